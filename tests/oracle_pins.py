"""Pins that tie the CPU oracle to facts outside itself.

Each ``pin_*`` takes the oracle module ``O`` and raises AssertionError on failure.  The pins
use the worked example the model page prints ("Attention mask layout": 16 tokens,
sliding_window=8, CSA m=4, HCA m'=8, index_topk=2), closed forms, invariants, library
routines (torch scaled_dot_product_attention in fp64, numpy sorts, math.cos/sin) and brute
force on tiny inputs.  test_oracle_mutations.py plants plausible mistakes in a copy of the
oracle and checks that every one of them trips at least one pin.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

HERE = os.path.dirname(__file__)
RNG = np.random.default_rng


def _worked():
    with open(os.path.join(HERE, "golden", "worked_example_16tok.json")) as f:
        return json.load(f)


def _close(a, b, tol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err} > {tol}"


# ----------------------------------------------------------------------------
# worked example on the page (visibility, sentinel, window cut)
# ----------------------------------------------------------------------------


def pin_worked_example_hca(O):
    g = _worked()
    S, m = g["S"], g["hca_m"]
    first = {int(k): v for k, v in g["stated"]["hca_entry_first_visible_query"].items()}
    for w, t0 in first.items():
        for t in range(S):
            vis = w < O.n_visible(t, m)
            assert vis == (t >= t0), (w, t)
    # the entries cover exactly the stated positions: mean pooling of one-hot tokens
    x = np.eye(S)  # token j carries a 1 in channel j
    pool = O.compress(x, np.zeros((S, S)), None, m, False)
    for w, (lo, hi) in g["stated"]["hca_entry_positions"].items():
        expect = np.zeros(S)
        expect[lo:hi + 1] = 1.0 / (hi - lo + 1)
        _close(pool[int(w)], expect, 1e-15, "hca entry coverage")


def pin_worked_example_csa(O):
    g = _worked()
    S, m, k = g["S"], g["csa_m"], g["index_topk"]
    rng = RNG(11)
    nI, cI = 3, 5
    q_idx = rng.standard_normal((1, S, nI, cI))
    w_idx = np.abs(rng.standard_normal((1, S, nI))) + 0.1
    k_pool = rng.standard_normal((1, S // m, cI))
    idx, _ = O.csa_index_topk(q_idx, w_idx, k_pool, [0], [S // m], m, k)
    idx = idx[0]
    for t in g["stated"]["csa_queries_with_no_entry"]:
        assert np.all(idx[t] == -1), (t, idx[t])
    for t in range(S):
        n_valid = int(np.sum(idx[t] >= 0))
        if t < m - 1:
            assert n_valid == 0
        elif t < 2 * m - 1:  # exactly one closed window: {0, -1}
            assert sorted(idx[t].tolist()) == [-1, 0], (t, idx[t])
        else:  # from t = 2m-1 on both slots fill
            assert n_valid == k, (t, idx[t])
        assert np.all(idx[t][idx[t] >= 0] < O.n_visible(t, m))


def pin_worked_example_sliding(O):
    g = _worked()
    S, W = g["S"], g["sliding_window"]
    cut_from = g["stated"]["sliding_lower_left_cut_from_query"]
    for t in range(S):
        rows = list(O.window_rows(t, W))
        assert rows[-1] == t, "causal: the query sees its own K=V"
        # the lower-left triangle is cut exactly from t >= window on
        assert (rows[0] > 0) == (t >= cut_from), (t, rows)
        assert rows == list(range(rows[0], t + 1))
    assert len(list(O.window_rows(S - 1, W))) == W


# ----------------------------------------------------------------------------
# RoPE (interleaved pairs on the trailing channels)
# ----------------------------------------------------------------------------


def pin_rope_closed_form(O):
    # single pair, base irrelevant for pair 0: angle = pos
    for pos in (1, 2, 7, -3):
        y = O.rope(np.array([1.0, 0.0]), pos, 2, 10000.0)
        _close(y, [math.cos(pos), math.sin(pos)], 1e-15, "rope pair0")
        y = O.rope(np.array([0.0, 1.0]), pos, 2, 10000.0)
        _close(y, [-math.sin(pos), math.cos(pos)], 1e-15, "rope pair0 (y)")
    # pair i rotates at base**(-2i/r); only its own two channels move; nope channels fixed
    C, r, base = 10, 6, 100.0
    for i in range(r // 2):
        x = np.zeros(C)
        x[C - r + 2 * i] = 1.0
        pos = 3
        y = O.rope(x, pos, r, base)
        ang = pos * base ** (-2.0 * i / r)
        expect = np.zeros(C)
        expect[C - r + 2 * i] = math.cos(ang)
        expect[C - r + 2 * i + 1] = math.sin(ang)
        _close(y, expect, 1e-15, f"rope pair {i}")


def pin_rope_group(O):
    rng = RNG(3)
    x = rng.standard_normal((4, 24))
    r, base = 8, 10000.0
    _close(O.rope(x, 0, r, base), x, 0.0, "rope(0) identity")
    _close(np.linalg.norm(O.rope(x, 123, r, base), axis=-1), np.linalg.norm(x, axis=-1), 1e-12,
           "rope isometry")
    _close(O.rope(O.rope(x, 17, r, base), 29, r, base), O.rope(x, 46, r, base), 1e-12,
           "rope composition")
    _close(O.rope(x, 5, 0, base), x, 0.0, "rope_dim 0")


# ----------------------------------------------------------------------------
# compressor
# ----------------------------------------------------------------------------


def pin_compress_mean_and_geometry(O):
    rng = RNG(5)
    S, C, m = 23, 6, 4  # S not a multiple of m: the trailing partial window emits nothing
    x = rng.standard_normal((S, C))
    z = np.zeros((S, C))
    # CSA: windows of 2m overlapping by m; entry w = [(w-1)m, (w+1)m) clipped at 0
    pool = O.compress(x, z, None, m, True)
    assert pool.shape == (S // m, C)
    for w in range(S // m):
        lo, hi = max(0, (w - 1) * m), (w + 1) * m
        _close(pool[w], x[lo:hi].mean(axis=0), 1e-14, f"csa mean entry {w}")
    # HCA: non-overlapping windows of m
    pool = O.compress(x, z, None, m, False)
    for w in range(S // m):
        _close(pool[w], x[w * m:(w + 1) * m].mean(axis=0), 1e-14, f"hca mean entry {w}")
    # tail tokens never contribute
    x2 = x.copy()
    x2[(S // m) * m:] += 100.0
    _close(O.compress(x2, z, None, m, True), O.compress(x, z, None, m, True), 0.0, "tail")


def pin_compress_known_weights(O):
    rng = RNG(6)
    S, C, m = 16, 5, 4
    x = rng.standard_normal((S, C))
    wts = rng.uniform(0.1, 2.0, size=(S, C))
    pool = O.compress(x, np.log(wts), None, m, False)
    for w in range(S // m):
        sl = slice(w * m, (w + 1) * m)
        _close(pool[w], (wts[sl] * x[sl]).sum(0) / wts[sl].sum(0), 1e-14, "known weights")
    # per-slot bias with a zero gate: weights exp(bias[slot]); CSA slot = j - (w-1)m
    bias = rng.standard_normal((2 * m, C))
    pool = O.compress(x, np.zeros((S, C)), bias, m, True)
    for w in range(S // m):
        js = [j for j in range((w - 1) * m, (w + 1) * m) if j >= 0]
        ew = np.exp(bias[[j - (w - 1) * m for j in js]])
        _close(pool[w], (ew * x[js]).sum(0) / ew.sum(0), 1e-14, f"slot bias entry {w}")
    # a dominant gate copies that token
    g = np.zeros((S, C))
    g[9] = 60.0
    pool = O.compress(x, g, None, m, True)
    _close(pool[2], x[9], 1e-20 + 1e-24, "one-hot gate copy (entry 2 covers 4..11)")


def pin_compress_permutation(O):
    rng = RNG(7)
    S, C, m = 12, 3, 4
    x = rng.standard_normal((S, C))
    g = rng.standard_normal((S, C))
    perm = np.arange(S)
    perm[4:8] = perm[4:8][::-1]  # reorder tokens inside HCA window 1
    a = O.compress(x, g, None, m, False)
    b = O.compress(x[perm], g[perm], None, m, False)
    _close(a, b, 1e-14, "permutation invariance")


def pin_compress_rope_position(O):
    # constant tokens, zero gate: entry w equals the token rotated at (w+1)m - 1 + offset
    S, C, m, r, base, off = 20, 8, 4, 4, 50.0, 7
    x = np.tile(np.arange(1.0, C + 1.0), (S, 1))
    pool = O.compress(x, np.zeros((S, C)), None, m, True, r, base, off)
    for w in range(S // m):
        p = (w + 1) * m - 1 + off
        e = x[0].copy()
        for i in range(r // 2):
            ang = p * base ** (-2.0 * i / r)
            a, b = x[0, C - r + 2 * i], x[0, C - r + 2 * i + 1]
            e[C - r + 2 * i] = a * math.cos(ang) - b * math.sin(ang)
            e[C - r + 2 * i + 1] = a * math.sin(ang) + b * math.cos(ang)
        _close(pool[w], e, 1e-12, f"entry {w} rotated at its closing position")


# ----------------------------------------------------------------------------
# indexer scores and top-k
# ----------------------------------------------------------------------------


def pin_index_single_head(O):
    rng = RNG(8)
    q = rng.standard_normal((1, 7))
    K = rng.standard_normal((20, 7))
    s = O.index_scores(q, np.array([1.0]), K)
    _close(s, [max(0.0, float(np.dot(q[0], K[w]))) for w in range(20)], 1e-13, "relu(q.k)")
    s2 = O.index_scores(q, np.array([2.5]), K)
    _close(s2, 2.5 * s, 1e-13, "head weight scales")
    s3 = O.index_scores(q, np.array([-1.0]), K)
    _close(s3, -s, 1e-13, "negative head weight")
    # a key with a negative dot product contributes nothing (ReLU), not a negative score
    Kn = -np.sign(q) * np.abs(rng.standard_normal((3, 7)))
    _close(O.index_scores(q, np.array([1.0]), Kn), np.zeros(3), 0.0, "relu cut")


def pin_index_heads_additive(O):
    rng = RNG(9)
    q = rng.standard_normal((4, 6))
    wv = rng.standard_normal(4)
    K = rng.standard_normal((15, 6))
    full = O.index_scores(q, wv, K)
    parts = O.index_scores(q[:2], wv[:2], K) + O.index_scores(q[2:], wv[2:], K)
    _close(full, parts, 1e-13, "heads add")


def pin_topk_bruteforce(O):
    rng = RNG(10)
    for trial in range(40):
        V = int(rng.integers(0, 12))
        k = int(rng.integers(1, 8))
        s = rng.integers(-3, 4, size=V).astype(np.float64)  # many exact ties
        if V:
            s[rng.random(V) < 0.3] = -0.0
        sel = O.topk_select(s, k)
        assert sel.shape == (k,)
        valid = sel[sel >= 0]
        assert np.all(sel[len(valid):] == -1), "valid first, then -1"
        assert len(valid) == min(k, V)
        # library sort: stable sort on the negated score keeps the lower index first on ties
        ref = np.argsort(-(s + 0.0), kind="stable")[:min(k, V)]
        assert set(valid.tolist()) == set(ref.tolist()), (s, k, sel, ref)
        # definition, by brute force over all subsets of that size (small V only)
        if V <= 9:
            def key(sub):
                return (sorted((-s[i] + 0.0 for i in sub)), sorted(sub))
            best = min(itertools.combinations(range(V), min(k, V)), key=key)
            assert set(best) == set(valid.tolist())


def pin_topk_signed_zero(O):
    s = np.array([0.0, -0.0, 1.0, -0.0, 0.0, -2.0])
    sel = O.topk_select(s, 3)
    assert set(sel.tolist()) == {2, 0, 1}, sel  # zeros tie, lower index wins
    sel = O.topk_select(np.array([-0.0, 0.0]), 1)
    assert sel.tolist() == [0]


# ----------------------------------------------------------------------------
# attention: dense SDPA in fp64, sink closed forms, eq. 26 shift invariance
# ----------------------------------------------------------------------------


def _sdpa_reference(O, q_rot, keys, mask_keep, sink, scale):
    """torch SDPA in fp64 with separate (equal) K and V, plus a zero-valued sink column."""
    import torch

    T, H, D = q_rot.shape
    n = keys.shape[0]
    Kx = np.concatenate([keys, np.zeros((1, D))], axis=0)
    bias = np.where(mask_keep, 0.0, -np.inf)  # [T, n]
    full = np.empty((H, T, n + 1))
    full[:, :, :n] = bias[None]
    full[:, :, n] = np.asarray(sink)[:, None]  # logit of the zero key is exactly s_h
    qt = torch.tensor(q_rot.transpose(1, 0, 2))  # [H, T, D]
    kt = torch.tensor(Kx)[None].expand(H, n + 1, D).contiguous()
    vt = torch.tensor(Kx.copy())[None].expand(H, n + 1, D).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt,
                                                          attn_mask=torch.tensor(full),
                                                          scale=scale)
    return o.numpy().transpose(1, 0, 2)  # [T, H, D]


def pin_hca_equals_dense_sdpa(O):
    rng = RNG(12)
    S, H, D, r, m, W, base = 40, 3, 12, 4, 8, 6, 10000.0
    q = rng.standard_normal((1, S, H, D))
    kv = rng.standard_normal((1, S, D))
    gate = rng.standard_normal((1, S, D))
    bias = rng.standard_normal((m, D))
    sink = rng.standard_normal(H)
    kv_win = O.swa_concat(kv, [0], r, base)
    pool = O.csa_compress(kv, gate, bias, m, False, r, base)
    N = pool.shape[1]
    out = O.hca_attend(q, kv_win, [0], pool, [N], m, sink, [0], W, r, base)
    keys = np.concatenate([kv_win[0], pool[0]], axis=0)
    keep = np.zeros((S, S + N), dtype=bool)
    for t in range(S):
        keep[t, max(0, t - W + 1):t + 1] = True
        keep[t, S:S + (t + 1) // m] = True
    q_rot = O.rope(q[0], np.arange(S)[:, None], r, base)
    ref = _sdpa_reference(O, q_rot, keys, keep, sink, 1.0 / math.sqrt(D))
    ref = O.rope(ref, -np.arange(S)[:, None], r, base)
    _close(out[0], ref, 1e-12, "HCA vs dense SDPA")


def pin_sliding_and_sink(O):
    rng = RNG(13)
    S, H, D, r, W, base = 20, 4, 8, 4, 5, 10000.0
    q = rng.standard_normal((1, S, H, D))
    kv = rng.standard_normal((1, S, D))
    sink = rng.standard_normal(H)
    kv_win = O.swa_concat(kv, [0], r, base)
    out = O.hca_attend(q, kv_win, [0], None, None, 128, sink, [0], W, r, base)
    # t = 0: one key and the sink -> o = sigmoid(z - s) * v, with v = the token at position 0
    z = (q[0, 0] @ kv[0, 0]) / math.sqrt(D)  # rotation at position 0 is the identity
    _close(out[0, 0], (1.0 / (1.0 + np.exp(sink - z)))[:, None] * kv[0, 0][None], 1e-13,
           "single key + sink")
    # sink -> -inf is plain softmax over the window
    out_ns = O.hca_attend(q, kv_win, [0], None, None, 128, np.full(H, -np.inf), [0], W, r, base)
    t = 11
    keys = kv_win[0, t - W + 1:t + 1]
    qr = O.rope(q[0, t], t, r, base)
    logits = qr @ keys.T / math.sqrt(D)
    p = np.exp(logits - logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    _close(out_ns[0, t], O.rope(p @ keys, -t, r, base), 1e-13, "no-sink softmax")
    # the sink only ever shrinks the weights: output = (1 - p_sink) * no-sink output
    lse = np.log(np.exp(logits - logits.max(1, keepdims=True)).sum(1)) + logits.max(1)
    frac = 1.0 / (1.0 + np.exp(sink - lse))
    _close(out[0, t], frac[:, None] * out_ns[0, t], 1e-13, "sink as zero-value logit")


def _csa_inputs(seed, S=33, H=2, D=8, r=4, m=4, nI=2, cI=6):
    rng = RNG(seed)
    return dict(
        q=rng.standard_normal((1, S, H, D)), kv=rng.standard_normal((1, S, D)),
        gate=rng.standard_normal((1, S, D)), q_idx=rng.standard_normal((1, S, nI, cI)),
        k_idx=rng.standard_normal((1, S, cI)), g_idx=rng.standard_normal((1, S, cI)),
        w_idx=rng.standard_normal((1, S, nI)), bias=rng.standard_normal((2 * m, D)),
        bias_idx=rng.standard_normal((2 * m, cI)), bias_hca=rng.standard_normal((8, D)),
        sink=rng.standard_normal(H))


class _Cfg:
    def __init__(self, **kw):
        self.__dict__.update(kw)


def pin_csa_full_k_equals_dense(O):
    inp = _csa_inputs(14)
    cfg = _Cfg(m=4, r=4, base=10000.0, k=64, W=5, m_hca=4)
    out, idx, aux = O.csa_layer(inp, cfg)
    pool = aux["pool"]
    dense = O.hca_attend(inp["q"], aux["kv_win"], [0], pool, [pool.shape[1]], cfg.m, inp["sink"],
                         [0], cfg.W, cfg.r, cfg.base)
    _close(out, dense, 1e-12, "CSA with k >= V(t) equals the dense range")


def pin_eq26_shift_invariance(O):
    inp = _csa_inputs(15)
    cfg = _Cfg(m=4, r=4, base=10000.0, k=3, W=5, m_hca=8)
    a, ia, _ = O.csa_layer(inp, cfg, pos_offset=0)
    for delta in (1, 977, 1_000_003):
        b, ib, _ = O.csa_layer(inp, cfg, pos_offset=delta)
        assert np.array_equal(ia, ib)
        _close(a, b, 2e-9, f"CSA shift {delta}")
    h0, _ = O.hca_layer(inp, cfg)
    h1, _ = O.hca_layer(inp, cfg, pos_offset=4242)
    _close(h0, h1, 2e-9, "HCA shift")
    # the rotation itself is not trivial: without the output counter-rotation the results move
    assert np.max(np.abs(O.rope(a, 5, cfg.r, cfg.base) - a)) > 1e-3


def pin_csa_sparse_selection(O):
    """Only the selected entries contribute: un-selected entries can change freely."""
    inp = _csa_inputs(16)
    cfg = _Cfg(m=4, r=4, base=10000.0, k=2, W=3, m_hca=8)
    out, idx, aux = O.csa_layer(inp, cfg)
    pool = aux["pool"].copy()
    t = 30
    chosen = set(idx[0, t][idx[0, t] >= 0].tolist())
    others = [w for w in range(O.n_visible(t, cfg.m)) if w not in chosen]
    pool2 = pool.copy()
    pool2[0, others] += 50.0
    o1 = O.csa_attend(inp["q"], aux["kv_win"], [0], pool, idx, inp["sink"], [0], cfg.W, cfg.r,
                      cfg.base, rows=[(0, t)])
    o2 = O.csa_attend(inp["q"], aux["kv_win"], [0], pool2, idx, inp["sink"], [0], cfg.W, cfg.r,
                      cfg.base, rows=[(0, t)])
    _close(o1, o2, 0.0, "unselected entries")
    pool3 = pool.copy()
    pool3[0, sorted(chosen)[0]] += 1.0
    o3 = O.csa_attend(inp["q"], aux["kv_win"], [0], pool3, idx, inp["sink"], [0], cfg.W, cfg.r,
                      cfg.base, rows=[(0, t)])
    assert np.max(np.abs(o3 - o1)) > 1e-6, "a selected entry must matter"


def pin_round_bf16(O):
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -3.0e-5, 0.0, 65504.0])
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even significand wins (1.0)
    expect = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0, -3.0e-5, 0.0, 65536.0])
    got = O.round_bf16(vals)
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == expect[2] and got[3] == 1.0
    assert abs(got[4] - expect[4]) <= 2 ** -8 * 3.0e-5
    assert got[5] == 0.0 and got[6] == 65536.0



# ----------------------------------------------------------------------------
# compressor variant R4b: separate projections for the two halves of a CSA window
# ----------------------------------------------------------------------------


def pin_compress_split_halves(O):
    """R4b reduces to R4 when both projections agree; the earlier half reads only the second
    projection and the later half only the first; a dominant gate copies one slot's value."""
    r = RNG(31)
    S, C, m = 21, 5, 4
    x, g = r.standard_normal((S, C)), r.standard_normal((S, C))
    bias = r.standard_normal((2 * m, C))
    same = O.compress(x, g, bias, m, True, x_prev=x, gate_prev=g)
    _close(same, O.compress(x, g, bias, m, True), 0.0, "R4b with equal projections")
    xp, gp = r.standard_normal((S, C)), r.standard_normal((S, C))
    base = O.compress(x, g, bias, m, True, x_prev=xp, gate_prev=gp)
    w = 3  # tokens 8..11 form its earlier half, 12..15 its later half
    x2 = x.copy(); x2[8:12] += 5.0; g2 = g.copy(); g2[8:12] -= 3.0
    _close(O.compress(x2, g2, bias, m, True, x_prev=xp, gate_prev=gp)[w], base[w], 0.0,
           "earlier half ignores the first projection")
    xp2 = xp.copy(); xp2[12:16] += 5.0; gp2 = gp.copy(); gp2[12:16] -= 3.0
    _close(O.compress(x, g, bias, m, True, x_prev=xp2, gate_prev=gp2)[w], base[w], 0.0,
           "later half ignores the second projection")
    for j, src in ((9, "prev"), (14, "cur")):
        gq, gpq = np.zeros((S, C)), np.zeros((S, C))
        (gpq if src == "prev" else gq)[j] = 80.0
        e = O.compress(x, gq, None, m, True, x_prev=xp, gate_prev=gpq)[w]
        _close(e, (xp if src == "prev" else x)[j], 1e-12, f"one-hot slot {j} from {src}")


# ----------------------------------------------------------------------------
# grouped output projection
# ----------------------------------------------------------------------------


def _oproj_case(seed, T=3, H=4, D=3, groups=2, rank=5, hidden=6):
    r = RNG(seed)
    attn = r.standard_normal((T, H, D))
    w_a = r.standard_normal((groups, rank, H // groups * D))
    w_b = r.standard_normal((hidden, groups * rank))
    return attn, w_a, w_b, groups


def pin_oproj_bruteforce(O):
    """Explicit loops over every output element on a tiny non-square case."""
    attn, w_a, w_b, G = _oproj_case(11)
    T, H, D = attn.shape
    rank, hidden, hpg = w_a.shape[1], w_b.shape[0], H // G
    out, mid = O.grouped_out_proj(attn, w_a, w_b, G)
    want_mid = np.zeros((T, G * rank))
    for t in range(T):
        for g in range(G):
            for j in range(rank):
                acc = 0.0
                for hh in range(hpg):
                    for d in range(D):
                        acc += attn[t, g * hpg + hh, d] * w_a[g, j, hh * D + d]
                want_mid[t, g * rank + j] = acc
    want = np.zeros((T, hidden))
    for t in range(T):
        for o in range(hidden):
            want[t, o] = sum(want_mid[t, i] * w_b[o, i] for i in range(G * rank))
    _close(mid, want_mid, 1e-12, "intermediate")
    _close(out, want, 1e-12, "output")


def pin_oproj_group_locality(O):
    """Changing the heads of one group changes only that group's rank slice; a one-hot head
    lands in the slice of the group of consecutive heads that holds it."""
    attn, w_a, w_b, G = _oproj_case(12, H=6, groups=3)
    _, mid0 = O.grouped_out_proj(attn, w_a, w_b, G)
    rank, hpg = w_a.shape[1], attn.shape[1] // G
    for g in range(G):
        a2 = attn.copy()
        a2[:, g * hpg:(g + 1) * hpg] += 1.0
        _, mid1 = O.grouped_out_proj(a2, w_a, w_b, G)
        changed = np.abs(mid1 - mid0).max(axis=0) > 0
        assert changed[g * rank:(g + 1) * rank].all()
        assert not np.delete(changed, np.s_[g * rank:(g + 1) * rank]).any(), g
    one = np.zeros_like(attn)
    one[0, 1, 0] = 1.0  # head 1 belongs to group 0 (heads 0, 1)
    _, mid = O.grouped_out_proj(one, w_a, w_b, G)
    _close(mid[0, :rank], w_a[0, :, attn.shape[2]], 1e-15, "one-hot head 1")
    assert not mid[0, rank:].any()


def pin_oproj_identity(O):
    """One group, identity weights: the output is the attention output itself."""
    r = RNG(13)
    attn = r.standard_normal((4, 2, 3))
    K = 6
    out, mid = O.grouped_out_proj(attn, np.eye(K)[None], np.eye(K), 1)
    _close(out, attn.reshape(4, K), 0.0, "identity")
    _close(mid, attn.reshape(4, K), 0.0, "identity intermediate")


# ----------------------------------------------------------------------------
# input projections (readings R23/R24)
# ----------------------------------------------------------------------------

_INPROJ_WIDTH = {"q_a": 4, "kv": 3, "gate": 3, "k_idx": 2, "g_idx": 2, "w_idx": 2, "q": 5, "q_idx": 6}


def _inproj_case(seed, kind, T=3, hidden=7):
    """Tiny distinct widths, so a name wired to the wrong weight changes a shape or a value."""
    r = RNG(seed)
    x = r.standard_normal((T, hidden))
    ws = {}
    for n in _inproj_names(kind):
        fan_in = _INPROJ_WIDTH["q_a"] if n in ("q", "q_idx") else hidden
        ws[n] = r.standard_normal((_INPROJ_WIDTH[n], fan_in))
    return x, ws


def _inproj_names(kind):
    return {"sliding": ("q_a", "kv", "q"), "hca": ("q_a", "kv", "gate", "q"),
            "csa": ("q_a", "kv", "gate", "k_idx", "g_idx", "w_idx", "q", "q_idx")}[kind]


def pin_inproj_bruteforce(O):
    """Explicit loops over every output element: the latent from x, q and q_idx from the
    latent, the others from x; each layer type lists exactly its own outputs."""
    for kind in ("csa", "hca", "sliding"):
        x, ws = _inproj_case(21, kind)
        got = O.input_projections(x, ws, kind)
        T, hidden = x.shape
        lat = np.zeros((T, _INPROJ_WIDTH["q_a"]))
        for t in range(T):
            for j in range(lat.shape[1]):
                lat[t, j] = sum(x[t, k] * ws["q_a"][j, k] for k in range(hidden))
        want = {"c_q": lat}
        for n in _inproj_names(kind):
            if n == "q_a":
                continue
            src = lat if n in ("q", "q_idx") else x
            y = np.zeros((T, _INPROJ_WIDTH[n]))
            for t in range(T):
                for j in range(y.shape[1]):
                    y[t, j] = sum(src[t, k] * ws[n][j, k] for k in range(src.shape[1]))
            want[n] = y
        assert sorted(got) == sorted(want), (kind, sorted(got))
        for n in want:
            _close(got[n], want[n], 1e-12, f"{kind} {n}")


def pin_inproj_one_hot_rows(O):
    """Row x = e_j gives column j of every weight read from x, and q / q_idx of the latent
    W_qa[:, j] (a wrong weight, a transposed one or a wrong input fails here)."""
    x, ws = _inproj_case(22, "csa", T=1)
    hidden = x.shape[1]
    for j in range(hidden):
        e = np.zeros((1, hidden))
        e[0, j] = 1.0
        got = O.input_projections(e, ws, "csa")
        _close(got["c_q"][0], ws["q_a"][:, j], 0.0, f"c_q e_{j}")
        for n in ("kv", "gate", "k_idx", "g_idx", "w_idx"):
            _close(got[n][0], ws[n][:, j], 0.0, f"{n} e_{j}")
        for n in ("q", "q_idx"):
            _close(got[n][0], ws[n] @ ws["q_a"][:, j], 1e-12, f"{n} e_{j}")


def pin_inproj_merged_query_weight(O):
    """The two query factors compose to the single product x (W_qb W_qa)^T, and with an
    identity first factor the query is the one-factor projection of x."""
    x, ws = _inproj_case(23, "hca", T=4)
    got = O.input_projections(x, ws, "hca")
    _close(got["q"], x @ (ws["q"] @ ws["q_a"]).T, 1e-12, "merged query weight")
    ws2 = dict(ws, q_a=np.eye(x.shape[1]), q=RNG(24).standard_normal((5, x.shape[1])))
    _close(O.input_projections(x, ws2, "hca")["q"], x @ ws2["q"].T, 1e-12, "identity first factor")
    _close(O.input_projections(x, ws2, "hca")["c_q"], x, 0.0, "identity latent")


def pin_inproj_token_locality(O):
    """Each output row depends on its own token's hidden state only."""
    x, ws = _inproj_case(25, "csa", T=5)
    base = O.input_projections(x, ws, "csa")
    x2 = x.copy()
    x2[2] += 1.0
    moved = O.input_projections(x2, ws, "csa")
    for n in base:
        d = np.abs(moved[n] - base[n]).max(axis=1)
        assert d[2] > 0 and not np.delete(d, 2).any(), n


# ----------------------------------------------------------------------------
# positions, buffer origins and pool capacities (the arguments decode and chunked prefill use)
# ----------------------------------------------------------------------------


def _rot_rows(x, pos, r, base):
    """Interleaved-pair rotation of the trailing r channels written out with math.cos/sin per
    element (independent of the oracle's rope): rows x[i] at positions pos[i]."""
    x = np.array(x, dtype=np.float64, copy=True)
    C = x.shape[-1]
    flat = x.reshape(-1, C)
    pos = np.broadcast_to(np.asarray(pos, dtype=np.float64), flat.shape[:1])
    for n in range(flat.shape[0]):
        for i in range(r // 2):
            ang = pos[n] * base ** (-2.0 * i / r)
            a, b = flat[n, C - r + 2 * i], flat[n, C - r + 2 * i + 1]
            flat[n, C - r + 2 * i] = a * math.cos(ang) - b * math.sin(ang)
            flat[n, C - r + 2 * i + 1] = a * math.sin(ang) + b * math.cos(ang)
    return flat.reshape(x.shape)


def _dense_ref(q_rows, q_pos, keys, keep, sink, r, base, D):
    """Masked attention of queries at sequence indices q_pos over rotated keys, by torch SDPA in
    fp64 (K and V separate but equal, sink as a zero-value column), counter-rotated."""
    T, H = q_rows.shape[:2]
    q_rot = np.stack([_rot_rows(q_rows[t], q_pos[t], r, base) for t in range(T)])
    o = _sdpa_reference(None, q_rot, keys, keep, sink, 1.0 / math.sqrt(D))
    return np.stack([_rot_rows(o[t], -q_pos[t], r, base) for t in range(T)])


def pin_window_buffer_origin_and_clipping(O):
    """A window buffer whose row 0 is sequence index kv_pos0 and which holds S_buf rows: the
    query at p attends the rows of sequence indices max(0, p-W+1) .. p that the buffer holds
    and nothing else (origin at 0, inside the window, past some queries; a buffer that ends
    early), for queries starting at q_pos0 > 0 too."""
    rng = RNG(41)
    S, H, D, r, W, base = 30, 2, 8, 4, 6, 10000.0
    q = rng.standard_normal((1, S, H, D))
    kv = rng.standard_normal((S, D))
    sink = rng.standard_normal(H)
    rot = _rot_rows(kv, np.arange(S), r, base)
    for kv_pos0, S_buf in ((0, S), (3, S - 3), (12, 10), (25, 5), (9, 2)):
        buf = rot[kv_pos0:kv_pos0 + S_buf][None]
        for q_pos0 in (0, 7):
            qs = q[:, q_pos0:]
            p = q_pos0 + np.arange(S - q_pos0)
            keep = np.zeros((len(p), S), dtype=bool)
            for n, pt in enumerate(p):
                for j in range(max(0, pt - W + 1), pt + 1):
                    keep[n, j] = kv_pos0 <= j < kv_pos0 + S_buf
            ref = _dense_ref(qs[0], p, rot, keep, sink, r, base, D)
            got = O.hca_attend(qs, buf, [kv_pos0], None, None, 128, sink, [q_pos0], W, r, base)
            _close(got[0], ref, 1e-12, f"window buffer at {kv_pos0} ({S_buf} rows), q from {q_pos0}")
            # the CSA call takes the same window rows (with no entry selected)
            none = np.full((1, len(p), 2), -1)
            got_c = O.csa_attend(qs, buf, [kv_pos0], np.zeros((1, 1, D)), none, sink, [q_pos0], W,
                                 r, base)
            _close(got_c[0], ref, 1e-12, f"CSA window buffer at {kv_pos0}, q from {q_pos0}")


def pin_index_topk_positions_and_capacity(O):
    """csa_index_topk for queries starting at q_pos0 > 0 and pools whose valid count n_pool
    cuts the visible entries: explicit score loops and a stable library sort."""
    rng = RNG(42)
    B, T, nI, cI, m, N_cap = 2, 9, 3, 5, 4, 12
    q_idx = rng.standard_normal((B, T, nI, cI))
    w_idx = rng.standard_normal((B, T, nI))
    k_pool = rng.standard_normal((B, N_cap, cI))
    q_pos0, n_pool = [17, 30], [5, 12]
    for k in (3, 6):
        idx, sc = O.csa_index_topk(q_idx, w_idx, k_pool, q_pos0, n_pool, m, k)
        for b in range(B):
            for t in range(T):
                V = min((q_pos0[b] + t + 1) // m, n_pool[b])
                s = np.zeros(V)
                for w in range(V):
                    for h in range(nI):
                        dot = sum(q_idx[b, t, h, c] * k_pool[b, w, c] for c in range(cI))
                        s[w] += w_idx[b, t, h] * max(dot, 0.0)
                ref = np.sort(np.argsort(-s, kind="stable")[:min(k, V)])
                row = idx[b, t]
                assert np.array_equal(row[:len(ref)], ref) and np.all(row[len(ref):] == -1), \
                    (k, b, t, row, ref)
                _close(sc[b, t, :len(ref)], s[ref], 1e-12, "scores of the kept entries")


def pin_swa_positions(O):
    """swa_concat rotates row i of sequence b at new_pos0[b] + i + offset (closed form)."""
    rng = RNG(43)
    kv = rng.standard_normal((2, 5, 6))
    new_pos0, r, base, off = [0, 37], 4, 100.0, 3
    got = O.swa_concat(kv, new_pos0, r, base, off)
    for b in range(2):
        for i in range(5):
            _close(got[b, i], _rot_rows(kv[b, i], new_pos0[b] + i + off, r, base), 1e-12,
                   f"window row {b},{i}")


def pin_hca_pool_capacity(O):
    """hca_attend with n_pool below the pool's rows: entry w is visible to the query at p iff
    w < min((p+1)//m, n_pool); fp64 SDPA with that mask."""
    rng = RNG(44)
    S, H, D, r, m, W, base = 40, 2, 8, 4, 8, 5, 10000.0
    q = rng.standard_normal((1, S, H, D))
    kv = rng.standard_normal((S, D))
    pool = rng.standard_normal((1, 5, D))
    sink = rng.standard_normal(H)
    rot = _rot_rows(kv, np.arange(S), r, base)
    for n_pool in (3, 5, 0):
        got = O.hca_attend(q, rot[None], [0], pool, [n_pool], m, sink, [0], W, r, base)
        keys = np.concatenate([rot, pool[0]], axis=0)
        keep = np.zeros((S, S + 5), dtype=bool)
        for t in range(S):
            keep[t, max(0, t - W + 1):t + 1] = True
            for w in range(min((t + 1) // m, n_pool)):
                keep[t, S + w] = True
        ref = _dense_ref(q[0], np.arange(S), keys, keep, sink, r, base, D)
        _close(got[0], ref, 1e-12, f"HCA with n_pool = {n_pool}")


def pin_decode_layout_equals_prefill_row(O):
    """The decode layout (one query at L-1, a window buffer holding positions L-W .. L-1, a
    pool whose first L//m rows are valid and the rest arbitrary) gives row L-1 of the one-shot
    prefill layer, for CSA and HCA."""
    inp = _csa_inputs(45, S=33)
    cfg = _Cfg(m=4, r=4, base=10000.0, k=3, W=5, m_hca=8)
    out, idx, aux = O.csa_layer(inp, cfg)
    junk = RNG(46).standard_normal
    for L in (33, 20, 4, 3):
        t = L - 1
        n = L // cfg.m
        win = aux["kv_win"][:, L - cfg.W:L] if L >= cfg.W else aux["kv_win"][:, :L]
        kv0 = max(L - cfg.W, 0)
        k_pool = np.concatenate([aux["k_pool"][:, :n], junk((1, 4, aux["k_pool"].shape[2]))], axis=1)
        pool = np.concatenate([aux["pool"][:, :n], junk((1, 4, aux["pool"].shape[2]))], axis=1)
        di, _ = O.csa_index_topk(inp["q_idx"][:, t:t + 1], inp["w_idx"][:, t:t + 1], k_pool, [t], [n],
                                 cfg.m, cfg.k)
        assert np.array_equal(di[0, 0], idx[0, t]), (L, di[0, 0], idx[0, t])
        do = O.csa_attend(inp["q"][:, t:t + 1], win, [kv0], pool, di, inp["sink"], [t], cfg.W, cfg.r,
                          cfg.base)
        _close(do[0, 0], out[0, t], 1e-12, f"CSA decode row at L={L}")
    hout, haux = O.hca_layer(inp, cfg)
    hp = haux["pool"]
    for L in (33, 16, 9):
        t, n = L - 1, L // cfg.m_hca
        pool = np.concatenate([hp[:, :n], junk((1, 3, hp.shape[2]))], axis=1)
        do = O.hca_attend(inp["q"][:, t:t + 1], haux["kv_win"][:, L - cfg.W:L], [L - cfg.W], pool, [n],
                          cfg.m_hca, inp["sink"], [t], cfg.W, cfg.r, cfg.base)
        _close(do[0, 0], hout[0, t], 1e-12, f"HCA decode row at L={L}")


def pin_chunked_prefill_equals_one_shot(O):
    """Prefill in chunks of queries (entries pooled chunk by chunk through entry ranges, each
    chunk's window buffer starting W-1 rows before it, the pool's valid count growing) equals
    the one-shot layer, for CSA and HCA."""
    inp = _csa_inputs(47, S=33)
    cfg = _Cfg(m=4, r=4, base=10000.0, k=3, W=5, m_hca=8)
    out, idx, aux = O.csa_layer(inp, cfg)
    hout, haux = O.hca_layer(inp, cfg)
    S = 33
    D = inp["kv"].shape[2]
    pool = np.zeros((1, S // cfg.m, D))
    k_pool = np.zeros((1, S // cfg.m, inp["k_idx"].shape[2]))
    hpool = np.zeros((1, S // cfg.m_hca, D))
    got, hgot = [], []
    for c0, c1 in ((0, 12), (12, 25), (25, 33)):
        e0, e1 = c0 // cfg.m, c1 // cfg.m
        pool[:, e0:e1] = O.csa_compress(inp["kv"][:, :c1], inp["gate"][:, :c1], inp["bias"], cfg.m,
                                        True, cfg.r, cfg.base, 0, e0, e1)
        k_pool[:, e0:e1] = O.csa_compress(inp["k_idx"][:, :c1], inp["g_idx"][:, :c1], inp["bias_idx"],
                                          cfg.m, True, 0, 10000.0, 0, e0, e1)
        h0, h1 = c0 // cfg.m_hca, c1 // cfg.m_hca
        hpool[:, h0:h1] = O.csa_compress(inp["kv"][:, :c1], inp["gate"][:, :c1], inp["bias_hca"],
                                         cfg.m_hca, False, cfg.r, cfg.base, 0, h0, h1)
        kv0 = max(c0 - cfg.W + 1, 0)
        win = O.swa_concat(inp["kv"][:, kv0:c1], [kv0], cfg.r, cfg.base)
        ci, _ = O.csa_index_topk(inp["q_idx"][:, c0:c1], inp["w_idx"][:, c0:c1], k_pool, [c0], [e1],
                                 cfg.m, cfg.k)
        assert np.array_equal(ci[0], idx[0, c0:c1])
        got.append(O.csa_attend(inp["q"][:, c0:c1], win, [kv0], pool, ci, inp["sink"], [c0], cfg.W,
                                cfg.r, cfg.base)[0])
        hgot.append(O.hca_attend(inp["q"][:, c0:c1], win, [kv0], hpool, [h1], cfg.m_hca, inp["sink"],
                                 [c0], cfg.W, cfg.r, cfg.base)[0])
    _close(np.concatenate(got), out[0], 1e-12, "chunked CSA")
    _close(np.concatenate(hgot), hout[0], 1e-12, "chunked HCA")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

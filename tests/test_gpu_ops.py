"""Per-call GPU parity: each C-ABI entry point against the CPU oracle on the same inputs.

Inputs come from the seeded workload generator (keyed by test name); the oracle receives the
exact fp64 values of the stored inputs.  Tolerances: fp32 |d| <= 1e-5 max|ref|; bf16
|d| <= 2e-2 max|ref| (and pool / window rows within one bf16 ulp of the exact value); top-k
sets exact except within the 1e-4 relative band around the k-th score.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import (assert_bf16_ulp, assert_close, check_topk_row, dev, enc, host,
                      torch_dtype)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU machines only to be skipped
    pytest.skip("no GPU", allow_module_level=True)

import long_context_sparse_09_amd as L  # noqa: E402


def normal(name, shape, seed=101):
    return W.normal_tensor(seed, 0, name, shape).astype(np.float64)


def i32(v):
    return torch.tensor(np.asarray(v, dtype=np.int32), device="cuda")


# ---------------------------------------------------------------------------- compress

COMPRESS_CASES = [
    # dtype, B, S, C, m, overlap, rope, bias, entries
    ("fp32", 1, 259, 64, 4, True, 16, True, None),     # tiny-CSA shape, ragged tail
    ("fp32", 1, 256, 32, 4, True, 0, True, None),      # tiny indexer keys
    ("fp32", 2, 37, 6, 2, True, 2, True, None),        # C not a multiple of 8
    ("bf16", 1, 1030, 512, 4, True, 64, True, None),   # CSA K=V pool
    ("bf16", 2, 1030, 128, 4, True, 0, True, None),    # indexer keys, B = 2
    ("bf16", 1, 1000, 512, 128, False, 64, True, None),  # HCA, 7 entries + tail
    ("bf16", 1, 700, 512, 128, False, 64, False, None),  # HCA, no bias
    ("bf16", 1, 300, 512, 4, True, 64, True, (20, 41)),  # entry sub-range (chunked prefill)
    ("bf16", 1, 90, 96, 3, True, 8, False, None),      # odd rate
    ("bf16", 2, 515, 64, 4, True, 16, True, None),     # m=4 at C=64: the register-window kernel
    ("bf16", 1, 301, 256, 4, True, 32, True, None),    # staged, two wavefronts per workgroup
    ("bf16", 1, 203, 384, 4, True, 64, True, None),    # 48-lane chunks: the generic kernel
]


@pytest.mark.parametrize("case", COMPRESS_CASES, ids=lambda c: "-".join(map(str, c[:7])))
def test_csa_compress(case):
    dt, B, S, C, m, overlap, r, use_bias, entries = case
    x = normal("x", (B, S, C))
    g = normal("g", (B, S, C))
    span = 2 * m if overlap else m
    bias = normal("bias", (span, C)).astype(np.float32) if use_bias else None
    xs, gs = enc(x, dt), enc(g, dt)
    x64, g64 = W.to_f64(xs), W.to_f64(gs)
    N = S // m
    e0, e1 = entries if entries else (0, N)
    base, off = 10000.0, 37
    pool = torch.full((B, N, C), 7.0, dtype=torch_dtype(dt), device="cuda")
    L.csa_compress(dev(xs), dev(gs), None if bias is None else dev(bias), pool, m, overlap, e0, e1,
                   r, base, off)
    got = host(pool)
    ref = oracle.csa_compress(x64, g64, None if bias is None else bias.astype(np.float64), m,
                              overlap, r, base, off, e0, e1)
    assert np.all(got[:, :e0] == 7.0) and np.all(got[:, e1:] == 7.0), "rows outside the range"
    assert_close(got[:, e0:e1], ref, dt, "pool")
    if dt == "bf16":
        assert_bf16_ulp(got[:, e0:e1], ref, "pool")


SPLIT_CASES = [
    # dtype, B, S, C, m, rope, bias, entries
    ("fp32", 1, 259, 64, 4, 16, True, None),
    ("bf16", 2, 1030, 512, 4, 64, True, None),
    ("bf16", 1, 1030, 128, 4, 0, True, (30, 200)),
    ("bf16", 1, 700, 512, 128, 64, False, None),      # long windows: slots split over thread groups
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "-".join(map(str, c[:6])))
def test_csa_compress_split_halves(case):
    """R4b: the earlier half of every overlapping window reads the second projection."""
    dt, B, S, C, m, r, use_bias, entries = case
    x, g = normal("x", (B, S, C)), normal("g", (B, S, C))
    xp, gp = normal("xp", (B, S, C)), normal("gp", (B, S, C))
    bias = normal("bias", (2 * m, C)).astype(np.float32) if use_bias else None
    enc4 = [enc(a, dt) for a in (x, g, xp, gp)]
    N = S // m
    e0, e1 = entries if entries else (0, N)
    pool = torch.full((B, N, C), 7.0, dtype=torch_dtype(dt), device="cuda")
    L.csa_compress(dev(enc4[0]), dev(enc4[1]), None if bias is None else dev(bias), pool, m, True, e0, e1,
                   r, 10000.0, 5, x_prev=dev(enc4[2]), gate_prev=dev(enc4[3]))
    got = host(pool)
    x64, g64, xp64, gp64 = (W.to_f64(a) for a in enc4)
    ref = oracle.csa_compress(x64, g64, None if bias is None else bias.astype(np.float64), m, True, r,
                              10000.0, 5, e0, e1, x_prev=xp64, gate_prev=gp64)
    assert np.all(got[:, :e0] == 7.0) and np.all(got[:, e1:] == 7.0), "rows outside the range"
    assert_close(got[:, e0:e1], ref, dt, "pool (split halves)")
    if dt == "bf16":
        assert_bf16_ulp(got[:, e0:e1], ref, "pool (split halves)")


def test_cache_update_split_halves_decode():
    """Token-by-token decode of the R4b compressor: rings of both projections, an entry
    closed every m tokens, sequences of different lengths (a finished sequence gets length 0
    and is left alone), against the oracle's pool of each whole history."""
    B, C, m, r = 3, 128, 4, 16
    S_b = [23, 30, 9]
    S = max(S_b)
    x, g = normal("x", (B, S, C)), normal("g", (B, S, C))
    xp, gp = normal("xp", (B, S, C)), normal("gp", (B, S, C))
    bias = normal("bias", (2 * m, C)).astype(np.float32)
    e = [enc(a, "bf16") for a in (x, g, xp, gp)]
    N_cap = S // m
    rings = [torch.zeros(B, 2 * m, C, dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    pool = torch.zeros(B, N_cap, C, dtype=torch.bfloat16, device="cuda")
    for t in range(S):
        lens = np.array([t + 1 if t < S_b[b] else 0 for b in range(B)], dtype=np.int32)
        tok = [np.ascontiguousarray(a[:, t]) for a in e]
        L.compressor_cache_update(dev(tok[0]), dev(tok[1]), rings[0], rings[1], dev(bias), pool,
                                  i32(lens), m, True, r, 10000.0, 0, emit=True,
                                  x_prev_new=dev(tok[2]), gate_prev_new=dev(tok[3]),
                                  x_prev_ring=rings[2], gate_prev_ring=rings[3])
    torch.cuda.synchronize()
    got = host(pool)
    for b in range(B):
        n = S_b[b] // m
        x64, g64, xp64, gp64 = (W.to_f64(a[b:b + 1, :S_b[b]]) for a in e)
        ref = oracle.csa_compress(x64, g64, bias.astype(np.float64), m, True, r, 10000.0, 0,
                                  x_prev=xp64, gate_prev=gp64)[0]
        assert_bf16_ulp(got[b, :n], ref, f"pool from decode (split halves), sequence {b}")
        assert np.all(got[b, n:] == 0.0), "entries beyond the sequence's closed windows"


def test_cache_update_pair_matches_two_calls_and_oracle():
    """The K=V and indexer-key compressors of a CSA layer updated by one launch
    (compressor_cache_update_pair): token by token, sequences of different lengths, entries
    closed every m tokens.  Each pool equals the one two separate calls build (bit for bit) and
    the oracle's pool of the whole history (one bf16 ulp)."""
    B, C1, C2, m, r = 3, 512, 128, 4, 64
    S_b = [21, 30, 8]
    S = max(S_b)
    print(f"cache update pair B={B} C={C1},{C2} m={m} S={S_b}", flush=True)
    xs = [normal(n, (B, S, c)) for n, c in (("x1", C1), ("g1", C1), ("x2", C2), ("g2", C2))]
    b1, b2 = (normal(n, (2 * m, c)).astype(np.float32) for n, c in (("b1", C1), ("b2", C2)))
    e = [enc(a, "bf16") for a in xs]
    N_cap = S // m

    def state():
        rings = [torch.zeros(B, 2 * m, c, dtype=torch.bfloat16, device="cuda") for c in (C1, C1, C2, C2)]
        pools = [torch.zeros(B, N_cap, c, dtype=torch.bfloat16, device="cuda") for c in (C1, C2)]
        return rings, pools

    (ra, pa), (rb, pb) = state(), state()
    for t in range(S):
        lens = i32([t + 1 if t < S_b[b] else 0 for b in range(B)])
        tok = [dev(np.ascontiguousarray(a[:, t])) for a in e]
        L.compressor_cache_update_pair(
            {"x_new": tok[0], "gate_new": tok[1], "x_ring": ra[0], "gate_ring": ra[1], "bias": dev(b1),
             "pool": pa[0], "rope_dim": r},
            {"x_new": tok[2], "gate_new": tok[3], "x_ring": ra[2], "gate_ring": ra[3], "bias": dev(b2),
             "pool": pa[1], "rope_dim": 0},
            lens, m, True, 10000.0)
        L.compressor_cache_update(tok[0], tok[1], rb[0], rb[1], dev(b1), pb[0], lens, m, True, r, 10000.0)
        L.compressor_cache_update(tok[2], tok[3], rb[2], rb[3], dev(b2), pb[1], lens, m, True, 0)
    torch.cuda.synchronize()
    for i, (bias, rd) in enumerate(((b1, r), (b2, 0))):
        got, two = host(pa[i]), host(pb[i])
        assert np.array_equal(got, two), f"compressor {i}: one launch differs from two calls"
        for b in range(B):
            n = S_b[b] // m
            x64, g64 = (W.to_f64(a[b:b + 1, :S_b[b]]) for a in e[2 * i:2 * i + 2])
            ref = oracle.csa_compress(x64, g64, bias.astype(np.float64), m, True, rd, 10000.0, 0)[0]
            assert_bf16_ulp(got[b, :n], ref, f"compressor {i}, sequence {b}")


# ---------------------------------------------------------------------------- swa_concat

@pytest.mark.parametrize("dt,D,r", [("fp32", 64, 16), ("bf16", 512, 64), ("bf16", 512, 0)])
def test_swa_concat(dt, D, r):
    B, S_new, S_cap = 2, 300, 400
    kv = normal("kv", (B, S_new, D))
    kvs = enc(kv, dt)
    kv_pos0, new_pos0, off = [0, 50], [0, 60], 12345
    win = torch.full((B, S_cap, D), 3.0, dtype=torch_dtype(dt), device="cuda")
    L.swa_concat(dev(kvs), win, i32(kv_pos0), i32(new_pos0), r, 10000.0, off)
    got = host(win)
    ref = oracle.swa_concat(W.to_f64(kvs), new_pos0, r, 10000.0, off)
    for b in range(B):
        r0 = new_pos0[b] - kv_pos0[b]
        assert np.all(got[b, :r0] == 3.0) and np.all(got[b, r0 + S_new:] == 3.0)
        assert_close(got[b, r0:r0 + S_new], ref[b], dt, f"window b={b}")
        if dt == "bf16":
            assert_bf16_ulp(got[b, r0:r0 + S_new], ref[b], "window")


def test_swa_concat_in_place_and_clipped():
    B, S, D, r = 1, 64, 512, 64
    kvs = enc(normal("kv", (B, S, D)), "bf16")
    t = dev(kvs)
    L.swa_concat(t, t, i32([0]), i32([0]), r, 10000.0, 0)  # in place
    assert_close(host(t), oracle.swa_concat(W.to_f64(kvs), [0], r, 10000.0), "bf16", "in place")
    # rows landing outside [0, S_cap) are skipped
    win = torch.zeros(B, 16, D, dtype=torch.bfloat16, device="cuda")
    L.swa_concat(dev(kvs), win, i32([40]), i32([30]), r, 10000.0, 0)
    ref = oracle.swa_concat(W.to_f64(kvs), [30], r, 10000.0)
    assert_close(host(win)[0], ref[0, 10:26], "bf16", "clipped rows")


# ---------------------------------------------------------------------------- index + top-k

def _topk_case(dt, B, T, nI, cI, N_cap, k, m, q_pos0, n_pool, seed, ties=False,
               few_rows=()):
    q = normal("q_idx", (B, T, nI, cI), seed)
    w = normal("w_idx", (B, T, nI), seed).astype(np.float32)
    kp = normal("k_pool", (B, N_cap, cI), seed)
    for b in few_rows:
        # every key row is one of 6 distinct rows: only 6 distinct scores per query, so the
        # k-th slot sits inside a block of thousands of exact ties (lowest indices must win)
        pick = np.random.default_rng(seed + b).integers(0, 6, N_cap)
        kp[b] = kp[b, :6][pick]
    if ties:
        # positive queries and weights; entries >= 10 are all -1, so their score is exactly 0:
        # the k-th slot falls inside a block of exact zero ties (lowest indices must win);
        # entry 5 duplicates entry 3 (an exact tie among positive scores)
        q, w = np.abs(q), np.abs(w)
        kp[:, 10:] = -1.0
        kp[:, 5] = kp[:, 3]
    qs, ks = enc(q, dt), enc(kp, dt)
    k_eff = k
    idx = torch.empty(B, T, k_eff, dtype=torch.int32, device="cuda")
    sc = torch.empty(B, T, k_eff, dtype=torch.float32, device="cuda")
    ws = torch.empty(L.csa_index_topk_workspace_size(B, T, N_cap, k_eff), dtype=torch.uint8,
                     device="cuda")
    L.csa_index_topk(dev(qs), dev(w), dev(ks), i32(q_pos0), i32(n_pool), idx, sc, m, ws)
    gi, gs = idx.cpu().numpy(), sc.cpu().numpy()
    q64, k64 = W.to_f64(qs), W.to_f64(ks)
    swaps = 0
    for b in range(B):
        for t in range(T):
            V = oracle.n_visible(q_pos0[b] + t, m, min(n_pool[b], N_cap))
            s = oracle.index_scores(q64[b, t], w[b, t], k64[b, :V])
            swaps += check_topk_row(gi[b, t], s, k_eff, f"b={b} t={t}")
            valid = gi[b, t] >= 0
            if valid.any():
                ref = s[gi[b, t][valid]]
                assert np.allclose(gs[b, t][valid], ref, rtol=1e-4, atol=1e-4 * np.abs(s).max())
            assert np.all(gs[b, t][~valid] == 0.0)
    return swaps


def test_index_topk_tiny_fp32():
    w = W.workload(1)
    _topk_case("fp32", 1, w.S, w.nI, w.cI, w.S // w.m, w.k, w.m, [0], [w.S // w.m], 5)


def test_index_topk_prefill_bf16_mfma():
    # 64 heads x 128 (MFMA path), T not a multiple of the 8-query block, k > some V(t)
    _topk_case("bf16", 1, 1003, 64, 128, 250, 100, 4, [0], [250], 6)


def test_index_topk_prefill_offset_batches():
    # two sequences with different start positions and pool fill levels
    _topk_case("bf16", 2, 72, 64, 128, 700, 64, 4, [2000, 5], [650, 700], 7)


def test_index_topk_decode_split():
    # T = 1 per sequence: the split-N decode path; n_pool caps visibility
    _topk_case("bf16", 3, 1, 64, 128, 2300, 512, 4, [4000, 9000, 200], [1000, 2250, 50], 8)


def test_index_topk_decode_long_rows():
    # V = 40000 and 33001: more keys than the top-k kernel keeps in registers and more than
    # one compaction segment; sequence 1 has only 6 distinct scores (exact ties everywhere)
    _topk_case("bf16", 2, 1, 64, 128, 40000, 512, 4, [159999, 132003], [40000, 40000], 11,
               few_rows=(1,))


def test_index_topk_long_rows_ragged_visibility():
    # few long rows (the block-per-row top-k): a row with fewer visible entries than k (300),
    # one with 5100 and a full row (20000) of a 20000-entry pool
    _topk_case("bf16", 3, 1, 64, 128, 20000, 512, 4, [1199, 20399, 79999], [20000, 20000, 20000], 13)


def test_index_topk_long_rows_other_scorers():
    # few long rows (the block-per-row selection) scored by the other two scoring kernels:
    # fp32 on the generic scorer (row 1 has 250 visible entries), and T = 16 on the MFMA
    # scorer with exact ties at the k-th slot
    _topk_case("fp32", 2, 1, 4, 32, 9000, 64, 4, [35999, 1000], [9000, 9000], 15)
    _topk_case("bf16", 1, 16, 64, 128, 12000, 512, 4, [47980], [12000], 16, few_rows=(0,))


def test_index_topk_prefill_rows_4k_to_8k():
    # many rows of 4097..8192 visible entries (the block-per-row selection with every key in
    # registers): a near-full 8192-entry pool, and a second sequence whose rows hold ~4250
    # entries with only 6 distinct scores (thousands of exact ties at the k-th slot)
    _topk_case("bf16", 2, 40, 64, 128, 8192, 512, 4, [32700, 17000], [8192, 6000], 14,
               few_rows=(1,))


def test_index_topk_small_T_stream_path():
    # T = 3 queries per sequence on the streaming scorer (T < 8), ragged entry counts
    _topk_case("bf16", 2, 3, 64, 128, 3000, 300, 4, [7001, 4096], [1800, 3000], 12)


def test_index_topk_many_rows_past_registers():
    # 2048 rows of ~5000-5500 entries on a 9000-entry pool: the one-wave-per-row selection,
    # whose key strides past the 64 it holds in registers are re-read from the score row on
    # every pass (the fp32 generic scorer keeps the oracle cheap); then the same rows with only
    # 6 distinct scores, so that the k-th slot lies inside thousands of exact ties
    _topk_case("fp32", 1, 2048, 4, 32, 9000, 64, 4, [20000], [9000], 17)
    _topk_case("fp32", 1, 2048, 4, 32, 9000, 64, 4, [20000], [9000], 18, few_rows=(0,))


def test_index_topk_exact_ties():
    _topk_case("bf16", 1, 40, 64, 128, 60, 16, 4, [300], [60], 9, ties=True)
    _topk_case("fp32", 1, 40, 4, 32, 60, 16, 4, [300], [60], 10, ties=True)


# ---------------------------------------------------------------------------- attention

def _attend_case(dt, csa, B, T, H, D, r, Wn, S_kv, kv_pos0, q_pos0, N_cap, k=0, n_pool=None,
                 m_hca=16, seed=20, shuffle_invalid=False, split=False, full_lists=False):
    q = normal("q", (B, T, H, D), seed)
    win = normal("win", (B, S_kv, D), seed)
    pool = normal("pool", (B, max(N_cap, 1), D), seed)[:, :N_cap]
    sink = normal("sink", (H,), seed).astype(np.float32)
    if csa:
        topk = W.random_index_lists(seed, "topk", B, T, k, N_cap, shuffle_invalid, full_lists)
        if full_lists and k % 4:
            # the entries of the slots past the last multiple of 4 get large rows, so that
            # attending any other entry in their place moves the output far
            for b in range(B):
                tail = topk[b, :, k & ~3:k]
                pool[b, np.unique(tail[tail >= 0])] *= 3.0
    qs, ws_, ps = enc(q, dt), enc(win, dt), enc(pool, dt)
    base, off = 10000.0, 11
    out = torch.empty(B, T, H, D, dtype=torch_dtype(dt), device="cuda")
    pool_t = dev(ps) if N_cap > 0 else None
    wsp = None
    if split:  # key ranges of each query on separate workgroups, merged afterwards
        nb = L.attend_workspace_size(B, T, H, D)
        assert nb > 0, "the split path should apply to this few queries"
        wsp = torch.empty(nb, dtype=torch.uint8, device="cuda")
    if csa:
        L.csa_attend(dev(qs), dev(ws_), i32(kv_pos0), pool_t, dev(topk), dev(sink), i32(q_pos0),
                     out, Wn, r, base, off, workspace=wsp)
        ref = oracle.csa_attend(W.to_f64(qs), W.to_f64(ws_), kv_pos0, W.to_f64(ps), topk, sink,
                                q_pos0, Wn, r, base, off)
    else:
        L.hca_attend(dev(qs), dev(ws_), i32(kv_pos0), pool_t,
                     i32(n_pool) if n_pool is not None else None, m_hca, dev(sink), i32(q_pos0),
                     out, Wn, r, base, off, workspace=wsp)
        ref = oracle.hca_attend(W.to_f64(qs), W.to_f64(ws_), kv_pos0,
                                W.to_f64(ps) if N_cap > 0 else None,
                                n_pool if n_pool is not None else ([N_cap] * B if N_cap else None),
                                m_hca, sink, q_pos0, Wn, r, base, off)
    return assert_close(host(out), ref, dt, "attention output")


def test_csa_attend_mfma():
    # 64 x 512 MFMA path; window + up to 96 selected keys (ragged tile counts), two sequences
    _attend_case("bf16", True, 2, 37, 64, 512, 64, 128, 300, [0, 40], [150, 100], 300, k=96)


def test_csa_attend_mfma_unordered_sentinels():
    # -1 slots anywhere in the list are masked, valid slots anywhere are used
    _attend_case("bf16", True, 1, 20, 64, 512, 64, 128, 200, [0], [180], 200, k=64, seed=21,
                 shuffle_invalid=True)


def test_csa_attend_generic_fp32():
    _attend_case("fp32", True, 2, 30, 8, 64, 16, 32, 100, [0, 5], [60, 40], 64, k=16, seed=22)


def test_hca_attend_mfma():
    _attend_case("bf16", False, 2, 33, 64, 512, 64, 128, 400, [0, 0], [300, 7], 40,
                 n_pool=[25, 40], m_hca=8, seed=23)


def test_sliding_attend_mfma_window_edges():
    # no pool; queries at the start of the sequence (fewer than W keys) and W > S
    _attend_case("bf16", False, 1, 40, 64, 512, 64, 128, 40, [0], [0], 0, seed=24)
    _attend_case("bf16", False, 1, 40, 64, 512, 64, 1000, 40, [0], [0], 0, seed=25)


def test_attend_rope_zero_and_generic_bf16():
    _attend_case("bf16", False, 1, 16, 64, 512, 0, 128, 60, [0], [40], 10, n_pool=[10], m_hca=4,
                 seed=26)
    _attend_case("bf16", True, 1, 16, 16, 128, 32, 20, 60, [0], [40], 30, k=8, seed=27)


def test_decode_shaped_attend():
    # one query per sequence at the end of its window buffer (decode layout)
    B, Wn = 4, 128
    L_b = [5000, 70000, 129, 20000]
    _attend_case("bf16", True, B, 1, 64, 512, 64, Wn, Wn, [x - Wn for x in L_b],
                 [x - 1 for x in L_b], 500, k=512, seed=28)


def test_decode_shaped_attend_split():
    # the same with each query's keys cut into ranges on separate workgroups and merged
    B, Wn = 4, 128
    L_b = [5000, 70000, 129, 20000]
    _attend_case("bf16", True, B, 1, 64, 512, 64, Wn, Wn, [x - Wn for x in L_b],
                 [x - 1 for x in L_b], 500, k=512, seed=28, split=True)


def test_split_attend_short_and_empty_queries():
    # HCA, one query per sequence: a long one, one with fewer tiles than ranges (empty ranges
    # run a masked tile), one whose window rows all lie outside the buffer and whose pool is
    # empty (the sink alone: output 0)
    _attend_case("bf16", False, 3, 1, 64, 512, 64, 128, 128, [3000, 40, 500], [3127, 60, 300],
                 600, n_pool=[600, 2, 0], m_hca=8, seed=29, split=True)


def test_split_attend_csa_two_queries_per_sequence():
    _attend_case("bf16", True, 3, 2, 64, 512, 64, 128, 256, [0, 100, 7], [200, 300, 40], 300,
                 k=128, seed=30, split=True, shuffle_invalid=True)


@pytest.mark.parametrize("ns", [2, 3, 5, 6, 7])
def test_split_attend_every_range_count(ns):
    # the merge is compiled once per range count (2 .. 8), and the count is the device's
    # compute units over the queries: these query counts give each remaining count once (8 and
    # 4 come from the tests above and the 64-sequence decode)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    B = cus // ns
    if B < 1 or min(8, cus // B) != ns:
        pytest.skip(f"{cus} compute units give no query count with {ns} ranges")
    L_b = [300 + 37 * b for b in range(B)]
    _attend_case("bf16", True, B, 1, 64, 512, 64, 128, 128, [x - 128 for x in L_b],
                 [x - 1 for x in L_b], 200, k=64, seed=40 + ns, split=True)


@pytest.mark.parametrize("k", [510, 6, 509])
@pytest.mark.parametrize("split", [False, True])
def test_csa_attend_list_length_not_multiple_of_4(k, split):
    # full lists whose last slots (k & ~3 .. k - 1) hold valid entries: the list copy into LDS
    # must deliver those slots, not zeros (entry 0) from a load that crosses the list's end
    B, T = (3, 2) if split else (1, 24)
    _attend_case("bf16", True, B, T, 64, 512, 64, 128, 700, [0] * B, [600] * B, 700, k=k,
                 seed=31 + k, split=split, full_lists=True)


# ---------------------------------------------------------------------------- errors

def test_argument_errors_do_not_launch():
    x = torch.zeros(1, 16, 64, dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros(1, 4, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(L.DSV4Error) as e:
        L.csa_compress(x, x, None, pool, 4, True, 0, 5)  # entry 4 needs tokens up to 19
    assert e.value.status == 1
    with pytest.raises(L.DSV4Error) as e:
        L.csa_compress(x, x, None, pool, 4, True, rope_dim=3)
    assert e.value.status == 1
    q = torch.zeros(1, 2, 4, 8, dtype=torch.float32, device="cuda")
    kp = torch.zeros(1, 10, 8, dtype=torch.float32, device="cuda")
    idx = torch.zeros(1, 2, 4, dtype=torch.int32, device="cuda")
    w = torch.zeros(1, 2, 4, dtype=torch.float32, device="cuda")
    z = i32([0])
    small = torch.empty(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(L.DSV4Error) as e:
        L.csa_index_topk(q, w, kp, z, i32([10]), idx, None, 4, small)
    assert e.value.status == 4

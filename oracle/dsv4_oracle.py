"""CPU oracle for the DeepSeek-V4 hybrid attention core (CSA + HCA + sliding window).

TEST INFRASTRUCTURE ONLY.  Plain, slow, fp64 numpy.  Only the test-suite, the smoke
check and the benchmark's CPU-baseline leg may import this module; the product path
(the HIP library and its binding) never does, and this module imports nothing from it.

Source: the Hugging Face Transformers model page "DeepSeek-V4" (all five language
mirrors carry the same text).  Sections cited below are that page's headings:
  "Hybrid attention (§2.3)"      - the three layer types and the shared skeleton
  "Attention mask layout"        - the sliding / CSA / HCA visibility rules
  "Cache layers"                 - compressor + indexer state
  "DeepseekV4Config"             - parameter meanings (index_topk, sliding_window, ...)
The page names eqs. 13-17, 26 and 27 but prints none of them.  Each function states the
reading it computes (R1 ... R24) in its docstring.

Everything is computed in float64 with no intermediate rounding, except where a caller
asks to model a storage rounding explicitly (``round_bf16``), which follows the path's
stated storage types (pool, indexer keys and the rotated window are stored in bf16).

Parity status per function (what pins it, see tests/test_oracle_pins.py):
  rope                     pinned: isometry, composition, identity at 0, closed-form angle
  compress                 pinned: mean pooling, one-hot copy, window geometry, known weights,
                           permutation invariance; the R4b variant: equal to R4 when both
                           projections agree, half locality, one-hot copy from each half.  Exact gate/bias form (R1) is a reading:
                           the page prints no compressor formula, so its constants are
                           parity unpinned by the page itself.
  index_scores             pinned: single-head closed form, head additivity, ReLU cut-off.
                           The ReLU/weight form (R8) is a reading: parity unpinned by the
                           page's printed values (it prints none).
  topk_select              pinned: brute force over a full stable sort, worked example
  visibility               pinned: the page's 16-token worked example
  csa_index_topk           pinned: queries starting at q_pos0 > 0 and an n_pool below the
                           visible count against explicit score loops and a stable sort
  swa_concat               pinned: rows at new_pos0 + i against the closed-form rotation
  csa_attend / hca_attend  pinned: window buffers whose row 0 is kv_pos0 (at 0, inside the
                           window, past the query) or that end early, queries at q_pos0 > 0,
                           and HCA pools capped by n_pool, all against fp64 SDPA with the
                           explicit mask; the decode layout (one query at L-1, a buffer of the
                           last W positions, a pool with unused rows) and chunked prefill
                           (entry ranges, halo buffers, a growing pool) equal the one-shot layer
  attend_query             pinned: torch SDPA (fp64) with explicit K=V and sink column,
                           sink closed forms, eq. 26 shift invariance
  grouped_out_proj         pinned: brute-force loops on tiny shapes, group locality (a group's
                           heads reach only its rank slice), identity weights.  The grouping
                           of consecutive heads and the linear-layer weight layout are
                           readings (R22); the page prints no values for them.
  input_projections        pinned: brute-force loops on tiny shapes, one-hot rows pick each
                           weight's column (which output reads which weight), the merged
                           query weight (W_qb W_qa) closed form, token locality.  Which
                           input feeds each projection and the absence of a norm are readings
                           (R23/R24); the page prints no values for them.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

# ----------------------------------------------------------------------------
# storage rounding (used only when a caller models bf16 storage of intermediates)
# ----------------------------------------------------------------------------


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even), returned as fp64.

    bf16 keeps 8 significant bits.  Written from the definition: scale each value by a power
    of two so that its significand is an integer of at most 8 bits, round half-to-even,
    scale back.  Subnormals of bf16 share float32's exponent range and do not occur here.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    m, e = np.frexp(x[nz])  # x = m * 2**e, 0.5 <= |m| < 1
    scaled = np.ldexp(m, 8)  # 8 significant bits -> integer part
    out[nz] = np.ldexp(np.round(scaled), e - 8)  # np.round: half to even
    out[~nz] = x[~nz]
    return out


# ----------------------------------------------------------------------------
# R10: partial RoPE on interleaved pairs of the trailing rope_dim channels
# ----------------------------------------------------------------------------


def rope(x: np.ndarray, pos, rope_dim: int, base: float) -> np.ndarray:
    """Rotate the trailing ``rope_dim`` channels of x in interleaved pairs.

    "Hybrid attention (§2.3)", partial RoPE bullet: the rotation acts on the last
    qk_rope_head_dim channels of each head, pairs interleaved.  Reading R10: pair i is
    channels (C-r+2i, C-r+2i+1), frequency theta_i = base**(-2i/r), angle pos*theta_i,
    (a, b) -> (a cos - b sin, a sin + b cos).  ``pos`` broadcasts against x[..., 0].
    """
    x = np.array(x, dtype=np.float64, copy=True)
    r = int(rope_dim)
    if r == 0:
        return x
    C = x.shape[-1]
    assert r % 2 == 0 and r <= C
    i = np.arange(r // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / r)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    a = x[..., C - r::2].copy()
    b = x[..., C - r + 1::2].copy()
    x[..., C - r::2] = a * c - b * s
    x[..., C - r + 1::2] = a * s + b * c
    return x


# ----------------------------------------------------------------------------
# R1-R6: the KV compressor
# ----------------------------------------------------------------------------


def compress(x: np.ndarray, gate: np.ndarray, bias: Optional[np.ndarray], m: int, overlap: bool,
             rope_dim: int = 0, base: float = 10000.0, pos_offset: int = 0,
             entry_begin: int = 0, entry_end: Optional[int] = None,
             x_prev: Optional[np.ndarray] = None, gate_prev: Optional[np.ndarray] = None) -> np.ndarray:
    """Pool tokens [S, C] into compressed entries [N, C], N = S // m.

    "Hybrid attention (§2.3)": CSA pools at rate m with overlapping windows, HCA at rate m'
    with non-overlapping windows; "Attention mask layout", HCA paragraph: entry w covers
    positions w*m .. (w+1)*m-1 and closes at (w+1)*m-1.
    Readings:
      R1 per-channel softmax-gated pooling: for channel c the slot weights are
         softmax over the window's tokens of gate[j, c] + bias[slot(j), c], and the entry is
         the weighted sum of x[j, c].  bias None means zero.
      R2 CSA window of entry w: tokens [(w-1)m, (w+1)m) (2m slots, overlapping by m);
         slots before token 0 do not exist and are left out of the softmax.
         HCA window: tokens [w m, (w+1) m) (m slots).
      R3 a trailing partial window (S mod m tokens) emits no entry.
      R5 RoPE (rope_dim > 0) after pooling, at position (w+1)m - 1 + pos_offset.
      R4 one token projection (x, gate) serves both halves of a CSA window.  Variant R4b
         ("separate-projection overlap halves"): with x_prev / gate_prev given, the earlier
         half (slots 0..m-1, tokens (w-1)m .. wm-1) takes its values and gates from them and
         the later half from x / gate; one softmax still spans all 2m slots.
    Returns entries [entry_begin, entry_end) as rows of an [entry_end - entry_begin, C] array.
    """
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(gate, dtype=np.float64)
    split = overlap and x_prev is not None
    if split:
        xp = np.asarray(x_prev, dtype=np.float64)
        gp = np.asarray(gate_prev, dtype=np.float64)
    S, C = x.shape
    N = S // m
    entry_end = N if entry_end is None else entry_end
    assert 0 <= entry_begin <= entry_end <= N
    span = 2 * m if overlap else m
    out = np.zeros((entry_end - entry_begin, C))
    for w in range(entry_begin, entry_end):
        lo = (w - 1) * m if overlap else w * m
        js = [j for j in range(lo, lo + span) if 0 <= j < S]
        slots = [j - lo for j in js]
        a = g[js].copy()
        xs = x[js]
        if split:  # the earlier half's slots read the second projection
            early = np.array([s_ < m for s_ in slots])
            a[early] = gp[js][early]
            xs = xs.copy()
            xs[early] = xp[js][early]
        if bias is not None:
            a += np.asarray(bias, dtype=np.float64)[slots]
        a -= a.max(axis=0, keepdims=True)
        e = np.exp(a)
        pi = e / e.sum(axis=0, keepdims=True)
        out[w - entry_begin] = (pi * xs).sum(axis=0)
    if rope_dim:
        pos = (np.arange(entry_begin, entry_end) + 1) * m - 1 + pos_offset
        out = rope(out, pos, rope_dim, base)
    return out


# ----------------------------------------------------------------------------
# R7: visibility of compressed entries
# ----------------------------------------------------------------------------


def n_visible(t: int, m: int, n_pool: Optional[int] = None) -> int:
    """Number of compressed entries visible to the query at sequence index t.

    "Attention mask layout", HCA paragraph: entry w is visible once its window closed,
    i.e. w < (t+1)//m; CSA paragraph: a query before the first window closes (t < m-1)
    gets nothing.  Reading R7 uses the same rule for both layer types, capped by the number
    of entries that exist.
    """
    v = (t + 1) // m
    if n_pool is not None:
        v = min(v, n_pool)
    return max(v, 0)


def window_rows(t: int, window: int) -> range:
    """Sequence indices of the sliding-window keys of query t (reading R11: W keys incl. self).

    "Attention mask layout", sliding paragraph: causal, with the lower-left triangle cut once
    t >= window.
    """
    return range(max(0, t - window + 1), t + 1)


# ----------------------------------------------------------------------------
# R8-R9: Lightning Indexer scores and top-k
# ----------------------------------------------------------------------------


def index_scores(q_idx_t: np.ndarray, w_idx_t: np.ndarray, k_pool: np.ndarray) -> np.ndarray:
    """Indexer score of one query against entries k_pool [V, cI]  ->  [V].

    "Hybrid attention (§2.3)", CSA item and "DeepseekV4Config" index_n_heads / index_head_dim:
    n_h^I indexer heads of width c^I score each query against the pooled entries.  Reading
    R8 (the page names eqs. 13-16 without printing them): score[w] =
    sum_h w_idx[h] * max(0, q_idx[h] . k_pool[w]), no scale, no rotation.
    """
    q = np.asarray(q_idx_t, dtype=np.float64)  # [nI, cI]
    wv = np.asarray(w_idx_t, dtype=np.float64)  # [nI]
    K = np.asarray(k_pool, dtype=np.float64)  # [V, cI]
    if K.shape[0] == 0:
        return np.zeros(0)
    dots = q @ K.T  # [nI, V]
    return (wv[:, None] * np.maximum(dots, 0.0)).sum(axis=0)


def topk_select(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the min(k, V) largest scores, then -1 padding  ->  int64 [k].

    "Attention mask layout", CSA paragraph: the indexer fills k slots per query and marks
    empty slots with the sentinel -1.  Reading R9: exact ties go to the lower entry index,
    -0.0 counts as +0.0; valid indices come first (here ascending), then -1.
    """
    s = np.asarray(scores, dtype=np.float64) + 0.0  # -0.0 + 0.0 == +0.0
    V = s.shape[0]
    order = sorted(range(V), key=lambda w: (-s[w], w))
    sel = sorted(order[:min(k, V)])
    out = np.full(k, -1, dtype=np.int64)
    out[:len(sel)] = sel
    return out


# ----------------------------------------------------------------------------
# R11-R16: shared-K=V attention with sink, sliding branch and counter-rotation
# ----------------------------------------------------------------------------


def attend_query(q_t: np.ndarray, keys: np.ndarray, sink: np.ndarray, p_t: float, rope_dim: int,
                 base: float, scale: Optional[float] = None) -> np.ndarray:
    """Output [H, D] of one query over keys [n, D] that are already rotated.

    "Hybrid attention (§2.3)", shared skeleton:
      * one K=V head read as both key and value (R15);
      * partial RoPE on q's trailing channels at its position p_t (R10);
      * a learnable per-head sink (eq. 27), read as an extra logit s_h in the scaled-logit
        space whose value is zero (R13);
      * the output's rope slice rotated at position -p_t (eq. 26, R16).
    Softmax scale 1/sqrt(D) unless given (R12).
    """
    q = np.asarray(q_t, dtype=np.float64)
    K = np.asarray(keys, dtype=np.float64)
    s = np.asarray(sink, dtype=np.float64)
    H, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    qr = rope(q, p_t, rope_dim, base)
    z = (qr @ K.T) * scale  # [H, n]
    M = np.maximum(s, z.max(axis=1) if K.shape[0] else -np.inf)
    e = np.exp(z - M[:, None])
    denom = np.exp(s - M) + e.sum(axis=1)
    o = (e @ K) / denom[:, None]
    return rope(o, -p_t, rope_dim, base)


# ----------------------------------------------------------------------------
# the library's five operations, with the same argument meaning (batch loops)
# ----------------------------------------------------------------------------


def csa_compress(x, gate, bias, m, overlap, rope_dim=0, base=10000.0, pos_offset=0,
                 entry_begin=0, entry_end=None, x_prev=None, gate_prev=None):
    """Batched compress: x, gate [B, S, C] -> pool rows [B, entry_end - entry_begin, C];
    x_prev, gate_prev [B, S, C] select the R4b variant."""
    x = np.asarray(x)
    return np.stack([compress(x[b], gate[b], bias, m, overlap, rope_dim, base, pos_offset,
                              entry_begin, entry_end,
                              None if x_prev is None else x_prev[b],
                              None if gate_prev is None else gate_prev[b])
                     for b in range(x.shape[0])])


def swa_concat(kv_raw, new_pos0, rope_dim, base, pos_offset=0):
    """Rotated window rows: token i of sequence b sits at sequence index new_pos0[b] + i.

    "Hybrid attention (§2.3)", sliding-window branch bullet: the raw K=V of the local window
    (rotated like every key, R10) forms the first block of keys; the compressor's output is
    concatenated after it.  Returns [B, S_new, D].
    """
    kv = np.asarray(kv_raw, dtype=np.float64)
    B, S_new, D = kv.shape
    out = np.empty_like(kv)
    for b in range(B):
        pos = new_pos0[b] + np.arange(S_new) + pos_offset
        out[b] = rope(kv[b], pos, rope_dim, base)
    return out


def csa_index_topk(q_idx, w_idx, k_pool, q_pos0, n_pool, m, k, rows=None):
    """Top-k entry indices [B, T, k] (and their scores, NaN where -1) per query.

    V(t) = min((q_pos0[b] + t + 1) // m, n_pool[b]) entries are candidates (R7).
    ``rows`` optionally restricts to a list of (b, t) pairs (sampled checks); the result is
    then [len(rows), k].
    """
    q_idx = np.asarray(q_idx)
    B, T = q_idx.shape[:2]
    pairs = [(b, t) for b in range(B) for t in range(T)] if rows is None else list(rows)
    idx = np.full((len(pairs), k), -1, dtype=np.int64)
    sc = np.full((len(pairs), k), np.nan)
    for n, (b, t) in enumerate(pairs):
        V = n_visible(int(q_pos0[b]) + t, m, int(n_pool[b]))
        s = index_scores(q_idx[b, t], w_idx[b, t], np.asarray(k_pool)[b, :V])
        sel = topk_select(s, k)
        idx[n] = sel
        valid = sel >= 0
        sc[n, valid] = s[sel[valid]]
    if rows is None:
        return idx.reshape(B, T, k), sc.reshape(B, T, k)
    return idx, sc


def _window_keys(kv_win_b, kv_pos0_b, qpos, window):
    """Window rows of the query at sequence index qpos held by a buffer whose row 0 is
    sequence index kv_pos0_b.  Rows the buffer does not hold are skipped (the library's
    documented boundary rule for a window buffer that starts late or ends early)."""
    lo = max(0, qpos - window + 1)
    r0 = max(lo - kv_pos0_b, 0)
    r1 = min(qpos + 1 - kv_pos0_b, kv_win_b.shape[0])
    return kv_win_b[r0:max(r0, r1)]


def csa_attend(q, kv_win, kv_pos0, pool, topk_idx, sink, q_pos0, window, rope_dim, base,
               pos_offset=0, scale=None, rows=None):
    """CSA core attention: keys = sliding window rows || the pool entries the indexer chose.

    "Attention mask layout", CSA paragraph: query t attends only to the k slots the indexer
    filled for it; -1 slots are masked.  Reading R14: one softmax over the concatenation,
    no de-duplication between a window token and an entry covering it.
    Returns [B, T, H, D] (or [len(rows), H, D] for sampled (b, t) pairs).
    """
    q = np.asarray(q)
    B, T, H, D = q.shape
    pairs = [(b, t) for b in range(B) for t in range(T)] if rows is None else list(rows)
    out = np.empty((len(pairs), H, D))
    for n, (b, t) in enumerate(pairs):
        qpos = int(q_pos0[b]) + t
        wk = _window_keys(np.asarray(kv_win[b], dtype=np.float64), int(kv_pos0[b]), qpos, window)
        sel = np.asarray(topk_idx[b][t])
        sel = sel[sel >= 0]
        ck = np.asarray(pool[b], dtype=np.float64)[sel]
        keys = np.concatenate([wk, ck], axis=0)
        out[n] = attend_query(q[b, t], keys, sink, qpos + pos_offset, rope_dim, base, scale)
    return out.reshape(B, T, H, D) if rows is None else out


def hca_attend(q, kv_win, kv_pos0, pool, n_pool, m_hca, sink, q_pos0, window, rope_dim, base,
               pos_offset=0, scale=None, rows=None):
    """HCA (and sliding, with no pool) core attention: keys = window rows || visible entries.

    "Attention mask layout", HCA paragraph: no indexer; every cached entry is potentially
    visible and entry w is visible once w < (t+1)//m'.  "Hybrid attention (§2.3)": in HCA
    every pool entry contributes.  A sliding-only layer is the same with no pool.
    """
    q = np.asarray(q)
    B, T, H, D = q.shape
    pairs = [(b, t) for b in range(B) for t in range(T)] if rows is None else list(rows)
    out = np.empty((len(pairs), H, D))
    for n, (b, t) in enumerate(pairs):
        qpos = int(q_pos0[b]) + t
        wk = _window_keys(np.asarray(kv_win[b], dtype=np.float64), int(kv_pos0[b]), qpos, window)
        if pool is None:
            ck = np.zeros((0, D))
        else:
            npb = np.asarray(pool).shape[1] if n_pool is None else int(n_pool[b])
            V = n_visible(qpos, m_hca, npb)
            ck = np.asarray(pool[b][:V], dtype=np.float64)
        keys = np.concatenate([wk, ck], axis=0)
        out[n] = attend_query(q[b, t], keys, sink, qpos + pos_offset, rope_dim, base, scale)
    return out.reshape(B, T, H, D) if rows is None else out


# ----------------------------------------------------------------------------
# whole layers, as the three layer types compose the operations
# ----------------------------------------------------------------------------


def csa_layer(inp: dict, cfg, rows=None, round_intermediates: bool = False, pos_offset: int = 0):
    """One CSA prefill layer on fp64 inputs (single sequence block, positions 0..S-1).

    inp: q [B,S,H,D], kv, gate [B,S,D], q_idx [B,S,nI,cI], k_idx, g_idx [B,S,cI],
    w_idx [B,S,nI], bias [2m,D], bias_idx [2m,cI], sink [H].
    ``round_intermediates`` models bf16 storage of the pool, the indexer keys and the
    rotated window (the stored types of the bf16 path).  Returns (out, topk_idx, aux).
    """
    B, S = inp["kv"].shape[:2]
    rnd = round_bf16 if round_intermediates else (lambda a: a)
    pool = rnd(csa_compress(inp["kv"], inp["gate"], inp["bias"], cfg.m, True, cfg.r, cfg.base,
                            pos_offset))
    k_pool = rnd(csa_compress(inp["k_idx"], inp["g_idx"], inp["bias_idx"], cfg.m, True, 0))
    kv_win = rnd(swa_concat(inp["kv"], [0] * B, cfg.r, cfg.base, pos_offset))
    zeros = [0] * B
    npool = [pool.shape[1]] * B
    if rows is None:
        idx, sc = csa_index_topk(inp["q_idx"], inp["w_idx"], k_pool, zeros, npool, cfg.m, cfg.k)
        out = csa_attend(inp["q"], kv_win, zeros, pool, idx, inp["sink"], zeros, cfg.W, cfg.r,
                         cfg.base, pos_offset)
    else:
        idx, sc = csa_index_topk(inp["q_idx"], inp["w_idx"], k_pool, zeros, npool, cfg.m, cfg.k,
                                 rows=rows)
        tk = {}
        for n, (b, t) in enumerate(rows):
            tk.setdefault(b, {})[t] = idx[n]
        out = np.stack([csa_attend(inp["q"], kv_win, zeros, pool, {b: tk[b]}, inp["sink"], zeros,
                                   cfg.W, cfg.r, cfg.base, pos_offset, rows=[(b, t)])[0]
                        for (b, t) in rows])
    return out, idx, dict(pool=pool, k_pool=k_pool, kv_win=kv_win, scores=sc)


def hca_layer(inp: dict, cfg, rows=None, round_intermediates: bool = False, pos_offset: int = 0,
              sliding: bool = False):
    """One HCA (or, with sliding=True, sliding-only) prefill layer.  Returns (out, aux)."""
    B, S = inp["kv"].shape[:2]
    rnd = round_bf16 if round_intermediates else (lambda a: a)
    kv_win = rnd(swa_concat(inp["kv"], [0] * B, cfg.r, cfg.base, pos_offset))
    zeros = [0] * B
    if sliding:
        pool, npool = None, None
    else:
        pool = rnd(csa_compress(inp["kv"], inp["gate"], inp["bias_hca"], cfg.m_hca, False, cfg.r,
                                cfg.base, pos_offset))
        npool = [pool.shape[1]] * B
    out = hca_attend(inp["q"], kv_win, zeros, pool, npool, cfg.m_hca, inp["sink"], zeros, cfg.W,
                     cfg.r, cfg.base, pos_offset, rows=rows)
    return out, dict(pool=pool, kv_win=kv_win)


# ----------------------------------------------------------------------------
# grouped low-rank output projection (the step right after the attention core)
# ----------------------------------------------------------------------------


def grouped_out_proj(attn, w_a, w_b, groups: int, round_intermediate: bool = False):
    """Grouped low-rank output projection.

    "Hybrid attention (§2.3)", grouped output projection item (o_groups head groups ->
    o_lora_rank per group -> hidden_size, a grouped linear o_a_proj then o_b_proj) and
    "DeepseekV4Config" (o_groups, o_lora_rank, hidden_size).  Reading R22: the H heads split
    into `groups` runs of H/groups consecutive heads; group g's head outputs, concatenated
    (H/groups * D values), are multiplied by its own matrix w_a[g] of shape
    [rank, H/groups * D] (a linear layer's [out, in] layout); the groups' rank vectors,
    concatenated in group order, are multiplied by w_b [hidden, groups * rank].  No bias
    (attention_bias is False) and nothing between the two products.
    ``round_intermediate`` models bf16 storage of the [T, groups * rank] intermediate.

    attn [T, H, D] or [T, H * D]; returns (out [T, hidden], intermediate [T, groups * rank]).
    """
    a = np.asarray(attn, dtype=np.float64)
    T = a.shape[0]
    a = a.reshape(T, -1)
    w_a = np.asarray(w_a, dtype=np.float64)
    w_b = np.asarray(w_b, dtype=np.float64)
    assert w_a.shape[0] == groups and a.shape[1] == groups * w_a.shape[2], (a.shape, w_a.shape)
    rank = w_a.shape[1]
    kg = w_a.shape[2]
    mid = np.empty((T, groups * rank))
    for g in range(groups):
        mid[:, g * rank:(g + 1) * rank] = a[:, g * kg:(g + 1) * kg] @ w_a[g].T
    if round_intermediate:
        mid = round_bf16(mid)
    return mid @ w_b.T, mid


# ----------------------------------------------------------------------------
# input projections of one attention layer
# ----------------------------------------------------------------------------

# Which projections a layer of each type has, in the order the outputs are listed.  Those of
# the first group read the hidden state x; those of the second read the query latent c_q.
INPROJ_FROM_X = {
    "sliding": ("q_a", "kv"),
    "hca": ("q_a", "kv", "gate"),
    "csa": ("q_a", "kv", "gate", "k_idx", "g_idx", "w_idx"),
}
INPROJ_FROM_LATENT = {"sliding": ("q",), "hca": ("q",), "csa": ("q", "q_idx")}


def input_projections(x, weights, kind: str, round_latent: bool = False):
    """The projections that produce the attention core's per-token inputs from the layer's
    hidden state.

    "Hybrid attention (§2.3)" (kv_proj makes the single K=V head; CSA's compressor with its
    gate and the Lightning Indexer of eqs. 13-17 with index_n_heads query heads of
    index_head_dim and per-head weights) and "DeepseekV4Config" (q_lora_rank: the query goes
    through a rank-q_lora_rank factorisation; attention_bias False: no bias anywhere).
    Readings R23/R24: every projection is a plain linear map with a linear layer's
    [out, in] weight and nothing between the two query factors (the page names no norm);
    the query latent c_q = x W_qa^T feeds both the attention query q = c_q W_qb^T and the
    indexer query q_idx = c_q W_q_idx^T, while kv, the compressor gate, the indexer key
    content k_idx, its gate g_idx and the indexer head weights w_idx project x directly.
    ``round_latent`` models bf16 storage of c_q before the second factor.

    x [T, hidden]; ``weights`` maps each name of INPROJ_FROM_X[kind] and
    INPROJ_FROM_LATENT[kind] to its [width, in] matrix ("q_a" is [q_rank, hidden]).
    Returns {"c_q": [T, q_rank], name: [T, width] for every other name}.
    """
    x = np.asarray(x, dtype=np.float64)
    W = {k: np.asarray(v, dtype=np.float64) for k, v in weights.items()}
    out = {}
    for name in INPROJ_FROM_X[kind]:
        out["c_q" if name == "q_a" else name] = x @ W[name].T
    lat = round_bf16(out["c_q"]) if round_latent else out["c_q"]
    for name in INPROJ_FROM_LATENT[kind]:
        out[name] = lat @ W[name].T
    return out

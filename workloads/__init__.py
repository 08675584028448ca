"""Seeded synthetic workloads for the DeepSeek-V4 hybrid attention core.

This module is shared by the GPU path's callers (tests, bench) and by the CPU
oracle. It holds no arithmetic of the method itself: it only defines the five
workload shapes and draws seeded, counter-based random tensors for them, then
encodes them in their storage type (bf16 bit patterns or fp32).

Generation recipe
-----------------
* Every tensor is keyed by ``(seed, layer, name)``.  Rows along the leading
  token/entry axis are drawn in blocks of ``ROW_BLOCK`` rows; each block comes
  from its own ``numpy.random.Philox`` stream keyed by
  ``SeedSequence([seed, layer, crc32(name), block])``.  Any block can therefore be
  regenerated on its own, which is what lets a CPU check recompute a few sampled
  query rows of a multi-GB tensor without drawing the rest.
* Values are standard normal, drawn as float32 and rounded to nearest-even
  into the storage type (bf16 for the bf16 workloads).
* The tiny fp32 workload projects a hidden state x ~ N(0,1) of width d = H*D
  through weights W ~ N(0, 1/d) (std 1/sqrt(d)), in fp64, and rounds the
  projections to fp32; this stands in for the model's upstream projections,
  which are not part of the attention core.
"""
from __future__ import annotations

import dataclasses
import os
import zlib
from typing import Dict, Iterable, Optional, Sequence

import numpy as np

ROW_BLOCK = 64

# ----------------------------------------------------------------------------
# storage encodings (not part of the method: input quantisation only)
# ----------------------------------------------------------------------------


def _bf16_rne(u: np.ndarray) -> np.ndarray:
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    rounding = ((u >> 16) & 1) + 0x7FFF
    out = ((u + rounding) >> 16).astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    flat = u.reshape(-1)
    if flat.size < (1 << 24):
        return _bf16_rne(flat).reshape(u.shape)
    out = np.empty(flat.size, dtype=np.uint16)
    step = 1 << 22
    import concurrent.futures as cf

    def conv(i):
        out[i:i + step] = _bf16_rne(flat[i:i + step])

    with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(conv, range(0, flat.size, step)))
    return out.reshape(u.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f64(arr: np.ndarray) -> np.ndarray:
    """Exact fp64 values of a stored tensor (uint16 = bf16 bits, else a float array)."""
    if arr.dtype == np.uint16:
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


# ----------------------------------------------------------------------------
# workload definitions
# ----------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes of one workload.  Symbols follow the model's config fields."""

    ident: int
    name: str
    dtype: str  # "fp32" or "bf16"
    B: int
    S: int  # tokens per sequence (prefill) / allocated pool rows (decode)
    H: int  # num_attention_heads
    D: int  # head_dim
    r: int  # qk_rope_head_dim
    m: int  # CSA compress rate
    m_hca: int  # HCA compress rate
    nI: int  # index_n_heads
    cI: int  # index_head_dim
    k: int  # index_topk
    W: int  # sliding_window
    base: float  # rope base
    seed: int
    kind: str  # "csa", "hca", "decode", "stack"
    layer_types: tuple = ()
    chunk: int = 0  # prefill query chunk (stack workload)
    n_seq: int = 0  # decode: number of sequences
    L_min: int = 0
    L_max: int = 0
    o_groups: int = 8  # grouped output projection: head groups
    o_rank: int = 1024  # o_lora_rank
    hidden: int = 4096  # hidden_size
    q_rank: int = 1024  # q_lora_rank


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "tiny_csa_fp32_S256", "fp32", 1, 256, 8, 64, 16, 4, 128, 4, 32, 16, 32,
                10000.0, 0, "csa", o_groups=4, o_rank=32, hidden=64, q_rank=32),
    2: Workload(2, "csa_prefill_bf16_S8192", "bf16", 1, 8192, 64, 512, 64, 4, 128, 64, 128, 512,
                128, 10000.0, 2, "csa"),
    3: Workload(3, "hca_prefill_bf16_S65536", "bf16", 1, 65536, 64, 512, 64, 4, 128, 64, 128,
                512, 128, 10000.0, 3, "hca"),
    4: Workload(4, "csa_decode_bf16_64seq_16K-128K", "bf16", 64, 32768, 64, 512, 64, 4, 128, 64,
                128, 512, 128, 10000.0, 4, "decode", n_seq=64, L_min=16384, L_max=131072),
    5: Workload(5, "stack8_bf16_S32768", "bf16", 1, 32768, 64, 512, 64, 4, 128, 64, 128, 512,
                128, 10000.0, 5, "stack",
                layer_types=("sliding", "sliding", "csa", "hca", "csa", "hca", "csa", "hca"),
                chunk=4096),
}


def workload(i: int) -> Workload:
    return WORKLOADS[i]


def scaled(w: Workload, **over) -> Workload:
    """A copy of a workload with some fields replaced (smaller test sizes)."""
    return dataclasses.replace(w, **over)


# ----------------------------------------------------------------------------
# keyed block generator
# ----------------------------------------------------------------------------


def _block_gen(seed: int, layer: int, name: str, block: int) -> np.random.Generator:
    ss = np.random.SeedSequence([seed, layer, zlib.crc32(name.encode()), block])
    return np.random.Generator(np.random.Philox(ss))


def normal_rows(seed: int, layer: int, name: str, row_shape: Sequence[int],
                rows: Iterable[int] | slice, n_rows: Optional[int] = None) -> np.ndarray:
    """float32 N(0,1) rows of a keyed tensor [n_rows, *row_shape].

    ``rows`` is a slice (contiguous range) or an iterable of row indices.
    The values of row i do not depend on n_rows or on which other rows are asked for.
    """
    row_shape = tuple(int(v) for v in row_shape)
    per_row = int(np.prod(row_shape)) if row_shape else 1
    if isinstance(rows, slice):
        start, stop, step = rows.indices(n_rows if n_rows is not None else rows.stop)
        assert step == 1
        idx = np.arange(start, stop)
    else:
        idx = np.asarray(list(rows), dtype=np.int64)
    out = np.empty((len(idx), per_row), dtype=np.float32)
    if len(idx) == 0:
        return out.reshape((0,) + row_shape)
    blocks = idx // ROW_BLOCK
    contiguous = bool(np.all(np.diff(idx) == 1))

    def fill(b):
        gen = _block_gen(seed, layer, name, int(b))
        b0 = int(b) * ROW_BLOCK
        if contiguous and idx[0] <= b0 and b0 + ROW_BLOCK <= idx[-1] + 1:
            # whole block lands contiguously in the output: draw in place
            gen.standard_normal(out=out[b0 - idx[0]:b0 - idx[0] + ROW_BLOCK], dtype=np.float32)
            return
        blk = gen.standard_normal(size=(ROW_BLOCK, per_row), dtype=np.float32)
        sel = np.nonzero(blocks == b)[0]
        out[sel] = blk[idx[sel] - b0]

    ub = np.unique(blocks)
    if len(ub) * ROW_BLOCK * per_row >= (1 << 22):  # large draws: blocks in parallel (fills release the GIL)
        import concurrent.futures as cf

        with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, ub))
    else:
        for b in ub:
            fill(b)
    return out.reshape((len(idx),) + row_shape)


def normal_tensor(seed: int, layer: int, name: str, shape: Sequence[int]) -> np.ndarray:
    """Whole keyed tensor, leading axis = rows."""
    return normal_rows(seed, layer, name, shape[1:], slice(0, shape[0]), shape[0])


def encode(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    return np.ascontiguousarray(x32, dtype=np.float32)


# ----------------------------------------------------------------------------
# per-workload tensors
# ----------------------------------------------------------------------------

# Names of the per-token activation tensors of one attention layer and their per-row shapes.
def _row_shapes(w: Workload) -> Dict[str, tuple]:
    return {
        "q": (w.H, w.D),  # query heads, un-rotated
        "kv": (w.D,),  # single shared K=V head, raw (un-rotated)
        "gate": (w.D,),  # compressor gate logits for the K=V pool
        "q_idx": (w.nI, w.cI),  # indexer query heads
        "k_idx": (w.cI,),  # indexer key content
        "g_idx": (w.cI,),  # indexer compressor gate logits
        "w_idx": (w.nI,),  # indexer head weights (fp32)
    }


FP32_ALWAYS = ("w_idx", "bias", "bias_idx", "sink", "bias_hca")


def _projected_rows(w: Workload, layer: int, name: str, rows) -> np.ndarray:
    """Tiny fp32 workload: project hidden x ~ N(0,1) [S, d] with W ~ N(0, 1/d), in fp64."""
    d = w.H * w.D
    shape = _row_shapes(w)[name]
    width = int(np.prod(shape))
    x = normal_rows(w.seed, layer, "hidden", (d,), rows, w.S).astype(np.float64)
    Wm = normal_tensor(w.seed, layer, "W_" + name, (d, width)).astype(np.float64) / np.sqrt(d)
    y = x @ Wm
    return y.astype(np.float32).reshape((len(x),) + shape)


def activation_rows(w: Workload, layer: int, name: str, rows) -> np.ndarray:
    """Storage-encoded rows of a per-token activation tensor (b folded into rows)."""
    shape = _row_shapes(w)[name]
    if w.ident == 1:
        y = _projected_rows(w, layer, name, rows)
    else:
        y = normal_rows(w.seed, layer, name, shape, rows, w.B * w.S)
    if name == "w_idx":
        return np.ascontiguousarray(y, dtype=np.float32)
    return encode(y, w.dtype)


def param(w: Workload, layer: int, name: str) -> np.ndarray:
    """Per-layer parameters (always fp32): compressor slot biases and per-head sinks."""
    if name == "bias":  # CSA K=V compressor bias [2m, D]
        shape = (2 * w.m, w.D)
    elif name == "bias_idx":  # indexer compressor bias [2m, cI]
        shape = (2 * w.m, w.cI)
    elif name == "bias_hca":  # HCA compressor bias [m', D]
        shape = (w.m_hca, w.D)
    elif name == "sink":
        shape = (w.H,)
    else:
        raise KeyError(name)
    return normal_tensor(w.seed, layer, name, shape).astype(np.float32)


def layer_inputs(w: Workload, layer: int = 0, S: Optional[int] = None,
                 names: Optional[Sequence[str]] = None) -> Dict[str, np.ndarray]:
    """All activations [B, S, ...] (storage-encoded) plus fp32 parameters for one layer."""
    S = w.S if S is None else S
    names = list(_row_shapes(w)) if names is None else list(names)
    out: Dict[str, np.ndarray] = {}
    for n in names:
        shape = _row_shapes(w)[n]
        if w.B == 1:
            rows = slice(0, S)
        else:
            rows = np.concatenate([np.arange(b * w.S, b * w.S + S) for b in range(w.B)])
        out[n] = activation_rows(w, layer, n, rows).reshape((w.B, S) + shape)
    for p in ("bias", "bias_idx", "bias_hca", "sink"):
        out[p] = param(w, layer, p)
    return out


# ----------------------------------------------------------------------------
# decode workload: pre-generated caches
# ----------------------------------------------------------------------------


def decode_lengths(w: Workload) -> np.ndarray:
    """Context length per sequence, uniform on [L_min, L_max] (seeded)."""
    g = _block_gen(w.seed, 0, "lengths", 0)
    return g.integers(w.L_min, w.L_max, size=w.n_seq, endpoint=True).astype(np.int64)


def decode_inputs(w: Workload, n_seq: Optional[int] = None, pool_rows: Optional[int] = None,
                  lengths: Optional[np.ndarray] = None, seqs: Optional[Sequence[int]] = None
                  ) -> Dict[str, np.ndarray]:
    """Caches and one new token per sequence (sequence b keyed on its own).

    pool   [B, N_cap, D]  pooled K=V cache (treated as already rotated), first L//m rows valid
    k_pool [B, N_cap, cI] indexer key cache, first L//m rows valid
    window [B, W, D]      sliding K=V cache rows for positions L-W .. L-1 (treated as rotated);
                          the last row is rewritten from kv_new by the window kernel
    kv_new [B, 1, D]      raw K=V of the token at position L-1
    q [B,1,H,D], q_idx [B,1,nI,cI], w_idx [B,1,nI], sink [H]
    Rows of pool / k_pool at or beyond L//m are zero.  ``seqs`` selects a subset of sequences
    (their values do not depend on which others are drawn).
    """
    B_all = w.n_seq if n_seq is None else n_seq
    L_all = decode_lengths(w)[:B_all] if lengths is None else np.asarray(lengths, dtype=np.int64)
    seqs = list(range(B_all)) if seqs is None else list(seqs)
    L = L_all[seqs]
    N_cap = (w.L_max // w.m) if pool_rows is None else pool_rows
    B = len(seqs)
    sdt = np.uint16 if w.dtype == "bf16" else np.float32
    pool = np.zeros((B, N_cap, w.D), dtype=sdt)
    k_pool = np.zeros((B, N_cap, w.cI), dtype=sdt)
    window = np.empty((B, w.W, w.D), dtype=sdt)
    kv_new = np.empty((B, 1, w.D), dtype=sdt)
    q = np.empty((B, 1, w.H, w.D), dtype=sdt)
    q_idx = np.empty((B, 1, w.nI, w.cI), dtype=sdt)
    w_idx = np.empty((B, 1, w.nI), dtype=np.float32)
    for i, b in enumerate(seqs):
        n = min(int(L[i]) // w.m, N_cap)
        tag = "/%d" % b
        pool[i, :n] = encode(normal_rows(w.seed, 0, "pool" + tag, (w.D,), slice(0, n), n), w.dtype)
        k_pool[i, :n] = encode(normal_rows(w.seed, 0, "k_pool" + tag, (w.cI,), slice(0, n), n), w.dtype)
        window[i] = encode(normal_rows(w.seed, 0, "window" + tag, (w.D,), slice(0, w.W), w.W), w.dtype)
        kv_new[i] = encode(normal_rows(w.seed, 0, "kv_new" + tag, (w.D,), slice(0, 1), 1), w.dtype)
        q[i] = encode(normal_rows(w.seed, 0, "q" + tag, (w.H, w.D), slice(0, 1), 1), w.dtype)
        q_idx[i] = encode(normal_rows(w.seed, 0, "q_idx" + tag, (w.nI, w.cI), slice(0, 1), 1), w.dtype)
        w_idx[i] = normal_rows(w.seed, 0, "w_idx" + tag, (w.nI,), slice(0, 1), 1)
    return {"lengths": L, "pool": pool, "k_pool": k_pool, "window": window, "kv_new": kv_new,
            "q": q, "q_idx": q_idx, "w_idx": w_idx, "sink": param(w, 0, "sink")}


def random_index_lists(seed: int, name: str, B: int, T: int, k: int, N: int,
                       shuffle: bool = False, full: bool = False) -> np.ndarray:
    """int32 [B, T, k] lists of distinct entries < N, a random number (0..min(k, N)) per row
    (exactly min(k, N) with full=True), padded with -1 (after the valid entries, or scattered
    among them when shuffle=True).  Synthetic inputs for the attention call, which takes index
    lists as given."""
    gen = _block_gen(seed, 0, name, 0)
    out = np.full((B, T, k), -1, dtype=np.int32)
    for b in range(B):
        for t in range(T):
            n = min(k, N) if full else int(gen.integers(0, min(k, N) + 1))
            out[b, t, :n] = gen.choice(N, size=n, replace=False)
            if shuffle:
                gen.shuffle(out[b, t])
    return out


# ----------------------------------------------------------------------------
# grouped output projection inputs
# ----------------------------------------------------------------------------


def oproj_inputs(w: Workload, T: Optional[int] = None, rows=None, layer: int = 0) -> Dict[str, np.ndarray]:
    """Inputs of the grouped output projection: ``attn`` [T, H, D] standing for the attention
    output, N(0, 1); ``w_a`` [o_groups, o_rank, H/o_groups * D] ~ N(0, 1/fan_in) and ``w_b``
    [hidden, o_groups * o_rank] ~ N(0, 1/fan_in), the fan-in scaling of a linear layer's
    initialisation (no trained weights exist here).  ``rows`` selects token rows of attn (their
    values do not depend on which others are drawn)."""
    T = w.S * w.B if T is None else T
    kg = w.H // w.o_groups * w.D
    rsel = slice(0, T) if rows is None else rows
    attn = normal_rows(w.seed, layer, "o_attn", (w.H, w.D), rsel, T)
    wa = normal_tensor(w.seed, layer, "w_oa", (w.o_groups * w.o_rank, kg)) / np.sqrt(kg)
    wb = normal_tensor(w.seed, layer, "w_ob", (w.hidden, w.o_groups * w.o_rank)) / np.sqrt(w.o_groups * w.o_rank)
    return {"attn": encode(attn, w.dtype),
            "w_a": encode(wa.astype(np.float32).reshape(w.o_groups, w.o_rank, kg), w.dtype),
            "w_b": encode(wb.astype(np.float32), w.dtype)}


# Projections of one attention layer, by the input they read, in the order the library stacks
# their weights (rows of w_x, then rows of w_lat).
INPROJ_X_ORDER = {"sliding": ("q_a", "kv"), "hca": ("q_a", "kv", "gate"),
                  "csa": ("q_a", "kv", "gate", "k_idx", "g_idx", "w_idx")}
INPROJ_LAT_ORDER = {"sliding": ("q",), "hca": ("q",), "csa": ("q", "q_idx")}


def inproj_widths(w: Workload) -> Dict[str, int]:
    return {"q_a": w.q_rank, "kv": w.D, "gate": w.D, "k_idx": w.cI, "g_idx": w.cI, "w_idx": w.nI,
            "q": w.H * w.D, "q_idx": w.nI * w.cI}


def inproj_inputs(w: Workload, kind: str, T: Optional[int] = None, rows=None,
                  layer: int = 0) -> Dict[str, np.ndarray]:
    """Inputs of a layer's input projections: ``x`` [T, hidden] ~ N(0, 1) standing for the
    layer's hidden state, and one [width, in] weight per projection ~ N(0, 1/in) (fan-in
    scaling; no trained weights exist here), ``in`` = hidden for those reading x and q_rank for
    those reading the query latent.  Also ``w_x`` / ``w_lat``: the same weights stacked
    row-wise in the library's order.  Storage-encoded in the workload's dtype."""
    T = w.S * w.B if T is None else T
    rsel = slice(0, T) if rows is None else rows
    wd = inproj_widths(w)
    out = {"x": encode(normal_rows(w.seed, layer, "inproj_x", (w.hidden,), rsel, T), w.dtype)}
    for name in INPROJ_X_ORDER[kind] + INPROJ_LAT_ORDER[kind]:
        fan_in = w.q_rank if name in INPROJ_LAT_ORDER["csa"] else w.hidden
        wt = normal_tensor(w.seed, layer, "W_in_" + name, (wd[name], fan_in)) / np.sqrt(fan_in)
        out[name] = encode(wt.astype(np.float32), w.dtype)
    out["w_x"] = np.ascontiguousarray(np.concatenate([out[n] for n in INPROJ_X_ORDER[kind]], axis=0))
    out["w_lat"] = np.ascontiguousarray(np.concatenate([out[n] for n in INPROJ_LAT_ORDER[kind]], axis=0))
    return out

#!/usr/bin/env python3
"""Benchmark of the hybrid attention core on one MI355X.

Headline (one JSON line): CSA prefill query-tokens/s on the S=8192 workload (64 heads x 512,
rope 64, m=4, 64 x 128 indexer, top-512, window 128, bf16).  One step = the whole CSA hot
path over one batch: csa_compress (K=V pool) + csa_compress (indexer keys) + csa_index_topk +
swa_concat + csa_attend, inputs resident in HBM.  `value` = S / (wall time of K back-to-back
steps / K).

Also reported in the same line ("workloads"): HCA prefill query-tokens/s at S=65536, CSA
decode us/step for 64 sequences of 16K-128K context (pre-generated caches, and the same shape
decoded through the per-layer cache), the mixed eight-layer stack (sliding, sliding, CSA, HCA,
CSA, HCA, CSA, HCA) at S=32768 prefilled in 4096-query chunks, and the projections around the
core.

Kernel timing protocol: every launch is bracketed by HIP events on the stream it is enqueued
on (torch's current stream, which every library call uses); at least 10 launches per kernel
after 3 warm-ups; median, minimum and mean are reported and fractions use the median.  Before
each timed launch of a kernel whose working set is below 512 MB the 256 MB Infinity Cache and
the L2s are flushed by reading a 1 GiB buffer (outside the events), so such kernels read HBM,
not a warm cache.  Decode steps are timed the same way, one step per event pair, flushed.

"roofline" is for the dominant kernel (csa_attend): algorithmic flops per launch over the
launch's mean duration (plus median and min), and the rocprofv3 average of the same source
when profiles/ holds one.  "cpu_baseline" is the fp64 CPU oracle, single-threaded (BLAS
limited to one thread), on bounded samples of configs 1-4.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu] [--copy-calib MiB]
                [--only WORKLOAD]

--copy-calib launches one plain device-to-device copy of that many MiB before the timed work,
so that a counter run (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE) sees a kernel of known traffic
to scale the other kernels' counters by.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15  # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12   # MI355X HBM3E, B/s
FLUSH_BYTES = 1 << 30
CACHE_LIMIT = 512 << 20  # working sets below this are timed after a cache flush
KERNEL_REPS = 10


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- work counts

def csa_keys_per_query(S, W_, m, k, q0=0):
    t = np.arange(q0, q0 + S, dtype=np.int64)
    win = np.minimum(t + 1, W_)
    sel = np.minimum(k, (t + 1) // m)
    return win, sel


def attend_flops(n_keys_total, H, D):
    return 4.0 * H * D * float(n_keys_total)  # QK^T and PV, 2 flops per MAC each


def index_flops(S, m, nI, cI, q0=0):
    t = np.arange(q0, q0 + S, dtype=np.int64)
    return 2.0 * nI * cI * float(((t + 1) // m).sum())


def compress_bytes(S, C, m, overlap, N, elt=2):
    """Read x and gate once, the slot biases once, write the pool once."""
    span = 2 * m if overlap else m
    return 2 * S * C * elt + span * C * 4 + N * C * elt


def kernel_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "long_context_sparse_09_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_profile(kernel: str, src_hash: str):
    """Measured figures per launch from profiles/traffic.json (rocprofv3 kernel trace and
    FETCH_SIZE / WRITE_SIZE counters), if they were taken on this source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return {}
    try:
        d = json.load(open(p)).get(kernel)
    except (ValueError, OSError):
        return {}
    if not d or d.get("source_hash") != src_hash:
        return {}
    return d


# ----------------------------------------------------------------------------- timing helpers

class Clock:
    """HIP events around single launches on torch's current stream (the stream every library
    call is enqueued on), with an optional cache flush before each timed launch."""

    def __init__(self, torch):
        self.torch = torch
        self.flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()

    def flush(self):
        # 1 GiB of reads evicts the Infinity Cache and the L2s with clean lines (a write would
        # leave dirty lines whose write-back overlaps the timed launch)
        self.flush_buf.sum()

    def launches(self, fn, reps=KERNEL_REPS, warm=3, flush=True):
        """Durations (ms) of `reps` launches of fn, each between two events."""
        torch = self.torch
        for _ in range(warm):
            fn()
        pairs = []
        for _ in range(reps):
            if flush:
                self.flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in pairs]


def stats(ms_list, flushed):
    a = np.asarray(ms_list, dtype=np.float64)
    return {"ms": float(np.median(a)), "ms_min": float(a.min()), "ms_mean": float(a.mean()),
            "reps": int(a.size), "cache": "flushed" if flushed else "not flushed (working set >= 512 MB)"}


def kernel_entry(st, bound, alg_flops=None, alg_bytes=None, **extra):
    """Per-kernel record: durations plus achieved rate and fraction of the bounding peak (from
    the median), and the other fraction where both matter."""
    e = dict(st)
    e["bound"] = bound
    if alg_flops is not None:
        e["alg_flops"] = alg_flops
        e["TFLOP/s"] = alg_flops / st["ms"] / 1e9
        e["mfma_frac"] = alg_flops / st["ms"] / 1e-3 / PEAK_BF16
    if alg_bytes is not None:
        e["alg_bytes"] = alg_bytes
        e["GB/s"] = alg_bytes / st["ms"] / 1e6
        e["hbm_frac"] = alg_bytes / st["ms"] / 1e-3 / PEAK_HBM
    e["frac"] = e["mfma_frac"] if bound == "mfma" else e["hbm_frac"]
    e.update(extra)
    return e


def time_ops(clock, ops, working_set):
    """Per-kernel statistics of a dict of launches; flushed where the working set is small."""
    out = {}
    for name, fn in ops.items():
        fl = working_set[name] < CACHE_LIMIT
        out[name] = stats(clock.launches(fn, flush=fl), fl)
    return out


def wall_steps(torch, step, steps, warmup):
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


# ----------------------------------------------------------------------------- workloads

def run_csa_prefill(torch, clock, steps, warmup):
    import workloads as W
    from long_context_sparse_09_amd import (csa_attend, csa_compress, csa_index_topk, layers,
                                            swa_concat)

    w = W.workload(2)
    S = w.S
    log(f"[bench] CSA prefill S={S}: generating inputs")
    inp = layers.to_device(W.layer_inputs(w, 0))
    sh = layers.LayerShape(w.B, S, w.H, w.D, w.r, w.m, w.m_hca, w.nI, w.cI, w.k, w.W, w.base,
                           torch.bfloat16)
    buf = layers.LayerBuffers(sh, kinds=("csa",))
    z = buf.zeros_b
    ops = {
        "csa_compress_kv": lambda: csa_compress(inp["kv"], inp["gate"], inp["bias"], buf.pool, w.m,
                                                True, rope_dim=w.r, rope_theta=w.base),
        "csa_compress_idx": lambda: csa_compress(inp["k_idx"], inp["g_idx"], inp["bias_idx"],
                                                 buf.k_pool, w.m, True),
        "csa_index_topk": lambda: csa_index_topk(inp["q_idx"], inp["w_idx"], buf.k_pool, z,
                                                 buf.n_pool, buf.topk_idx, None, w.m,
                                                 buf.workspace),
        "swa_concat": lambda: swa_concat(inp["kv"], buf.kv_win, z, z, w.r, w.base),
        "csa_attend": lambda: csa_attend(inp["q"], buf.kv_win, z, buf.pool, buf.topk_idx,
                                         inp["sink"], z, buf.out, w.W, w.r, w.base),
    }

    def step():
        for fn in ops.values():
            fn()

    log(f"[bench] CSA prefill: timing {steps} steps")
    wall = wall_steps(torch, step, steps, warmup)
    N = S // w.m
    win, sel = csa_keys_per_query(S, w.W, w.m, w.k)
    a_flops = attend_flops((win + sel).sum(), w.H, w.D)
    i_flops = index_flops(S, w.m, w.nI, w.cI)
    b_kv = compress_bytes(S, w.D, w.m, True, N)
    b_idx = compress_bytes(S, w.cI, w.m, True, N)
    b_swa = 2 * S * w.D * 2
    vis = float(((np.arange(S) + 1) // w.m).sum())
    b_index = S * w.nI * w.cI * 2 + S * w.nI * 4 + N * w.cI * 2 + S * w.k * 4
    b_att = S * w.H * w.D * 2 * 2 + S * w.D * 2 + N * w.D * 2 + S * w.k * 4
    wset = {"csa_compress_kv": b_kv, "csa_compress_idx": b_idx, "swa_concat": b_swa,
            "csa_index_topk": b_index, "csa_attend": b_att}
    log("[bench] CSA prefill: per-kernel launches")
    st = time_ops(clock, ops, wset)
    kern = {
        "csa_compress_kv": kernel_entry(st["csa_compress_kv"], "hbm", alg_bytes=b_kv),
        "csa_compress_idx": kernel_entry(st["csa_compress_idx"], "hbm", alg_bytes=b_idx),
        "csa_index_topk": kernel_entry(st["csa_index_topk"], "mfma", alg_flops=i_flops,
                                       alg_bytes=b_index, visible_pairs=vis),
        "swa_concat": kernel_entry(st["swa_concat"], "hbm", alg_bytes=b_swa),
        "csa_attend": kernel_entry(st["csa_attend"], "mfma", alg_flops=a_flops, alg_bytes=b_att,
                                   keys_per_query=float((win + sel).mean())),
    }
    del inp, buf
    return w, wall, kern


def run_hca_prefill(torch, clock, steps, warmup):
    import workloads as W
    from long_context_sparse_09_amd import csa_compress, hca_attend, hca_attend_pairs, layers, swa_concat

    w = W.workload(3)
    S = w.S
    log(f"[bench] HCA prefill S={S}: generating inputs")
    inp = layers.to_device(W.layer_inputs(w, 0, names=["q", "kv", "gate"]))
    inp.update(layers.to_device({"bias_hca": W.param(w, 0, "bias_hca"), "sink": W.param(w, 0, "sink")}))
    sh = layers.LayerShape(w.B, S, w.H, w.D, w.r, w.m, w.m_hca, w.nI, w.cI, w.k, w.W, w.base,
                           torch.bfloat16)
    buf = layers.LayerBuffers(sh, kinds=("hca",))
    z = buf.zeros_b
    ops = {
        "hca_compress": lambda: csa_compress(inp["kv"], inp["gate"], inp["bias_hca"], buf.pool_h,
                                             w.m_hca, False, rope_dim=w.r, rope_theta=w.base),
        "swa_concat": lambda: swa_concat(inp["kv"], buf.kv_win, z, z, w.r, w.base),
        "hca_attend": lambda: hca_attend(inp["q"], buf.kv_win, z, buf.pool_h, buf.n_pool_h,
                                         w.m_hca, inp["sink"], z, buf.out, w.W, w.r, w.base),
    }

    def step():
        for fn in ops.values():
            fn()

    wall = wall_steps(torch, step, steps, warmup)
    t = np.arange(S, dtype=np.int64)
    keys = np.minimum(t + 1, w.W) + np.minimum((t + 1) // w.m_hca, S // w.m_hca)
    fl = attend_flops(keys.sum(), w.H, w.D)
    N = S // w.m_hca
    b_att = S * w.H * w.D * 2 * 2 + S * w.D * 2 + N * w.D * 2  # q + out + window + pool, once each
    b_cmp = compress_bytes(S, w.D, w.m_hca, False, N)
    b_swa = 2 * S * w.D * 2
    st = time_ops(clock, ops, {"hca_compress": b_cmp, "swa_concat": b_swa, "hca_attend": b_att})
    # the query-pair kernel on the same inputs, for comparison (not part of the step)
    pairs = {"hca_attend_pairs": lambda: hca_attend_pairs(inp["q"], buf.kv_win, z, buf.pool_h, buf.n_pool_h,
                                                          w.m_hca, inp["sink"], z, buf.out, w.W, w.r, w.base)}
    st.update(time_ops(clock, pairs, {"hca_attend_pairs": b_att}))
    del inp, buf
    return {
        "workload": w.name, "query_tokens_per_s": S / wall, "ms_per_step": wall * 1e3,
        "kernels": {
            "hca_compress": kernel_entry(st["hca_compress"], "hbm", alg_bytes=b_cmp),
            "swa_concat": kernel_entry(st["swa_concat"], "hbm", alg_bytes=b_swa),
            # AI = 380 flop/B, near the ridge (315): both fractions are reported
            "hca_attend": kernel_entry(st["hca_attend"], "mfma", alg_flops=fl, alg_bytes=b_att,
                                       keys_per_query=float(keys.mean())),
            "hca_attend_pairs (comparison, not in the step)": kernel_entry(
                st["hca_attend_pairs"], "mfma", alg_flops=fl, alg_bytes=b_att),
        },
    }


def _decode_bytes(w, L):
    n_valid = L // w.m
    idx_bytes = float(n_valid.sum()) * w.cI * 2 + len(L) * (w.nI * w.cI * 2 + w.nI * 4)
    k_sel = np.minimum(w.k, n_valid)
    att_bytes = float((k_sel * w.D * 2).sum()) + len(L) * (w.W * w.D * 2 + 2 * w.H * w.D * 2)
    return idx_bytes, att_bytes


def run_decode(torch, clock, steps, warmup):
    """Config 4 with pre-generated caches: swa_concat of the new token + csa_index_topk +
    csa_attend (key-range split), one step per event pair, cache flushed before each step."""
    import workloads as W
    from long_context_sparse_09_amd import csa_attend, csa_index_topk, layers, swa_concat

    w = W.workload(4)
    log("[bench] CSA decode 64 sequences: generating caches")
    d = W.decode_inputs(w)
    L = d.pop("lengths")
    t = layers.to_device(d)
    sh = layers.LayerShape(w.n_seq, 1, w.H, w.D, w.r, w.m, w.m_hca, w.nI, w.cI, w.k, w.W, w.base,
                           torch.bfloat16)
    st = layers.DecodeState(t, sh, L)
    reps = max(steps, 20)
    step_ms = clock.launches(lambda: layers.csa_decode_step(st), reps=reps, warm=warmup, flush=True)
    back_to_back = wall_steps(torch, lambda: layers.csa_decode_step(st), reps, 0)
    ops = {
        "swa_concat": lambda: swa_concat(t["kv_new"], t["window"], st.kv_pos0, st.q_pos0, sh.r,
                                         sh.base),
        "csa_index_topk": lambda: csa_index_topk(t["q_idx"], t["w_idx"], t["k_pool"], st.q_pos0,
                                                 st.n_pool, st.topk_idx, None, sh.m, st.workspace),
        "csa_attend": lambda: csa_attend(t["q"], t["window"], st.kv_pos0, t["pool"], st.topk_idx,
                                         t["sink"], st.q_pos0, st.out, sh.W, sh.r, sh.base,
                                         workspace=st.attend_ws),
    }
    per = {n: stats(clock.launches(fn, flush=True), True) for n, fn in ops.items()}
    idx_bytes, att_bytes = _decode_bytes(w, L)
    s = stats(step_ms, True)
    del t, st
    return {"workload": w.name, "us_per_step": s["ms"] * 1e3, "us_per_step_min": s["ms_min"] * 1e3,
            "us_per_step_mean": s["ms_mean"] * 1e3, "steps_timed": s["reps"],
            "cache": "flushed before every step",
            "us_per_step_back_to_back": back_to_back * 1e6,
            "alg_bytes": {"index_scan": idx_bytes, "attend": att_bytes},
            "hbm_frac_whole_step": (idx_bytes + att_bytes) / (s["ms"] * 1e-3) / PEAK_HBM,
            "kernels": {
                "swa_concat": dict(per["swa_concat"], bound="hbm"),
                "csa_index_topk": kernel_entry(per["csa_index_topk"], "hbm", alg_bytes=idx_bytes),
                "csa_attend": kernel_entry(per["csa_attend"], "hbm", alg_bytes=att_bytes),
            }}


def run_decode_cache(torch, clock, steps, warmup):
    """Config 4's shape decoded through the per-layer cache (DecodeCache.step: the compressor
    ring updates of the K=V pool and the indexer keys, the window append, the indexer and the
    attention; the step's per-sequence integers are uploaded from the host each step).  The
    caches are pre-generated N(0,1) contents (pools, rings, window) of sequences of the same
    lengths; every step appends one token per sequence.  One step per event pair, flushed."""
    import workloads as W
    from long_context_sparse_09_amd import layers
    from long_context_sparse_09_amd.cache import DecodeCache

    w = W.workload(4)
    L = W.decode_lengths(w)[:w.n_seq]
    B = w.n_seq
    sh = layers.LayerShape(B, 1, w.H, w.D, w.r, w.m, w.m_hca, w.nI, w.cI, w.k, w.W, w.base,
                           torch.bfloat16)
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed * 1000 + 404)
    rn = lambda *s: torch.randn(s, generator=g, device="cuda").to(torch.bfloat16)  # noqa: E731
    params = {"bias": torch.randn((2 * w.m, w.D), generator=g, device="cuda"),
              "bias_idx": torch.randn((2 * w.m, w.cI), generator=g, device="cuda"),
              "sink": torch.randn((w.H,), generator=g, device="cuda")}
    n_cap = w.L_max // w.m
    cache = DecodeCache("csa", sh, params, n_cap, G=256)
    cache.pool.copy_(rn(B, n_cap, w.D))
    cache.k_pool.copy_(rn(B, n_cap, w.cI))
    cache.win[cache.cur].copy_(rn(B, w.W + cache.G, w.D))
    for ring in cache.ring.values():
        ring.copy_(rn(*ring.shape))
    cache.L[:] = L - 1  # each step appends the token at position L - 1, L, ...
    n_steps = max(steps, 20) + warmup
    toks = [{"q": rn(B, 1, w.H, w.D), "kv": rn(B, 1, w.D), "gate": rn(B, 1, w.D),
             "k_idx": rn(B, 1, w.cI), "g_idx": rn(B, 1, w.cI), "q_idx": rn(B, 1, w.nI, w.cI),
             "w_idx": torch.randn((B, 1, w.nI), generator=g, device="cuda")} for _ in range(4)]
    it = iter(range(n_steps))
    ms = clock.launches(lambda: cache.step(toks[next(it) % 4]), reps=n_steps - warmup, warm=warmup,
                        flush=True)
    s = stats(ms, True)
    del cache
    return {"workload": f"{w.name} through DecodeCache.step", "us_per_step": s["ms"] * 1e3,
            "us_per_step_min": s["ms_min"] * 1e3, "steps_timed": s["reps"],
            "cache": "flushed before every step",
            "note": "includes the compressor ring updates and the host upload of the step's lengths"}


def run_stack(torch, clock, steps, warmup):
    """The mixed eight-layer stack at S=32768, prefilled in 4096-query chunks (chunk-major).

    Inputs are generated on the device (torch's Philox generator, seeded per layer and tensor,
    N(0,1) rounded to bf16; fp32 biases, sinks and indexer weights), the same distribution as
    the keyed host generator the parity tests use: regenerating 17 GB of activations on the
    host would dominate the run."""
    import workloads as W
    from long_context_sparse_09_amd import layers

    w = W.workload(5)
    S, kinds = w.S, list(w.layer_types)
    log(f"[bench] stack {kinds} S={S} chunk={w.chunk}: generating inputs on the device")
    sh = layers.LayerShape(w.B, S, w.H, w.D, w.r, w.m, w.m_hca, w.nI, w.cI, w.k, w.W, w.base,
                           torch.bfloat16)
    shapes = {"q": (w.H, w.D), "kv": (w.D,), "gate": (w.D,), "q_idx": (w.nI, w.cI),
              "k_idx": (w.cI,), "g_idx": (w.cI,)}
    need = {"sliding": ("q", "kv"), "hca": ("q", "kv", "gate"), "csa": tuple(shapes)}
    inps, bufs = [], []
    for ell, kind in enumerate(kinds):
        g = torch.Generator(device="cuda")
        g.manual_seed(w.seed * 1000 + ell)
        d = {n: torch.randn((1, S) + shapes[n], generator=g, device="cuda",
                            dtype=torch.float32).to(torch.bfloat16) for n in need[kind]}
        d["w_idx"] = torch.randn((1, S, w.nI), generator=g, device="cuda")
        d["sink"] = torch.randn((w.H,), generator=g, device="cuda")
        d["bias"] = torch.randn((2 * w.m, w.D), generator=g, device="cuda")
        d["bias_idx"] = torch.randn((2 * w.m, w.cI), generator=g, device="cuda")
        d["bias_hca"] = torch.randn((w.m_hca, w.D), generator=g, device="cuda")
        inps.append(d)
        bufs.append(layers.LayerBuffers(sh, kinds=(kind,)))
    torch.cuda.synchronize()

    def step():
        layers.stack_prefill_chunked(kinds, inps, bufs, w.chunk)

    log(f"[bench] stack: timing {steps} steps")
    wall = wall_steps(torch, step, steps, warmup)
    # each layer's chunk loop between events, per layer type (3 passes)
    per_kind = {}
    for _ in range(3):
        for ell, kind in enumerate(kinds):
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            ev0.record()
            layers.prefill_chunked(kind, inps[ell], bufs[ell], w.chunk)
            ev1.record()
            per_kind.setdefault(kind, []).append((ev0, ev1))
    torch.cuda.synchronize()
    layer_ms = {k: float(np.median([a.elapsed_time(b) for a, b in v])) for k, v in per_kind.items()}
    win, sel = csa_keys_per_query(S, w.W, w.m, w.k)
    t = np.arange(S, dtype=np.int64)
    hkeys = np.minimum(t + 1, w.W) + (t + 1) // w.m_hca
    fl = {"csa": attend_flops((win + sel).sum(), w.H, w.D) + index_flops(S, w.m, w.nI, w.cI),
          "hca": attend_flops(hkeys.sum(), w.H, w.D),
          "sliding": attend_flops(win.sum(), w.H, w.D)}
    qo = S * w.H * w.D * 2 * 2  # q read + out written
    by = {"sliding": qo + 3 * S * w.D * 2,
          "hca": qo + 3 * S * w.D * 2 + S * w.D * 2 + (S // w.m_hca) * w.D * 2 * 2,
          "csa": qo + 3 * S * w.D * 2 + 2 * S * (w.D + w.cI) * 2 + S * w.nI * (w.cI * 2 + 4)}
    layers_out = {}
    for k in layer_ms:
        ms = layer_ms[k]
        e = {"ms": ms, "alg_flops": fl[k], "alg_bytes": by[k],
             "mfma_frac": fl[k] / (ms * 1e-3) / PEAK_BF16, "hbm_frac": by[k] / (ms * 1e-3) / PEAK_HBM}
        e["bound"] = "mfma" if fl[k] / by[k] > PEAK_BF16 / PEAK_HBM else "hbm"
        e["frac"] = e["mfma_frac"] if e["bound"] == "mfma" else e["hbm_frac"]
        layers_out[k] = e
    total = sum(fl[k] for k in kinds)
    del inps, bufs
    return {"workload": w.name, "layer_types": kinds, "chunk": w.chunk,
            "query_tokens_per_s": S / wall, "ms_per_step": wall * 1e3,
            "layers": layers_out,
            "alg_flops_per_step": total, "TFLOP/s": total / wall / 1e12,
            "mfma_frac_whole_step": total / wall / PEAK_BF16,
            "inputs": "device-generated N(0,1), torch Philox, seeded per layer"}


def run_oproj(torch, clock, steps, warmup):
    """The grouped low-rank output projection after the S=8192 CSA layer: 8192 tokens of
    64 heads x 512 -> 8 groups x rank 1024 -> hidden 4096 (DeepseekV4Config defaults).  Inputs
    are generated on the device (N(0,1) attention output, fan-in-scaled N(0,1) weights, bf16)."""
    import workloads as W
    from long_context_sparse_09_amd import grouped_out_proj

    w = W.workload(2)
    T, G, rk, hid = w.S, w.o_groups, w.o_rank, w.hidden
    kg = w.H // G * w.D
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed * 1000 + 77)
    attn = torch.randn((T, w.H, w.D), generator=g, device="cuda").to(torch.bfloat16)
    w_a = (torch.randn((G, rk, kg), generator=g, device="cuda") / kg ** 0.5).to(torch.bfloat16)
    w_b = (torch.randn((hid, G * rk), generator=g, device="cuda") / (G * rk) ** 0.5).to(torch.bfloat16)
    mid = torch.empty((T, G * rk), device="cuda", dtype=torch.bfloat16)
    out = torch.empty((T, hid), device="cuda", dtype=torch.bfloat16)
    st = stats(clock.launches(lambda: grouped_out_proj(attn, w_a, w_b, mid, out), warm=warmup,
                              flush=False), False)
    flops = 2.0 * T * (G * rk * kg + hid * G * rk)
    e = kernel_entry(st, "mfma", alg_flops=flops)
    e.update(workload="grouped_out_proj T=8192: 64x512 -> 8x1024 -> 4096 (bf16)",
             tokens_per_s=T / st["ms"] * 1e3)
    return e


def run_inproj(torch, clock, steps, warmup):
    """The input projections of the S=8192 CSA layer: 8192 tokens of hidden 4096 -> the query
    latent (q_lora_rank 1024), K=V head and compressor gate (512 each), indexer key content and
    gate (128 each) and head weights (64, fp32); then the latent -> 64 x 512 query heads and
    64 x 128 indexer query heads (DeepseekV4Config defaults).  Inputs are generated on the
    device (N(0,1) hidden state, fan-in-scaled N(0,1) weights, bf16)."""
    import workloads as W
    from long_context_sparse_09_amd import input_projections

    w = W.workload(2)
    T, hid, qr = w.S, w.hidden, w.q_rank
    wd = W.inproj_widths(w)
    n_x = sum(wd[n] for n in W.INPROJ_X_ORDER["csa"])
    n_lat = sum(wd[n] for n in W.INPROJ_LAT_ORDER["csa"])
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed * 1000 + 91)
    x = torch.randn((T, hid), generator=g, device="cuda").to(torch.bfloat16)
    w_x = (torch.randn((n_x, hid), generator=g, device="cuda") / hid ** 0.5).to(torch.bfloat16)
    w_lat = (torch.randn((n_lat, qr), generator=g, device="cuda") / qr ** 0.5).to(torch.bfloat16)
    e = lambda *sh, dt=torch.bfloat16: torch.empty(*sh, dtype=dt, device="cuda")  # noqa: E731
    out = dict(c_q=e(T, qr), q=e(T, w.H, w.D), kv=e(T, w.D), gate=e(T, w.D), q_idx=e(T, w.nI, w.cI),
               k_idx=e(T, w.cI), g_idx=e(T, w.cI), w_idx=e(T, w.nI, dt=torch.float32))
    st = stats(clock.launches(lambda: input_projections("csa", x, w_x, w_lat, **out), warm=warmup,
                              flush=False), False)
    flops = 2.0 * T * (n_x * hid + n_lat * qr)
    r = kernel_entry(st, "mfma", alg_flops=flops)
    r.update(workload=f"input_projections T=8192 CSA: 4096 -> {n_x} (latent, kv, gate, indexer k/g/w); "
                      f"1024 -> {n_lat} (q, indexer q) (bf16)", tokens_per_s=T / st["ms"] * 1e3)
    return r


# ----------------------------------------------------------------------------- CPU oracle

def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _oracle_csa_rows(oracle, W, w, layer, rows, pool, k_pool, kv_win, sink):
    N = pool.shape[1]
    for t in rows:
        qi = W.to_f64(W.activation_rows(w, layer, "q_idx", [t]))
        wi = W.activation_rows(w, layer, "w_idx", [t])
        idx, _ = oracle.csa_index_topk(qi[None], wi[None], k_pool, [t], [N], w.m, w.k)
        q = W.to_f64(W.activation_rows(w, layer, "q", [t]))
        oracle.csa_attend(q[None], kv_win, [0], pool, idx, sink, [t], w.W, w.r, w.base)


def cpu_baseline(n2=320, n3=64):
    """The fp64 oracle on this host, single-threaded (numpy's BLAS pool limited to one thread;
    the oracle's own loops are plain Python).  Config 2 (the headline): pooling and window
    rotation of all 8192 tokens, then index / top-k / attention for n2 evenly spaced queries,
    extrapolated.  Config 1: the whole tiny layer.  Config 3: pooling of all 65536 tokens, then
    window rotation and attention for n3 evenly spaced queries, extrapolated.  Config 4: one
    decode step of all 64 sequences (index scan, top-k, attention), cache generation excluded."""
    import oracle
    import workloads as W

    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
        threads = 1
    except Exception:  # noqa: BLE001
        limiter, threads = None, None
    try:
        res = {}
        # ---- config 1, whole layer
        w1 = W.workload(1)
        inp = W.layer_inputs(w1, 0)
        f64 = {k: W.to_f64(v) for k, v in inp.items()}
        t0 = time.perf_counter()
        oracle.csa_layer(f64, w1)
        t1 = time.perf_counter() - t0
        res["config1"] = {"value": w1.S / t1, "unit": "query-tokens/s", "seconds": t1,
                          "sample": f"whole layer, S={w1.S}"}
        # ---- config 2, headline
        w = W.workload(2)
        S = w.S
        inp = W.layer_inputs(w, 0, names=["kv", "gate", "k_idx", "g_idx"])
        f = {k: W.to_f64(inp[k]) for k in ("kv", "gate", "k_idx", "g_idx")}
        t0 = time.perf_counter()
        pool = oracle.csa_compress(f["kv"], f["gate"], inp["bias"], w.m, True, w.r, w.base)
        k_pool = oracle.csa_compress(f["k_idx"], f["g_idx"], inp["bias_idx"], w.m, True, 0)
        kv_win = oracle.swa_concat(f["kv"], [0], w.r, w.base)
        t_full = time.perf_counter() - t0
        rows = np.linspace(0, S - 1, n2).astype(int)
        t0 = time.perf_counter()
        _oracle_csa_rows(oracle, W, w, 0, rows, pool, k_pool, kv_win, inp["sink"])
        t_rows = time.perf_counter() - t0
        est2 = t_full + t_rows / n2 * S
        res["config2"] = {"value": S / est2, "unit": "query-tokens/s", "seconds": t_full + t_rows,
                          "sample": f"S={S} CSA layer: pooling + window rotation of all tokens, "
                                    f"index/top-k/attention for {n2} of {S} queries (evenly spaced), "
                                    "extrapolated"}
        # ---- config 3, HCA
        w3 = W.workload(3)
        S3 = w3.S
        inp3 = W.layer_inputs(w3, 0, names=["kv", "gate"])
        kv3 = W.to_f64(inp3["kv"])
        t0 = time.perf_counter()
        hpool = oracle.csa_compress(kv3, W.to_f64(inp3["gate"]), inp3["bias_hca"], w3.m_hca, False,
                                    w3.r, w3.base)
        t_pool = time.perf_counter() - t0
        rows3 = np.linspace(0, S3 - 1, n3).astype(int)
        t0 = time.perf_counter()
        for t in rows3:
            lo = max(0, t - w3.W + 1)
            win = oracle.swa_concat(kv3[:, lo:t + 1], [lo], w3.r, w3.base)
            q = W.to_f64(W.activation_rows(w3, 0, "q", [t]))
            oracle.hca_attend(q[None], win, [lo], hpool, [hpool.shape[1]], w3.m_hca, inp3["sink"], [t],
                              w3.W, w3.r, w3.base)
        t_rows3 = time.perf_counter() - t0
        est3 = t_pool + t_rows3 / n3 * S3
        res["config3"] = {"value": S3 / est3, "unit": "query-tokens/s", "seconds": t_pool + t_rows3,
                          "sample": f"S={S3} HCA layer: pooling of all tokens, window rotation and "
                                    f"attention for {n3} of {S3} queries (evenly spaced), extrapolated"}
        del kv3, hpool, inp3
        # ---- config 4, one decode step of every sequence
        w4 = W.workload(4)
        Ls = W.decode_lengths(w4)[:w4.n_seq]
        t_dec = 0.0
        for b in range(w4.n_seq):
            one = W.decode_inputs(w4, seqs=[b])
            fo = {k: W.to_f64(v) if v.dtype == np.uint16 else v for k, v in one.items()}
            Lb = int(Ls[b])
            n = Lb // w4.m
            t0 = time.perf_counter()
            win = fo["window"].copy()
            win[0, -1] = oracle.swa_concat(fo["kv_new"], [Lb - 1], w4.r, w4.base)[0, 0]
            idx, _ = oracle.csa_index_topk(fo["q_idx"], fo["w_idx"], fo["k_pool"], [Lb - 1], [n], w4.m,
                                           w4.k)
            oracle.csa_attend(fo["q"], win, [Lb - w4.W], fo["pool"], idx, fo["sink"], [Lb - 1], w4.W,
                              w4.r, w4.base)
            t_dec += time.perf_counter() - t0
        res["config4"] = {"value": t_dec * 1e6, "unit": "us/step", "seconds": t_dec,
                          "sample": f"one decode step of all {w4.n_seq} sequences (cache generation "
                                    "excluded)"}
    finally:
        if limiter is not None:
            limiter.unregister()
    head = res["config2"]
    return {"value": head["value"], "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
            "sample": head["sample"], "seconds_measured": sum(r["seconds"] for r in res.values()),
            "threads": threads, "host_cores": len(os.sched_getaffinity(0)),
            "host_cpu_count": os.cpu_count(), "cpu_model": _cpu_model(),
            "configs": res}


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true", help="skip the HCA / decode / stack workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", choices=["csa_prefill", "hca_prefill", "csa_decode", "decode_cache",
                                       "stack", "oproj", "inproj"],
                    default=None, help="run one workload alone (for profiling); prints its figures only")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MiB",
                    help="launch one device copy of this size first (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path would shard by query ranges (one all-gather of the pooled K=V)", file=sys.stderr)
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calib > 0:
        n = args.copy_calib << 18  # fp32 elements
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {n * 4} bytes read, {n * 4} bytes written")
        del src, dst
    clock = Clock(torch)
    others = {"hca_prefill": run_hca_prefill, "csa_decode": run_decode, "decode_cache": run_decode_cache,
              "stack": run_stack, "oproj": run_oproj, "inproj": run_inproj}
    if args.only in others:
        print(json.dumps({"only": args.only, **others[args.only](torch, clock, args.steps, args.warmup)}),
              flush=True)
        return
    w, wall, kern = run_csa_prefill(torch, clock, args.steps, args.warmup)
    if args.only == "csa_prefill":
        print(json.dumps({"only": args.only, "query_tokens_per_s": w.S / wall,
                          "ms_per_step": wall * 1e3, "kernels": kern}), flush=True)
        return
    extra = {}
    if not args.no_extra:
        torch.cuda.empty_cache()
        extra["hca_prefill"] = run_hca_prefill(torch, clock, max(3, args.steps // 4), 1)
        torch.cuda.empty_cache()
        extra["csa_decode"] = run_decode(torch, clock, args.steps, args.warmup)
        torch.cuda.empty_cache()
        extra["csa_decode_cache"] = run_decode_cache(torch, clock, args.steps, args.warmup)
        torch.cuda.empty_cache()
        extra["stack8_prefill"] = run_stack(torch, clock, max(2, args.steps // 10), 1)
        torch.cuda.empty_cache()
        extra["grouped_out_proj"] = run_oproj(torch, clock, args.steps, args.warmup)
        extra["input_projections"] = run_inproj(torch, clock, args.steps, args.warmup)
        torch.cuda.empty_cache()
    att = kern["csa_attend"]
    src = kernel_hash("attend_mfma.hip", "common.h")
    prof = load_profile("csa_prefill/csa_attend", src)
    roof = {"kernel": "csa_attend", "bound": "mfma",
            "achieved": att["alg_flops"] / att["ms_mean"] / 1e9, "peak": PEAK_BF16 / 1e12,
            "unit": "TFLOP/s", "frac": att["alg_flops"] / att["ms_mean"] / 1e-3 / PEAK_BF16,
            "traffic": prof.get("bytes_per_launch"),
            "alg_flops_per_launch": att["alg_flops"], "launch_ms_mean": att["ms_mean"],
            "launch_ms_median": att["ms"], "launch_ms_min": att["ms_min"],
            "frac_median": att["mfma_frac"], "source_hash": src}
    if prof.get("rocprof_avg_us"):
        roof["rocprof_avg_us"] = prof["rocprof_avg_us"]
        roof["frac_rocprof"] = att["alg_flops"] / (prof["rocprof_avg_us"] * 1e-6) / PEAK_BF16
    res = {
        "metric": "CSA prefill query-tokens/s (S=8192); HCA prefill query-tokens/s and CSA decode "
                  "us/step in 'workloads'",
        "value": w.S / wall,
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "S": w.S, "H": w.H, "D": w.D, "rope": w.r,
                   "m": w.m, "index_heads": w.nI, "index_dim": w.cI, "topk": w.k,
                   "window": w.W, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "kernels": kern,
        "workloads": extra,
    }
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline()
    else:
        res["cpu_baseline"] = None
    # release the device and host buffers before the line is printed, so the process exits
    # promptly once it is read (bench.py starts no other process)
    del clock, w
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the hybrid attention core on one MI355X.

Headline (one JSON line): CSA prefill query-tokens/s on the S=8192 workload (64 heads x 512,
rope 64, m=4, 64 x 128 indexer, top-512, window 128, bf16).  One step = the whole CSA hot
path over one batch: csa_compress (K=V pool) + csa_compress (indexer keys) + csa_index_topk +
swa_concat + csa_attend, inputs resident in HBM.

Also reported in the same line ("workloads"): HCA prefill query-tokens/s at S=65536, CSA
decode us/step for 64 sequences of 16K-128K context, and the mixed eight-layer stack
(sliding, sliding, CSA, HCA, CSA, HCA, CSA, HCA) at S=32768 prefilled in 4096-query chunks,
plus per-kernel times and roofline
fractions.  "roofline" is for the dominant kernel (csa_attend): algorithmic flops per launch
over the launch's average duration (HIP events on the launch stream).  "cpu_baseline" is the
fp64 CPU oracle timed on this host's cores over a bounded sample of the same workload.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu] [--copy-calib MiB]

--copy-calib launches one plain device-to-device copy of that many MiB before the timed work,
so that a counter run (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE) sees a kernel of known traffic
to scale the attention kernel's counters by.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15  # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12   # MI355X HBM3E, B/s


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


def kernel_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "long_context_sparse_09_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, src_hash: str):
    """Measured HBM bytes per launch from profiles/traffic.json, if taken on this source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p)).get(kernel)
    except (ValueError, OSError):
        return None
    if not d or d.get("source_hash") != src_hash:
        return None
    return d.get("bytes_per_launch")


# ----------------------------------------------------------------------------- timing helpers

class Timer:
    """HIP events on torch's current stream (the stream every library call is enqueued on)."""

    def __init__(self, torch):
        self.torch = torch
        self.acc = {}

    def __call__(self, name, fn):
        ev0 = self.torch.cuda.Event(enable_timing=True)
        ev1 = self.torch.cuda.Event(enable_timing=True)
        ev0.record()
        fn()
        ev1.record()
        self.acc.setdefault(name, []).append((ev0, ev1))

    def means_ms(self):
        self.torch.cuda.synchronize()
        return {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in self.acc.items()}


def run_csa_prefill(torch, steps, warmup):
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

    def step(timer=None):
        for name, fn in ops.items():
            if timer is None:
                fn()
            else:
                timer(name, fn)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] CSA prefill: timing {steps} steps")
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    # per-kernel launch durations (separate pass, events around each launch)
    timer = Timer(torch)
    for _ in range(max(3, steps)):
        step(timer)
    per = timer.means_ms()

    win, sel = csa_keys_per_query(S, w.W, w.m, w.k)
    a_flops = attend_flops((win + sel).sum(), w.H, w.D)
    i_flops = index_flops(S, w.m, w.nI, w.cI)
    N = S // w.m
    bytes_kv = 2 * S * w.D * 2 + 2 * w.m * w.D * 4 + N * w.D * 2
    bytes_idx = 2 * S * w.cI * 2 + 2 * w.m * w.cI * 4 + N * w.cI * 2
    bytes_swa = 2 * S * w.D * 2
    kern = {
        "csa_compress_kv": {"ms": per["csa_compress_kv"], "bound": "hbm", "alg_bytes": bytes_kv,
                            "GB/s": bytes_kv / per["csa_compress_kv"] / 1e6},
        "csa_compress_idx": {"ms": per["csa_compress_idx"], "bound": "hbm",
                             "alg_bytes": bytes_idx, "GB/s": bytes_idx / per["csa_compress_idx"] / 1e6},
        "csa_index_topk": {"ms": per["csa_index_topk"], "bound": "mfma", "alg_flops": i_flops,
                           "TFLOP/s": i_flops / per["csa_index_topk"] / 1e9},
        "swa_concat": {"ms": per["swa_concat"], "bound": "hbm", "alg_bytes": bytes_swa,
                       "GB/s": bytes_swa / per["swa_concat"] / 1e6},
        "csa_attend": {"ms": per["csa_attend"], "bound": "mfma", "alg_flops": a_flops,
                       "TFLOP/s": a_flops / per["csa_attend"] / 1e9,
                       "keys_per_query": float((win + sel).mean())},
    }
    for v in kern.values():
        v["frac"] = (v["TFLOP/s"] * 1e12 / PEAK_BF16) if v["bound"] == "mfma" else (v["GB/s"] * 1e9 / PEAK_HBM)
    return w, wall, kern


def run_hca_prefill(torch, steps, warmup):
    import workloads as W
    from long_context_sparse_09_amd import csa_compress, hca_attend, layers, swa_concat

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
    for _ in range(warmup):
        for fn in ops.values():
            fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        for fn in ops.values():
            fn()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    timer = Timer(torch)
    for _ in range(max(3, steps)):
        for n, fn in ops.items():
            timer(n, fn)
    per = timer.means_ms()
    t = np.arange(S, dtype=np.int64)
    keys = np.minimum(t + 1, w.W) + np.minimum((t + 1) // w.m_hca, S // w.m_hca)
    fl = attend_flops(keys.sum(), w.H, w.D)
    N = S // w.m_hca
    b_att = S * w.H * w.D * 2 * 2 + S * w.D * 2 + N * w.D * 2  # q + out + window + pool, once each
    b_cmp = 2 * S * w.D * 2 + w.m_hca * w.D * 4 + N * w.D * 2
    del inp, buf
    return {
        "workload": w.name, "query_tokens_per_s": S / wall, "ms_per_step": wall * 1e3,
        "kernels": {
            "hca_compress": {"ms": per["hca_compress"], "bound": "hbm", "alg_bytes": b_cmp,
                             "GB/s": b_cmp / per["hca_compress"] / 1e6,
                             "frac": b_cmp / per["hca_compress"] / 1e-3 / PEAK_HBM},
            "swa_concat": {"ms": per["swa_concat"], "bound": "hbm",
                           "GB/s": 2 * S * w.D * 2 / per["swa_concat"] / 1e6,
                           "frac": 2 * S * w.D * 2 / per["swa_concat"] / 1e-3 / PEAK_HBM},
            "hca_attend": {"ms": per["hca_attend"], "bound": "mfma", "alg_flops": fl,
                           "TFLOP/s": fl / per["hca_attend"] / 1e9,
                           "frac": fl / per["hca_attend"] / 1e-3 / PEAK_BF16,
                           "alg_bytes": b_att,
                           "hbm_frac": b_att / per["hca_attend"] / 1e-3 / PEAK_HBM,
                           "keys_per_query": float(keys.mean())},
        },
    }


def run_decode(torch, steps, warmup):
    import workloads as W
    from long_context_sparse_09_amd import layers

    w = W.workload(4)
    log("[bench] CSA decode 64 sequences: generating caches")
    d = W.decode_inputs(w)
    L = d.pop("lengths")
    t = layers.to_device(d)
    sh = layers.LayerShape(w.n_seq, 1, w.H, w.D, w.r, w.m, w.m_hca, w.nI, w.cI, w.k, w.W, w.base,
                           torch.bfloat16)
    st = layers.DecodeState(t, sh, L)
    for _ in range(warmup):
        layers.csa_decode_step(st)
    torch.cuda.synchronize()
    n = max(steps, 20)
    t0 = time.perf_counter()
    for _ in range(n):
        layers.csa_decode_step(st)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / n
    n_valid = (L // w.m)
    idx_bytes = float(n_valid.sum()) * w.cI * 2 + w.n_seq * w.nI * w.cI * 2
    att_bytes = w.n_seq * (w.k * w.D * 2 + w.W * w.D * 2 + 2 * w.H * w.D * 2)
    del t, st
    return {"workload": w.name, "us_per_step": wall * 1e6,
            "alg_bytes": {"index_scan": idx_bytes, "attend": att_bytes},
            "hbm_frac_whole_step": (idx_bytes + att_bytes) / wall / PEAK_HBM}


def run_stack(torch, steps, warmup):
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

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] stack: timing {steps} steps")
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    # one step with events around each layer's chunk loop, per layer type
    per_kind = {}
    for ell, kind in enumerate(kinds):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        layers.prefill_chunked(kind, inps[ell], bufs[ell], w.chunk)
        ev1.record()
        per_kind.setdefault(kind, []).append((ev0, ev1))
    torch.cuda.synchronize()
    layer_ms = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in per_kind.items()}
    win, sel = csa_keys_per_query(S, w.W, w.m, w.k)
    t = np.arange(S, dtype=np.int64)
    hkeys = np.minimum(t + 1, w.W) + (t + 1) // w.m_hca
    fl = {"csa": attend_flops((win + sel).sum(), w.H, w.D) + index_flops(S, w.m, w.nI, w.cI),
          "hca": attend_flops(hkeys.sum(), w.H, w.D),
          "sliding": attend_flops(win.sum(), w.H, w.D)}
    total = sum(fl[k] for k in kinds)
    del inps, bufs
    return {"workload": w.name, "layer_types": kinds, "chunk": w.chunk,
            "query_tokens_per_s": S / wall, "ms_per_step": wall * 1e3,
            "layer_ms": layer_ms,
            "alg_flops_per_step": total, "TFLOP/s": total / wall / 1e12,
            "mfma_frac_whole_step": total / wall / PEAK_BF16,
            "inputs": "device-generated N(0,1), torch Philox, seeded per layer"}


# ----------------------------------------------------------------------------- CPU oracle

def cpu_baseline(n_sample=640):
    """The fp64 oracle on this host: full pooling of all 8192 tokens plus index / top-k /
    attention for n_sample queries spread over the sequence; extrapolated to all queries."""
    import oracle
    import workloads as W

    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = 1
    w = W.workload(2)
    S = w.S
    inp = W.layer_inputs(w, 0, names=["kv", "gate", "k_idx", "g_idx"])
    f = {k: W.to_f64(inp[k]) for k in ("kv", "gate", "k_idx", "g_idx")}
    t0 = time.perf_counter()
    pool = oracle.csa_compress(f["kv"], f["gate"], inp["bias"], w.m, True, w.r, w.base)
    k_pool = oracle.csa_compress(f["k_idx"], f["g_idx"], inp["bias_idx"], w.m, True, 0)
    kv_win = oracle.swa_concat(f["kv"], [0], w.r, w.base)
    t_full = time.perf_counter() - t0
    rows = np.linspace(0, S - 1, n_sample).astype(int)
    N = pool.shape[1]
    t1 = time.perf_counter()
    for t in rows:
        qi = W.to_f64(W.activation_rows(w, 0, "q_idx", [t]))
        wi = W.activation_rows(w, 0, "w_idx", [t])
        idx, _ = oracle.csa_index_topk(qi[None], wi[None], k_pool, [t], [N], w.m, w.k)
        q = W.to_f64(W.activation_rows(w, 0, "q", [t]))
        oracle.csa_attend(q[None], kv_win, [0], pool, idx, inp["sink"], [t], w.W, w.r, w.base)
    t_rows = time.perf_counter() - t1
    est = t_full + t_rows / n_sample * S
    return {"value": S / est, "unit": "query-tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"S=8192 CSA layer: pooling + window rotation of all tokens, index/top-k/"
                      f"attention for {n_sample} of {S} queries (evenly spaced), extrapolated; "
                      f"{t_full + t_rows:.1f} s measured",
            "seconds_measured": t_full + t_rows}


# ----------------------------------------------------------------------------- main

def run_oproj(torch, steps, warmup):
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
    for _ in range(warmup):
        grouped_out_proj(attn, w_a, w_b, mid, out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        grouped_out_proj(attn, w_a, w_b, mid, out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 2.0 * T * (G * rk * kg + hid * G * rk)
    return {"workload": "grouped_out_proj T=8192: 64x512 -> 8x1024 -> 4096 (bf16)", "ms": ms,
            "alg_flops": flops, "TFLOP/s": flops / ms / 1e9, "bound": "mfma",
            "frac": flops / ms / 1e9 / (PEAK_BF16 / 1e12), "tokens_per_s": T / ms * 1e3}


def run_inproj(torch, steps, warmup):
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
    for _ in range(warmup):
        input_projections("csa", x, w_x, w_lat, **out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        input_projections("csa", x, w_x, w_lat, **out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 2.0 * T * (n_x * hid + n_lat * qr)
    return {"workload": f"input_projections T=8192 CSA: 4096 -> {n_x} (latent, kv, gate, indexer k/g/w); "
                        f"1024 -> {n_lat} (q, indexer q) (bf16)", "ms": ms,
            "alg_flops": flops, "TFLOP/s": flops / ms / 1e9, "bound": "mfma",
            "frac": flops / ms / 1e9 / (PEAK_BF16 / 1e12), "tokens_per_s": T / ms * 1e3}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true", help="skip the HCA / decode workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", choices=["csa_prefill", "hca_prefill", "csa_decode", "stack", "oproj", "inproj"],
                    default=None,
                    help="run one workload alone (for profiling); prints its figures only")
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
    if args.only in ("hca_prefill", "csa_decode", "stack", "oproj", "inproj"):
        fn = {"hca_prefill": run_hca_prefill, "csa_decode": run_decode,
              "stack": run_stack, "oproj": run_oproj, "inproj": run_inproj}[args.only]
        print(json.dumps({"only": args.only, **fn(torch, args.steps, args.warmup)}), flush=True)
        return
    w, wall, kern = run_csa_prefill(torch, args.steps, args.warmup)
    if args.only == "csa_prefill":
        print(json.dumps({"only": args.only, "query_tokens_per_s": w.S / wall,
                          "ms_per_step": wall * 1e3, "kernels": kern}), flush=True)
        return
    extra = {}
    if not args.no_extra:
        extra["hca_prefill"] = run_hca_prefill(torch, max(3, args.steps // 4), 1)
        torch.cuda.empty_cache()
        extra["csa_decode"] = run_decode(torch, args.steps, args.warmup)
        torch.cuda.empty_cache()
        extra["stack8_prefill"] = run_stack(torch, max(2, args.steps // 5), 1)
        torch.cuda.empty_cache()
        extra["grouped_out_proj"] = run_oproj(torch, args.steps, args.warmup)
        extra["input_projections"] = run_inproj(torch, args.steps, args.warmup)
        torch.cuda.empty_cache()
    att = kern["csa_attend"]
    src = kernel_hash("attend_mfma.hip", "common.h")
    traffic = load_traffic("csa_attend", src)
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
        "roofline": {"kernel": "csa_attend", "bound": "mfma",
                     "achieved": att["TFLOP/s"], "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                     "frac": att["frac"], "traffic": traffic,
                     "alg_flops_per_launch": att["alg_flops"], "launch_ms": att["ms"],
                     "source_hash": src},
        "kernels": kern,
        "workloads": extra,
    }
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline()
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

"""Helpers for the GPU parity tests: device transfer, tolerances, top-k comparison."""
from __future__ import annotations

import numpy as np

import workloads as W

# Tolerances on attention-like outputs: |d| <= TOL * max|ref| over the whole output tensor.
TOL = {"bf16": 2e-2, "fp32": 1e-5}
TOPK_REL_BAND = 1e-4


def torch_dtype(dt: str):
    import torch

    return torch.bfloat16 if dt == "bf16" else torch.float32


def dev(a: np.ndarray, device="cuda"):
    """Storage-encoded numpy array -> contiguous device tensor."""
    import torch

    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def host(t) -> np.ndarray:
    """Device tensor -> fp64 numpy (exact for bf16 / fp32 values)."""
    import torch

    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


def enc(x64: np.ndarray, dt: str) -> np.ndarray:
    return W.encode(np.asarray(x64, dtype=np.float32), dt)


def assert_close(got, ref, dt: str, what: str, tol=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    tol = TOL[dt] if tol is None else tol
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    assert err <= tol * scale + 1e-30, f"{what}: max|d| {err:.3e} > {tol} * max|ref| {scale:.3e}"
    return err / max(scale, 1e-30)


def assert_bf16_ulp(got, ref, what: str, ulps: float = 1.0):
    """Each bf16 element within `ulps` bf16 ulps of the exact value (fp64 reference), plus an
    absolute floor of 1e-6 * max|ref| for the fp32 accumulation error of results that cancel
    to near zero (the kernels accumulate in fp32, then round once to bf16)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    mag = np.maximum(np.abs(ref), 1e-30)
    ulp = np.exp2(np.floor(np.log2(mag)) - 7)
    floor = 1e-6 * float(np.abs(ref).max()) if ref.size else 0.0
    bad = np.abs(got - ref) > ulps * ulp + floor
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond {ulps} bf16 ulp; " \
        f"worst |d|={float(np.abs(got - ref)[bad].max()):.3e}"


def check_topk_row(gpu_row: np.ndarray, scores: np.ndarray, k: int, what: str) -> int:
    """GPU top-k list of one query against the oracle's scores of all V candidates.

    Valid indices first, then -1; exactly min(k, V) valid, distinct, < V.  The set must equal
    the oracle's (ties to the lower index) except for entries whose score lies within
    TOPK_REL_BAND (relative) of the oracle's k-th score; exact ties are never excused.
    Returns the number of excused swaps.
    """
    V = len(scores)
    kk = min(k, V)
    g = gpu_row[gpu_row >= 0]
    assert len(g) == kk, f"{what}: {len(g)} valid entries, expected {kk}"
    assert np.all(gpu_row[:kk] >= 0) and np.all(gpu_row[kk:] == -1), f"{what}: -1 not at the end"
    assert len(set(g.tolist())) == kk and np.all(g < V), f"{what}: duplicate or invisible entry"
    if kk == 0:
        return 0
    s = np.asarray(scores, dtype=np.float64) + 0.0
    order = np.lexsort((np.arange(V), -s))
    O = set(order[:kk].tolist())
    G = set(g.tolist())
    if G == O:
        return 0
    s_k = s[order[kk - 1]]
    band = TOPK_REL_BAND * abs(s_k)
    diff = G ^ O
    for x in diff:
        exact_tie = s[x] == s_k
        assert abs(s[x] - s_k) <= band and not exact_tie, \
            f"{what}: entry {x} score {s[x]!r} vs k-th {s_k!r} (band {band:.3e})"
    return len(diff) // 2


def check_keys(gpu_keys, ref_keys, dt: str, what: str):
    """Compressed keys computed on the GPU against the oracle's: within one bf16 ulp on the
    bf16 path (storage rounding of an fp32 result), 1e-5 * max|ref| on the fp32 path."""
    if dt == "bf16":
        assert_bf16_ulp(gpu_keys, ref_keys, what)
    else:
        assert_close(gpu_keys, ref_keys, "fp32", what)


def staged_topk_row(gpu_row, q_idx_t, w_idx_t, gpu_keys, k: int, what: str) -> int:
    """Top-k stage on its own: the oracle scores the query against the GPU's compressed keys
    gpu_keys [V, cI] (already held to the oracle's own keys by check_keys), so both sides
    select from the same bf16 values, and the GPU's list must be that selection (ties to the
    lower index; swaps only inside the relative band of the k-th score)."""
    s = oracle_index_scores(q_idx_t, w_idx_t, gpu_keys)
    return check_topk_row(gpu_row, s, k, what)


def oracle_index_scores(q_idx_t, w_idx_t, keys):
    import oracle

    return oracle.index_scores(q_idx_t, w_idx_t, keys)

"""Whole layers on the GPU (the five calls chained) against the CPU oracle's layers.

The oracle models the path's storage types (pool, indexer keys, rotated window in bf16) with
round_intermediates for the bf16 path.  CSA parity is stage-wise: the GPU's pool and indexer
keys are held to the oracle's (one bf16 ulp); the oracle then scores the GPU's indexer keys, so
both sides select from the same values, and the GPU's top-k lists must be that selection
(exact sets except inside the 1e-4 relative band of the k-th score); the oracle's attention
then runs on the GPU's lists, so an excused swap cannot move the output check.  Outputs:
|d| <= tol * max|ref| over the whole output tensor.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_close, check_keys, host, staged_topk_row

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from long_context_sparse_09_amd import layers  # noqa: E402


def _shape(w, S):
    return layers.LayerShape(w.B, S, w.H, w.D, w.r, w.m, w.m_hca, w.nI, w.cI, w.k, w.W, w.base,
                             torch.bfloat16 if w.dtype == "bf16" else torch.float32)


def _run(kind, w, S, layer=0, pos_offset=0):
    inp = W.layer_inputs(w, layer, S=S)
    d = layers.to_device(inp)
    buf = layers.LayerBuffers(_shape(w, S), kinds=(kind,))
    fn = {"csa": layers.csa_layer, "hca": layers.hca_layer, "sliding": layers.sliding_layer}[kind]
    if kind == "csa":
        out = fn(d, buf, rope_pos_offset=pos_offset, with_scores=True)
    else:
        out = fn(d, buf, rope_pos_offset=pos_offset)
    torch.cuda.synchronize()
    return inp, buf, host(out)


def _check_csa_stages(f64, w, buf, out, aux, S, dt, what):
    """Stage-wise CSA parity over every query of the layer (see the module docstring)."""
    gpu_keys = host(buf.k_pool)
    check_keys(host(buf.pool), aux["pool"], dt, f"{what} pool")
    check_keys(gpu_keys, aux["k_pool"], dt, f"{what} indexer keys")
    gpu_idx = buf.topk_idx.cpu().numpy()
    for t in range(S):
        V = oracle.n_visible(t, w.m, gpu_keys.shape[1])
        staged_topk_row(gpu_idx[0, t], f64["q_idx"][0, t], f64["w_idx"][0, t], gpu_keys[0, :V],
                        gpu_idx.shape[2], f"{what} t={t}")
    ref = oracle.csa_attend(f64["q"], aux["kv_win"], [0], aux["pool"], gpu_idx, f64["sink"], [0],
                            w.W, w.r, w.base)
    assert_close(out, ref, dt, f"{what} output")


def test_tiny_csa_layer_fp32_full():
    """The tiny fp32 CSA workload in full: every output element, every top-k list."""
    w = W.workload(1)
    inp, buf, out = _run("csa", w, w.S)
    f64 = {k: W.to_f64(v) for k, v in inp.items()}
    _, _, aux = oracle.csa_layer(f64, w)
    _check_csa_stages(f64, w, buf, out, aux, w.S, "fp32", "tiny CSA")


@pytest.mark.parametrize("S", [1100, 263])
def test_csa_layer_bf16(S):
    """Production head shape (64 x 512, rope 64, 64 x 128 indexer, k = 512) at a short S."""
    w = W.workload(2)
    inp, buf, out = _run("csa", w, S)
    f64 = {k: W.to_f64(v) for k, v in inp.items()}
    _, _, aux = oracle.csa_layer(f64, w, round_intermediates=True)
    _check_csa_stages(f64, w, buf, out, aux, S, "bf16", "CSA")


def test_hca_layer_bf16():
    w = W.workload(3)
    S = 1500  # 11 HCA entries + a partial window
    inp, buf, out = _run("hca", w, S, layer=1)
    f64 = {k: W.to_f64(v) for k, v in inp.items()}
    ref, aux = oracle.hca_layer(f64, w, round_intermediates=True)
    assert_close(out, ref, "bf16", "HCA output")


def test_sliding_layer_bf16():
    w = W.workload(2)
    S = 700
    inp, buf, out = _run("sliding", w, S, layer=2)
    f64 = {k: W.to_f64(v) for k, v in inp.items()}
    ref, aux = oracle.hca_layer(f64, w, round_intermediates=True, sliding=True)
    assert_close(out, ref, "bf16", "sliding output")


def test_eq26_shift_invariance_on_gpu():
    """A global position shift leaves the layer output unchanged (eq. 26) on the GPU path too."""
    w = W.workload(2)
    S = 300
    _, _, a = _run("csa", w, S)
    _, _, b = _run("csa", w, S, pos_offset=100_000)
    assert_close(b, a, "bf16", "shifted vs unshifted")

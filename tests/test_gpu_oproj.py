"""Grouped low-rank output projection and the dense product behind it, on the GPU, against
the CPU oracle (reading R22 of the grouped output projection item of "Hybrid attention
(§2.3)").

Cases: the MFMA path at small sizes with a ragged token count (two 256-row tiles, the second
partial), the plain kernel for shapes outside it (fp32, and bf16 with a rank that is not a
multiple of 256), an empty batch, and the full DeepseekV4Config shape (64 heads x 512,
8 groups, rank 1024, hidden 4096) over 8192 tokens, checked on sampled token rows (each row
of the output depends on its own attention row only).

Tolerances: bf16 outputs |d| <= 2e-2 * max|ref| (the path's bf16 bar), and each output element
within 2 bf16 ulps of the exact value plus 2e-3 * max|ref| for fp32 accumulation over up to
8192 terms; the intermediate is compared the same way.  fp32: 1e-5 * max|ref|.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_close, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import long_context_sparse_09_amd as L  # noqa: E402

R = oracle.round_bf16


def _check(got, ref, dt, what):
    assert_close(got, ref, dt, what)
    if dt == "bf16":
        scale = float(np.abs(ref).max())
        mag = np.maximum(np.abs(ref), 1e-30)
        ulp = np.exp2(np.floor(np.log2(mag)) - 7)
        bad = np.abs(got - ref) > 2 * ulp + 2e-3 * scale
        assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond 2 ulp + 2e-3 max|ref|"


def _run(w, T, dt):
    print(f"[oproj] {w.name} T={T} groups={w.o_groups} rank={w.o_rank} hidden={w.hidden}", flush=True)
    inp = W.oproj_inputs(w, T=T)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    mid = torch.empty(T, w.o_groups * w.o_rank, dtype=tdt, device="cuda")
    out = torch.empty(T, w.hidden, dtype=tdt, device="cuda")
    L.grouped_out_proj(dev(inp["attn"]), dev(inp["w_a"]), dev(inp["w_b"]), mid, out)
    torch.cuda.synchronize()
    ref_out, ref_mid = oracle.grouped_out_proj(W.to_f64(inp["attn"]), W.to_f64(inp["w_a"]),
                                               W.to_f64(inp["w_b"]), w.o_groups,
                                               round_intermediate=(dt == "bf16"))
    # the intermediate as stored: compare with the unrounded product
    _, exact_mid = oracle.grouped_out_proj(W.to_f64(inp["attn"]), W.to_f64(inp["w_a"]),
                                           W.to_f64(inp["w_b"]), w.o_groups)
    _check(host(mid), exact_mid, dt, "intermediate")
    _check(host(out), ref_out, dt, "output")


def test_oproj_mfma_path_ragged_tokens():
    w = W.scaled(W.workload(2), H=16, o_groups=4, o_rank=256, hidden=512)
    _run(w, 300, "bf16")


def test_oproj_mfma_path_one_group_and_deep_k():
    w = W.scaled(W.workload(2), H=8, o_groups=1, o_rank=512, hidden=256)
    _run(w, 64, "bf16")


def test_oproj_generic_fp32_tiny_config():
    _run(W.workload(1), 256, "fp32")


def test_oproj_generic_bf16_odd_rank():
    w = W.scaled(W.workload(2), H=4, D=48, o_groups=2, o_rank=96, hidden=80)
    _run(w, 37, "bf16")


def test_oproj_empty_batch():
    w = W.workload(2)
    z = torch.empty(0, w.H, w.D, dtype=torch.bfloat16, device="cuda")
    inp = W.oproj_inputs(W.scaled(w, H=8, o_groups=1, o_rank=256, hidden=256), T=1)
    L.grouped_out_proj(z[:, :8], dev(inp["w_a"]), dev(inp["w_b"]),
                       torch.empty(0, 256, dtype=torch.bfloat16, device="cuda"),
                       torch.empty(0, 256, dtype=torch.bfloat16, device="cuda"))


def test_linear_bt_matches_single_group_projection():
    print("[oproj] linear_bt 300 x 512 x 192", flush=True)
    rng = np.random.default_rng(5)
    x = W.encode(rng.standard_normal((300, 192)).astype(np.float32), "bf16")
    wt = W.encode(rng.standard_normal((512, 192)).astype(np.float32), "bf16")
    y = torch.empty(300, 512, dtype=torch.bfloat16, device="cuda")
    L.linear_bt(dev(x), dev(wt), y)
    _, ref = oracle.grouped_out_proj(W.to_f64(x), W.to_f64(wt)[None], np.eye(512), 1)
    _check(host(y), ref, "bf16", "linear_bt")


SAMPLE = [0, 1, 255, 256, 4095, 4096, 8190, 8191]


def test_oproj_full_config_sampled_rows():
    w = W.workload(2)
    T = w.S
    print(f"[oproj] full: T={T} H={w.H} D={w.D} groups={w.o_groups} rank={w.o_rank} hidden={w.hidden}", flush=True)
    inp = W.oproj_inputs(w, T=T)
    mid = torch.empty(T, w.o_groups * w.o_rank, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(T, w.hidden, dtype=torch.bfloat16, device="cuda")
    L.grouped_out_proj(dev(inp["attn"]), dev(inp["w_a"]), dev(inp["w_b"]), mid, out)
    torch.cuda.synchronize()
    ref_out, ref_mid = oracle.grouped_out_proj(W.to_f64(inp["attn"][SAMPLE]), W.to_f64(inp["w_a"]),
                                               W.to_f64(inp["w_b"]), w.o_groups, round_intermediate=True)
    _, exact_mid = oracle.grouped_out_proj(W.to_f64(inp["attn"][SAMPLE]), W.to_f64(inp["w_a"]),
                                           W.to_f64(inp["w_b"]), w.o_groups)
    _check(host(mid[SAMPLE]), exact_mid, "bf16", "intermediate (sampled rows)")
    _check(host(out[SAMPLE]), ref_out, "bf16", "output (sampled rows)")


@pytest.mark.parametrize("M,N", [(1500, 1024), (2048, 2048), (700, 768)])
def test_linear_bt_tile_orders(M, N):
    """Grids whose tile count is a multiple of 8 take the XCD-grouped tile order, including a
    last group of fewer tile rows (1500 x 1024: 6 x 4 tiles); others take row-major ranks
    (700 x 768: 3 x 3).  Every output tile must be written once, with its own values."""
    print(f"[oproj] linear_bt {M} x {N} x 128", flush=True)
    rng = np.random.default_rng(M + N)
    x = W.encode(rng.standard_normal((M, 128)).astype(np.float32), "bf16")
    wt = W.encode((rng.standard_normal((N, 128)) / np.sqrt(128)).astype(np.float32), "bf16")
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    L.linear_bt(dev(x), dev(wt), y)
    torch.cuda.synchronize()
    _, ref = oracle.grouped_out_proj(W.to_f64(x), W.to_f64(wt)[None], np.eye(N), 1)
    _check(host(y), ref, "bf16", f"linear_bt {M}x{N}")

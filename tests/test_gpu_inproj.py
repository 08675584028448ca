"""Input projections of an attention layer (the query latent and query, K=V head, compressor
gate, indexer query / key / gate / head weights) on the GPU, against the CPU oracle (readings
R23/R24 of "Hybrid attention (§2.3)" and "DeepseekV4Config": q_lora_rank, index_n_heads,
index_head_dim), and the multi-output product behind them.

Cases: the MFMA path with a ragged token count and a ragged last tile column of the stacked
weight (672 = 2 x 256 + 160 columns), every layer type, fp32 outputs next to bf16 ones, the
plain kernel for widths that are not multiples of 32, the fp32 tiny config, an empty batch,
and the full DeepseekV4Config shape (hidden 4096, q_lora_rank 1024, 64 x 512 query heads,
64 x 128 indexer heads) over 8192 tokens, checked on sampled token rows (each output row
depends on its own token's hidden state only).

Tolerances: bf16 outputs |d| <= 2e-2 * max|ref| (the path's bf16 bar) and each element within
2 bf16 ulps of the exact value plus 2e-3 * max|ref| (fp32 accumulation over up to 4096
terms, then one rounding); q and q_idx are compared with the oracle fed the latent rounded
to bf16, as the path stores it.  fp32 outputs (w_idx, and the fp32 config): 1e-5 * max|ref|.
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


def _check(got, ref, dt, what):
    assert_close(got, ref, dt, what)
    if dt == "bf16":
        scale = float(np.abs(ref).max())
        mag = np.maximum(np.abs(ref), 1e-30)
        ulp = np.exp2(np.floor(np.log2(mag)) - 7)
        bad = np.abs(got - ref) > 2 * ulp + 2e-3 * scale
        assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond 2 ulp + 2e-3 max|ref|"


def _alloc(w, kind, T):
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    e = lambda *s, dt=tdt: torch.empty(*s, dtype=dt, device="cuda")  # noqa: E731
    out = {"c_q": e(T, w.q_rank), "q": e(T, w.H, w.D), "kv": e(T, w.D)}
    if kind != "sliding":
        out["gate"] = e(T, w.D)
    if kind == "csa":
        out.update(q_idx=e(T, w.nI, w.cI), k_idx=e(T, w.cI), g_idx=e(T, w.cI),
                   w_idx=e(T, w.nI, dt=torch.float32))
    return out


def _run(w, kind, T, sample=None):
    print(f"[inproj] {w.name} kind={kind} T={T} hidden={w.hidden} q_rank={w.q_rank} "
          f"H={w.H} D={w.D} nI={w.nI} cI={w.cI}", flush=True)
    inp = W.inproj_inputs(w, kind, T=T)
    out = _alloc(w, kind, T)
    L.input_projections(kind, dev(inp["x"]), dev(inp["w_x"]), dev(inp["w_lat"]), **out)
    torch.cuda.synchronize()
    rows = np.arange(T) if sample is None else np.asarray(sample)
    ws = {n: W.to_f64(inp[n]) for n in W.INPROJ_X_ORDER[kind] + W.INPROJ_LAT_ORDER[kind]}
    ref = oracle.input_projections(W.to_f64(inp["x"][rows]), ws, kind,
                                   round_latent=(w.dtype == "bf16"))
    assert sorted(ref) == sorted(out), (sorted(ref), sorted(out))
    for name, t in out.items():
        got = host(t).reshape(T, -1)[rows]
        dt = "fp32" if t.dtype == torch.float32 else "bf16"
        _check(got, ref[name], dt, name)


def _small(**over):
    base = dict(H=4, D=128, nI=32, cI=64, hidden=256, q_rank=256)
    base.update(over)
    return W.scaled(W.workload(2), **base)


@pytest.mark.parametrize("kind", ["csa", "hca", "sliding"])
def test_inproj_mfma_path_ragged_tokens_and_columns(kind):
    _run(_small(), kind, 300)


def test_inproj_plain_kernel_for_narrow_widths():
    # w_idx 4 wide and k_idx 48 wide: not multiples of 32, the first product runs the plain kernel
    _run(_small(nI=4, cI=48, q_rank=192), "csa", 70)


def test_inproj_fp32_tiny_config():
    for kind in ("csa", "hca", "sliding"):
        _run(W.workload(1), kind, 256)


def test_inproj_empty_batch():
    w = _small()
    inp = W.inproj_inputs(w, "csa", T=1)
    out = _alloc(w, "csa", 0)
    L.input_projections("csa", torch.empty(0, w.hidden, dtype=torch.bfloat16, device="cuda"),
                        dev(inp["w_x"]), dev(inp["w_lat"]), **out)
    torch.cuda.synchronize()


def test_linear_bt_multi_mixed_output_types():
    print("[inproj] linear_bt_multi 300 x (96 bf16 | 64 fp32 | 160 bf16) x 128", flush=True)
    rng = np.random.default_rng(9)
    x = W.encode(rng.standard_normal((300, 128)).astype(np.float32), "bf16")
    wt = W.encode((rng.standard_normal((320, 128)) / np.sqrt(128)).astype(np.float32), "bf16")
    outs = [torch.empty(300, 96, dtype=torch.bfloat16, device="cuda"),
            torch.empty(300, 64, dtype=torch.float32, device="cuda"),
            torch.empty(300, 160, dtype=torch.bfloat16, device="cuda")]
    L.linear_bt_multi(dev(x), dev(wt), outs)
    torch.cuda.synchronize()
    _, ref = oracle.grouped_out_proj(W.to_f64(x), W.to_f64(wt)[None], np.eye(320), 1)
    _check(host(outs[0]), ref[:, :96], "bf16", "segment 0")
    _check(host(outs[1]), ref[:, 96:160], "fp32", "segment 1")
    _check(host(outs[2]), ref[:, 160:], "bf16", "segment 2")


SAMPLE = [0, 1, 255, 256, 4095, 4096, 8190, 8191]


def test_inproj_full_config_sampled_rows():
    w = W.workload(2)
    _run(w, "csa", w.S, sample=SAMPLE)


def test_inproj_single_token_full_shape():
    """One token (a decode step) through the full DeepseekV4Config shapes: a tile row with one
    live row, every other row of the tile outside the buffers."""
    w = W.workload(2)
    _run(w, "csa", 1)


def test_linear_bt_multi_eight_segments():
    print("[inproj] linear_bt_multi 70 x 8 segments x 64", flush=True)
    rng = np.random.default_rng(10)
    widths = [32, 64, 32, 96, 32, 32, 64, 32]
    f32 = [0, 1, 0, 0, 1, 0, 1, 0]
    N = sum(widths)
    x = W.encode(rng.standard_normal((70, 64)).astype(np.float32), "bf16")
    wt = W.encode((rng.standard_normal((N, 64)) / 8.0).astype(np.float32), "bf16")
    outs = [torch.empty(70, n, dtype=torch.float32 if f else torch.bfloat16, device="cuda")
            for n, f in zip(widths, f32)]
    L.linear_bt_multi(dev(x), dev(wt), outs)
    torch.cuda.synchronize()
    _, ref = oracle.grouped_out_proj(W.to_f64(x), W.to_f64(wt)[None], np.eye(N), 1)
    c0 = 0
    for i, (n, f) in enumerate(zip(widths, f32)):
        _check(host(outs[i]), ref[:, c0:c0 + n], "fp32" if f else "bf16", f"segment {i}")
        c0 += n

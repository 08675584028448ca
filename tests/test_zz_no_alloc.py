"""csa_index_topk_noalloc (the indexer with the library's static score scratch) against
csa_index_topk with a caller workspace: identical lists and scores, bit for bit (the same
kernels run on the same inputs), on two calls in a row, the second one smaller, so a call
after a larger one must not read what the earlier call left in the shared array.  A request
beyond the scratch size is refused before anything is enqueued."""
import numpy as np
import pytest

import workloads as W
from gpu_util import dev, enc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import long_context_sparse_09_amd as L  # noqa: E402


def _case(seed, B, T, N_cap, k, q_pos0, n_pool):
    nI, cI, m = 64, 128, 4
    q = enc(W.normal_tensor(seed, 0, "q_idx", (B, T, nI, cI)), "bf16")
    wi = W.normal_tensor(seed, 0, "w_idx", (B, T, nI)).astype(np.float32)
    kp = enc(W.normal_tensor(seed, 0, "k_pool", (B, N_cap, cI)), "bf16")
    i32 = lambda v: torch.tensor(np.asarray(v, dtype=np.int32), device="cuda")  # noqa: E731
    args = (dev(q), dev(wi), dev(kp), i32(q_pos0), i32(n_pool))
    outs = []
    for noalloc in (True, False):
        idx = torch.full((B, T, k), -7, dtype=torch.int32, device="cuda")
        sc = torch.full((B, T, k), -7.0, dtype=torch.float32, device="cuda")
        if noalloc:
            print(f"[noalloc] csa_index_topk_noalloc B={B} T={T} N_cap={N_cap} k={k}", flush=True)
            L.csa_index_topk_noalloc(*args, idx, sc, m)
        else:
            nb = L.csa_index_topk_workspace_size(B, T, N_cap, k)
            ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
            L.csa_index_topk(*args, idx, sc, m, ws)
        torch.cuda.synchronize()
        outs.append((idx.cpu().numpy(), sc.cpu().numpy()))
    (ia, sa), (ib, sb) = outs
    assert np.array_equal(ia, ib), f"lists differ at {np.argwhere(ia != ib)[:4]}"
    assert np.array_equal(sa.view(np.uint32), sb.view(np.uint32)), "scores differ"
    assert (ia >= 0).any(), "the case selects something"


def test_noalloc_matches_workspace_entry_point_twice():
    # first call: prefill-shaped (MFMA scorer, one wave per row selection), 4.9 MB of scores
    _case(61, 2, 300, 2048, 512, [0, 7000], [2048, 1900])
    # second call, smaller: decode-shaped (streaming scorer, block-per-row selection), 144 KB
    _case(62, 4, 1, 9000, 512, [35999, 20000, 3000, 100], [9000, 5000, 750, 25])


def test_noalloc_refuses_requests_beyond_the_scratch():
    B, T, N_cap, k = 1, 4096, 8192, 512  # 128 MiB of scores
    assert L.csa_index_topk_workspace_size(B, T, N_cap, k) > L.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, T, 64, 128, dtype=torch.bfloat16, device="cuda")
    wi = torch.zeros(B, T, 64, dtype=torch.float32, device="cuda")
    kp = torch.zeros(B, N_cap, 128, dtype=torch.bfloat16, device="cuda")
    z = torch.zeros(B, dtype=torch.int32, device="cuda")
    idx = torch.empty(B, T, k, dtype=torch.int32, device="cuda")
    with pytest.raises(L.DSV4Error) as e:
        L.csa_index_topk_noalloc(q, wi, kp, z, z, idx, None, 4)
    assert e.value.status == 2

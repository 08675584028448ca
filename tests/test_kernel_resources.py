"""Register budget of the MFMA kernels, checked at compile time (no GPU needed).

The attention kernel runs ten wavefronts per CU with a 168-register budget per lane; a source
change that pushes the compiler past it spills registers to scratch memory, which measured
about 1.8x slower with identical results (the parity tests cannot see it).  This test compiles
the kernel sources for gfx950 with the compiler's resource-usage remarks and requires zero
scratch bytes for every MFMA kernel."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_sparse_09_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

KERNELS = {  # source file -> mangled-name fragments of kernels that must not use scratch
    "attend_mfma.hip": ["attend_mfma_kernel"],
    "attend_dense.hip": ["attend_dense_kernel"],
    "index_topk.hip": ["index_score_mfma", "index_score_stream", "topk_wave", "topk_radix"],
}


def _usage(src):
    from long_context_sparse_09_amd import build as b

    cmd = [HIPCC, *b.FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c",
           os.path.join(CSRC, src), "-o", os.devnull]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    usage, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            usage[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^]]*\])?: (\d+)", line)
        if m and name:
            usage[name][m.group(1).strip()] = int(m.group(2))
    return usage


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", sorted(KERNELS))
def test_mfma_kernels_use_no_scratch(src):
    usage = _usage(src)
    for frag in KERNELS[src]:
        hits = {n: u for n, u in usage.items() if frag in n}
        assert hits, f"no kernel matching {frag} in {src}"
        for n, u in hits.items():
            assert u.get("ScratchSize", 0) == 0, f"{n}: {u.get('ScratchSize')} scratch bytes per lane"

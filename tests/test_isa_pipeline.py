"""The k loops of the matrix-core GEMM and the weight-gradient GEMM keep
their LDS copies in flight across steps: no `s_waitcnt vmcnt(0)` may sit
directly before an LDS read in those kernels.

Such a wait would drain every outstanding global -> LDS copy (the stages
still being filled as well as the one about to be read), serialising the
pipeline.  The compiler inserts one whenever it cannot prove that the read
stage's copies were already awaited, e.g. when a copy is issued on only some
paths into the loop, or when ordinary loads are in flight next to the LDS
copies.  The check compiles the two sources for gfx950 (host-only, no GPU)
and scans the assembly of every instantiated kernel.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "element_routed_moe_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _assembly(src: str, out: str) -> str:
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-w", "-I" + CSRC, "-S", "--cuda-device-only", os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    return open(out).read()


def _kernels(asm: str, pattern: str):
    for name in re.findall(r"^(_ZN4mlip\S*" + pattern + r"\S+):", asm, re.M):
        i = asm.index(name + ":")
        j = asm.index(".Lfunc_end", i)
        lines = [l.strip() for l in asm[i:j].split("\n") if l.strip() and not l.strip().startswith(";")]
        yield name, lines


def _drains_before_lds_reads(lines):
    return [k for k, l in enumerate(lines[:-1])
            if l.startswith("s_waitcnt") and "vmcnt(0)" in l and lines[k + 1].startswith("ds_read")]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src,pattern,expect", [("gemm.hip", "gemm_kernel", 12), ("gemm.hip", "gemm_pair_kernel", 2),
                                                ("gemm.hip", "gemm_pair_tall_kernel", 2), ("second.hip", "wgrad_kernel", 8)])
def test_no_counter_drain_before_lds_reads(tmp_path, src, pattern, expect):
    asm = _assembly(src, str(tmp_path / (src + ".s")))
    found = list(_kernels(asm, pattern))
    assert len(found) == expect, [n for n, _ in found]
    bad = {name: _drains_before_lds_reads(lines) for name, lines in found}
    bad = {k: v for k, v in bad.items() if v}
    assert not bad, bad
    # every kernel copies global -> LDS directly
    for name, lines in found:
        assert any(l.startswith("global_load_lds_dwordx4") for l in lines), name

"""CPU check of the GEMM kernels' gfx950 assembly (built here from source):
the direct global->LDS loads take their LDS address from M0, which the
kernels set in the same inline-asm statement as each load.  The compiler
treats M0 as reserved and cannot be told about that write, so the kernels
stay correct only while no compiler-generated instruction relies on M0.
This test fails if a change makes the compiler use M0 (dynamic register
indexing, its own LDS-DMA, messages) anywhere in gemm.hip's device code."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# instructions that read M0 without naming it
IMPLICIT_M0 = re.compile(r"\b(s_set_gpr_idx_\w+|s_movrel\w*|v_movrel\w*|s_sendmsg\w*|ds_gws\w*|"
                         r"v_interp\w*|ds_\w+_addtid\w*|s_ttracedata)\b")


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "gemm.s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", out,
           os.path.join(ROOT, "combine_dispatch_amd", "csrc", "gemm.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return open(out).read().splitlines()


def test_m0_is_only_written_by_the_direct_loads(gemm_asm):
    insts = []
    for line in gemm_asm:
        s = line.split(";")[0].strip()
        if s and not s.startswith(".") and not s.endswith(":"):
            insts.append(s)
        elif line.strip().startswith(";;#ASM"):
            insts.append(line.strip())
    n_loads = 0
    for i, s in enumerate(insts):
        if re.search(r"\bm0\b", s):
            assert re.match(r"^s_mov_b32 m0, s\d+$", s), s
        assert not IMPLICIT_M0.search(s), s
        if s.startswith("global_load_lds_") or re.match(r"^buffer_load_\w+.*\blds\b", s):
            n_loads += 1
            # the same asm statement: s_mov_b32 m0, ...; s_nop 0; the load
            assert insts[i - 1] == "s_nop 0" and insts[i - 2].startswith("s_mov_b32 m0,"), insts[i - 3:i + 1]
    assert n_loads > 100  # both GEMM kernels' main loops were compiled

"""Checks on the generated gfx950 code of the direct-load GEMM kernels (CPU
only): nf4f_kernel (y = x W), nf4t_kernel (dx = dy W), bf16f_kernel
(C = A B^T in bf16) and bf16t_kernel (C = A B in bf16).

The kernels' direct global -> LDS loads are inline asm that set M0 without
saving it; that is only correct while the compiler itself uses M0 nowhere in
the kernel.  The kernels must also keep their accumulators in registers: no
scratch access in the main loop."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CSRC = os.path.join(os.path.dirname(__file__), "..", "layer_streamed_nf4_double_amd", "csrc")
KERNELS = {"nf4f_kernel": "gemm_nf4f.hip", "nf4t_kernel": "gemm_nf4t.hip",
           "bf16f_kernel": "gemm_bf16.hip", "bf16t_kernel": "gemm_bf16.hip"}


@pytest.fixture(scope="module", params=sorted(KERNELS))
def asm(request):
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        src = os.path.join(CSRC, KERNELS[request.param])
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", src, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return request.param, open(out).read()


def _kernels(asm):
    """(name, body, metadata) of every instantiation of the kernel (one per
    output form)."""
    kernel, asm = asm
    names = re.findall(r"^(_ZN3lsn%d%sI\w+E):" % (len(kernel), kernel), asm, re.M)
    assert len(names) >= 2, f"{kernel} instantiations not found"
    out = []
    for name in names:
        start = asm.index(f"{name}:")
        body = asm[start:asm.index(".Lfunc_end", start)]
        i = asm.index(f".name:           {name}")
        meta = asm[asm.rindex("- .agpr_count", 0, i):i + 2000]
        out.append((name, body, meta))
    return out


def test_m0_only_in_direct_loads(asm):
    for name, body, _ in _kernels(asm):
        inside = False
        for line in body.splitlines():
            if "ASMSTART" in line:
                inside = True
                continue
            if "ASMEND" in line:
                inside = False
                continue
            code = line.split(";")[0]
            if not inside:
                assert not re.search(r"\bm0\b", code), f"{name}: compiler uses M0: {line.strip()}"
        assert body.count("global_load_lds_dwordx4") >= 10, name


def test_no_scratch_in_main_loop(asm):
    """The instantiations the forward pass uses (fp32 output, split-k partial
    sums) use no scratch at all; the others may spill in their epilogue but
    never between the direct loads of the main loop."""
    for name, body, meta in _kernels(asm):
        if "ILi0E" in name or "ILin1E" in name:  # C_F32, split-k partials
            assert re.search(r"\.private_segment_fixed_size:\s+0\b", meta), f"{name} uses scratch"
        lines = body.splitlines()
        dma = [i for i, l in enumerate(lines) if "global_load_lds" in l]
        loop = lines[dma[0]:dma[-1]]
        assert not any("scratch_" in l for l in loop), f"{name}: scratch access in the main loop"

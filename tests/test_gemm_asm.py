"""Build-level check of the GEMM mainloops (CPU only: hipcc cross-compiles for
gfx950).  The HBM->LDS copies are inline asm, which the compiler does not
count; a compiler-inserted `s_waitcnt vmcnt(0)` inside a mainloop (for example
for a spill reload) would wait for every copy in flight on every K tile.  The
check compiles fng_gemm.hip to assembly and asserts that no basic block holding
the K loop's MFMAs has such a wait or any scratch (spill) access."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "attention_fng_prenorm_amd", "csrc", "fng_gemm.hip")


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "fng_gemm.s"
    cmd = [hipcc, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-I", os.path.join(ROOT, "include"), "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           SRC, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return out.read_text().split("\n")


def _mainloop_blocks(lines):
    """(kernel symbol, block label, instructions) of every basic block that
    holds at least 4 of the 32x32x16 bf16 MFMAs (the K loop bodies)."""
    out = []
    kern, label, ins = None, None, []
    def flush():
        if kern and label and sum("v_mfma_f32_32x32x16_bf16" in x for x in ins) >= 4:
            out.append((kern, label, list(ins)))
    for ln in lines:
        m = re.match(r"^(_ZN3fng11gemm_kernel\S+):", ln)
        if m:
            flush()
            kern, label, ins = m.group(1), None, []
            continue
        if re.match(r"^\.LBB\S+:", ln):
            flush()
            label, ins = ln.split(":")[0], []
            continue
        t = ln.strip()
        if t and not t.startswith(";") and not t.startswith("."):
            ins.append(t)
    flush()
    return out


def test_no_full_wait_or_spill_in_gemm_mainloops(gemm_asm):
    blocks = _mainloop_blocks(gemm_asm)
    kernels = {k for k, _, _ in blocks}
    assert len(kernels) >= 20, "expected the GEMM kernel instantiations in the assembly"
    bad = [(k, b) for k, b, ins in blocks
           if any(re.search(r"vmcnt\(0\)", x) for x in ins) or any(x.startswith("scratch_") for x in ins)]
    assert not bad, f"mainloop blocks with a full memory wait or a spill access: {bad[:5]}"

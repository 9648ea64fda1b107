"""The fp8 forward's tile barrier leaves tile t+2's V loads in flight (s_waitcnt vmcnt(4), then
s_barrier).  That wait is right only if those four loads are the last vector memory instructions
the wavefront issues before the barrier; otherwise it could pass the barrier with the next K
tile's transfers into LDS unfinished.  The order is fixed by the compiler, so this test compiles
fwd_fp8.hip to gfx950 assembly with the library's own flags and checks it before every such
barrier (no GPU needed)."""
import os
import re
import shutil
import subprocess

import pytest

from exact_tiled_attention_15_amd import build

SRC = os.path.join(build.CSRC, "fwd_fp8.hip")
VMEM = re.compile(r"(global_|buffer_|flat_|scratch_)\w+")


def _kernels(asm):
    for m in re.finditer(r"^(_ZN3eta14fwd_fp8_kernel\S+):", asm, re.M):
        end = asm.index(".Lfunc_end", m.end())
        yield m.group(1), asm[m.end():end].splitlines()


@pytest.mark.skipif(not shutil.which(build.HIPCC) and not os.path.exists(build.HIPCC),
                    reason="hipcc is not installed")
def test_v_loads_last_before_partial_wait(tmp_path):
    out = tmp_path / "fwd_fp8.s"
    flags = [f for f in build.COMMON_FLAGS if f != "-fPIC"] + build.EXTRA_FLAGS.get("fwd_fp8.hip", [])
    subprocess.run([build.HIPCC, *flags, "--cuda-device-only", "-S", SRC, "-o", str(out)],
                   check=True, capture_output=True, timeout=600)
    asm = out.read_text()
    sites = 0
    for name, body in _kernels(asm):
        for i, line in enumerate(body):
            if line.strip() != "s_waitcnt vmcnt(4) lgkmcnt(0)" or body[i + 1].strip() != "s_barrier":
                continue
            sites += 1
            vmem = []
            for prev in reversed(body[:i]):
                t = prev.strip()
                if t == "s_barrier":
                    break
                if VMEM.match(t):
                    vmem.append(t.split()[0])
            # instructions in layout order, last first: the V loads of the whole-tile path and of
            # the partial-tile path (each four global_load_dwordx2) must come after everything else
            tail = 0
            for op in vmem:
                if op != "global_load_dwordx2":
                    break
                tail += 1
            assert tail >= 4 and tail % 4 == 0, (name, vmem[:12])
            assert len(vmem) > tail, (name, "no K transfers before the V loads")
    # one such barrier in each fp8-Q.K instantiation: 2 head sizes x 2 masks x 4 P.V forms
    assert sites == 16, sites

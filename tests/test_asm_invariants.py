"""Invariants of the generated gfx950 code that the C++ source cannot state.

The streamed sweeps (output and backward) issue their LDS DMAs through an
inline-asm helper that overwrites M0.  That is safe only while those kernels
have no other M0 user, so the compiled code is checked: in every such kernel,
each M0 write is the helper's (followed by its global_load_lds) and nothing
else reads M0.  Compiles the sources with hipcc (CPU only, no GPU needed).
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "entropic_ot_banded_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"

# instructions that read M0 on gfx9 besides the LDS DMA
M0_READERS = re.compile(r"\b(s_movrel|v_movrel|s_sendmsg|ds_gws|ds_ordered|v_interp|s_ttracedata)")


def _device_asm(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O3", "--cuda-device-only", "-S",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", src, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _functions(asm, prefix):
    funcs, name, body = {}, None, []
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):\s*(;.*)?$", line)
        if m:
            name, body = m.group(1), []
            continue
        if name is not None:
            if line.startswith(".Lfunc_end"):
                funcs[name] = body
                name = None
            else:
                body.append(line.strip())
    return {k: v for k, v in funcs.items() if prefix in k}


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src,kernel", [("backward.hip", "bw_sweep_kernel"), ("forward.hip", "output_sweep_kernel")])
def test_lds_dma_helper_is_the_only_m0_user(src, kernel, tmp_path):
    funcs = _functions(_device_asm(os.path.join(CSRC, src), tmp_path), kernel)
    assert funcs, f"no {kernel} instance found"
    for name, body in funcs.items():
        dma = 0
        for i, ins in enumerate(body):
            if re.match(r"s_(mov|add)_\w+\s+m0,", ins):
                # the helper: m0 set, one s_nop, then the DMA
                nxt = [b for b in body[i + 1:i + 4] if b and not b.startswith(";")]
                assert any(b.startswith("global_load_lds") for b in nxt), (name, ins, nxt)
                dma += 1
            assert not M0_READERS.search(ins), (name, ins)
        assert dma > 0, f"{name}: no LDS DMA found"

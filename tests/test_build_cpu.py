"""Properties of the built bf16 and FP8 kernels that their code relies on (CPU only: hipcc
cross-compiles).

The kernels address LDS with plain byte addresses from 0, which holds because they declare no
static LDS: their whole LDS is the dynamic block, which then starts at address 0.
"""
import os
import re
import subprocess

import pytest

from long_sequence_dit_amd import build as lib_build


def _device_asm(tmp_path, src):
    out = tmp_path / "k.s"
    cmd = [lib_build.HIPCC] + [f for f in lib_build.COMMON if f != "-fPIC"] + [
        "-x", "hip", "-S", "--cuda-device-only", os.path.join(lib_build.CSRC, src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        pytest.skip("hipcc unavailable: %s" % res.stderr[-300:])
    return out.read_text()


@pytest.mark.parametrize("src,kernel,count", [("attn_fwd_bf16.hip", "fwd_bf16_kernel", 2),  # D = 64, 128
                                              ("attn_fwd_fp8.hip", "fwd_fp8_kernel", 1)])
def test_forward_kernels_have_no_static_lds(tmp_path, src, kernel, count):
    asm = _device_asm(tmp_path, src)
    blocks = re.findall(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", asm, re.S)
    names = [n for n, _ in blocks if kernel in n]
    assert len(names) == count, names
    for name, body in blocks:
        if kernel in name:
            m = re.search(r"\.amdhsa_group_segment_fixed_size (\d+)", body)
            assert m and int(m.group(1)) == 0, (name, m and m.group(0))
            assert re.search(r"\.amdhsa_private_segment_fixed_size 0\b", body), name  # no scratch either

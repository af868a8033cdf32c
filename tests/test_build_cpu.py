"""Properties of the built bf16 kernel that its code relies on (CPU only: hipcc cross-compiles).

The kernel addresses LDS with plain byte addresses from 0, which holds because it declares no
static LDS: its whole LDS is the dynamic block, which then starts at address 0.
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


def test_bf16_kernel_has_no_static_lds(tmp_path):
    asm = _device_asm(tmp_path, "attn_fwd_bf16.hip")
    blocks = re.findall(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", asm, re.S)
    names = [n for n, _ in blocks if "fwd_bf16_kernel" in n]
    assert len(names) == 2, names  # D = 64 and D = 128
    for name, body in blocks:
        if "fwd_bf16_kernel" in name:
            m = re.search(r"\.amdhsa_group_segment_fixed_size (\d+)", body)
            assert m and int(m.group(1)) == 0, (name, m and m.group(0))
            assert re.search(r"\.amdhsa_private_segment_fixed_size 0\b", body), name  # no scratch either

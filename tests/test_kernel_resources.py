"""Resources of the gfx950 kernels, read from the device assembly of this
repository's own sources (CPU only; hipcc cross-compiles).

- No kernel has a private (scratch) segment: every record stays in
  registers or LDS, and scratch would sit on dependent-latency paths.
- No packed-fp32 VALU forms (v_pk_fma_f32, v_pk_mul_f32, v_pk_add_f32): the
  sources build with that feature switched off."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from speculative_sampling_verification_vocab_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    tmp = tmp_path_factory.mktemp("asm")
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]

    def one(src):
        out = os.path.join(str(tmp), os.path.basename(src) + ".s")
        subprocess.check_call([B.HIPCC, *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"),
                               "-o", out, src], stderr=subprocess.DEVNULL)
        return os.path.basename(src), open(out).read()

    with ThreadPoolExecutor(4) as ex:
        return dict(ex.map(one, B.sources()))


def test_every_kernel_has_no_private_segment(device_asm):
    kernels = 0
    for name, asm in device_asm.items():
        for m in re.finditer(r"\.name:\s+(\S+)\s*\n(?:.*\n)*?\s+\.private_segment_fixed_size:\s+(\d+)", asm):
            kernels += 1
            assert int(m.group(2)) == 0, (name, m.group(1), m.group(2))
    assert kernels > 40


def test_no_packed_fp32_valu(device_asm):
    for name, asm in device_asm.items():
        assert not re.search(r"\bv_pk_(fma|mul|add)_f32\b", asm), name


def test_shortlist_head_fits_three_blocks_per_cu(device_asm):
    # Three 4-wave blocks per CU: LDS (53.4 KB each) allows three, and the
    # register file must too (512 per SIMD lane / 3 waves, in units of 8).
    asm = device_asm["sv_head.hip"]
    found = 0
    for m in re.finditer(r"\.name:\s+(_ZN\S*head_mfma_kernel\S*)\s*\n(?:.*\n)*?\s+\.vgpr_count:\s+(\d+)", asm):
        found += 1
        assert int(m.group(2)) <= 168, (m.group(1), m.group(2))
    assert found == 2

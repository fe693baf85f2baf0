"""CPU checks on the gfx950 code the kernels compile to (no GPU needed).

* Only the matrix-core shapes the kernels are written for appear: bf16
  v_mfma_f32_16x16x32_bf16 and v_mfma_f32_16x16x16_bf16, fp32
  v_mfma_f32_16x16x4_f32.
* No 16x16x16 reads a 16x16x32 result as its accumulator within 5 wait states
  (that pair is not interlocked by gfx950 and was seen to read stale
  accumulators), and no VALU instruction reads a matrix-core result before
  its measured latency.
* No source applies __builtin_bit_cast to one element of a vector value: the
  device compiler was seen to read element 0 for every index in that form.
"""
from __future__ import annotations

import os
import re
import shutil

import pytest

from gated_delta_rule_92_amd import build as kbuild
from tests import isa_hazards

HIP_SOURCES = [s for s in kbuild.SOURCES if s.endswith(".hip")]
ALLOWED_MFMA = {"v_mfma_f32_16x16x32_bf16", "v_mfma_f32_16x16x16_bf16", "v_mfma_f32_16x16x4_f32"}

pytestmark = pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc") and shutil.which("hipcc") is None,
                                reason="hipcc not available")


@pytest.fixture(scope="module", params=HIP_SOURCES)
def asm(request):
    src = os.path.join(kbuild.CSRC, request.param)
    flags = [f for f in kbuild.COMMON_FLAGS if f not in ("-fPIC",)]
    return request.param, isa_hazards.compile_to_asm(src, flags, kbuild.hipcc())


def test_only_known_mfma_shapes(asm):
    name, text = asm
    used = set(re.findall(r"^\s*(v_mfma_\w+)", text, flags=re.M))
    assert used <= ALLOWED_MFMA, f"{name}: unexpected matrix-core shapes {sorted(used - ALLOWED_MFMA)}"


def test_no_unpadded_mfma_result_reads(asm):
    name, text = asm
    bad = {fn: p for fn, p in isa_hazards.scan_asm(text).items() if p}
    assert not bad, f"{name}: {bad}"


BITCAST_ELEMENT = re.compile(r"__builtin_bit_cast\(\s*[^,()]+,\s*[A-Za-z_][\w\.]*(\[[^\]]*\]|\.[xyzw])+\s*\)")


@pytest.mark.parametrize("src", sorted(f for f in os.listdir(kbuild.CSRC) if f.endswith((".hip", ".h", ".cpp"))))
def test_no_bit_cast_of_vector_element(src):
    text = open(os.path.join(kbuild.CSRC, src)).read()
    hits = [m.group(0) for m in BITCAST_ELEMENT.finditer(text)]
    assert not hits, f"{src}: {hits}"

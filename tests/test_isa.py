"""Instruction-level checks of the gfx950 code built from csrc/dq4.hip (CPU only).

The separate rounding of the scale multiply and the offset add, and of the
value product before its conversion, is what the bitwise contract rests on
(bitsandbytes issue "Fuse nested scale reconstruction into SM103 4-bit
dequantization", section "Correctness requirements").  These checks read the
AMD assembly of this library's own build and require:
  * no fused or mixed multiply-add of any kind (v_fma*, v_fmac*, v_mad*,
    v_mac*, v_fma_mix*, v_mad_mix*, v_dot*), so every product is rounded to
    FP32 on its own;
  * no packed FP32 arithmetic (v_pk_*_f32) and no round-toward-zero FP16 pack
    (v_cvt_pkrtz_f16_f32);
  * every kernel runs in round-to-nearest-even with FP32 and FP16 subnormals
    kept (float_round_mode 0, float_denorm_mode 3).
Integer multiply-adds (v_mad_u64_u32 and similar) are address arithmetic and
allowed.
"""
import re
import tempfile

import pytest

from block_wise_bit_amd import build as dq4_build

FORBIDDEN = re.compile(
    r"\b(v_fma\w*|v_fmac\w*|v_mad_f\w*|v_mad_legacy\w*|v_mad_mix\w*|v_mac_\w*|v_dot\w*|"
    r"v_pk_fma_f32|v_pk_mul_f32|v_pk_add_f32|v_cvt_pkrtz\w*)\b")


@pytest.fixture(scope="module")
def asm():
    with tempfile.TemporaryDirectory() as d:
        return dq4_build.device_assembly(d)


def _kernel_bodies(asm):
    bodies = {}
    for m in re.finditer(r"^(_Z\w+):.*?$(.*?)^\s*s_endpgm", asm, flags=re.M | re.S):
        bodies[m.group(1)] = m.group(2)
    return bodies


def test_kernels_present(asm):
    names = list(_kernel_bodies(asm))
    assert sum("dq4_tile_kernel" in n for n in names) == 3
    assert sum("dq4_elem_kernel" in n for n in names) == 3


def test_no_fused_or_packed_fp_instructions(asm):
    for name, body in _kernel_bodies(asm).items():
        code = "\n".join(l.split(";")[0] for l in body.splitlines())
        found = sorted(set(FORBIDDEN.findall(code)))
        assert not found, f"{name}: {found}"
        assert "v_mul_f32" in code and "v_add_f32" in code, name


def test_ieee_float_modes(asm):
    for key in ("float_round_mode_32", "float_round_mode_16_64"):
        vals = re.findall(r"\.amdhsa_%s (\d+)" % key, asm)
        assert vals and all(v == "0" for v in vals), (key, vals)
    for key in ("float_denorm_mode_32", "float_denorm_mode_16_64"):
        vals = re.findall(r"\.amdhsa_%s (\d+)" % key, asm)
        assert vals and all(v == "3" for v in vals), (key, vals)


def test_no_scratch(asm):
    """The scale lives in registers: no private (scratch) segment is used."""
    vals = re.findall(r"\.amdhsa_private_segment_fixed_size (\d+)", asm)
    assert vals and all(v == "0" for v in vals)

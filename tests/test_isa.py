"""Instruction-level checks of the gfx950 code built from csrc/dq4.hip (CPU only).

The separate rounding of the scale multiply and the offset add, and of the
value product before its conversion, is what the bitwise contract rests on
(bitsandbytes issue "Fuse nested scale reconstruction into SM103 4-bit
dequantization", section "Correctness requirements").  These checks read the
AMD assembly of this library's own build and require:
  * no fused or mixed multiply-add of any kind (v_fma*, v_fmac*, v_mad*,
    v_mac*, v_fma_mix*, v_mad_mix*, v_dot*), so every product is rounded to
    FP32 on its own.  One exception: the out_prod kernel for a single dst row
    (out_prod_direct_kernel<1, 2, *>) accumulates b * W + acc with v_fmac_f32
    on the vector unit, where the other out_prod kernels fuse that product
    and sum inside the matrix instructions; its W is still the separate,
    rounded v_mul_f32 of the decode;
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
    return dq4_build.kernel_bodies(asm)


def test_kernels_present(asm):
    names = list(_kernel_bodies(asm))
    for kernel, count in (("dq4_tile_kernel", 3), ("dq4_elem_kernel", 3),
                          ("dq4_value_tile_kernel", 3), ("dq4_value_elem_kernel", 3),
                          ("dq4_scale_codes_kernel", 1), ("dq4_add_offset_kernel", 1),
                          ("zero_fill_kernel", 1), ("int8_prep_kernel", 1),
                          ("out_prod_fused_kernel", 8), ("out_prod_direct_kernel", 28),
                          ("out_prod_reduce_kernel", 1), ("src1_transpose_kernel", 1),
                          ("out_prod_zero_kernel", 1), ("dq4_memory_twin_kernel", 1),
                          ("dq4_shift_tile_kernel", 23)):
        assert sum(kernel in n for n in names) == count, kernel


def test_no_fused_or_packed_fp_instructions(asm):
    for name, code in _kernel_bodies(asm).items():
        found = set(FORBIDDEN.findall(code))
        if re.search(r"out_prod_direct_kernelILi1ELi2E", name):  # the vector-unit row
            assert found == {"v_fmac_f32_e32"} or found == {"v_fmac_f32_e32", "v_fma_f32"}, \
                (name, found)
            found = set()
        assert not found, f"{name}: {sorted(found)}"
        if "add_offset" in name or "reduce" in name:
            assert "v_add_f32" in code, name
        elif "src1_transpose" in name:  # a bit copy of src1: no FP32 arithmetic at all
            assert not re.search(r"\bv_(mul|add|sub|fma\w*|mac)_f32", code), name
        elif "zero_fill" not in name and "zero_kernel" not in name and "memory_twin" not in name:
            assert "v_mul_f32" in code, name
        if ("dq4_tile_kernel" in name or "dq4_elem_kernel" in name or "out_prod_fused" in name
                or "out_prod_direct" in name):
            assert "v_add_f32" in code, name   # the scale is rebuilt in the fused kernels
        if "out_prod_fused" in name or "out_prod_direct" in name:  # FP32 matrix cores only
            if re.search(r"out_prod_direct_kernelILi\dELi2E", name):  # the vector-unit row
                want = set()
            elif re.search(r"out_prod_direct_kernelILi\dELi1E", name):  # the 4-row sets
                want = {"v_mfma_f32_4x4x1_16b_f32"}
            elif "kernelILi16E" in name or "out_prod_direct" in name:
                want = {"v_mfma_f32_16x16x4_f32"}
            else:
                want = {"v_mfma_f32_32x32x2_f32"}
            assert set(re.findall(r"\bv_mfma\w*", code)) == want, name


def test_kernel_digests_written_by_build():
    """build() records the instruction digest of every kernel next to the
    library, so a measurement can be tied to the exact code it ran."""
    import json
    import os
    from libs import ensure_hip_library
    ensure_hip_library()
    if not os.path.exists(dq4_build.KERNEL_DIGESTS):
        dq4_build.build()
    with open(dq4_build.KERNEL_DIGESTS) as fh:
        digests = json.load(fh)
    assert any("dq4_tile_kernelILi1" in k for k in digests)
    assert all(len(v) == 16 for v in digests.values())


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


def test_tile_kernels_stream_their_memory_traffic(asm):
    """The vector paths write every output unit with a 16-byte buffer store
    marked nt and sc1 (the measured-fastest store policy on MI355X), and no
    other kind of 16-byte store appears in them; so does their memory twin.  The packed data is read
    with non-temporal loads for FP16/BF16 output (instantiations 1 and 2) and
    with plain loads for FP32 output (instantiation 0), as measured fastest."""
    for name, code in _kernel_bodies(asm).items():
        if ("dq4_tile_kernel" not in name and "dq4_value_tile_kernel" not in name
                and "dq4_memory_twin_kernel" not in name):
            continue
        stores = re.findall(r"^\s*(buffer_store_dwordx4|global_store_dwordx4)\b(.*)$", code,
                            re.M)
        assert stores, name
        for op, operands in stores:
            assert op == "buffer_store_dwordx4", (name, op)
            flags = set(operands.split())
            assert {"nt", "sc1"} <= flags and "sc0" not in flags, (name, operands)
        packed = re.findall(r"^\s*global_load_(?:dword|ushort)\b(.*)$", code, re.M)
        assert packed, name
        if "ILi0E" in name:
            assert not any(" nt" in p for p in packed), name
        else:
            assert any(" nt" in p for p in packed), name

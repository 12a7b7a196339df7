// dq4_device.h -- pieces shared by the library's HIP sources (internal; not
// part of the C ABI).  Everything here keeps the FP32 operation order of the
// bitsandbytes issue "Fuse nested scale reconstruction into SM103 4-bit
// dequantization" (section "Correctness requirements"): every multiply and
// add is a separately rounded FP32 operation, and every conversion to FP16 or
// BF16 is one IEEE round-to-nearest-even step of an FP32 value.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

#include "dq4.h"

#pragma clang fp contract(off)

namespace dq4 {

constexpr int kNestedLog2 = 8;  // 256 outer blocks per nested absmax
// Largest element count an entry point accepts: far beyond any device's
// memory, and small enough that index and tile arithmetic stays in int64.
constexpr int64_t kMaxElems = int64_t{1} << 62;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Scale of one outer block: a rounded multiply, then a rounded add.
__device__ __forceinline__ float block_scale(float scale_codebook_value, float absmax,
                                             float offset)
{
    const float t = scale_codebook_value * absmax;
    return t + offset;
}

// The FP32 product must be rounded to FP32 before it is converted: without
// this fence the compiler folds "multiply, then convert to FP16" into one
// mixed-precision fused multiply-add (v_fma_mix*), which rounds the exact
// product once, straight to FP16 -- a different result in about one element
// in 20 000.  The empty asm makes the FP32 value opaque; it emits nothing.
__device__ __forceinline__ float rounded_fp32(float x)
{
    __asm__("" : "+v"(x));
    return x;
}

__device__ __forceinline__ _Float16 to_f16(float x)
{
    return static_cast<_Float16>(rounded_fp32(x));  // IEEE round to nearest even
}

__device__ __forceinline__ __bf16 to_bf16(float x)
{
    return static_cast<__bf16>(rounded_fp32(x));    // IEEE round to nearest even
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi)
{
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, to_f16(lo))) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, to_f16(hi))) << 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, to_bf16(lo))) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, to_bf16(hi))) << 16);
}

// The vector paths work in "units": the elements one lane turns into one
// 16-byte store.  A unit is 8 elements (one packed dword) for FP16/BF16 output
// and 4 elements (one packed 16-bit word) for FP32 output, so that every store
// instruction of a wavefront writes 64 x 16 contiguous bytes for every output
// type.  Since units start on multiples of 4 elements and blocksize >= 32,
// the elements of a unit share one outer block.
template <int OUT>
struct Unit {
    static constexpr int kElems = OUT == DQ4_F32 ? 4 : 8;
    using Word = typename std::conditional<OUT == DQ4_F32, uint16_t, uint32_t>::type;
};

// Memory policy of the vector paths, by output type (measured on MI355X with
// cold inputs).  With FP16/BF16 output (4 B written per 1 B read) the packed
// loads are non-temporal and tiles sharing a line of scale codes are placed
// on one XCD; each was worth ~0.5 % at 28672 x 8192.  With FP32 output (8 B
// written per 1 B read) both made the kernel slower -- ~13 % together at
// 28672 x 8192 -- so that instantiation uses plain loads in dispatch order.
template <int OUT>
constexpr bool kStreamPolicy = OUT != DQ4_F32;

// Unit u (0 .. kUnits-1) of lane t within a tile of kUnits * 256 units.
// Either way every wavefront load and store instruction covers 64 consecutive
// units.  FP16/BF16: unit u * 256 + t, so a wave's two stores are 4 KiB apart.
// FP32: each wave's units are contiguous, ((t / 64) * kUnits + u) * 64 + t % 64;
// ~3 % faster at 28672 x 8192 for FP32 and neutral for FP16.
template <int OUT, int kUnits>
__device__ __forceinline__ int tile_unit(int u, int t)
{
    if constexpr (kStreamPolicy<OUT>)
        return u * 256 + t;
    else
        return (((t >> 6) * kUnits + u) << 6) + (t & 63);
}

// Address of packed word tile_unit(u, t) of a tile whose first word is p.
template <int OUT, int kUnits, typename Word>
__device__ __forceinline__ const Word *tile_word(const Word *p, int u, int t)
{
    if constexpr (kStreamPolicy<OUT>)
        return p + u * 256 + t;
    else
        return p + tile_unit<OUT, kUnits>(u, t);
}

template <int OUT, typename Word>
__device__ __forceinline__ Word load_packed(const Word *p)
{
    if constexpr (kStreamPolicy<OUT>)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

// Output stores of the vector paths go through a raw buffer resource that
// covers the units of one tile, with two cache-policy bits set: nt (streamed,
// not kept for reuse) and sc1 (device scope).  On MI355X, 16-byte stores with
// nt and sc1 measured ~3 % faster over a whole dequantization than stores with
// nt alone, and sc1 without nt was slower than both.  A raw buffer store also
// drops any access past the resource's byte range instead of writing there.
//
// Dword 3 of the resource: 32-bit data format (bits 18:15 = 4), no index
// stride, no swizzle -- the plain untyped-buffer layout of the gfx9 family.
constexpr int kRawBufferWord3 = 0x00020000;
// Cache-policy immediate of a gfx950 vector memory instruction.
constexpr int kPolicyNT = 2;    // non-temporal
constexpr int kPolicySC1 = 16;  // scope bit 1 (device scope)

// The buffer for n_units 16-byte units of `out` starting at unit u0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t unit_buffer(void *out, int64_t u0,
                                                              uint32_t n_units)
{
    return __builtin_amdgcn_make_buffer_rsrc(static_cast<char *>(out) + u0 * 16, 0,
                                             n_units * 16, kRawBufferWord3);
}

// The decoded FP32 values of one unit, written as output type OUT with one
// 16-byte store at unit `ul` of the buffer.
template <int OUT>
__device__ __forceinline__ void store_unit(__amdgpu_buffer_rsrc_t dst, uint32_t ul,
                                           const float (&v)[Unit<OUT>::kElems])
{
    u32x4 q;
    if constexpr (OUT == DQ4_F32)
        q = __builtin_bit_cast(u32x4, f32x4{v[0], v[1], v[2], v[3]});
    else if constexpr (OUT == DQ4_F16)
        q = u32x4{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]), pack_f16x2(v[4], v[5]),
                  pack_f16x2(v[6], v[7])};
    else
        q = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                  pack_bf16x2(v[6], v[7])};
    __builtin_amdgcn_raw_buffer_store_b128(q, dst, ul * 16, 0, kPolicyNT | kPolicySC1);
}
template <int OUT>
__device__ __forceinline__ void store1(void *out, int64_t j, float v)
{
    if constexpr (OUT == DQ4_F32) {
        static_cast<float *>(out)[j] = v;
    } else if constexpr (OUT == DQ4_F16) {
        static_cast<_Float16 *>(out)[j] = to_f16(v);
    } else {
        static_cast<__bf16 *>(out)[j] = to_bf16(v);
    }
}

// ---------------------------------------------------------------------------
// host-side helpers shared by the entry points (defined in dq4.hip)
// ---------------------------------------------------------------------------
// Output type, blocksize (power of two 32..4096) and nested layout (256).
dq4_status_t validate_layout(int32_t blocksize, int32_t nested_blocksize, int32_t out_dtype,
                             int *log2_block);
// Record a HIP failure for dq4_last_hip_error() and return DQ4_EHIP.
dq4_status_t hip_failed(hipError_t e);
// Compute units of `device` (cached).
int compute_units(int device);
// HIP error code of this thread's last DQ4_EHIP.
int32_t last_hip_error();

}  // namespace dq4

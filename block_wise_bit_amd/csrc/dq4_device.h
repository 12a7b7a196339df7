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

// The decoded FP32 values of unit u, written as output type OUT with a
// streaming 16-byte store (unit u covers elements [u * kElems, ...)).
template <int OUT>
__device__ __forceinline__ void store_unit(void *out, int64_t u,
                                           const float (&v)[Unit<OUT>::kElems])
{
    if constexpr (OUT == DQ4_F32) {
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]},
                                    reinterpret_cast<f32x4 *>(out) + u);
    } else if constexpr (OUT == DQ4_F16) {
        __builtin_nontemporal_store(u32x4{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]),
                                          pack_f16x2(v[4], v[5]), pack_f16x2(v[6], v[7])},
                                    reinterpret_cast<u32x4 *>(out) + u);
    } else {
        __builtin_nontemporal_store(u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                          pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])},
                                    reinterpret_cast<u32x4 *>(out) + u);
    }
}

// One FP32 value written as output type OUT at element index j.
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

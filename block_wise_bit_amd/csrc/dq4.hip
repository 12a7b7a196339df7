// dq4.hip -- nested (double-quantized) block-wise 4-bit dequantization for
// MI355X (gfx950), and the C ABI declared in include/dq4.h.
//
// The operation is the fused nested dequantization of the bitsandbytes issue
// "Fuse nested scale reconstruction into SM103 4-bit dequantization"
// (section "Proposed experiment"): every block scale is rebuilt inside the
// value pass as fl32(fl32(scale_codebook[code] * nested_absmax[group]) +
// offset) and every value is cvt(fl32(codebook4[nibble] * scale)).  Section
// "Correctness requirements" fixes the separate rounding of the multiply and
// the add: contraction is switched off for this whole file (pragma below and
// -ffp-contract=off on the command line), and the build is checked for the
// absence of fused multiply-add instructions in the emitted gfx950 code.
//
// Design (HBM-bound stream; no matrix cores: nothing here is a contraction):
//  * one workgroup of 256 lanes handles tiles of 256 * U packed dwords; lane
//    t takes dword u * 256 + t of the tile, so every load instruction of a
//    wavefront reads 256 contiguous bytes and every store instruction writes
//    64 contiguous 16-byte (FP16/BF16) or 32-byte (FP32) pieces;
//  * a dword holds 8 elements, and since blocksize >= 32 and the window
//    starts on a multiple of 8, the 8 elements share one outer block: one
//    code byte, one absmax and one rebuilt scale per lane and dword;
//  * the 256-entry scale codebook and the 16-entry value codebook sit in LDS;
//    a 16-entry table covers 16 distinct banks, so lookups never conflict;
//  * the grid is a few workgroups per compute unit, striding over the tiles
//    so that the LDS tables are filled once per workgroup;
//  * a tile that is not full, and any window that does not meet the
//    alignment of the vector path, goes through a per-element path that
//    computes the same bits.
// No scratch memory: the scale never leaves registers.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>

#include "dq4.h"

#pragma clang fp contract(off)

namespace {

constexpr int kThreads = 256;
constexpr int kNestedLog2 = 8;            // 256 outer blocks per nested absmax
constexpr int kTileDwordsPerLane = 4;     // U
constexpr int kTileElems = kThreads * kTileDwordsPerLane * 8;
constexpr int kBlocksPerCU = 8;

struct Args {
    const uint8_t *packed;
    const uint8_t *scale_codes;
    const float *nested_absmax;
    const float *scale_codebook;
    const float *codebook4;
    void *out;
    int64_t e0;      // global index of the first element of the window
    int64_t count;   // elements in the window
    float offset;
    int log2_block;
};

// Scale of outer block b: a rounded multiply, then a rounded add.
__device__ __forceinline__ float block_scale(const float *lds_scb, const Args &a,
                                             uint32_t code, float absmax)
{
    const float t = lds_scb[code] * absmax;
    return t + a.offset;
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
    const _Float16 l = to_f16(lo);
    const _Float16 h = to_f16(hi);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h)) << 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const __bf16 l = to_bf16(lo);
    const __bf16 h = to_bf16(hi);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h)) << 16);
}

// One element, any alignment: used for partial tiles and unaligned windows.
template <int OUT>
__device__ __forceinline__ void one_element(const Args &a, const float *lds_scb,
                                            const float *lds_cb4, int64_t j)
{
    const int64_t i = a.e0 + j;
    const int64_t b = i >> a.log2_block;
    const float s = block_scale(lds_scb, a, a.scale_codes[b], a.nested_absmax[b >> kNestedLog2]);
    const uint32_t byte = a.packed[i >> 1];
    const uint32_t k = (i & 1) ? (byte >> 4) : (byte & 0xFu);
    const float v = lds_cb4[k] * s;
    if constexpr (OUT == DQ4_F32) {
        static_cast<float *>(a.out)[j] = v;
    } else if constexpr (OUT == DQ4_F16) {
        static_cast<_Float16 *>(a.out)[j] = to_f16(v);
    } else {
        static_cast<__bf16 *>(a.out)[j] = to_bf16(v);
    }
}

__device__ __forceinline__ void load_tables(const Args &a, float *lds_scb, float *lds_cb4)
{
    const int t = threadIdx.x;
    lds_scb[t] = a.scale_codebook[t];
    if (t < 16)
        lds_cb4[t] = a.codebook4[t];
    __syncthreads();
}

// Vector path.  Requires: e0 % 8 == 0, packed + e0/2 4-byte aligned, out
// 16-byte aligned.  Tiles [0, n_full) are full; tile n_full (if any) is the
// partial last tile.
template <int OUT>
__global__ __launch_bounds__(kThreads) void dq4_vec_kernel(Args a, int64_t n_full,
                                                           int64_t n_tiles)
{
    __shared__ float lds_scb[256];
    __shared__ float lds_cb4[16];
    load_tables(a, lds_scb, lds_cb4);

    const int t = threadIdx.x;
    const uint32_t *words = reinterpret_cast<const uint32_t *>(a.packed + (a.e0 >> 1));
    constexpr int U = kTileDwordsPerLane;

    for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
        const int64_t tile_dword0 = tile * (kThreads * U);
        if (tile >= n_full) {
            // partial last tile: element by element
            const int64_t first = tile_dword0 * 8;
            for (int64_t j = first + t; j < a.count; j += kThreads)
                one_element<OUT>(a, lds_scb, lds_cb4, j);
            continue;
        }

        uint32_t w[U];
        uint32_t code[U];
        float absmax[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t d = tile_dword0 + u * kThreads + t;
            w[u] = words[d];
            const int64_t b = (a.e0 + d * 8) >> a.log2_block;
            code[u] = a.scale_codes[b];
            absmax[u] = a.nested_absmax[b >> kNestedLog2];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t d = tile_dword0 + u * kThreads + t;
            const float s = block_scale(lds_scb, a, code[u], absmax[u]);
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = lds_cb4[(w[u] >> (4 * e)) & 0xFu] * s;
            if constexpr (OUT == DQ4_F32) {
                float4 *o = reinterpret_cast<float4 *>(a.out) + d * 2;
                o[0] = make_float4(v[0], v[1], v[2], v[3]);
                o[1] = make_float4(v[4], v[5], v[6], v[7]);
            } else if constexpr (OUT == DQ4_F16) {
                uint4 *o = reinterpret_cast<uint4 *>(a.out) + d;
                *o = make_uint4(pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]),
                                pack_f16x2(v[4], v[5]), pack_f16x2(v[6], v[7]));
            } else {
                uint4 *o = reinterpret_cast<uint4 *>(a.out) + d;
                *o = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
            }
        }
    }
}

// Per-element path for windows the vector path cannot take.
template <int OUT>
__global__ __launch_bounds__(kThreads) void dq4_elem_kernel(Args a)
{
    __shared__ float lds_scb[256];
    __shared__ float lds_cb4[16];
    load_tables(a, lds_scb, lds_cb4);
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t j = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; j < a.count;
         j += stride)
        one_element<OUT>(a, lds_scb, lds_cb4, j);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];
thread_local int32_t t_last_hip_error = 0;

int compute_units(int device)
{
    if (device < 0 || device >= kMaxDevices)
        return 256;
    int cus = g_cu_count[device].load(std::memory_order_relaxed);
    if (cus > 0)
        return cus;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        cus <= 0)
        cus = 256;
    g_cu_count[device].store(cus, std::memory_order_relaxed);
    return cus;
}

int log2_if_pow2(int32_t x)
{
    if (x <= 0 || (x & (x - 1)) != 0)
        return -1;
    int r = 0;
    while ((1 << r) != x)
        ++r;
    return r;
}

dq4_status_t validate_common(int32_t blocksize, int32_t nested_blocksize, int32_t out_dtype,
                             int *log2_block)
{
    if (out_dtype != DQ4_F32 && out_dtype != DQ4_F16 && out_dtype != DQ4_BF16)
        return DQ4_EINVAL;
    const int lb = log2_if_pow2(blocksize);
    if (lb < 5 || lb > 12)
        return DQ4_EUNSUPPORTED;
    if (nested_blocksize != (1 << kNestedLog2))
        return DQ4_EUNSUPPORTED;
    *log2_block = lb;
    return DQ4_OK;
}

dq4_status_t hip_failed(hipError_t e)
{
    t_last_hip_error = static_cast<int32_t>(e);
    (void)hipGetLastError();  // the failure is reported through the status code
    return DQ4_EHIP;
}

template <int OUT>
dq4_status_t launch_typed(const Args &a, hipStream_t stream)
{
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess)
        return hip_failed(e);
    const int64_t max_grid = static_cast<int64_t>(compute_units(device)) * kBlocksPerCU;

    const bool vec = (a.e0 % 8 == 0) &&
                     (reinterpret_cast<uintptr_t>(a.packed + (a.e0 >> 1)) % 4 == 0) &&
                     (reinterpret_cast<uintptr_t>(a.out) % 16 == 0);
    Args args = a;
    if (vec) {
        const int64_t n_full = a.count / kTileElems;
        const int64_t n_tiles = (a.count + kTileElems - 1) / kTileElems;
        const int64_t grid = n_tiles < max_grid ? n_tiles : max_grid;
        void *params[] = {&args, const_cast<int64_t *>(&n_full), const_cast<int64_t *>(&n_tiles)};
        e = hipLaunchKernel(reinterpret_cast<const void *>(&dq4_vec_kernel<OUT>),
                            dim3(static_cast<uint32_t>(grid)), dim3(kThreads), params, 0, stream);
    } else {
        const int64_t want = (a.count + kThreads - 1) / kThreads;
        const int64_t grid = want < max_grid ? want : max_grid;
        void *params[] = {&args};
        e = hipLaunchKernel(reinterpret_cast<const void *>(&dq4_elem_kernel<OUT>),
                            dim3(static_cast<uint32_t>(grid)), dim3(kThreads), params, 0, stream);
    }
    if (e != hipSuccess)
        return hip_failed(e);
    return DQ4_OK;
}

dq4_status_t launch(const Args &a, int32_t out_dtype, void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (out_dtype) {
    case DQ4_F32:
        return launch_typed<DQ4_F32>(a, s);
    case DQ4_F16:
        return launch_typed<DQ4_F16>(a, s);
    default:
        return launch_typed<DQ4_BF16>(a, s);
    }
}

bool any_null(const void *a, const void *b, const void *c, const void *d, const void *e,
              const void *f)
{
    return !a || !b || !c || !d || !e || !f;
}

}  // namespace

extern "C" {

dq4_status_t dq4_nested_dequant(const uint8_t *packed, const uint8_t *scale_codes,
                                const float *nested_absmax, const float *scale_codebook,
                                const float *codebook4, float offset, int64_t n,
                                int32_t blocksize, int32_t nested_blocksize, int32_t out_dtype,
                                void *out, void *stream)
{
    int log2_block = 0;
    const dq4_status_t st = validate_common(blocksize, nested_blocksize, out_dtype, &log2_block);
    if (st != DQ4_OK)
        return st;
    if (n < 0)
        return DQ4_EINVAL;
    if (n == 0)
        return DQ4_OK;
    if (any_null(packed, scale_codes, nested_absmax, scale_codebook, codebook4, out))
        return DQ4_EINVAL;
    const Args a{packed, scale_codes, nested_absmax, scale_codebook, codebook4, out,
                 0, n, offset, log2_block};
    return launch(a, out_dtype, stream);
}

dq4_status_t dq4_nested_dequant_rows(const uint8_t *packed, const uint8_t *scale_codes,
                                     const float *nested_absmax, const float *scale_codebook,
                                     const float *codebook4, float offset, int64_t n_rows,
                                     int64_t n_cols, int64_t r0, int64_t rows, int32_t blocksize,
                                     int32_t nested_blocksize, int32_t out_dtype, void *out,
                                     void *stream)
{
    int log2_block = 0;
    const dq4_status_t st = validate_common(blocksize, nested_blocksize, out_dtype, &log2_block);
    if (st != DQ4_OK)
        return st;
    if (n_rows < 0 || n_cols < 0 || r0 < 0 || rows < 0 || r0 > n_rows || rows > n_rows - r0)
        return DQ4_EINVAL;
    if (n_cols != 0 && n_rows > INT64_MAX / n_cols)
        return DQ4_EINVAL;
    const int64_t count = rows * n_cols;
    if (count == 0)
        return DQ4_OK;
    if (any_null(packed, scale_codes, nested_absmax, scale_codebook, codebook4, out))
        return DQ4_EINVAL;
    const Args a{packed, scale_codes, nested_absmax, scale_codebook, codebook4, out,
                 r0 * n_cols, count, offset, log2_block};
    return launch(a, out_dtype, stream);
}

int64_t dq4_rows_per_block(int64_t n_cols, int64_t elem_bytes, int64_t budget_bytes)
{
    if (n_cols <= 0 || elem_bytes <= 0 || budget_bytes <= 0)
        return 1;
    if (n_cols > INT64_MAX / elem_bytes)
        return 1;
    const int64_t r = budget_bytes / (n_cols * elem_bytes);
    return r < 1 ? 1 : r;
}

const char *dq4_status_string(dq4_status_t status)
{
    switch (status) {
    case DQ4_OK:
        return "DQ4_OK";
    case DQ4_EINVAL:
        return "DQ4_EINVAL: invalid argument";
    case DQ4_EUNSUPPORTED:
        return "DQ4_EUNSUPPORTED: unsupported block layout";
    case DQ4_EHIP:
        return "DQ4_EHIP: kernel launch failed";
    default:
        return "DQ4: unknown status";
    }
}

int32_t dq4_last_hip_error(void)
{
    return t_last_hip_error;
}

}  // extern "C"

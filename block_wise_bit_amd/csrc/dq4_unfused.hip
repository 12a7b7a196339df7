// dq4_unfused.hip -- the unfused three-launch nested dequantization, kept as
// the comparison baseline of the fused kernel in dq4.hip.
//
// This is the existing sequence of the bitsandbytes issue "Fuse nested scale
// reconstruction into SM103 4-bit dequantization" (section "Problem"):
//   launch 1: the uint8 scale codes become FP32 values in a scale buffer,
//             scale[b] = fl32(scale_codebook[code[b]] * nested_absmax[b / 256]);
//   launch 2: the nested offset is added by a separate elementwise pass,
//             scale[b] = fl32(scale[b] + offset);
//   launch 3: the 4-bit values are decoded against the materialized buffer,
//             out[i] = cvt(fl32(codebook4[nibble] * scale[i / blocksize])).
// Every operation is the same separately rounded FP32 step as in the fused
// kernel, so the results are bit-identical; what differs is the extra HBM
// traffic of the FP32 buffer (4 B written, 4 B read + 4 B written, 4 B read
// per block) and two extra launches -- the cost the fusion removes.
//
// Launch 3 has the same tile structure as the fused kernel (256 lanes, 4096
// elements per workgroup, the same load policy per output type, the same
// nt + sc1 output stores), so the comparison measures the fusion and nothing
// else.  (The fused kernel also places tiles that share a line of scale
// codes on one XCD; here each tile reads its own lines of the FP32 buffer,
// so there is nothing to pair.)

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>
#include <mutex>

#include "dq4.h"
#include "dq4_device.h"

#pragma clang fp contract(off)

namespace dq4 {
namespace {

constexpr int kThreads = 256;
constexpr int kDwordsPerLane = 2;
constexpr int kTileDwords = kThreads * kDwordsPerLane;
constexpr int kTileElems = kTileDwords * 8;
constexpr int kMaxTileBlocks = kTileElems / 32 + 1;

// launch 1: scale codes -> FP32 scale buffer
__global__ __launch_bounds__(kThreads) void dq4_scale_codes_kernel(
    const uint8_t *scale_codes, const float *nested_absmax, const float *scale_codebook,
    float *scale, int64_t n_blocks)
{
    const int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (b < n_blocks)
        scale[b] = scale_codebook[scale_codes[b]] * nested_absmax[b >> kNestedLog2];
}

// launch 2: the nested offset, a separate elementwise add
__global__ __launch_bounds__(kThreads) void dq4_add_offset_kernel(float *scale, float offset,
                                                                  int64_t n_blocks)
{
    const int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (b < n_blocks)
        scale[b] = scale[b] + offset;
}

// launch 3, vector path (packed 4-byte aligned, out 16-byte aligned): the
// fused kernel's tile loop with the block scales read from the buffer.
template <int OUT>
__global__ __launch_bounds__(kThreads) void dq4_value_tile_kernel(
    const uint8_t *packed, const float *scale, const float *codebook4, void *out, int64_t n,
    int log2_block, int64_t n_full, int64_t n_tiles)
{
    __shared__ float lds_cb4[16];
    __shared__ float lds_scale[kMaxTileBlocks];
    const int t = threadIdx.x;

    const int64_t edge = n_tiles - n_full;  // 1 or 0
    for (int64_t slot = blockIdx.x; slot < n_tiles; slot += gridDim.x) {
        if (slot != blockIdx.x)
            __syncthreads();  // LDS still holds the previous tile of this workgroup
        // the partial tile, if any, goes to the first slot, as in the fused kernel
        const int64_t tile = slot < edge ? n_full : slot - edge;
        const int64_t d0 = tile * kTileDwords;
        const float cv = t < 16 ? codebook4[t] : 0.0f;
        if (tile >= n_full) {
            if (t < 16)
                lds_cb4[t] = cv;
            __syncthreads();
            for (int64_t i = d0 * 8 + t; i < n; i += kThreads) {
                const uint32_t byte = packed[i >> 1];
                const uint32_t k = (i & 1) ? (byte >> 4) : (byte & 0xFu);
                store1<OUT>(out, i, lds_cb4[k] * scale[i >> log2_block]);
            }
            continue;
        }
        using Word = typename Unit<OUT>::Word;
        constexpr int E = Unit<OUT>::kElems;
        constexpr int kUnits = kDwordsPerLane * 8 / E;  // units per lane and tile
        const Word *wp = reinterpret_cast<const Word *>(packed);
        const int64_t u0 = d0 * 8 / E;
        Word w[kUnits];
        // the fused kernel's load-phase wave priority, for FP16/BF16 as there
        if constexpr (kStreamPolicy<OUT>)
            __builtin_amdgcn_s_setprio(3);
#pragma unroll
        for (int u = 0; u < kUnits; ++u)
            w[u] = load_packed<OUT>(tile_word<OUT, kUnits>(wp + u0, u, t));
        const int64_t b0 = (d0 * 8) >> log2_block;
        const uint32_t r = static_cast<uint32_t>(d0 * 8 - (b0 << log2_block));
        const int n_blocks = static_cast<int>((r + kTileElems - 1) >> log2_block) + 1;
        if (t < n_blocks)
            lds_scale[t] = scale[b0 + t];
        if (t + kThreads < n_blocks)
            lds_scale[t + kThreads] = scale[b0 + t + kThreads];
        if (t < 16)
            lds_cb4[t] = cv;
        if constexpr (kStreamPolicy<OUT>)
            __builtin_amdgcn_s_setprio(0);
        __syncthreads();
        const __amdgpu_buffer_rsrc_t dst = unit_buffer(out, u0, kUnits * kThreads);
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const uint32_t ul = tile_unit<OUT, kUnits>(u, t);
            const float s = lds_scale[(r + ul * E) >> log2_block];
            float v[E];
#pragma unroll
            for (int e = 0; e < E; ++e)
                v[e] = lds_cb4[(static_cast<uint32_t>(w[u]) >> (4 * e)) & 0xFu] * s;
            store_unit<OUT>(dst, ul, v);
        }
    }
}

// launch 3, any alignment: one element per lane, grid-stride
template <int OUT>
__global__ __launch_bounds__(kThreads) void dq4_value_elem_kernel(
    const uint8_t *packed, const float *scale, const float *codebook4, void *out, int64_t n,
    int log2_block)
{
    __shared__ float lds_cb4[16];
    if (threadIdx.x < 16)
        lds_cb4[threadIdx.x] = codebook4[threadIdx.x];
    __syncthreads();
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n;
         i += stride) {
        const uint32_t byte = packed[i >> 1];
        const uint32_t k = (i & 1) ? (byte >> 4) : (byte & 0xFu);
        store1<OUT>(out, i, lds_cb4[k] * scale[i >> log2_block]);
    }
}

template <int OUT>
hipError_t launch_value(const uint8_t *packed, const float *scale, const float *codebook4,
                        void *out, int64_t n, int log2_block, hipStream_t stream)
{
    const bool vec = (reinterpret_cast<uintptr_t>(packed) % 4 == 0) &&
                     (reinterpret_cast<uintptr_t>(out) % 16 == 0);
    if (vec) {
        int64_t n_full = n / kTileElems;
        int64_t n_tiles = (n + kTileElems - 1) / kTileElems;
        const int64_t grid = n_tiles < 0x7FFFFFFF ? n_tiles : 0x7FFFFFFF;
        int lb = log2_block;
        void *params[] = {&packed, &scale, &codebook4, &out, &n, &lb, &n_full, &n_tiles};
        return hipLaunchKernel(reinterpret_cast<const void *>(&dq4_value_tile_kernel<OUT>),
                               dim3(static_cast<uint32_t>(grid)), dim3(kThreads), params, 0,
                               stream);
    }
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess)
        return e;
    const int64_t max_grid = static_cast<int64_t>(compute_units(device)) * 8;
    const int64_t want = (n + kThreads - 1) / kThreads;
    const int64_t grid = want < max_grid ? want : max_grid;
    int lb = log2_block;
    void *params[] = {&packed, &scale, &codebook4, &out, &n, &lb};
    return hipLaunchKernel(reinterpret_cast<const void *>(&dq4_value_elem_kernel<OUT>),
                           dim3(static_cast<uint32_t>(grid)), dim3(kThreads), params, 0, stream);
}

// The three launches over a caller-provided FP32 scale buffer of
// ceil(n / 2^log2_block) values (arguments already validated).
dq4_status_t launch_unfused(const uint8_t *packed, const uint8_t *scale_codes,
                            const float *nested_absmax, const float *scale_codebook,
                            const float *codebook4, float offset, int64_t n, int log2_block,
                            int32_t out_dtype, float *scale_workspace, void *out,
                            hipStream_t s)
{
    int64_t n_blocks = ((n - 1) >> log2_block) + 1;
    const int64_t grid = (n_blocks + kThreads - 1) / kThreads;
    if (grid > 0x7FFFFFFF)
        return DQ4_EINVAL;
    {
        void *params[] = {&scale_codes, &nested_absmax, &scale_codebook, &scale_workspace,
                          &n_blocks};
        const hipError_t e =
            hipLaunchKernel(reinterpret_cast<const void *>(&dq4_scale_codes_kernel),
                            dim3(static_cast<uint32_t>(grid)), dim3(kThreads), params, 0, s);
        if (e != hipSuccess)
            return hip_failed(e);
    }
    {
        void *params[] = {&scale_workspace, &offset, &n_blocks};
        const hipError_t e =
            hipLaunchKernel(reinterpret_cast<const void *>(&dq4_add_offset_kernel),
                            dim3(static_cast<uint32_t>(grid)), dim3(kThreads), params, 0, s);
        if (e != hipSuccess)
            return hip_failed(e);
    }
    hipError_t e;
    switch (out_dtype) {
    case DQ4_F32:
        e = launch_value<DQ4_F32>(packed, scale_workspace, codebook4, out, n, log2_block, s);
        break;
    case DQ4_F16:
        e = launch_value<DQ4_F16>(packed, scale_workspace, codebook4, out, n, log2_block, s);
        break;
    default:
        e = launch_value<DQ4_BF16>(packed, scale_workspace, codebook4, out, n, log2_block, s);
        break;
    }
    if (e != hipSuccess)
        return hip_failed(e);
    return DQ4_OK;
}

// Validation shared by both unfused entry points (the workspace pointer
// aside); sets *log2_block.
dq4_status_t validate_unfused(const uint8_t *packed, const uint8_t *scale_codes,
                              const float *nested_absmax, const float *scale_codebook,
                              const float *codebook4, int64_t n, int32_t blocksize,
                              int32_t nested_blocksize, int32_t out_dtype, const void *out,
                              int *log2_block)
{
    const dq4_status_t st = validate_layout(blocksize, nested_blocksize, out_dtype, log2_block);
    if (st != DQ4_OK)
        return st;
    if (n < 0 || n > kMaxElems)
        return DQ4_EINVAL;
    if (n == 0)
        return DQ4_OK;
    if (!packed || !scale_codes || !nested_absmax || !scale_codebook || !codebook4 || !out)
        return DQ4_EINVAL;
    return DQ4_OK;
}

// ---------------------------------------------------------------------------
// Scratch of dq4_nested_dequant_unfused_noalloc: the FP32 block scales of up
// to DQ4_NOALLOC_MAX_BLOCKS outer blocks (32 MiB), a file-scope device array
// that each GPU the library runs on holds until the process ends.  In host
// code `scratch` only names the symbol; its device address, one per device,
// comes from hipGetSymbolAddress on that device's first call and is the only
// form in which it reaches a kernel or any other HIP call.
// ---------------------------------------------------------------------------
static __device__ __align__(256) float scratch[DQ4_NOALLOC_MAX_BLOCKS];

constexpr int kMaxScratchDevices = 64;
std::atomic<float *> g_scratch[kMaxScratchDevices];
std::mutex g_scratch_mutex;

// This device's address of `scratch` (looked up once per device).
dq4_status_t scratch_on_current_device(float **ptr)
{
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess)
        return hip_failed(e);
    if (device < 0 || device >= kMaxScratchDevices)
        return DQ4_EUNSUPPORTED;
    float *p = g_scratch[device].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch[device].load(std::memory_order_relaxed);
        if (!p) {
            void *addr = nullptr;
            e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
            if (e != hipSuccess)
                return hip_failed(e);
            if (!addr)
                return hip_failed(hipErrorInvalidSymbol);
            p = static_cast<float *>(addr);
            g_scratch[device].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return DQ4_OK;
}

}  // namespace
}  // namespace dq4

extern "C" {

int64_t dq4_unfused_workspace_bytes(int64_t n, int32_t blocksize)
{
    if (n <= 0 || n > dq4::kMaxElems || blocksize <= 0)
        return 0;
    return ((n + blocksize - 1) / blocksize) * static_cast<int64_t>(sizeof(float));
}

dq4_status_t dq4_nested_dequant_unfused(const uint8_t *packed, const uint8_t *scale_codes,
                                        const float *nested_absmax,
                                        const float *scale_codebook, const float *codebook4,
                                        float offset, int64_t n, int32_t blocksize,
                                        int32_t nested_blocksize, int32_t out_dtype,
                                        float *scale_workspace, void *out, void *stream)
{
    int log2_block = 0;
    const dq4_status_t st =
        dq4::validate_unfused(packed, scale_codes, nested_absmax, scale_codebook, codebook4, n,
                              blocksize, nested_blocksize, out_dtype, out, &log2_block);
    if (st != DQ4_OK || n == 0)
        return st;
    if (!scale_workspace)
        return DQ4_EINVAL;
    return dq4::launch_unfused(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                               offset, n, log2_block, out_dtype, scale_workspace, out,
                               static_cast<hipStream_t>(stream));
}

dq4_status_t dq4_nested_dequant_unfused_noalloc(const uint8_t *packed,
                                                const uint8_t *scale_codes,
                                                const float *nested_absmax,
                                                const float *scale_codebook,
                                                const float *codebook4, float offset, int64_t n,
                                                int32_t blocksize, int32_t nested_blocksize,
                                                int32_t out_dtype, void *out, void *stream)
{
    int log2_block = 0;
    const dq4_status_t st =
        dq4::validate_unfused(packed, scale_codes, nested_absmax, scale_codebook, codebook4, n,
                              blocksize, nested_blocksize, out_dtype, out, &log2_block);
    if (st != DQ4_OK || n == 0)
        return st;
    if (((n - 1) >> log2_block) + 1 > DQ4_NOALLOC_MAX_BLOCKS)
        return DQ4_ESCRATCH;
    float *scales = nullptr;
    const dq4_status_t sst = dq4::scratch_on_current_device(&scales);
    if (sst != DQ4_OK)
        return sst;
    return dq4::launch_unfused(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                               offset, n, log2_block, out_dtype, scales, out,
                               static_cast<hipStream_t>(stream));
}

}  // extern "C"

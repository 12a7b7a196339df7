// dq4_out_prod_fused.hip -- out_prod with the dequantization fused into an
// FP32 matrix-core GEMM: no dequantized copy of the weight touches HBM.
//
// llama.cpp PR "cuda: out_prod dequantizes a 2D weight in row blocks": the
// row-blocked route (dq4_gemm.hip) dequantizes each block of weight rows to
// an F32 buffer and runs a GEMM on it; the approving review names the fused
// dequant-in-GEMM route as the follow-on.  The sum is the same,
//
//   dst[i][j] = sum_r B[r][i] * W[r][j]     dst: m x n_cols FP32, row-major
//
// but each workgroup decodes the 4-bit weight of its tile straight into LDS
// as the very FP32 values the dequantization kernel writes (bitsandbytes
// issue "Fuse nested scale reconstruction into SM103 4-bit dequantization",
// section "Proposed experiment": W = fl32(codebook4[k] * scale) with scale =
// fl32(fl32(scale_codebook[code] * absmax) + offset)), and feeds them to
// v_mfma_f32_32x32x2_f32.
//
// Design:
//  * a workgroup (4 waves) owns a 64 x 128 tile of dst (64 values of i, the
//    src1 columns; 128 of j, the weight columns) and one split of the rows r;
//    each wave computes a 32 x 64 sub-tile as two 32 x 32 MFMA blocks that
//    share their A operand;
//  * per stage of 16 weight rows every lane decodes 8 consecutive weight
//    elements (one packed dword when n_cols % 8 == 0) with their one or two
//    block scales, and stages 4 src1 values; the global loads of the next
//    stage are issued before the MFMAs of the current one;
//  * when the tiles alone cannot fill the GPU, the rows are split and each
//    split writes its partial tile to the caller's workspace; a second kernel
//    adds the partials in split order.  The result is deterministic for a
//    given device and workspace size.
// The FP32 sum order differs from the blocked route's library GEMM; both are
// within the FP32 summation bound of the exact sum.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "dq4.h"
#include "dq4_device.h"

#pragma clang fp contract(off)

namespace dq4 {
namespace {

constexpr int kThreads = 256;
constexpr int kTileI = 64;          // dst rows (src1 columns) per workgroup
constexpr int kTileJ = 128;         // dst columns (weight columns) per workgroup
constexpr int kStage = 16;          // weight rows per LDS stage
constexpr int kLdsW = kTileJ + 4;   // padded LDS row of decoded weights
constexpr int kLdsB = kTileI + 4;   // padded LDS row of src1 values
constexpr int kTargetGroupsPerCU = 8;
constexpr int64_t kMinRowsPerSplit = 256;

typedef float f32x16 __attribute__((ext_vector_type(16)));

struct FusedArgs {
    const uint8_t *packed;
    const uint8_t *scale_codes;
    const float *nested_absmax;
    const float *scale_codebook;
    const float *codebook4;
    const float *src1;
    float *part;             // dst when there is one split, else splits x m x n_cols
    int64_t n_rows;
    int64_t n_cols;
    int64_t m;
    int64_t ld;
    int64_t rows_per_split;  // a multiple of kStage
    float offset;
    int log2_block;
    int tiles_i;
    int tiles_j;
    int aligned8;            // n_cols % 8 == 0 and packed 4-byte aligned: a lane's 8
                             // elements are one aligned packed dword
};

// What one lane loads from HBM for one stage, before decoding it.
struct StageLoad {
    uint32_t packed4;   // 8 nibbles (aligned8) ...
    uint8_t bytes[8];   // ... or the byte holding each element (otherwise)
    uint32_t code_lo, code_hi;
    float absmax_lo, absmax_hi;
    float b[4];
};

template <bool kSrc1Transposed>
__device__ __forceinline__ void load_stage(const FusedArgs &a, int64_t k0, int64_t k_end,
                                           int64_t i0, int64_t j0, int t, StageLoad &ld)
{
    // weight: row k0 + t / 16, columns j0 + (t % 16) * 8 .. + 7
    const int64_t r = k0 + (t >> 4);
    const int64_t j = j0 + (t & 15) * 8;
    const int lb = a.log2_block;
    ld.code_lo = ld.code_hi = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q)
        ld.bytes[q] = 0;
    ld.absmax_lo = ld.absmax_hi = 0.0f;
    ld.packed4 = 0;
    if (r < k_end && j < a.n_cols) {
        const int64_t e = r * a.n_cols + j;
        const int64_t e_last = e + (min(a.n_cols - j, int64_t{8}) - 1);
        if (a.aligned8) {
            ld.packed4 = *reinterpret_cast<const uint32_t *>(a.packed + (e >> 1));
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q)
                ld.bytes[q] = e + q <= e_last ? a.packed[(e + q) >> 1] : 0;
        }
        const int64_t b_lo = e >> lb, b_hi = e_last >> lb;  // at most two blocks
        ld.code_lo = a.scale_codes[b_lo];
        ld.absmax_lo = a.nested_absmax[b_lo >> kNestedLog2];
        ld.code_hi = a.scale_codes[b_hi];
        ld.absmax_hi = a.nested_absmax[b_hi >> kNestedLog2];
    }
    // src1 values of the stage
    if constexpr (!kSrc1Transposed) {
        // B[r][i] = src1[r * ld + i]: row k0 + t / 16, columns i0 + (t % 16) * 4 .. + 3
        const int64_t rb = k0 + (t >> 4);
        const int64_t ib = i0 + (t & 15) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            ld.b[q] = (rb < k_end && ib + q < a.m) ? a.src1[rb * a.ld + ib + q] : 0.0f;
    } else {
        // B[r][i] = src1[i * ld + r]: column i0 + t / 4, rows k0 + (t % 4) * 4 .. + 3
        const int64_t ib = i0 + (t >> 2);
        const int64_t rb = k0 + (t & 3) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            ld.b[q] = (rb + q < k_end && ib < a.m) ? a.src1[ib * a.ld + rb + q] : 0.0f;
    }
}

template <bool kSrc1Transposed>
__device__ __forceinline__ void decode_stage(const FusedArgs &a, int64_t k0, int64_t k_end,
                                             int64_t j0, int t, const StageLoad &ld,
                                             const float *lds_scb, const float *lds_cb4,
                                             float (*lds_w)[kLdsW], float (*lds_b)[kLdsB])
{
    const int row = t >> 4, col = (t & 15) * 8;
    const int64_t r = k0 + row;
    const int64_t j = j0 + col;
    float v[8];
    if (r < k_end && j < a.n_cols) {
        const int lb = a.log2_block;
        const int64_t e = r * a.n_cols + j;
        const int64_t n_valid = min(a.n_cols - j, int64_t{8});
        const float s_lo = block_scale(lds_scb[ld.code_lo], ld.absmax_lo, a.offset);
        const float s_hi = block_scale(lds_scb[ld.code_hi], ld.absmax_hi, a.offset);
        // position of element e in its block; element e + q is in the next block
        // once off + q reaches the block size
        const uint32_t off = static_cast<uint32_t>(e & ((int64_t{1} << lb) - 1));
        const uint32_t odd = static_cast<uint32_t>(e & 1);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            uint32_t k;
            if (a.aligned8)
                k = (ld.packed4 >> (4 * q)) & 0xFu;
            else
                k = ((odd + q) & 1) ? (ld.bytes[q] >> 4) : (ld.bytes[q] & 0xFu);
            const float s = ((off + q) >> lb) == 0 ? s_lo : s_hi;
            v[q] = q < n_valid ? lds_cb4[k] * s : 0.0f;
        }
    } else {
#pragma unroll
        for (int q = 0; q < 8; ++q)
            v[q] = 0.0f;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
        lds_w[row][col + q] = v[q];
    if constexpr (!kSrc1Transposed) {
        const int br = t >> 4, bc = (t & 15) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            lds_b[br][bc + q] = ld.b[q];
    } else {
        const int bc = t >> 2, br = (t & 3) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            lds_b[br + q][bc] = ld.b[q];
    }
}

template <bool kSrc1Transposed>
__global__ __launch_bounds__(kThreads) void out_prod_fused_kernel(FusedArgs a)
{
    __shared__ float lds_w[kStage][kLdsW];
    __shared__ float lds_b[kStage][kLdsB];
    __shared__ float lds_scb[256];
    __shared__ float lds_cb4[16];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int ti = static_cast<int>(blockIdx.x % static_cast<uint32_t>(a.tiles_i));
    const uint32_t rest = blockIdx.x / static_cast<uint32_t>(a.tiles_i);
    const int tj = static_cast<int>(rest % static_cast<uint32_t>(a.tiles_j));
    const int split = static_cast<int>(rest / static_cast<uint32_t>(a.tiles_j));
    const int64_t i0 = int64_t{ti} * kTileI, j0 = int64_t{tj} * kTileJ;
    const int64_t k_begin = int64_t{split} * a.rows_per_split;
    const int64_t k_end = min(a.n_rows, k_begin + a.rows_per_split);

    lds_scb[t] = a.scale_codebook[t];
    if (t < 16)
        lds_cb4[t] = a.codebook4[t];

    // wave sub-tile: i in [32 wi, 32 wi + 32), j in [64 wj, 64 wj + 64)
    const int wi = wave & 1, wj = wave >> 1;
    const int kl = lane >> 5, cl = lane & 31;
    f32x16 acc0 = {}, acc1 = {};

    StageLoad ld;
    load_stage<kSrc1Transposed>(a, k_begin, k_end, i0, j0, t, ld);
    __syncthreads();  // the codebooks are in LDS
    for (int64_t k0 = k_begin; k0 < k_end; k0 += kStage) {
        decode_stage<kSrc1Transposed>(a, k0, k_end, j0, t, ld, lds_scb, lds_cb4, lds_w, lds_b);
        __syncthreads();
        if (k0 + kStage < k_end)  // next stage's loads fly during this stage's MFMAs
            load_stage<kSrc1Transposed>(a, k0 + kStage, k_end, i0, j0, t, ld);
#pragma unroll
        for (int kk = 0; kk < kStage; kk += 2) {
            const float av = lds_b[kk + kl][32 * wi + cl];
            const float w0 = lds_w[kk + kl][64 * wj + cl];
            const float w1 = lds_w[kk + kl][64 * wj + 32 + cl];
            acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av, w0, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av, w1, acc1, 0, 0, 0);
        }
        __syncthreads();  // LDS is rewritten by the next stage
    }

    // accumulator register v of lane l holds row 8 (v / 4) + 4 (l / 32) + v % 4,
    // column l % 32 of the 32 x 32 block
    float *out = a.part + int64_t{split} * a.m * a.n_cols;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int64_t i = i0 + 32 * wi + 8 * (v >> 2) + 4 * kl + (v & 3);
        const int64_t j = j0 + 64 * wj + cl;
        if (i < a.m) {
            if (j < a.n_cols)
                out[i * a.n_cols + j] = acc0[v];
            if (j + 32 < a.n_cols)
                out[i * a.n_cols + j + 32] = acc1[v];
        }
    }
}

// dst[x] = part[0][x] + part[1][x] + ... in split order
__global__ __launch_bounds__(kThreads) void out_prod_reduce_kernel(const float *part, float *dst,
                                                                   int64_t count, int splits)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t x = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; x < count;
         x += stride) {
        float sum = part[x];
        for (int s = 1; s < splits; ++s)
            sum = sum + part[int64_t{s} * count + x];
        dst[x] = sum;
    }
}

__global__ __launch_bounds__(kThreads) void out_prod_zero_kernel(float *dst, int64_t count)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t x = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; x < count;
         x += stride)
        dst[x] = 0.0f;
}

int64_t ceil_div(int64_t a, int64_t b)
{
    return (a + b - 1) / b;
}

// The split of the rows the fused kernel uses: enough workgroups to fill the
// device, at least kMinRowsPerSplit rows each, and no more partial tiles than
// max_partials (the workspace's capacity).  Returns the rows per split.
int64_t rows_per_split(int64_t n_rows, int64_t tiles, int cus, int64_t max_partials)
{
    int64_t splits = ceil_div(int64_t{kTargetGroupsPerCU} * cus, tiles);
    splits = min(splits, ceil_div(n_rows, kMinRowsPerSplit));
    splits = min(splits, max_partials);
    if (splits < 1)
        splits = 1;
    return ceil_div(ceil_div(n_rows, splits), kStage) * kStage;
}

dq4_status_t grid_size(int64_t count, int device, uint32_t *grid)
{
    int64_t g = ceil_div(count, kThreads);
    const int64_t cap = int64_t{compute_units(device)} * 8;
    *grid = static_cast<uint32_t>(g < cap ? g : cap);
    return DQ4_OK;
}

}  // namespace
}  // namespace dq4

extern "C" {

int64_t dq4_out_prod_fused_workspace_bytes(int64_t n_rows, int64_t n_cols, int64_t m)
{
    if (n_rows <= 0 || n_cols <= 0 || m <= 0 || n_cols > INT64_MAX / m ||
        m * n_cols > INT64_MAX / 4 / 1024)
        return 0;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess)
        return 0;
    const int64_t tiles = dq4::ceil_div(m, dq4::kTileI) * dq4::ceil_div(n_cols, dq4::kTileJ);
    const int64_t rps = dq4::rows_per_split(n_rows, tiles, dq4::compute_units(device), 1024);
    const int64_t splits = dq4::ceil_div(n_rows, rps);
    return splits > 1 ? splits * m * n_cols * 4 : 0;
}

dq4_status_t dq4_out_prod_fused(const uint8_t *packed, const uint8_t *scale_codes,
                                const float *nested_absmax, const float *scale_codebook,
                                const float *codebook4, float offset, int64_t n_rows,
                                int64_t n_cols, int32_t blocksize, int32_t nested_blocksize,
                                const float *src1, int64_t m, int64_t ld_src1,
                                int32_t src1_transposed, float *dst, float *workspace,
                                int64_t workspace_bytes, void *stream)
{
    int log2_block = 0;
    const dq4_status_t st = dq4::validate_layout(blocksize, nested_blocksize, DQ4_F32,
                                                 &log2_block);
    if (st != DQ4_OK)
        return st;
    if (n_rows < 0 || n_cols < 0 || m < 0 || (src1_transposed != 0 && src1_transposed != 1) ||
        workspace_bytes < 0)
        return DQ4_EINVAL;
    if (m == 0 || n_cols == 0)
        return DQ4_OK;  // dst is empty
    if (!dst || n_cols > INT64_MAX / m || (n_rows > 0 && n_cols > INT64_MAX / n_rows))
        return DQ4_EINVAL;
    const int64_t count = m * n_cols;
    const int64_t tiles_i = dq4::ceil_div(m, dq4::kTileI);
    const int64_t tiles_j = dq4::ceil_div(n_cols, dq4::kTileJ);
    if (n_rows > 0) {
        if (!packed || !scale_codes || !nested_absmax || !scale_codebook || !codebook4 || !src1)
            return DQ4_EINVAL;
        if (src1_transposed ? ld_src1 < n_rows : ld_src1 < m)
            return DQ4_EINVAL;
        if (workspace_bytes > 0 && !workspace)
            return DQ4_EINVAL;
        if (tiles_i > 0x7FFFFFFF || tiles_j > 0x7FFFFFFF || tiles_i * tiles_j > 0x7FFFFFFF)
            return DQ4_EUNSUPPORTED;
    }
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess)
        return dq4::hip_failed(e);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (n_rows == 0) {  // an empty sum: dst = 0
        uint32_t grid = 0;
        dq4::grid_size(count, device, &grid);
        float *d = dst;
        int64_t c = count;
        void *params[] = {&d, &c};
        e = hipLaunchKernel(reinterpret_cast<const void *>(&dq4::out_prod_zero_kernel),
                            dim3(grid), dim3(dq4::kThreads), params, 0, s);
        return e == hipSuccess ? DQ4_OK : dq4::hip_failed(e);
    }
    const int64_t max_partials = workspace_bytes / 4 / count;
    const int64_t rps = dq4::rows_per_split(n_rows, tiles_i * tiles_j,
                                            dq4::compute_units(device), max_partials);
    const int64_t splits = dq4::ceil_div(n_rows, rps);
    const int64_t groups = splits * tiles_i * tiles_j;
    if (groups > 0x7FFFFFFF)
        return DQ4_EUNSUPPORTED;

    dq4::FusedArgs a{packed, scale_codes, nested_absmax, scale_codebook, codebook4, src1,
                     splits > 1 ? workspace : dst, n_rows, n_cols, m, ld_src1, rps, offset,
                     log2_block, static_cast<int>(tiles_i), static_cast<int>(tiles_j),
                     (n_cols % 8 == 0 && reinterpret_cast<uintptr_t>(packed) % 4 == 0) ? 1 : 0};
    void *params[] = {&a};
    const void *kernel =
        src1_transposed ? reinterpret_cast<const void *>(&dq4::out_prod_fused_kernel<true>)
                        : reinterpret_cast<const void *>(&dq4::out_prod_fused_kernel<false>);
    e = hipLaunchKernel(kernel, dim3(static_cast<uint32_t>(groups)), dim3(dq4::kThreads), params,
                        0, s);
    if (e != hipSuccess)
        return dq4::hip_failed(e);
    if (splits > 1) {
        uint32_t grid = 0;
        dq4::grid_size(count, device, &grid);
        const float *p = workspace;
        float *d = dst;
        int64_t c = count;
        int sp = static_cast<int>(splits);
        void *rparams[] = {&p, &d, &c, &sp};
        e = hipLaunchKernel(reinterpret_cast<const void *>(&dq4::out_prod_reduce_kernel),
                            dim3(grid), dim3(dq4::kThreads), rparams, 0, s);
        if (e != hipSuccess)
            return dq4::hip_failed(e);
    }
    return DQ4_OK;
}

}  // extern "C"

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
// but each workgroup decodes the 4-bit weight of its tile on chip as the
// very FP32 values the dequantization kernel writes (bitsandbytes issue
// "Fuse nested scale reconstruction into SM103 4-bit dequantization",
// section "Proposed experiment": W = fl32(codebook4[k] * scale) with scale =
// fl32(fl32(scale_codebook[code] * absmax) + offset)) and feeds them to the
// FP32 matrix instructions.
//
// Design:
//  * the aligned path (n_cols % 8 == 0, packed 4-byte aligned) takes the
//    direct kernel (out_prod_direct_kernel): each lane decodes a packed
//    dword of 8 weights, which share one block scale, straight into the
//    operand registers of the matrix instruction, with no LDS staging of the
//    weights and no barrier in its main loop.  A tile is 4 or 8 dst rows
//    (v_mfma_f32_4x4x1_16b_f32) or 16, 32, 48 or 64 rows
//    (v_mfma_f32_16x16x4_f32) by 128 columns; m > 64 is split into whole
//    64-row tiles and one launch for the rest with the smallest tile that
//    holds it (row_ranges), since the 64-row tile costs no more per dst row
//    than any wider staged tile.  Full steps address the split from one
//    buffer per array with 32-bit offsets when those fit, and the split's
//    last step, or every step when they do not, takes checked 64-bit loads;
//  * the byte path (odd widths) takes the staged kernel
//    (out_prod_fused_kernel): a workgroup (4 waves) owns a kTileI x 128 tile
//    of dst (kTileI = 256, 128 or 64 from a cost rule, tile_cost, or 16 for
//    decode-sized m) and one split of the rows; per stage of 16 weight rows
//    every lane decodes 8 consecutive elements byte by byte (one or two
//    block scales) into LDS and stages the tile's src1 values, and the
//    waves' 32 x 32 (or 16 x 16) MFMA blocks read both from LDS; two LDS
//    buffers, so the next stage is decoded while the MFMAs read the current
//    one, with one barrier per stage and the stage after that already
//    loading;
//  * the rows are split when that fills the GPU's resident workgroup slots
//    (sized from the kernel's occupancy) better than the tiles alone; each
//    split writes its partial tile to the caller's workspace, and a second
//    kernel adds the partials in split order, so the result is deterministic
//    for a given device and workspace size.
// The FP32 sum order differs from the blocked route's library GEMM; both are
// within the FP32 summation bound of the exact sum.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "dq4.h"
#include "dq4_device.h"

#pragma clang fp contract(off)

namespace dq4 {
namespace {

constexpr int kThreads = 256;
constexpr int kTileJ = 128;         // dst columns (weight columns) per workgroup
constexpr int kLog2Stage = 4;
constexpr int kStage = 1 << kLog2Stage;  // weight rows per LDS stage
constexpr int kLdsW = kTileJ + 4;   // padded LDS row of decoded weights
constexpr int64_t kMinRowsPerSplit = 256;
constexpr int64_t kMaxSplits = 64;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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
    int full_stages;         // 1: the direct kernel's full steps take the unchecked loads
};

// Tile shape: a workgroup owns kTileI x kTileJ of dst and its 4 waves split
// it into kWavesI x kWavesJ sub-tiles of MFMA blocks.  kTileI = 64, 128 or
// 256: 2 x 2 waves of 32 x 32 blocks (v_mfma_f32_32x32x2_f32, 2 rows per
// instruction).  kTileI = 16, for decode-sized m on the byte path: 1 x 4
// waves of 16 x 16 blocks (v_mfma_f32_16x16x4_f32, 4 rows per instruction);
// the staged kernel serves the byte path (n_cols % 8 != 0, or packed not
// 4-byte aligned); the aligned path takes out_prod_direct_kernel.
template <int kTileI>
struct Shape {
    static constexpr bool kSmall = kTileI == 16;
    static constexpr int kBlk = kSmall ? 16 : 32;           // MFMA block edge
    static constexpr int kK = kSmall ? 4 : 2;               // weight rows per MFMA
    static constexpr int kWavesI = kSmall ? 1 : 2;
    static constexpr int kWaveI = kTileI / kWavesI;
    static constexpr int kWaveJ = kTileJ / (4 / kWavesI);
    static constexpr int kBlocksI = kWaveI / kBlk;
    static constexpr int kBlocksJ = kWaveJ / kBlk;
    static constexpr int kAccRegs = kBlk * kBlk / 64;        // accumulator values per lane
    static constexpr int kLdsB = kTileI + 4;                 // padded LDS row of src1 values
    static constexpr int kB = kStage * kTileI / kThreads;    // src1 values per lane and stage
    using Acc = typename std::conditional<kSmall, f32x4, f32x16>::type;
    // Accumulator sets per block.  The 16-row tile has only two blocks per
    // wave, so with one set each MFMA of a stage waited on the one just
    // issued before it, and the compiler shuffled the accumulators between
    // registers on every stage; consecutive steps in alternate sets (added
    // together at the end) remove both (~3 % at m <= 16).  The wider tiles
    // already interleave enough blocks.
    static constexpr int kSets = kSmall ? 2 : 1;
    // Waves per SIMD the register allocation must allow: the wide tiles'
    // LDS already caps them at 2 (256 rows) and 4 (128 rows) per SIMD, and
    // left alone the compiler spends registers on hoisted LDS addresses until
    // fewer fit.  The 16- and 64-row tiles are left to the compiler.
    static constexpr int kMinWaves = kTileI == 256 ? 2 : kTileI == 128 ? 4 : 1;

    // one MFMA: acc += A (kBlk x kK) x B (kK x kBlk); lane l holds A[l % kBlk][l / kBlk]
    // and B[l / kBlk][l % kBlk]
    __device__ static Acc mma(float a, float b, Acc acc)
    {
        if constexpr (kSmall)
            return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
    // the block row held by accumulator register v of lane l (its column is l % kBlk)
    __device__ static int acc_row(int v, int l)
    {
        if constexpr (kSmall)
            return 4 * (l >> 4) + v;
        else
            return 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
    }
};

// What one lane loads from HBM for one stage, before decoding it.
template <int kTileI>
struct StageLoad {
    uint8_t bytes[8];   // the byte holding each element
    uint32_t code_lo, code_hi;
    float absmax_lo, absmax_hi;
    float b[Shape<kTileI>::kB];
};

template <int kTileI, bool kSrc1Transposed>
__device__ __forceinline__ void load_stage_b(const FusedArgs &a, int64_t k0, int64_t k_end,
                                             int64_t i0, int t, StageLoad<kTileI> &ld);

// A lane's 8 consecutive elements, byte by byte: a row's elements need not
// start on a byte (odd n_cols) and may span two blocks.
template <int kTileI, bool kSrc1Transposed>
__device__ __forceinline__ void load_stage(const FusedArgs &a, int64_t k0, int64_t k_end,
                                           int64_t i0, int64_t j0, int t,
                                           StageLoad<kTileI> &ld)
{
    // weight: row k0 + t / 16, columns j0 + (t % 16) * 8 .. + 7
    const int64_t r = k0 + (t >> 4);
    const int64_t j = j0 + (t & 15) * 8;
    const int lb = a.log2_block;
    if (r < k_end && j < a.n_cols) {
        const int64_t e = r * a.n_cols + j;
        const int64_t e_last = e + (min(a.n_cols - j, int64_t{8}) - 1);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            ld.bytes[q] = e + q <= e_last ? a.packed[(e + q) >> 1] : 0;
        const int64_t b_lo = e >> lb, b_hi = e_last >> lb;  // at most two blocks
        ld.code_lo = a.scale_codes[b_lo];
        ld.absmax_lo = a.nested_absmax[b_lo >> kNestedLog2];
        ld.code_hi = a.scale_codes[b_hi];
        ld.absmax_hi = a.nested_absmax[b_hi >> kNestedLog2];
    }
    load_stage_b<kTileI, kSrc1Transposed>(a, k0, k_end, i0, t, ld);
}

// The src1 values of one stage, with bounds checks: B[r][i] for the stage's
// rows below k_end and columns below m, 0 elsewhere.
template <int kTileI, bool kSrc1Transposed>
__device__ __forceinline__ void load_stage_b(const FusedArgs &a, int64_t k0, int64_t k_end,
                                             int64_t i0, int t, StageLoad<kTileI> &ld)
{
    constexpr int kB = Shape<kTileI>::kB;
    if constexpr (!kSrc1Transposed) {
        // B[r][i] = src1[r * ld + i]: one stage row, kB consecutive columns
        constexpr int kLanesPerRow = kTileI / kB;
        const int64_t rb = k0 + t / kLanesPerRow;
        const int64_t ib = i0 + (t % kLanesPerRow) * kB;
        const float *p = a.src1 + rb * a.ld + ib;
        if (rb < k_end && ib + kB <= a.m) {
#pragma unroll
            for (int q = 0; q < kB; ++q)
                ld.b[q] = p[q];
        } else {
#pragma unroll
            for (int q = 0; q < kB; ++q)
                ld.b[q] = (rb < k_end && ib + q < a.m) ? p[q] : 0.0f;
        }
    } else {
        // B[r][i] = src1[i * ld + r]: one column i, kB consecutive stage rows
        constexpr int kLanesPerCol = kStage / kB;
        const int64_t ib = i0 + t / kLanesPerCol;
        const int64_t rb = k0 + (t % kLanesPerCol) * kB;
        const float *p = a.src1 + ib * a.ld + rb;
        if (ib < a.m && rb + kB <= k_end) {
#pragma unroll
            for (int q = 0; q < kB; ++q)
                ld.b[q] = p[q];
        } else {
#pragma unroll
            for (int q = 0; q < kB; ++q)
                ld.b[q] = (rb + q < k_end && ib < a.m) ? p[q] : 0.0f;
        }
    }
}

// The 8 weights of one packed dword (element 2p in the low nibble of byte
// p, element 2p + 1 in its high nibble), all in the block of scale s:
// v[q] = fl32(codebook4[nibble q] * s).  One 8-byte LDS read from the
// 256-entry table of codebook pairs returns both entries of a byte.
__device__ __forceinline__ void decode8(uint32_t packed4, float s, const f32x2 *lds_pair,
                                        float (&v)[8])
{
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t off = ((packed4 >> (8 * p)) & 0xFFu) << 3;
        const f32x2 e =
            *reinterpret_cast<const f32x2 *>(reinterpret_cast<const char *>(lds_pair) + off);
        v[2 * p] = e.x * s;
        v[2 * p + 1] = e.y * s;
    }
}

// The lane's src1 values of one stage into LDS (lds_b[r][i] = B[r][i]).
template <int kTileI, bool kSrc1Transposed>
__device__ __forceinline__ void store_stage_b(int t, const StageLoad<kTileI> &ld,
                                              float (*lds_b)[Shape<kTileI>::kLdsB])
{
    constexpr int kB = Shape<kTileI>::kB;
    if constexpr (!kSrc1Transposed) {
        constexpr int kLanesPerRow = kTileI / kB;
        const int br = t / kLanesPerRow, bc = (t % kLanesPerRow) * kB;
#pragma unroll
        for (int q = 0; q < kB; ++q)
            lds_b[br][bc + q] = ld.b[q];
    } else {
        constexpr int kLanesPerCol = kStage / kB;
        const int bc = t / kLanesPerCol, br = (t % kLanesPerCol) * kB;
#pragma unroll
        for (int q = 0; q < kB; ++q)
            lds_b[br + q][bc] = ld.b[q];
    }
}

template <int kTileI, bool kSrc1Transposed>
__device__ __forceinline__ void decode_stage(const FusedArgs &a, int64_t k0, int64_t k_end,
                                             int64_t j0, int t, const StageLoad<kTileI> &ld,
                                             const float *lds_scb, const float *lds_cb4,
                                             float (*lds_w)[kLdsW],
                                             float (*lds_b)[Shape<kTileI>::kLdsB])
{
    const int row = t >> 4, col = (t & 15) * 8;
    const int64_t r = k0 + row;
    const int64_t j = j0 + col;
    float v[8];
    if (r < k_end && j < a.n_cols) {
        const float s_lo = block_scale(lds_scb[ld.code_lo], ld.absmax_lo, a.offset);
        const int lb = a.log2_block;
        const int64_t e = r * a.n_cols + j;
        const float s_hi = block_scale(lds_scb[ld.code_hi], ld.absmax_hi, a.offset);
        // position of element e in its block; element e + q is in the next
        // block once off + q reaches the block size
        const uint32_t off = static_cast<uint32_t>(e & ((int64_t{1} << lb) - 1));
        const int64_t n_valid = min(a.n_cols - j, int64_t{8});
        const uint32_t odd = static_cast<uint32_t>(e & 1);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t k = ((odd + q) & 1) ? (ld.bytes[q] >> 4) : (ld.bytes[q] & 0xFu);
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
    store_stage_b<kTileI, kSrc1Transposed>(t, ld, lds_b);
}

// A raw buffer over `bytes` bytes from `base`: each load through it is one
// scalar base plus 32-bit offsets, with no 64-bit address arithmetic.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_buffer(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0,
                                             static_cast<int>(bytes), kRawBufferWord3);
}

// The float at byte_offset + extra; `extra` is a compile-time constant that
// goes into the instruction's scalar offset, not into a vector register.
__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t buf, uint32_t byte_offset,
                                          int extra = 0)
{
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_raw_buffer_load_b32(buf, byte_offset, extra, 0));
}

// The MFMAs of one stage: acc[bi][bj] += A(i block bi) x W(j block bj) over
// the stage's kStage rows, kK rows per instruction; each step's operands
// are read from LDS one step ahead of its MFMAs.  (The raised wave priority
// around this call is a scheduling hint within the kernel, not a stream
// priority.)
template <int kTileI>
__device__ __forceinline__ void mma_stage(
    const float (*lds_w)[kLdsW], const float (*lds_b)[Shape<kTileI>::kLdsB], int wi, int wj,
    int kl, int cl,
    typename Shape<kTileI>::Acc (&acc)[Shape<kTileI>::kSets][Shape<kTileI>::kBlocksI]
                                      [Shape<kTileI>::kBlocksJ])
{
    using S = Shape<kTileI>;
    const int ia = S::kWaveI * wi + cl, jw = S::kWaveJ * wj + cl;
    float av[2][S::kBlocksI], wv[2][S::kBlocksJ];
#pragma unroll
    for (int bi = 0; bi < S::kBlocksI; ++bi)
        av[0][bi] = lds_b[kl][ia + S::kBlk * bi];
#pragma unroll
    for (int bj = 0; bj < S::kBlocksJ; ++bj)
        wv[0][bj] = lds_w[kl][jw + S::kBlk * bj];
#pragma unroll
    for (int kk = 0; kk < kStage; kk += S::kK) {
        const int cur = (kk / S::kK) & 1, nxt = cur ^ 1;
        if (kk + S::kK < kStage) {
#pragma unroll
            for (int bi = 0; bi < S::kBlocksI; ++bi)
                av[nxt][bi] = lds_b[kk + S::kK + kl][ia + S::kBlk * bi];
#pragma unroll
            for (int bj = 0; bj < S::kBlocksJ; ++bj)
                wv[nxt][bj] = lds_w[kk + S::kK + kl][jw + S::kBlk * bj];
        }
        const int set = (kk / S::kK) % S::kSets;
#pragma unroll
        for (int bi = 0; bi < S::kBlocksI; ++bi)
#pragma unroll
            for (int bj = 0; bj < S::kBlocksJ; ++bj)
                acc[set][bi][bj] = S::mma(av[cur][bi], wv[cur][bj], acc[set][bi][bj]);
        if (kk + S::kK < kStage) {
            // keep the next step's LDS reads ahead of this step's MFMAs (the
            // compiler otherwise issues them just before their use)
            __builtin_amdgcn_sched_group_barrier(0x100, S::kBlocksI + S::kBlocksJ, 0);  // DS read
            __builtin_amdgcn_sched_group_barrier(0x008, S::kBlocksI * S::kBlocksJ, 0);  // MFMA
        }
    }
}

// Two LDS buffers: while the waves multiply one stage, they decode the next
// into the other buffer, so one barrier per stage suffices.  The stage loop
// is unrolled by two, so that each step's LDS buffers are known at compile
// time and every LDS address is a lane-constant register plus an immediate.
template <int kTileI, bool kSrc1Transposed>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Shape<kTileI>::kMinWaves)))
void out_prod_fused_kernel(FusedArgs a)
{
    using S = Shape<kTileI>;
    __shared__ float lds_w[2][kStage][kLdsW];
    __shared__ float lds_b[2][kStage][S::kLdsB];
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

    const int wi = wave % S::kWavesI, wj = wave / S::kWavesI;
    const int kl = lane / S::kBlk, cl = lane % S::kBlk;
    typename S::Acc acc[S::kSets][S::kBlocksI][S::kBlocksJ];
#pragma unroll
    for (int q = 0; q < S::kSets; ++q)
#pragma unroll
        for (int bi = 0; bi < S::kBlocksI; ++bi)
#pragma unroll
            for (int bj = 0; bj < S::kBlocksJ; ++bj)
                acc[q][bi][bj] = typename S::Acc{};

    // stage s holds rows k_begin + kStage * s .. (stage counts are below
    // 2^31: the host caps the rows of a split)
    const int64_t rows = k_end - k_begin;  // > 0
    const int n_stages =
        __builtin_amdgcn_readfirstlane(static_cast<int>((rows + kStage - 1) >> kLog2Stage));

    StageLoad<kTileI> ld;
    const auto load = [&](int s) {
        load_stage<kTileI, kSrc1Transposed>(a, k_begin + kStage * s, k_end, i0, j0, t, ld);
    };
    const auto decode = [&](int s, auto buffer) {
        constexpr int q = decltype(buffer)::value;
        decode_stage<kTileI, kSrc1Transposed>(a, k_begin + kStage * s, k_end, j0, t, ld,
                                              lds_scb, lds_cb4, lds_w[q], lds_b[q]);
    };
    // one step: the MFMAs of stage s (in buffer q), then stage s + 1 decoded
    // into the other buffer and the loads of stage s + 2 issued
    const auto step = [&](int s, auto buffer) {
        constexpr int q = decltype(buffer)::value;
        // a wave issuing MFMAs goes first among the SIMD's waves, so the matrix
        // unit is fed while other waves decode (~2 % at m >= 512)
        __builtin_amdgcn_s_setprio(1);
        mma_stage<kTileI>(lds_w[q], lds_b[q], wi, wj, kl, cl, acc);
        __builtin_amdgcn_s_setprio(0);
        if (s + 1 < n_stages) {
            decode(s + 1, std::integral_constant<int, q ^ 1>{});
            if (s + 2 < n_stages)
                load(s + 2);
        }
        __syncthreads();
    };

    load(0);
    __syncthreads();  // the codebooks are in LDS
    decode(0, std::integral_constant<int, 0>{});
    if (n_stages > 1)
        load(1);
    __syncthreads();
    // even stages in buffer 0, odd ones in buffer 1
    int s = 0;
    for (; s + 1 < n_stages; s += 2) {
        step(s, std::integral_constant<int, 0>{});
        step(s + 1, std::integral_constant<int, 1>{});
    }
    if (s < n_stages)
        step(s, std::integral_constant<int, 0>{});

    float *out = a.part + int64_t{split} * a.m * a.n_cols;
#pragma unroll
    for (int bi = 0; bi < S::kBlocksI; ++bi)
#pragma unroll
        for (int v = 0; v < S::kAccRegs; ++v) {
            const int64_t i = i0 + S::kWaveI * wi + S::kBlk * bi + S::acc_row(v, lane);
            if (i >= a.m)
                continue;
#pragma unroll
            for (int bj = 0; bj < S::kBlocksJ; ++bj) {
                const int64_t j = j0 + S::kWaveJ * wj + S::kBlk * bj + cl;
                if (j < a.n_cols)
                {
                    float sum = acc[0][bi][bj][v];
#pragma unroll
                    for (int q = 1; q < S::kSets; ++q)
                        sum = sum + acc[q][bi][bj][v];
                    out[i * a.n_cols + j] = sum;
                }
            }
        }
}

// ---------------------------------------------------------------------------
// Direct tiles on the aligned path, up to 64 dst rows each (a wider m repeats
// the tile over the rows).  With few dst rows each decoded weight feeds only a
// tile's products, and staging the weights through LDS (a write and a read
// per element) made the LDS the limit at m = 16.  Here each lane decodes its
// packed dword straight into the operand layout of v_mfma_f32_16x16x4_f32: a
// step covers 4 weight rows (the instruction's k) and the tile's 128 columns
// as 8 blocks of 16, lane l taking row l / 16 and columns 8 (l % 16) .. + 7,
// so that its 8 decoded values are its operands of the 8 blocks (block bj's
// column c is weight column 8c + bj).  The tile's 16 * kBI dst rows (kBI =
// 1 .. 4) are kBI blocks of 16 in the same way (block bi's row c is dst row
// kBI c + bi), so a lane's src1 operands of one step are kBI consecutive
// floats of one src1 row, loaded straight from global memory.  The store
// undoes both permutations.  The 4 waves of a workgroup take every fourth
// step of the split's rows and add their partial tiles at the end in a fixed
// order ((w0 + w2) + (w1 + w3)), so the result stays deterministic.  Only the
// codebooks live in LDS during the main loop, which has no barrier.
//
// kMode selects how a step's products are summed.  Mode 0 is the above.
// In mode 1 (4-row sets), for m <= 8, the same steps feed v_mfma_f32_4x4x1_16b_f32
// instead: 16 independent 4 x 4 blocks of k = 1, block b = l / 4 made of
// lanes 4b .. 4b + 3.  The weight operand keeps its place (lane l's value q
// is column j = l % 4 of its block), and the src1 operand of lane l is src1
// column 4 bi + l % 4 of the lane's own weight row, so block b sums products
// of one weight row only.  The tile's 4 kBI dst rows are kBI sets of 4 (set
// bi's row v is dst row 4 bi + v, accumulator register v), and the lanes of
// the four weight rows of a step hold partial sums of the same dst elements;
// they are added across lanes at the end, (g0 + g1) + (g2 + g3) over the lane
// groups l / 16.  The instruction does a quarter of the 16 x 16 x 4 one's
// products in a quarter of its matrix-pipe time (8 cycles against 32, by
// counters), but the decode's vector instructions, which do not overlap FP32
// matrix instructions, are the same per step: on the output head m <= 4
// takes 0.16 ms and m <= 8 0.22 ms against 0.26 ms for the 16-row tile, and
// three sets (m <= 12) measured slower than the 16-row tile, which keeps them.
//
// Mode 2, for m == 1, sums on the vector unit: each lane adds b * W for its
// 8 weights with fused multiply-adds into 8 accumulators, and the lane groups
// and waves are added as in mode 1.  Each weight W is still its own rounded
// product fl32(codebook4[k] * scale); only the accumulation is fused, as it
// is inside the matrix instructions.  The step's 8 FMAs issue in 32 cycles
// against the 64 of its 8 matrix instructions (0.13 against 0.16 ms on the
// output head); from m = 2 on they would cost as much.
constexpr int kDirectK = 4;   // weight rows per step (n_steps uses >> 2)

template <int kBI>
struct DirectLoad {
    uint32_t packed4;
    uint32_t code;
    float absmax;
    float b[kBI];
};

template <int kBI, int kMode>
struct Direct {
    static constexpr bool kQuad = kMode == 1;  // 4-row sets on the 4 x 4 x 1 instruction
    static constexpr bool kVec = kMode == 2;   // one dst row on the vector unit
    static constexpr int kRows = kVec ? 1 : (kQuad ? 4 : 16) * kBI;  // dst rows of the tile
    static constexpr int kAccV = kVec ? 1 : 4;  // accumulator values per block and lane
    static constexpr int kMinWaves = kBI >= 3 && kMode == 0 ? 2 : 1;

    // the tile row of the lane's src1 operand of block (or set) bi
    static __device__ __forceinline__ uint32_t src1_row(int lane, int bi)
    {
        if constexpr (kVec)
            return 0u;
        return kQuad ? static_cast<uint32_t>(4 * bi + (lane & 3))
                     : static_cast<uint32_t>(kBI * (lane & 15) + bi);
    }

    static __device__ __forceinline__ f32x4 mma(float b, float w, f32x4 acc)
    {
        if constexpr (kVec) {
            acc[0] = __builtin_fmaf(b, w, acc[0]);
            return acc;
        } else if constexpr (kQuad) {
            return __builtin_amdgcn_mfma_f32_4x4x1f32(b, w, acc, 0, 0, 0);
        } else {
            return __builtin_amdgcn_mfma_f32_16x16x4f32(b, w, acc, 0, 0, 0);
        }
    }
};

// The 4 x 4 transpose of x across the four 16-lane rows of a wave: lane row r
// holds x = (M[r][0], .., M[r][3]) and gets out[t] = M[t][r].  Swapping rows
// 2-3 of one register with rows 0-1 of another, then odd rows with even rows,
// is the usual two-level block transpose.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void transpose_rows4(u32x4 x, float (&out)[4])
{
    // x holds the loaded bits as integers: a bit_cast of a single element of
    // a float vector read element 0 for every element with this compiler
    uint32_t v0 = x[0], v1 = x[1], v2 = x[2], v3 = x[3];
    auto p = __builtin_amdgcn_permlane32_swap(v0, v2, false, false);
    v0 = p[0];
    v2 = p[1];
    p = __builtin_amdgcn_permlane32_swap(v1, v3, false, false);
    v1 = p[0];
    v3 = p[1];
    p = __builtin_amdgcn_permlane16_swap(v0, v1, false, false);
    v0 = p[0];
    v1 = p[1];
    p = __builtin_amdgcn_permlane16_swap(v2, v3, false, false);
    v2 = p[0];
    v3 = p[1];
    out[0] = __builtin_bit_cast(float, v0);
    out[1] = __builtin_bit_cast(float, v1);
    out[2] = __builtin_bit_cast(float, v2);
    out[3] = __builtin_bit_cast(float, v3);
}

template <int kBI>
struct SuperLoad {
    uint32_t packed4[4];
    uint32_t code[4];
    float absmax[4];
    u32x4 b[kBI];  // src1 bits
};

template <int kBI, int kMode, bool kSrc1Transposed, bool kWholeBlocks>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(Direct<kBI, kMode>::kMinWaves)))
void out_prod_direct_kernel(FusedArgs a)
{
    using D = Direct<kBI, kMode>;
    __shared__ float lds_scb[256];
    __shared__ f32x2 lds_pair[256];                  // (entry of low nibble, high nibble)
    __shared__ float lds_red[kBI * 32 * 64];         // a wave's partial tile

    const int t = threadIdx.x;
    // the wave index is uniform within a wave; saying so keeps the steps'
    // addresses in scalar registers
    const int lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
    // Workgroups go to the 8 XCDs in turn (blockIdx % 8), each XCD with its
    // own L2.  With one i-tile, XCD x takes the x-th eighth of the tile order
    // instead, so that a split's column tiles, which share the lines of its
    // codes and src1 rows and (two by two) of its packed rows, share an L2:
    // on the output head that cuts the call's HBM reads from 2.3-2.8 x its
    // algorithmic bytes to 1.1-1.2 x, and the time by 4-9 % at m <= 4 (within
    // 2 % at m = 8 .. 64: the decode, not HBM, bounds those).  With several
    // i-tiles (m > 64) the round-robin order measured 2 % faster for a
    // transposed src1, so it stays.
    uint32_t order = blockIdx.x;
    if (a.tiles_i == 1) {
        const uint32_t g_all = gridDim.x, xcd = blockIdx.x & 7u;
        order = xcd * (g_all >> 3) + min(xcd, g_all & 7u) + (blockIdx.x >> 3);
    }
    const int ti = static_cast<int>(order % static_cast<uint32_t>(a.tiles_i));
    const uint32_t rest = order / static_cast<uint32_t>(a.tiles_i);
    const int tj = static_cast<int>(rest % static_cast<uint32_t>(a.tiles_j));
    const int split = static_cast<int>(rest / static_cast<uint32_t>(a.tiles_j));
    const int64_t i0 = int64_t{ti} * D::kRows, j0 = int64_t{tj} * kTileJ;
    const int64_t k_begin = int64_t{split} * a.rows_per_split;
    const int64_t k_end = min(a.n_rows, k_begin + a.rows_per_split);

    lds_scb[t] = a.scale_codebook[t];
    lds_pair[t] = f32x2{a.codebook4[t & 15], a.codebook4[t >> 4]};
    __syncthreads();

    // lane constants: row of the step, first of 8 weight columns, src1
    // columns (lanes past n_cols read column j0, and src1 columns past m read
    // column m - 1: in range, and their products reach only dst elements that
    // are never stored)
    const int row = lane >> 4, c = lane & 15;
    const uint32_t n_cols = static_cast<uint32_t>(a.n_cols);
    const uint32_t ld_src1 = static_cast<uint32_t>(a.ld);
    const uint32_t col_in = j0 + 8 * c < a.n_cols ? 8u * c : 0u;
    const uint32_t w_elem = static_cast<uint32_t>(row) * n_cols + col_in;
    const uint32_t i_last = static_cast<uint32_t>(min(a.m - i0, int64_t{D::kRows}) - 1);
    uint32_t b_off[kBI];  // bytes from the step's first src1 element
#pragma unroll
    for (int bi = 0; bi < kBI; ++bi) {
        const uint32_t il = min(D::src1_row(lane, bi), i_last);
        b_off[bi] = kSrc1Transposed ? 4u * (il * ld_src1 + row) : 4u * (row * ld_src1 + il);
    }
    const int lb = a.log2_block;

    const int64_t rows = k_end - k_begin;  // > 0
    const int n_steps =
        __builtin_amdgcn_readfirstlane(static_cast<int>((rows + kDirectK - 1) >> 2));
    const int n_full =
        a.full_stages ? __builtin_amdgcn_readfirstlane(static_cast<int>(rows >> 2)) : 0;

    // A full step: no bounds checks, one buffer per array for the whole split
    // and 32-bit offsets, the step's part of them uniform (the instruction's
    // scalar offset, or added once for the lanes' shared block index).  The
    // host allows full steps only when the split's offsets below stay under
    // 2^32: rows * n_cols weight elements plus the block offset bl0 < 4096,
    // and rows * ld (or kRows * ld when transposed) src1 floats.  Rebuilding
    // the buffers at every step instead cost about 40 scalar instructions a
    // step, up to 18 % of the call at m <= 8.
    const int64_t e_split = k_begin * a.n_cols + j0;  // the split's first element of the tile
    const int64_t bh0 = e_split >> lb;
    const uint32_t rows32 = static_cast<uint32_t>(rows);
    const uint32_t span_e = rows32 * n_cols;  // elements from e_split to the split's end
    const __amdgpu_buffer_rsrc_t packed_b =
        span_buffer(a.packed + (e_split >> 1), span_e / 2 + 64);
    const uint32_t bl0 = static_cast<uint32_t>(e_split & ((int64_t{1} << lb) - 1));
    const uint32_t c_span = ((bl0 + span_e + 128u) >> lb) + 1u;
    const __amdgpu_buffer_rsrc_t code_b = span_buffer(a.scale_codes + bh0, c_span);
    const uint32_t g0 = static_cast<uint32_t>(bh0 & ((1 << kNestedLog2) - 1));
    const __amdgpu_buffer_rsrc_t absmax_b =
        span_buffer(a.nested_absmax + (bh0 >> kNestedLog2),
                    4u * (((g0 + c_span) >> kNestedLog2) + 1u));
    const __amdgpu_buffer_rsrc_t src1_b =
        kSrc1Transposed
            ? span_buffer(a.src1 + (i0 * a.ld + k_begin), 4u * (D::kRows * ld_src1 + rows32))
            : span_buffer(a.src1 + (k_begin * a.ld + i0), 4u * (rows32 * ld_src1 + D::kRows));
    const uint32_t w_byte = w_elem >> 1, c_lane = bl0 + w_elem;
    const uint32_t step_elems = kDirectK * n_cols;
    const uint32_t step_b = kSrc1Transposed ? 4u * kDirectK : 4u * kDirectK * ld_src1;
    // When a step spans whole blocks (kWholeBlocks: kDirectK * n_cols is a
    // multiple of the block size), the lane's block at step s is its block at
    // step 0 plus s times the step's block count: the code's offset is then a
    // lane constant plus a uniform part, and only the absmax index needs
    // vector instructions (3 instead of 5 a step).
    const uint32_t cb_lane = c_lane >> lb, ga_lane = g0 + cb_lane;
    const uint32_t step_blocks = step_elems >> lb;
    // the code and absmax of the lane's block at the step starting d elements
    // past the split's first row (d = s * step_elems)
    const auto load_meta = [&](uint32_t s, uint32_t d, uint32_t &code, float &absmax) {
        if constexpr (kWholeBlocks) {
            const uint32_t sblk = s * step_blocks;
            code = __builtin_amdgcn_raw_buffer_load_b8(code_b, cb_lane, sblk, 0);
            absmax = load_f32(absmax_b, 4u * ((ga_lane + sblk) >> kNestedLog2));
        } else {
            const uint32_t cb = (c_lane + d) >> lb;  // the lane's block, from bh0
            code = __builtin_amdgcn_raw_buffer_load_b8(code_b, cb, 0, 0);
            absmax = load_f32(absmax_b, 4u * ((g0 + cb) >> kNestedLog2));
        }
    };
    const auto load_full = [&](int s) {
        DirectLoad<kBI> ld;
        const uint32_t d = static_cast<uint32_t>(s) * step_elems;  // the step's first element
        ld.packed4 = __builtin_amdgcn_raw_buffer_load_b32(packed_b, w_byte, d >> 1, 0);
        load_meta(static_cast<uint32_t>(s), d, ld.code, ld.absmax);
        const uint32_t sb = static_cast<uint32_t>(s) * step_b;
#pragma unroll
        for (int bi = 0; bi < kBI; ++bi)
            ld.b[bi] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(src1_b, b_off[bi], sb, 0));
        return ld;
    };

    f32x4 acc[kBI][8];
#pragma unroll
    for (int bi = 0; bi < kBI; ++bi)
#pragma unroll
        for (int bj = 0; bj < 8; ++bj)
            acc[bi][bj] = f32x4{};
    const auto decode = [&](const DirectLoad<kBI> &ld, float (&v)[8]) {
        decode8(ld.packed4, block_scale(lds_scb[ld.code], ld.absmax, a.offset), lds_pair, v);
    };
    const auto full_step = [&](const DirectLoad<kBI> &ld) {
        float v[8];
        decode(ld, v);
#pragma unroll
        for (int bj = 0; bj < 8; ++bj)
#pragma unroll
            for (int bi = 0; bi < kBI; ++bi)
                acc[bi][bj] =
                    D::mma(ld.b[bi], v[bj], acc[bi][bj]);
    };
    // a loaded step that may lie past n_full: its operands zeroed there, so
    // that the accumulators are updated unconditionally (see below)
    const auto masked_step = [&](const DirectLoad<kBI> &ld, bool use) {
        float v[8];
        decode(ld, v);
#pragma unroll
        for (int bj = 0; bj < 8; ++bj)
#pragma unroll
            for (int bi = 0; bi < kBI; ++bi)
                acc[bi][bj] = D::mma(use ? ld.b[bi] : 0.0f, use ? v[bj] : 0.0f, acc[bi][bj]);
    };

    // The full steps run in two banks of loads that alternate: the steps of
    // one bank are computed while the loads of the other fly.  (Written so
    // that no loaded value is copied between registers -- a copy would wait
    // for the load -- and so that the loop body updates the accumulators
    // unconditionally: a conditional update keeps the old value live and made
    // the compiler copy every accumulator on every step.)
    int first_tail = n_full;  // the checked steps start here
    if constexpr (kSrc1Transposed && kMode == 0 && kBI <= 2) {
        // A transposed src1 in the 16- and 32-row tiles: each of a step's
        // src1 loads reads 16 separate rows of src1 (one line each).  Here a
        // wave takes super-steps of 16 consecutive weight rows (4 steps; wave
        // w takes super-steps w, w + 4, ..), lane row r loads rows
        // 16 S + 4 r .. + 3 of its src1 column at once (16 bytes), and the
        // wave's four lane rows swap them into place (transpose_rows4), so the
        // src1 loads read 4 x fewer lines.  On the output head this made the
        // 16- and 32-row tiles' time flat in m: m = 16 and 32 8 % faster, m =
        // 28 4 %, and at most 2 % slower for a sparse tile (m = 9), whose
        // clamped columns already share lines.  The 4- and 8-row sets, whose
        // loads read only 4 rows of src1 each, were 3-8 % slower with it, and
        // the 64-row tile 2.5 % faster at m = 64 but 1.5 % slower at m = 512.
        const int n_super = n_full >> 2;
        first_tail = n_super << 2;
        uint32_t bq_off[kBI];
#pragma unroll
        for (int bi = 0; bi < kBI; ++bi) {
            const uint32_t il = min(D::src1_row(lane, bi), i_last);
            bq_off[bi] = 4u * (il * ld_src1 + 4u * static_cast<uint32_t>(row));
        }
        const auto load_super = [&](int S) {
            SuperLoad<kBI> ld;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t d = static_cast<uint32_t>(4 * S + t) * step_elems;
                ld.packed4[t] = __builtin_amdgcn_raw_buffer_load_b32(packed_b, w_byte, d >> 1, 0);
                load_meta(static_cast<uint32_t>(4 * S + t), d, ld.code[t], ld.absmax[t]);
            }
            const uint32_t sb = static_cast<uint32_t>(S) * (16u * 4u);
#pragma unroll
            for (int bi = 0; bi < kBI; ++bi)
                ld.b[bi] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(src1_b, bq_off[bi], sb, 0));
            return ld;
        };
        const auto super_step = [&](const SuperLoad<kBI> &ld, bool use) {
            float av[kBI][4];
#pragma unroll
            for (int bi = 0; bi < kBI; ++bi)
                transpose_rows4(ld.b[bi], av[bi]);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                float v[8];
                decode8(ld.packed4[t],
                        block_scale(lds_scb[ld.code[t]], ld.absmax[t], a.offset), lds_pair, v);
#pragma unroll
                for (int bj = 0; bj < 8; ++bj)
#pragma unroll
                    for (int bi = 0; bi < kBI; ++bi)
                        acc[bi][bj] = D::mma(use ? av[bi][t] : 0.0f, use ? v[bj] : 0.0f,
                                             acc[bi][bj]);
            }
        };
        SuperLoad<kBI> sl0, sl1;
        if (n_super > 0) {
            sl0 = load_super(min(wave, n_super - 1));
            __builtin_amdgcn_sched_barrier(0);
            sl1 = load_super(min(wave + 4, n_super - 1));
            __builtin_amdgcn_sched_barrier(0);
        }
        int S0 = wave;  // the super-step in sl0
        for (; S0 + 4 < n_super; S0 += 8) {
            super_step(sl0, true);
            sl0 = load_super(min(S0 + 8, n_super - 1));
            __builtin_amdgcn_sched_barrier(0);
            super_step(sl1, true);
            sl1 = load_super(min(S0 + 12, n_super - 1));
            __builtin_amdgcn_sched_barrier(0);
        }
        if (n_super > 0)
            super_step(sl0, S0 < n_super);  // at most one left, in sl0
    } else {
        // wave w takes steps w, w + 4, w + 8, ... below n_full, kDepth steps
        // per bank: at kBI >= 3 one for a row-major src1 (fewer registers, 3 %
        // faster at m = 48 and 64), two for a transposed one, whose kBI loads
        // per step are kBI separate rows (3 % slower with one)
        constexpr int kDepth = kBI >= 3 ? (kSrc1Transposed ? 2 : 1) : 3;
        constexpr int kBank = 4 * kDepth;  // steps of one bank
        DirectLoad<kBI> bank0[kDepth], bank1[kDepth];
        if (n_full > 0) {
            // unconditional as in the loop (past n_full: step n_full - 1, unused),
            // and issued in the loop's order: the counts of loads in flight that
            // the loop waits for hold on entry too (left to reorder these loads,
            // the compiler made the loop wait for all but a few of them)
    #pragma unroll
            for (int d = 0; d < kDepth; ++d) {
                bank0[d] = load_full(min(wave + 4 * d, n_full - 1));
                __builtin_amdgcn_sched_barrier(0);
            }
    #pragma unroll
            for (int d = 0; d < kDepth; ++d) {
                bank1[d] = load_full(min(wave + kBank + 4 * d, n_full - 1));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        int s0 = wave;  // first step of bank0
        for (; s0 + kBank + 4 * (kDepth - 1) < n_full; s0 += 2 * kBank) {
            // Every step of both banks is below n_full.  The next loads are
            // issued unconditionally (a step past n_full reloads step n_full - 1,
            // unused): conditional loads would make the compiler's count of loads
            // in flight inexact, and it then waits for all of them.  The
            // scheduling barriers keep each step's loads right after its use of
            // the registers they refill; left alone, the scheduler sank all of
            // them to the end of the loop body, where the next iteration waited
            // for them at once.
    #pragma unroll
            for (int d = 0; d < kDepth; ++d) {
                full_step(bank0[d]);
                bank0[d] = load_full(min(s0 + 2 * kBank + 4 * d, n_full - 1));
                __builtin_amdgcn_sched_barrier(0);
            }
    #pragma unroll
            for (int d = 0; d < kDepth; ++d) {
                full_step(bank1[d]);
                bank1[d] = load_full(min(s0 + 3 * kBank + 4 * d, n_full - 1));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // at most 2 * kDepth - 1 full steps are left, all loaded
        if (n_full > 0) {
    #pragma unroll
            for (int d = 0; d < kDepth; ++d)
                masked_step(bank0[d], s0 + 4 * d < n_full);
    #pragma unroll
            for (int d = 0; d < kDepth - 1; ++d)
                masked_step(bank1[d], s0 + kBank + 4 * d < n_full);
        }
    }
    // the rest (the split's last, partial step; every step when the host
    // could not allow the full ones): 64-bit indices, both operands of a row
    // past the split zeroed
    for (int s = first_tail + ((wave - first_tail) & 3); s < n_steps; s += 4) {
        const int64_t r = k_begin + int64_t{kDirectK} * s + row;
        const bool valid = r < k_end;
        DirectLoad<kBI> ld{};
        if (valid) {
            const int64_t e = r * a.n_cols + j0 + col_in;
            ld.packed4 = *reinterpret_cast<const uint32_t *>(a.packed + (e >> 1));
            ld.code = a.scale_codes[e >> lb];
            ld.absmax = a.nested_absmax[(e >> lb) >> kNestedLog2];
#pragma unroll
            for (int bi = 0; bi < kBI; ++bi) {
                const int64_t i = i0 + min(D::src1_row(lane, bi), i_last);
                ld.b[bi] = kSrc1Transposed ? a.src1[i * a.ld + r] : a.src1[r * a.ld + i];
            }
        }
        float v[8];
        decode(ld, v);
#pragma unroll
        for (int bj = 0; bj < 8; ++bj)
#pragma unroll
            for (int bi = 0; bi < kBI; ++bi)
                acc[bi][bj] = D::mma(valid ? ld.b[bi] : 0.0f, valid ? v[bj] : 0.0f, acc[bi][bj]);
    }

    // partial tiles: (w0 + w2) + (w1 + w3), through one LDS buffer in three
    // rounds (a buffer per pair of waves would double the kernel's LDS and
    // cost resident workgroups); lds_red[q * 64 + lane], q = (bi * 8 + bj) * 4 + v
    const auto put = [&]() {
#pragma unroll
        for (int bi = 0; bi < kBI; ++bi)
#pragma unroll
            for (int bj = 0; bj < 8; ++bj)
#pragma unroll
                for (int v = 0; v < D::kAccV; ++v)
                    lds_red[((bi * 8 + bj) * 4 + v) * 64 + lane] = acc[bi][bj][v];
    };
    const auto add = [&]() {
#pragma unroll
        for (int bi = 0; bi < kBI; ++bi)
#pragma unroll
            for (int bj = 0; bj < 8; ++bj)
#pragma unroll
                for (int v = 0; v < D::kAccV; ++v)
                    acc[bi][bj][v] = acc[bi][bj][v] + lds_red[((bi * 8 + bj) * 4 + v) * 64 + lane];
    };
    if (wave == 2)
        put();
    __syncthreads();
    if (wave == 0)
        add();  // w0 + w2
    __syncthreads();
    if (wave == 3)
        put();
    __syncthreads();
    if (wave == 1)
        add();  // w1 + w3
    __syncthreads();
    if (wave == 1)
        put();
    __syncthreads();
    if (wave != 0)
        return;
    float *out = a.part + int64_t{split} * a.m * a.n_cols;
    if constexpr (D::kQuad || D::kVec) {
        // the lane groups of the four weight rows, (g0 + g1) + (g2 + g3), with
        // every lane of the wave still active for the exchanges
#pragma unroll
        for (int bi = 0; bi < kBI; ++bi)
#pragma unroll
            for (int bj = 0; bj < 8; ++bj)
#pragma unroll
                for (int v = 0; v < D::kAccV; ++v) {
                    float x = acc[bi][bj][v] + lds_red[((bi * 8 + bj) * 4 + v) * 64 + lane];
                    x = x + __shfl_xor(x, 16);
                    acc[bi][bj][v] = x + __shfl_xor(x, 32);
                }
        if (row != 0 || j0 + 8 * c >= a.n_cols)
            return;
#pragma unroll
        for (int bi = 0; bi < kBI; ++bi)
#pragma unroll
            for (int v = 0; v < D::kAccV; ++v) {
                const int64_t i = i0 + 4 * bi + v;  // the accumulator's row v of set bi
                if (i >= a.m)
                    continue;
                float *o = out + i * a.n_cols + j0 + 8 * c;
#pragma unroll
                for (int bj = 0; bj < 8; ++bj)
                    o[bj] = acc[bi][bj][v];
            }
    } else {
        if (j0 + 8 * c >= a.n_cols)
            return;
#pragma unroll
        for (int bi = 0; bi < kBI; ++bi)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                // the accumulator's row 4 * row + v (see Shape::acc_row) of block bi
                const int64_t i = i0 + kBI * (4 * row + v) + bi;
                if (i >= a.m)
                    continue;
                float *o = out + i * a.n_cols + j0 + 8 * c;
#pragma unroll
                for (int bj = 0; bj < 8; ++bj)
                    o[bj] = acc[bi][bj][v] + lds_red[((bi * 8 + bj) * 4 + v) * 64 + lane];
            }
    }
}

// dst[x] = part[0][x] + part[1][x] + ... in split order.  Each thread loads
// kReduceBatch partials before adding them in order, so that the loads
// overlap (one at a time, the call was bound by their latency: 14 us for 36
// splits of a 16 x 5376 dst); the sum is the plain loop's.
constexpr int kReduceBatch = 8;

__global__ __launch_bounds__(kThreads) void out_prod_reduce_kernel(const float *part, float *dst,
                                                                   int64_t count, int splits)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t x = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; x < count;
         x += stride) {
        float sum = part[x];
        int s = 1;
        for (; s + kReduceBatch <= splits; s += kReduceBatch) {
            float v[kReduceBatch];
#pragma unroll
            for (int q = 0; q < kReduceBatch; ++q)
                v[q] = part[int64_t{s + q} * count + x];
#pragma unroll
            for (int q = 0; q < kReduceBatch; ++q)
                sum = sum + v[q];
        }
        for (; s < splits; ++s)
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

// A transposed src1 (m rows of n_rows floats, leading dimension ld) copied
// into a row-major n_rows x m buffer: out[r * m + i] = src1[i * ld + r].  One
// workgroup moves a 64 x 64 tile through LDS: it reads 64 consecutive floats
// of each src1 row and writes each out row's run of the tile's columns (for
// m <= 64 the tile's rows of out are one contiguous span).  Bit copies only.
constexpr int kTrTile = 64;

// The grid is (tiles of 64 rows r, tiles of 64 columns i).
__global__ __launch_bounds__(kThreads) void src1_transpose_kernel(const float *src1, int64_t ld,
                                                                  int64_t m, int64_t n_rows,
                                                                  float *out)
{
    __shared__ float tile[kTrTile][kTrTile + 1];
    const int t = threadIdx.x;
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kTrTile;
    const int64_t i0 = static_cast<int64_t>(blockIdx.y) * kTrTile;
    const int nr = static_cast<int>(min(int64_t{kTrTile}, n_rows - r0));
    const int ni = static_cast<int>(min(int64_t{kTrTile}, m - i0));
    // every lane's 16 loads are issued before any is stored (a loop that
    // stored each load before the next ran the copy at about 3 TB/s)
    constexpr int kPer = kTrTile * kTrTile / kThreads;
    float v[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int k = t + q * kThreads;
        const int ii = k / kTrTile, rr = k % kTrTile;
        v[q] = ii < ni && rr < nr ? src1[(i0 + ii) * ld + r0 + rr] : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int k = t + q * kThreads;
        tile[k / kTrTile][k % kTrTile] = v[q];
    }
    __syncthreads();
    // lanes step through the tile's rows in runs of the next power of two
    // of ni (shifts, not a division: the compiler expands a 32-bit division
    // into floating-point instructions); nr << lg <= 64 * 64
    const int lg = 32 - __clz(ni - 1);  // ni >= 1; ni == 1 gives 0
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int k = t + q * kThreads;
        const int rr = k >> lg, ii = k & ((1 << lg) - 1);
        if (rr < nr && ii < ni)
            out[(r0 + rr) * m + i0 + ii] = tile[ii][rr];
    }
}

int64_t ceil_div(int64_t a, int64_t b)
{
    return (a + b - 1) / b;
}

// The kernel for a launch (see plan_for).  `variant` (0..43) indexes the
// kernel for the occupancy cache.
struct Plan {
    const void *kernel;
    int tile_i;
    int variant;
    bool direct;  // out_prod_direct_kernel (its full steps may take unchecked loads)
};

template <int kTileI>
const void *staged_kernel(bool transposed)
{
    return transposed ? reinterpret_cast<const void *>(&out_prod_fused_kernel<kTileI, true>)
                      : reinterpret_cast<const void *>(&out_prod_fused_kernel<kTileI, false>);
}

// Relative work per dst row of each staged i-tile width, measured on the
// output head with m a multiple of the width (FP32 TFLOP/s 128 / 109 / 93 at
// widths 256 / 128 / 64): the decode cost of a stage is shared by more rows
// in a wider tile.  A ragged m pays for its padded rows, so the width that
// minimizes padded rows x relative cost wins.
double tile_cost(int64_t m, int64_t tile_i)
{
    const double rel = tile_i == 256 ? 1.0 : tile_i == 128 ? 1.17 : 1.37;
    return static_cast<double>(ceil_div(m, tile_i) * tile_i) * rel;
}

template <int kBI, int kMode = 0>
const void *direct_kernel(bool transposed, bool whole)
{
    if (whole)
        return transposed
                   ? reinterpret_cast<const void *>(&out_prod_direct_kernel<kBI, kMode, true, true>)
                   : reinterpret_cast<const void *>(&out_prod_direct_kernel<kBI, kMode, false, true>);
    return transposed
               ? reinterpret_cast<const void *>(&out_prod_direct_kernel<kBI, kMode, true, false>)
               : reinterpret_cast<const void *>(&out_prod_direct_kernel<kBI, kMode, false, false>);
}

// The kernel for m dst rows.  The aligned path takes the direct kernel's
// tiles: the vector-unit row for m == 1, the 4-row sets for m <= 8, then 16,
// 32, 48 or 64 rows (m > 64 repeats the 64-row tile over the rows; the call
// splits such m into whole 64-row tiles and a smaller rest, see row_ranges).
// The byte path takes the staged kernel.  `whole`: a direct step of 4 weight
// rows spans whole blocks (4 * n_cols is a multiple of the block size).
Plan plan_for(int64_t m, bool transposed, bool aligned8, bool whole)
{
    const int t = (transposed ? 1 : 0) + (whole ? 14 : 0);
    if (aligned8) {
        if (m == 1)
            return {direct_kernel<1, 2>(transposed, whole), 1, 28 + t, true};
        if (m <= 4)
            return {direct_kernel<1, 1>(transposed, whole), 4, 24 + t, true};
        if (m <= 8)
            return {direct_kernel<2, 1>(transposed, whole), 8, 26 + t, true};
        if (m <= 16)
            return {direct_kernel<1>(transposed, whole), 16, 16 + t, true};
        if (m <= 32)
            return {direct_kernel<2>(transposed, whole), 32, 18 + t, true};
        if (m <= 48)
            return {direct_kernel<3>(transposed, whole), 48, 22 + t, true};
        return {direct_kernel<4>(transposed, whole), 64, 20 + t, true};
    }
    const int ts = transposed ? 1 : 0;
    if (m <= 16)
        return {staged_kernel<16>(transposed), 16, 2 * ts, false};
    int64_t best = 64;
    for (const int64_t w : {128, 256})
        if (tile_cost(m, w) < tile_cost(m, best))
            best = w;
    if (best == 256)
        return {staged_kernel<256>(transposed), 256, 12 + 2 * ts, false};
    if (best == 128)
        return {staged_kernel<128>(transposed), 128, 8 + 2 * ts, false};
    return {staged_kernel<64>(transposed), 64, 4 + 2 * ts, false};
}

constexpr int kVariants = 44;
constexpr int kMaxDevices = 64;
std::atomic<int> g_resident[kMaxDevices][kVariants];

// Workgroups of the plan's kernel resident at once on one CU of `device` (at
// least 1), asked of the runtime once per device and kernel.  The kernels use
// no dynamic LDS, so the answer depends on the kernel alone.
int resident_per_cu(const Plan &plan, int device)
{
    std::atomic<int> *slot = device >= 0 && device < kMaxDevices
                                 ? &g_resident[device][plan.variant]
                                 : nullptr;
    int n = slot ? slot->load(std::memory_order_relaxed) : 0;
    if (n > 0)
        return n;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, plan.kernel, kThreads, 0) !=
            hipSuccess ||
        n < 1) {
        (void)hipGetLastError();
        return 1;  // not cached: the next call asks again
    }
    if (slot)
        slot->store(n, std::memory_order_relaxed);
    return n;
}

// The split of the rows.  Workgroups all do the same work, so the kernel
// takes ceil(groups / resident) rounds of resident workgroups; the preferred
// split count is the smallest that brings the fraction of occupied slots,
// groups / (rounds * resident), within 2 % of the best reachable with at most
// kMaxSplits splits and at least kMinRowsPerSplit rows per split.  The call
// takes the largest count up to that one whose partial tiles the workspace
// holds (max_partials), so a workspace of the preferred size gives the
// preferred split.  Returns the rows per split.
int64_t rows_per_split(int64_t n_rows, int64_t tiles, int64_t resident, int64_t max_partials)
{
    const auto occupied = [&](int64_t splits) {
        const int64_t groups = tiles * splits;
        return static_cast<double>(groups) /
               static_cast<double>(ceil_div(groups, resident) * resident);
    };
    const int64_t s_max = min(ceil_div(n_rows, kMinRowsPerSplit), kMaxSplits);
    double best = occupied(1);
    for (int64_t s = 2; s <= s_max; ++s)
        best = std::max(best, occupied(s));
    int64_t splits = 1;
    while (splits < s_max && occupied(splits) < 0.98 * best)
        ++splits;
    splits = max(int64_t{1}, min(splits, max_partials));
    return ceil_div(ceil_div(n_rows, splits), kStage) * kStage;
}

// Whether the direct kernel's full steps may address a split of `rows` rows
// (at most) from one base per array with 32-bit offsets: its rows * n_cols
// weight elements plus a block offset under 4096 (and the lanes' columns),
// and the floats of src1 it reads -- rows * ld + tile_i, or tile_i * ld +
// rows when transposed -- as bytes.  Otherwise every step takes the checked
// loads.
bool direct_split_fits(int64_t rows, int64_t n_cols, int64_t ld, int tile_i, bool transposed)
{
    constexpr int64_t k32 = int64_t{1} << 32, kFloats = k32 / 4;
    if (rows >= k32 / n_cols || rows * n_cols + 8192 >= k32)
        return false;
    return transposed ? ld < kFloats / tile_i && tile_i * ld + rows < kFloats
                      : ld < kFloats / rows && rows * ld + tile_i < kFloats;
}

// A call's dst rows are covered by at most two ranges, each with its own plan
// and launches: dst row i depends on src1 column i alone, so a range is the
// same operation on a column slice of src1.  On the aligned path m > 64
// takes whole 64-row direct tiles for its first 64 * floor(m / 64) rows and
// the best smaller tile for the rest.  The 64-row direct tile costs no more
// per dst row than the staged kernel's 256-row tile (output head, row-major
// src1: 1.58 against 1.67 ms at m = 128, 6.19 against 6.41 ms at m = 512,
// 12.09 against 12.79 ms at m = 1024), and the rest pays for its own rows
// rather than for a padded wide tile (m = 192: 2.37 against 3.58 ms).
struct RowRange {
    int64_t i_begin;  // first dst row (src1 column) of the range
    int64_t m;        // its dst rows
    Plan plan;
};

int row_ranges(int64_t m, bool transposed, bool aligned8, bool whole_blocks, RowRange (&r)[2])
{
    if (aligned8 && m > 64) {
        const int64_t whole = m / 64 * 64;
        r[0] = {0, whole, plan_for(64, transposed, true, whole_blocks)};
        if (whole == m)
            return 1;
        r[1] = {whole, m - whole, plan_for(m - whole, transposed, true, whole_blocks)};
        return 2;
    }
    r[0] = {0, m, plan_for(m, transposed, aligned8, whole_blocks)};
    return 1;
}

// Bytes of partial tiles the preferred row split of each of the ranges
// writes (0 when each prefers one split); the ranges use the workspace one
// after the other, so the largest counts.
int64_t partial_bytes(const RowRange *r, int n_ranges, int64_t n_rows, int64_t n_cols,
                      int device)
{
    int64_t bytes = 0;
    for (int k = 0; k < n_ranges; ++k) {
        const int64_t tiles = ceil_div(r[k].m, r[k].plan.tile_i) * ceil_div(n_cols, kTileJ);
        const int64_t resident =
            int64_t{compute_units(device)} * resident_per_cu(r[k].plan, device);
        const int64_t rps = rows_per_split(n_rows, tiles, resident, kMaxSplits);
        const int64_t splits = ceil_div(n_rows, rps);
        if (splits > 1)
            bytes = std::max(bytes, splits * r[k].m * n_cols * 4);
    }
    return bytes;
}

int64_t preferred_partial_bytes(int64_t n_rows, int64_t n_cols, int64_t m, bool transposed,
                                bool aligned8, bool whole, int device)
{
    RowRange ranges[2];
    const int n_ranges = row_ranges(m, transposed, aligned8, whole, ranges);
    return partial_bytes(ranges, n_ranges, n_rows, n_cols, device);
}

// Bytes of a row-major copy of `cols` columns of a transposed src1 in the
// workspace (rounded so that the partials after it stay 256-byte aligned).
int64_t src1_copy_bytes(int64_t n_rows, int64_t cols)
{
    return (n_rows * cols * 4 + 255) / 256 * 256;
}

// A transposed src1 in the 48- and 64-row direct tiles reads 16 lines per
// load where a row-major one reads 4, and a row-major copy of the range's
// columns pays for itself in every 64-row range and in a 48-row one with at
// least 40 rows.  Measured on the output head against the in-place read:
// m = 44 .. 64 and whole 64-row ranges 1.4-7 % faster with the copy (m = 50
// .. 54, a 64-row tile at 3/4 use, 1.4-1.7 %), m = 40 .. 42 within 1 %, and
// m = 33 .. 36 (a sparse 48-row tile, whose unused lanes share lines with
// the used ones) 0.5 % slower.  The narrower tiles (4-row sets, and the 16-
// and 32-row tiles with their super-steps) were within 1 % either way.
bool copy_pays(const RowRange &r)
{
    return r.plan.direct && (r.plan.tile_i == 64 || (r.plan.tile_i == 48 && r.m >= 40));
}

// For a transposed src1 on the aligned path: marks the ranges whose columns
// go through the row-major copy, re-plans them row-major, and sets the
// copied columns [*c0, *c1) (the copied ranges are adjacent).  Returns the
// copy's bytes (0: nothing is copied).
int64_t plan_copy(int64_t n_rows, int64_t m, bool whole, RowRange (&r)[2], int n_ranges,
                  bool (&copied)[2], int64_t *c0, int64_t *c1)
{
    *c0 = *c1 = 0;
    copied[0] = copied[1] = false;
    if (m <= 1 || n_rows > INT64_MAX / 8 / m)
        return 0;
    for (int k = 0; k < n_ranges; ++k) {
        if (!copy_pays(r[k]))
            continue;
        if (*c1 == *c0)
            *c0 = r[k].i_begin;
        *c1 = r[k].i_begin + r[k].m;
        copied[k] = true;
        r[k].plan = plan_for(r[k].m, false, true, whole);
    }
    return *c1 > *c0 ? src1_copy_bytes(n_rows, *c1 - *c0) : 0;
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

int64_t dq4_out_prod_fused_workspace_bytes(int64_t n_rows, int64_t n_cols, int64_t m,
                                           int32_t src1_transposed)
{
    if (n_rows <= 0 || n_cols <= 0 || m <= 0 || n_cols > INT64_MAX / m ||
        m * n_cols > INT64_MAX / 4 / dq4::kMaxSplits || n_rows > INT64_MAX / 8 / m ||
        (src1_transposed != 0 && src1_transposed != 1))
        return 0;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess)
        return 0;
    // a one-column src1 reads the same memory in either orientation
    const bool transposed = src1_transposed != 0 && m > 1;
    // the largest partials any kernel variant would write for this shape and
    // orientation (packed alignment and block size are not known here)
    int64_t bytes = 0;
    for (int v = 0; v < 4; ++v)
        bytes = std::max(bytes, dq4::preferred_partial_bytes(n_rows, n_cols, m, transposed,
                                                             (v & 1) != 0, (v & 2) != 0, device));
    // a transposed src1 on an aligned weight: the row-major copy of the
    // columns whose tiles take it, and the partials of the plan that reads it
    if (transposed && n_cols % 8 == 0)
        for (int whole = 0; whole < 2; ++whole) {
            dq4::RowRange ranges[2];
            const int n_ranges = dq4::row_ranges(m, true, true, whole != 0, ranges);
            bool copied[2];
            int64_t c0 = 0, c1 = 0;
            const int64_t copy =
                dq4::plan_copy(n_rows, m, whole != 0, ranges, n_ranges, copied, &c0, &c1);
            if (copy > 0)
                bytes = std::max(bytes, copy + dq4::partial_bytes(ranges, n_ranges, n_rows,
                                                                  n_cols, device));
        }
    return bytes;
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
    const bool aligned8 = n_cols % 8 == 0 && reinterpret_cast<uintptr_t>(packed) % 4 == 0;
    bool transposed = src1_transposed != 0;
    // blocksize is a power of two >= 32, so 4 * n_cols is a multiple of it
    // exactly when n_cols is a multiple of a quarter of it
    const bool whole_blocks = n_cols % (blocksize / dq4::kDirectK) == 0;
    dq4::RowRange ranges[2];
    int n_ranges = dq4::row_ranges(m, transposed, aligned8, whole_blocks, ranges);
    const int64_t tiles_j = dq4::ceil_div(n_cols, dq4::kTileJ);
    if (n_rows > 0) {
        if (!packed || !scale_codes || !nested_absmax || !scale_codebook || !codebook4 || !src1)
            return DQ4_EINVAL;
        if (transposed ? ld_src1 < n_rows : ld_src1 < m)
            return DQ4_EINVAL;
        if (workspace_bytes > 0 && !workspace)
            return DQ4_EINVAL;
        for (int k = 0; k < n_ranges; ++k) {
            const int64_t tiles_i = dq4::ceil_div(ranges[k].m, ranges[k].plan.tile_i);
            if (tiles_i > 0x7FFFFFFF || tiles_j > 0x7FFFFFFF || tiles_i * tiles_j > 0x7FFFFFFF)
                return DQ4_EUNSUPPORTED;
        }
    }
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess)
        return dq4::hip_failed(e);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // each range's src1: where its values are, their leading dimension and
    // orientation
    const float *r_src[2];
    int64_t r_ld[2];
    bool r_tr[2];
    for (int k = 0; k < n_ranges; ++k) {
        r_tr[k] = transposed;
        r_ld[k] = ld_src1;
        r_src[k] = transposed ? src1 + ranges[k].i_begin * ld_src1 : src1 + ranges[k].i_begin;
    }
    if (n_rows > 0 && transposed && m == 1) {
        // one src1 row: B[r][0] = src1[r], the row-major layout with ld 1
        r_tr[0] = false;
        r_ld[0] = 1;
        r_src[0] = src1;
        n_ranges = dq4::row_ranges(m, false, aligned8, whole_blocks, ranges);
    } else if (n_rows > 0 && transposed && aligned8) {
        // The ranges whose tiles read a transposed src1 badly (copy_pays) take
        // a row-major copy of their columns when the workspace holds it and the
        // partials of the plan that reads it: one more kernel writes the copy
        // at the start of the workspace, and those ranges run as for a
        // row-major src1 on it, with the rest of the workspace.
        dq4::RowRange planned[2];
        for (int k = 0; k < n_ranges; ++k)
            planned[k] = ranges[k];
        bool copied[2];
        int64_t c0 = 0, c1 = 0;
        const int64_t copy_bytes = dq4::plan_copy(n_rows, m, whole_blocks, planned, n_ranges,
                                                  copied, &c0, &c1);
        const int64_t tiles_r = dq4::ceil_div(n_rows, dq4::kTrTile);
        const int64_t tiles_c = dq4::ceil_div(c1 - c0, dq4::kTrTile);
        if (copy_bytes > 0 && tiles_r <= 0x7FFFFFFF && tiles_c <= 65535 &&
            workspace_bytes >= copy_bytes + dq4::partial_bytes(planned, n_ranges, n_rows,
                                                               n_cols, device)) {
            const float *in = src1 + c0 * ld_src1;
            int64_t ld_in = ld_src1, cols = c1 - c0, nr = n_rows;
            float *copy = workspace;
            void *params[] = {&in, &ld_in, &cols, &nr, &copy};
            e = hipLaunchKernel(reinterpret_cast<const void *>(&dq4::src1_transpose_kernel),
                                dim3(static_cast<uint32_t>(tiles_r),
                                     static_cast<uint32_t>(tiles_c)),
                                dim3(dq4::kThreads), params, 0, s);
            if (e != hipSuccess)
                return dq4::hip_failed(e);
            for (int k = 0; k < n_ranges; ++k) {
                ranges[k] = planned[k];
                if (copied[k]) {
                    r_tr[k] = false;
                    r_ld[k] = cols;
                    r_src[k] = copy + (ranges[k].i_begin - c0);
                }
            }
            workspace += copy_bytes / 4;
            workspace_bytes -= copy_bytes;
        }
    }
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

    // every range's launch is set up (and checked) before the first is enqueued
    struct Launch {
        dq4::FusedArgs args;
        int64_t groups, splits, count;
        float *dst;  // the range's first dst row
    } launches[2];
    for (int k = 0; k < n_ranges; ++k) {
        const dq4::RowRange &r = ranges[k];
        const dq4::Plan &plan = r.plan;
        const int64_t tiles_i = dq4::ceil_div(r.m, plan.tile_i);
        const int64_t r_count = r.m * n_cols;
        const int64_t max_partials = workspace_bytes / 4 / r_count;
        const int64_t resident =
            int64_t{dq4::compute_units(device)} * dq4::resident_per_cu(plan, device);
        const int64_t rps =
            dq4::rows_per_split(n_rows, tiles_i * tiles_j, resident, max_partials);
        const int64_t splits = dq4::ceil_div(n_rows, rps);
        const int64_t groups = splits * tiles_i * tiles_j;
        // the kernels count a split's stages (16 rows) or steps (4 rows) in 32 bits
        if (groups > 0x7FFFFFFF || dq4::ceil_div(rps, dq4::kDirectK) > 0x7FFFFFFF)
            return DQ4_EUNSUPPORTED;
        const bool full = plan.direct && dq4::direct_split_fits(rps, n_cols, r_ld[k],
                                                                 plan.tile_i, r_tr[k]);
        float *r_dst = dst + r.i_begin * n_cols;
        launches[k] = {{packed, scale_codes, nested_absmax, scale_codebook, codebook4, r_src[k],
                        splits > 1 ? workspace : r_dst, n_rows, n_cols, r.m, r_ld[k], rps,
                        offset, log2_block, static_cast<int>(tiles_i),
                        static_cast<int>(tiles_j), full ? 1 : 0},
                       groups, splits, r_count, r_dst};
    }
    // the ranges run one after the other on the stream, so the second reuses
    // the workspace once the first range's reduction has read it
    for (int k = 0; k < n_ranges; ++k) {
        Launch &l = launches[k];
        void *params[] = {&l.args};
        e = hipLaunchKernel(ranges[k].plan.kernel, dim3(static_cast<uint32_t>(l.groups)),
                            dim3(dq4::kThreads), params, 0, s);
        if (e != hipSuccess)
            return dq4::hip_failed(e);
        if (l.splits > 1) {
            uint32_t grid = 0;
            dq4::grid_size(l.count, device, &grid);
            const float *p = workspace;
            float *d = l.dst;
            int64_t c = l.count;
            int sp = static_cast<int>(l.splits);
            void *rparams[] = {&p, &d, &c, &sp};
            e = hipLaunchKernel(reinterpret_cast<const void *>(&dq4::out_prod_reduce_kernel),
                                dim3(grid), dim3(dq4::kThreads), rparams, 0, s);
            if (e != hipSuccess)
                return dq4::hip_failed(e);
        }
    }
    return DQ4_OK;
}

}  // extern "C"

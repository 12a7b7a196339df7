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
// Design (an HBM-bound stream, 0.5 B read per 2 or 4 B written; no matrix
// cores: nothing here is a contraction):
//  * one workgroup of 256 lanes per tile of 4096 elements (2 KiB packed in,
//    8 or 16 KiB out).  The tile is cut into "units" of 8 elements (one
//    packed dword) for FP16/BF16 output or 4 elements (one packed 16-bit
//    word) for FP32 output; lane t takes unit u * 256 + t (FP16/BF16) or one
//    of its wave's contiguous run of units (FP32), so each wavefront load is
//    contiguous and each store instruction writes 64 x 16 contiguous bytes
//    for every output type.  One tile per workgroup, in dispatch order,
//    keeps the set of addresses being written compact; on MI355X this writes
//    markedly faster than a persistent grid-stride loop, and 4096-element
//    tiles measured faster than 2048 (by ~45 %), 6144 (~0.3 %) and 8192
//    (~10 %) elements;
//  * the packed loads are issued first (non-temporal for FP16/BF16 output:
//    each byte is read once); while they are in flight the workgroup rebuilds the scale of each outer block its tile touches (at
//    most 129), one block per lane, into LDS -- so the scale is computed once
//    per block, never stored to HBM, and the value pass reads it from LDS;
//  * the 256-entry scale codebook and the 16-entry value codebook sit in LDS;
//    the 16-entry table covers 16 distinct banks, so lookups never conflict;
//  * since blocksize >= 32 and the window starts on a multiple of 8, the
//    elements of a unit share one outer block;
//  * outputs are written with 16-byte buffer stores marked nt and sc1
//    (streamed at device scope; ~3 % faster than nt alone on MI355X);
//  * with blocksize >= 64, neighbouring tiles read the same 128-byte line of
//    scale codes; for FP16/BF16 output the slot -> tile map puts such tiles
//    on one XCD so that the line is fetched from HBM once (workgroups go to
//    the 8 XCDs in turn, and each XCD has its own L2).  FP32 output measured
//    faster with plain loads in dispatch order (kStreamPolicy);
//  * the partial last tile goes through a per-element path that computes the
//    same bits; windows that miss the alignment of this path take a general
//    vector path (dq4_shift_tile_kernel, output-aligned tiles with
//    funnel-shifted packed words), and only outputs that are not even
//    element-aligned take the per-element path throughout.
// No scratch memory: nothing but the inputs and the output touches HBM.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>

#include "dq4.h"
#include "dq4_device.h"

#pragma clang fp contract(off)

namespace dq4 {
namespace {

constexpr int kThreads = 256;
constexpr int kDwordsPerLane = 2;
constexpr int kTileDwords = kThreads * kDwordsPerLane;
constexpr int kTileElems = kTileDwords * 8;    // 4096
constexpr int kMaxTileBlocks = kTileElems / 32 + 1;  // blocksize 32, tile not block-aligned
constexpr int kElemBlocksPerCU = 8;            // grid of the per-element path
constexpr int kOutAlign = 128;    // output alignment of the vector tiles (bytes)
constexpr int kXcds = 8;          // MI355X: 8 accelerator dies, each with its own L2
constexpr int kLog2MaxShare = 3;  // pair up at most 8 tiles per line of scale codes

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

// Fill the two codebooks in LDS (every lane must call it; ends on a barrier).
__device__ __forceinline__ void load_tables(const Args &a, float *lds_scb, float *lds_cb4)
{
    const int t = threadIdx.x;
    const float sv = a.scale_codebook[t];
    const float cv = t < 16 ? a.codebook4[t] : 0.0f;
    lds_scb[t] = sv;
    if (t < 16)
        lds_cb4[t] = cv;
    __syncthreads();
}

// One element, any alignment: used for the partial last tile and for windows
// the vector path cannot take.  j is the index within the window.
template <int OUT>
__device__ __forceinline__ void one_element(const Args &a, const float *lds_scb,
                                            const float *lds_cb4, int64_t j)
{
    const int64_t i = a.e0 + j;
    const int64_t b = i >> a.log2_block;
    const float s = block_scale(lds_scb[a.scale_codes[b]], a.nested_absmax[b >> kNestedLog2],
                                a.offset);
    const uint32_t byte = a.packed[i >> 1];
    const uint32_t k = (i & 1) ? (byte >> 4) : (byte & 0xFu);
    store1<OUT>(a.out, j, lds_cb4[k] * s);
}

// Workgroups are dispatched to the XCDs in turn (workgroup i to XCD i mod 8),
// and each XCD has its own L2.  With blocksize 2^lb, 2^(lb-5) consecutive
// tiles read the same 128-byte line of scale codes; this bijection of each
// aligned group of 8 * 2^s slots gives those 2^s tiles slots that are 8
// apart, hence one XCD, so the line is fetched from HBM once, not 2^s times.
__device__ __forceinline__ int64_t xcd_paired_tile(int64_t slot, int s)
{
    const int64_t group = slot & ~((int64_t{kXcds} << s) - 1);
    const int64_t x = slot - group;
    return group | ((x % kXcds) << s) | (x / kXcds);
}

// Vector path.  Requires e0 % 8 == 0, packed + e0/2 4-byte aligned and out
// 16-byte aligned (the launcher sends it 128-byte aligned outputs only, see
// kOutAlign).  Tiles [0, n_full) are full; tile n_full (if any) is the
// partial last tile, run by slot 0.  Normally gridDim.x == n_tiles and each workgroup runs
// one tile; the loop only matters for grids capped below the tile count.
template <int OUT>
__global__ __launch_bounds__(kThreads) void dq4_tile_kernel(Args a, int64_t n_full,
                                                            int64_t n_tiles)
{
    __shared__ float lds_scb[256];
    __shared__ float lds_cb4[16];
    __shared__ float lds_scale[kMaxTileBlocks];

    const int t = threadIdx.x;
    const int lb = a.log2_block;

    // FP16/BF16: tiles that read the same 128-byte line of scale codes run on
    // one XCD (FP32 keeps dispatch order; see kStreamPolicy)
    const int log2_share = min(lb - 5, kLog2MaxShare);  // tiles per line of codes
    const int64_t n_paired =
        kStreamPolicy<OUT> ? n_full & ~((int64_t{kXcds} << log2_share) - 1) : 0;
    // the partial tile, if any, goes to the first slot: dispatched last, its
    // per-element work would add to the end of the launch
    const int64_t edge = n_tiles - n_full;  // 1 or 0
    for (int64_t slot = blockIdx.x; slot < n_tiles; slot += gridDim.x) {
        if (slot < edge) {
            load_tables(a, lds_scb, lds_cb4);
            for (int64_t j = n_full * kTileElems + t; j < a.count; j += kThreads)
                one_element<OUT>(a, lds_scb, lds_cb4, j);
            __syncthreads();
            continue;
        }
        const int64_t fs = slot - edge;  // full-tile slot
        const int64_t tile = fs < n_paired ? xcd_paired_tile(fs, log2_share) : fs;
        const int64_t d0 = tile * kTileDwords;  // first packed dword of the tile

        // 1. packed data first: the longest-latency loads.  The waves issue
        //    this tile's loads at raised priority (an issue-arbitration hint
        //    within the CU), ahead of waves busy in their value pass: a
        //    workgroup's life is mostly the wait for these loads, and the
        //    FP16 launch measured ~0.4 % faster.  FP32 output keeps the
        //    default priority: raised, it ran ~7 % slower
        if constexpr (kStreamPolicy<OUT>)
            __builtin_amdgcn_s_setprio(3);
        using Word = typename Unit<OUT>::Word;
        constexpr int E = Unit<OUT>::kElems;
        constexpr int kUnits = kDwordsPerLane * 8 / E;  // units per lane and tile
        const Word *words = reinterpret_cast<const Word *>(a.packed + (a.e0 >> 1));
        const int64_t u0 = d0 * 8 / E;  // first unit of the tile
        Word w[kUnits];
#pragma unroll
        for (int u = 0; u < kUnits; ++u)
            w[u] = load_packed<OUT>(tile_word<OUT, kUnits>(words + u0, u, t));

        // 2. metadata of the outer blocks this tile touches, one block per lane
        const int64_t e_tile = a.e0 + d0 * 8;
        const int64_t b0 = e_tile >> lb;
        const uint32_t r = static_cast<uint32_t>(e_tile - (b0 << lb));  // offset in block b0
        const int n_blocks = static_cast<int>((r + kTileElems - 1) >> lb) + 1;
        const bool has0 = t < n_blocks;
        const bool has1 = t + kThreads < n_blocks;
        uint32_t code0 = 0, code1 = 0;
        float absmax0 = 0.0f, absmax1 = 0.0f;
        if (has0) {
            code0 = a.scale_codes[b0 + t];
            absmax0 = a.nested_absmax[(b0 + t) >> kNestedLog2];
        }
        if (has1) {
            code1 = a.scale_codes[b0 + t + kThreads];
            absmax1 = a.nested_absmax[(b0 + t + kThreads) >> kNestedLog2];
        }

        // 3. codebooks to LDS, then every block's scale to LDS
        load_tables(a, lds_scb, lds_cb4);
        if constexpr (kStreamPolicy<OUT>)
            __builtin_amdgcn_s_setprio(0);
        if (has0)
            lds_scale[t] = block_scale(lds_scb[code0], absmax0, a.offset);
        if (has1)
            lds_scale[t + kThreads] = block_scale(lds_scb[code1], absmax1, a.offset);
        __syncthreads();

        // 4. value pass: E elements per unit, one 16-byte store per unit
        const __amdgpu_buffer_rsrc_t dst = unit_buffer(a.out, u0, kUnits * kThreads);
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const uint32_t ul = tile_unit<OUT, kUnits>(u, t);
            const float s = lds_scale[(r + ul * E) >> lb];
            float v[E];
#pragma unroll
            for (int e = 0; e < E; ++e)
                v[e] = lds_cb4[(static_cast<uint32_t>(w[u]) >> (4 * e)) & 0xFu] * s;
            store_unit<OUT>(dst, ul, v);
        }
        __syncthreads();  // LDS is rewritten by the next tile of this workgroup
    }
}

// General vector path, for windows that miss the alignment of dq4_tile_kernel
// (start element, packed or output pointer) but whose output is
// element-aligned.  Tiles are aligned to the output instead of the packed
// bytes: the first `head` outputs (up to the first 128-byte boundary of
// `out`; stores that start mid-line run ~40 % slower on MI355X) and the last
// partial tile are computed element by element by the workgroup of slot 0,
// so that their latency overlaps the full tiles; every full tile of 4096
// outputs after the head is a dq4_tile_kernel tile whose units take their
// nibbles from two neighbouring packed dwords, funnel-shifted by a bit
// offset that is the same for the whole window (one dword when that offset
// is 0), and whose elements pick one of two block scales, since a unit may
// straddle two outer blocks.  Every unit starts c = (e0 + head) mod E
// elements past a multiple of E and outer blocks are multiples of E long, so
// a block boundary inside a unit always falls just before its element
// kK0 = E - c: elements below kK0 take the scale of the unit's first element,
// the rest that of its last (the same scale when no boundary falls inside).
// kK0 is a template parameter, so that choice costs nothing per element; a
// per-element compare and select cost ~4 % of the launch.  kK0 == 0 is the
// instantiation for windows whose units each lie in one packed dword (FP32:
// half of one) and one block: one load and one scale per unit, as in
// dq4_tile_kernel.  Compiled separately, it ran an 8-element output shift of
// the 28672 x 8192 headline shape in 93.8-94.1 us against 98.9-99.1 us
// through the general code (a runtime branch inside one kernel gained
// nothing).  The packed bytes are read through a buffer resource that ends
// at the last dword holding a needed nibble: reads past it return zero.
template <int OUT, int kK0>
__global__ __launch_bounds__(kThreads) void dq4_shift_tile_kernel(Args a, int64_t head,
                                                                  int64_t n_full,
                                                                  int64_t n_tiles)
{
    __shared__ float lds_scb[256];
    __shared__ float lds_cb4[16];
    __shared__ float lds_scale[kMaxTileBlocks];

    const int t = threadIdx.x;
    const int lb = a.log2_block;
    constexpr int E = Unit<OUT>::kElems;
    constexpr int kUnits = kDwordsPerLane * 8 / E;  // units per lane and tile
    constexpr int kOutBytes = OUT == DQ4_F32 ? 4 : 2;
    // plain loads: marking these buffer loads non-temporal measured ~14 %
    // slower here (the neighbouring dword each unit also reads is then
    // fetched again rather than found in cache)
    constexpr int kLoadPolicy = 0;

    // packed bits from a 4-byte aligned base: element g's nibble starts at
    // bit base_bits + 4 g
    const uintptr_t p_addr = reinterpret_cast<uintptr_t>(a.packed);
    const uint8_t *pb = a.packed - (p_addr & 3);
    const int64_t base_bits = static_cast<int64_t>(p_addr & 3) * 8;
    const int64_t last_byte = (a.e0 + a.count - 1) >> 1;  // of the needed packed bytes
    const int64_t span = (p_addr & 3) + last_byte + 1;
    const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(pb), 0, static_cast<int32_t>((span + 3) & ~int64_t{3}),
        kRawBufferWord3);
    // the first slot takes the head and the tail when there are any
    const int64_t edge = n_tiles - n_full;  // 1 or 0

    // FP16/BF16: tiles that read the same 128-byte line of scale codes run on
    // one XCD, as in dq4_tile_kernel
    const int log2_share = min(lb - 5, kLog2MaxShare);
    const int64_t n_paired =
        kStreamPolicy<OUT> ? n_full & ~((int64_t{kXcds} << log2_share) - 1) : 0;
    for (int64_t slot = blockIdx.x; slot < n_tiles; slot += gridDim.x) {
        if (slot < edge) {
            load_tables(a, lds_scb, lds_cb4);
            for (int64_t j = t; j < head; j += kThreads)
                one_element<OUT>(a, lds_scb, lds_cb4, j);
            for (int64_t j = head + n_full * kTileElems + t; j < a.count; j += kThreads)
                one_element<OUT>(a, lds_scb, lds_cb4, j);
            __syncthreads();
            continue;
        }
        const int64_t fs = slot - edge;  // full-tile slot
        const int64_t tile = fs < n_paired ? xcd_paired_tile(fs, log2_share) : fs;

        // 1. packed words: unit ul covers global elements g .. g + E - 1,
        //    g = e_tile + ul * E, i.e. bits [4 g, 4 g + 4 E) after the base
        const int64_t e_tile = a.e0 + head + tile * kTileElems;
        const int64_t bit0 = base_bits + 4 * e_tile;
        const uint32_t sh = static_cast<uint32_t>(bit0 & 31);  // the same for every unit
        uint32_t lo[kUnits], hi[kUnits];
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const int64_t bit = bit0 + int64_t{4 * E} * tile_unit<OUT, kUnits>(u, t);
            const int32_t byte = static_cast<int32_t>((bit >> 5) << 2);
            lo[u] = __builtin_amdgcn_raw_buffer_load_b32(src, byte, 0, kLoadPolicy);
            // with sh == 0 every unit's nibbles lie in its first dword
            hi[u] = kK0 != 0 && sh != 0
                        ? __builtin_amdgcn_raw_buffer_load_b32(src, byte + 4, 0, kLoadPolicy)
                        : 0u;
        }

        // 2. metadata of the outer blocks this tile touches, one block per lane
        const int64_t b0 = e_tile >> lb;
        const uint32_t r = static_cast<uint32_t>(e_tile - (b0 << lb));  // offset in block b0
        const int n_blocks = static_cast<int>((r + kTileElems - 1) >> lb) + 1;
        const bool has0 = t < n_blocks;
        const bool has1 = t + kThreads < n_blocks;
        uint32_t code0 = 0, code1 = 0;
        float absmax0 = 0.0f, absmax1 = 0.0f;
        if (has0) {
            code0 = a.scale_codes[b0 + t];
            absmax0 = a.nested_absmax[(b0 + t) >> kNestedLog2];
        }
        if (has1) {
            code1 = a.scale_codes[b0 + t + kThreads];
            absmax1 = a.nested_absmax[(b0 + t + kThreads) >> kNestedLog2];
        }

        // 3. codebooks to LDS, then every block's scale to LDS
        load_tables(a, lds_scb, lds_cb4);
        if (has0)
            lds_scale[t] = block_scale(lds_scb[code0], absmax0, a.offset);
        if (has1)
            lds_scale[t + kThreads] = block_scale(lds_scb[code1], absmax1, a.offset);
        __syncthreads();

        // 4. value pass: the unit's nibbles funnel-shifted out of (hi, lo);
        //    element e of the unit is in the unit's first block or the next
        void *out_tile = static_cast<char *>(a.out) + (head + tile * kTileElems) * kOutBytes;
        const __amdgpu_buffer_rsrc_t dst = unit_buffer(out_tile, 0, kUnits * kThreads);
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const uint32_t ul = tile_unit<OUT, kUnits>(u, t);
            const uint32_t first = r + ul * E;             // offset from block b0's start
            float v[E];
            if constexpr (kK0 == 0) {
                // one dword (FP32: half of one) and one block per unit
                const uint32_t word = lo[u] >> ((sh + 4 * E * ul) & 31);
                const float s = lds_scale[first >> lb];
#pragma unroll
                for (int e = 0; e < E; ++e)
                    v[e] = lds_cb4[(word >> (4 * e)) & 0xFu] * s;
            } else {
                const uint32_t ush = (sh + 4 * E * ul) & 31;  // FP32 units start mid-dword
                const uint32_t word = __builtin_amdgcn_alignbit(hi[u], lo[u], ush);
                const float s_lo = lds_scale[first >> lb];
                const float s_hi = kK0 < E ? lds_scale[(first + E - 1) >> lb] : s_lo;
#pragma unroll
                for (int e = 0; e < E; ++e)
                    v[e] = lds_cb4[(word >> (4 * e)) & 0xFu] * (e < kK0 ? s_lo : s_hi);
            }
            store_unit<OUT>(dst, ul, v);
        }
        __syncthreads();  // LDS is rewritten by the next tile of this workgroup
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

// Memory twin of dq4_tile_kernel<F16> at block size 64: the same 4096-element
// tiles, tile order, non-temporal packed loads and nt sc1 output stores, with
// the dequantization taken out -- each packed dword is written four times
// into its 16-byte output unit.  It moves the headline call's packed and
// output bytes (all but its scale codes, absmax and codebooks) in the same
// pattern, so its time is the ceiling that access pattern reaches on the
// machine it runs on.  A diagnostic: nothing of the method runs here.
__global__ __launch_bounds__(kThreads) void dq4_memory_twin_kernel(const uint32_t *words,
                                                                   void *out, int64_t n_tiles)
{
    constexpr int kUnits = kDwordsPerLane;  // FP16 units: one packed dword each
    const int t = threadIdx.x;
    const int64_t n_paired = n_tiles & ~((int64_t{kXcds} << 1) - 1);  // B = 64: 2 tiles/line
    for (int64_t slot = blockIdx.x; slot < n_tiles; slot += gridDim.x) {
        const int64_t tile = slot < n_paired ? xcd_paired_tile(slot, 1) : slot;
        const int64_t u0 = tile * kTileDwords;
        uint32_t w[kUnits];
#pragma unroll
        for (int u = 0; u < kUnits; ++u)
            w[u] = load_packed<DQ4_F16>(tile_word<DQ4_F16, kUnits>(words + u0, u, t));
        const __amdgpu_buffer_rsrc_t dst = unit_buffer(out, u0, kUnits * kThreads);
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const uint32_t ul = tile_unit<DQ4_F16, kUnits>(u, t);
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[u], w[u], w[u], w[u]}, dst, ul * 16,
                                                   0, kPolicyNT | kPolicySC1);
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {
constexpr int kMaxDevices = 64;
constexpr int64_t kMaxGrid = 0x7FFFFFFF;
std::atomic<int> g_cu_count[kMaxDevices];
thread_local int32_t t_last_hip_error = 0;

int log2_if_pow2(int32_t x)
{
    if (x <= 0 || (x & (x - 1)) != 0)
        return -1;
    int r = 0;
    while ((1 << r) != x)
        ++r;
    return r;
}
}  // namespace

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

dq4_status_t validate_layout(int32_t blocksize, int32_t nested_blocksize, int32_t out_dtype,
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

int32_t last_hip_error()
{
    return t_last_hip_error;
}

namespace {
// The shifted vector path needs an element-aligned output, at least one full
// tile after the head, and packed bytes that a buffer resource can span
// (offsets below 2^31).
bool shift_path_fits(const Args &a, int64_t out_bytes)
{
    if (reinterpret_cast<uintptr_t>(a.out) % out_bytes != 0)
        return false;
    if (a.count < kTileElems + kOutAlign)
        return false;
    const int64_t span = static_cast<int64_t>(reinterpret_cast<uintptr_t>(a.packed) & 3) +
                         ((a.e0 + a.count - 1) >> 1) + 1;
    return span + 8 < (int64_t{1} << 31);
}

// dq4_shift_tile_kernel<OUT, k0> for k0 in 0 .. E (E = 8 for FP16/BF16, 4
// for FP32)
template <int OUT>
const void *shift_kernel(int k0)
{
    switch (k0) {
    case 0: return reinterpret_cast<const void *>(&dq4_shift_tile_kernel<OUT, 0>);
    case 1: return reinterpret_cast<const void *>(&dq4_shift_tile_kernel<OUT, 1>);
    case 2: return reinterpret_cast<const void *>(&dq4_shift_tile_kernel<OUT, 2>);
    case 3: return reinterpret_cast<const void *>(&dq4_shift_tile_kernel<OUT, 3>);
    case 4: return reinterpret_cast<const void *>(&dq4_shift_tile_kernel<OUT, 4>);
    default: break;
    }
    if constexpr (Unit<OUT>::kElems == 8) {
        switch (k0) {
        case 5: return reinterpret_cast<const void *>(&dq4_shift_tile_kernel<OUT, 5>);
        case 6: return reinterpret_cast<const void *>(&dq4_shift_tile_kernel<OUT, 6>);
        case 7: return reinterpret_cast<const void *>(&dq4_shift_tile_kernel<OUT, 7>);
        case 8: return reinterpret_cast<const void *>(&dq4_shift_tile_kernel<OUT, 8>);
        default: break;
        }
    }
    return nullptr;
}

template <int OUT>
dq4_status_t launch_typed(const Args &a, hipStream_t stream)
{
    Args args = a;
    hipError_t e;
    // dq4_tile_kernel: aligned start, packed dwords and a 128-byte aligned
    // output (16-byte aligned stores that start mid-line run ~40 % slower)
    const bool vec = (a.e0 % 8 == 0) &&
                     (reinterpret_cast<uintptr_t>(a.packed + (a.e0 >> 1)) % 4 == 0) &&
                     (reinterpret_cast<uintptr_t>(a.out) % kOutAlign == 0);
    if (vec) {
        int64_t n_full = a.count / kTileElems;
        int64_t n_tiles = (a.count + kTileElems - 1) / kTileElems;
        const int64_t grid = n_tiles < kMaxGrid ? n_tiles : kMaxGrid;
        void *params[] = {&args, &n_full, &n_tiles};
        e = hipLaunchKernel(reinterpret_cast<const void *>(&dq4_tile_kernel<OUT>),
                            dim3(static_cast<uint32_t>(grid)), dim3(kThreads), params, 0, stream);
    } else if (shift_path_fits(a, OUT == DQ4_F32 ? 4 : 2)) {
        const int64_t out_bytes = OUT == DQ4_F32 ? 4 : 2;
        int64_t head = ((kOutAlign - static_cast<int64_t>(reinterpret_cast<uintptr_t>(a.out) %
                                                           kOutAlign)) % kOutAlign) / out_bytes;
        int64_t n_full = (a.count - head) / kTileElems;
        const bool edge = head > 0 || head + n_full * kTileElems < a.count;
        int64_t n_tiles = n_full + (edge ? 1 : 0);  // slot 0 takes head and tail
        const int64_t grid = n_tiles < kMaxGrid ? n_tiles : kMaxGrid;
        void *params[] = {&args, &head, &n_full, &n_tiles};
        // the first full tile decides for all (tiles are 4096 elements apart):
        // whole units when each lies in one packed dword and one block, else
        // the split point kK0 of every unit's elements between two blocks
        constexpr int E = Unit<OUT>::kElems;
        const int64_t e_first = a.e0 + head;
        const int64_t sh =
            (static_cast<int64_t>(reinterpret_cast<uintptr_t>(a.packed) & 3) * 8 + 4 * e_first) & 31;
        const int k0 = E - static_cast<int>(e_first % E);
        const void *kernel = shift_kernel<OUT>(sh % (4 * E) == 0 && k0 == E ? 0 : k0);
        if (!kernel)
            return hip_failed(hipErrorInvalidDeviceFunction);  // k0 is always 0 .. E
        e = hipLaunchKernel(kernel, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), params, 0,
                            stream);
    } else {
        int device = 0;
        e = hipGetDevice(&device);
        if (e != hipSuccess)
            return hip_failed(e);
        const int64_t max_grid = static_cast<int64_t>(compute_units(device)) * kElemBlocksPerCU;
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
}  // namespace dq4

using dq4::Args;
constexpr int kTileElemsPublic = dq4::kTileElems;
constexpr int kThreadsPublic = dq4::kThreads;

extern "C" {

dq4_status_t dq4_nested_dequant(const uint8_t *packed, const uint8_t *scale_codes,
                                const float *nested_absmax, const float *scale_codebook,
                                const float *codebook4, float offset, int64_t n,
                                int32_t blocksize, int32_t nested_blocksize, int32_t out_dtype,
                                void *out, void *stream)
{
    int log2_block = 0;
    const dq4_status_t st = dq4::validate_layout(blocksize, nested_blocksize, out_dtype, &log2_block);
    if (st != DQ4_OK)
        return st;
    if (n < 0 || n > dq4::kMaxElems)
        return DQ4_EINVAL;
    if (n == 0)
        return DQ4_OK;
    if (dq4::any_null(packed, scale_codes, nested_absmax, scale_codebook, codebook4, out))
        return DQ4_EINVAL;
    const Args a{packed, scale_codes, nested_absmax, scale_codebook, codebook4, out,
                 0, n, offset, log2_block};
    return dq4::launch(a, out_dtype, stream);
}

dq4_status_t dq4_nested_dequant_rows(const uint8_t *packed, const uint8_t *scale_codes,
                                     const float *nested_absmax, const float *scale_codebook,
                                     const float *codebook4, float offset, int64_t n_rows,
                                     int64_t n_cols, int64_t r0, int64_t rows, int32_t blocksize,
                                     int32_t nested_blocksize, int32_t out_dtype, void *out,
                                     void *stream)
{
    int log2_block = 0;
    const dq4_status_t st = dq4::validate_layout(blocksize, nested_blocksize, out_dtype, &log2_block);
    if (st != DQ4_OK)
        return st;
    if (n_rows < 0 || n_cols < 0 || r0 < 0 || rows < 0 || r0 > n_rows || rows > n_rows - r0)
        return DQ4_EINVAL;
    if (n_cols != 0 && n_rows > dq4::kMaxElems / n_cols)
        return DQ4_EINVAL;
    const int64_t count = rows * n_cols;
    if (count == 0)
        return DQ4_OK;
    if (dq4::any_null(packed, scale_codes, nested_absmax, scale_codebook, codebook4, out))
        return DQ4_EINVAL;
    const Args a{packed, scale_codes, nested_absmax, scale_codebook, codebook4, out,
                 r0 * n_cols, count, offset, log2_block};
    return dq4::launch(a, out_dtype, stream);
}

dq4_status_t dq4_memory_twin_f16(const uint8_t *packed, int64_t n, void *out, void *stream)
{
    if (n < 0 || n % kTileElemsPublic != 0)
        return DQ4_EINVAL;
    if (n == 0)
        return DQ4_OK;
    if (!packed || !out || reinterpret_cast<uintptr_t>(packed) % 4 != 0 ||
        reinterpret_cast<uintptr_t>(out) % 16 != 0)
        return DQ4_EINVAL;
    const uint32_t *words = reinterpret_cast<const uint32_t *>(packed);
    int64_t n_tiles = n / kTileElemsPublic;
    if (n_tiles > 0x7FFFFFFF)
        return DQ4_EUNSUPPORTED;
    void *o = out;
    void *params[] = {&words, &o, &n_tiles};
    const hipError_t e = hipLaunchKernel(
        reinterpret_cast<const void *>(&dq4::dq4_memory_twin_kernel),
        dim3(static_cast<uint32_t>(n_tiles)), dim3(kThreadsPublic), params, 0,
        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DQ4_OK : dq4::hip_failed(e);
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

int64_t dq4_row_window(int64_t n_rows, int64_t n_cols, int64_t elem_bytes, int64_t budget_bytes,
                       int64_t k, int64_t *r0, int64_t *rows)
{
    if (n_rows <= 0)
        return 0;
    const int64_t rpb = dq4_rows_per_block(n_cols, elem_bytes, budget_bytes);
    const int64_t count = n_rows / rpb + (n_rows % rpb != 0 ? 1 : 0);
    if (k >= 0 && k < count) {
        const int64_t first = k * rpb;
        const int64_t left = n_rows - first;
        if (r0)
            *r0 = first;
        if (rows)
            *rows = left < rpb ? left : rpb;
    }
    return count;
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
    case DQ4_EBLAS:
        return "DQ4_EBLAS: library GEMM failed";
    case DQ4_ESCRATCH:
        return "DQ4_ESCRATCH: more outer blocks than the static scratch holds";
    default:
        return "DQ4: unknown status";
    }
}

int32_t dq4_last_hip_error(void)
{
    return dq4::last_hip_error();
}

}  // extern "C"

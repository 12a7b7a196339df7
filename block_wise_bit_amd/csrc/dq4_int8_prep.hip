// dq4_int8_prep.hip -- LLM.int8 correction-operand preparation in one kernel.
//
// bitsandbytes issue "Fuse LLM.int8 correction operand preparation into one
// CUDA kernel" (sections "Summary", "Bounded method" and "Exact correctness
// oracle"): the eager chain
//     subA = A[:, cols]
//     subB = fp16(int8_vectorwise_dequant(CB[:, cols], SCB)).t()
// becomes one launch that writes the two final contiguous operands of the
// correction GEMM directly:
//     subA[r][l] = A[r][cols[l]]                               (raw 16-bit copy)
//     subB[l][n] = fp16(fl32(fl32(CB[n][cols[l]] * SCB[n]) * R127))
// with the eager chain's FP32 order (a multiply by the row scale, then a
// separately rounded multiply by the reciprocal-127 constant, then one
// round-to-nearest-even conversion).  R127 is the FP32 value nearest 1/127.
//
// Mapping: a bounded grid-stride loop over the two output regions, laid end
// to end, as the page asks (no persistent scheduler, no shape dispatch).
// Each lane writes one 16-bit output; consecutive lanes write consecutive
// outputs, so both regions are stored coalesced.  The subB reads are one
// byte per row of CB (rows are K bytes apart); rows touched by several
// columns are served from cache.
//
// Column indices are checked in the kernel: an index outside [0, K) reads
// nothing and writes an FP16 NaN (0x7E00) to the outputs it feeds, so a bad
// index never faults (the Python binding can also reject such indices on
// the host, on request: that check reads them back, a synchronization).

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "dq4.h"
#include "dq4_device.h"

#pragma clang fp contract(off)

namespace dq4 {
namespace {

constexpr int kThreads = 256;
constexpr uint32_t kR127Bits = 0x3C010204u;  // the FP32 value nearest 1/127
constexpr uint16_t kBadIndex = 0x7E00u;      // FP16 quiet NaN

// 32-bit indexing: the host guarantees that M*K, N*K and the two regions
// (plus one grid stride) stay below 2^31.
using Index = int32_t;

__global__ __launch_bounds__(kThreads) void int8_prep_kernel(
    const uint16_t *A, Index M, Index K, const int8_t *CB, const float *SCB, Index N,
    const int64_t *cols, Index L, uint16_t *subA, uint16_t *subB)
{
    const float r127 = __builtin_bit_cast(float, kR127Bits);
    const Index n_a = M * L;
    const Index total = n_a + L * N;
    const Index stride = static_cast<Index>(gridDim.x) * kThreads;
    for (Index i = static_cast<Index>(blockIdx.x) * kThreads + threadIdx.x; i < total;
         i += stride) {
        if (i < n_a) {
            // activation gather: output (r, l), l fastest
            const Index r = i / L;
            const Index l = i - r * L;
            const int64_t c = cols[l];
            subA[i] = (c >= 0 && c < K) ? A[r * K + static_cast<Index>(c)] : kBadIndex;
        } else {
            // weight gather + dequantization + conversion: output (l, n), n fastest
            const Index j = i - n_a;
            const Index l = j / N;
            const Index n = j - l * N;
            const int64_t c = cols[l];
            if (c < 0 || c >= K) {
                subB[j] = kBadIndex;
                continue;
            }
            const float code = static_cast<float>(CB[n * K + static_cast<Index>(c)]);
            const float scaled = code * SCB[n];
            const float v = scaled * r127;
            subB[j] = __builtin_bit_cast(uint16_t, to_f16(v));
        }
    }
}

}  // namespace
}  // namespace dq4

extern "C" {

dq4_status_t dq4_int8_prep(const uint16_t *A, int64_t M, int64_t K, const int8_t *CB,
                           const float *SCB, int64_t N, const int64_t *cols, int64_t L,
                           uint16_t *subA, uint16_t *subB, void *stream)
{
    if (M < 0 || K < 0 || N < 0 || L < 0)
        return DQ4_EINVAL;
    if (L == 0 || (M == 0 && N == 0))
        return DQ4_OK;  // nothing to prepare: the empty-outlier path launches nothing
    if (!cols || (M > 0 && (!A || !subA)) || (N > 0 && (!CB || !SCB || !subB)))
        return DQ4_EINVAL;
    if (K == 0)
        return DQ4_EINVAL;  // no column index can be valid
    // sizes of the arrays the kernel indexes, and of its two output regions
    if (M > INT64_MAX / K || N > INT64_MAX / K || M > INT64_MAX / L || N > INT64_MAX / L)
        return DQ4_EINVAL;
    const int64_t total = M * L + N * L;
    if (total < 0)
        return DQ4_EINVAL;
    // the kernel indexes in 32 bits (64-bit integer division would bring the
    // compiler's float-based division sequence into the kernel)
    const int64_t kLimit = INT32_MAX - (int64_t{1} << 24);
    if (M * K >= kLimit || N * K >= kLimit || total >= kLimit)
        return DQ4_EUNSUPPORTED;
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess)
        return dq4::hip_failed(e);
    int64_t grid = (total + dq4::kThreads - 1) / dq4::kThreads;
    const int64_t max_grid = static_cast<int64_t>(dq4::compute_units(device)) * 8;
    if (grid > max_grid)
        grid = max_grid;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t m = static_cast<int32_t>(M), k = static_cast<int32_t>(K), n = static_cast<int32_t>(N),
            l = static_cast<int32_t>(L);
    void *params[] = {&A, &m, &k, &CB, &SCB, &n, &cols, &l, &subA, &subB};
    e = hipLaunchKernel(reinterpret_cast<const void *>(&dq4::int8_prep_kernel),
                        dim3(static_cast<uint32_t>(grid)), dim3(dq4::kThreads), params, 0, s);
    return e == hipSuccess ? DQ4_OK : dq4::hip_failed(e);
}

}  // extern "C"

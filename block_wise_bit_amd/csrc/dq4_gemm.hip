// dq4_gemm.hip -- the consumers of the dequantized weight that end in a
// plain library GEMM (rocBLAS): the row-blocked out_prod and the
// dequantize-plus-linear forward / grad_A.
//
// 1. Row-blocked out_prod.
// llama.cpp PR "cuda: out_prod dequantizes a 2D weight in row blocks"
// (section "What" and the approving review): out_prod sums over the weight's
// rows, so the weight is dequantized to F32 one block of rows at a time into
// a bounded buffer (at most 256 MiB there), and each block's GEMM
// accumulates into the destination -- beta 0 for the first block, 1 after.
// The sum over blocks is the sum over all rows.
//
//   dst[i][j] = sum_r B[r][i] * W[r][j]     dst: m x n_cols FP32, row-major
//
// W is the n_rows x n_cols nested 4-bit weight (dequantized by this
// library's own kernel, bit-identical to the whole-tensor call); B is src1,
// FP32, in either orientation the review names: stored n_rows x m (a block
// starts r0 * ld_src1 into it, the GEMM reads it transposed) or stored
// m x n_rows (a block starts r0 into it).  The GEMM is a plain FP32 library
// GEMM.
//
// 2. Dequantize-plus-linear (bitsandbytes issue "Fuse nested scale
// reconstruction into SM103 4-bit dequantization", section "Problem": the
// dequantize-plus-linear fallback that materializes the full weight before
// F.linear, and the MatMul4Bit.backward path for grad_A that runs the same
// dequantization).  The whole weight is dequantized once, bit-identical to
// dq4_nested_dequant, into a caller-provided FP16/BF16 buffer, then one GEMM
// with FP32 accumulation:
//   forward  Y = X W^T   (X: m x n_in,  Y: m x n_out)
//   grad_A   Y = G W     (G: m x n_out, Y: m x n_in)

#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <stdint.h>

#include <unordered_map>

#include "dq4.h"
#include "dq4_device.h"

namespace dq4 {
namespace {

__global__ __launch_bounds__(256) void zero_fill_kernel(float *p, int64_t count)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < count; i += stride)
        p[i] = 0.0f;
}

// One rocBLAS handle per (thread, device), created on first use: rocBLAS
// handles must not be shared between threads.  They are never destroyed; a
// thread_local destructor can run after the HIP runtime has shut down at
// process exit, so each thread that calls a GEMM entry point keeps its
// handles (a few KB of host state and rocBLAS's device workspace per device)
// until the process ends.
thread_local std::unordered_map<int, rocblas_handle> t_handles;
thread_local int32_t t_last_blas_status = 0;

rocblas_handle blas_handle(int device)
{
    auto it = t_handles.find(device);
    if (it != t_handles.end())
        return it->second;
    rocblas_handle h = nullptr;
    if (rocblas_create_handle(&h) != rocblas_status_success)
        return nullptr;
    t_handles.emplace(device, h);
    return h;
}

bool fits_i32(int64_t v)
{
    return v >= 0 && v <= 0x7FFFFFFF;
}

// The handle for this thread's current device, bound to `stream`.
dq4_status_t blas_on_stream(hipStream_t s, rocblas_handle *out)
{
    int device = 0;
    const hipError_t he = hipGetDevice(&device);
    if (he != hipSuccess)
        return hip_failed(he);
    rocblas_handle h = blas_handle(device);
    if (!h)
        return DQ4_EBLAS;
    const rocblas_status bs = rocblas_set_stream(h, s);
    if (bs != rocblas_status_success) {
        t_last_blas_status = static_cast<int32_t>(bs);
        return DQ4_EBLAS;
    }
    *out = h;
    return DQ4_OK;
}

}  // namespace
}  // namespace dq4

extern "C" {

int32_t dq4_last_blas_status(void)
{
    return dq4::t_last_blas_status;
}

dq4_status_t dq4_out_prod_rows(const uint8_t *packed, const uint8_t *scale_codes,
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
    if (n_rows < 0 || n_cols < 0 || m < 0 || (src1_transposed != 0 && src1_transposed != 1))
        return DQ4_EINVAL;
    if (m == 0 || n_cols == 0)
        return DQ4_OK;  // dst is empty
    if (!dst)
        return DQ4_EINVAL;
    if (n_cols > INT64_MAX / m || !dq4::fits_i32(n_cols) || !dq4::fits_i32(m))
        return DQ4_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (n_rows == 0) {  // an empty sum: dst = 0
        const int64_t count = m * n_cols;
        int64_t grid = (count + 255) / 256;
        if (grid > 65536)
            grid = 65536;
        float *d = dst;
        int64_t c = count;
        void *params[] = {&d, &c};
        const hipError_t e =
            hipLaunchKernel(reinterpret_cast<const void *>(&dq4::zero_fill_kernel),
                            dim3(static_cast<uint32_t>(grid)), dim3(256), params, 0, s);
        return e == hipSuccess ? DQ4_OK : dq4::hip_failed(e);
    }
    if (!packed || !scale_codes || !nested_absmax || !scale_codebook || !codebook4 || !src1 ||
        !workspace)
        return DQ4_EINVAL;
    if (ld_src1 < (src1_transposed ? n_rows : m) || !dq4::fits_i32(ld_src1))
        return DQ4_EINVAL;
    if (n_cols > INT64_MAX / 4 || workspace_bytes < n_cols * 4)
        return DQ4_EINVAL;  // the workspace must hold at least one F32 row
    const int64_t rows_per_block = dq4_rows_per_block(n_cols, 4, workspace_bytes);
    if (!dq4::fits_i32(rows_per_block < n_rows ? rows_per_block : n_rows))
        return DQ4_EINVAL;

    rocblas_handle h = nullptr;
    const dq4_status_t hs = dq4::blas_on_stream(s, &h);
    if (hs != DQ4_OK)
        return hs;

    const float alpha = 1.0f;
    for (int64_t r0 = 0; r0 < n_rows; r0 += rows_per_block) {
        const int64_t rows = n_rows - r0 < rows_per_block ? n_rows - r0 : rows_per_block;
        const dq4_status_t ds = dq4_nested_dequant_rows(
            packed, scale_codes, nested_absmax, scale_codebook, codebook4, offset, n_rows, n_cols,
            r0, rows, blocksize, nested_blocksize, DQ4_F32, workspace, stream);
        if (ds != DQ4_OK)
            return ds;
        // column-major view: dst is (n_cols x m), ld n_cols; the window is
        // (n_cols x rows), ld n_cols; B is read as (rows x m)
        const float beta = r0 == 0 ? 0.0f : 1.0f;
        const float *b = src1_transposed ? src1 + r0 : src1 + r0 * ld_src1;
        const rocblas_operation op_b =
            src1_transposed ? rocblas_operation_none : rocblas_operation_transpose;
        const rocblas_status bs = rocblas_sgemm(h, rocblas_operation_none, op_b, static_cast<rocblas_int>(n_cols),
                           static_cast<rocblas_int>(m), static_cast<rocblas_int>(rows), &alpha,
                           workspace, static_cast<rocblas_int>(n_cols), b,
                           static_cast<rocblas_int>(ld_src1), &beta, dst,
                           static_cast<rocblas_int>(n_cols));
        if (bs != rocblas_status_success) {
            dq4::t_last_blas_status = static_cast<int32_t>(bs);
            return DQ4_EBLAS;
        }
    }
    return DQ4_OK;
}

dq4_status_t dq4_dequant_linear(const uint8_t *packed, const uint8_t *scale_codes,
                                const float *nested_absmax, const float *scale_codebook,
                                const float *codebook4, float offset, int64_t n_out,
                                int64_t n_in, int32_t blocksize, int32_t nested_blocksize,
                                int32_t dtype, int32_t op, const void *x, int64_t m, void *y,
                                void *w_workspace, void *stream)
{
    int log2_block = 0;
    const dq4_status_t st = dq4::validate_layout(blocksize, nested_blocksize, dtype, &log2_block);
    if (st != DQ4_OK)
        return st;
    if (dtype != DQ4_F16 && dtype != DQ4_BF16)
        return DQ4_EINVAL;
    if (op != DQ4_LINEAR_FORWARD && op != DQ4_LINEAR_GRAD_A)
        return DQ4_EINVAL;
    if (n_out < 0 || n_in < 0 || m < 0)
        return DQ4_EINVAL;
    if (!dq4::fits_i32(n_out) || !dq4::fits_i32(n_in) || !dq4::fits_i32(m))
        return DQ4_EINVAL;
    const int64_t y_cols = op == DQ4_LINEAR_FORWARD ? n_out : n_in;
    const int64_t k = op == DQ4_LINEAR_FORWARD ? n_in : n_out;
    if (m == 0 || y_cols == 0)
        return DQ4_OK;  // Y is empty
    if (!x || !y || !w_workspace)
        return DQ4_EINVAL;
    if (k > 0 && (!packed || !scale_codes || !nested_absmax || !scale_codebook || !codebook4))
        return DQ4_EINVAL;
    if (n_out > INT64_MAX / (n_in > 0 ? n_in : 1))
        return DQ4_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (k > 0) {
        const dq4_status_t ds =
            dq4_nested_dequant(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                               offset, n_out * n_in, blocksize, nested_blocksize, dtype,
                               w_workspace, stream);
        if (ds != DQ4_OK)
            return ds;
    }
    rocblas_handle h = nullptr;
    const dq4_status_t hs = dq4::blas_on_stream(s, &h);
    if (hs != DQ4_OK)
        return hs;
    const rocblas_datatype t =
        dtype == DQ4_F16 ? rocblas_datatype_f16_r : rocblas_datatype_bf16_r;
    const float alpha = 1.0f, beta = 0.0f;
    // column-major views: W (n_out x n_in, row-major) is Wc = (n_in x n_out), ld n_in
    rocblas_status bs;
    if (op == DQ4_LINEAR_FORWARD) {
        // Y^T (n_out x m) = Wc^T (n_out x n_in) * X^T (n_in x m)
        bs = rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none,
                             static_cast<rocblas_int>(n_out), static_cast<rocblas_int>(m),
                             static_cast<rocblas_int>(n_in), &alpha, w_workspace, t,
                             static_cast<rocblas_int>(n_in > 0 ? n_in : 1), x, t,
                             static_cast<rocblas_int>(n_in > 0 ? n_in : 1), &beta, y, t,
                             static_cast<rocblas_int>(n_out), y, t,
                             static_cast<rocblas_int>(n_out), rocblas_datatype_f32_r,
                             rocblas_gemm_algo_standard, 0, 0);
    } else {
        // Y^T (n_in x m) = Wc (n_in x n_out) * G^T (n_out x m)
        bs = rocblas_gemm_ex(h, rocblas_operation_none, rocblas_operation_none,
                             static_cast<rocblas_int>(n_in), static_cast<rocblas_int>(m),
                             static_cast<rocblas_int>(n_out), &alpha, w_workspace, t,
                             static_cast<rocblas_int>(n_in), x, t,
                             static_cast<rocblas_int>(n_out > 0 ? n_out : 1), &beta, y, t,
                             static_cast<rocblas_int>(n_in), y, t,
                             static_cast<rocblas_int>(n_in), rocblas_datatype_f32_r,
                             rocblas_gemm_algo_standard, 0, 0);
    }
    if (bs != rocblas_status_success) {
        dq4::t_last_blas_status = static_cast<int32_t>(bs);
        return DQ4_EBLAS;
    }
    return DQ4_OK;
}

}  // extern "C"

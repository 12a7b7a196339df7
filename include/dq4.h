/*
 * dq4.h -- C ABI of the MI355X (gfx950) nested 4-bit dequantization library.
 *
 * The operation (bitsandbytes issue "Fuse nested scale reconstruction into
 * SM103 4-bit dequantization", section "Proposed experiment"): for every
 * element i of a flat row-major tensor of packed 4-bit codes
 *
 *     b     = i / blocksize                 outer block
 *     g     = b / nested_blocksize          nested group, counted in outer blocks
 *     t     = fl32(scale_codebook[scale_codes[b]] * nested_absmax[g])
 *     s     = fl32(t + offset)              rounded separately: no fused multiply-add
 *     k     = nibble of element i           byte i/2; low nibble for even i, high for odd i
 *     out_i = cvt(fl32(codebook4[k] * s))   cvt: identity (F32) or IEEE
 *                                           round-to-nearest-even to F16 / BF16,
 *                                           subnormals kept
 *
 * fl32() is one IEEE binary32 round-to-nearest-even step.  The section
 * "Correctness requirements" of that issue fixes the separate rounding of the
 * multiply and the add, and requires the result to be bitwise identical to the
 * three-step sequence of its section "Problem" (scale codes to an FP32 buffer,
 * a separate offset add, then the value pass).  The per-block scale is rebuilt
 * in registers inside the value pass: no FP32 scale tensor is written.
 *
 * Buffers (all of them caller-owned; device memory unless stated otherwise):
 *   packed          ceil(n/2) bytes.  For odd n the high nibble of the last
 *                   byte is read and ignored.
 *   scale_codes     ceil(n/blocksize) bytes, one uint8 code per outer block.
 *   nested_absmax   ceil(ceil(n/blocksize)/nested_blocksize) FP32 values.
 *   scale_codebook  256 FP32 values (indexed by the scale code).
 *   codebook4       16 FP32 values (the NF4 or FP4 decode table, indexed by
 *                   the 4-bit code; any 16 values are accepted).
 *   offset          host FP32 scalar, passed by value.
 *   out             n elements of the output type, densely packed.
 * No pointer has to be aligned.  A 4-byte aligned `packed`, a 128-byte
 * aligned `out` and a window starting at a multiple of 8 elements take the
 * fastest path; other element-aligned outputs a general vector path (a few
 * percent slower: 2-4 % at 28672 x 8192); anything else a per-element path.
 * All of them give bitwise identical results.
 * Input and output ranges must not overlap.
 *
 * Ownership and ordering: the library allocates nothing, frees nothing, keeps
 * no handle to any buffer and never synchronizes.  (Two exceptions, each
 * documented at its call: the GEMM routes keep a rocBLAS handle per thread and
 * device, and dq4_nested_dequant_unfused_noalloc uses a static device array
 * that the runtime sets up with the library's code.)  Each fused call enqueues
 * exactly one kernel on `stream` (a hipStream_t; NULL means the legacy
 * default stream) and returns; the output is ready when that stream reaches
 * the kernel.  Calls are reentrant and thread-safe.
 *
 * Errors: validation happens on the host before anything is enqueued.  A call
 * that returns anything but DQ4_OK has enqueued nothing and left `out`
 * untouched, except DQ4_EHIP, which reports that the launch itself failed
 * (the HIP error code is kept, per thread, for dq4_last_hip_error()).
 */
#ifndef DQ4_H
#define DQ4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t dq4_status_t;

enum {
    DQ4_OK = 0,
    DQ4_EINVAL = 1,        /* null pointer with work to do, negative size or
                              more than 2^62 elements, bad row window,
                              unknown output type */
    DQ4_EUNSUPPORTED = 2,  /* blocksize not a power of two in [32, 4096], or
                              nested_blocksize other than 256 */
    DQ4_EHIP = 3,          /* the kernel launch failed */
    DQ4_EBLAS = 4,         /* the library GEMM (rocBLAS) failed */
    DQ4_ESCRATCH = 5       /* the call needs more than the library's static
                              scratch holds (dq4_nested_dequant_unfused_noalloc) */
};

/* Outer blocks whose FP32 scales fit in the static scratch of
 * dq4_nested_dequant_unfused_noalloc (32 MiB per device). */
#define DQ4_NOALLOC_MAX_BLOCKS (1 << 23)

enum {
    DQ4_F32 = 0,
    DQ4_F16 = 1,
    DQ4_BF16 = 2
};

enum {
    DQ4_LINEAR_FORWARD = 0,  /* Y = X W^T */
    DQ4_LINEAR_GRAD_A = 1    /* Y = G W   */
};

/*
 * Whole-tensor dequantization of n elements (the fused nested dequantization
 * of the bitsandbytes issue above, section "Proposed experiment").
 *
 * blocksize: outer block size, a power of two from 32 to 4096 (section
 *   "Correctness requirements": block sizes 32 through 4096).
 * nested_blocksize: outer blocks per nested absmax; 256 is the only nested
 *   layout supported (section "Proposed experiment", the routing guard
 *   state2.blocksize == 256).
 * out_dtype: DQ4_F32, DQ4_F16 or DQ4_BF16.
 * n == 0 is a no-op that returns DQ4_OK without touching the GPU.
 */
dq4_status_t dq4_nested_dequant(const uint8_t *packed, const uint8_t *scale_codes,
                                const float *nested_absmax, const float *scale_codebook,
                                const float *codebook4, float offset, int64_t n,
                                int32_t blocksize, int32_t nested_blocksize,
                                int32_t out_dtype, void *out, void *stream);

/*
 * Row-window dequantization (llama.cpp PR "cuda: out_prod dequantizes a 2D
 * weight in row blocks", section "What" and the review): rows [r0, r0 + rows)
 * of an n_rows x n_cols row-major weight, so a large weight can stream through
 * one bounded output buffer.  Output element (r - r0) * n_cols + j is global
 * element r * n_cols + j of the whole-tensor call; block and group indices
 * come from the global element index, and the metadata pointers are those of
 * the whole tensor.  `out` holds rows * n_cols elements.
 * Requires 0 <= r0, 0 <= rows, r0 + rows <= n_rows; rows == 0 is a no-op.
 */
dq4_status_t dq4_nested_dequant_rows(const uint8_t *packed, const uint8_t *scale_codes,
                                     const float *nested_absmax,
                                     const float *scale_codebook, const float *codebook4,
                                     float offset, int64_t n_rows, int64_t n_cols,
                                     int64_t r0, int64_t rows, int32_t blocksize,
                                     int32_t nested_blocksize, int32_t out_dtype, void *out,
                                     void *stream);

/*
 * Rows per transient block (llama.cpp PR above, review): the largest row count
 * whose rows * n_cols * elem_bytes fits in budget_bytes, and at least 1.
 * Non-positive arguments return 1.  Host only.
 */
int64_t dq4_rows_per_block(int64_t n_cols, int64_t elem_bytes, int64_t budget_bytes);

/*
 * The host's row-block loop of the same PR (review: the weight is walked in
 * consecutive blocks of rows_per_block rows, the last one partial): window k
 * of an n_rows-row weight is rows [k * rpb, k * rpb + min(rpb, n_rows - k *
 * rpb)), rpb = dq4_rows_per_block(n_cols, elem_bytes, budget_bytes).
 * Returns the number of windows, ceil(n_rows / rpb), or 0 for n_rows <= 0.
 * When 0 <= k < that count, writes window k's first row to *r0 and its row
 * count to *rows (either pointer may be NULL); otherwise writes nothing.
 * Feeding each window to dq4_nested_dequant_rows covers every row once, in
 * order.  Host only.
 */
int64_t dq4_row_window(int64_t n_rows, int64_t n_cols, int64_t elem_bytes, int64_t budget_bytes,
                       int64_t k, int64_t *r0, int64_t *rows);

/*
 * Diagnostic, not part of the method: the memory twin of the FP16 whole-tensor
 * call at block size 64.  It reads the n/2 packed bytes and writes 2n bytes
 * to `out` in exactly the tiles, tile order, load policy and store policy of
 * dq4_nested_dequant's vector path, with the dequantization taken out: each
 * packed dword is written four times into its 16-byte output unit
 * (out as uint32: out[4u + i] = packed_as_uint32[u], i < 4).  Its time is
 * the ceiling that the dequantization's access pattern reaches on the GPU at
 * hand, the reference beside the nominal HBM peak (the pages' evidence plan
 * asks for effective bandwidth; this gives the attainable one).
 * Requires n % 4096 == 0, `packed` 4-byte and `out` 16-byte aligned
 * (DQ4_EINVAL otherwise); n == 0 is a no-op.  One kernel on `stream`.
 */
dq4_status_t dq4_memory_twin_f16(const uint8_t *packed, int64_t n, void *out, void *stream);

/*
 * Unfused three-launch form, kept as the comparison baseline of
 * dq4_nested_dequant: the existing sequence of the bitsandbytes issue above
 * (section "Problem") -- (1) scale codes to an FP32 scale buffer,
 * scale[b] = fl32(scale_codebook[code[b]] * nested_absmax[b / 256]); (2) a
 * separate elementwise add, scale[b] = fl32(scale[b] + offset); (3) the
 * value pass reading that buffer.  Results are bitwise identical to
 * dq4_nested_dequant; the cost is the FP32 buffer's HBM traffic and two more
 * launches, which is what the fused call removes.
 *
 * scale_workspace: caller-owned device buffer of at least
 *   dq4_unfused_workspace_bytes(n, blocksize) bytes; overwritten.  Three
 *   kernels are enqueued on `stream`, in order.  Other arguments, errors and
 *   the n == 0 no-op are as for dq4_nested_dequant.
 */
dq4_status_t dq4_nested_dequant_unfused(const uint8_t *packed, const uint8_t *scale_codes,
                                        const float *nested_absmax,
                                        const float *scale_codebook, const float *codebook4,
                                        float offset, int64_t n, int32_t blocksize,
                                        int32_t nested_blocksize, int32_t out_dtype,
                                        float *scale_workspace, void *out, void *stream);

/*
 * dq4_nested_dequant_unfused without a workspace argument, for callers that
 * cannot allocate device memory: code being captured into a HIP graph, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments (less
 * scale_workspace), same three kernels, same results, bit for bit.
 *
 * The FP32 scale buffer is a static device array inside the library,
 * DQ4_NOALLOC_MAX_BLOCKS floats (32 MiB), one copy per GPU, held from the
 * first call on that GPU until the process ends.  The call itself allocates
 * nothing (no hipMalloc, no allocating library routine); its first call on a
 * device looks up that device's address of the array (hipGetSymbolAddress).
 *
 * Limit: ceil(n / blocksize) <= DQ4_NOALLOC_MAX_BLOCKS, else DQ4_ESCRATCH
 * and nothing is enqueued (e.g. n <= 2^29 at blocksize 64).  Every call on
 * one GPU shares that GPU's array: calls that overlap in time on one GPU
 * (different streams or threads) race and give wrong results; serialize
 * them.  Nothing in the array needs to start at zero: the first kernel
 * writes every scale the third one reads.  Other errors as for
 * dq4_nested_dequant_unfused.
 */
dq4_status_t dq4_nested_dequant_unfused_noalloc(const uint8_t *packed,
                                                const uint8_t *scale_codes,
                                                const float *nested_absmax,
                                                const float *scale_codebook,
                                                const float *codebook4, float offset, int64_t n,
                                                int32_t blocksize, int32_t nested_blocksize,
                                                int32_t out_dtype, void *out, void *stream);

/* Bytes of FP32 scale workspace dq4_nested_dequant_unfused needs: 4 * ceil(n /
 * blocksize); 0 for non-positive arguments or n above 2^62.  Host only. */
int64_t dq4_unfused_workspace_bytes(int64_t n, int32_t blocksize);

/*
 * Row-blocked out_prod of a nested 4-bit weight (llama.cpp PR "cuda: out_prod
 * dequantizes a 2D weight in row blocks", section "What" and the review):
 *
 *     dst[i][j] = sum over r in [0, n_rows) of B[r][i] * W[r][j]
 *
 * W is the n_rows x n_cols nested 4-bit weight described by the first ten
 * arguments (as for dq4_nested_dequant_rows).  B is src1, FP32 device memory:
 *   src1_transposed == 0: B[r][i] = src1[r * ld_src1 + i]   (stored n_rows x m, ld_src1 >= m)
 *   src1_transposed == 1: B[r][i] = src1[i * ld_src1 + r]   (stored m x n_rows, ld_src1 >= n_rows)
 * dst: m x n_cols FP32 row-major device memory, overwritten (n_rows == 0
 * writes zeros).  workspace: caller-owned device buffer of workspace_bytes
 * bytes, at least one F32 row (n_cols * 4); the weight is dequantized to F32
 * in consecutive windows of dq4_rows_per_block(n_cols, 4, workspace_bytes)
 * rows into it, and for each window an FP32 GEMM (rocBLAS) adds
 * B[r0:r0+rows]^T * window into dst, with beta 0 for the first window and 1
 * after -- the same sum as one GEMM over the whole dequantized weight.
 *
 * Everything is enqueued on `stream`; nothing is synchronized.  The first
 * call on a thread and device creates a rocBLAS handle for it (rocBLAS
 * manages that handle's own device memory); nothing else is allocated.
 * Returns DQ4_EBLAS (code in dq4_last_blas_status()) if rocBLAS fails,
 * DQ4_EINVAL for bad sizes, a leading dimension that is too small or a
 * workspace smaller than one row, or any size above 2^31 - 1 that rocBLAS's
 * 32-bit interface cannot take.
 */
dq4_status_t dq4_out_prod_rows(const uint8_t *packed, const uint8_t *scale_codes,
                               const float *nested_absmax, const float *scale_codebook,
                               const float *codebook4, float offset, int64_t n_rows,
                               int64_t n_cols, int32_t blocksize, int32_t nested_blocksize,
                               const float *src1, int64_t m, int64_t ld_src1,
                               int32_t src1_transposed, float *dst, float *workspace,
                               int64_t workspace_bytes, void *stream);

/*
 * out_prod with the dequantization fused into the GEMM (llama.cpp PR "cuda:
 * out_prod dequantizes a 2D weight in row blocks": the approving review names
 * the fused dequant-in-GEMM route as the follow-on of the row-blocked path).
 * Same sum, same arguments and same layouts as dq4_out_prod_rows:
 *
 *     dst[i][j] = sum over r in [0, n_rows) of B[r][i] * W[r][j]
 *
 * but no dequantized copy of W is written: each workgroup decodes its part
 * of the 4-bit weight into on-chip memory as exactly the FP32 values
 * dq4_nested_dequant writes, and multiplies on the matrix cores in FP32.
 * The summation order differs from dq4_out_prod_rows; both are within the
 * FP32 summation bound of the exact sum.
 *
 * The dst rows may be computed in two ranges one after the other (dst row i
 * depends on src1 column i alone): on the aligned path (n_cols % 8 == 0,
 * packed 4-byte aligned) m > 64 takes whole 64-row tiles, then the rest.
 *
 * workspace: optional caller-owned device memory for partial sums.  When the
 * dst tiles alone cannot fill the GPU, the rows r are split and each split's
 * partial of the range's dst rows (at most m * n_cols FP32) goes to the
 * workspace, then one more kernel adds the partials in split order into dst;
 * the ranges reuse the workspace in turn.  The number of splits is the
 * largest of those the workspace holds up to the preferred count
 * (dq4_out_prod_fused_workspace_bytes); with workspace_bytes == 0 there is
 * one split and dst is written directly.  A transposed src1 on the aligned
 * path: the dst-row ranges whose tiles are 64 rows, or 48 rows with at
 * least 40 used, read a transposed src1 slowly, so when the workspace holds a
 * row-major copy of those ranges' src1 columns (rounded up to 256 bytes)
 * plus the partials of the resulting plan (dq4_out_prod_fused_workspace_bytes
 * with src1_transposed = 1 is enough), the call first copies those columns
 * to the start of the workspace (one more kernel) and those ranges run
 * exactly as for a row-major src1, with the rest of the workspace; other
 * ranges, or every range when the workspace is smaller, read src1 in place.
 * With m == 1 both orientations are the same memory and take the row-major
 * path.  The workspace changes speed only; the result is deterministic for a
 * given device, orientation and workspace size.
 *
 * dst is overwritten (n_rows == 0 writes zeros); m == 0 or n_cols == 0 is a
 * no-op.  Everything is enqueued on `stream`; nothing is allocated or
 * synchronized.  Errors: DQ4_EINVAL for bad sizes, a leading dimension that
 * is too small, a null pointer, or workspace_bytes > 0 with a null
 * workspace; DQ4_EUNSUPPORTED for a tile grid of more than 2^31 - 1
 * workgroups or a split of more than 4 * (2^31 - 1) rows; layout errors as
 * for dq4_nested_dequant.
 */
dq4_status_t dq4_out_prod_fused(const uint8_t *packed, const uint8_t *scale_codes,
                                const float *nested_absmax, const float *scale_codebook,
                                const float *codebook4, float offset, int64_t n_rows,
                                int64_t n_cols, int32_t blocksize, int32_t nested_blocksize,
                                const float *src1, int64_t m, int64_t ld_src1,
                                int32_t src1_transposed, float *dst, float *workspace,
                                int64_t workspace_bytes, void *stream);

/* Workspace bytes at which dq4_out_prod_fused uses its preferred number of
 * row splits on the current device for a src1 of the given orientation (0
 * when one split is preferred, or for non-positive or oversized arguments or
 * a src1_transposed other than 0 or 1).  For a transposed src1 and
 * n_cols % 8 == 0 this includes the row-major copy of src1 columns that
 * dq4_out_prod_fused then makes (see there).  Host only; queries the current
 * device. */
int64_t dq4_out_prod_fused_workspace_bytes(int64_t n_rows, int64_t n_cols, int64_t m,
                                           int32_t src1_transposed);

/*
 * Dequantize-plus-linear (bitsandbytes issue above, section "Problem": the
 * dequantize-plus-linear fallback that materializes the full weight before
 * F.linear, and MatMul4Bit.backward's grad_A, which uses the same
 * dequantization).  W is the n_out x n_in nested 4-bit weight (row-major,
 * first ten arguments as for dq4_nested_dequant with n = n_out * n_in).  It is
 * dequantized whole into w_workspace (n_out * n_in elements of `dtype`,
 * caller-owned device memory; bit-identical to dq4_nested_dequant), then one
 * GEMM (rocBLAS, FP32 accumulation, inputs and output in `dtype`):
 *   op == DQ4_LINEAR_FORWARD:  Y[i][o] = sum_k X[i][k] W[o][k]   x: m x n_in,  y: m x n_out
 *   op == DQ4_LINEAR_GRAD_A:   Y[i][k] = sum_o X[i][o] W[o][k]   x: m x n_out, y: m x n_in
 * x and y are dense row-major device arrays of `dtype` (DQ4_F16 or DQ4_BF16).
 * Everything is enqueued on `stream`.  An empty Y (m or its width 0) is a
 * no-op.  Sizes above 2^31 - 1 are DQ4_EINVAL (rocBLAS's 32-bit interface);
 * rocBLAS failures are DQ4_EBLAS.  The rocBLAS handle is as for
 * dq4_out_prod_rows.
 */
dq4_status_t dq4_dequant_linear(const uint8_t *packed, const uint8_t *scale_codes,
                                const float *nested_absmax, const float *scale_codebook,
                                const float *codebook4, float offset, int64_t n_out,
                                int64_t n_in, int32_t blocksize, int32_t nested_blocksize,
                                int32_t dtype, int32_t op, const void *x, int64_t m, void *y,
                                void *w_workspace, void *stream);

/*
 * LLM.int8 correction-operand preparation in one kernel (bitsandbytes issue
 * "Fuse LLM.int8 correction operand preparation into one CUDA kernel",
 * sections "Bounded method" and "Exact correctness oracle"):
 *     subA[r][l] = A[r][cols[l]]                                  r < M, l < L
 *     subB[l][n] = fp16(fl32(fl32(CB[n][cols[l]] * SCB[n]) * R127))  n < N
 * A: M x K FP16 (16-bit values, copied bit for bit), CB: N x K int8, SCB: N
 * FP32 row scales, cols: L int64 column indices (any order, repeats allowed),
 * all dense row-major device arrays.  subA: M x L and subB: L x N (the
 * transposed layout the correction GEMM consumes), FP16, caller-owned.
 * R127 is the FP32 value nearest 1/127; the multiply by the row scale and the
 * multiply by R127 are separately rounded FP32 operations, and the FP16
 * conversion is round-to-nearest-even.  One kernel on `stream`; L == 0 (no
 * outlier columns) launches nothing and returns DQ4_OK.  A column index
 * outside [0, K) is not read: the outputs it feeds are set to FP16 NaN
 * (0x7E00).  DQ4_EINVAL for negative sizes, K == 0 with L > 0, or a null
 * pointer an output needs; DQ4_EUNSUPPORTED when M*K, N*K or (M+N)*L reaches
 * 2^31 - 2^24 (the kernel indexes in 32 bits).
 */
dq4_status_t dq4_int8_prep(const uint16_t *A, int64_t M, int64_t K, const int8_t *CB,
                           const float *SCB, int64_t N, const int64_t *cols, int64_t L,
                           uint16_t *subA, uint16_t *subB, void *stream);

/* rocBLAS status of this thread's last DQ4_EBLAS, 0 if none. */
int32_t dq4_last_blas_status(void);

/* Static, human-readable name of a status code (never NULL). */
const char *dq4_status_string(dq4_status_t status);

/* HIP error code of this thread's last DQ4_EHIP, 0 if none. */
int32_t dq4_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DQ4_H */

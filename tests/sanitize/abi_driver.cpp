// Sanitizer driver for the C ABI's host-side validation (a test, built by
// tests/test_sanitizers.py with AddressSanitizer and UBSan on the host code
// only).  Every call here must be rejected, or be a no-op, before anything
// reaches the GPU, so it runs on a machine without one.
#include <stdint.h>
#include <stdio.h>

#include "dq4.h"

static int failures = 0;
static void expect(int got, int want, const char *what)
{
    if (got != want) {
        printf("%s: got %d want %d\n", what, got, want);
        ++failures;
    }
}

int main()
{
    uint8_t *p8 = reinterpret_cast<uint8_t *>(0x1000);
    float *pf = reinterpret_cast<float *>(0x1000);
    void *pv = reinterpret_cast<void *>(0x1000);
    expect(dq4_nested_dequant(p8, p8, pf, pf, pf, 0.f, 0, 64, 256, DQ4_F16, pv, nullptr), DQ4_OK, "n=0");
    expect(dq4_nested_dequant(p8, p8, pf, pf, pf, 0.f, -1, 64, 256, DQ4_F16, pv, nullptr), DQ4_EINVAL, "n<0");
    expect(dq4_nested_dequant(nullptr, p8, pf, pf, pf, 0.f, 8, 64, 256, DQ4_F16, pv, nullptr), DQ4_EINVAL, "null");
    expect(dq4_nested_dequant(p8, p8, pf, pf, pf, 0.f, 8, 48, 256, DQ4_F16, pv, nullptr), DQ4_EUNSUPPORTED, "bs 48");
    expect(dq4_nested_dequant(p8, p8, pf, pf, pf, 0.f, 8, 64, 128, DQ4_F16, pv, nullptr), DQ4_EUNSUPPORTED, "nested 128");
    expect(dq4_nested_dequant(p8, p8, pf, pf, pf, 0.f, 8, 64, 256, 9, pv, nullptr), DQ4_EINVAL, "dtype");
    expect(dq4_nested_dequant_rows(p8, p8, pf, pf, pf, 0.f, INT64_MAX, 2, 0, 1, 64, 256, DQ4_F32, pv, nullptr), DQ4_EINVAL, "rows overflow");
    expect(dq4_nested_dequant_rows(p8, p8, pf, pf, pf, 0.f, 10, 10, 5, 6, 64, 256, DQ4_F32, pv, nullptr), DQ4_EINVAL, "window");
    expect(dq4_nested_dequant_rows(p8, p8, pf, pf, pf, 0.f, 10, 10, 10, 0, 64, 256, DQ4_F32, pv, nullptr), DQ4_OK, "empty window");
    expect(dq4_nested_dequant_unfused(p8, p8, pf, pf, pf, 0.f, 8, 64, 256, DQ4_F16, nullptr, pv, nullptr), DQ4_EINVAL, "no workspace");
    expect(dq4_out_prod_rows(p8, p8, pf, pf, pf, 0.f, 10, 64, 64, 256, pf, 4, 3, 0, pf, pf, 1 << 20, nullptr), DQ4_EINVAL, "ld < m");
    expect(dq4_out_prod_rows(p8, p8, pf, pf, pf, 0.f, 10, 64, 64, 256, pf, 0, 4, 0, pf, pf, 1 << 20, nullptr), DQ4_OK, "m=0");
    expect(dq4_out_prod_fused(p8, p8, pf, pf, pf, 0.f, 10, 64, 64, 256, pf, 4, 3, 0, pf, nullptr, 0, nullptr), DQ4_EINVAL, "fused ld < m");
    expect(dq4_out_prod_fused(p8, p8, pf, pf, pf, 0.f, 10, 64, 64, 256, pf, 0, 4, 0, pf, nullptr, 0, nullptr), DQ4_OK, "fused m=0");
    expect(dq4_out_prod_fused(p8, p8, pf, pf, pf, 0.f, 10, 64, 64, 256, pf, 4, 4, 0, pf, nullptr, 64, nullptr), DQ4_EINVAL, "fused size without workspace");
    expect(static_cast<int>(dq4_out_prod_fused_workspace_bytes(INT64_MAX, INT64_MAX, 2, 0)), 0, "fused workspace overflow");
    expect(static_cast<int>(dq4_out_prod_fused_workspace_bytes(INT64_MAX, 64, 2, 1)), 0, "fused workspace copy overflow");
    expect(static_cast<int>(dq4_out_prod_fused_workspace_bytes(100, 64, 8, 2)), 0, "fused workspace orientation");
    expect(dq4_dequant_linear(p8, p8, pf, pf, pf, 0.f, 64, 64, 64, 256, DQ4_F32, 0, pv, 4, pv, pv, nullptr), DQ4_EINVAL, "linear f32");
    expect(dq4_int8_prep(nullptr, 4, 64, nullptr, nullptr, 8, nullptr, 0, nullptr, nullptr, nullptr), DQ4_OK, "int8 L=0");
    expect(dq4_int8_prep(reinterpret_cast<uint16_t *>(pv), 1 << 20, 1 << 12, reinterpret_cast<int8_t *>(pv), pf, 8,
                         reinterpret_cast<int64_t *>(pv), 2, reinterpret_cast<uint16_t *>(pv), reinterpret_cast<uint16_t *>(pv), nullptr),
           DQ4_EUNSUPPORTED, "int8 too large");
    expect(dq4_rows_per_block(5376, 4, 268435456), 12483, "rows per block");
    expect(dq4_rows_per_block(INT64_MAX, 4, 1), 1, "rows per block overflow");
    expect(static_cast<int>(dq4_unfused_workspace_bytes(INT64_MAX / 2, 32) > 0), 1, "workspace bytes");
    for (int st = -1; st < 6; ++st)
        if (!dq4_status_string(st))
            ++failures;
    printf("abi sanitizer driver: %d failures\n", failures);
    return failures != 0;
}

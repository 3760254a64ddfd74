/* C99 client of include/mxq.h that runs on the GPU: device memory and a stream
 * from the HIP runtime's C API, the library's entry points called directly
 * (no Python, no PyTorch), and every output byte compared with the CPU oracle
 * (oracle/mxq_oracle.h, test infrastructure linked only into this test).
 *
 * Covered: mx_quant_grouped (MXFP8 and NVFP4, linear and swizzled, ragged
 * rows, a strided source), the same entries through mx_quant_grouped_batch
 * (two launches, the second chained), nvfp4_quant_split_row_scaled (empty and ragged
 * experts, swizzled) and rmsnorm_quant_fused (MXFP8, swizzled; 1, 3 and 20
 * rows).  Prints
 * "ok: N checks" and exits 0 when everything matches. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "mxq.h"
#include "mxq_oracle.h"

static int checks = 0, fails = 0;

#define HIP_OK(call)                                                                   \
    do {                                                                               \
        hipError_t e_ = (call);                                                        \
        if (e_ != hipSuccess) {                                                        \
            printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
            exit(2);                                                                   \
        }                                                                              \
    } while (0)

static void expect_bytes(const char *what, const void *got, const void *want, size_t n) {
    ++checks;
    if (memcmp(got, want, n) != 0) {
        const uint8_t *a = got, *b = want;
        size_t i = 0;
        while (a[i] == b[i]) ++i;
        printf("FAIL %s: first difference at byte %zu of %zu (%u vs %u)\n", what, i, n, a[i],
               b[i]);
        ++fails;
    }
}

static void expect_status(const char *what, int st) {
    ++checks;
    if (st != MXQ_OK) {
        printf("FAIL %s: %s\n", what, mxq_status_str(st));
        ++fails;
    }
}

/* splitmix64: a seeded stream of finite bf16 values with a spread of scales */
static uint64_t rng_state = 0x1234567ULL;
static uint64_t next_u64(void) {
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ULL);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}
static uint16_t next_bf16(int row_exp) {
    const uint64_t r = next_u64();
    const uint32_t sign = (uint32_t)(r & 1) << 15;
    const int exp = 127 + row_exp + (int)((r >> 1) % 9) - 4; /* 2^(row_exp +- 4) */
    const uint32_t mant = (uint32_t)((r >> 8) & 0x7F);
    return (uint16_t)(sign | ((uint32_t)exp << 7) | mant);
}
static void fill(uint16_t *x, int64_t rows, int64_t cols, int64_t ld) {
    for (int64_t r = 0; r < rows; ++r) {
        const int row_exp = (int)(next_u64() % 17) - 8;
        for (int64_t c = 0; c < ld; ++c) x[r * ld + c] = next_bf16(row_exp);
    }
    (void)cols;
}

static void *dmalloc(size_t n) {
    void *p = NULL;
    HIP_OK(hipMalloc(&p, n ? n : 16));
    return p;
}
static void *hmalloc(size_t n) {
    void *p = malloc(n ? n : 16);
    if (!p) exit(2);
    return p;
}

static void grouped(hipStream_t s, int fmt, int layout, int batched) {
    enum { N = 3 };
    const int64_t cols = 768, rows[N] = {130, 1, 64}, ld[N] = {768, 1024, 768};
    const int64_t pw = fmt == MXQ_MXFP8 ? cols : cols / 2;
    mxq_entry e[N];
    uint16_t *h_src[N];
    float h_g[N];
    float *d_g = dmalloc(sizeof h_g);
    for (int i = 0; i < N; ++i) {
        h_src[i] = hmalloc((size_t)(rows[i] * ld[i] * 2));
        fill(h_src[i], rows[i], cols, ld[i]);
        h_g[i] = orc_nvfp4_encode_scale(orc_tensor_amax(h_src[i], rows[i], cols, ld[i]));
    }
    HIP_OK(hipMemcpy(d_g, h_g, sizeof h_g, hipMemcpyHostToDevice));
    for (int i = 0; i < N; ++i) {
        const int64_t sb = mxq_scale_bytes(rows[i], cols, fmt, layout);
        e[i].src = dmalloc((size_t)(rows[i] * ld[i] * 2));
        e[i].payload = dmalloc((size_t)(rows[i] * pw));
        e[i].scales = dmalloc((size_t)sb);
        e[i].global_scale = fmt == MXQ_NVFP4 ? d_g + i : NULL;
        e[i].rows = rows[i];
        e[i].src_ld = ld[i];
        HIP_OK(hipMemcpy((void *)e[i].src, h_src[i], (size_t)(rows[i] * ld[i] * 2),
                         hipMemcpyHostToDevice));
    }
    if (batched)
        expect_status("mx_quant_grouped_batch",
                      mx_quant_grouped_batch(fmt, layout, cols, e, N, 2, MXQ_CHAIN, s));
    else
        expect_status("mx_quant_grouped", mx_quant_grouped(fmt, layout, cols, e, N, s));
    HIP_OK(hipStreamSynchronize(s));
    for (int i = 0; i < N; ++i) {
        const int64_t sb = mxq_scale_bytes(rows[i], cols, fmt, layout);
        uint8_t *got_p = hmalloc((size_t)(rows[i] * pw)), *want_p = hmalloc((size_t)(rows[i] * pw));
        uint8_t *got_s = hmalloc((size_t)sb), *want_s = hmalloc((size_t)sb);
        HIP_OK(hipMemcpy(got_p, e[i].payload, (size_t)(rows[i] * pw), hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(got_s, e[i].scales, (size_t)sb, hipMemcpyDeviceToHost));
        orc_quantize(fmt, layout, h_src[i], rows[i], cols, ld[i], h_g[i], want_p, want_s);
        expect_bytes("grouped payload", got_p, want_p, (size_t)(rows[i] * pw));
        expect_bytes("grouped scales", got_s, want_s, (size_t)sb);
        free(got_p); free(want_p); free(got_s); free(want_s);
        HIP_OK(hipFree((void *)e[i].src));
        HIP_OK(hipFree(e[i].payload));
        HIP_OK(hipFree(e[i].scales));
        free(h_src[i]);
    }
    HIP_OK(hipFree(d_g));
}

static void split_row_scaled(hipStream_t s) {
    enum { N = 5 };
    const int64_t split[N] = {0, 5, 140, 0, 1};
    const int64_t T = 146, cols = 512, pw = cols / 2;
    const int64_t sb = mxq_split_scale_offset(split, N, N, cols, MXQ_NVFP4, MXQ_SF_SWIZZLED);
    uint16_t *h_x = hmalloc((size_t)(T * cols * 2));
    fill(h_x, T, cols, cols);
    void *d_x = dmalloc((size_t)(T * cols * 2)), *d_p = dmalloc((size_t)(T * pw));
    void *d_s = dmalloc((size_t)sb);
    float *d_a = dmalloc((size_t)T * 4);
    HIP_OK(hipMemcpy(d_x, h_x, (size_t)(T * cols * 2), hipMemcpyHostToDevice));
    expect_status("nvfp4_quant_split_row_scaled",
                  nvfp4_quant_split_row_scaled(d_x, T, cols, split, N, d_p, d_s, d_a,
                                               MXQ_SF_SWIZZLED, s));
    HIP_OK(hipStreamSynchronize(s));
    uint8_t *got_p = hmalloc((size_t)(T * pw)), *want_p = hmalloc((size_t)(T * pw));
    uint8_t *got_s = hmalloc((size_t)sb), *want_s = hmalloc((size_t)sb);
    float *got_a = hmalloc((size_t)T * 4), *want_a = hmalloc((size_t)T * 4);
    HIP_OK(hipMemcpy(got_p, d_p, (size_t)(T * pw), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(got_s, d_s, (size_t)sb, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(got_a, d_a, (size_t)T * 4, hipMemcpyDeviceToHost));
    orc_split(MXQ_NVFP4, 1, h_x, T, cols, split, N, 1.0f, MXQ_SF_SWIZZLED, want_p, want_s,
              want_a);
    expect_bytes("split payload", got_p, want_p, (size_t)(T * pw));
    expect_bytes("split scales", got_s, want_s, (size_t)sb);
    expect_bytes("split row amax", got_a, want_a, (size_t)T * 4);
    free(h_x); free(got_p); free(want_p); free(got_s); free(want_s); free(got_a); free(want_a);
    HIP_OK(hipFree(d_x)); HIP_OK(hipFree(d_p)); HIP_OK(hipFree(d_s)); HIP_OK(hipFree(d_a));
}

static void fused(hipStream_t s, int64_t T) {
    const int64_t H = 256;
    const int64_t sb = mxq_scale_bytes(T, H, MXQ_MXFP8, MXQ_SF_SWIZZLED);
    const size_t nb = (size_t)(T * H * 2);
    uint16_t *h_x = hmalloc(nb), *h_r = hmalloc(nb), *h_gm = hmalloc((size_t)H * 2);
    fill(h_x, T, H, H);
    fill(h_r, T, H, H);
    for (int64_t c = 0; c < H; ++c) h_gm[c] = (uint16_t)(0x3F80 + (next_u64() % 32) - 16);
    void *d_x = dmalloc(nb), *d_r = dmalloc(nb), *d_gm = dmalloc((size_t)H * 2);
    void *d_ro = dmalloc(nb), *d_no = dmalloc(nb), *d_p = dmalloc((size_t)(T * H));
    void *d_s = dmalloc((size_t)sb);
    HIP_OK(hipMemcpy(d_x, h_x, nb, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_r, h_r, nb, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_gm, h_gm, (size_t)H * 2, hipMemcpyHostToDevice));
    expect_status("rmsnorm_quant_fused",
                  rmsnorm_quant_fused(MXQ_MXFP8, MXQ_SF_SWIZZLED, d_x, d_r, d_gm, 1e-6f, T, H,
                                      NULL, d_ro, d_no, d_p, d_s, s));
    HIP_OK(hipStreamSynchronize(s));
    uint16_t *ro = hmalloc(nb), *no = hmalloc(nb), *want_ro = hmalloc(nb), *want_no = hmalloc(nb);
    uint8_t *got_p = hmalloc((size_t)(T * H)), *want_p = hmalloc((size_t)(T * H));
    uint8_t *got_s = hmalloc((size_t)sb), *want_s = hmalloc((size_t)sb);
    HIP_OK(hipMemcpy(ro, d_ro, nb, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(no, d_no, nb, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(got_p, d_p, (size_t)(T * H), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(got_s, d_s, (size_t)sb, hipMemcpyDeviceToHost));
    orc_add_rmsnorm(h_x, h_r, h_gm, 1e-6f, T, H, want_ro, want_no);
    expect_bytes("fused residual_out", ro, want_ro, nb);
    /* norm_out: within one bf16 ulp of the oracle's (same sign, so a bit-pattern distance) */
    ++checks;
    for (int64_t k = 0; k < T * H; ++k) {
        const int d = (int)no[k] - (int)want_no[k];
        if (d > 1 || d < -1 || ((no[k] ^ want_no[k]) & 0x8000)) {
            printf("FAIL fused norm_out at %lld: %04x vs %04x\n", (long long)k, no[k], want_no[k]);
            ++fails;
            break;
        }
    }
    /* the quantized form is the quantization of the GPU's own norm_out */
    orc_quantize(MXQ_MXFP8, MXQ_SF_SWIZZLED, no, T, H, H, 1.0f, want_p, want_s);
    expect_bytes("fused payload", got_p, want_p, (size_t)(T * H));
    expect_bytes("fused scales", got_s, want_s, (size_t)sb);
    free(h_x); free(h_r); free(h_gm); free(ro); free(no); free(want_ro); free(want_no);
    free(got_p); free(want_p); free(got_s); free(want_s);
    HIP_OK(hipFree(d_x)); HIP_OK(hipFree(d_r)); HIP_OK(hipFree(d_gm)); HIP_OK(hipFree(d_ro));
    HIP_OK(hipFree(d_no)); HIP_OK(hipFree(d_p)); HIP_OK(hipFree(d_s));
}

int main(void) {
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    for (int fmt = 0; fmt < 2; ++fmt)
        for (int layout = 0; layout < 2; ++layout) {
            printf("grouped fmt %d layout %d\n", fmt, layout);
            fflush(stdout);
            grouped(s, fmt, layout, 0);
            printf("grouped batch, chained, fmt %d layout %d\n", fmt, layout);
            fflush(stdout);
            grouped(s, fmt, layout, 1);
        }
    printf("row-scaled split\n");
    fflush(stdout);
    split_row_scaled(s);
    /* 1 and 20 rows run the one-workgroup-per-row kernel, 3 the general one */
    const int64_t fused_rows[] = {1, 3, 20};
    for (int i = 0; i < 3; ++i) {
        printf("fused epilogue, %lld rows\n", (long long)fused_rows[i]);
        fflush(stdout);
        fused(s, fused_rows[i]);
    }
    HIP_OK(hipStreamDestroy(s));
    printf("ok: %d checks, %d failed\n", checks, fails);
    return fails ? 1 : 0;
}

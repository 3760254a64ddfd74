/* C99 client of include/mxq.h: compiles against the header with a plain C
 * compiler, links libmxq.so and checks host-side behaviour that needs no GPU
 * (every compute call here fails validation or is a no-op, so nothing is
 * launched).  Exit status 0 when every check passes. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mxq.h"

static int fails = 0;

#define EXPECT(expr, want)                                                          \
    do {                                                                            \
        long long got_ = (long long)(expr);                                         \
        if (got_ != (long long)(want)) {                                            \
            printf("FAIL %s = %lld, want %lld\n", #expr, got_, (long long)(want));  \
            ++fails;                                                                \
        }                                                                           \
    } while (0)

int main(void) {
    /* a 16-byte aligned address that is never dereferenced */
    void *A = (void *)(uintptr_t)0x10000;
    mxq_entry e;
    int64_t split[5] = {0, 1, 129, 0, 3};
    int slots[2] = {0, 2};

    memset(&e, 0, sizeof e);
    e.src = A;
    e.payload = A;
    e.scales = A;
    e.global_scale = (const float *)A;
    e.rows = 4;
    e.src_ld = 64;

    /* sizes: swizzled pads rows to 128 and scale columns to 4 */
    EXPECT(mxq_scale_bytes(130, 64, MXQ_MXFP8, MXQ_SF_SWIZZLED), 256 * 4);
    EXPECT(mxq_scale_bytes(130, 64, MXQ_MXFP8, MXQ_SF_LINEAR), 130 * 2);
    EXPECT(mxq_scale_bytes(3, 7168, MXQ_NVFP4, MXQ_SF_SWIZZLED), 128 * 448);
    EXPECT(mxq_scale_bytes(3, 48, MXQ_MXFP8, MXQ_SF_LINEAR), -1);
    EXPECT(mxq_split_scale_offset(split, 5, 0, 64, MXQ_MXFP8, MXQ_SF_SWIZZLED), 0);
    EXPECT(mxq_split_scale_offset(split, 5, 2, 64, MXQ_MXFP8, MXQ_SF_SWIZZLED), 512);
    EXPECT(mxq_split_scale_offset(split, 5, 5, 64, MXQ_MXFP8, MXQ_SF_SWIZZLED), 512 + 1024 + 512);
    EXPECT(mxq_split_scale_offset(split, 5, 5, 64, MXQ_MXFP8, MXQ_SF_LINEAR), 133 * 2);
    EXPECT(mxq_split_scale_offset(split, 5, 6, 64, MXQ_MXFP8, MXQ_SF_LINEAR), -1);

    /* validation */
    EXPECT(mx_quant_grouped(MXQ_MXFP8, MXQ_SF_LINEAR, 64, NULL, 1, NULL), MXQ_EINVAL);
    EXPECT(mx_quant_grouped(MXQ_MXFP8, MXQ_SF_LINEAR, 64, &e, 0, NULL), MXQ_EINVAL);
    EXPECT(mx_quant_grouped(MXQ_MXFP8, MXQ_SF_LINEAR, 48, &e, 1, NULL), MXQ_ESHAPE);
    EXPECT(mx_quant_grouped(7, MXQ_SF_LINEAR, 64, &e, 1, NULL), MXQ_EINVAL);
    e.src_ld = 60;
    EXPECT(mx_quant_grouped(MXQ_MXFP8, MXQ_SF_LINEAR, 64, &e, 1, NULL), MXQ_ESHAPE);
    e.src_ld = 64;
    e.rows = 0;  /* nothing to do: no launch */
    EXPECT(mx_quant_grouped(MXQ_NVFP4, MXQ_SF_SWIZZLED, 64, &e, 1, NULL), MXQ_OK);
    e.rows = 4;
    EXPECT(nvfp4_quant_grouped_auto(MXQ_SF_LINEAR, 64, &e, 2, slots, 2, (float *)A, (float *)A,
                                    NULL), MXQ_EINVAL);  /* slot 2 of 2 */
    EXPECT(nvfp4_quant_grouped_auto(MXQ_SF_LINEAR, 64, &e, 1, NULL, 1, NULL, (float *)A, NULL),
           MXQ_EINVAL);
    EXPECT(nvfp4_quant_split(A, 8, 64, split, 5, (const float *)A, A, A, NULL, MXQ_SF_LINEAR,
                             NULL), MXQ_EINVAL);  /* splits add up to 133 */
    EXPECT(nvfp4_quant_split_row_scaled(A, 133, 64, split, 5, A, A, NULL, MXQ_SF_LINEAR, NULL),
           MXQ_EINVAL);  /* row amax is required */
    EXPECT(mxfp8_quant_split(A, 133, 48, split, 5, A, A, NULL, MXQ_SF_LINEAR, NULL),
           MXQ_ESHAPE);
    EXPECT(rmsnorm_quant_fused(MXQ_MXFP8, MXQ_SF_SWIZZLED, A, A, A, 0.0f, 4, 256, NULL, A, A, A,
                               A, NULL), MXQ_EINVAL);  /* eps must be > 0 */
    EXPECT(rmsnorm_quant_fused(MXQ_MXFP8, MXQ_SF_SWIZZLED, A, A, A, 1e-6f, 4, 96, NULL, A, A, A,
                               A, NULL), MXQ_ESHAPE);  /* would pad scale columns */
    EXPECT(scale_swizzle(A, 4, 0, A, NULL), MXQ_EINVAL);
    EXPECT(scale_swizzle(NULL, 0, 4, NULL, NULL), MXQ_OK);
    EXPECT(strcmp(mxq_status_str(MXQ_OK), "ok"), 0);
    EXPECT(mxq_status_str(12345) != NULL, 1);

    printf("%s: %d failed\n", fails ? "FAIL" : "ok", fails);
    return fails != 0;
}

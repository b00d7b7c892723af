/* A plain C99 client of the C ABI: it includes include/tea.h, links
 * libtea.so and calls the entry points on arguments that every one of them
 * rejects, or answers, before any HIP call (argument validation, workspace
 * sizes, status strings), so it runs without a GPU.  Prints "c client ok"
 * on success; on a mismatch prints the failing check and exits 1. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tea.h"

static int failures = 0;

#define EXPECT(expr, want)                                                                       \
    do {                                                                                         \
        long long got_ = (long long)(expr);                                                      \
        if (got_ != (long long)(want)) {                                                         \
            fprintf(stderr, "%s:%d: %s = %lld, expected %lld\n", __FILE__, __LINE__, #expr, got_, \
                    (long long)(want));                                                          \
            ++failures;                                                                          \
        }                                                                                        \
    } while (0)

int main(void)
{
    /* fake, 16-byte aligned device addresses, far apart: never dereferenced */
    void* const a = (void*)(uintptr_t)0x10000000u;
    void* const b = (void*)(uintptr_t)0x20000000u;
    void* const c = (void*)(uintptr_t)0x30000000u;
    void* const d = (void*)(uintptr_t)0x40000000u;
    void* const e = (void*)(uintptr_t)0x50000000u;

    EXPECT(tea_abi_version() >= 1, 1);
    for (int s = TEA_OK; s <= TEA_ENOSPACE; ++s) EXPECT(tea_status_string(s) != NULL && strlen(tea_status_string(s)) > 0, 1);

    /* row_softmax: negative size, unknown dtype, null pointers, unsupported block; empty is a no-op */
    EXPECT(row_softmax(a, b, -1, 8, TEA_F32, 8, NULL, NULL, NULL), TEA_EINVAL);
    EXPECT(row_softmax(a, b, 4, 8, 7, 8, NULL, NULL, NULL), TEA_EINVAL);
    EXPECT(row_softmax(NULL, b, 4, 8, TEA_F32, 8, NULL, NULL, NULL), TEA_EINVAL);
    EXPECT(row_softmax(a, b, 4, 8, TEA_F32, 3, NULL, NULL, NULL), TEA_EUNSUPPORTED);
    EXPECT(row_softmax(a, b, 0, 8, TEA_F32, 8, NULL, NULL, NULL), TEA_OK);
    EXPECT(row_softmax_variant(a, b, 4, 8, TEA_F32, 8, 9, NULL, NULL, NULL), TEA_EINVAL);

    /* attn_fwd: head dimension, causal shape, scale; an empty batch is a no-op */
    EXPECT(attn_fwd(a, b, c, d, 1, 1, 8, 8, 96, 0.1f, 0, TEA_BF16, NULL, NULL), TEA_EUNSUPPORTED);
    EXPECT(attn_fwd(a, b, c, d, 1, 1, 8, 16, 64, 0.1f, 1, TEA_BF16, NULL, NULL), TEA_EUNSUPPORTED);
    EXPECT(attn_fwd(a, b, c, d, 1, 1, 8, 8, 64, 0.0f, 0, TEA_BF16, NULL, NULL), TEA_EINVAL);
    EXPECT(attn_fwd(a, b, c, d, 1, 1, 8, 8, 64, -1.0f, 0, TEA_BF16, NULL, NULL), TEA_EINVAL);
    EXPECT(attn_fwd(a, b, c, d, 0, 1, 8, 8, 64, 0.1f, 0, TEA_BF16, NULL, NULL), TEA_OK);
    EXPECT(attn_fwd(NULL, b, c, d, 1, 1, 8, 8, 64, 0.1f, 0, TEA_BF16, NULL, NULL), TEA_EINVAL);

    /* split-K workspace sizes and limits */
    EXPECT(attn_fwd_splitk_workspace_bytes(1, 1, 8, 64, 65), 0);
    EXPECT(attn_fwd_splitk_workspace_bytes(1, 1, 8, 64, 4) >= (size_t)8 * 4 * (64 + 2) * 4, 1);
    EXPECT(attn_fwd_splitk(a, b, c, d, 1, 1, 8, 8, 64, 0.1f, 0, 4, TEA_BF16, NULL, e, 16, NULL), TEA_EINVAL);

    /* decode: workspace size, splits, the allocation-free form's limit */
    EXPECT(attn_decode_workspace_bytes(16, 32, 128, 64) >= (size_t)16 * 32 * 64 * (128 + 2) * 4, 1);
    EXPECT(attn_decode_workspace_bytes(1, 1, 128, 0), 0);
    EXPECT(attn_decode_splitkv(a, b, c, (const int32_t*)d, e, 2, 2, 100, 128, 0, 0.1f, TEA_BF16, e, 0, NULL),
           TEA_EINVAL);
    EXPECT(attn_decode_workspace_bytes(64, 32, 128, 64) > TEA_DECODE_NOALLOC_MAX_BYTES, 1);
    EXPECT(attn_decode_splitkv_noalloc(a, b, c, (const int32_t*)d, e, 64, 32, 100, 128, 64, 0.1f, TEA_BF16, NULL),
           TEA_ENOSPACE);
    EXPECT(attn_decode_fused(a, b, c, (const int32_t*)d, e, 2, 2, 100, 128, 65, 0.1f, TEA_BF16, NULL), TEA_EINVAL);

    /* merge_partials: the output may not overlap the inputs; nothing to merge is a no-op */
    EXPECT(merge_partials((const float*)a, (const float*)b, (const float*)c, 4, 8, 8, NULL, NULL, c, TEA_F32, 1,
                          NULL),
           TEA_EINVAL);
    EXPECT(merge_partials((const float*)a, (const float*)b, (const float*)c, 0, 8, 8, NULL, NULL, d, TEA_F32, 1,
                          NULL),
           TEA_OK);

    if (failures) return 1;
    printf("c client ok\n");
    return 0;
}

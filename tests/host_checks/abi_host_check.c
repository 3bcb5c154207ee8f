/* Host-side checks of the C ABI, built with AddressSanitizer and UndefinedBehavior-
 * Sanitizer on the host code of every library source (device code is not built, and
 * nothing here launches a kernel): argument validation of every entry point, zero-size
 * calls, the kernel-coverage queries, and the pure host arithmetic of the workspace and
 * split plans over a sweep of shapes.  Exit status 0 when every expectation holds. */
#include <stdint.h>
#include <stdio.h>

#include "gqa_attn.h"

#define A16 ((void *)0x10000) /* aligned, never dereferenced: validation fails first */
#define F16 ((float *)0x10000)
#define MIS ((void *)0x10004) /* not 16-byte aligned */

static int fails = 0;
#define EXPECT(call, code)                                                               \
    do {                                                                                 \
        long rc_ = (long)(call);                                                         \
        if (rc_ != (long)(code)) {                                                       \
            printf("FAIL line %d: %s -> %ld, want %ld\n", __LINE__, #call, rc_, (long)(code)); \
            ++fails;                                                                     \
        }                                                                                \
    } while (0)

int main(void) {
    /* prefill: each argument outside its domain */
    EXPECT(attn_prefill(A16, A16, A16, F16, -1, 2, 1, 4, 8, 0.5f, 1, GQA_BF16, NULL), GQA_EINVAL);
    EXPECT(attn_prefill(A16, A16, A16, F16, 1, 0, 1, 4, 8, 0.5f, 1, GQA_BF16, NULL), GQA_EINVAL);
    EXPECT(attn_prefill(A16, A16, A16, F16, 1, 2, 0, 4, 8, 0.5f, 1, GQA_BF16, NULL), GQA_EINVAL);
    EXPECT(attn_prefill(A16, A16, A16, F16, 1, 3, 2, 4, 8, 0.5f, 1, GQA_BF16, NULL), GQA_EINVAL);
    EXPECT(attn_prefill(A16, A16, A16, F16, 1, 2, 1, -4, 8, 0.5f, 1, GQA_BF16, NULL), GQA_EINVAL);
    EXPECT(attn_prefill(A16, A16, A16, F16, 1, 2, 1, 4, 0, 0.5f, 1, GQA_BF16, NULL), GQA_EINVAL);
    EXPECT(attn_prefill(A16, A16, A16, F16, 1, 2, 1, 4, 257, 0.5f, 1, GQA_BF16, NULL), GQA_EUNSUPPORTED);
    EXPECT(attn_prefill(A16, A16, A16, F16, 1, 2, 1, 4, 8, 1.0f / 0.0f, 1, GQA_BF16, NULL), GQA_EINVAL);
    EXPECT(attn_prefill(A16, A16, A16, F16, 1, 2, 1, 4, 8, 0.5f, 2, GQA_BF16, NULL), GQA_EINVAL);
    EXPECT(attn_prefill(A16, A16, A16, F16, 1, 2, 1, 4, 8, 0.5f, 1, 7, NULL), GQA_EINVAL);
    EXPECT(attn_prefill(NULL, A16, A16, F16, 1, 2, 1, 4, 8, 0.5f, 1, GQA_BF16, NULL), GQA_EINVAL);
    EXPECT(attn_prefill(A16, A16, MIS, F16, 1, 2, 1, 4, 8, 0.5f, 1, GQA_BF16, NULL), GQA_EINVAL);
    EXPECT(attn_prefill(A16, A16, A16, F16, 70000, 70000, 1, 4, 8, 0.5f, 1, GQA_BF16, NULL), GQA_EUNSUPPORTED);
    EXPECT(attn_prefill_ex(A16, A16, A16, F16, 1, 2, 1, 4, 8, 0.5f, 1, GQA_BF16, 9, NULL), GQA_EINVAL);
    EXPECT(attn_prefill_window(A16, A16, A16, F16, 1, 2, 1, 4, 8, 0.5f, 0, GQA_BF16, NULL), GQA_EINVAL);
    EXPECT(attn_prefill_lse(A16, A16, A16, F16, (float *)0x10002, 1, 2, 1, 4, 8, 0.5f, 1, GQA_BF16, NULL),
           GQA_EINVAL);
    /* empty tensors: nothing to do, NULL pointers accepted */
    EXPECT(attn_prefill(NULL, NULL, NULL, NULL, 0, 2, 1, 4, 8, 0.5f, 1, GQA_BF16, NULL), GQA_OK);
    EXPECT(attn_prefill(NULL, NULL, NULL, NULL, 3, 2, 1, 0, 8, 0.5f, 1, GQA_F32, NULL), GQA_OK);
    /* kernel coverage, asked with empty calls */
    for (int d = 1; d <= 256; ++d) {
        const int mf = d % 16 == 0 && d <= 128;
        EXPECT(attn_prefill_ex(NULL, NULL, NULL, NULL, 0, 4, 2, 1, d, 1.0f, 1, GQA_BF16, GQA_ALGO_MFMA, NULL),
               mf ? GQA_OK : GQA_EUNSUPPORTED);
        EXPECT(attn_prefill_ex(NULL, NULL, NULL, NULL, 0, 4, 2, 1, d, 1.0f, 1, GQA_BF16, GQA_ALGO_MFMA_SPLIT, NULL),
               mf ? GQA_OK : GQA_EUNSUPPORTED);
        EXPECT(attn_prefill_ex(NULL, NULL, NULL, NULL, 0, 4, 2, 1, d, 1.0f, 1, GQA_F32, GQA_ALGO_MFMA_SPLIT, NULL),
               mf ? GQA_OK : GQA_EUNSUPPORTED);
        EXPECT(attn_prefill_ex(NULL, NULL, NULL, NULL, 0, 4, 2, 1, d, 1.0f, 1, GQA_F32, GQA_ALGO_GENERIC, NULL),
               GQA_OK);
    }

    /* decode rejections and empty calls */
    EXPECT(attn_decode_cached(A16, A16, A16, F16, 2, 10, 9, 4, 2, 64, 1, GQA_BF16, A16, 1 << 20, NULL), GQA_EINVAL);
    EXPECT(attn_decode_cached(A16, A16, A16, F16, -1, 10, 0, 4, 2, 64, 1, GQA_BF16, A16, 1 << 20, NULL), GQA_EINVAL);
    EXPECT(attn_decode_cached(A16, A16, A16, F16, 1, 10, -1, 4, 2, 64, 1, GQA_BF16, A16, 1 << 20, NULL), GQA_EINVAL);
    EXPECT(attn_decode_cached(A16, A16, A16, F16, 1, 10, 9, 4, 3, 64, 1, GQA_BF16, A16, 1 << 20, NULL), GQA_EINVAL);
    EXPECT(attn_decode_cached(A16, A16, A16, F16, 1, 4096, 4095, 32, 8, 128, 64, GQA_BF16, NULL, 0, NULL),
           GQA_EWORKSPACE);
    EXPECT(attn_decode_cached(A16, A16, A16, F16, 1, 4096, 4095, 32, 8, 128, 64, GQA_BF16, A16, 16, NULL),
           GQA_EWORKSPACE);
    EXPECT(attn_decode_cached(NULL, NULL, NULL, NULL, 0, 10, 10, 4, 2, 64, 1, GQA_BF16, NULL, 0, NULL), GQA_OK);
    EXPECT(attn_decode_window(A16, A16, A16, F16, 1, 10, 9, 4, 2, 64, 1, 0, GQA_BF16, A16, 1 << 20, NULL),
           GQA_EINVAL);
    EXPECT(attn_decode_cached_noalloc(A16, A16, A16, F16, 64, 32768, 32768 - 64, 32, 8, 128, 64, GQA_BF16, NULL),
           GQA_ESCRATCH);
    EXPECT(attn_decode_cached_noalloc(A16, A16, A16, F16, 2, 10, 9, 4, 2, 64, 1, GQA_BF16, NULL), GQA_EINVAL);
    EXPECT(attn_decode_cached_noalloc(NULL, NULL, NULL, NULL, 0, 10, 10, 4, 2, 64, 1, GQA_BF16, NULL), GQA_OK);

    /* paged decode rejections */
    int tab[4] = {0, 1, 2, 3}, lens[1] = {40};
    EXPECT(attn_decode_paged(A16, A16, A16, tab, lens, F16, 1, 1, 4, 2, 64, 0, 4, 4, GQA_BF16, A16, 1 << 20, NULL),
           GQA_EINVAL);
    EXPECT(attn_decode_paged(A16, A16, A16, tab, lens, F16, 1, 1, 4, 2, 64, 24, 4, 4, GQA_BF16, A16, 1 << 20, NULL),
           GQA_EUNSUPPORTED);
    EXPECT(attn_decode_paged(A16, A16, A16, tab, lens, F16, 1, 1, 4, 2, 64, 16, 4, 4, GQA_F32, A16, 1 << 20, NULL),
           GQA_EUNSUPPORTED);
    EXPECT(attn_decode_blocks(A16, A16, A16, NULL, lens, F16, 1, 1, 4, 2, 64, 16, 4, 4, GQA_BF16, A16, 1 << 20, NULL),
           GQA_EINVAL);

    /* append and backward rejections */
    EXPECT(attn_kv_append((float *)A16, (float *)A16, A16, A16, NULL, 1, 2, 2, 12, 10, 0, 10000.f, GQA_BF16, NULL),
           GQA_EUNSUPPORTED);
    EXPECT(attn_kv_append((float *)A16, (float *)A16, A16, A16, NULL, 1, 2, 2, 64, 10, 9, 10000.f, GQA_BF16, NULL),
           GQA_EINVAL);
    EXPECT(attn_backward(A16, A16, A16, F16, F16, F16, F16, F16, F16, 1, 2, 1, 8, 64, 0.5f, 1, GQA_BF16, NULL, 0, NULL),
           GQA_EWORKSPACE);
    EXPECT(attn_backward(A16, A16, A16, F16, F16, F16, F16, F16, F16, 1, 2, 1, 8, 64, 0.5f, 3, GQA_BF16, A16, 1 << 20,
                         NULL),
           GQA_EINVAL);

    /* the split plan: workspace = B * Hq * n * splits * (d + 2) floats for bf16 caches,
       nothing for fp32 ones (the vector kernel), 0 for rejected shapes */
    const int Bs[] = {1, 3, 64}, ns[] = {1, 4, 17}, Ls[] = {1, 31, 32, 33, 4096, 32768};
    const int heads[][2] = {{4, 1}, {8, 2}, {32, 8}, {6, 6}};
    for (int ib = 0; ib < 3; ++ib)
        for (int in = 0; in < 3; ++in)
            for (int il = 0; il < 6; ++il)
                for (int ih = 0; ih < 4; ++ih)
                    for (int d = 16; d <= 128; d += 16) {
                        const int B = Bs[ib], n = ns[in], L = Ls[il], Hq = heads[ih][0], Hkv = heads[ih][1];
                        const size_t ws = attn_decode_workspace_bytes(B, n, L, Hq, Hkv, d, GQA_BF16);
                        const int sp = attn_decode_num_splits(B, n, L, Hq, Hkv, d, GQA_BF16);
                        if (n > L) {
                            EXPECT(ws, 0);
                            EXPECT(sp, 0);
                            continue;
                        }
                        if (sp < 1 || (long)sp * 32 > (long)L + 31) {
                            printf("FAIL: splits %d for L=%d\n", sp, L);
                            ++fails;
                        }
                        EXPECT(ws, (size_t)B * Hq * n * sp * (d + 2) * 4);
                        EXPECT(attn_decode_workspace_bytes(B, n, L, Hq, Hkv, d, GQA_F32), 0);
                        EXPECT(attn_decode_paged_workspace_bytes(B, n, Hq, Hkv, d, 16, (L + 15) / 16, GQA_BF16) > 0,
                               1);
                    }
    EXPECT(attn_decode_workspace_bytes(1, 1, 10, 4, 3, 64, GQA_BF16), 0);
    EXPECT(attn_decode_window_workspace_bytes(1, 1, 10, 4, 2, 64, 0, GQA_BF16), 0);
    EXPECT(attn_backward_workspace_bytes(2, 16, 8, 4096, 128, GQA_BF16) > 0, 1);
    EXPECT(attn_backward_workspace_bytes(2, 16, 7, 4096, 128, GQA_BF16), 0);

    for (int code = 1; code >= -6; --code)
        if (!attn_strerror(code) || !attn_strerror(code)[0]) {
            printf("FAIL: empty strerror(%d)\n", code);
            ++fails;
        }
    printf("abi host checks: %d failures\n", fails);
    return fails ? 1 : 0;
}

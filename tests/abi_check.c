/* A plain C program against libpqkv: it includes only include/pqkv.h, links the
 * shared library and exercises the host-side contract (status strings, workspace
 * sizes, argument validation) without touching a GPU. */
#include <stdio.h>
#include <string.h>

#include "pqkv.h"

static int fails = 0;
#define EXPECT(cond)                                           \
    do {                                                       \
        if (!(cond)) {                                         \
            printf("FAIL line %d: %s\n", __LINE__, #cond);     \
            ++fails;                                           \
        }                                                      \
    } while (0)

int main(void) {
    pqkv_dims d = {128, 2, 256, 32, 32};
    pqkv_dims bad = {96, 2, 256, 32, 32};
    void* fake = (void*)0x10000; /* never dereferenced: validation fails first */

    EXPECT(strcmp(pqkv_status_str(PQKV_OK), "ok") == 0);
    EXPECT(pqkv_decode_workspace_bytes(&d, 1, 32768) == (size_t)(32 * 8 * 132 * 4 + 256));
    EXPECT(pqkv_decode_workspace_bytes(&bad, 1, 32768) == 0);
    {
        pqkv_decode_plan_info pi;
        memset(&pi, 0, sizeof(pi));
        EXPECT(pqkv_decode_plan(&d, 1, 32768, &pi) == PQKV_OK);
        EXPECT(pi.splits == 8 && pi.split_tokens == 4096 && pi.rounds == 8 && pi.build_rounds == 8);
        EXPECT(pi.q_heads_per_group == 1 && pi.work_groups == 256 && pi.device_plan == 0);
        EXPECT(pi.workspace_bytes == pqkv_decode_workspace_bytes(&d, 1, 32768));
        EXPECT(pqkv_decode_plan(&d, 1, 32768, NULL) == PQKV_ERR_INVALID);
        EXPECT(pqkv_decode_plan(&bad, 1, 32768, &pi) == PQKV_ERR_UNSUPPORTED);
        EXPECT(pqkv_decode_plan(&d, 0, 32768, &pi) == PQKV_ERR_INVALID);
    }
    EXPECT(pqkv_encode(&bad, fake, PQKV_F16, 1, 10, 0, 4096, 128, fake, fake, 64, 0, NULL) == PQKV_ERR_UNSUPPORTED);
    EXPECT(pqkv_encode(&d, NULL, PQKV_F16, 1, 10, 0, 4096, 128, fake, fake, 64, 0, NULL) == PQKV_ERR_INVALID);
    EXPECT(pqkv_encode(&d, NULL, PQKV_F16, 1, 0, 0, 4096, 128, NULL, NULL, 64, 0, NULL) == PQKV_OK);
    EXPECT(pqkv_merge(0, 128, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == PQKV_OK);
    EXPECT(pqkv_merge(4, 2048, fake, fake, fake, fake, fake, fake, NULL) == PQKV_ERR_UNSUPPORTED);
    EXPECT(pqkv_fit_codebooks(&d, fake, PQKV_F16, 0, 4096, 128, fake, 10, fake, NULL, NULL) == PQKV_ERR_INVALID);
    EXPECT(pqkv_append_kv(&d, 0, NULL, NULL, NULL, NULL, PQKV_F16, 128, NULL, NULL, NULL, NULL, 64, NULL, NULL,
                          NULL, NULL, 4096, 100, NULL) == PQKV_OK);
    {
        int32_t lens[4];
        EXPECT(pqkv_append_kv(&d, 1, fake, fake, fake, fake, PQKV_F16, 128, lens, lens + 1, lens, lens + 3, 64, fake,
                              fake, fake, fake, 4096, 100, NULL) == PQKV_ERR_INVALID); /* out aliases in */
    }
    EXPECT(pqkv_decode_attention(&d, 1, fake, PQKV_F16, NULL, fake, fake, fake, fake, 32768, fake, 32768, fake,
                                 fake, PQKV_F16, 128, fake, 0.088f, fake, fake, NULL, 0, NULL) == PQKV_ERR_WORKSPACE);
    /* a history needs its lengths; with no history they may be NULL */
    EXPECT(pqkv_decode_attention(&d, 1, fake, PQKV_F16, NULL, fake, fake, fake, fake, 32768, NULL, 32768, fake,
                                 fake, PQKV_F16, 128, fake, 0.088f, fake, fake, fake, 1 << 20, NULL) == PQKV_ERR_INVALID);
    EXPECT(pqkv_decode_attention(&d, 1, fake, PQKV_F16, NULL, NULL, NULL, NULL, NULL, 0, NULL, 0, fake, fake,
                                 PQKV_F16, 128, fake, 0.088f, fake, fake, NULL, 0, NULL) == PQKV_ERR_WORKSPACE);
    /* misaligned query */
    EXPECT(pqkv_decode_attention(&d, 1, (char*)fake + 4, PQKV_F16, NULL, fake, fake, fake, fake, 32768, fake, 32768,
                                 fake, fake, PQKV_F16, 128, fake, 0.088f, fake, fake, fake, 1 << 20,
                                 NULL) == PQKV_ERR_INVALID);
    /* a table in place of the key codebook */
    EXPECT(pqkv_decode_attention(&d, 1, fake, PQKV_F16, fake, NULL, fake, fake, fake, 32768, fake, 32768, fake,
                                 fake, PQKV_F16, 128, fake, 0.088f, fake, fake, NULL, 0, NULL) == PQKV_ERR_WORKSPACE);
    /* 4096 tokens, 32 heads: 8 splits per head; the counters (one per query head) come first */
    EXPECT(pqkv_decode_workspace_bytes(&d, 1, 4096) == (size_t)(256 + 32 * 8 * 132 * 4));
    printf(fails ? "abi_check: %d failures\n" : "abi_check: ok\n", fails);
    return fails != 0;
}

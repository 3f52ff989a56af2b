/* Host-side error paths of every entry point of include/wall.h, for a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitize.py).
 * Each call has one bad argument and must return its status before any HIP
 * call; pointers are fake, aligned and never dereferenced.  Exits 0 when every
 * status matches, 1 (naming the first mismatch) otherwise. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "wall.h"

#define FAKE(n) ((void *)(uintptr_t)((n) << 20))
#define INVALID WALL_ERR_INVALID_ARG
#define UNSUP WALL_ERR_UNSUPPORTED

static int failures = 0;

static void expect(const char *what, wall_status_t got, wall_status_t want) {
    if (got != want) {
        fprintf(stderr, "%s: got %s, want %s\n", what, wall_status_string(got), wall_status_string(want));
        ++failures;
    }
}

static wall_status_t scan(const void *x, wall_dtype_t dt, int64_t B, int64_t T, int64_t C, const int32_t *cu,
                          int64_t nseq, void *ws, size_t wsb) {
    return wall_prefix_scan(x, dt, (float *)FAKE(2), B, T, C, cu, nseq, 1.4426950f, ws, wsb, NULL);
}

static wall_status_t fwd(const void *q, int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t V,
                         const int32_t *cu, int64_t nseq, int64_t maxlen, void *ws, size_t wsb) {
    return wall_attn_fwd(q, FAKE(2), FAKE(3), WALL_BF16, (const float *)FAKE(4), NULL, NULL, FAKE(5),
                         (float *)FAKE(6), B, T, HQ, H, K, V, 0.088f, 0, cu, nseq, maxlen, ws, wsb, NULL);
}

static wall_status_t bwd(const void *dq, const float *G, void *dgs, int64_t K, size_t wsb) {
    return wall_attn_bwd(FAKE(1), FAKE(2), FAKE(3), WALL_BF16, (const float *)FAKE(4), G, NULL, FAKE(5),
                         (const float *)FAKE(6), FAKE(7), dq, FAKE(9), FAKE(10), FAKE(11), dgs, WALL_BF16, NULL,
                         1, 256, 4, 2, K, 128, 0.088f, 0, NULL, 0, 0, FAKE(13), wsb, NULL);
}

static wall_status_t decode(int64_t B, int64_t T, int64_t T_cap, int64_t HQ, int64_t K, int64_t C,
                            size_t wsb, int noalloc) {
    if (noalloc)
        return wall_attn_decode_noalloc(FAKE(1), FAKE(2), WALL_BF16, (const float *)FAKE(3), 0, FAKE(4),
                                        (const float *)FAKE(5), NULL, FAKE(6), NULL, B, T, T_cap, HQ, 1, K, 128,
                                        C, 0.088f, NULL);
    return wall_attn_decode(FAKE(1), FAKE(2), WALL_BF16, (const float *)FAKE(3), 0, FAKE(4),
                            (const float *)FAKE(5), NULL, FAKE(6), NULL, B, T, T_cap, HQ, 1, K, 128, C, 0.088f,
                            FAKE(7), wsb, NULL);
}

int main(void) {
    /* status names and sizes */
    if (strcmp(wall_status_string(WALL_OK), "WALL_OK") != 0 ||
        strcmp(wall_status_string((wall_status_t)99), "WALL_ERR_UNKNOWN") != 0 ||
        strcmp(wall_status_string(WALL_ERR_SCRATCH), "WALL_ERR_SCRATCH") != 0) {
        fprintf(stderr, "wall_status_string\n");
        ++failures;
    }
    if (wall_prefix_scan_workspace_size(0, 1, 1) != 0 || wall_attn_fwd_workspace_size(WALL_BF16, 1, 1, 0, 1, 64, 64, 0) != 0 ||
        wall_attn_bwd_workspace_size(1, 0, 1, 64, 0) != 0 || wall_attn_decode_workspace_size(1, 1, 1, 0) != 0) {
        fprintf(stderr, "workspace sizes of invalid shapes are not 0\n");
        ++failures;
    }
    const size_t sws = wall_prefix_scan_workspace_size(2, 300, 512);
    const size_t fws = wall_attn_fwd_workspace_size(WALL_BF16, 2, 300, 4, 2, 128, 128, 0);
    const size_t bws = wall_attn_bwd_workspace_size(1, 256, 4, 128, 0);
    const size_t dws = wall_attn_decode_workspace_size(2, 300, 4, 128);
    const int32_t *cu = (const int32_t *)FAKE(9);

    /* prefix scan */
    expect("scan null x", scan(NULL, WALL_BF16, 2, 300, 512, NULL, 0, FAKE(3), sws), INVALID);
    expect("scan B=0", scan(FAKE(1), WALL_BF16, 0, 300, 512, NULL, 0, FAKE(3), sws), INVALID);
    expect("scan short workspace", scan(FAKE(1), WALL_BF16, 2, 300, 512, NULL, 0, FAKE(3), sws - 1), INVALID);
    expect("scan misaligned", scan((char *)FAKE(1) + 2, WALL_BF16, 2, 300, 512, NULL, 0, FAKE(3), sws), INVALID);
    expect("scan varlen with B=2", scan(FAKE(1), WALL_BF16, 2, 300, 512, cu, 2, FAKE(3), sws), INVALID);
    expect("scan dtype", scan(FAKE(1), (wall_dtype_t)5, 2, 300, 512, NULL, 0, FAKE(3), sws), UNSUP);
    expect("append null out", wall_prefix_append(FAKE(1), WALL_BF16, 24, NULL, 0, NULL, 24, 2, 3, 8, 1.f, NULL),
           INVALID);

    /* forward */
    expect("fwd null q", fwd(NULL, 2, 300, 4, 2, 128, 128, NULL, 0, 300, FAKE(8), fws), INVALID);
    expect("fwd HQ % H", fwd(FAKE(1), 2, 300, 6, 4, 128, 128, NULL, 0, 300, FAKE(8), fws), INVALID);
    expect("fwd K=96", fwd(FAKE(1), 2, 300, 4, 2, 96, 128, NULL, 0, 300, FAKE(8), fws), UNSUP);
    expect("fwd short workspace", fwd(FAKE(1), 2, 300, 4, 2, 128, 128, NULL, 0, 300, FAKE(8), fws - 1), INVALID);
    expect("fwd varlen B=2", fwd(FAKE(1), 2, 300, 4, 2, 128, 128, cu, 2, 300, FAKE(8), fws), INVALID);
    expect("fwd varlen max_seqlen > T", fwd(FAKE(1), 1, 300, 4, 2, 128, 128, cu, 2, 301, FAKE(8), fws), INVALID);
    expect("fwd misaligned workspace", fwd(FAKE(1), 2, 300, 4, 2, 128, 128, NULL, 0, 300, (char *)FAKE(8) + 16, fws),
           INVALID);
    expect("fwd prepare null P", wall_attn_fwd_prepare(FAKE(1), FAKE(2), FAKE(3), WALL_BF16, NULL, 2, 300, 4, 2, 128,
                                                       128, 0.088f, NULL, 0, FAKE(8), fws, NULL), INVALID);
    expect("fwd run null k", wall_attn_fwd_run(FAKE(1), NULL, FAKE(3), WALL_BF16, (const float *)FAKE(4), NULL, NULL,
                                               FAKE(5), NULL, 2, 300, 4, 2, 128, 128, 0.088f, 0, NULL, 0, 300,
                                               FAKE(8), fws, NULL), INVALID);

    /* backward */
    expect("bwd null dq", bwd(NULL, NULL, NULL, 128, bws), INVALID);
    expect("bwd G without dg_scalar", bwd(FAKE(8), (const float *)FAKE(14), NULL, 128, bws), INVALID);
    expect("bwd K=96", bwd(FAKE(8), NULL, NULL, 96, bws), UNSUP);
    expect("bwd short workspace", bwd(FAKE(8), NULL, NULL, 128, bws - 1), INVALID);

    /* decode cache, streaming append, decode */
    expect("cache t0 >= t1", wall_kv_cache_build(FAKE(1), WALL_BF16, (const float *)FAKE(2), FAKE(3),
                                                 (float *)FAKE(4), 2, 300, 4, 2, 128, 64, 10, 10, NULL), INVALID);
    expect("cache chunk 32", wall_kv_cache_build(FAKE(1), WALL_BF16, (const float *)FAKE(2), FAKE(3),
                                                 (float *)FAKE(4), 2, 300, 4, 2, 128, 32, 0, 10, NULL), UNSUP);
    expect("append t1 > T_cap", wall_stream_append(FAKE(1), WALL_BF16, FAKE(2), WALL_BF16, (float *)FAKE(3),
                                                   FAKE(4), (float *)FAKE(5), 2, 300, 4, 2, 128, 64, 299, 301,
                                                   1.f, NULL), INVALID);
    expect("decode T > T_cap", decode(2, 301, 300, 4, 128, 64, dws, 0), INVALID);
    expect("decode short workspace", decode(2, 300, 300, 4, 128, 64, dws - 1, 0), INVALID);
    expect("decode K=96", decode(2, 300, 300, 4, 96, 64, dws, 0), UNSUP);
    expect("decode without allocation B*HQ > 65535", decode(8192, 64, 64, 16, 128, 64, 0, 1), INVALID);
    expect("decode without allocation past its scratch", decode(512, 64, 64, 16, 128, 64, 0, 1), WALL_ERR_SCRATCH);

    if (failures) {
        fprintf(stderr, "%d mismatches\n", failures);
        return 1;
    }
    printf("all statuses as declared\n");
    return 0;
}

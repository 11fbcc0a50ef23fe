/*
 * Host-side argument validation of libgdn2's C ABI, run under AddressSanitizer
 * and UndefinedBehaviorSanitizer (built host-only: no kernel is ever
 * launched). Every call here must be refused before anything is enqueued, so
 * device pointers are stand-in addresses that are never dereferenced. Exits
 * non-zero on the first status that differs from the one expected.
 */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/gdn2.h"

static int fails = 0;

#define EXPECT(call, want)                                                                  \
    do {                                                                                    \
        const int got_ = (call);                                                            \
        if (got_ != (want)) {                                                               \
            fprintf(stderr, "line %d: %s -> %d, expected %d\n", __LINE__, #call, got_, want); \
            ++fails;                                                                        \
        }                                                                                   \
    } while (0)

int main(void)
{
    /* stand-in device addresses: 16-byte aligned, one misaligned */
    void *A = (void *)(uintptr_t)0x100000, *M = (void *)(uintptr_t)0x100004;
    float *F = (float *)A;
    const int32_t *CU = (const int32_t *)A;
    const int BF = GDN2_BF16, F32 = GDN2_F32;

    for (int s = -3; s <= 8; ++s) {
        const char *msg = gdn2_status_string(s);
        if (!msg || !strlen(msg)) { fprintf(stderr, "empty status string %d\n", s); ++fails; }
    }
    EXPECT(gdn2_set_stream(NULL), GDN2_OK);
    if (gdn2_get_stream() != NULL) { fprintf(stderr, "stream not reset\n"); ++fails; }

    /* workspace sizes: valid sizes are positive, invalid ones 0 */
    if (gdn2_chunk_fwd_workspace_bytes(1, 65536, 1, 16, 128, 128, BF, 0) == 0) ++fails;
    if (gdn2_chunk_fwd_workspace_bytes(1, 0, 1, 16, 128, 128, BF, 0) == 0) ++fails;
    const int bad_dims[][8] = {
        {0, 64, 1, 1, 128, 128, 1, 0}, {1, -1, 1, 1, 128, 128, 1, 0}, {1, 64, 0, 1, 128, 128, 1, 0},
        {1, 64, 1, 0, 128, 128, 1, 0}, {1, 64, 1, 1, 0, 128, 1, 0},   {1, 64, 1, 1, 128, -5, 1, 0},
        {2, 64, 1, 1, 128, 128, 1, 0}, {2, 64, 3, 1, 128, 128, 1, 1}, {1, 64, 1, 1, 96, 128, 1, 0},
        {1, 64, 1, 1, 128, 256, 1, 0}, {1, 64, 1, 1, 16, 16, 1, 0},   {1, 64, 1, 70000, 128, 128, 1, 0},
        {1, INT_MAX, 1, 16, 128, 128, 1, 0}, {INT_MAX, INT_MAX, INT_MAX, 16, 128, 128, 1, 0},
        {1, 64, 1, 1, 128, 128, 7, 0}};
    for (size_t i = 0; i < sizeof bad_dims / sizeof bad_dims[0]; ++i) {
        const int *d = bad_dims[i];
        const size_t ws = gdn2_chunk_fwd_workspace_bytes(d[0], d[1], d[2], d[3], d[4], d[5], d[6], d[7]);
        if (ws != 0) { fprintf(stderr, "bad dims %zu accepted (%zu bytes)\n", i, ws); ++fails; }
        if (gdn2_chunk_bwd_workspace_bytes(d[0], d[1], d[2], d[3], d[4], d[5], d[6], d[7]) != 0) {
            fprintf(stderr, "bad dims %zu accepted by the backward\n", i);
            ++fails;
        }
    }
    for (int chunk = -64; chunk <= 256; chunk += 32) {
        const size_t ws = gdn2_chunk_fwd_sized_workspace_bytes(1, 1000, 1, 4, 64, 64, BF, 0, chunk);
        const int ok = chunk == 32 || chunk == 64 || chunk == 128;
        if ((ws != 0) != ok) { fprintf(stderr, "chunk %d: workspace %zu\n", chunk, ws); ++fails; }
    }
    /* fp32 inputs, dk = 128, 128-token chunks: valid but not built */
    if (gdn2_chunk_fwd_sized_workspace_bytes(1, 1000, 1, 4, 128, 128, F32, 0, 128) != 0) ++fails;

    /* prefill forward */
    const size_t need = gdn2_chunk_fwd_workspace_bytes(2, 100, 2, 4, 64, 64, BF, 0);
    EXPECT(gdn2_chunk_fwd(NULL, A, A, F, A, A, NULL, A, NULL, NULL, 2, 100, 2, 4, 64, 64, BF, F32, A, need),
           GDN2_ERR_INVALID);
    EXPECT(gdn2_chunk_fwd(A, A, A, F, A, A, NULL, NULL, NULL, NULL, 2, 100, 2, 4, 64, 64, BF, F32, A, need),
           GDN2_ERR_INVALID);
    EXPECT(gdn2_chunk_fwd(A, M, A, F, A, A, NULL, A, NULL, NULL, 2, 100, 2, 4, 64, 64, BF, F32, A, need),
           GDN2_ERR_INVALID);
    EXPECT(gdn2_chunk_fwd(A, A, A, F, A, A, (float *)M, A, NULL, NULL, 2, 100, 2, 4, 64, 64, BF, F32, A, need),
           GDN2_ERR_INVALID);
    EXPECT(gdn2_chunk_fwd(A, A, A, F, A, A, NULL, A, NULL, NULL, 2, 100, 2, 4, 64, 64, BF, F32, NULL, need),
           GDN2_ERR_WORKSPACE);
    EXPECT(gdn2_chunk_fwd(A, A, A, F, A, A, NULL, A, NULL, NULL, 2, 100, 2, 4, 64, 64, BF, F32, A, need - 1),
           GDN2_ERR_WORKSPACE);
    EXPECT(gdn2_chunk_fwd(A, A, A, F, A, A, NULL, A, NULL, NULL, 2, 100, 2, 4, 64, 64, BF, BF, A, need),
           GDN2_ERR_UNSUPPORTED);
    EXPECT(gdn2_chunk_fwd(A, A, A, F, A, A, NULL, A, NULL, NULL, 2, 100, 2, 4, 64, 64, BF, 9, A,
                          need),
           GDN2_ERR_INVALID);
    EXPECT(gdn2_chunk_fwd(A, A, A, F, A, A, NULL, A, NULL, NULL, 2, 100, 3, 4, 64, 64, BF, F32, A, need),
           GDN2_ERR_INVALID);
    EXPECT(gdn2_chunk_fwd(A, A, A, F, A, A, NULL, A, NULL, CU, 2, 100, 2, 4, 64, 64, BF, F32, A, need),
           GDN2_ERR_INVALID);
    EXPECT(gdn2_chunk_fwd(A, A, A, F, A, A, NULL, A, NULL, (const int32_t *)M, 1, 100, 2, 4, 64, 64, BF, F32, A,
                          1u << 30),
           GDN2_ERR_INVALID);
    EXPECT(gdn2_chunk_fwd(A, A, A, F, A, A, NULL, A, NULL, NULL, 2, 100, 2, 4, 48, 64, BF, F32, A, need),
           GDN2_ERR_UNSUPPORTED);
    EXPECT(gdn2_chunk_fwd_gates(A, A, A, F, A, A, 8, NULL, A, NULL, NULL, 2, 100, 2, 4, 64, 64, BF, F32, A, need),
           GDN2_ERR_INVALID);
    EXPECT(gdn2_chunk_fwd_sized(A, A, A, F, A, A, NULL, A, NULL, NULL, 2, 100, 2, 4, 64, 64, BF, F32, 48, A, need),
           GDN2_ERR_INVALID);

    /* fused prologue: taps required, history all-or-none */
    gdn2_short_conv conv;
    memset(&conv, 0, sizeof conv);
    EXPECT(gdn2_chunk_fwd_prologue(A, A, A, F, A, A, NULL, NULL, A, NULL, NULL, 2, 100, 2, 4, 64, 64, BF, F32, A,
                                   need),
           GDN2_ERR_INVALID);
    EXPECT(gdn2_chunk_fwd_prologue(A, A, A, F, A, A, &conv, NULL, A, NULL, NULL, 2, 100, 2, 4, 64, 64, BF, F32, A,
                                   need),
           GDN2_ERR_INVALID);
    conv.weight_q = conv.weight_k = conv.weight_v = F;
    conv.state_in_q = A;
    EXPECT(gdn2_chunk_fwd_prologue(A, A, A, F, A, A, &conv, NULL, A, NULL, NULL, 2, 100, 2, 4, 64, 64, BF, F32, A,
                                   need),
           GDN2_ERR_INVALID);
    conv.state_in_k = conv.state_in_v = A;
    conv.bias_k = (const float *)M;
    EXPECT(gdn2_chunk_fwd_prologue(A, A, A, F, A, A, &conv, NULL, A, NULL, NULL, 2, 100, 2, 4, 64, 64, BF, F32, A,
                                   need),
           GDN2_ERR_INVALID);
    conv.bias_k = NULL;
    EXPECT(gdn2_chunk_fwd_prologue(A, A, A, F, A, A, &conv, NULL, A, NULL, NULL, 2, 100, 2, 4, 64, 64, BF, F32, A,
                                   need - 1),
           GDN2_ERR_WORKSPACE);

    /* decode */
    EXPECT(gdn2_decode_step(A, A, A, F, A, A, NULL, A, 4, 2, 64, 64, BF, F32), GDN2_ERR_INVALID);
    EXPECT(gdn2_decode_step(A, A, A, F, A, M, F, A, 4, 2, 64, 64, BF, F32), GDN2_ERR_INVALID);
    EXPECT(gdn2_decode_step(A, A, A, F, A, A, F, A, 0, 2, 64, 64, BF, F32), GDN2_ERR_INVALID);
    EXPECT(gdn2_decode_step(A, A, A, F, A, A, F, A, 4, 2, 64, 80, BF, F32), GDN2_ERR_UNSUPPORTED);
    EXPECT(gdn2_decode_step(A, A, A, F, A, A, F, A, 4, 2, 64, 64, BF, BF), GDN2_ERR_UNSUPPORTED);
    EXPECT(gdn2_decode_step(A, A, A, F, A, A, F, A, INT_MAX, INT_MAX, 64, 64, BF, F32), GDN2_ERR_UNSUPPORTED);
    EXPECT(gdn2_decode_step_gates(A, A, A, F, A, A, 16, F, A, 4, 2, 64, 64, BF, F32), GDN2_ERR_INVALID);
    EXPECT(gdn2_decode_step_prologue(A, A, A, F, A, A, NULL, F, A, 4, 2, 64, 64, BF, F32), GDN2_ERR_INVALID);

    /* backward */
    const size_t bneed = gdn2_chunk_bwd_workspace_bytes(2, 100, 2, 4, 64, 64, BF, 0);
    if (bneed == 0) ++fails;
    EXPECT(gdn2_chunk_bwd(A, A, A, F, A, A, NULL, F, NULL, NULL, 2, 100, 2, 4, 64, 64, BF, F, F, F, F, F, NULL,
                          NULL, A, bneed),
           GDN2_ERR_INVALID);
    EXPECT(gdn2_chunk_bwd(A, A, A, F, A, A, NULL, F, NULL, NULL, 2, 100, 2, 4, 64, 64, BF, F, F, F, F, F, F, NULL,
                          A, bneed - 1),
           GDN2_ERR_WORKSPACE);
    EXPECT(gdn2_chunk_bwd(A, A, A, F, A, A, NULL, (const float *)M, NULL, NULL, 2, 100, 2, 4, 64, 64, BF, F, F, F,
                          F, F, F, NULL, A, bneed),
           GDN2_ERR_INVALID);

    /* profiling: bounds of the call count, no kernel recorded */
    EXPECT(gdn2_profile_begin(0), GDN2_ERR_INVALID);
    EXPECT(gdn2_profile_begin(4097), GDN2_ERR_INVALID);
    EXPECT(gdn2_profile_end(), 0);
    const char *name = NULL;
    int launches = -1;
    double ms = -1.0;
    EXPECT(gdn2_profile_kernel(0, &name, &launches, &ms), GDN2_ERR_INVALID);
    EXPECT(gdn2_profile_kernel(-1, &name, &launches, &ms), GDN2_ERR_INVALID);

    if (fails) fprintf(stderr, "%d validation expectations failed\n", fails);
    else printf("abi validation: all expectations met\n");
    return fails ? 1 : 0;
}

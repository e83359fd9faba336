/* Drives libkda's host layer through its C ABI with arguments that every
 * entry point must reject on the host (no kernel is ever launched: there need
 * be no GPU), plus the size queries at their limits.  Built against a copy of
 * the library whose host code carries AddressSanitizer and
 * UndefinedBehaviorSanitizer; exits non-zero if a call returns an unexpected
 * status.  Pointers are fake device addresses that are never dereferenced. */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kda.h"

static int failures = 0;

static void expect(const char *what, kda_status got, kda_status want) {
    if (got != want) {
        printf("FAIL %s: %s (%s), expected %s\n", what, kda_status_string(got), kda_last_error(),
               kda_status_string(want));
        ++failures;
    } else if (got != KDA_OK && kda_last_error()[0] == '\0') {
        printf("FAIL %s: no detail string\n", what);
        ++failures;
    }
}

#define P(i) ((void *)(((uintptr_t)1 << 40) + ((uintptr_t)(i) << 36)))
#define PF(i) ((float *)P(i))
#define PI(i) ((int *)P(i))

int main(void) {
    const kda_dtype F = KDA_F32, BF = KDA_BF16;
    /* status strings and the error slot */
    for (int s = 0; s <= 9; ++s)
        if (!kda_status_string((kda_status)s)) ++failures;
    if (kda_abi_version() != KDA_ABI_VERSION) ++failures;
    (void)kda_last_error();

    /* size queries, including arguments they must reject (return 0) */
    const int dims[][5] = {{1, 64, 2, 32, 0},        {1, 4096, 32, 128, 1}, {1, 1048576, 32, 128, 1},
                           {8, 32768, 32, 128, 1},   {0, 64, 2, 32, 0},     {1, INT_MAX, 1, 128, 1},
                           {INT_MAX, INT_MAX, INT_MAX, 128, 1}, {1, 16, 1, 48, 0}, {1, -5, 2, 32, 0}};
    for (size_t i = 0; i < sizeof dims / sizeof dims[0]; ++i) {
        const int B = dims[i][0], T = dims[i][1], H = dims[i][2], d = dims[i][3];
        const kda_dtype dt = dims[i][4] ? BF : F;
        size_t a = kda_chunk_prefill_workspace_bytes(B, T, H, d, d, dt);
        size_t b = kda_chunk_prefill_paged_workspace_bytes(B, T, H, d, d, dt);
        size_t c = kda_chunk_backward_workspace_bytes(B, T, H, d, d, dt);
        size_t e = kda_chunk_prefill_segmented_workspace_bytes(B, T, H, d, d, 8, dt);
        int r = kda_chunk_prefill_segments(B, T, H, d, d, dt);
        printf("sizes %d %d %d %d: %zu %zu %zu %zu %d\n", B, T, H, d, a, b, c, e, r);
    }

    /* prefill */
    expect("prefill q NULL",
           kda_chunk_prefill(NULL, P(1), P(2), P(3), PF(4), PF(5), -5.f, NULL, P(7), PF(8), 1, 64,
                             2, 32, 32, F, P(9), (size_t)1 << 33, NULL),
           KDA_ERR_NULL_POINTER);
    expect("prefill shape",
           kda_chunk_prefill(P(0), P(1), P(2), P(3), PF(4), PF(5), -5.f, NULL, P(7), PF(8), 1, 0,
                             2, 32, 32, F, P(9), (size_t)1 << 33, NULL),
           KDA_ERR_INVALID_SHAPE);
    expect("prefill huge",
           kda_chunk_prefill(P(0), P(1), P(2), P(3), PF(4), PF(5), -5.f, NULL, P(7), PF(8),
                             INT_MAX, INT_MAX, INT_MAX, 32, 32, F, P(9), (size_t)1 << 33, NULL),
           KDA_ERR_INVALID_SHAPE);
    expect("prefill g_min",
           kda_chunk_prefill(P(0), P(1), P(2), P(3), PF(4), PF(5), -7.f, NULL, P(7), PF(8), 1, 64,
                             2, 32, 32, F, P(9), (size_t)1 << 33, NULL),
           KDA_ERR_INVALID_VALUE);
    expect("prefill head size",
           kda_chunk_prefill(P(0), P(1), P(2), P(3), PF(4), PF(5), -5.f, NULL, P(7), PF(8), 1, 64,
                             2, 64, 64, F, P(9), (size_t)1 << 33, NULL),
           KDA_ERR_UNSUPPORTED);
    expect("prefill misaligned",
           kda_chunk_prefill((char *)P(0) + 4, P(1), P(2), P(3), PF(4), PF(5), -5.f, NULL, P(7),
                             PF(8), 1, 64, 2, 32, 32, F, P(9), (size_t)1 << 33, NULL),
           KDA_ERR_MISALIGNED);
    expect("prefill aliasing",
           kda_chunk_prefill(P(0), P(1), P(2), P(3), PF(4), PF(5), -5.f, NULL, P(0), PF(8), 1, 64,
                             2, 32, 32, F, P(9), (size_t)1 << 33, NULL),
           KDA_ERR_ALIASING);
    expect("prefill workspace",
           kda_chunk_prefill(P(0), P(1), P(2), P(3), PF(4), PF(5), -5.f, NULL, P(7), PF(8), 1,
                             4096, 32, 128, 128, BF, P(9), 16, NULL),
           KDA_ERR_WORKSPACE_TOO_SMALL);
    expect("prefill noalloc beyond the scratch",
           kda_chunk_prefill_noalloc(P(0), P(1), P(2), P(3), PF(4), PF(5), -5.f, NULL, P(7), PF(8),
                                     1, 16384, 32, 128, 128, BF, NULL),
           KDA_ERR_WORKSPACE_TOO_SMALL);
    expect("prefill noalloc NULL",
           kda_chunk_prefill_noalloc(P(0), NULL, P(2), P(3), PF(4), PF(5), -5.f, NULL, P(7), PF(8),
                                     1, 64, 2, 32, 32, F, NULL),
           KDA_ERR_NULL_POINTER);
    expect("segmented divisor",
           kda_chunk_prefill_segmented(P(0), P(1), P(2), P(3), PF(4), PF(5), -5.f, NULL, P(7),
                                       PF(8), 1, 100, 2, 32, 32, 7, F, P(9), (size_t)1 << 33, NULL),
           KDA_ERR_INVALID_SHAPE);
    expect("segmented workspace",
           kda_chunk_prefill_segmented(P(0), P(1), P(2), P(3), PF(4), PF(5), -5.f, NULL, P(7),
                                       PF(8), 1, 96, 2, 32, 32, 4, F, P(9), 8, NULL),
           KDA_ERR_WORKSPACE_TOO_SMALL);
    /* decode, verify */
    expect("decode S NULL",
           kda_decode_step(P(0), P(1), P(2), P(3), PF(4), PF(5), -5.f, NULL, P(7), 4, 2, 128, 128,
                           BF, NULL),
           KDA_ERR_NULL_POINTER);
    expect("decode aliasing",
           kda_decode_step(P(0), P(1), P(2), P(3), PF(4), PF(5), -5.f, PF(6), P(6), 4, 2, 128, 128,
                           BF, NULL),
           KDA_ERR_ALIASING);
    expect("tokens T",
           kda_decode_tokens(P(0), P(1), P(2), P(3), PF(4), PF(5), -5.f, PF(6), PF(7), P(8), 4,
                             KDA_MAX_DECODE_TOKENS + 1, 2, 32, 32, F, NULL),
           KDA_ERR_INVALID_SHAPE);
    expect("tokens partial overlap",
           kda_decode_tokens(P(0), P(1), P(2), P(3), PF(4), PF(5), -5.f, PF(6),
                             (float *)((char *)P(6) + 64), P(8), 4, 3, 2, 32, 32, F, NULL),
           KDA_ERR_ALIASING);
    /* paged */
    expect("paged prefill n_slots",
           kda_chunk_prefill_paged(P(0), P(1), P(2), P(3), PF(4), PF(5), -5.f, PF(6), 0, PI(7),
                                   PI(7), P(8), 1, 64, 2, 32, 32, F, P(9), (size_t)1 << 33, NULL),
           KDA_ERR_INVALID_SHAPE);
    expect("paged prefill workspace",
           kda_chunk_prefill_paged(P(0), P(1), P(2), P(3), PF(4), PF(5), -5.f, PF(6), 4, PI(7),
                                   PI(7), P(8), 1, 65536, 32, 128, 128, BF, P(9), 1024, NULL),
           KDA_ERR_WORKSPACE_TOO_SMALL);
    expect("paged decode table",
           kda_decode_step_paged(P(0), P(1), P(2), P(3), PF(4), PF(5), -5.f, PF(6), 4, NULL, P(8),
                                 2, 2, 32, 32, F, NULL),
           KDA_ERR_NULL_POINTER);
    expect("paged tokens pool overlaps o",
           kda_decode_tokens_paged(P(0), P(1), P(2), P(3), PF(4), PF(5), -5.f, PF(6), 4, PI(7),
                                   PI(7), P(6), 2, 3, 2, 32, 32, F, NULL),
           KDA_ERR_ALIASING);
    /* backward */
    expect("backward dO NULL",
           kda_chunk_backward(P(0), P(1), P(2), P(3), PF(4), PF(5), -5.f, NULL, NULL, NULL, P(9),
                              P(10), P(11), P(12), PF(13), PF(14), NULL, 1, 64, 2, 32, 32, F,
                              P(16), (size_t)1 << 33, NULL),
           KDA_ERR_NULL_POINTER);
    expect("backward workspace",
           kda_chunk_backward(P(0), P(1), P(2), P(3), PF(4), PF(5), -5.f, NULL, P(7), NULL, P(9),
                              P(10), P(11), P(12), PF(13), PF(14), NULL, 1, 64, 2, 32, 32, F,
                              P(16), 0, NULL),
           KDA_ERR_WORKSPACE_TOO_SMALL);
    expect("backward aliasing",
           kda_chunk_backward(P(0), P(1), P(2), P(3), PF(4), PF(5), -5.f, NULL, P(7), NULL, P(0),
                              P(10), P(11), P(12), PF(13), PF(14), NULL, 1, 64, 2, 32, 32, F,
                              P(16), (size_t)1 << 33, NULL),
           KDA_ERR_ALIASING);
    /* diagnostics */
    expect("gate aliasing",
           kda_gate_chunk_cumsum(P(0), PF(1), -5.f, PF(0), 1, 16, 1, 32, F, NULL), KDA_ERR_ALIASING);
    expect("intra g_min",
           kda_intra_chunk(P(0), P(1), P(2), PF(3), PF(4), -6.f, PF(5), PF(6), PF(7), 1, 16, 1, 32,
                           F, NULL),
           KDA_ERR_INVALID_VALUE);
    expect("dtype", kda_gate_chunk_cumsum(P(0), PF(1), -5.f, PF(2), 1, 16, 1, 32, (kda_dtype)9,
                                          NULL),
           KDA_ERR_UNSUPPORTED);
    printf("%s (%d failures)\n", failures ? "FAILED" : "OK", failures);
    return failures ? 1 : 0;
}

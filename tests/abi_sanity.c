/*
 * abi_sanity.c -- host-only checks of the C ABI, built and run under
 * AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py
 * (linked against a copy of the library whose host code is instrumented).
 * Every call below fails argument validation, so nothing is launched and no
 * GPU is needed; the sanitizers watch the validation, sizing and plan code.
 * Exits 0 when every status matches the documented one.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "la.h"

static int failures = 0;

#define EXPECT(call, want)                                                                     \
    do {                                                                                       \
        int got_ = (int)(call);                                                                \
        if (got_ != (int)(want)) {                                                             \
            fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, \
                    got_, (int)(want));                                                        \
            ++failures;                                                                        \
        }                                                                                      \
    } while (0)

/* 16-byte aligned addresses that are never dereferenced */
#define P(i) ((void *)(uintptr_t)((1ull << 32) + ((uint64_t)(i) << 24)))

int main(void) {
    const int64_t shapes[][5] = {{1, 1, 1, 32, 32},      {1, 8, 65536, 64, 64}, {16, 8, 784, 32, 32},
                                 {256, 8, 1, 64, 64},    {3, 5, 4097, 64, 32},  {1, 1, 1 << 20, 32, 32},
                                 {64, 16, 512, 32, 64},  {1, 2, 40000, 64, 64}};
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) {
        const int64_t *s = shapes[i];
        for (int op = 0; op <= 5; ++op)
            for (int dt = 0; dt <= 1; ++dt) {
                size_t n = la_workspace_size((la_op_t)op, s[0], s[1], s[2], s[3], s[4], (la_dtype_t)dt);
                if (n == 0 || n % 256 != 0) {
                    fprintf(stderr, "workspace size %zu for op %d shape %zu\n", n, op, i);
                    ++failures;
                }
            }
    }
    EXPECT(la_workspace_size(LA_OP_FWD_CAUSAL, 0, 1, 1, 32, 32, LA_DTYPE_F32), 0);
    EXPECT(la_workspace_size((la_op_t)9, 1, 1, 1, 32, 32, LA_DTYPE_F32), 0);
    EXPECT(la_workspace_size(LA_OP_FWD_CAUSAL, 1, 1, 1, 40, 32, LA_DTYPE_F32), 0);
    EXPECT(la_workspace_size(LA_OP_BWD_CAUSAL, 1, 1, 1, 40, 32, LA_DTYPE_F32), 0);
    if (la_workspace_size(LA_OP_BWD_CAUSAL, 1, 1, 100, 48, 32, LA_DTYPE_F32) == 0) ++failures;
    EXPECT(la_workspace_size(LA_OP_FWD_CAUSAL_POLY2, 1, 1, 1, 48, 32, LA_DTYPE_F32), 0);
    if (la_workspace_size(LA_OP_FWD_CAUSAL, 1, 1, 100, 48, 128, LA_DTYPE_F32) == 0) ++failures;
    EXPECT(la_workspace_size(LA_OP_FWD_CAUSAL, INT64_MAX, INT64_MAX, INT64_MAX, 32, 32, LA_DTYPE_F32), 0);

    /* forwards */
    EXPECT(la_forward_causal(NULL, P(1), P(2), P(3), 1, 1, 8, 32, 32, LA_DTYPE_F32, P(4), 1 << 20, 0),
           LA_ERR_INVALID_ARGUMENT);
    EXPECT(la_forward_causal(P(0), P(1), P(2), P(3), 1, 1, 0, 32, 32, LA_DTYPE_F32, P(4), 1 << 20, 0),
           LA_ERR_INVALID_ARGUMENT);
    EXPECT(la_forward_causal(P(0), P(1), P(2), P(3), 1, 1, 8, 40, 32, LA_DTYPE_F32, P(4), 1 << 20, 0),
           LA_ERR_UNSUPPORTED);
    EXPECT(la_forward_causal(P(0), P(1), P(2), P(3), 1, 1, 8, 32, 144, LA_DTYPE_F32, P(4), 1 << 20, 0),
           LA_ERR_UNSUPPORTED);
    EXPECT(la_forward_causal(P(0), P(1), P(2), P(3), 1, 1, 8, 32, 32, (la_dtype_t)7, P(4), 1 << 20, 0),
           LA_ERR_UNSUPPORTED);
    EXPECT(la_forward_causal(P(0), P(1), P(2), P(0), 1, 1, 8, 32, 32, LA_DTYPE_F32, P(4), 1 << 20, 0),
           LA_ERR_INVALID_ARGUMENT);
    EXPECT(la_forward_causal(P(0), P(1), P(2), P(3), 1, 1, 8, 32, 32, LA_DTYPE_F32, P(4), 16, 0),
           LA_ERR_WORKSPACE);
    EXPECT(la_forward_noncausal(P(0), P(1), P(2), P(3), 1, 1, 8, 32, 32, LA_DTYPE_BF16, NULL, 1 << 20, 0),
           LA_ERR_WORKSPACE);
    EXPECT(la_forward_causal_features(P(0), P(1), P(2), (char *)P(3) + 8, 1, 1, 8, 32, 32, LA_DTYPE_F32, P(4),
                                      1 << 20, 0),
           LA_ERR_INVALID_ARGUMENT);
    EXPECT(la_forward_causal_state(P(0), P(1), P(2), P(3), (const float *)P(4), NULL, NULL, NULL, 1, 1, 8, 32, 32,
                                   LA_DTYPE_F32, P(8), 1 << 20, 0),
           LA_ERR_INVALID_ARGUMENT);
    EXPECT(la_forward_causal_state(P(0), P(1), P(2), P(3), NULL, NULL, (float *)P(0), (float *)P(5), 1, 1, 8, 32,
                                   32, LA_DTYPE_F32, P(8), 1 << 20, 0),
           LA_ERR_INVALID_ARGUMENT);
    EXPECT(la_forward_causal_poly2(P(0), P(1), P(2), P(3), 1, 1, 8, 48, 32, LA_DTYPE_BF16, P(4), 1 << 20, 0),
           LA_ERR_UNSUPPORTED);
    EXPECT(la_forward_noncausal_poly2(P(0), P(1), P(2), P(3), 1, 1, 8, 32, 32, LA_DTYPE_BF16, P(4), 16, 0),
           LA_ERR_WORKSPACE);
    EXPECT(la_forward_causal_poly2_state(P(0), P(1), P(2), P(3), NULL, 1, 1, 8, 32, 32, LA_DTYPE_BF16, P(4),
                                         1 << 20, 0),
           LA_ERR_INVALID_ARGUMENT);
    EXPECT(la_decode_step_poly2(P(0), P(1), P(2), (float *)P(3), P(3), 2, 2, 32, 32, LA_DTYPE_BF16, 0),
           LA_ERR_INVALID_ARGUMENT);
    EXPECT(la_decode_step_poly2(P(0), P(1), P(2), (float *)P(3), P(4), 2, 2, 48, 32, LA_DTYPE_BF16, 0),
           LA_ERR_UNSUPPORTED);
    EXPECT(la_poly2_state_floats(32, 32), (33 * 2 + 4) * 256);
    EXPECT(la_poly2_state_floats(40, 32), 0);
    EXPECT(la_rff_features(P(0), (const float *)P(1), (const float *)P(2), P(0), 1, 1, 8, 32, 32, LA_DTYPE_F32, 0),
           LA_ERR_INVALID_ARGUMENT);

    /* backwards and decode */
    EXPECT(la_backward_causal(P(0), P(1), P(2), P(3), P(4), P(5), P(4), 1, 1, 8, 32, 32, LA_DTYPE_F32, P(8),
                              1 << 20, 0),
           LA_ERR_INVALID_ARGUMENT);
    EXPECT(la_backward_noncausal(P(0), P(1), P(2), P(3), P(4), P(5), P(6), 1, 1, 8, 32, 32, LA_DTYPE_F32, P(8), 64,
                                 0),
           LA_ERR_WORKSPACE);
    EXPECT(la_decode_step(P(0), P(1), P(2), (float *)P(3), (float *)P(3), P(5), 2, 2, 32, 32, LA_DTYPE_BF16, 0),
           LA_ERR_INVALID_ARGUMENT);
    EXPECT(la_decode_step(P(0), P(1), P(2), (float *)P(3), (float *)P(4), P(5), 2, 2, 32, 100, LA_DTYPE_BF16, 0),
           LA_ERR_UNSUPPORTED);

    /* the no-allocation forward: a workspace beyond its scratch (about 17 MB) */
    EXPECT(la_forward_causal_noalloc(P(0), P(64), P(128), P(192), 1, 255, 32768, 64, 64, LA_DTYPE_BF16, 0),
           LA_ERR_WORKSPACE);
    EXPECT(la_forward_causal_noalloc(P(0), P(1), P(2), P(0), 1, 1, 8, 32, 32, LA_DTYPE_F32, 0),
           LA_ERR_INVALID_ARGUMENT);

    /* diagnostics */
    EXPECT(la_workspace_check(NULL, 1 << 20, 0, 0), LA_ERR_WORKSPACE);
    EXPECT(la_workspace_check((char *)P(0) + 16, 1 << 20, 0, 0), LA_ERR_WORKSPACE);
    EXPECT(la_workspace_check(P(0), 255, 1, 0), LA_ERR_WORKSPACE);
    EXPECT(la_set_wait_limit(7), 1 << 20);
    EXPECT(la_set_wait_limit(-1), 7);
    for (int s = 0; s <= 6; ++s)
        if (strlen(la_status_string((la_status_t)s)) == 0) ++failures;
    EXPECT(la_abi_version(), LA_ABI_VERSION);

    printf(failures ? "abi sanity: %d FAILED\n" : "abi sanity: ok\n", failures);
    return failures ? 1 : 0;
}

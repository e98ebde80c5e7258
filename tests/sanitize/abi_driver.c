/*
 * Drives the host side of the library's C ABI -- argument validation, workspace sizing and
 * status strings -- for a host-only build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py builds and runs it; no GPU).  Every
 * call here is one that must return before touching the device: invalid arguments with
 * their expected status, and size queries over the extremes of every limit (the size
 * arithmetic must neither overflow nor read out of bounds).
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dspark.h"

static int failures = 0;
#define EXPECT(call, want)                                                               \
    do {                                                                                 \
        int got_ = (int)(call);                                                          \
        if (got_ != (want)) {                                                            \
            fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call,  \
                    got_, (int)(want));                                                  \
            ++failures;                                                                  \
        }                                                                                \
    } while (0)

int main(void) {
    void* P = (void*)(uintptr_t)256;   /* non-null, never dereferenced on these paths */
    const int32_t Bs[] = {1, 2, 31, 32, 33, 128, 129, 256, 257, 4096, 65535};
    const int32_t Gs[] = {1, 2, 5, 16, 64};
    const int32_t Vs[] = {2, 3, 1023, 4096, 151936, 262144, 1 << 28};
    const int32_t rs[] = {8, 16, 256, 1024};
    size_t acc = 0;
    for (unsigned a = 0; a < sizeof Bs / sizeof *Bs; ++a)
        for (unsigned g = 0; g < sizeof Gs / sizeof *Gs; ++g)
            for (unsigned v = 0; v < sizeof Vs / sizeof *Vs; ++v)
                for (unsigned q = 0; q < sizeof rs / sizeof *rs; ++q) {
                    dspark_dims d = {Bs[a], Gs[g], Vs[v], rs[q], 4096};
                    for (int op = -1; op <= 5; ++op) acc += dspark_workspace_bytes(op, &d);
                    acc += dspark_loop_workspace_bytes(&d);
                }
    dspark_dims bad[] = {{0, 4, 1024, 16, 64}, {4, 0, 1024, 16, 64}, {4, 65, 1024, 16, 64},
                         {4, 4, 1, 16, 64}, {4, 4, 1024, 12, 64}, {4, 4, 1024, 0, 64},
                         {65536, 4, 1024, 16, 64}, {4, 4, (1 << 28) + 1, 16, 64},
                         {4, 4, 1024, 16, -1}, {4, 4, 1024, 2048, 64}};
    for (unsigned i = 0; i < sizeof bad / sizeof *bad; ++i) {
        for (int op = 0; op <= 4; ++op) EXPECT(dspark_workspace_bytes(op, &bad[i]), 0);
        EXPECT(dspark_loop_workspace_bytes(&bad[i]), 0);
    }
    EXPECT(dspark_workspace_bytes(0, NULL), 0);
    EXPECT(dspark_loop_workspace_bytes(NULL), 0);
    const int32_t ns[] = {-1, 0, 1, 1000, 1 << 22, (1 << 22) + 1};
    for (unsigned i = 0; i < sizeof ns / sizeof *ns; ++i) {
        acc += dspark_sts_workspace_bytes(ns[i], 256, 15);
        acc += dspark_sts_workspace_bytes(ns[i], 65535, 256);
        acc += dspark_sts_workspace_bytes(ns[i], 0, 0);
        acc += dspark_loss_workspace_bytes(ns[i], 16, 151936);
        acc += dspark_loss_workspace_bytes(128, 64, ns[i]);
    }
    for (int s = -2; s <= 8; ++s) acc += strlen(dspark_status_string(s));
    acc += (size_t)dspark_version();

    dspark_dims d = {4, 4, 1024, 16, 64};
    /* draft */
    EXPECT(dspark_draft_markov(NULL, P, P, P, 0, P, NULL, 1.f, 1, P, P, P, P, 1 << 30, NULL),
           DSPARK_E_NULL);
    EXPECT(dspark_draft_markov(&bad[0], P, P, P, 0, P, NULL, 1.f, 1, P, P, P, P, 1 << 30, NULL),
           DSPARK_E_SHAPE);
    EXPECT(dspark_draft_markov(&d, P, P, P, 9, P, NULL, 1.f, 1, P, P, P, P, 1 << 30, NULL),
           DSPARK_E_DTYPE);
    EXPECT(dspark_draft_markov(&d, P, P, P, 0, P, NULL, -1.f, 1, P, P, P, P, 1 << 30, NULL),
           DSPARK_E_VALUE);
    EXPECT(dspark_draft_markov(&d, P, P, P, 0, P, NULL, 1.f, 1, P, P, P, P, 8, NULL),
           DSPARK_E_WORKSPACE);
    /* confidence */
    EXPECT(dspark_confidence(&d, NULL, 0, P, 0, P, 0, P, P, P, NULL), DSPARK_E_NULL);
    EXPECT(dspark_confidence(&bad[1], P, 0, P, 0, P, 0, P, P, P, NULL), DSPARK_E_SHAPE);
    EXPECT(dspark_confidence(&d, P, 5, P, 0, P, 0, P, P, P, NULL), DSPARK_E_DTYPE);
    EXPECT(dspark_confidence_calibrated(&d, P, 0, P, 0, P, 0, P, P, NULL, P, NULL),
           DSPARK_E_NULL);
    /* calibration */
    EXPECT(dspark_sts_calibrate(10, 4, NULL, P, P, 4, 15, P, P, P, 1 << 20, NULL),
           DSPARK_E_NULL);
    EXPECT(dspark_sts_calibrate(0, 4, P, P, P, 4, 15, P, P, P, 1 << 20, NULL), DSPARK_E_SHAPE);
    EXPECT(dspark_sts_calibrate(10, 4, P, P, P, 4, 0, P, P, P, 1 << 20, NULL), DSPARK_E_SHAPE);
    EXPECT(dspark_sts_calibrate(10, 4, P, P, P, 4, 15, P, P, P, 0, NULL), DSPARK_E_WORKSPACE);
    /* scheduler */
    EXPECT(dspark_schedule(4, 4, NULL, P, 0, P, P, P, NULL, 0, NULL), DSPARK_E_NULL);
    EXPECT(dspark_schedule(4097, 1, P, P, 0, P, P, P, NULL, 0, NULL), DSPARK_E_SHAPE);
    EXPECT(dspark_schedule(4, 4, P, P, DSPARK_SCHED_TOPK_DELAYED, P, P, P, NULL, 0, NULL),
           DSPARK_E_VALUE);
    EXPECT(dspark_schedule_topk(4, 4, P, P, -1, P, P, P, NULL, 0, NULL), DSPARK_E_VALUE);
    EXPECT(dspark_schedule_topk(0, 4, P, P, 1, P, P, P, NULL, 0, NULL), DSPARK_E_SHAPE);
    /* verify and TV */
    EXPECT(dspark_verify(&d, P, P, P, 0, P, P, P, P, NULL, P, 1.f, 1, P, P, NULL, P, 1 << 30,
                         NULL), DSPARK_E_NULL);
    EXPECT(dspark_verify(&bad[2], P, P, P, 0, P, P, P, P, P, P, 1.f, 1, P, P, NULL, P, 1 << 30,
                         NULL), DSPARK_E_SHAPE);
    EXPECT(dspark_verify(&d, P, P, P, 0, P, P, P, P, P, P, 0.f, 1, P, P, NULL, P, 1 << 30,
                         NULL), DSPARK_E_VALUE);
    EXPECT(dspark_verify(&d, P, P, P, 0, P, P, P, P, P, P, 1.f, 1, P, P, NULL, P, 1, NULL),
           DSPARK_E_WORKSPACE);
    EXPECT(dspark_accept_rate_tv(&d, P, P, P, 0, P, P, P, P, 1.f, NULL, P, 1 << 30, NULL),
           DSPARK_E_NULL);
    dspark_dims wide = {4096, 64, 1024, 16, 64};   /* B * gamma above the TV limit */
    EXPECT(dspark_accept_rate_tv(&wide, P, P, P, 0, P, P, P, P, 1.f, P, P, 1 << 30, NULL),
           DSPARK_E_SHAPE);
    /* loss */
    EXPECT(dspark_draft_loss(4, 4, 1024, NULL, P, P, P, 0.1, 0.9, 1.0, P, NULL, NULL, NULL, P,
                             1 << 30, NULL), DSPARK_E_NULL);
    EXPECT(dspark_draft_loss(4, 4, 0, P, P, P, P, 0.1, 0.9, 1.0, P, NULL, NULL, NULL, P,
                             1 << 30, NULL), DSPARK_E_SHAPE);
    EXPECT(dspark_draft_loss(4, 4, 1024, P, P, P, P, 0.0 / 0.0, 0.9, 1.0, P, NULL, NULL, NULL,
                             P, 1 << 30, NULL), DSPARK_E_VALUE);
    /* closed loop */
    dspark_dims many = {128, 64, 1024, 16, 64};   /* B * gamma above the scheduler's limit */
    EXPECT(dspark_closed_loop(&many, P, P, P, 0, P, 0, P, 0, P, P, 0, 1.f, 1, 0.5f, 2, 3, NULL,
                              P, P, P, NULL, P, P, P, NULL, P, (size_t)1 << 40, NULL),
           DSPARK_E_SHAPE);
    EXPECT(dspark_closed_loop(&d, P, P, P, 0, P, 0, P, 0, P, P, 3, 1.f, 1, 0.5f, 2, 3, NULL,
                              P, P, P, NULL, P, P, P, NULL, P, (size_t)1 << 40, NULL),
           DSPARK_E_VALUE);
    EXPECT(dspark_closed_loop(&d, P, P, P, 0, P, 0, P, 0, P, P, 0, 1.f, 1, 0.5f, 2, 0, NULL,
                              P, P, P, NULL, P, P, P, NULL, P, (size_t)1 << 40, NULL),
           DSPARK_E_SHAPE);
    /* hooks */
    EXPECT(dspark_rng_uniforms(1, 0, 1, 0, 0, 16, NULL, NULL), DSPARK_E_NULL);
    EXPECT(dspark_rng_uniforms(1, 0, 1, 0, 0, -1, P, NULL), DSPARK_E_SHAPE);
    EXPECT(dspark_gumbel_lattice(3, P, NULL), DSPARK_E_VALUE);
    EXPECT(dspark_profile_start(0), DSPARK_E_VALUE);
    EXPECT(dspark_profile_stop(NULL, NULL, NULL), DSPARK_E_NULL);
    double ms;
    EXPECT(dspark_stream_read_probe(P, 1 << 20, 17, 1, P, &ms, NULL), DSPARK_E_SHAPE);
    EXPECT(dspark_stream_read_probe(P, 1 << 20, 1 << 16, 0, P, &ms, NULL), DSPARK_E_VALUE);
    printf("abi driver: %d failures (size checksum %zu)\n", failures, acc);
    return failures ? 1 : 0;
}

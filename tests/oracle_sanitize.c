/*
 * oracle_sanitize.c -- runs every function of the CPU oracle (oracle/oracle.c, included below)
 * on small inputs that reach its edge cases, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitizers.py compiles and runs it with gcc).
 * The inputs are the failure modes "PR #39593: [Bug]: Fix FlashInfer CUTLASS BF16 + CUDA graphs
 * IMA" (Root cause) names: NaN logit rows, repeated expert ids in one token, and out-of-range ids;
 * plus empty experts, expert-parallel ranks with no local rows, k = E, all-zero and NaN
 * quantisation groups.  Each call's results are checked against simple invariants; the exit
 * status is the number of failed checks (the sanitizers abort on their own findings).
 * Test infrastructure only.
 */
#include "../oracle/oracle.c"

#include <stdio.h>

static int failures = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            failures++;                                                 \
        }                                                               \
    } while (0)

static uint16_t bf16_of(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static uint32_t lcg = 12345u;
static float frand(void) { /* uniform in [-1, 1) */
    lcg = lcg * 1664525u + 1013904223u;
    return (float)((lcg >> 8) & 0xffff) / 32768.0f - 1.0f;
}

int main(void) {
    enum { T = 9, H = 256, I = 128, E = 6, K = 3 };
    /* router: a NaN row, a row of equal values, k = E */
    float logits[T * E];
    for (int i = 0; i < T * E; i++) logits[i] = frand() * 4.0f;
    for (int e = 0; e < E; e++) logits[2 * E + e] = NAN;
    for (int e = 0; e < E; e++) logits[4 * E + e] = 0.5f;
    logits[7 * E + 1] = INFINITY;
    logits[7 * E + 2] = -INFINITY;
    int32_t ids[T * K];
    double w[T * K];
    for (int sc = 0; sc < 2; sc++)
        for (int rn = 0; rn < 2; rn++) {
            oracle_router_topk(logits, 0, T, E, K, sc, rn, ids, w);
            for (int t = 0; t < T; t++)
                for (int a = 0; a < K; a++)
                    for (int b = a + 1; b < K; b++) CHECK(ids[t * K + a] != ids[t * K + b]);
            CHECK(ids[2 * K] == 0 && ids[2 * K + 1] == 1 && ids[2 * K + 2] == 2);
        }
    int32_t all_ids[T * E];
    double all_w[T * E];
    oracle_router_topk(logits, 0, T, E, E, 0, 1, all_ids, all_w);
    int32_t gids[T * 2];
    double gw[T * 2];
    oracle_router_topk_grouped(logits, 0, T, E, 2, 3, 1, 0, 1, gids, gw);
    for (int t = 0; t < T; t++) CHECK(gids[t * 2] / 2 == gids[t * 2 + 1] / 2);

    /* router linear */
    uint16_t x[T * H], wr[E * H];
    for (int i = 0; i < T * H; i++) x[i] = bf16_of(frand());
    for (int i = 0; i < E * H; i++) wr[i] = bf16_of(frand() * 0.05f);
    float lg[T * E];
    oracle_router_logits(x, wr, T, H, E, lg);
    CHECK(oracle_rows_per_expert_estimate(288, 6, 400) == 5);

    /* grouping: repeated ids, out-of-range ids, two ranks (one with no local rows) */
    int32_t cid[T * K] = {1, 1, 1, -1, 6, 0, 2, 2, 5, 0, 0, 0, 7, -3, 1, 4, 4, 4, 5, 5, 5, 3, 1, 0, 2, 2, 2};
    int32_t counts[E], offsets[E + 1], perm[T * K], inv[T * K];
    long long dropped = 0;
    oracle_route_permute(T, K, E, 1, 0, cid, counts, offsets, perm, inv, &dropped);
    CHECK(dropped == 4);
    CHECK(offsets[E] == T * K - 4);
    for (int p = 0; p < offsets[E]; p++) CHECK(inv[perm[p]] == p);
    oracle_route_permute(T, K, E, 3, 1, cid, counts, offsets, perm, inv, &dropped);
    CHECK(offsets[2] == counts[0] + counts[1]);
    int32_t far[T * K];
    for (int i = 0; i < T * K; i++) far[i] = 5;
    oracle_route_permute(T, K, E, 3, 0, far, counts, offsets, perm, inv, &dropped);
    CHECK(offsets[2] == 0);

    /* quantisation: an all-zero group, a NaN value, a value beyond 448 */
    float qx[2 * 256];
    for (int i = 0; i < 512; i++) qx[i] = frand() * 1000.0f;
    for (int i = 128; i < 256; i++) qx[i] = 0.0f;
    qx[300] = NAN;
    uint8_t q[512];
    float s[4];
    oracle_act_quant(qx, 2, 256, q, s);
    CHECK(s[1] == 1.0f && q[130] == 0);
    CHECK(q[300] == 0x7E);
    for (int c = 0; c < 256; c++) CHECK(oracle_e4m3_encode(oracle_e4m3_decode((uint8_t)c)) == c || (c & 0x7F) == 0x7F);

    /* experts, bf16 and FP8, with the repeated and out-of-range ids, on both ranks */
    uint16_t wg[E * I * H], wu[E * I * H], wd[E * H * I];
    uint8_t qg[E * I * H], qu[E * I * H], qd[E * H * I];
    float sg[E * (I / 128) * (H / 128)], su[E * (I / 128) * (H / 128)], sd[E * (H / 128) * (I / 128)];
    for (int i = 0; i < E * I * H; i++) {
        wg[i] = bf16_of(frand() * 0.05f);
        wu[i] = bf16_of(frand() * 0.05f);
        wd[i] = bf16_of(frand() * 0.05f);
        qg[i] = (uint8_t)(lcg >> 3) & 0x77;
        qu[i] = (uint8_t)(lcg >> 5) & 0x77;
        qd[i] = (uint8_t)(lcg >> 7) & 0x77;
        frand();
    }
    for (int i = 0; i < E * 2; i++) sg[i] = su[i] = sd[i] = 0.001f * (float)(i + 1);
    double cw[T * K];
    for (int i = 0; i < T * K; i++) cw[i] = 0.25;
    int32_t tok[T];
    for (int t = 0; t < T; t++) tok[t] = T - 1 - t;
    double out[T * H];
    oracle_moe_tokens(T, H, I, E, K, 1, 0, 0, x, cid, cw, wg, wu, wd, sg, su, sd, tok, T, out);
    for (int i = 0; i < T * H; i++) CHECK(isfinite(out[i]));
    oracle_moe_tokens(T, H, I, E, K, 3, 2, 1, x, cid, cw, qg, qu, qd, sg, su, sd, tok, T, out);
    for (int i = 0; i < T * H; i++) CHECK(isfinite(out[i]));
    oracle_moe_tokens(T, H, I, E, K, 3, 0, 0, x, far, cw, wg, wu, wd, sg, su, sd, tok, T, out);
    for (int i = 0; i < T * H; i++) CHECK(out[i] == 0.0);

    /* grouped GEMM stages, both dtypes */
    double g0[T * K * I], g1[T * K * H];
    int R = oracle_grouped_gemm(0, T, K, E, 1, 0, I, H, 0, cid, x, NULL, 0, wg, wu, NULL, NULL, g0);
    CHECK(R == T * K - 4);
    uint8_t hq[T * K * I];
    float hs[T * K];
    for (int i = 0; i < T * K * I; i++) hq[i] = (uint8_t)(i * 37) & 0x77;
    for (int i = 0; i < T * K; i++) hs[i] = 0.5f;
    R = oracle_grouped_gemm(1, T, K, E, 3, 1, H, I, 1, cid, hq, hs, 1, qd, NULL, sd, NULL, g1);
    CHECK(R >= 0);
    oracle_set_num_threads(1);
    CHECK(oracle_num_threads() == 1);
    if (failures) fprintf(stderr, "%d checks failed\n", failures);
    else printf("oracle sanitizer run: all checks passed\n");
    return failures;
}

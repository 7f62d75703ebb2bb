/*
 * oracle.c -- plain, slow reference implementation of the fused mixture-of-experts
 * layer (router top-k -> per-expert grouping -> SwiGLU experts -> weighted combine).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * constant with the GPU library: everything here is written from the definitions.
 *
 * Arithmetic: IEEE double for every sum, product, exponential and division of the
 * layer, except where a floating-point value decides an integer or a stored code:
 *   - router logits of the tiny layer are an fp32 fused-multiply-add chain (they
 *     decide the expert ids, and fmaf is correctly rounded on both sides);
 *   - expert selection compares the fp32 logits themselves;
 *   - FP8 activation quantisation (scale, reciprocal, scaled value, e4m3 code) is
 *     fp32, the precision the layer stores its scales in.
 *
 * Sources (web pages; cited by title and section):
 *   [PR39593] "PR #39593: [Bug]: Fix FlashInfer CUTLASS BF16 + CUDA graphs IMA",
 *             sections Root cause, Fix, Test Plan (micro-benchmark).
 *   [H20]     "vLLM Community Traces H20 MoE Scheduling Inefficiency to Expert-Load
 *             Kernel Selection", paragraphs 2-3 (API, workload estimate).
 *   [LAB6]    "Lab notes #6: We tuned vLLM's MoE kernels on an H100 ...", intro
 *             (fp8_w8a8, block_shape [128,128], E=128, N=768).
 *   The workload definitions of the layer (SwiGLU experts, weights renormalised after
 *   softmax top-k, ties to the lower index) are stated where they are used.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -shared -fPIC oracle.c -o liboracle.so -lm
 */
#include <float.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_E4M3_MAX 448.0f /* largest finite OCP E4M3FN value, the clamp bound in [PR39593] Root cause */

/* ------------------------------------------------------------------ scalar formats */

/* bfloat16 is the top half of an IEEE binary32: widening is exact. */
float oracle_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* OCP E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
 * holds subnormals m * 2^-9; S.1111.111 is NaN; there are no infinities. */
float oracle_e4m3_decode(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return (float)(s ? -v : v);
}

/* Encode a finite fp32 value to the nearest E4M3FN value; an exact midpoint goes to the
 * code with an even mantissa; magnitudes above 448 saturate to 448.  Written as a plain
 * nearest-value search over the 127 finite non-negative codes (sorted by value). */
uint8_t oracle_e4m3_encode(float x) {
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs((double)x);
    if (a >= OR_E4M3_MAX) return sign | 0x7E;
    int lo = 0, hi = 0x7E; /* invariant: value(lo) <= a < value(hi) once narrowed */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if ((double)oracle_e4m3_decode((uint8_t)mid) <= a) lo = mid; else hi = mid;
    }
    double vlo = oracle_e4m3_decode((uint8_t)lo), vhi = oracle_e4m3_decode((uint8_t)hi);
    int code;
    if (a - vlo < vhi - a) code = lo;
    else if (a - vlo > vhi - a) code = hi;
    else code = (lo & 1) ? hi : lo; /* tie: even mantissa */
    return sign | (uint8_t)code;
}

/* ------------------------------------------------------------------ router */

/* Router linear of the tiny layer: logits[t,e] = sum_h x[t,h] * Wr[e,h], as an fp32
 * fused-multiply-add chain over ascending h starting from 0 (x, Wr are bf16). */
void oracle_router_logits(const uint16_t* x, const uint16_t* wr, int T, int H, int E, float* logits) {
    for (int t = 0; t < T; t++)
        for (int e = 0; e < E; e++) {
            float acc = 0.0f;
            for (int h = 0; h < H; h++)
                acc = fmaf(oracle_bf16_to_f32(x[(size_t)t * H + h]), oracle_bf16_to_f32(wr[(size_t)e * H + h]), acc);
            logits[(size_t)t * E + e] = acc;
        }
}

/* Sanitised logit ([PR39593] Fix: NaN becomes -FLT_MAX before scoring and selection).
 * Infinities are clamped to +-FLT_MAX so that differences stay finite; -0 compares
 * equal to +0 (it is a float comparison). */
static float sanitize(float v) {
    if (isnan(v)) return -FLT_MAX;
    if (v > FLT_MAX) return FLT_MAX;
    if (v < -FLT_MAX) return -FLT_MAX;
    return v;
}

/* Top-k router ([PR39593] Fix and Test Plan: K distinct expert ids per token, never a
 * repeated id, also for all-NaN rows).
 *   logits: [T,E], fp32 (is_bf16 = 0) or bf16 (is_bf16 = 1), row-major.
 *   scoring: 0 = softmax, 1 = sigmoid.  renorm: weights of the k picks divided by their sum.
 * Selection: indices ordered by sanitised logit, larger first, lower index first among
 * equal values; the first k are the ids, best first.  Softmax and sigmoid are strictly
 * increasing, so this is the order of the scores.
 * Weights (double):
 *   softmax: p_e = exp(v_e - m) / sum_{e'<E} exp(v_e' - m), m = max_e v_e; renormalised:
 *            w_j = exp(v_{id_j} - m) / sum_{j'<k} exp(v_{id_j'} - m).
 *   sigmoid: s_e = 1 / (1 + exp(-v_e)); renormalised w_j = s_j / sum s; when that sum is
 *            0 (all picks at -FLT_MAX), every weight is 1/k. */
void oracle_router_topk(const void* logits, int is_bf16, int T, int E, int k, int scoring, int renorm,
                        int32_t* ids, double* w) {
    float* v = (float*)malloc(sizeof(float) * (size_t)E);
    char* taken = (char*)malloc((size_t)E);
    for (int t = 0; t < T; t++) {
        for (int e = 0; e < E; e++) {
            float raw = is_bf16 ? oracle_bf16_to_f32(((const uint16_t*)logits)[(size_t)t * E + e])
                                : ((const float*)logits)[(size_t)t * E + e];
            v[e] = sanitize(raw);
            taken[e] = 0;
        }
        /* k rounds of "largest remaining value, lowest index among equals" */
        for (int j = 0; j < k; j++) {
            int best = -1;
            for (int e = 0; e < E; e++) {
                if (taken[e]) continue;
                if (best < 0 || v[e] > v[best]) best = e;
            }
            taken[best] = 1;
            ids[(size_t)t * k + j] = best;
        }
        const int32_t* id = ids + (size_t)t * k;
        double* wt = w + (size_t)t * k;
        if (scoring == 0) {
            double m = v[id[0]]; /* the first pick holds the row maximum */
            double denom = 0.0;
            if (renorm) for (int j = 0; j < k; j++) denom += exp((double)v[id[j]] - m);
            else for (int e = 0; e < E; e++) denom += exp((double)v[e] - m);
            for (int j = 0; j < k; j++) wt[j] = exp((double)v[id[j]] - m) / denom;
        } else {
            double sum = 0.0;
            for (int j = 0; j < k; j++) {
                wt[j] = 1.0 / (1.0 + exp(-(double)v[id[j]]));
                sum += wt[j];
            }
            if (renorm) {
                for (int j = 0; j < k; j++) wt[j] = (sum > 0.0) ? wt[j] / sum : 1.0 / k;
            }
        }
    }
    free(v);
    free(taken);
}

/* Grouped (group-limited) top-k.  [PR39593] names a grouped top-k beside the plain one without
 * defining it; this is the plain reading, written out (and listed with the other readings of
 * the pages):
 *   1. the E experts form n_group groups of E/n_group consecutive indices;
 *   2. a group's key is the largest sanitised logit among its experts;
 *   3. the topk_group groups with the largest keys are kept, the lower group index first
 *      among equal keys;
 *   4. the k ids are picked as in oracle_router_topk, among the kept groups' experts only;
 *   5. the weights are those of oracle_router_topk for these ids (softmax without
 *      renormalisation still normalises over all E experts).
 * Requires E % n_group == 0, 1 <= topk_group <= n_group and k <= topk_group * E / n_group,
 * so the k ids are distinct.  With n_group == 1 or topk_group == n_group it is
 * oracle_router_topk. */
void oracle_router_topk_grouped(const void* logits, int is_bf16, int T, int E, int k, int n_group, int topk_group,
                                int scoring, int renorm, int32_t* ids, double* w) {
    const int gsz = E / n_group;
    float* v = (float*)malloc(sizeof(float) * (size_t)E);
    char* taken = (char*)malloc((size_t)E);
    float* gkey = (float*)malloc(sizeof(float) * (size_t)n_group);
    char* gkept = (char*)malloc((size_t)n_group);
    for (int t = 0; t < T; t++) {
        for (int e = 0; e < E; e++) {
            float raw = is_bf16 ? oracle_bf16_to_f32(((const uint16_t*)logits)[(size_t)t * E + e])
                                : ((const float*)logits)[(size_t)t * E + e];
            v[e] = sanitize(raw);
        }
        /* step 2: group keys */
        for (int g = 0; g < n_group; g++) {
            gkey[g] = v[g * gsz];
            for (int e = g * gsz + 1; e < (g + 1) * gsz; e++)
                if (v[e] > gkey[g]) gkey[g] = v[e];
            gkept[g] = 0;
        }
        /* step 3: topk_group rounds of "largest remaining key, lowest group among equals" */
        for (int j = 0; j < topk_group; j++) {
            int best = -1;
            for (int g = 0; g < n_group; g++) {
                if (gkept[g]) continue;
                if (best < 0 || gkey[g] > gkey[best]) best = g;
            }
            gkept[best] = 1;
        }
        /* step 4: the plain selection, with the experts of dropped groups already taken */
        for (int e = 0; e < E; e++) taken[e] = !gkept[e / gsz];
        for (int j = 0; j < k; j++) {
            int best = -1;
            for (int e = 0; e < E; e++) {
                if (taken[e]) continue;
                if (best < 0 || v[e] > v[best]) best = e;
            }
            taken[best] = 1;
            ids[(size_t)t * k + j] = best;
        }
        /* step 5: weights as the plain router */
        const int32_t* id = ids + (size_t)t * k;
        double* wt = w + (size_t)t * k;
        if (scoring == 0) {
            double m = v[0];
            for (int e = 1; e < E; e++) if (v[e] > m) m = v[e];
            double denom = 0.0;
            if (renorm) for (int j = 0; j < k; j++) denom += exp((double)v[id[j]] - m);
            else for (int e = 0; e < E; e++) denom += exp((double)v[e] - m);
            for (int j = 0; j < k; j++) wt[j] = exp((double)v[id[j]] - m) / denom;
        } else {
            double sum = 0.0;
            for (int j = 0; j < k; j++) {
                wt[j] = 1.0 / (1.0 + exp(-(double)v[id[j]]));
                sum += wt[j];
            }
            if (renorm) {
                for (int j = 0; j < k; j++) wt[j] = (sum > 0.0) ? wt[j] / sum : 1.0 / k;
            }
        }
    }
    free(v);
    free(taken);
    free(gkey);
    free(gkept);
}

/* ------------------------------------------------------------------ grouping */

/* Rows per expert estimate of [H20] paragraph 3: ceil(tokens * top_k / total physical
 * experts), at least 1. */
int oracle_rows_per_expert_estimate(long long T, long long k, long long E) {
    long long num = T * k;
    long long est = (num + E - 1) / E;
    return (int)(est < 1 ? 1 : est);
}

/* Per-expert grouping of the T*k assignments of this expert-parallel rank.
 * Expert range of the rank: [ep_rank*E_loc, (ep_rank+1)*E_loc), E_loc = E/ep_size ([H20]
 * paragraph 2: expert-parallel size and rank).  Flat assignment i = t*k + j.
 *   counts[l]      rows of local expert l
 *   offsets[l]     exclusive prefix sum; offsets[E_loc] = R (all local rows)
 *   perm_src[p]    flat index of the p-th grouped row: experts ascending, and inside an
 *                  expert flat index ascending (a stable counting sort)
 *   inv_perm[i]    grouped row of assignment i, or -1 when it is not local
 * Ids outside [0,E) are not local and are counted in *dropped. */
void oracle_route_permute(int T, int k, int E, int ep_size, int ep_rank, const int32_t* ids,
                          int32_t* counts, int32_t* offsets, int32_t* perm_src, int32_t* inv_perm,
                          long long* dropped) {
    int El = E / ep_size;
    long long n = (long long)T * k, bad = 0;
    for (int l = 0; l < El; l++) counts[l] = 0;
    for (long long i = 0; i < n; i++) {
        int id = ids[i];
        if (id < 0 || id >= E) { bad++; continue; }
        int l = id - ep_rank * El;
        if (l >= 0 && l < El) counts[l]++;
    }
    offsets[0] = 0;
    for (int l = 0; l < El; l++) offsets[l + 1] = offsets[l] + counts[l];
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)(El > 0 ? El : 1));
    for (int l = 0; l < El; l++) cursor[l] = offsets[l];
    for (long long i = 0; i < n; i++) {
        int id = ids[i];
        int l = id - ep_rank * El;
        if (id < 0 || id >= E || l < 0 || l >= El) { inv_perm[i] = -1; continue; }
        int p = cursor[l]++;
        perm_src[p] = (int32_t)i;
        inv_perm[i] = p;
    }
    free(cursor);
    if (dropped) *dropped = bad;
}

/* ------------------------------------------------------------------ FP8 activation quantisation */

/* Per row, per group of 128 consecutive columns ([LAB6] fp8_w8a8: per-token, per-128-column
 * activation scales in fp32): amax = max |x| over the group; s = amax / 448 (s = 1 when
 * amax = 0); inv = 1 / s; q = e4m3(max(min(x * inv, 448), -448)).  The min/max clamp is the
 * saturating conversion of [PR39593] Root cause: a NaN input becomes +448.  All fp32. */
void oracle_act_quant(const float* x, int rows, int cols, uint8_t* q, float* s) {
    int G = cols / 128;
    for (int r = 0; r < rows; r++)
        for (int g = 0; g < G; g++) {
            const float* xg = x + (size_t)r * cols + (size_t)g * 128;
            float amax = 0.0f;
            for (int c = 0; c < 128; c++) {
                float a = fabsf(xg[c]);
                if (a > amax) amax = a; /* NaN never compares greater */
            }
            float sc = (amax == 0.0f) ? 1.0f : amax / OR_E4M3_MAX;
            float inv = 1.0f / sc;
            s[(size_t)r * G + g] = sc;
            for (int c = 0; c < 128; c++) {
                float y = xg[c] * inv;
                y = fminf(y, OR_E4M3_MAX);
                y = fmaxf(y, -OR_E4M3_MAX);
                q[(size_t)r * cols + (size_t)g * 128 + c] = oracle_e4m3_encode(y);
            }
        }
}

/* ------------------------------------------------------------------ experts */

typedef struct {
    int T, H, I, E, k, ep_size, ep_rank, fp8;
    const uint16_t* x;                 /* [T,H] bf16 */
    const void *wg, *wu, *wd;          /* bf16 or e4m3 codes: [E_loc,I,H], [E_loc,I,H], [E_loc,H,I] */
    const float *sg, *su, *sd;         /* fp8 block scales [E_loc,I/128,H/128], same, [E_loc,H/128,I/128] */
} or_layer;

/* Dequantised weight W[l, n, kk] of a [E_loc, N, K] tensor (bf16, or e4m3 code times the
 * fp32 scale of its [128,128] block, [H20] paragraph 2 and [LAB6] block_shape). */
static double wval(const void* w, const float* sc, int fp8, int l, int n, int kk, int N, int K) {
    size_t idx = ((size_t)l * N + n) * K + kk;
    if (!fp8) return oracle_bf16_to_f32(((const uint16_t*)w)[idx]);
    double q = oracle_e4m3_decode(((const uint8_t*)w)[idx]);
    return q * (double)sc[((size_t)l * (N / 128) + n / 128) * (K / 128) + kk / 128];
}

/* One SwiGLU expert on one token: y = W_down * (silu(W_gate x) * (W_up x)), silu(g) =
 * g / (1 + exp(-g)).  In the FP8 layer both expert inputs (x and the activation) are first
 * quantised per 128 columns (oracle_act_quant) and used dequantised (code * scale). */
static void expert_token(const or_layer* L, int t, int l, double* y /* [H] */) {
    int H = L->H, I = L->I;
    float* xf = (float*)malloc(sizeof(float) * (size_t)H);
    double* xh = (double*)malloc(sizeof(double) * (size_t)H);
    double* a = (double*)malloc(sizeof(double) * (size_t)I);
    for (int h = 0; h < H; h++) xf[h] = oracle_bf16_to_f32(L->x[(size_t)t * H + h]);
    if (L->fp8) {
        uint8_t* q = (uint8_t*)malloc((size_t)H);
        float* s = (float*)malloc(sizeof(float) * (size_t)(H / 128));
        oracle_act_quant(xf, 1, H, q, s);
        for (int h = 0; h < H; h++) xh[h] = (double)oracle_e4m3_decode(q[h]) * (double)s[h / 128];
        free(q); free(s);
    } else {
        for (int h = 0; h < H; h++) xh[h] = xf[h];
    }
    for (int n = 0; n < I; n++) {
        double g = 0.0, u = 0.0;
        for (int h = 0; h < H; h++) {
            g += xh[h] * wval(L->wg, L->sg, L->fp8, l, n, h, I, H);
            u += xh[h] * wval(L->wu, L->su, L->fp8, l, n, h, I, H);
        }
        a[n] = g / (1.0 + exp(-g)) * u;
    }
    if (L->fp8) {
        float* af = (float*)malloc(sizeof(float) * (size_t)I);
        uint8_t* q = (uint8_t*)malloc((size_t)I);
        float* s = (float*)malloc(sizeof(float) * (size_t)(I / 128));
        for (int n = 0; n < I; n++) af[n] = (float)a[n];
        oracle_act_quant(af, 1, I, q, s);
        for (int n = 0; n < I; n++) a[n] = (double)oracle_e4m3_decode(q[n]) * (double)s[n / 128];
        free(af); free(q); free(s);
    }
    for (int h = 0; h < H; h++) {
        double acc = 0.0;
        for (int n = 0; n < I; n++) acc += a[n] * wval(L->wd, L->sd, L->fp8, l, h, n, H, I);
        y[h] = acc;
    }
    free(xf); free(xh); free(a);
}

/* Layer output for the listed tokens:
 *   out[r, :] = sum_{j ascending, id local} w[t,j] * expert_{id - ep_rank*E_loc}(x[t])
 * for t = tokens[r]; ids outside [0,E) or outside the rank's range add nothing, so a token
 * with no local pick gets a zero row.  Tokens are independent: OpenMP over the list. */
void oracle_moe_tokens(int T, int H, int I, int E, int k, int ep_size, int ep_rank, int fp8,
                       const uint16_t* x, const int32_t* ids, const double* w,
                       const void* wg, const void* wu, const void* wd,
                       const float* sg, const float* su, const float* sd,
                       const int32_t* tokens, int ntok, double* out) {
    or_layer L = {T, H, I, E, k, ep_size, ep_rank, fp8, x, wg, wu, wd, sg, su, sd};
    int El = E / ep_size;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < ntok; r++) {
        int t = tokens[r];
        double* o = out + (size_t)r * H;
        double* y = (double*)malloc(sizeof(double) * (size_t)H);
        for (int h = 0; h < H; h++) o[h] = 0.0;
        for (int j = 0; j < k; j++) {
            int id = ids[(size_t)t * k + j];
            int l = id - ep_rank * El;
            if (id < 0 || id >= E || l < 0 || l >= El) continue;
            expert_token(&L, t, l, y);
            for (int h = 0; h < H; h++) o[h] += w[(size_t)t * k + j] * y[h];
        }
        free(y);
    }
}

/* One grouped GEMM stage of the layer on given operands, rows in the grouped order of
 * oracle_route_permute (local experts ascending, flat index ascending inside an expert):
 *   stage 0 (gate/up): grouped row p of flat assignment i = perm_src[p], token t = i / k,
 *     local expert l:  g_n = sum_h a[t,h] Wg[l,n,h],  u_n = sum_h a[t,h] Wu[l,n,h],
 *     out[p,n] = g_n / (1 + exp(-g_n)) * u_n       (SiLU on the gate times up; n < N = I)
 *   stage 1 (down): out[p,n] = sum_i a[p,i] Wd[l,n,i]  (n < N = H; a holds grouped rows)
 * a is bf16 (a_fp8 = 0: uint16 bit patterns) or e4m3 codes times the fp32 scale of their
 * 128-column group (a_fp8 = 1: a_scale [rows, K/128]); weights as in oracle_moe_tokens
 * (w1/s1 unused in stage 1).  Double arithmetic, sums in ascending reduction index.  Writes
 * out[0..R-1] ([R, N], R = local rows) and returns R. */
int oracle_grouped_gemm(int stage, int T, int k, int E, int ep_size, int ep_rank, int N, int K, int a_fp8,
                        const int32_t* ids, const void* a, const float* a_scale, int w_fp8, const void* w0,
                        const void* w1, const float* s0, const float* s1, double* out) {
    int El = E / ep_size;
    long long n = (long long)T * k;
    int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)(El > 0 ? El : 1));
    int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(El + 1));
    int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    int32_t* inv = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    oracle_route_permute(T, k, E, ep_size, ep_rank, ids, counts, offsets, perm, inv, NULL);
    int R = offsets[El];
    int G = K / 128;
#pragma omp parallel for schedule(dynamic, 4)
    for (int p = 0; p < R; p++) {
        int l = 0;
        while (offsets[l + 1] <= p) l++; /* the expert whose rows hold p */
        int row = (stage == 0) ? perm[p] / k : p;
        double* av = (double*)malloc(sizeof(double) * (size_t)K);
        for (int c = 0; c < K; c++) {
            size_t idx = (size_t)row * K + c;
            av[c] = a_fp8 ? (double)oracle_e4m3_decode(((const uint8_t*)a)[idx]) * (double)a_scale[(size_t)row * G + c / 128]
                          : (double)oracle_bf16_to_f32(((const uint16_t*)a)[idx]);
        }
        for (int f = 0; f < N; f++) {
            double acc0 = 0.0, acc1 = 0.0;
            for (int c = 0; c < K; c++) {
                acc0 += av[c] * wval(w0, s0, w_fp8, l, f, c, N, K);
                if (stage == 0) acc1 += av[c] * wval(w1, s1, w_fp8, l, f, c, N, K);
            }
            out[(size_t)p * N + f] = (stage == 0) ? acc0 / (1.0 + exp(-acc0)) * acc1 : acc0;
        }
        free(av);
    }
    free(counts); free(offsets); free(perm); free(inv);
    return R;
}

/* Thread count of the OpenMP loops above (the benchmark times the oracle on one core and on
 * all of them); 0 or less keeps the current setting. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Threads OpenMP would use for oracle_moe_tokens (reported beside its timings). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

// abi.cpp -- the extern "C" entry points of libfmoe: argument checks, the plan (rows per
// expert estimate and tile size), worst-case workspace layout, and kernel launches.
//
// Plan ("vLLM Community Traces H20 MoE Scheduling Inefficiency to Expert-Load Kernel
// Selection", paragraph 3): the workspace is laid out for the worst case first (every
// assignment local, any imbalance); then the rows-per-expert estimate
// max(1, ceil(T*top_k/E)) with E the total physical expert slots picks the largest light row
// tile (16 or 32 rows).  The grouping kernel sorts each expert by its real row count on the
// device: one light tile when it fits, heavy tiles of up to 256 rows otherwise (the hot
// experts of a concentrated routing, every expert of a large batch), without a host round
// trip.  Both GEMM kernels run; the one with an empty tile list exits at once.  FP8: when no
// expert can hold more than a few light tiles' rows (router ids are distinct per token, so an
// expert holds at most T rows; caller ids at most T*top_k), heavier experts are cut into
// several light tiles instead and the heavy-tile launches are left out.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/fmoe.h"
#include "launch.hpp"

using namespace fmoe;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Worst-case workspace layout of one call.
struct Layout {
    size_t hdr, ids, wts, counts, offsets, perm, inv, rank, grp, mtiles, xq, xs, h, hq, hs, y, total;
};

struct Plan {
    int T, H, I, E, k, El, lo;
    bool fp8;
    long long n;         // T*k assignments
    int rows_estimate;   // max(1, ceil(T*k/E))
    int tile_rows;       // largest light row tile: 16 or 32
    int light_cap;       // experts with up to this many rows get light tiles, heavier ones heavy tiles
    bool heavy_launch;   // some expert may exceed light_cap: run the heavy-tile kernels
    int heavy5;          // one tile for experts of 257..320 rows: -1 never, 1 always, 0 the grouping decides
    int max_light;       // bounds on light and heavy row tiles for any routing
    int max_heavy;
    int wk1, wk2;        // wavefronts splitting the reduction of the gate/up and down GEMMs
    int sparse_rows;     // > 0: the forward also launches the split gate/up kernel (split 2) for
                         // light tiles of fewer rows than this on average (decided on the device)
    bool down_combine;   // the down GEMM and the combine in one launch (small bf16 batches)
    Layout L;
};

int check_shape(const fmoe_shape* s) {
    if (!s) return FMOE_ERR_ARG;
    if (s->tokens < 0 || s->hidden <= 0 || s->inter <= 0 || s->experts <= 0 || s->top_k <= 0) return FMOE_ERR_ARG;
    if (s->hidden % 128 || s->inter % 128) return FMOE_ERR_UNSUPPORTED;
    if (s->hidden > FMOE_MAX_DIM || s->inter > FMOE_MAX_DIM) return FMOE_ERR_UNSUPPORTED;
    if (s->top_k > s->experts) return FMOE_ERR_ARG;
    if (s->top_k > FMOE_MAX_TOP_K) return FMOE_ERR_UNSUPPORTED;
    if (s->ep_size <= 0 || s->experts % s->ep_size || s->ep_rank < 0 || s->ep_rank >= s->ep_size) return FMOE_ERR_ARG;
    if (s->experts / s->ep_size > FMOE_MAX_EXPERTS || s->experts > FMOE_MAX_EXPERTS) return FMOE_ERR_UNSUPPORTED;
    if (s->weight_dtype != FMOE_BF16 && s->weight_dtype != FMOE_FP8_E4M3) return FMOE_ERR_UNSUPPORTED;
    if ((long long)s->tokens * s->top_k > FMOE_MAX_ASSIGNMENTS) return FMOE_ERR_UNSUPPORTED;
    return FMOE_OK;
}

// ov: tile plan overrides (nullptr: the heuristic alone); checked by check_plan first.
// max_expert_rows bounds the rows of one expert: T when the router made the ids (distinct
// experts per token), T*k (the default) for ids from the caller.  The workspace layout does not
// depend on it.
Plan make_plan(const fmoe_shape* s, const fmoe_plan* ov = nullptr, long long max_expert_rows = -1) {
    Plan p;
    p.T = s->tokens;
    p.H = s->hidden;
    p.I = s->inter;
    p.E = s->experts;
    p.k = s->top_k;
    p.El = s->experts / s->ep_size;
    p.lo = s->ep_rank * p.El;
    p.fp8 = s->weight_dtype == FMOE_FP8_E4M3;
    p.n = (long long)p.T * p.k;
    long long est = (p.n + p.E - 1) / p.E;
    p.rows_estimate = (int)(est < 1 ? 1 : est);
    // Largest row tile: 16 rows at one expected row per expert, 32 rows from two expected
    // rows on (the estimate plus three standard deviations of the per-expert count under
    // uniform routing, about sqrt(estimate), already exceeds 16 rows at 8).  The tile-space
    // sweep (bench.py --tile-sweep) measured 32 rows at two expected rows as fast as 16 under
    // uniform routing and faster under concentrated routing, where hot experts of up to 32 rows
    // stay light tiles (T=32 of the 128-expert layer: 212 / 95 us against 214 / 108); at
    // T <= 32 it also leaves no expert for the heavy-tile launches.  From 32 expected rows per
    // expert on, most experts exceed a light tile anyway, and the sweep measured the smallest
    // light tile best there (every expert above 16 rows goes to the heavy-tile kernel): 270
    // against 304 us at T=512.
    int tr = p.rows_estimate >= 2 ? kLightRows : 16;
    if (p.rows_estimate >= 32) tr = 16;
    // FP8 stages the tile's activation scales in LDS: keep them within 64 KB
    while (p.fp8 && tr > 16 && gemm_lds_bytes(true, p.H > p.I ? p.H : p.I, tr) > 65536) tr >>= 1;
    if (ov && ov->tile_rows) tr = ov->tile_rows;
    p.tile_rows = tr;
    // Split the reduction over 4 wavefronts when the expected tiles (about one per active
    // expert under uniform routing) times the 16-feature blocks leave the GPU's 1024 SIMDs
    // with fewer than one wavefront each.  Otherwise the streaming kernel (no split), except
    // where the tile-space sweep measured a split of 2 faster (bf16 weights): the gate/up GEMM
    // below 16 expected rows per expert (T=8: 133 -> 118 us, T=32: 225 -> 212 us) and from 32
    // on, where the light tiles are the few experts left below 17 rows (T=512: equal under
    // uniform routing, 311 -> 289 us under concentrated routing), and the down GEMM at one
    // expected row (T=8: 118 -> 111 us).  FP8 tiles stream best unsplit at a 2048-deep
    // reduction (T=128: 141 against 150 us split), but a gate/up reduction of 4096 or more
    // splits better in two (the 7168-wide expert shard at T=288: 433 against 440 us uniform,
    // 325 against 331 us concentrated).  At one expected row per expert (T=8) the bf16 gate/up
    // GEMM splits in two as well: 95.2 against 100.5 us with a split of 4 under uniform
    // routing, 45.4 against 43.2 us under concentrated routing (whole-line weight loads; with
    // per-step loads four had been as fast under uniform routing and faster when concentrated).
    const long long local_rows = (p.n * p.El + p.E - 1) / p.E;
    const long long active = local_rows < p.El ? local_rows : p.El;
    auto pick_wk = [&](int N, bool gate_up) {
        const long long tasks = active * (N / 16);
        if (tasks < 1024) return 4;
        // from 128 expected rows on the light tiles are the few experts left below 17 rows, each
        // a short stream: splits of 4 (gate/up) and 2 (down) measured best under uniform and
        // concentrated routing (T=4096: 537 / 603 us against 540 / 620 us with 2 and 1)
        if (!p.fp8 && p.rows_estimate >= 128) return gate_up ? 4 : 2;
        if (!p.fp8 && (gate_up ? p.rows_estimate < 16 || p.rows_estimate >= 32 : p.rows_estimate <= 1)) return 2;
        if (p.fp8 && gate_up && p.H >= 4096) return 2;
        return tasks < 2048 ? 2 : 1;
    };
    p.wk1 = ov && ov->split_gate_up ? ov->split_gate_up : pick_wk(p.I, true);
    p.wk2 = ov && ov->split_down ? ov->split_down : pick_wk(p.H, false);
    // Routing concentration, read on the device ([H20] paragraph 4): where the heuristic streams
    // the bf16 gate/up GEMM unsplit (16 to 31 expected rows per expert), the grouping hands the
    // light tiles to the split-reduction kernel instead when they hold fewer than a quarter of the
    // expected rows on average.  Those are the cold experts of a concentrated batch (one or two
    // rows each, their hot experts in heavy tiles); the tile-space sweep measured them faster
    // split in two (T=256 concentrated: 250.5 against 260.8 us) and uniform routing, whose light
    // tiles hold about the expected rows, faster streamed (254.3 against 290.1 us).  The launch
    // of the kernel left without tiles costs about a microsecond and a half.
    p.sparse_rows = (!p.fp8 && p.wk1 == 1 && !(ov && ov->split_gate_up) && p.rows_estimate >= 8)
                        ? p.rows_estimate / 4 : 0;
    // FP8: several light tiles per expert (up to kMaxLightPerExpert) when that bounds every
    // expert.  The heavy-tile launches are then left out, and the gate/up kernel writes the
    // quantised activation itself (no quantisation launch, no fp32 activation); the light tiles
    // of one expert share its weights in one XCD's L2.  The tile-space sweep measured this
    // faster at T=64-256 of the 128-expert layer under uniform and concentrated routing alike
    // (T=256 concentrated: 160 against 175 us).  bf16 has no quantisation to save, and under
    // concentrated routing its hot experts ran faster as heavy tiles (T=256: 262 against
    // 283 us), so bf16 keeps one light tile per expert.
    if (max_expert_rows < 0) max_expert_rows = p.n;
    const int per = ov && ov->light_tiles ? ov->light_tiles : p.fp8 ? kMaxLightPerExpert : 1;
    p.light_cap = max_expert_rows <= (long long)per * tr ? per * tr : tr;
    p.heavy_launch = max_expert_rows > p.light_cap;
    // light tiles: ceil(c/tile_rows) per expert with 1..light_cap rows, at most
    // min(n, El + n/16) in all; heavy tiles: at most ceil(c/256) per expert with c > tile_rows
    // rows, at most n/256 + n/(tile_rows+1) in all (bounded with the smallest light tile,
    // 16 rows, so one workspace fits every tile plan); no tile is empty
    long long nl = p.El + p.n / 16;
    if (nl > p.n) nl = p.n;
    p.heavy5 = p.fp8 ? -1 : ov && ov->heavy_rows ? (ov->heavy_rows == kHeavyRows5 ? 1 : -1) : 0;
    long long nh = p.n / kHeavyRows + (p.n / 17 < p.El ? p.n / 17 : p.El) + 1;
    if (nh > p.n) nh = p.n;
    p.max_light = (int)(nl < 1 ? 1 : nl);
    p.max_heavy = (int)(nh < 1 ? 1 : nh);
    // A few assignments (bf16): the down GEMM is a matrix-vector stream, and the combine joins
    // it in the same launch (down_combine.hip), unless a plan asks for a down split.
    p.down_combine = down_combine_fits(p.fp8, p.n, p.I) && !(ov && ov->split_down);

    Layout& L = p.L;
    size_t o = 0;
    const size_t n = (size_t)(p.n > 0 ? p.n : 1);
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align_up(o + bytes);
        return at;
    };
    L.hdr = take(sizeof(DevHeader));
    L.ids = take(n * 4);
    L.wts = take(n * 4);
    L.counts = take((size_t)p.El * 4);
    L.offsets = take((size_t)(p.El + 1) * 4);
    L.perm = take(n * 4);
    L.inv = take(n * 4);
    L.rank = take(n * 4);
    L.grp = take(group_scratch_bytes((long long)n, p.El));
    L.mtiles = take((size_t)(p.max_light + p.max_heavy) * sizeof(MTile));
    if (p.fp8) {
        L.xq = take((size_t)p.T * p.H);
        L.xs = take((size_t)p.T * (p.H / 128) * 4);
        L.h = take(n * p.I * 4);  // fp32 activation before its quantisation
        L.hq = take(n * p.I);
        L.hs = take(n * (p.I / 128) * 4);
    } else {
        L.xq = L.xs = L.hq = L.hs = 0;
        L.h = take(n * p.I * 2);
    }
    L.y = take(n * p.H * 2);
    L.total = o;
    return p;
}

int device_cus() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        cache[dev] = cus;
    }
    return cache[dev];
}

// FMOE_LOG=1 in the environment (read once): every layer call prints its plan to stderr, one
// line, before it launches anything.
bool log_enabled() {
    static const int on = [] {
        const char* v = std::getenv("FMOE_LOG");
        return (v && *v && std::strcmp(v, "0") != 0) ? 1 : 0;
    }();
    return on != 0;
}

// The 256-row heavy tiles from which the grouping cuts an expert of 257..320 rows as one tile
// of five row groups (INT_MAX: never): enough tiles that the GEMM with the fewer 128-column
// blocks (gate/up 2*I/128, down H/128) gives every compute unit four tasks.  There the launch is
// bound by the copies into LDS, which one task in place of two cuts by the second task's weight
// stream (128 experts of 272 rows, 2048 deep: 290 against 360 us for the gate/up GEMM as one
// tile and as two); with fewer tasks the launch is as long as its longest task, which a tile of
// five groups lengthens (the hot experts of a concentrated batch: 81 against 64 us).
int heavy5_min_tiles(const Plan& p) {
    if (p.heavy5 < 0) return INT_MAX;
    if (p.heavy5 > 0) return 0;
    const int nb = 2 * p.I < p.H ? 2 * p.I / 128 : p.H / 128;
    return (4 * device_cus() + nb - 1) / nb;
}

void log_plan(const char* who, const Plan& p) {
    if (!log_enabled()) return;
    std::fprintf(stderr,
                 "[fmoe] %s: T=%d H=%d I=%d E=%d k=%d E_loc=%d first_expert=%d %s | rows_estimate=%d "
                 "tile_rows=%d light_cap=%d heavy_launch=%d heavy5=%d split_gate_up=%d split_down=%d "
                 "sparse_rows=%d down_combine=%d max_light_tiles=%d max_heavy_tiles=%d workspace=%zu B\n",
                 who, p.T, p.H, p.I, p.E, p.k, p.El, p.lo, p.fp8 ? "fp8" : "bf16", p.rows_estimate, p.tile_rows,
                 p.light_cap, (int)p.heavy_launch, p.heavy5, p.wk1, p.wk2, p.sparse_rows, (int)p.down_combine, p.max_light,
                 p.max_heavy,
                 p.L.total);
}

int hip_status(hipError_t e) { return e == hipSuccess ? FMOE_OK : FMOE_ERR_HIP; }

#define FMOE_TRY(expr)                          \
    do {                                        \
        hipError_t e_ = (expr);                 \
        if (e_ != hipSuccess) return FMOE_ERR_HIP; \
    } while (0)

int check_weights(const Plan& p, const fmoe_weights* w) {
    if (!w || !w->gate || !w->up || !w->down) return FMOE_ERR_ARG;
    if (!aligned16(w->gate) || !aligned16(w->up) || !aligned16(w->down)) return FMOE_ERR_ARG;
    const bool scales = w->gate_scale && w->up_scale && w->down_scale;
    const bool none = !w->gate_scale && !w->up_scale && !w->down_scale;
    if (p.fp8 ? !scales : !none) return FMOE_ERR_ARG;
    return FMOE_OK;
}

void record(void* const* ev, int i, hipStream_t st) {
    if (ev && ev[i]) (void)hipEventRecord((hipEvent_t)ev[i], st);
}

// Grouping, expert GEMMs and combine for routing already in ids/wts (device pointers).
// grouped: the fused router + grouping launch has already written the grouping; x_quantised:
// the router launch has already written the FP8 codes and scales of x.
int run_experts(const Plan& p, const void* x, const int32_t* ids, const float* wts, const fmoe_weights* w, void* out,
                char* ws, hipStream_t st, void* const* ev, bool grouped = false, bool x_quantised = false) {
    const Layout& L = p.L;
    DevHeader* hdr = (DevHeader*)(ws + L.hdr);
    int32_t* perm = (int32_t*)(ws + L.perm);
    int32_t* inv = (int32_t*)(ws + L.inv);
    MTile* mtiles = (MTile*)(ws + L.mtiles);
    const int cus = device_cus();

    record(ev, FMOE_STAGE_GROUP, st);
    MTile* mtiles_heavy = mtiles + p.max_light;
    if (!grouped)
        FMOE_TRY(launch_group(ids, (int)p.n, p.E, p.El, p.lo, p.tile_rows, p.light_cap, heavy5_min_tiles(p), p.rows_estimate,
                              p.sparse_rows, (int32_t*)(ws + L.counts),
                          (int32_t*)(ws + L.offsets), perm, inv, (int32_t*)(ws + L.rank), (int*)(ws + L.grp), mtiles,
                          mtiles_heavy, hdr, st));
    const bool heavy_possible = p.heavy_launch;
    // FP8 with light tiles only and the streaming gate/up kernel: that kernel writes the e4m3
    // codes and scales of h itself, so the quantisation launch and the fp32 h are left out
    const bool fused_quant_h = p.fp8 && !heavy_possible && p.wk1 == 1;

    record(ev, FMOE_STAGE_QUANT_X, st);
    if (p.fp8 && !x_quantised)
        FMOE_TRY(launch_quant_rows(x, true, p.T, p.H, (uint8_t*)(ws + L.xq), (float*)(ws + L.xs), nullptr, st));

    record(ev, FMOE_STAGE_GEMM1, st);
    GemmArgs g1;
    g1.A = p.fp8 ? (const void*)(ws + L.xq) : x;
    g1.A_scale = p.fp8 ? (const float*)(ws + L.xs) : nullptr;
    g1.perm_src = perm;
    g1.topk = p.k;
    g1.W0 = w->gate;
    g1.W1 = w->up;
    g1.S0 = w->gate_scale;
    g1.S1 = w->up_scale;
    g1.N = p.I;
    g1.K = p.H;
    g1.out = fused_quant_h ? ws + L.hq : ws + L.h;
    g1.out_scale = fused_quant_h ? (float*)(ws + L.hs) : nullptr;
    g1.mtiles = mtiles;
    g1.tile_count = &hdr->m_tiles;
    GemmArgs g1h = g1;
    g1h.mtiles = mtiles_heavy;
    g1h.tile_count = &hdr->m_tiles_heavy;
    if (p.wk1 == 1) {
        GemmArgs g1s = g1;  // the light tiles' other kernel (the grouping gives all of them to one)
        if (p.sparse_rows > 0) {
            g1.tile_count = &hdr->m_tiles_stream;
            g1s.tile_count = &hdr->m_tiles_split;
        }
        FMOE_TRY(launch_grouped_gemm_stream(true, p.fp8, fused_quant_h ? kOutE4M3 : p.fp8 ? kOutF32 : kOutBf16, g1,
                                            p.tile_rows, p.max_light, cus, st));
        record(ev, FMOE_STAGE_GEMM1_SPLIT, st);
        if (p.sparse_rows > 0) FMOE_TRY(launch_grouped_gemm(true, p.fp8, p.fp8, g1s, p.tile_rows, 2, p.max_light, cus, st));
    } else {
        FMOE_TRY(launch_grouped_gemm(true, p.fp8, p.fp8, g1, p.tile_rows, p.wk1, p.max_light, cus, st));
        record(ev, FMOE_STAGE_GEMM1_SPLIT, st);
    }
    record(ev, FMOE_STAGE_GEMM1_HEAVY, st);
    if (heavy_possible) FMOE_TRY(launch_grouped_gemm_tiled(true, p.fp8, p.fp8, g1h, p.max_heavy, cus, st));

    record(ev, FMOE_STAGE_QUANT_H, st);
    if (p.fp8 && !fused_quant_h)
        FMOE_TRY(launch_quant_rows(ws + L.h, false, p.n, p.I, (uint8_t*)(ws + L.hq), (float*)(ws + L.hs), hdr, st));

    record(ev, FMOE_STAGE_GEMM2, st);
    if (p.down_combine) {
        FMOE_TRY(launch_down_combine(ws + L.h, w->down, p.H, p.I, mtiles, mtiles_heavy, hdr, inv, wts, p.T, p.k, out,
                                     st));
        record(ev, FMOE_STAGE_GEMM2_HEAVY, st);
        record(ev, FMOE_STAGE_COMBINE, st);
        record(ev, FMOE_NUM_STAGES, st);
        return FMOE_OK;
    }
    GemmArgs g2;
    g2.A = p.fp8 ? (const void*)(ws + L.hq) : (const void*)(ws + L.h);
    g2.A_scale = p.fp8 ? (const float*)(ws + L.hs) : nullptr;
    g2.perm_src = nullptr;
    g2.topk = p.k;
    g2.W0 = w->down;
    g2.W1 = nullptr;
    g2.S0 = w->down_scale;
    g2.S1 = nullptr;
    g2.N = p.H;
    g2.K = p.I;
    g2.out = ws + L.y;
    g2.out_scale = nullptr;
    g2.mtiles = mtiles;
    g2.tile_count = &hdr->m_tiles;
    GemmArgs g2h = g2;
    g2h.mtiles = mtiles_heavy;
    g2h.tile_count = &hdr->m_tiles_heavy;
    if (p.wk2 == 1) FMOE_TRY(launch_grouped_gemm_stream(false, p.fp8, kOutBf16, g2, p.tile_rows, p.max_light, cus, st));
    else FMOE_TRY(launch_grouped_gemm(false, p.fp8, false, g2, p.tile_rows, p.wk2, p.max_light, cus, st));
    record(ev, FMOE_STAGE_GEMM2_HEAVY, st);
    if (heavy_possible) FMOE_TRY(launch_grouped_gemm_tiled(false, p.fp8, false, g2h, p.max_heavy, cus, st));

    record(ev, FMOE_STAGE_COMBINE, st);
    FMOE_TRY(launch_combine(ws + L.y, inv, wts, p.T, p.k, p.H, out, st));
    record(ev, FMOE_NUM_STAGES, st);
    return FMOE_OK;
}

// One GEMM stage of run_experts on caller operands (fmoe_grouped_gemm): grouping of ids, then
// the light and heavy launches of that stage.  stage 0: a = [T, H] rows gathered through
// perm_src, out [n, I]; stage 1: a = [n, I] grouped rows, out [n, H] bf16.  out_mode for
// stage 0: kOutBf16 (bf16), kOutF32 or kOutE4M3 (FP8: fused into the streaming kernel when it
// alone runs, else the fp32 activation in ws.h and then the quantisation kernel).
int run_stage(const Plan& p, int stage, const int32_t* ids, const void* a, const float* a_scale,
              const fmoe_weights* w, int out_mode, void* out, float* out_scale, char* ws, hipStream_t st) {
    const Layout& L = p.L;
    DevHeader* hdr = (DevHeader*)(ws + L.hdr);
    int32_t* perm = (int32_t*)(ws + L.perm);
    MTile* mtiles = (MTile*)(ws + L.mtiles);
    MTile* mtiles_heavy = mtiles + p.max_light;
    const int cus = device_cus();
    FMOE_TRY(launch_group(ids, (int)p.n, p.E, p.El, p.lo, p.tile_rows, p.light_cap, heavy5_min_tiles(p), p.rows_estimate, 0,
                          (int32_t*)(ws + L.counts), (int32_t*)(ws + L.offsets), perm, (int32_t*)(ws + L.inv),
                          (int32_t*)(ws + L.rank), (int*)(ws + L.grp), mtiles, mtiles_heavy, hdr, st));
    GemmArgs g;
    g.A = a;
    g.A_scale = p.fp8 ? a_scale : nullptr;
    g.topk = p.k;
    g.out_scale = nullptr;
    g.mtiles = mtiles;
    g.tile_count = &hdr->m_tiles;
    if (stage == 0) {
        g.perm_src = perm;
        g.W0 = w->gate;
        g.W1 = w->up;
        g.S0 = w->gate_scale;
        g.S1 = w->up_scale;
        g.N = p.I;
        g.K = p.H;
        const bool fused = out_mode == kOutE4M3 && !p.heavy_launch && p.wk1 == 1;
        const bool via_f32 = out_mode == kOutE4M3 && !fused;
        g.out = via_f32 ? (void*)(ws + L.h) : out;
        g.out_scale = fused ? out_scale : nullptr;
        GemmArgs gh = g;
        gh.mtiles = mtiles_heavy;
        gh.tile_count = &hdr->m_tiles_heavy;
        const bool f32 = p.fp8;  // FP8 writes fp32 (or codes), bf16 writes bf16
        if (p.wk1 == 1)
            FMOE_TRY(launch_grouped_gemm_stream(true, p.fp8, fused ? kOutE4M3 : f32 ? kOutF32 : kOutBf16, g,
                                                p.tile_rows, p.max_light, cus, st));
        else FMOE_TRY(launch_grouped_gemm(true, p.fp8, f32, g, p.tile_rows, p.wk1, p.max_light, cus, st));
        if (p.heavy_launch) FMOE_TRY(launch_grouped_gemm_tiled(true, p.fp8, f32, gh, p.max_heavy, cus, st));
        if (via_f32) FMOE_TRY(launch_quant_rows(ws + L.h, false, p.n, p.I, (uint8_t*)out, out_scale, hdr, st));
        return FMOE_OK;
    }
    g.perm_src = nullptr;
    g.W0 = w->down;
    g.W1 = nullptr;
    g.S0 = w->down_scale;
    g.S1 = nullptr;
    g.N = p.H;
    g.K = p.I;
    g.out = out;
    GemmArgs gh = g;
    gh.mtiles = mtiles_heavy;
    gh.tile_count = &hdr->m_tiles_heavy;
    if (p.wk2 == 1) FMOE_TRY(launch_grouped_gemm_stream(false, p.fp8, kOutBf16, g, p.tile_rows, p.max_light, cus, st));
    else FMOE_TRY(launch_grouped_gemm(false, p.fp8, false, g, p.tile_rows, p.wk2, p.max_light, cus, st));
    if (p.heavy_launch) FMOE_TRY(launch_grouped_gemm_tiled(false, p.fp8, false, gh, p.max_heavy, cus, st));
    return FMOE_OK;
}

// Values a tile plan may force; the FP8 split kernel's LDS limit for 32-row tiles.
int check_plan(const fmoe_shape* s, const fmoe_plan* ov) {
    if (!ov) return FMOE_OK;
    auto split_ok = [](int v) { return v == 0 || v == 1 || v == 2 || v == 4; };
    if (!(ov->tile_rows == 0 || ov->tile_rows == 16 || ov->tile_rows == 32)) return FMOE_ERR_ARG;
    if (!split_ok(ov->split_gate_up) || !split_ok(ov->split_down)) return FMOE_ERR_ARG;
    if (!(ov->light_tiles == 0 || ov->light_tiles == 1 || ov->light_tiles == kMaxLightPerExpert)) return FMOE_ERR_ARG;
    if (!(ov->heavy_rows == 0 || ov->heavy_rows == kHeavyRows || ov->heavy_rows == kHeavyRows5)) return FMOE_ERR_ARG;
    if (s->weight_dtype == FMOE_FP8_E4M3 && ov->heavy_rows == kHeavyRows5) return FMOE_ERR_UNSUPPORTED;
    const int K = s->hidden > s->inter ? s->hidden : s->inter;
    if (s->weight_dtype == FMOE_FP8_E4M3 && ov->tile_rows == 32 && gemm_lds_bytes(true, K, 32) > 65536)
        return FMOE_ERR_UNSUPPORTED;
    return FMOE_OK;
}

int forward_impl(const fmoe_shape* s, const void* x, const void* logits, int32_t logits_dtype, int32_t scoring,
                 int32_t renormalize, const fmoe_weights* w, void* out, int32_t* ids_out, float* wts_out, void* ws,
                 size_t ws_bytes, void* stream, void* const* ev, const fmoe_plan* ov = nullptr) {
    int rc = check_shape(s);
    if (rc) return rc;
    if ((rc = check_plan(s, ov))) return rc;
    if (logits_dtype != FMOE_BF16 && logits_dtype != FMOE_FP32) return FMOE_ERR_UNSUPPORTED;
    if (scoring != FMOE_SOFTMAX && scoring != FMOE_SIGMOID) return FMOE_ERR_ARG;
    Plan p = make_plan(s, ov, s->tokens);
    if ((rc = check_weights(p, w))) return rc;
    if (p.T == 0) return FMOE_OK;
    if (!x || !logits || !out || !ws) return FMOE_ERR_ARG;
    if (!aligned16(x) || !aligned16(out) || !aligned16(ws)) return FMOE_ERR_ARG;
    if (ws_bytes < p.L.total) return FMOE_ERR_WORKSPACE;
    log_plan(ov ? "fmoe_forward_planned" : "fmoe_forward", p);
    hipStream_t st = (hipStream_t)stream;
    char* wsb = (char*)ws;
    int32_t* ids = ids_out ? ids_out : (int32_t*)(wsb + p.L.ids);
    float* wts = wts_out ? wts_out : (float*)(wsb + p.L.wts);
    record(ev, FMOE_STAGE_ROUTER, st);
    const bool bf16 = logits_dtype == FMOE_BF16;
    // FP8: the router launch quantises x as well (one token row per wavefront)
    const XQuant xq = {x, p.H, (uint8_t*)(wsb + p.L.xq), (float*)(wsb + p.L.xs)};
    const XQuant* xqp = p.fp8 ? &xq : nullptr;
    if (route_group_fits((int)p.T, p.k, p.E, p.El)) {  // small batch: router and grouping in one launch
        const Layout& L = p.L;
        MTile* mtiles = (MTile*)(wsb + L.mtiles);
        FMOE_TRY(launch_route_group(logits, bf16, (int)p.T, p.E, p.k, scoring, renormalize != 0, ids, wts, p.El, p.lo,
                                    p.tile_rows, p.light_cap, heavy5_min_tiles(p), p.rows_estimate, p.sparse_rows,
                                    (int32_t*)(wsb + L.counts),
                                    (int32_t*)(wsb + L.offsets), (int32_t*)(wsb + L.perm), (int32_t*)(wsb + L.inv),
                                    mtiles, mtiles + p.max_light, (DevHeader*)(wsb + L.hdr), st, xqp));
        return run_experts(p, x, ids, wts, w, out, wsb, st, ev, true, p.fp8);
    }
    FMOE_TRY(launch_router_topk(logits, bf16, p.T, p.E, p.k, scoring, renormalize != 0, ids, wts, st, 1, 1, xqp));
    return run_experts(p, x, ids, wts, w, out, wsb, st, ev, false, p.fp8);
}

}  // namespace

// Workspace of fmoe_forward_noalloc: a static device buffer, one copy per GPU (the code object
// is loaded on every device the library runs on).  Host code never passes this name to a
// kernel or a copy: the name is a host-side stand-in, and only the device address that
// hipGetSymbolAddress returns for the current device is used.
static __device__ __align__(256) unsigned char scratch[FMOE_NOALLOC_MAX_WORKSPACE];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up once per device.
int scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FMOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return FMOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FMOE_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return FMOE_OK;
}

}  // namespace

extern "C" {

int fmoe_abi_version(void) { return FMOE_ABI_VERSION; }

const char* fmoe_status_string(int status) {
    switch (status) {
        case FMOE_OK: return "ok";
        case FMOE_ERR_ARG: return "invalid argument";
        case FMOE_ERR_UNSUPPORTED: return "unsupported size or dtype";
        case FMOE_ERR_WORKSPACE: return "workspace too small";
        case FMOE_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

int fmoe_workspace_bytes(const fmoe_shape* shape, size_t* bytes) {
    int rc = check_shape(shape);
    if (rc) return rc;
    if (!bytes) return FMOE_ERR_ARG;
    *bytes = make_plan(shape).L.total;
    return FMOE_OK;
}

int fmoe_router_logits(const void* x, const void* w_r, int32_t T, int32_t H, int32_t E, float* logits, void* stream) {
    if (T < 0 || H <= 0 || E <= 0) return FMOE_ERR_ARG;
    if (T == 0) return FMOE_OK;
    if (!x || !w_r || !logits) return FMOE_ERR_ARG;
    if ((long long)T * E > INT_MAX) return FMOE_ERR_UNSUPPORTED;
    return hip_status(launch_router_logits(x, w_r, T, H, E, logits, (hipStream_t)stream));
}

int fmoe_router_topk(const void* logits, int32_t logits_dtype, int32_t T, int32_t E, int32_t k, int32_t scoring,
                     int32_t renormalize, int32_t* topk_ids, float* topk_weights, void* stream) {
    if (T < 0 || E <= 0 || k <= 0 || k > E) return FMOE_ERR_ARG;
    if (E > FMOE_MAX_EXPERTS || k > FMOE_MAX_TOP_K) return FMOE_ERR_UNSUPPORTED;
    if (logits_dtype != FMOE_BF16 && logits_dtype != FMOE_FP32) return FMOE_ERR_UNSUPPORTED;
    if (scoring != FMOE_SOFTMAX && scoring != FMOE_SIGMOID) return FMOE_ERR_ARG;
    if (T == 0) return FMOE_OK;
    if (!logits || !topk_ids || !topk_weights) return FMOE_ERR_ARG;
    return hip_status(launch_router_topk(logits, logits_dtype == FMOE_BF16, T, E, k, scoring, renormalize != 0,
                                         topk_ids, topk_weights, (hipStream_t)stream));
}

int fmoe_router_topk_grouped(const void* logits, int32_t logits_dtype, int32_t T, int32_t E, int32_t k,
                             int32_t n_group, int32_t topk_group, int32_t scoring, int32_t renormalize,
                             int32_t* topk_ids, float* topk_weights, void* stream) {
    if (T < 0 || E <= 0 || k <= 0 || k > E) return FMOE_ERR_ARG;
    if (E > FMOE_MAX_EXPERTS || k > FMOE_MAX_TOP_K) return FMOE_ERR_UNSUPPORTED;
    if (n_group > 64) return FMOE_ERR_UNSUPPORTED;
    if (n_group < 1 || E % n_group || topk_group < 1 || topk_group > n_group) return FMOE_ERR_ARG;
    if ((long long)k > (long long)topk_group * (E / n_group)) return FMOE_ERR_ARG;
    if (logits_dtype != FMOE_BF16 && logits_dtype != FMOE_FP32) return FMOE_ERR_UNSUPPORTED;
    if (scoring != FMOE_SOFTMAX && scoring != FMOE_SIGMOID) return FMOE_ERR_ARG;
    if (T == 0) return FMOE_OK;
    if (!logits || !topk_ids || !topk_weights) return FMOE_ERR_ARG;
    return hip_status(launch_router_topk(logits, logits_dtype == FMOE_BF16, T, E, k, scoring, renormalize != 0,
                                         topk_ids, topk_weights, (hipStream_t)stream, n_group, topk_group));
}

int fmoe_route_permute(const fmoe_shape* shape, const int32_t* topk_ids, int32_t* counts, int32_t* offsets,
                       int32_t* perm_src, int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_shape(shape);
    if (rc) return rc;
    Plan p = make_plan(shape);
    if (p.T == 0) return FMOE_OK;
    if (!topk_ids || !counts || !offsets || !perm_src || !inv_perm || !ws) return FMOE_ERR_ARG;
    if (!aligned16(ws)) return FMOE_ERR_ARG;
    if (ws_bytes < p.L.total) return FMOE_ERR_WORKSPACE;
    char* wsb = (char*)ws;
    MTile* mt = (MTile*)(wsb + p.L.mtiles);
    return hip_status(launch_group(topk_ids, (int)p.n, p.E, p.El, p.lo, p.tile_rows, p.light_cap, heavy5_min_tiles(p),
                                   p.rows_estimate, p.sparse_rows, counts, offsets,
                                   perm_src, inv_perm, (int32_t*)(wsb + p.L.rank), (int*)(wsb + p.L.grp), mt,
                                   mt + p.max_light, (DevHeader*)(wsb + p.L.hdr), (hipStream_t)stream));
}

int fmoe_experts(const fmoe_shape* shape, const void* x, const int32_t* topk_ids, const float* topk_weights,
                 const fmoe_weights* w, void* out, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_shape(shape);
    if (rc) return rc;
    Plan p = make_plan(shape);
    if ((rc = check_weights(p, w))) return rc;
    if (p.T == 0) return FMOE_OK;
    if (!x || !topk_ids || !topk_weights || !out || !ws) return FMOE_ERR_ARG;
    if (!aligned16(x) || !aligned16(out) || !aligned16(ws)) return FMOE_ERR_ARG;
    if (ws_bytes < p.L.total) return FMOE_ERR_WORKSPACE;
    log_plan("fmoe_experts", p);
    return run_experts(p, x, topk_ids, topk_weights, w, out, (char*)ws, (hipStream_t)stream, nullptr);
}

int fmoe_forward(const fmoe_shape* shape, const void* x, const void* logits, int32_t logits_dtype, int32_t scoring,
                 int32_t renormalize, const fmoe_weights* w, void* out, int32_t* topk_ids_out,
                 float* topk_weights_out, void* ws, size_t ws_bytes, void* stream) {
    return forward_impl(shape, x, logits, logits_dtype, scoring, renormalize, w, out, topk_ids_out,
                        topk_weights_out, ws, ws_bytes, stream, nullptr);
}

int fmoe_forward_profiled(const fmoe_shape* shape, const void* x, const void* logits, int32_t logits_dtype,
                          int32_t scoring, int32_t renormalize, const fmoe_weights* w, void* out,
                          int32_t* topk_ids_out, float* topk_weights_out, void* ws, size_t ws_bytes, void* stream,
                          void* const* stage_events) {
    if (!stage_events) return FMOE_ERR_ARG;
    return forward_impl(shape, x, logits, logits_dtype, scoring, renormalize, w, out, topk_ids_out,
                        topk_weights_out, ws, ws_bytes, stream, stage_events);
}

int fmoe_forward_planned(const fmoe_shape* shape, const void* x, const void* logits, int32_t logits_dtype,
                         int32_t scoring, int32_t renormalize, const fmoe_weights* w, void* out,
                         int32_t* topk_ids_out, float* topk_weights_out, void* ws, size_t ws_bytes, void* stream,
                         const fmoe_plan* plan) {
    return forward_impl(shape, x, logits, logits_dtype, scoring, renormalize, w, out, topk_ids_out,
                        topk_weights_out, ws, ws_bytes, stream, nullptr, plan);
}

int fmoe_act_quant(const void* x, int32_t x_dtype, int64_t rows, int32_t cols, uint8_t* q, float* s, void* stream) {
    if (rows < 0 || cols <= 0) return FMOE_ERR_ARG;
    if (cols % 128 || cols > FMOE_MAX_DIM) return FMOE_ERR_UNSUPPORTED;
    if (x_dtype != FMOE_BF16 && x_dtype != FMOE_FP32) return FMOE_ERR_UNSUPPORTED;
    if (rows * (cols / 128) > (long long)INT_MAX * 4) return FMOE_ERR_UNSUPPORTED;  // grid size
    if (rows == 0) return FMOE_OK;
    if (!x || !q || !s) return FMOE_ERR_ARG;
    if (!aligned16(x) || !aligned16(q) || ((uintptr_t)s & 3u)) return FMOE_ERR_ARG;
    return hip_status(launch_quant_rows(x, x_dtype == FMOE_BF16, rows, cols, q, s, nullptr, (hipStream_t)stream));
}

int fmoe_workspace_layout(const fmoe_shape* shape, fmoe_layout* out) {
    int rc = check_shape(shape);
    if (rc) return rc;
    if (!out) return FMOE_ERR_ARG;
    const Plan p = make_plan(shape);
    const Layout& L = p.L;
    std::memset(out, 0, sizeof(*out));
    if (p.fp8) {
        out->x_codes = L.xq;
        out->x_scales = L.xs;
        out->h_f32 = L.h;
        out->h_codes = L.hq;
        out->h_scales = L.hs;
    } else {
        out->h_bf16 = L.h;
    }
    out->y = L.y;
    out->perm_src = L.perm;
    out->inv_perm = L.inv;
    out->total = L.total;
    return FMOE_OK;
}

int fmoe_grouped_gemm(const fmoe_shape* shape, const fmoe_plan* plan, int32_t stage, const int32_t* topk_ids,
                      const void* a, const float* a_scale, const fmoe_weights* w, int32_t out_dtype, void* out,
                      float* out_scale, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_shape(shape);
    if (rc) return rc;
    if ((rc = check_plan(shape, plan))) return rc;
    if (stage != 0 && stage != 1) return FMOE_ERR_ARG;
    Plan p = make_plan(shape, plan);
    if ((rc = check_weights(p, w))) return rc;
    int mode;
    if (stage == 1) {
        if (out_dtype != FMOE_BF16) return FMOE_ERR_ARG;
        mode = kOutBf16;
    } else if (!p.fp8) {
        if (out_dtype != FMOE_BF16) return FMOE_ERR_ARG;
        mode = kOutBf16;
    } else {
        if (out_dtype == FMOE_FP32) mode = kOutF32;
        else if (out_dtype == FMOE_FP8_E4M3) mode = kOutE4M3;
        else return FMOE_ERR_ARG;
    }
    if (p.T == 0) return FMOE_OK;
    if (!topk_ids || !a || !out || !ws) return FMOE_ERR_ARG;
    if (p.fp8 && !a_scale) return FMOE_ERR_ARG;
    if (mode == kOutE4M3 && !out_scale) return FMOE_ERR_ARG;
    if (!aligned16(a) || !aligned16(out) || !aligned16(ws)) return FMOE_ERR_ARG;
    if (ws_bytes < p.L.total) return FMOE_ERR_WORKSPACE;
    log_plan(stage == 0 ? "fmoe_grouped_gemm gate/up" : "fmoe_grouped_gemm down", p);
    return run_stage(p, stage, topk_ids, a, a_scale, w, mode, out, out_scale, (char*)ws, (hipStream_t)stream);
}

int fmoe_forward_noalloc(const fmoe_shape* shape, const void* x, const void* logits, int32_t logits_dtype,
                         int32_t scoring, int32_t renormalize, const fmoe_weights* w, void* out,
                         int32_t* topk_ids_out, float* topk_weights_out, void* stream) {
    int rc = check_shape(shape);
    if (rc) return rc;
    if (make_plan(shape).L.total > FMOE_NOALLOC_MAX_WORKSPACE) return FMOE_ERR_WORKSPACE;
    void* ws = nullptr;
    if (shape->tokens > 0 && (rc = scratch_of_current_device(&ws))) return rc;
    return forward_impl(shape, x, logits, logits_dtype, scoring, renormalize, w, out, topk_ids_out, topk_weights_out,
                        ws, FMOE_NOALLOC_MAX_WORKSPACE, stream, nullptr);
}

int fmoe_read_stats(const void* ws, void* stream, fmoe_stats* out) {
    if (!ws || !out) return FMOE_ERR_ARG;
    DevHeader h;
    hipStream_t st = (hipStream_t)stream;
    if (hipMemcpyAsync(&h, ws, sizeof(h), hipMemcpyDeviceToHost, st) != hipSuccess) return FMOE_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return FMOE_ERR_HIP;
    std::memset(out, 0, sizeof(*out));
    out->dropped_ids = h.dropped;
    out->local_rows = h.local_rows;
    out->max_rows = h.max_rows;
    out->empty_experts = h.empty_experts;
    out->m_tiles = h.m_tiles + h.m_tiles_heavy;
    out->heavy_tiles = h.m_tiles_heavy;
    out->heavy_rows = h.heavy_rows;
    out->tile_rows = h.tile_rows;
    out->rows_estimate = h.rows_estimate;
    out->light_rows = h.light_rows;
    out->split_light_tiles = h.m_tiles_split;
    return FMOE_OK;
}

}  // extern "C"

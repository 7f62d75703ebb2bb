// gemm_tiled.hip -- grouped expert GEMMs for heavy row tiles, both operands tiled through LDS.
//
// Same operation as gemm.hip (gate/up with SiLU-and-mul, or down; bf16 or FP8 block-scaled),
// for experts that hold more rows than a light tile: large batches, and the hot experts of a
// concentrated routing ("vLLM Community Traces H20 MoE Scheduling Inefficiency to
// Expert-Load Kernel Selection", paragraph 4: concentrated routing needs another kernel choice
// than the average).  With up to 320 rows per tile the work is a dense contraction, so the
// kernel is built around the matrix cores rather than the weight stream.
//
// Shape: one workgroup of 8 wavefronts computes a tile of up to 256 rows (320 for a bf16 expert
// of 257..320 rows cut as one tile) times 128 weight columns (gate/up: 64 features of each
// matrix, so SiLU-and-mul happens in registers).  The tile's rows are staged in NA groups of 64
// (NA = 1..5, FP8 1..4); the wavefronts form a 4 x 2 grid, each owning 16*NA rows x 64 columns
// (4*NA accumulators of 16 x 16), so all 8 wavefronts, and all four SIMDs equally, carry MFMA
// work whatever the tile's size.
// Every 128-byte slice of the reduction (64 bf16 or 128 e4m3 per row) is one stage: the
// activation rows (gathered through the row map) and the weight rows are copied straight from
// global memory into LDS by direct global-to-LDS loads: the activations three stages deep (two
// for tiles of five row groups), the weights four stages deep for bf16 (160 KB in all) and three
// for FP8, so one or two activation and three (FP8: two) weight stages are in flight while one is
// read.  A stage row of 8 pieces of 16 bytes keeps piece c at position c ^ ((row >> 1) & 7): the
// 16 rows read by one MFMA fragment then fall in 16 different bank groups.  Every wait is an
// explicit count of the loads that must have landed.
//
// Per stage and wavefront (NA = 4): 8 fragment reads (16 KB) feed 32 MFMAs of 16x16x32 (bf16),
// or 4 + 4 double-width reads feed 16 MFMAs of 16x16x128 (FP8, one per 128-deep scale block,
// whose product is added times weight scale x activation scale).
//
// Work order: the tasks (row tile, column block) of one expert run column block first, then
// tile, and the persistent workgroups of one XCD (workgroup ids equal mod 8) take consecutive
// tasks, so the tiles that read the same weight block, and the column blocks that read the same
// tile's activations, tend to run at the same time behind one L2.
#include <type_traits>

#include "launch.hpp"

namespace fmoe {

namespace {

constexpr int kTgCols = 128;     // weight columns per workgroup
constexpr int kTgThreads = 512;  // 8 wavefronts
constexpr int kTgWPieces = kTgCols * 8;  // 16-byte pieces of one weight stage (16 KB)
constexpr int kTgPieces = 10240;         // 16-byte pieces of the LDS (160 KB)
// LDS layout for a tile of NA 64-row groups (16-byte pieces): NX activation buffers of
// tg_xstride pieces (NA <= 4: three of 32 KB; NA = 5, bf16 only: two of 40 KB), then the
// weight buffers of 16 KB (bf16: four, FP8: three), then (FP8) three buffers of 256 fp32
// activation scales.
template <int NA> constexpr int tg_nx() { return NA == 5 ? 2 : 3; }
template <int NA> constexpr int tg_xstride() { return NA == 5 ? 5 * 512 : 4 * 512; }
template <int NA> constexpr int tg_wbase() { return tg_nx<NA>() * tg_xstride<NA>(); }
constexpr int kTgSBase = 3 * 2048 + 3 * kTgWPieces;
static_assert(tg_wbase<4>() + 4 * kTgWPieces <= kTgPieces && tg_wbase<5>() + 4 * kTgWPieces <= kTgPieces &&
                  kTgSBase + 3 * 64 <= kTgPieces,
              "LDS layout");

// Global-to-LDS copies of 64 lanes (16 or 4 bytes each) to LDS byte address lds (wavefront-
// uniform, in M0, which nothing else in this kernel uses).  Written as inline assembly: the
// buffers are parts of one LDS array picked per tile size, and the compiler, which tracks its
// own copies per array, would otherwise wait for every copy into the array before each
// fragment read.  Every wait on these copies is an explicit count.  No memory clobber: a copy
// never writes a buffer read in the same step, and as volatile statements the copies keep
// their order against the stage barrier and the waits; the fragment reads of the current
// stage may then be scheduled among them.
__device__ __forceinline__ void tg_copy16(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src) : "m0");
}
__device__ __forceinline__ void tg_copy4(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(src) : "m0");
}

template <int N>
__device__ __forceinline__ void tg_wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void tg_fence() { asm volatile("" ::: "memory"); }
// Workgroup barrier without the full memory wait __syncthreads implies around LDS DMA.  The
// wavefront's own LDS reads finish first: after the barrier other wavefronts copy the next
// stage into the buffer those reads came from, and the scheduler may otherwise sink the
// reads' wait (with the MFMAs that use them) below the barrier.
__device__ __forceinline__ void tg_barrier() {
    tg_fence();
    __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
    tg_fence();
}

template <int I, int N, typename F>
__device__ __forceinline__ void tg_static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        tg_static_for<I + 1, N>(f);
    }
}

// f(0), f(1), .. while f returns true, each call nested in the previous one's success branch
template <int I, int N, typename F>
__device__ __forceinline__ void tg_static_chain(F&& f) {
    if constexpr (I < N) {
        if (f(std::integral_constant<int, I>{})) tg_static_chain<I + 1, N>(f);
    }
}


// position of piece c of stage row r
__device__ __forceinline__ int tg_slot(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

template <bool GATED, bool FP8, bool OUT_F32>
__global__ __launch_bounds__(kTgThreads) void k_grouped_gemm_tiled(GemmArgs g) {
    // bf16: three activation and four weight buffers, 3 x 32 KB + 4 x 16 KB = 160 KB of LDS
    // (tiles of five row groups: two of 40 KB and four); FP8 keeps three weight buffers (its
    // activation scales take the room of the fourth)
    constexpr int NW = FP8 ? 3 : 4;
    __shared__ i32x4 LDS[kTgPieces];
    const uint32_t lds0 = (uint32_t)(size_t)(void*)LDS;

    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = w >> 1, wn = w & 1;  // row group (16*NA rows) and column group (64 columns)
    const int r16 = lane & 15, kg = lane >> 4;
    const int K = g.K;
    const size_t rowbytes = (size_t)K * (FP8 ? 1 : 2);
    const int nkb = K / (FP8 ? 128 : 64);  // stages
    const int nkb128 = K >> 7;             // 128-deep scale blocks
    const int feat_per_task = GATED ? kTgCols / 2 : kTgCols;
    const int nblocks = g.N / feat_per_task;
    const int tasks = *g.tile_count * nblocks;
    const int topk = g.perm_src ? g.topk : 1;

    // workgroups of one XCD (ids equal mod 8) take consecutive tasks
    const int G = gridDim.x;
    const int li = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;

    // fragment read offset of this lane inside a 16-row block, for piece group q (0..1)
    int frag[2];
#pragma unroll
    for (int q = 0; q < 2; q++) frag[q] = tg_slot(r16, q * 4 + kg);

    for (int t = li; t < tasks; t += G) {
        // The tasks of an expert with m heavy tiles (tiles first .. first+m-1) are
        // [first*nblocks, (first+m)*nblocks), ordered column block first, then tile: the m tiles
        // that read the same weight block are consecutive tasks.  The tile list is read-only
        // here: scalar loads through the constant address space.
        const int i0 = t / nblocks;
        const i32x4 m0 = *(const __attribute__((address_space(4))) i32x4*)(g.mtiles + i0);
        // unsigned: an expert's tile count reaches 32768 (2^23 rows of 256), bit 31 of the field
        const int m = (int)((uint32_t)m0[3] >> 16), first = i0 - (m0[3] & 0xffff);
        const int tl = t - first * nblocks;
        const int nb = tl / m;
        const int tile = first + (tl - nb * m);
        const i32x4 mv = tile == i0 ? m0 : *(const __attribute__((address_space(4))) i32x4*)(g.mtiles + tile);
        const int expert = mv[0], row0 = mv[1], rows = mv[2];
        // every load of the previous task has landed and every wavefront is past its last
        // stage, so all buffers are free
        tg_wait_vmcnt<0>();
        __syncthreads();

        auto run = [&](auto NAc) {
            constexpr int NA = decltype(NAc)::value;  // activation loads per stage = 64-row groups
            constexpr int LX = NA + (FP8 ? 1 : 0);  // vector-memory instructions per activation stage
            constexpr int LW = 2;                   // and per weight stage
            constexpr int NX = tg_nx<NA>();         // activation buffers
            constexpr int XSTRIDE = tg_xstride<NA>(), WBASE = tg_wbase<NA>();
            static_assert(!FP8 || NA <= 4, "FP8 tiles have at most 256 rows");
            // activation pieces: load j of wavefront w covers stage rows (j*8 + w)*8 .. +8
            size_t xoff[NA];
#pragma unroll
            for (int j = 0; j < NA; j++) {
                const int r = (j * 8 + w) * 8 + (lane >> 3);
                const int p = row0 + min(r, rows - 1);
                const int src = (g.perm_src ? g.perm_src[p] : p) / topk;
                const int c = (lane & 7) ^ ((r >> 1) & 7);
                xoff[j] = (size_t)src * rowbytes + c * 16;
            }
            // weight pieces: load j covers weight columns (j*8 + w)*8 .. +8 of the block
            const uint8_t* wsrc[2];
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int q = (j * 8 + w) * 8 + (lane >> 3);
                const int c = (lane & 7) ^ ((q >> 1) & 7);
                const uint8_t* base;
                size_t wrow;
                if constexpr (GATED) {
                    base = (const uint8_t*)(q < 64 ? g.W0 : g.W1);
                    wrow = (size_t)expert * g.N + nb * 64 + (q & 63);
                } else {
                    base = (const uint8_t*)g.W0;
                    wrow = (size_t)expert * g.N + nb * kTgCols + q;
                }
                wsrc[j] = base + wrow * rowbytes + c * 16;
            }
            // FP8 activation scales: wavefront w stages the scales of rows (w & 3)*64 + lane
            int ssrc = 0;
            if constexpr (FP8) {
                const int r = (w & 3) * 64 + lane;
                const int p = row0 + min(r, rows - 1);
                ssrc = (g.perm_src ? g.perm_src[p] : p) / topk;
            }

            // activation stage kb into buffer X<B> (FP8: with its activation scales)
            auto issue_x = [&](auto Bc, int kb) {
                constexpr int B = decltype(Bc)::value;
                const uint32_t X = lds0 + (uint32_t)(B * XSTRIDE) * 16;
                const size_t ko = (size_t)kb * 128;
#pragma unroll
                for (int j = 0; j < NA; j++)
                    tg_copy16((const uint8_t*)g.A + xoff[j] + ko, X + (uint32_t)((j * 8 + w) * 64) * 16);
                if constexpr (FP8)
                    tg_copy4(g.A_scale + (size_t)ssrc * nkb128 + kb,
                             lds0 + (uint32_t)(kTgSBase + B * 64) * 16 + (uint32_t)(w & 3) * 64 * 4);
            };
            // weight stage kb into buffer W<B>
            auto issue_w = [&](auto Bc, int kb) {
                constexpr int B = decltype(Bc)::value;
                const uint32_t W = lds0 + (uint32_t)(WBASE + B * kTgWPieces) * 16;
                const size_t ko = (size_t)kb * 128;
#pragma unroll
                for (int j = 0; j < 2; j++) tg_copy16(wsrc[j] + ko, W + (uint32_t)((j * 8 + w) * 64) * 16);
            };

            f32x4 acc[NA][4];
#pragma unroll
            for (int i = 0; i < NA; i++)
#pragma unroll
                for (int c = 0; c < 4; c++) acc[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};

            // weight rows of column block c of this wavefront (gate/up: c = 0,1 gate, 2,3 up)
            auto wcol = [&](int c) { return GATED ? (c >> 1) * 64 + wn * 32 + (c & 1) * 16 : wn * 64 + c * 16; };
            const int rb0 = wm * 16 * NA;  // first tile row of this wavefront
            // FP8 weight scales of the block: one per matrix and 128-deep block
            const int fb = GATED ? nb / 2 : nb;
            const size_t sidx = ((size_t)expert * (g.N / 128) + fb) * nkb128;

            // issue(): the next stages' copies, placed after this stage's fragment reads so that
            // every wavefront starts its MFMAs before its copies queue up behind the others'
            auto compute = [&](auto BXc, auto BWc, int kb, auto issue) {
                constexpr int B = decltype(BXc)::value, BW = decltype(BWc)::value;
                const i32x4* X = LDS + B * XSTRIDE;
                const i32x4* W = LDS + WBASE + BW * kTgWPieces;
                if constexpr (!FP8) {
#pragma unroll
                    for (int q = 0; q < 2; q++) {
                        bf16x8 xa[NA], wb[4];
#pragma unroll
                        for (int i = 0; i < NA; i++)
                            xa[i] = __builtin_bit_cast(bf16x8, X[(rb0 + i * 16) * 8 + frag[q]]);
#pragma unroll
                        for (int c = 0; c < 4; c++) wb[c] = __builtin_bit_cast(bf16x8, W[wcol(c) * 8 + frag[q]]);
                        if (q == 1) issue();
#pragma unroll
                        for (int i = 0; i < NA; i++)
#pragma unroll
                            for (int c = 0; c < 4; c++)
                                acc[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[c], xa[i], acc[i][c], 0, 0, 0);
                    }
                } else {
                    const float* S = (const float*)(LDS + kTgSBase + B * 64);
                    const float ws0 = *(const __attribute__((address_space(4))) float*)(g.S0 + sidx + kb);
                    const float ws1 =
                        GATED ? *(const __attribute__((address_space(4))) float*)(g.S1 + sidx + kb) : ws0;
                    i32x8 xa[NA], wb[4];
#pragma unroll
                    for (int i = 0; i < NA; i++) {
                        const i32x4 lo = X[(rb0 + i * 16) * 8 + frag[0]], hi = X[(rb0 + i * 16) * 8 + frag[1]];
                        xa[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    }
#pragma unroll
                    for (int c = 0; c < 4; c++) {
                        const i32x4 lo = W[wcol(c) * 8 + frag[0]], hi = W[wcol(c) * 8 + frag[1]];
                        wb[c] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    }
                    issue();
                    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < NA; i++) {
                        const float sa = S[rb0 + i * 16 + r16];
#pragma unroll
                        for (int c = 0; c < 4; c++) {
                            const f32x4 pr =
                                __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wb[c], xa[i], zero, 0, 0, 0, 0, 0, 0);
                            const float cs = (GATED && c >= 2 ? ws1 : ws0) * sa;
#pragma unroll
                            for (int e = 0; e < 4; e++) acc[i][c][e] = __builtin_fmaf(pr[e], cs, acc[i][c][e]);
                        }
                    }
                }
            };

            // Stage s sits in X<s % NX> and W<s % NW>.  The step of stage s waits for it (this
            // wavefront's loads, then everyone's), which also means every wavefront is done with
            // stage s-1, whose buffers then take activation stage s+NX-1 and weight stage s+NW-1:
            // the weights run one or two stages further ahead than the activations.  Loads land in
            // issue order, so the wait is a count of the loads issued after the last one of stage
            // s: NX = 3, NW = 3 (issue order X0 W0 X1 W1, then X2 W2 X3 W3 ..): the next step's X
            // and W; NX = 3, NW = 4 (W0 X0 W1 X1 W2, then X2 W3 X3 W4 ..): a W, then the next X
            // and W; NX = 2, NW = 4 (W0 W1 X0 W2, then X1 W3 X2 W4 ..): the next step's W.  The
            // last steps reload the last stage (from L2) in place of the stages past the end.
            constexpr int WAIT = NX == 2 ? LW : NW == 3 ? LX + LW : LX + 2 * LW;
            auto step = [&](auto Jc, int kb) {
                constexpr int J = decltype(Jc)::value;
                tg_wait_vmcnt<WAIT>();
                tg_barrier();
                auto issue = [&] {
                    issue_x(std::integral_constant<int, (J + NX - 1) % NX>{}, min(kb + NX - 1, nkb - 1));
                    issue_w(std::integral_constant<int, (J + NW - 1) % NW>{}, min(kb + NW - 1, nkb - 1));
                };
                // with two activation buffers a copy has one stage to land: issue it first
                if constexpr (NX == 2) {
                    issue();
                    compute(std::integral_constant<int, J % NX>{}, std::integral_constant<int, J % NW>{}, kb, [] {});
                } else {
                    compute(std::integral_constant<int, J % NX>{}, std::integral_constant<int, J % NW>{}, kb, issue);
                }
            };

            if constexpr (NX == 2) {
                issue_w(std::integral_constant<int, 0>{}, 0);
                issue_w(std::integral_constant<int, 1>{}, min(1, nkb - 1));
                issue_x(std::integral_constant<int, 0>{}, 0);
                issue_w(std::integral_constant<int, 2>{}, min(2, nkb - 1));
            } else if constexpr (NW == 3) {
                issue_x(std::integral_constant<int, 0>{}, 0);
                issue_w(std::integral_constant<int, 0>{}, 0);
                issue_x(std::integral_constant<int, 1>{}, min(1, nkb - 1));
                issue_w(std::integral_constant<int, 1>{}, min(1, nkb - 1));
            } else {
                issue_w(std::integral_constant<int, 0>{}, 0);
                issue_x(std::integral_constant<int, 0>{}, 0);
                issue_w(std::integral_constant<int, 1>{}, min(1, nkb - 1));
                issue_x(std::integral_constant<int, 1>{}, min(1, nkb - 1));
                issue_w(std::integral_constant<int, 2>{}, min(2, nkb - 1));
            }
            // Whole cycles of both buffer rings, unrolled so every buffer index is a constant,
            // then the remaining steps as nested conditions: the path back to the loop head is
            // always a whole cycle, and a skipped step skips all later ones, so the compiler's
            // count of the loads in flight never merges two different paths before a step.
            constexpr int U = NX == 2 ? 4 : NW == 3 ? 3 : 12;  // lcm(NX, NW)
            int kb = 0;
            for (; kb + U <= nkb; kb += U)
                tg_static_for<0, U>([&](auto Jc) { step(Jc, kb + decltype(Jc)::value); });
            tg_static_chain<0, U - 1>([&](auto Jc) {
                if (kb + decltype(Jc)::value >= nkb) return false;
                step(Jc, kb + decltype(Jc)::value);
                return true;
            });

            // lane (r16, kg) holds, for row block i and column block c, row rb0 + 16 i + r16
            // and the 4 columns 16 c + 4 kg .. +3 of its column group
#pragma unroll
            for (int i = 0; i < NA; i++) {
                const int r = rb0 + i * 16 + r16;
                if (r >= rows) continue;
#pragma unroll
                for (int c = 0; c < (GATED ? 2 : 4); c++) {
                    const int f = GATED ? nb * 64 + wn * 32 + c * 16 + kg * 4 : nb * kTgCols + wn * 64 + c * 16 + kg * 4;
                    const size_t o = (size_t)(row0 + r) * g.N + f;
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; e++) v[e] = GATED ? silu_mul(acc[i][c][e], acc[i][c + 2][e]) : acc[i][c][e];
                    if (OUT_F32) {
                        *(f32x4*)((float*)g.out + o) = f32x4{v[0], v[1], v[2], v[3]};
                    } else {
                        uint2 pk;
                        pk.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
                        pk.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
                        *(uint2*)((uint16_t*)g.out + o) = pk;
                    }
                }
            }
        };
        const int groups = (rows + 63) >> 6;
        if constexpr (!FP8) {
            if (groups > 4) {
                run(std::integral_constant<int, 5>{});
                continue;
            }
        }
        if (groups > 3) run(std::integral_constant<int, 4>{});
        else if (groups > 2) run(std::integral_constant<int, 3>{});
        else if (groups > 1) run(std::integral_constant<int, 2>{});
        else run(std::integral_constant<int, 1>{});
    }
    // the last steps' loads into LDS land before the workgroup (and its LDS) goes away
    tg_wait_vmcnt<0>();
}

template <bool GATED, bool FP8, bool OUT_F32>
hipError_t launch_tiled(const GemmArgs& a, int max_tiles, int cus, hipStream_t st) {
    const int per_task = GATED ? kTgCols / 2 : kTgCols;
    long long grid = (long long)max_tiles * (a.N / per_task);
    if (grid > cus) grid = cus;  // one workgroup per CU (the stage buffers take 144 to 160 KB of LDS)
    if (grid < 1) grid = 1;
    k_grouped_gemm_tiled<GATED, FP8, OUT_F32><<<(unsigned)grid, kTgThreads, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm_tiled(bool gated, bool fp8, bool out_f32, const GemmArgs& a, int max_tiles, int cus,
                                     hipStream_t st) {
    if (gated) {
        if (fp8) return out_f32 ? launch_tiled<true, true, true>(a, max_tiles, cus, st)
                                : launch_tiled<true, true, false>(a, max_tiles, cus, st);
        return launch_tiled<true, false, false>(a, max_tiles, cus, st);
    }
    if (fp8) return launch_tiled<false, true, false>(a, max_tiles, cus, st);
    return launch_tiled<false, false, false>(a, max_tiles, cus, st);
}

}  // namespace fmoe

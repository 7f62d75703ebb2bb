// gemm_heavy.hip -- grouped expert GEMMs for heavy row tiles (more rows than a light tile, at
// most 256 rows of one expert).
//
// Same operation as gemm.hip (gate/up with SiLU-and-mul, or down; bf16 or FP8 block-scaled),
// for experts that hold more rows than a light tile: large batches, and the hot experts of a
// concentrated routing ("vLLM Community Traces H20 MoE Scheduling Inefficiency to
// Expert-Load Kernel Selection", paragraph 4: concentrated routing needs another kernel choice
// than the average).
//
// Shape: a workgroup of 8 wavefronts owns one row tile and 128 output features; wavefront v
// takes 16 of the features (two weight matrices' worth for gate/up) for all of the tile's rows,
// so every weight fragment it holds feeds up to 16 sub-blocks of 16 rows, a 256-row tile reads
// its weights from HBM once, and every weight byte is loaded by one wavefront only.  Two
// wavefronts per SIMD keep the matrix cores fed while the other waits.
//
// Weights stream from HBM straight into registers (the MFMA "A" operand, a ring of D steps per
// wavefront).  The tile's activation rows (the "B" operand) are staged in LDS by direct
// global-to-LDS loads: each load instruction gathers one 16-row x 64-byte MFMA fragment (rows
// through the gather map) and writes it in the order the MFMA reads it (lane i at byte 16 i),
// so reads are contiguous and conflict free.  Four chunk buffers are kept, three chunks ahead
// of the one being read, so the gathers (served by L2 or the Infinity Cache) never hold up the
// stream.  Each buffer is a separate LDS array, so the compiler knows that a read of one
// buffer does not depend on loads still landing in another; the waits before each step and
// each chunk are explicit counts of the loads that must have arrived.
//
// FP8 (e4m3 weights with one fp32 scale per [128,128] block, activations with one fp32 scale
// per row and 128 columns): one v_mfma_f32_16x16x128_f8f6f4 covers one 128-deep scale block;
// its exact product is added to the fp32 accumulator times (weight scale * activation scale).
// The tile's weight scales are read into LDS once per tile, the activation scales of a chunk
// are staged with it.
#include <type_traits>

#include "launch.hpp"

namespace fmoe {

namespace {

constexpr int kHvFeatures = 128;  // output features per workgroup: 8 wavefronts x 16
constexpr int kHvThreads = 512;
constexpr int kHvFrags = 32;      // 1 KB fragment pieces per chunk buffer

template <bool FP8>
struct HvCfg {
    using T = bf16x8;
    static constexpr int KSTEP = 32;   // reduction depth of one MFMA
    static constexpr int EB = 2;       // bytes per element
    static constexpr int LANE_B = 16;  // operand bytes per lane per step
    static constexpr int HALVES = 1;   // 16-byte pieces per lane fragment
    static constexpr int CS = 2;       // steps per staged chunk
};
template <>
struct HvCfg<true> {
    using T = i32x8;
    static constexpr int KSTEP = 128;
    static constexpr int EB = 1;
    static constexpr int LANE_B = 32;
    static constexpr int HALVES = 2;
    static constexpr int CS = 1;
};

__device__ __forceinline__ float silu_mul_h(float g, float u) { return g / (1.0f + expf(-g)) * u; }

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;

// s_waitcnt vmcnt(N) with the other counters left free (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// compiler-only fence: no memory access moves across it; emits nothing
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

constexpr int cmin(int a, int b) { return a < b ? a : b; }
constexpr int cap63(int n) { return n > 63 ? 63 : n; }

// Vector-memory instructions certainly issued after the weight loads of the step at position p
// (0 <= p < 4 CS) of the four-chunk loop body, when that step is computed.  A step's loads are
// issued right after the step D earlier is computed; after them come the weight loads of the
// D-1 steps in between and the staging group at the start of every chunk entered since (in the
// first pass, steps p < D were loaded in the prologue, after which only the groups of chunks
// 0..p/CS follow).
template <int p, int CS, int D, int WL, int QD>
constexpr int weight_wait() {
    constexpr int crossed = (p + 4 * CS) / CS - (p + 4 * CS - D) / CS;
    return cap63((D - 1) * WL + QD * cmin(crossed, p / CS + 1));
}

template <bool GATED, bool FP8>
constexpr int ring_depth() {
    return FP8 ? (GATED ? 2 : 4) : (GATED ? 4 : 8);
}

template <bool GATED, bool FP8, bool OUT_F32>
__global__ __launch_bounds__(kHvThreads) void k_grouped_gemm_heavy(GemmArgs g) {
    using C = HvCfg<FP8>;
    using FT = typename C::T;
    constexpr int NW = GATED ? 2 : 1;
    constexpr int CS = C::CS;
    constexpr int D = ring_depth<GATED, FP8>();
    constexpr int WL = NW * (FP8 ? 2 : 1);  // weight load instructions per step
    static_assert(4 * CS % D == 0, "ring slots repeat every four chunks");

    // four chunk buffers, each its own LDS array (see the header)
    __shared__ i32x4 X0[kHvFrags * 64], X1[kHvFrags * 64], X2[kHvFrags * 64], X3[kHvFrags * 64];
    __shared__ float A0[FP8 ? 256 : 1], A1[FP8 ? 256 : 1], A2[FP8 ? 256 : 1], A3[FP8 ? 256 : 1];
    __shared__ float WS[2][FP8 ? kMaxKBlocks : 1];
    __shared__ int split_last;  // this workgroup completed a split task's reduction

    const int lane = lane_id();
    const int v = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, kg = lane >> 4;
    const int K = g.K;
    const int nsteps = K / C::KSTEP;
    const int nkb = K >> 7;
    const int nch = (nsteps + CS - 1) / CS;
    const size_t rowbytes = (size_t)K * C::EB;
    const int nblocks = g.N / kHvFeatures;
    const int tasks = *g.tile_count * nblocks;
    const int topk = g.perm_src ? g.topk : 1;
    // Too few tasks for the GPU (a few hot experts): split each task's reduction over KS
    // workgroups, whole groups of four chunks each; every split leaves its fp32 partial in its
    // own slot and the last to finish adds them in split order (a fixed order, so the result does
    // not depend on which one is last) and writes the output.  The partials of a task (written
    // and read back: 2 KS rows 4 bytes per feature) stay within a quarter of its weight bytes
    // (K per feature, times the element size), with rows those of the largest tile.
    const int ngroups = ((nsteps + CS - 1) / CS + 3) / 4;
    const int slots = min((int)gridDim.x, kSplitSlots);
    int KS = 1;
    if (g.part != nullptr && tasks > 0 && 2 * tasks <= slots) {
        const int big = max(16, min(*g.max_rows, heavy_max_rows(FP8)));
        const int by_bytes = (int)(rowbytes / (32 * (size_t)big));
        KS = max(1, min(min(min(8, slots / tasks), ngroups), by_bytes));
    }
    const int total = tasks * KS;

    for (int tl = blockIdx.x; tl < total; tl += gridDim.x) {
        const int task = tl / KS;
        const int ks = tl - task * KS;
        const int mt = task / nblocks;
        const int nb = task - mt * nblocks;
        // the tile list is read-only here: a scalar load through the constant address space
        const i32x4 mv = *(const __attribute__((address_space(4))) i32x4*)(g.mtiles + mt);
        const int expert = mv[0], row0 = mv[1], rows = mv[2];

        // one tile of NS sub-blocks of 16 rows
        auto run = [&](auto NSc) {
            constexpr int NS = decltype(NSc)::value;
            constexpr int F = CS * NS * C::HALVES;       // fragment pieces per chunk
            constexpr int QX = F >= 8 ? F / 8 : 1;       // staging loads per wavefront per chunk
            constexpr int QD = QX + (FP8 ? 1 : 0);       // with the activation-scale load
            constexpr int NWAIT = cap63(2 * QD + cmin(2 * CS, D + CS) * WL);
            constexpr int NPRO = cap63(2 * QD + D * WL);
            // this split's chunks [cb, ce): whole groups of four
            const int cb = 4 * (ks * ngroups / KS), ce = 4 * ((ks + 1) * ngroups / KS);

            // staging sources: wavefront v loads pieces (v*QX + j) mod F; piece f is step
            // f / (NS HALVES) of the chunk, sub-block (f / HALVES) % NS, half f % HALVES (waves
            // past the F pieces repeat one, writing the same bytes to the same place)
            size_t xoff[QX];
            int xstep[QX], xpos[QX];
#pragma unroll
            for (int j = 0; j < QX; j++) {
                const int f = (v * QX + j) % F;
                const int sb = (f / C::HALVES) % NS;
                const int p = row0 + min(sb * 16 + r16, rows - 1);
                const int src = (g.perm_src ? g.perm_src[p] : p) / topk;
                xoff[j] = (size_t)src * rowbytes + kg * C::LANE_B + (f % C::HALVES) * 16;
                xstep[j] = f / (NS * C::HALVES);
                xpos[j] = f * 64;
            }
            // FP8 activation scales of a chunk: entry e = (v*64 + lane) mod 16 NS is tile row e
            int ascale_src = 0;
            if constexpr (FP8) {
                const int e = (v * 64 + lane) % (16 * NS);
                const int p = row0 + min(e, rows - 1);
                ascale_src = (g.perm_src ? g.perm_src[p] : p) / topk;
            }
            auto stage = [&](auto Bc, int c) {
                constexpr int B = decltype(Bc)::value;
                i32x4* X = B == 0 ? X0 : B == 1 ? X1 : B == 2 ? X2 : X3;
#pragma unroll
                for (int j = 0; j < QX; j++) {
                    const size_t step = (size_t)min(c * CS + xstep[j], nsteps - 1);
                    __builtin_amdgcn_global_load_lds(
                        (gbl_void*)((const uint8_t*)g.A + xoff[j] + step * (C::KSTEP * C::EB)),
                        (lds_void*)(X + xpos[j]), 16, 0, 0);
                }
                if constexpr (FP8) {
                    float* A = B == 0 ? A0 : B == 1 ? A1 : B == 2 ? A2 : A3;
                    const int kb = min(c, nkb - 1);  // CS = 1: chunk c is 128-deep block c
                    __builtin_amdgcn_global_load_lds((gbl_void*)(g.A_scale + (size_t)ascale_src * nkb + kb),
                                                     (lds_void*)(A + ((v * 64) % (16 * NS))), 4, 0, 0);
                }
            };

            // weights: lane row r16 of this wavefront's 16 features
            const size_t wrow = (size_t)expert * g.N + nb * kHvFeatures + v * 16 + r16;
            const uint8_t* wp[NW];
            wp[0] = (const uint8_t*)g.W0 + wrow * rowbytes + kg * C::LANE_B;
            if constexpr (GATED) wp[NW - 1] = (const uint8_t*)g.W1 + wrow * rowbytes + kg * C::LANE_B;
            FT bw[D][NW];
            auto issue_w = [&](int slot, int step) {
                const size_t o = (size_t)min(step, nsteps - 1) * (C::KSTEP * C::EB);
#pragma unroll
                for (int h = 0; h < NW; h++) bw[slot][h] = *(const FT*)(wp[h] + o);
            };

            f32x4 acc[NS][NW];
#pragma unroll
            for (int sb = 0; sb < NS; sb++)
#pragma unroll
                for (int h = 0; h < NW; h++) acc[sb][h] = f32x4{0.f, 0.f, 0.f, 0.f};

            // step s of the chunk in buffer B, weights from ring slot `slot`.  The activation
            // fragments are read in groups of GS sub-blocks, double-buffered, so the reads of
            // the next group are in flight while the current group's MFMAs run.
            constexpr int GS = NS < 4 ? NS : 4;
            constexpr int NG = NS / GS;
            auto compute = [&](auto Bc, int slot, int s, int step) {
                constexpr int B = decltype(Bc)::value;
                const i32x4* X = B == 0 ? X0 : B == 1 ? X1 : B == 2 ? X2 : X3;
                i32x4 xr[2][GS][C::HALVES];
                auto read_group = [&](auto Gc) {
                    constexpr int G = decltype(Gc)::value;
#pragma unroll
                    for (int q = 0; q < GS; q++)
#pragma unroll
                        for (int hf = 0; hf < C::HALVES; hf++)
                            xr[G & 1][q][hf] = X[((s * NS + G * GS + q) * C::HALVES + hf) * 64 + lane];
                };
                auto mfma_group = [&](auto Gc) {
                    constexpr int G = decltype(Gc)::value;
#pragma unroll
                    for (int q = 0; q < GS; q++) {
                        const int sb = G * GS + q;
                        if constexpr (!FP8) {
                            const bf16x8 xb = __builtin_bit_cast(bf16x8, xr[G & 1][q][0]);
#pragma unroll
                            for (int h = 0; h < NW; h++)
                                acc[sb][h] =
                                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(bw[slot][h], xb, acc[sb][h], 0, 0, 0);
                        } else {
                            const float* A = B == 0 ? A0 : B == 1 ? A1 : B == 2 ? A2 : A3;
                            const i32x4 lo = xr[G & 1][q][0], hi = xr[G & 1][q][C::HALVES - 1];
                            const i32x8 xb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                            const float sa = A[sb * 16 + r16];
                            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int h = 0; h < NW; h++) {
                                const f32x4 pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                    bw[slot][h], xb, zero, 0, 0, 0, 0, 0, 0);
                                const float cs = WS[h][step] * sa;
#pragma unroll
                                for (int i = 0; i < 4; i++) acc[sb][h][i] = __builtin_fmaf(pr[i], cs, acc[sb][h][i]);
                            }
                        }
                    }
                };
                read_group(std::integral_constant<int, 0>{});
                __builtin_amdgcn_sched_group_barrier(0x100, GS * C::HALVES, 0);
                static_for<0, NG>([&](auto Gc) {
                    constexpr int G = decltype(Gc)::value;
                    if constexpr (G + 1 < NG) {
                        read_group(std::integral_constant<int, G + 1>{});
                        __builtin_amdgcn_sched_group_barrier(0x100, GS * C::HALVES, 0);
                    }
                    mfma_group(Gc);
                    __builtin_amdgcn_sched_group_barrier(0x008, GS * NW, 0);
                });
            };

            // prologue: chunks 0..2 in flight, D weight steps in flight, chunk 0 landed
            __builtin_amdgcn_sched_barrier(0);
            stage(std::integral_constant<int, 0>{}, cb);
            __builtin_amdgcn_sched_barrier(0);
            stage(std::integral_constant<int, 1>{}, cb + 1);
            __builtin_amdgcn_sched_barrier(0);
            stage(std::integral_constant<int, 2>{}, cb + 2);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int d = 0; d < D; d++) issue_w(d, cb * CS + d);
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<NPRO>();
            compiler_fence();
            __builtin_amdgcn_s_barrier();
            compiler_fence();
            __builtin_amdgcn_sched_barrier(0);

            // chunk c from buffer B: stage chunk c+3 into the buffer read last, run the chunk's
            // steps, then wait for chunk c+1 and for every wavefront to be done with chunk c
            auto chunk = [&](auto Bc, int c) {
                constexpr int B = decltype(Bc)::value;
                stage(std::integral_constant<int, (B + 3) & 3>{}, c + 3);
                __builtin_amdgcn_sched_barrier(0);
                static_for<0, CS>([&](auto Sc) {
                    constexpr int s = decltype(Sc)::value;
                    constexpr int slot = (B * CS + s) % D;
                    const int step = c * CS + s;
                    // this step's weights have landed (an explicit count: with global-to-LDS
                    // loads in flight the compiler would otherwise wait for everything)
                    wait_vmcnt<weight_wait<B * CS + s, CS, D, WL, QD>()>();
                    if (step < nsteps) compute(Bc, slot, s, step);
                    __builtin_amdgcn_sched_barrier(0);
                    issue_w(slot, step + D);
                    __builtin_amdgcn_sched_barrier(0);
                });
                wait_vmcnt<NWAIT>();
                compiler_fence();
                __builtin_amdgcn_s_barrier();
                compiler_fence();
                __builtin_amdgcn_sched_barrier(0);
            };
            // whole groups of four chunks (an early exit would cost the exact wait counts the
            // compiler keeps across the loop); chunks past the end load clamped addresses and
            // compute nothing
            for (int c0 = cb; c0 < ce; c0 += 4) {
                chunk(std::integral_constant<int, 0>{}, c0);
                chunk(std::integral_constant<int, 1>{}, c0 + 1);
                chunk(std::integral_constant<int, 2>{}, c0 + 2);
                chunk(std::integral_constant<int, 3>{}, c0 + 3);
            }

            // output of tile row col (this lane's sub-block row), features nb*128 + v*16 + kg*4 + i
            auto store = [&](int col, const f32x4& a0, const f32x4& a1) {
                const size_t o = (size_t)(row0 + col) * g.N + nb * kHvFeatures + v * 16 + kg * 4;
                float r[4];
#pragma unroll
                for (int i = 0; i < 4; i++) r[i] = GATED ? silu_mul_h(a0[i], a1[i]) : a0[i];
                if (OUT_F32) {
                    *(f32x4*)((float*)g.out + o) = f32x4{r[0], r[1], r[2], r[3]};
                } else {
                    uint2 pk;
                    pk.x = (uint32_t)f32_to_bf16(r[0]) | ((uint32_t)f32_to_bf16(r[1]) << 16);
                    pk.y = (uint32_t)f32_to_bf16(r[2]) | ((uint32_t)f32_to_bf16(r[3]) << 16);
                    *(uint2*)((uint16_t*)g.out + o) = pk;
                }
            };

            if (KS == 1) {
                // epilogue: lane holds tile rows sb*16 + r16
#pragma unroll
                for (int sb = 0; sb < NS; sb++) {
                    const int col = sb * 16 + r16;
                    if (col < rows) store(col, acc[sb][0], acc[sb][NW - 1]);
                }
                return;
            }
            // split reduction: every split leaves its partial in its slot (slot tl holds
            // [2][part_rows][128] fp32), the last to arrive adds the KS partials in split order.
            // The partials move through device-scope (sc1) 16-byte buffer stores and loads, which
            // write through / bypass the per-XCD L2; a device-wide fence instead would write
            // back and invalidate the whole L2 under every other workgroup's weight stream.
            // Each lane's stores are acknowledged (vmcnt 0) before the workgroup barrier and the
            // arrival count, and the last workgroup reads only after it has counted every
            // arrival.  Offsets past the buffer are dropped by the hardware range check.
            const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
                g.part, (short)0, (int)((size_t)kSplitSlots * 2 * g.part_rows * kHvFeatures * 4), 0x00020000);
            auto slot_off = [&](int slot, int h, int col) {
                return (int)(((((size_t)slot * 2 + h) * g.part_rows + col) * kHvFeatures + v * 16 + kg * 4) * 4);
            };
            constexpr int kDeviceScope = 16;  // cache policy: sc1
            typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
            for (int sb = 0; sb < NS; sb++) {
                const int col = sb * 16 + r16;
                if (col >= rows) continue;
#pragma unroll
                for (int h = 0; h < NW; h++)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[sb][h]), prs,
                                                           slot_off(tl, h, col), 0, kDeviceScope);
            }
            wait_vmcnt<0>();
            __syncthreads();
            if (threadIdx.x == 0) {
                const int before = __hip_atomic_fetch_add(&g.sem[task], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                split_last = before == KS - 1;
                // ready for the next launch (kernel boundaries order it before any later use)
                if (before == KS - 1)
                    __hip_atomic_store(&g.sem[task], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
            if (!split_last) return;
            for (int sb = 0; sb < NS; sb++) {
                const int col = sb * 16 + r16;
                if (col >= rows) continue;
                f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
                for (int j = 0; j < KS; j++) {
                    s0 += __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(prs, slot_off(task * KS + j, 0, col), 0, kDeviceScope));
                    if constexpr (GATED)
                        s1 += __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                            prs, slot_off(task * KS + j, 1, col), 0, kDeviceScope));
                }
                store(col, s0, s1);
            }
        };

        if constexpr (FP8) {
            // the workgroup's 128 features are one 128-row weight block
            const size_t srow = ((size_t)expert * (g.N >> 7) + nb) * nkb;
            for (int q = threadIdx.x; q < nkb; q += kHvThreads) {
                WS[0][q] = g.S0[srow + q];
                if (GATED) WS[1][q] = g.S1[srow + q];
            }
        }
        // every load of the previous tile has landed (its last staging loads ran past its end)
        // and every wavefront is past it, so the staging buffers are free; the weight scales are
        // visible
        wait_vmcnt<0>();
        __syncthreads();
        const int nsub = (rows + 15) >> 4;  // sub-blocks of 16 rows
        if (nsub > 8) {
            if constexpr (heavy_max_rows(FP8) > 128) run(std::integral_constant<int, 16>{});
        } else if (nsub > 4) run(std::integral_constant<int, 8>{});
        else if (nsub > 2) run(std::integral_constant<int, 4>{});
        else if (nsub > 1) run(std::integral_constant<int, 2>{});
        else run(std::integral_constant<int, 1>{});
    }
}

template <bool GATED, bool FP8, bool OUT_F32>
hipError_t launch_heavy(const GemmArgs& a, int max_tiles, int cus, hipStream_t st) {
    static int per_cu = 0;
    if (per_cu == 0) {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_grouped_gemm_heavy<GATED, FP8, OUT_F32>, kHvThreads,
                                                          0) != hipSuccess || nb < 1)
            nb = 1;
        per_cu = nb;
    }
    long long grid = (long long)max_tiles * (a.N / kHvFeatures);
    const long long cap = (long long)cus * per_cu;
    if (grid > cap) grid = cap;
    // with partial-sum slots, enough workgroups to split the reductions of a few tiles
    if (a.part != nullptr && grid < (cap < kSplitSlots ? cap : kSplitSlots)) grid = cap < kSplitSlots ? cap : kSplitSlots;
    if (grid < 1) grid = 1;
    k_grouped_gemm_heavy<GATED, FP8, OUT_F32><<<(unsigned)grid, kHvThreads, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm_heavy(bool gated, bool fp8, bool out_f32, const GemmArgs& a, int max_tiles, int cus,
                                     hipStream_t st) {
    if (gated) {
        if (fp8) return out_f32 ? launch_heavy<true, true, true>(a, max_tiles, cus, st)
                                : launch_heavy<true, true, false>(a, max_tiles, cus, st);
        return launch_heavy<true, false, false>(a, max_tiles, cus, st);
    }
    if (fp8) return launch_heavy<false, true, false>(a, max_tiles, cus, st);
    return launch_heavy<false, false, false>(a, max_tiles, cus, st);
}

}  // namespace fmoe

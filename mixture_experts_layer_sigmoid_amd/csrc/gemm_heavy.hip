// gemm_heavy.hip -- grouped expert GEMMs for heavy row tiles (33..256 rows of one expert).
//
// Same operation as gemm.hip (gate/up with SiLU-and-mul, or down; bf16 or FP8 block-scaled),
// for experts that hold more rows than the light kernel's 32: large batches, and the hot
// experts of a concentrated routing ("vLLM Community Traces H20 MoE Scheduling Inefficiency
// to Expert-Load Kernel Selection", paragraph 4: concentrated routing needs another kernel
// choice than the average).
//
// Shape: a workgroup owns one row tile (up to 256 rows = 16 sub-blocks of 16) and 128 output
// features; each of its 4 wavefronts owns 32 features (two 16-row weight blocks per matrix)
// and all the tile's rows.  The tile's activation rows are staged through LDS in chunks of
// 256 bytes per row (128 bf16 or 256 e4m3 along the reduction), double-buffered and shared by
// the 4 wavefronts, so each activation byte crosses L2 once per workgroup instead of once per
// wavefront.  Weights are streamed from HBM straight into registers (a ring of D MFMA steps)
// as in the light kernel, and every weight fragment feeds up to 16 sub-blocks of MFMAs, so a
// 256-row tile reads each weight of its 128 features once.  A chunk's MFMA work (about 4k
// cycles at 256 rows) covers the latency of the next chunk's loads.
#include <type_traits>

#include "launch.hpp"

namespace fmoe {

namespace {

constexpr int kHeavyFeatures = 128;        // output features per workgroup (4 x 32)
constexpr int kChunkBytes = 256;           // bytes per activation row per chunk
constexpr int kRowStride = kChunkBytes + 16;  // LDS row stride: conflict-free 16-byte reads

__device__ __forceinline__ float silu_mul_h(float g, float u) { return g / (1.0f + expf(-g)) * u; }

template <bool FP8>
struct HCfg {
    using T = bf16x8;
    static constexpr int KSTEP = 32;   // reduction depth of one MFMA
    static constexpr int EB = 2;       // bytes per element
    static constexpr int FRAG = 16;    // bytes per lane per operand
    static constexpr int D = 4;        // weight ring depth (steps)
};
template <>
struct HCfg<true> {
    using T = i32x8;
    static constexpr int KSTEP = 128;
    static constexpr int EB = 1;
    static constexpr int FRAG = 32;
    static constexpr int D = 2;
};

struct HeavyLds {
    uint8_t tok[2][kHeavyRows][kRowStride];  // activation chunks
    float asc[2][kHeavyRows][2];             // FP8: activation scales of the chunk's 2 k-blocks
    float wsc[2][kMaxKBlocks];               // FP8: weight-block scales (gate, up) of the tile
    int src[kHeavyRows];                     // activation row of each tile row
};

template <bool FP8>
__device__ __forceinline__ typename HCfg<FP8>::T lds_frag(const uint8_t* p) {
    if constexpr (FP8) {
        const i32x4 a = *(const i32x4*)p;
        const i32x4 b = *(const i32x4*)(p + 16);
        return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else {
        return *(const bf16x8*)p;
    }
}

template <bool FP8>
__device__ __forceinline__ typename HCfg<FP8>::T gl_frag(const uint8_t* p) {
    if constexpr (FP8) return *(const i32x8*)p;
    else return *(const bf16x8*)p;
}

template <bool GATED, bool FP8, bool OUT_F32, int NS>
__device__ __forceinline__ void heavy_tile(const GemmArgs& g, const MTile& m, int nb, HeavyLds& L) {
    using C = HCfg<FP8>;
    using FT = typename C::T;
    constexpr int NW = GATED ? 2 : 1;
    constexpr int FB = 2;                               // 16-row weight blocks per wavefront
    constexpr int CS = kChunkBytes / (C::KSTEP * C::EB);  // MFMA steps per chunk: 4 (bf16) / 2 (fp8)
    // weight ring depth in MFMA steps: deep enough to cover HBM latency under load; smaller
    // when the tile's accumulators leave fewer registers
    constexpr int D = FP8 ? C::D : (NS >= 16 ? C::D : 2 * C::D);
    constexpr int PIECES = NS * 16 * (kChunkBytes / 16) / 256;  // 16-byte staging pieces per thread
    static_assert((2 * CS) % D == 0, "ring slots repeat every pair of chunks");
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, kg = lane >> 4;
    const int K = g.K;
    const int nsteps = K / C::KSTEP;
    const int nchunks = (nsteps + CS - 1) / CS;
    const int nkb = K >> 7;
    const size_t rowbytes = (size_t)K * C::EB;
    const int f0 = nb * kHeavyFeatures + w * 32;  // this wavefront's first feature

    // weights: lane row r16 of block fb, bytes kg*FRAG of each step
    const uint8_t* wbase0 = (const uint8_t*)g.W0 + ((size_t)m.expert * g.N + f0 + r16) * rowbytes + kg * C::FRAG;
    const uint8_t* wbase1 = GATED ? (const uint8_t*)g.W1 + ((size_t)m.expert * g.N + f0 + r16) * rowbytes + kg * C::FRAG
                                  : wbase0;
    const size_t fbstride = 16 * rowbytes;
    FT bw[D][FB][NW];
    auto issue_w = [&](int slot, int step) {
        const size_t o = (size_t)step * C::KSTEP * C::EB;
#pragma unroll
        for (int fb = 0; fb < FB; fb++) {
            bw[slot][fb][0] = gl_frag<FP8>(wbase0 + fb * fbstride + o);
            if constexpr (GATED) bw[slot][fb][NW - 1] = gl_frag<FP8>(wbase1 + fb * fbstride + o);
        }
    };

    // staging: thread t owns 16-byte piece (t & 15) of rows (t >> 4) + 16j, j < PIECES.  In LDS
    // the pieces of a row are stored transposed (step-minor): piece q = step*PP + j goes to
    // position j*CS + step, so the 16-byte reads of one MFMA step (lane = 16*kg + row) fall in
    // 16 distinct 4-bank groups for any grouping of 16 lanes by row or by kg.
    constexpr int COLS = kChunkBytes / 16;
    constexpr int PP = COLS / CS;  // pieces per MFMA step in a row
    const int scol = threadIdx.x % COLS, srow0 = threadIdx.x / COLS;
    const int spos = (scol % PP) * CS + scol / PP;
    i32x4 stage[PIECES];
    float sstage[2];
    auto load_chunk = [&](int c) {
        // the last chunk may be partial: columns past the row end re-read the row's last 16 bytes
        const size_t col = min((size_t)c * kChunkBytes + scol * 16, rowbytes - 16);
#pragma unroll
        for (int j = 0; j < PIECES; j++)
            stage[j] = *(const i32x4*)((const uint8_t*)g.A + (size_t)L.src[srow0 + (256 / COLS) * j] * rowbytes + col);
        if constexpr (FP8) {
            // activation scales of the chunk's 2 k-blocks: 16*NS rows x 2 entries
#pragma unroll
            for (int q = 0; q < 2; q++) {
                const int e = threadIdx.x + 256 * q;
                const int r = e >> 1, kb = min(c * 2 + (e & 1), nkb - 1);
                sstage[q] = (r < NS * 16) ? g.A_scale[(size_t)L.src[r] * nkb + kb] : 0.0f;
            }
        }
    };
    auto store_chunk = [&](int buf) {
#pragma unroll
        for (int j = 0; j < PIECES; j++) *(i32x4*)&L.tok[buf][srow0 + (256 / COLS) * j][spos * 16] = stage[j];
        if constexpr (FP8) {
#pragma unroll
            for (int q = 0; q < 2; q++) {
                const int e = threadIdx.x + 256 * q;
                if ((e >> 1) < NS * 16) L.asc[buf][e >> 1][e & 1] = sstage[q];
            }
        }
    };

    f32x4 acc[NS][FB][NW];
#pragma unroll
    for (int sb = 0; sb < NS; sb++)
#pragma unroll
        for (int fb = 0; fb < FB; fb++)
#pragma unroll
            for (int h = 0; h < NW; h++) acc[sb][fb][h] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int d = 0; d < D; d++) issue_w(d, min(d, nsteps - 1));
    load_chunk(0);
    store_chunk(0);
    __syncthreads();

    // one chunk: prefetch the next chunk into registers, run its MFMA steps from LDS buffer B,
    // then publish the prefetched chunk in the other buffer
    auto run_chunk = [&](auto Bc, int c) {
        constexpr int B = decltype(Bc)::value;
        load_chunk(min(c + 1, nchunks - 1));  // next chunk (the last one re-reads itself)
#pragma unroll
        for (int s = 0; s < CS; s++) {
            const int step = c * CS + s;
            const int slot = (B * CS + s) % D;
            if (step < nsteps) {
#pragma unroll
                for (int sb = 0; sb < NS; sb++) {
                    const uint8_t* row = &L.tok[B][sb * 16 + r16][0];
                    if constexpr (!FP8) {
                        const FT xb = lds_frag<FP8>(row + (kg * CS + s) * 16);
#pragma unroll
                        for (int fb = 0; fb < FB; fb++)
#pragma unroll
                            for (int h = 0; h < NW; h++)
                                acc[sb][fb][h] =
                                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(bw[slot][fb][h], xb, acc[sb][fb][h], 0, 0, 0);
                    } else {
                        const i32x4 lo = *(const i32x4*)(row + ((2 * kg) * CS + s) * 16);
                        const i32x4 hi = *(const i32x4*)(row + ((2 * kg + 1) * CS + s) * 16);
                        const FT xb = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        const float sa = L.asc[B][sb * 16 + r16][s];
                        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int h = 0; h < NW; h++) {
                            const float cs = L.wsc[h][step] * sa;
#pragma unroll
                            for (int fb = 0; fb < FB; fb++) {
                                const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bw[slot][fb][h], xb, zero,
                                                                                                  0, 0, 0, 0, 0, 0);
#pragma unroll
                                for (int i = 0; i < 4; i++) acc[sb][fb][h][i] = __builtin_fmaf(p[i], cs, acc[sb][fb][h][i]);
                            }
                        }
                    }
                }
            }
            issue_w(slot, min(step + D, nsteps - 1));
        }
        store_chunk(B ^ 1);
        __syncthreads();
    };
    for (int c = 0; c < nchunks; c += 2) {
        run_chunk(std::integral_constant<int, 0>{}, c);
        if (c + 1 < nchunks) run_chunk(std::integral_constant<int, 1>{}, c + 1);
    }

    // epilogue: lane holds token column sb*16 + r16, features f0 + fb*16 + kg*4 + i
#pragma unroll
    for (int sb = 0; sb < NS; sb++) {
        const int c = sb * 16 + r16;
        if (c >= m.rows) continue;
#pragma unroll
        for (int fb = 0; fb < FB; fb++) {
            const size_t o = (size_t)(m.row0 + c) * g.N + f0 + fb * 16 + kg * 4;
            float r[4];
#pragma unroll
            for (int i = 0; i < 4; i++) r[i] = GATED ? silu_mul_h(acc[sb][fb][0][i], acc[sb][fb][NW - 1][i]) : acc[sb][fb][0][i];
            if (OUT_F32) {
                *(f32x4*)((float*)g.out + o) = f32x4{r[0], r[1], r[2], r[3]};
            } else {
                uint2 pk;
                pk.x = (uint32_t)f32_to_bf16(r[0]) | ((uint32_t)f32_to_bf16(r[1]) << 16);
                pk.y = (uint32_t)f32_to_bf16(r[2]) | ((uint32_t)f32_to_bf16(r[3]) << 16);
                *(uint2*)((uint16_t*)g.out + o) = pk;
            }
        }
    }
}

template <bool GATED, bool FP8, bool OUT_F32>
__global__ __launch_bounds__(256) void k_grouped_gemm_heavy(GemmArgs g) {
    __shared__ HeavyLds L;
    const int nblocks = g.N / kHeavyFeatures;
    const int total = *g.tile_count * nblocks;
    const int nkb = g.K >> 7;
    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const int mt = tile / nblocks;
        const int nb = tile - mt * nblocks;
        const MTile m = g.mtiles[mt];
        const int nsub = (m.rows + 15) >> 4;
        const int NSr = nsub <= 4 ? 4 : (nsub <= 8 ? 8 : 16);
        if (threadIdx.x < NSr * 16) {
            const int p = m.row0 + min((int)threadIdx.x, m.rows - 1);
            L.src[threadIdx.x] = g.perm_src ? g.perm_src[p] / g.topk : p;
        }
        if constexpr (FP8) {
            // the workgroup's 128 features are one 128-row weight block
            const size_t srow = ((size_t)m.expert * (g.N >> 7) + nb) * nkb;
            for (int q = threadIdx.x; q < nkb; q += 256) {
                L.wsc[0][q] = g.S0[srow + q];
                if (GATED) L.wsc[1][q] = g.S1[srow + q];
            }
        }
        __syncthreads();
        if (nsub <= 4) {
            heavy_tile<GATED, FP8, OUT_F32, 4>(g, m, nb, L);
        } else if (nsub <= 8) {
            heavy_tile<GATED, FP8, OUT_F32, 8>(g, m, nb, L);
        } else if constexpr (GATED) {
            // 256 gate/up accumulators would not leave registers for the rest: two 128-row
            // halves, the second re-reading the tile's weights from cache
            MTile a = m, b = m;
            a.rows = 128;
            b.row0 = m.row0 + 128;
            b.rows = m.rows - 128;
            heavy_tile<GATED, FP8, OUT_F32, 8>(g, a, nb, L);
            if (threadIdx.x < 128) L.src[threadIdx.x] = L.src[128 + threadIdx.x];
            __syncthreads();
            heavy_tile<GATED, FP8, OUT_F32, 8>(g, b, nb, L);
        } else {
            heavy_tile<GATED, FP8, OUT_F32, 16>(g, m, nb, L);
        }
    }
}

template <bool GATED, bool FP8, bool OUT_F32>
hipError_t launch_heavy(const GemmArgs& a, int max_tiles, int cus, hipStream_t st) {
    static int per_cu = 0;
    if (per_cu == 0) {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_grouped_gemm_heavy<GATED, FP8, OUT_F32>, 256, 0) !=
                hipSuccess || nb < 1)
            nb = 1;
        per_cu = nb;
    }
    long long grid = (long long)max_tiles * (a.N / kHeavyFeatures);
    const long long cap = (long long)cus * per_cu;
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    k_grouped_gemm_heavy<GATED, FP8, OUT_F32><<<(unsigned)grid, 256, 0, st>>>(a);
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

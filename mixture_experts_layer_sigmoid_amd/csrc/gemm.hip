// gemm.hip -- grouped expert GEMMs on MFMA (gfx950).
//
// For each row tile (local expert l, grouped rows row0..row0+rows-1) and each block of
// output features of that expert:
//   gated (gate/up):  h[r, n] = silu(sum_k A[r,k] Wg[l,n,k]) * (sum_k A[r,k] Wu[l,n,k])
//   plain (down):     y[r, n] = sum_k A[r,k] Wd[l,n,k]
// A rows are gathered: grouped row p reads activation row perm_src[p] / top_k (the gather
// is fused into the operand load), or row p itself when no map is given.
//
// This light kernel takes row tiles of at most 32 rows (experts with few rows); heavier
// experts go to gemm_tiled.hip.
//
// Shape of the work: weights are the bytes that matter (at decode every weight byte is used
// by a handful of rows), so each wavefront streams its own 16 weight rows straight from HBM
// into registers as the MFMA "A" operand (16 rows x 8 consecutive k per lane, 16-byte
// loads), with the tokens as the MFMA "B" operand (16 tokens per 16x16 MFMA; up to BMS such
// sub-blocks per row tile reuse the weight registers).  Every wavefront keeps a ring of D
// reduction steps of operands in flight.
//
// The 4 wavefronts of a workgroup form a WN x WK grid: WN blocks of 16 output features
// (sharing the tile's activation rows), each reduced by WK wavefronts that split the
// reduction dimension and add their partial sums through LDS in a fixed order.  WK > 1 puts
// more wavefronts on each expert's weights when few experts are active (decode); WK = 1
// avoids the reduction when there are tiles enough to fill the GPU.  The host picks the
// grid from its estimate of the tile count.  Workgroups are persistent and walk the
// device-built tile list, whose length is only known on the device.
//
// FP8 (e4m3 weights with one fp32 scale per [128,128] block, activations with one fp32
// scale per row and 128 columns; "vLLM Community Traces H20 MoE ...", paragraph 2, and
// "Lab notes #6 ...", intro): one v_mfma_f32_16x16x128_f8f6f4 covers exactly one 128-deep
// scale block, so each block's exact-scale partial product is added to the fp32
// accumulator times (weight scale * activation scale).  The scales are arbitrary fp32, so
// the power-of-two-scaled MX form of the instruction is not used.  The tile's scales are
// staged in LDS first, so the ring of operand loads is not held up by small scale loads.
#include "launch.hpp"

namespace fmoe {


__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// MFMA operand fragment of one lane: 8 bf16 (16x16x32) or 32 e4m3 codes (16x16x128),
// consecutive along the reduction dimension.
template <bool FP8>
struct Frag {
    using T = bf16x8;
    static constexpr int KSTEP = 32;  // reduction depth of one MFMA
    static constexpr int LANE_K = 8;  // consecutive elements per lane
    static constexpr int REGS = 4;
    static constexpr int EB = 2;  // bytes per element
};
template <>
struct Frag<true> {
    using T = i32x8;
    static constexpr int KSTEP = 128;
    static constexpr int LANE_K = 32;
    static constexpr int REGS = 8;
    static constexpr int EB = 1;
};

template <bool FP8>
__device__ __forceinline__ typename Frag<FP8>::T load_frag(const void* base, size_t elem) {
    if constexpr (FP8) return *(const i32x8*)((const uint8_t*)base + elem);
    else return *(const bf16x8*)((const uint16_t*)base + elem);
}

// Bytes of dynamic LDS of one workgroup: FP8 weight-scale rows (gate/up) and the tile's
// activation scales.
size_t gemm_lds_bytes(bool fp8, int K, int tile_rows) {
    if (!fp8) return 0;
    const size_t nkb = (size_t)K / 128;
    return (2 * nkb + (size_t)tile_rows * nkb) * sizeof(float);
}

// One row tile: wavefront (wn, wk) computes 16 output features n0..n0+15 over its share of
// the reduction; NS = active 16-row sub-blocks (compile time, so the reduction loop has no
// per-step branches).
//
// LINE: weights by whole 128-byte lines, as in the streaming kernel (gemm_stream.hip): two
// non-temporal loads, one of rows 0-7 and one of rows 8-15 of the wavefront's 16, each
// giving a lower-half lane (r16 < 8) one piece of its own row and an upper-half lane one
// piece of the row 8 away; a select per dword and a rotation by 8 lanes within each 16-lane
// row put the MFMA's own pieces back in its lanes.  A line holds two bf16 reduction steps, so
// a wavefront's share of the reduction must start and end on even steps.
template <bool GATED, bool FP8, bool OUT_F32, int NS, int BMS, int WN, int WK, bool LINE>
__device__ __forceinline__ void tile_body(const GemmArgs& g, const MTile& m, int n0, int wn, int wk, float* red,
                                          const float* wsc, const float* asc) {
    using F = Frag<FP8>;
    using FT = typename F::T;
    constexpr int NW = GATED ? 2 : 1;
    constexpr int RING = 96 / ((NW + NS) * F::REGS);
    constexpr int D = RING < 1 ? 1 : (RING > 8 ? 8 : RING);
    const int lane = lane_id();
    const int r16 = lane & 15, kg = lane >> 4;

    const int nsteps = g.K / F::KSTEP;
    const int s0 = wk * nsteps / WK;
    const int n = (wk + 1) * nsteps / WK - s0;
    const int nkb = g.K >> 7;
    const bool lower = r16 < 8;
    // with LINE: the lane's load-A row and piece (an upper-half lane takes the second step's
    // piece, F::KSTEP elements on), and the distance to its load-B piece, in elements
    const size_t wrow = LINE ? ((size_t)m.expert * g.N + n0 + (r16 & 7)) * g.K + kg * F::LANE_K +
                                   (lower ? 0 : F::KSTEP) + (size_t)s0 * F::KSTEP
                             : ((size_t)m.expert * g.N + n0 + r16) * g.K + kg * F::LANE_K + (size_t)s0 * F::KSTEP;
    const long long lane_ab = 8 * (long long)g.K + (lower ? F::KSTEP : -F::KSTEP);

    static_assert(!(LINE && FP8), "whole-line loads: bf16 weights");
    constexpr int PAIR = LINE ? 2 : 1;
    static_assert(D % PAIR == 0, "the ring holds whole lines");
    FT bw0[D], bw1[D], bx[D][NS];
    float bsa[D][NS], bsw0[D], bsw1[D];
    // with LINE, slot pairs (s, s+1) load when their second step is issued
    auto issue_w = [&](int slot, int step) {
        if constexpr (!LINE) {
            bw0[slot] = load_frag<FP8>(g.W0, wrow + (size_t)step * F::KSTEP);
            if constexpr (GATED) bw1[slot] = load_frag<FP8>(g.W1, wrow + (size_t)step * F::KSTEP);
        } else {
            if (slot % PAIR != PAIR - 1) return;
            const size_t e = wrow + (size_t)(step - (PAIR - 1)) * F::KSTEP;
            auto two = [&](const void* W, FT* bw) {
                const uint8_t* p = (const uint8_t*)W + e * F::EB;
                bw[slot - 1] = __builtin_bit_cast(FT, __builtin_nontemporal_load((const i32x4*)p));
                bw[slot] = __builtin_bit_cast(FT, __builtin_nontemporal_load((const i32x4*)(p + lane_ab * F::EB)));
            };
            two(g.W0, bw0);
            if constexpr (GATED) two(g.W1, bw1);
        }
    };
    // loads A, B of a line into pieces X = lower ? A : B and Y = (lower ? B : A) rotated by 8
    // lanes within each 16-lane row (row_ror:8)
    auto regroup = [&](i32x4& a, i32x4& b) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int x = lower ? a[i] : b[i];
            const int z = lower ? b[i] : a[i];
            a[i] = x;
            b[i] = __builtin_amdgcn_update_dpp(0, z, 0x128, 0xf, 0xf, false);
        }
    };
    size_t xoff[NS];
    auto gather_rows = [&]() {
#pragma unroll
        for (int sb = 0; sb < NS; sb++) {
            const int p = m.row0 + min(sb * 16 + r16, m.rows - 1);
            const int src = g.perm_src ? g.perm_src[p] / g.topk : p;
            xoff[sb] = (size_t)src * g.K + kg * F::LANE_K + (size_t)s0 * F::KSTEP;
        }
    };
    auto issue_x = [&](int slot, int step) {
#pragma unroll
        for (int sb = 0; sb < NS; sb++) bx[slot][sb] = load_frag<FP8>(g.A, xoff[sb] + (size_t)step * F::KSTEP);
        if constexpr (FP8) {
            bsw0[slot] = wsc[s0 + step];
            if constexpr (GATED) bsw1[slot] = wsc[nkb + s0 + step];
#pragma unroll
            for (int sb = 0; sb < NS; sb++) bsa[slot][sb] = asc[(sb * 16 + r16) * nkb + s0 + step];
        }
    };

    f32x4 acc0[NS], acc1[NS];
#pragma unroll
    for (int sb = 0; sb < NS; sb++) {
        acc0[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc1[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // one reduction step on weight fragments w0 (w1) with the slot's activations
    auto mfma_step = [&](int slot, const FT& w0, const FT& w1) {
#pragma unroll
        for (int sb = 0; sb < NS; sb++) {
            if constexpr (!FP8) {
                acc0[sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, bx[slot][sb], acc0[sb], 0, 0, 0);
                if constexpr (GATED)
                    acc1[sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, bx[slot][sb], acc1[sb], 0, 0, 0);
            } else {
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                const f32x4 p0 =
                    __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w0, bx[slot][sb], zero, 0, 0, 0, 0, 0, 0);
                const float c0 = bsw0[slot] * bsa[slot][sb];
#pragma unroll
                for (int i = 0; i < 4; i++) acc0[sb][i] = __builtin_fmaf(p0[i], c0, acc0[sb][i]);
                if constexpr (GATED) {
                    const f32x4 p1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w1, bx[slot][sb], zero,
                                                                                       0, 0, 0, 0, 0, 0);
                    const float c1 = bsw1[slot] * bsa[slot][sb];
#pragma unroll
                    for (int i = 0; i < 4; i++) acc1[sb][i] = __builtin_fmaf(p1[i], c1, acc1[sb][i]);
                }
            }
        }
    };
    // step `slot`; with LINE the even slot of a pair runs both of its steps (in order) from
    // regrouped copies and the odd slot nothing, so no regrouped value has to outlive a branch
    // of the loop's tail
    auto compute = [&](int slot) {
        if constexpr (!LINE) {
            mfma_step(slot, bw0[slot], bw1[slot]);
        } else if (slot % 2 == 0) {
            i32x4 x[2], y[2];
#pragma unroll
            for (int h = 0; h < NW; h++) {
                x[h] = __builtin_bit_cast(i32x4, h ? bw1[slot] : bw0[slot]);
                y[h] = __builtin_bit_cast(i32x4, h ? bw1[slot + 1] : bw0[slot + 1]);
                regroup(x[h], y[h]);
            }
            mfma_step(slot, __builtin_bit_cast(FT, x[0]), __builtin_bit_cast(FT, x[NW - 1]));
            mfma_step(slot + 1, __builtin_bit_cast(FT, y[0]), __builtin_bit_cast(FT, y[NW - 1]));
        }
    };

    if (n >= D) {
        // Pipelined: the weight prologue goes first (its addresses do not depend on the gather
        // map), all D ring slots load unconditionally so the loop starts from a known number
        // of loads in flight, and every steady-state step computes one slot and refills it D
        // steps ahead with no branches.
#pragma unroll
        for (int d = 0; d < D; d++) issue_w(d, d);
        gather_rows();
#pragma unroll
        for (int d = 0; d < D; d++) issue_x(d, d);
        int base = 0;
        for (; base + 2 * D <= n; base += D) {
#pragma unroll
            for (int d = 0; d < D; d++) {
                compute(d);
                issue_w(d, base + d + D);
                issue_x(d, base + d + D);
            }
        }
        // tail: fewer than 2*D steps left
#pragma unroll
        for (int d = 0; d < D; d++) {
            if (base + d < n) {
                compute(d);
                if (base + d + D < n) {
                    issue_w(d, base + d + D);
                    issue_x(d, base + d + D);
                }
            }
        }
#pragma unroll
        for (int d = 0; d < D; d++)
            if (base + D + d < n) compute(d);
    } else {
        // Short share of the reduction (fewer steps than ring slots, possibly none): load all
        // of it, then compute.
#pragma unroll
        for (int d = 0; d < D; d++)
            if (d < n) issue_w(d, d);
        gather_rows();
#pragma unroll
        for (int d = 0; d < D; d++)
            if (d < n) issue_x(d, d);
#pragma unroll
        for (int d = 0; d < D; d++)
            if (d < n) compute(d);
    }

    // Epilogue: lane holds token column sb*16 + r16 and features n0 + 4*kg + i.
    auto store = [&](int sb, const f32x4& v0, const f32x4& v1) {
        const int c = sb * 16 + r16;
        if (c >= m.rows) return;
        const size_t o = (size_t)(m.row0 + c) * g.N + n0 + kg * 4;
        float r[4];
#pragma unroll
        for (int i = 0; i < 4; i++) r[i] = GATED ? silu_mul(v0[i], v1[i]) : v0[i];
        if (OUT_F32) {
            *(f32x4*)((float*)g.out + o) = f32x4{r[0], r[1], r[2], r[3]};
        } else {
            uint2 pk;
            pk.x = (uint32_t)f32_to_bf16(r[0]) | ((uint32_t)f32_to_bf16(r[1]) << 16);
            pk.y = (uint32_t)f32_to_bf16(r[2]) | ((uint32_t)f32_to_bf16(r[3]) << 16);
            *(uint2*)((uint16_t*)g.out + o) = pk;
        }
    };

    if constexpr (WK > 1) {
        // partial sums through LDS, added in wavefront order (fixed, so results are reproducible)
        auto at = [&](int k, int sb, int h, int i) { return ((((k * WN + wn) * BMS + sb) * NW + h) * 4 + i) * 64 + lane; };
#pragma unroll
        for (int sb = 0; sb < NS; sb++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                red[at(wk, sb, 0, i)] = acc0[sb][i];
                if (GATED) red[at(wk, sb, NW - 1, i)] = acc1[sb][i];
            }
        __syncthreads();
        for (int sb = wk; sb < NS; sb += WK) {
            f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < WK; q++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    v0[i] += red[at(q, sb, 0, i)];
                    if (GATED) v1[i] += red[at(q, sb, NW - 1, i)];
                }
            store(sb, v0, v1);
        }
    } else {
#pragma unroll
        for (int sb = 0; sb < NS; sb++) store(sb, acc0[sb], acc1[sb]);
    }
}

// Persistent workgroups walk the tiles (row tile x 16*WN features) of the device-built list.
template <bool GATED, bool FP8, bool OUT_F32, int BMS, int WN, int WK, bool LINE>
__global__ __launch_bounds__(256) void k_grouped_gemm(GemmArgs g) {
    static_assert(WN * WK == 4, "four wavefronts per workgroup");
    constexpr int NW = GATED ? 2 : 1;
    __shared__ float red[WK > 1 ? WK * WN * BMS * NW * 256 : 1];
    extern __shared__ float dyn[];
    const int w = uniform(threadIdx.x >> 6);
    const int wn = w % WN, wk = w / WN;
    const int nblocks = g.N / (16 * WN);
    const int total = *g.tile_count * nblocks;
    const int nkb = g.K >> 7;
    float* wsc = dyn;             // FP8: [2][nkb] gate/up weight-block scales of the tile
    float* asc = dyn + 2 * nkb;   // FP8: [16*BMS][nkb] activation scales of the tile rows
    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const int mt = tile / nblocks;
        const int nb = tile - mt * nblocks;
        const MTile m = g.mtiles[mt];
        const int nsub = (m.rows + 15) >> 4;
        if constexpr (FP8) {
            // all 16*WN rows of the tile sit in one 128-row weight block (16*WN divides 128)
            const size_t srow = ((size_t)m.expert * (g.N >> 7) + ((nb * 16 * WN) >> 7)) * nkb;
            for (int q = threadIdx.x; q < nkb; q += 256) {
                wsc[q] = g.S0[srow + q];
                if (GATED) wsc[nkb + q] = g.S1[srow + q];
            }
            const int rows_pad = min(BMS, nsub <= 1 ? 1 : nsub <= 2 ? 2 : nsub <= 4 ? 4 : 8) * 16;
            for (int q = threadIdx.x; q < rows_pad * nkb; q += 256) {
                const int r = q / nkb, kb = q - r * nkb;
                const int p = m.row0 + min(r, m.rows - 1);
                const int src = g.perm_src ? g.perm_src[p] / g.topk : p;
                asc[q] = g.A_scale[(size_t)src * nkb + kb];
            }
            __syncthreads();
        }
        const int n0 = nb * 16 * WN + wn * 16;
        // active sub-blocks rounded up to a power of two (extra columns repeat the last row
        // and are not stored)
        if (nsub <= 1 || BMS == 1) tile_body<GATED, FP8, OUT_F32, 1, BMS, WN, WK, LINE>(g, m, n0, wn, wk, red, wsc, asc);
        else if (nsub <= 2 || BMS == 2)
            tile_body<GATED, FP8, OUT_F32, (BMS >= 2 ? 2 : 1), BMS, WN, WK, LINE>(g, m, n0, wn, wk, red, wsc, asc);
        else if (nsub <= 4 || BMS == 4)
            tile_body<GATED, FP8, OUT_F32, (BMS >= 4 ? 4 : 1), BMS, WN, WK, LINE>(g, m, n0, wn, wk, red, wsc, asc);
        else tile_body<GATED, FP8, OUT_F32, (BMS >= 8 ? 8 : 1), BMS, WN, WK, LINE>(g, m, n0, wn, wk, red, wsc, asc);
        if (WK > 1 || FP8) __syncthreads();  // LDS is refilled by the next tile
    }
}

// Persistent grid: the number of workgroups that fit on the GPU at once (occupancy query,
// cached per instantiation and LDS size), at most the tile bound.
template <bool GATED, bool FP8, bool OUT_F32, int BMS, int WN, int WK, bool LINE>
static hipError_t launch_grid(const GemmArgs& a, int max_tiles, int cus, hipStream_t st) {
    const size_t lds = gemm_lds_bytes(FP8, a.K, 16 * BMS);
    static int per_cu = 0;
    static size_t per_cu_lds = 0;
    if (per_cu == 0 || per_cu_lds != lds) {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_grouped_gemm<GATED, FP8, OUT_F32, BMS, WN, WK, LINE>,
                                                          256, lds) != hipSuccess || nb < 1)
            nb = 1;
        per_cu = nb;
        per_cu_lds = lds;
    }
    long long grid = (long long)max_tiles * (a.N / (16 * WN));
    const long long cap = (long long)cus * per_cu;
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    k_grouped_gemm<GATED, FP8, OUT_F32, BMS, WN, WK, LINE><<<(unsigned)grid, 256, lds, st>>>(a);
    return hipGetLastError();
}

// Weight load form: whole lines for bf16 weights, per step for FP8 (there the rearrangement
// needs more registers than the split kernel's rings leave: the FP8 down GEMM went from 3 to 1
// wavefronts per SIMD and measured slower), and per step for a bf16 reduction whose four shares
// would not all start on an even step (K a multiple of 128 but not 256); splits of 1 and 2
// always do.
template <bool GATED, bool FP8, bool OUT_F32, int BMS, int WN, int WK>
static hipError_t launch_shape(const GemmArgs& a, int max_tiles, int cus, hipStream_t st) {
    if constexpr (FP8) {
        return launch_grid<GATED, FP8, OUT_F32, BMS, WN, WK, false>(a, max_tiles, cus, st);
    } else if constexpr (WK < 4) {
        return launch_grid<GATED, FP8, OUT_F32, BMS, WN, WK, true>(a, max_tiles, cus, st);
    } else {
        if ((a.K / Frag<FP8>::KSTEP) % (2 * WK) == 0)
            return launch_grid<GATED, FP8, OUT_F32, BMS, WN, WK, true>(a, max_tiles, cus, st);
        return launch_grid<GATED, FP8, OUT_F32, BMS, WN, WK, false>(a, max_tiles, cus, st);
    }
}

template <bool GATED, bool FP8, bool OUT_F32, int BMS>
static hipError_t launch_bms(const GemmArgs& a, int wk, int max_tiles, int cus, hipStream_t st) {
    if constexpr (BMS <= 2) {
        if (wk == 4) return launch_shape<GATED, FP8, OUT_F32, BMS, 1, 4>(a, max_tiles, cus, st);
        if (wk == 2) return launch_shape<GATED, FP8, OUT_F32, BMS, 2, 2>(a, max_tiles, cus, st);
    }
    return launch_shape<GATED, FP8, OUT_F32, BMS, 4, 1>(a, max_tiles, cus, st);
}

template <bool GATED, bool FP8, bool OUT_F32>
static hipError_t launch_kind(const GemmArgs& a, int tile_rows, int wk, int max_tiles, int cus, hipStream_t st) {
    switch (tile_rows) {
        case 16: return launch_bms<GATED, FP8, OUT_F32, 1>(a, wk, max_tiles, cus, st);
        case 32: return launch_bms<GATED, FP8, OUT_F32, 2>(a, wk, max_tiles, cus, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_grouped_gemm(bool gated, bool fp8, bool out_f32, const GemmArgs& a, int tile_rows, int wk,
                               int max_tiles, int cus, hipStream_t st) {
    if (gated) {
        if (fp8) return out_f32 ? launch_kind<true, true, true>(a, tile_rows, wk, max_tiles, cus, st)
                                : launch_kind<true, true, false>(a, tile_rows, wk, max_tiles, cus, st);
        return launch_kind<true, false, false>(a, tile_rows, wk, max_tiles, cus, st);
    }
    if (fp8) return launch_kind<false, true, false>(a, tile_rows, wk, max_tiles, cus, st);
    return launch_kind<false, false, false>(a, tile_rows, wk, max_tiles, cus, st);
}

}  // namespace fmoe

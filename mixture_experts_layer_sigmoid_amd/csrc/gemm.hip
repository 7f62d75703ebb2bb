// gemm.hip -- grouped expert GEMMs on MFMA (gfx950).
//
// For each row tile (local expert l, grouped rows row0..row0+rows-1) and each block of 16
// output features n0..n0+15 of that expert:
//   gated (gate/up):  h[r, n] = silu(sum_k A[r,k] Wg[l,n,k]) * (sum_k A[r,k] Wu[l,n,k])
//   plain (down):     y[r, n] = sum_k A[r,k] Wd[l,n,k]
// A rows are gathered: grouped row p reads activation row perm_src[p] / top_k (the gather
// is fused into the operand load), or row p itself when no map is given.
//
// Shape of the work: weights are the bytes that matter (at decode every weight byte is used
// by a handful of rows), so each wavefront streams its own 16 weight rows straight from HBM
// into registers as the MFMA "A" operand (16 rows x 8 consecutive k per lane, 16-byte
// loads), and the tokens are the MFMA "B" operand (16 tokens per 16x16 MFMA, up to BMS such
// sub-blocks per tile reuse the weight registers).  The KSPLIT wavefronts of a workgroup
// split the reduction dimension and add their partial sums through LDS in a fixed order
// before the epilogue, so more wavefronts stream weights when few experts are active.
// Workgroups are persistent and walk the device-built tile list, whose length is only
// known on the device (the tile list is cut from the real per-expert counts).
//
// FP8 (e4m3 weights with one fp32 scale per [128,128] block, activations with one fp32
// scale per row and 128 columns; "vLLM Community Traces H20 MoE ...", paragraph 2, and
// "Lab notes #6 ...", intro): one v_mfma_f32_16x16x128_f8f6f4 covers exactly one 128-deep
// scale block, so each block's exact-scale partial product is added to the fp32
// accumulator times (weight scale * activation scale).  The scales are arbitrary fp32, so
// the power-of-two-scaled MX form of the instruction is not used.
#include "launch.hpp"

namespace fmoe {


__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

template <bool GATED, bool FP8, bool OUT_F32, int BMS, int KSPLIT>
__global__ __launch_bounds__(64 * KSPLIT) void k_grouped_gemm(GemmArgs g) {
    constexpr int NW = GATED ? 2 : 1;
    __shared__ float red[KSPLIT > 1 ? KSPLIT : 1][BMS][NW][4][64];
    const int lane = lane_id(), w = threadIdx.x >> 6;
    const int r16 = lane & 15, kg = lane >> 4;
    const int nblocks = g.N >> 4;
    const int total = g.hdr->m_tiles * nblocks;

    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const int mt = tile / nblocks, nb = tile - mt * nblocks;
        const MTile m = g.mtiles[mt];
        const int nsub = (m.rows + 15) >> 4;
        const int n0 = nb << 4;

        int src[BMS];
#pragma unroll
        for (int sb = 0; sb < BMS; sb++) {
            const int p = m.row0 + min(sb * 16 + r16, m.rows - 1);
            src[sb] = g.perm_src ? g.perm_src[p] / g.topk : p;
        }

        f32x4 acc0[BMS], acc1[BMS];
#pragma unroll
        for (int sb = 0; sb < BMS; sb++) {
            acc0[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc1[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

        if constexpr (!FP8) {
            const size_t wrow = ((size_t)m.expert * g.N + n0 + r16) * g.K + kg * 8;
            const uint16_t* w0 = (const uint16_t*)g.W0 + wrow;
            const uint16_t* w1 = GATED ? (const uint16_t*)g.W1 + wrow : w0;
            const uint16_t* a = (const uint16_t*)g.A + kg * 8;
            const int nsteps = g.K >> 5;
            const int s0 = w * nsteps / KSPLIT, s1 = (w + 1) * nsteps / KSPLIT;
#pragma unroll 4
            for (int s = s0; s < s1; s++) {
                const bf16x8 wa0 = *(const bf16x8*)(w0 + s * 32);
                bf16x8 wa1;
                if (GATED) wa1 = *(const bf16x8*)(w1 + s * 32);
#pragma unroll
                for (int sb = 0; sb < BMS; sb++) {
                    if (sb < nsub) {
                        const bf16x8 xb = *(const bf16x8*)(a + (size_t)src[sb] * g.K + s * 32);
                        acc0[sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa0, xb, acc0[sb], 0, 0, 0);
                        if (GATED) acc1[sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa1, xb, acc1[sb], 0, 0, 0);
                    }
                }
            }
        } else {
            const int nkb = g.K >> 7;
            const size_t wrow = ((size_t)m.expert * g.N + n0 + r16) * g.K + kg * 32;
            const uint8_t* w0 = (const uint8_t*)g.W0 + wrow;
            const uint8_t* w1 = GATED ? (const uint8_t*)g.W1 + wrow : w0;
            const size_t srow = ((size_t)m.expert * (g.N >> 7) + (n0 >> 7)) * nkb;
            const float* sw0 = g.S0 + srow;
            const float* sw1 = GATED ? g.S1 + srow : sw0;
            const uint8_t* a = (const uint8_t*)g.A + kg * 32;
            const int kb0 = w * nkb / KSPLIT, kb1 = (w + 1) * nkb / KSPLIT;
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
            for (int kb = kb0; kb < kb1; kb++) {
                const i32x8 wa0 = *(const i32x8*)(w0 + kb * 128);
                i32x8 wa1;
                if (GATED) wa1 = *(const i32x8*)(w1 + kb * 128);
                const float s_w0 = sw0[kb];
                const float s_w1 = GATED ? sw1[kb] : 0.0f;
#pragma unroll
                for (int sb = 0; sb < BMS; sb++) {
                    if (sb < nsub) {
                        const i32x8 xb = *(const i32x8*)(a + (size_t)src[sb] * g.K + kb * 128);
                        const float s_a = g.A_scale[(size_t)src[sb] * nkb + kb];
                        const f32x4 p0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa0, xb, zero, 0, 0, 0, 0, 0, 0);
                        const float c0 = s_w0 * s_a;
#pragma unroll
                        for (int i = 0; i < 4; i++) acc0[sb][i] = __builtin_fmaf(p0[i], c0, acc0[sb][i]);
                        if (GATED) {
                            const f32x4 p1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa1, xb, zero, 0, 0, 0, 0, 0, 0);
                            const float c1 = s_w1 * s_a;
#pragma unroll
                            for (int i = 0; i < 4; i++) acc1[sb][i] = __builtin_fmaf(p1[i], c1, acc1[sb][i]);
                        }
                    }
                }
            }
        }

        // Epilogue for sub-block sb: lane holds token column sb*16 + r16 and features n0 + 4*kg + i.
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

        if constexpr (KSPLIT > 1) {
#pragma unroll
            for (int sb = 0; sb < BMS; sb++) {
                if (sb < nsub) {
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        red[w][sb][0][i][lane] = acc0[sb][i];
                        if (GATED) red[w][sb][NW - 1][i][lane] = acc1[sb][i];
                    }
                }
            }
            __syncthreads();
            for (int sb = w; sb < nsub; sb += KSPLIT) {
                f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
                for (int q = 0; q < KSPLIT; q++) {
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        v0[i] += red[q][sb][0][i][lane];
                        if (GATED) v1[i] += red[q][sb][NW - 1][i][lane];
                    }
                }
                store(sb, v0, v1);
            }
            __syncthreads();
        } else {
#pragma unroll
            for (int sb = 0; sb < BMS; sb++)
                if (sb < nsub) store(sb, acc0[sb], acc1[sb]);
        }
    }
}

// Launch shapes: KSPLIT wavefronts per workgroup for small row tiles (few rows, so more
// wavefronts share each weight block), one for large tiles.
template <bool GATED, bool FP8, bool OUT_F32, int BMS>
static hipError_t launch_bms(const GemmArgs& a, int max_tiles, int cus, hipStream_t st) {
    constexpr int KSPLIT = BMS <= 2 ? 4 : 1;
    constexpr int per_cu = KSPLIT == 4 ? 8 : 16;
    long long grid = (long long)max_tiles * (a.N >> 4);
    const long long cap = (long long)cus * per_cu;
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    k_grouped_gemm<GATED, FP8, OUT_F32, BMS, KSPLIT><<<(unsigned)grid, 64 * KSPLIT, 0, st>>>(a);
    return hipGetLastError();
}

template <bool GATED, bool FP8, bool OUT_F32>
static hipError_t launch_kind(const GemmArgs& a, int tile_rows, int max_tiles, int cus, hipStream_t st) {
    switch (tile_rows) {
        case 16: return launch_bms<GATED, FP8, OUT_F32, 1>(a, max_tiles, cus, st);
        case 32: return launch_bms<GATED, FP8, OUT_F32, 2>(a, max_tiles, cus, st);
        case 64: return launch_bms<GATED, FP8, OUT_F32, 4>(a, max_tiles, cus, st);
        case 128: return launch_bms<GATED, FP8, OUT_F32, 8>(a, max_tiles, cus, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_grouped_gemm(bool gated, bool fp8, bool out_f32, const GemmArgs& a, int tile_rows, int max_tiles,
                               int cus, hipStream_t st) {
    if (gated) {
        if (fp8) return out_f32 ? launch_kind<true, true, true>(a, tile_rows, max_tiles, cus, st)
                                : launch_kind<true, true, false>(a, tile_rows, max_tiles, cus, st);
        return launch_kind<true, false, false>(a, tile_rows, max_tiles, cus, st);
    }
    if (fp8) return launch_kind<false, true, false>(a, tile_rows, max_tiles, cus, st);
    return launch_kind<false, false, false>(a, tile_rows, max_tiles, cus, st);
}

}  // namespace fmoe

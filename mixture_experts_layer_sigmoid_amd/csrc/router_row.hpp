// router_row.hpp -- top-k routing of one token row by one 64-lane wavefront (device code
// shared by the router kernel and the fused router + grouping kernel).
//
// Top-k follows "PR #39593: [Bug]: Fix FlashInfer CUTLASS BF16 + CUDA graphs IMA", Fix:
// a NaN logit is replaced by -FLT_MAX in registers right after the load, before scoring
// and selection, so an all-NaN row still yields k distinct ids (0..k-1) instead of the
// same id k times.  The row sits in registers (expert e in lane e%64, slot e/64), each of
// the k rounds is a 64-bit max-reduction across the wavefront, and the picked lane retires
// its slot, so ids are distinct by construction.
//
// Grouped (group-limited) top-k: the pages name it beside the plain router without defining
// it; the reading taken: experts form n_group groups of consecutive indices, a group's key is
// its best expert key (largest sanitised logit, and among equal values the lower expert, so
// the lower group), the topk_group best groups are kept, and the plain k rounds then run over
// the kept groups' experts only.  One max-reduction per group, one per kept group, and the
// dropped groups' slots are retired before the k rounds.
#pragma once

#include <float.h>

#include "common.hpp"

namespace fmoe {

// Sanitised logit: NaN -> -FLT_MAX, +-inf -> +-FLT_MAX, -0 -> +0 (so equal values compare
// equal as keys).
__device__ __forceinline__ float sanitize(float v) {
    if (v != v) return -FLT_MAX;
    v = fminf(fmaxf(v, -FLT_MAX), FLT_MAX);
    return v == 0.0f ? 0.0f : v;
}

// Order-preserving map of a finite float to an unsigned key.
__device__ __forceinline__ uint32_t float_key(float v) {
    uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_float(uint32_t kb) {
    return __uint_as_float((kb & 0x80000000u) ? (kb & 0x7fffffffu) : ~kb);
}

// One step of the key max: each lane takes the larger of its key and the key the DPP control
// CTRL brings it from another lane (lanes whose source is outside the row, or whose row is not
// in ROWS, keep their own).
template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned long long key_max_step(unsigned long long v) {
    const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
    const uint32_t nlo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWS, 0xf, false);
    const uint32_t nhi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWS, 0xf, false);
    const unsigned long long n = ((unsigned long long)nhi << 32) | nlo;
    return n > v ? n : v;
}

// Largest 64-bit key of the wavefront, in every lane.  Row shifts by 1, 2, 4 and 8 leave each
// 16-lane row's maximum in its lane 15 (a max-scan: taking a key twice does not matter), the
// row broadcasts of lanes 15 and 31 carry it into the later rows, and lane 63 ends with the
// maximum of all 64 lanes, which is then read as a uniform value.  Everything runs on the
// vector ALU; a shuffle through the LDS crossbar per step would cost a round trip each.
__device__ __forceinline__ unsigned long long wave_max_key(unsigned long long v) {
    v = key_max_step<0x111, 0xf>(v);  // row_shr:1
    v = key_max_step<0x112, 0xf>(v);  // row_shr:2
    v = key_max_step<0x114, 0xf>(v);  // row_shr:4
    v = key_max_step<0x118, 0xf>(v);  // row_shr:8
    v = key_max_step<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v = key_max_step<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return ((unsigned long long)hi << 32) | lo;
}

// Token t by the calling wavefront: ids [*,k] and weights [*,k] of row t; also the ids into
// ids_lds[0..k) when ids_lds is not null.
template <int SLOTS, bool BF16_IN>
__device__ __forceinline__ void topk_row(const void* __restrict__ logits, int t, int E, int k, int scoring,
                                         int renorm, int n_group, int topk_group, int32_t* __restrict__ ids,
                                         float* __restrict__ weights, int32_t* ids_lds) {
    const int lane = lane_id();

    float v[SLOTS];
    unsigned long long key[SLOTS];
#pragma unroll
    for (int s = 0; s < SLOTS; s++) {
        int e = lane + 64 * s;
        float raw = -FLT_MAX;
        if (e < E) {
            if (BF16_IN) raw = bf16_to_f32(((const uint16_t*)logits)[(size_t)t * E + e]);
            else raw = ((const float*)logits)[(size_t)t * E + e];
        }
        v[s] = sanitize(raw);
        // key: value first, then the lower index; 0 marks a slot that cannot be picked
        key[s] = (e < E) ? (((unsigned long long)float_key(v[s]) << 32) | (uint32_t)(0xffffffffu - (uint32_t)e)) : 0ull;
    }

    if (topk_group < n_group) {  // grouped: retire the slots of the groups not kept
        const int gsz = E / n_group;
        int grp[SLOTS];
#pragma unroll
        for (int s = 0; s < SLOTS; s++) grp[s] = (lane + 64 * s < E) ? (lane + 64 * s) / gsz : 0;  // past E: key 0
        unsigned long long gk = 0ull;  // lane g < n_group holds the key of group g
        for (int g = 0; g < n_group; g++) {
            unsigned long long b = 0ull;
#pragma unroll
            for (int s = 0; s < SLOTS; s++) b = (grp[s] == g && key[s] > b) ? key[s] : b;
            b = wave_max_key(b);
            if (lane == g) gk = b;
        }
        unsigned long long kept = 0ull;  // bit g: group g kept
        for (int j = 0; j < topk_group; j++) {
            const unsigned long long b = wave_max_key(gk);  // group keys are distinct (distinct experts)
            const int g = __ffsll((long long)__ballot(gk == b && b != 0ull)) - 1;
            kept |= 1ull << g;
            if (lane == g) gk = 0ull;
        }
#pragma unroll
        for (int s = 0; s < SLOTS; s++)
            if (!((kept >> grp[s]) & 1ull)) key[s] = 0ull;
    }

    float my_v = -FLT_MAX;  // lane j < k keeps the value of pick j
    int my_id = 0;
    for (int j = 0; j < k; j++) {
        unsigned long long best = key[0];
#pragma unroll
        for (int s = 1; s < SLOTS; s++) best = key[s] > best ? key[s] : best;
        best = wave_max_key(best);
        const int e = (int)(0xffffffffu - (uint32_t)(best & 0xffffffffu));
        const float val = key_float((uint32_t)(best >> 32));
        if (lane == j) { my_v = val; my_id = e; }
#pragma unroll
        for (int s = 0; s < SLOTS; s++)
            if (lane + 64 * s == e) key[s] = 0ull;
    }

    const float m = __shfl(my_v, 0, 64);  // the first pick holds the row maximum (its group is kept)
    float w = 0.0f;
    if (scoring == 0) {
        float ex = (lane < k) ? expf(my_v - m) : 0.0f;
        float denom;
        if (renorm) {
            denom = wave_sum(ex);
        } else {
            float part = 0.0f;
#pragma unroll
            for (int s = 0; s < SLOTS; s++)
                if (lane + 64 * s < E) part += expf(v[s] - m);
            denom = wave_sum(part);
        }
        w = ex / denom;
    } else {
        float sg = (lane < k) ? 1.0f / (1.0f + expf(-my_v)) : 0.0f;
        if (renorm) {
            float sum = wave_sum(sg);
            w = (sum > 0.0f) ? sg / sum : 1.0f / (float)k;
        } else {
            w = sg;
        }
    }
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_id;
        weights[(size_t)t * k + lane] = w;
        if (ids_lds) ids_lds[lane] = my_id;
    }
}

}  // namespace fmoe

// combine.hip -- routing-weighted combine of the expert outputs back to token order:
//   out[t,:] = sum over j ascending, inv_perm[t*k+j] >= 0, of w[t,j] * Y[inv_perm[t*k+j],:]
// fp32 fused multiply-adds in that fixed order, one bf16 rounding at the end; a token with
// no local row gets zeros.  One workgroup per token, 8 bf16 (16 bytes) per lane per pass.
#include "launch.hpp"

namespace fmoe {

// The rows of a token are taken 8 at a time: their positions and weights are loaded together,
// then their 16-byte pieces, and only then added in j order, so a token waits for two memory
// round trips per 8 rows rather than two per row.
constexpr int kCombineBatch = 8;

__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ Y, const int32_t* __restrict__ inv_perm,
                                                 const float* __restrict__ w, int k, int H,
                                                 uint16_t* __restrict__ out) {
    const int t = blockIdx.x;
    for (int h0 = threadIdx.x * 8; h0 < H; h0 += 256 * 8) {
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; q++) acc[q] = 0.0f;
        for (int j0 = 0; j0 < k; j0 += kCombineBatch) {
            int p[kCombineBatch];
            float wt[kCombineBatch];
#pragma unroll
            for (int b = 0; b < kCombineBatch; b++) {
                const bool in = j0 + b < k;
                p[b] = in ? inv_perm[(size_t)t * k + j0 + b] : -1;
                wt[b] = in ? w[(size_t)t * k + j0 + b] : 0.0f;
            }
            i32x4 v[kCombineBatch];
#pragma unroll
            for (int b = 0; b < kCombineBatch; b++)
                v[b] = p[b] >= 0 ? *(const i32x4*)(Y + (size_t)p[b] * H + h0) : i32x4{0, 0, 0, 0};
#pragma unroll
            for (int b = 0; b < kCombineBatch; b++) {
                if (p[b] < 0) continue;
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    acc[2 * q] = __builtin_fmaf(wt[b], bf16_to_f32((uint16_t)(v[b][q] & 0xffff)), acc[2 * q]);
                    acc[2 * q + 1] =
                        __builtin_fmaf(wt[b], bf16_to_f32((uint16_t)((uint32_t)v[b][q] >> 16)), acc[2 * q + 1]);
                }
            }
        }
        i32x4 o;
#pragma unroll
        for (int q = 0; q < 4; q++)
            o[q] = (int)((uint32_t)f32_to_bf16(acc[2 * q]) | ((uint32_t)f32_to_bf16(acc[2 * q + 1]) << 16));
        *(i32x4*)(out + (size_t)t * H + h0) = o;
    }
}

hipError_t launch_combine(const void* Y, const int32_t* inv_perm, const float* w, int T, int k, int H, void* out,
                          hipStream_t st) {
    k_combine<<<T, 256, 0, st>>>((const uint16_t*)Y, inv_perm, w, k, H, (uint16_t*)out);
    return hipGetLastError();
}

}  // namespace fmoe

// router.hip -- router linear and the wavefront top-k router kernel (the per-row top-k is in
// router_row.hpp, shared with the fused router + grouping kernel of group.hip).
#include "launch.hpp"
#include "router_row.hpp"

namespace fmoe {

// logits[t,e] = fmaf chain over ascending h of x[t,h]*w[e,h] (bf16 inputs, fp32 result).
__global__ void k_router_logits(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                int T, int H, int E, float* __restrict__ logits) {
    long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long long)T * E) return;
    int t = (int)(i / E), e = (int)(i % E);
    const uint16_t* xr = x + (size_t)t * H;
    const uint16_t* wr = w + (size_t)e * H;
    float acc = 0.0f;
    for (int h = 0; h < H; h++) acc = __builtin_fmaf(bf16_to_f32(xr[h]), bf16_to_f32(wr[h]), acc);
    logits[i] = acc;
}

// One wavefront per token, 4 tokens per workgroup.  QX: the workgroups after the first
// ceil(T/4) quantise x instead, one 128-column group per wavefront.
template <int SLOTS, bool BF16_IN, bool QX>
__global__ __launch_bounds__(256) void k_router_topk(const void* __restrict__ logits, int T, int E, int k,
                                                     int scoring, int renorm, int n_group, int topk_group,
                                                     int32_t* __restrict__ ids, float* __restrict__ weights,
                                                     XQuant xq) {
    const int nr = (T + 3) / 4;  // routing workgroups
    if (QX && (int)blockIdx.x >= nr) {
        const long long g = (long long)(blockIdx.x - nr) * 4 + (threadIdx.x >> 6);
        if (g < (long long)T * (xq.H >> 7)) quant_group_bf16_wave((const uint16_t*)xq.x, xq.H, g, xq.q, xq.s);
        return;
    }
    const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (t >= T) return;  // whole wavefront leaves together
    topk_row<SLOTS, BF16_IN>(logits, t, E, k, scoring, renorm, n_group, topk_group, ids, weights, nullptr);
}

hipError_t launch_router_logits(const void* x, const void* w, int T, int H, int E, float* logits, hipStream_t st) {
    long long n = (long long)T * E;
    int blocks = (int)((n + 255) / 256);
    k_router_logits<<<blocks, 256, 0, st>>>((const uint16_t*)x, (const uint16_t*)w, T, H, E, logits);
    return hipGetLastError();
}

template <int SLOTS>
static void launch_topk_slots(const void* logits, bool bf16, int T, int E, int k, int scoring, int renorm, int ng,
                              int tg, int32_t* ids, float* weights, hipStream_t st, const XQuant* xq) {
    long long blocks = (T + 3) / 4;
    if (xq) blocks += ((long long)T * (xq->H / 128) + 3) / 4;
    const XQuant none = {nullptr, 0, nullptr, nullptr};
    const XQuant& q = xq ? *xq : none;
    auto kern = bf16 ? (xq ? k_router_topk<SLOTS, true, true> : k_router_topk<SLOTS, true, false>)
                     : (xq ? k_router_topk<SLOTS, false, true> : k_router_topk<SLOTS, false, false>);
    kern<<<(unsigned)blocks, 256, 0, st>>>(logits, T, E, k, scoring, renorm, ng, tg, ids, weights, q);
}

hipError_t launch_router_topk(const void* logits, bool bf16, int T, int E, int k, int scoring, int renorm,
                              int32_t* ids, float* weights, hipStream_t st, int n_group, int topk_group,
                              const XQuant* xq) {
    if (xq && (!xq->x || !xq->q || !xq->s || xq->H <= 0 || xq->H % 128)) return hipErrorInvalidValue;
    int slots = (E + 63) / 64;
    const int ng = n_group, tg = topk_group;
    if (slots <= 1) launch_topk_slots<1>(logits, bf16, T, E, k, scoring, renorm, ng, tg, ids, weights, st, xq);
    else if (slots <= 2) launch_topk_slots<2>(logits, bf16, T, E, k, scoring, renorm, ng, tg, ids, weights, st, xq);
    else if (slots <= 4) launch_topk_slots<4>(logits, bf16, T, E, k, scoring, renorm, ng, tg, ids, weights, st, xq);
    else if (slots <= 8) launch_topk_slots<8>(logits, bf16, T, E, k, scoring, renorm, ng, tg, ids, weights, st, xq);
    else launch_topk_slots<16>(logits, bf16, T, E, k, scoring, renorm, ng, tg, ids, weights, st, xq);
    return hipGetLastError();
}

}  // namespace fmoe

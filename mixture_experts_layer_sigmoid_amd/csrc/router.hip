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

// One wavefront per token, 4 tokens per workgroup.
template <int SLOTS, bool BF16_IN>
__global__ __launch_bounds__(256) void k_router_topk(const void* __restrict__ logits, int T, int E, int k,
                                                     int scoring, int renorm, int n_group, int topk_group,
                                                     int32_t* __restrict__ ids, float* __restrict__ weights) {
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
                              int tg, int32_t* ids, float* weights, hipStream_t st) {
    int blocks = (T + 3) / 4;
    if (bf16)
        k_router_topk<SLOTS, true><<<blocks, 256, 0, st>>>(logits, T, E, k, scoring, renorm, ng, tg, ids, weights);
    else
        k_router_topk<SLOTS, false><<<blocks, 256, 0, st>>>(logits, T, E, k, scoring, renorm, ng, tg, ids, weights);
}

hipError_t launch_router_topk(const void* logits, bool bf16, int T, int E, int k, int scoring, int renorm,
                              int32_t* ids, float* weights, hipStream_t st, int n_group, int topk_group) {
    int slots = (E + 63) / 64;
    const int ng = n_group, tg = topk_group;
    if (slots <= 1) launch_topk_slots<1>(logits, bf16, T, E, k, scoring, renorm, ng, tg, ids, weights, st);
    else if (slots <= 2) launch_topk_slots<2>(logits, bf16, T, E, k, scoring, renorm, ng, tg, ids, weights, st);
    else if (slots <= 4) launch_topk_slots<4>(logits, bf16, T, E, k, scoring, renorm, ng, tg, ids, weights, st);
    else if (slots <= 8) launch_topk_slots<8>(logits, bf16, T, E, k, scoring, renorm, ng, tg, ids, weights, st);
    else launch_topk_slots<16>(logits, bf16, T, E, k, scoring, renorm, ng, tg, ids, weights, st);
    return hipGetLastError();
}

}  // namespace fmoe

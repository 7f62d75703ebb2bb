// quant.hip -- per-row, per-128-column e4m3 quantisation of activations (the w8a8 scheme of
// "Lab notes #6: We tuned vLLM's MoE kernels on an H100 ...", intro: fp8_w8a8 with
// block_shape [128,128]; activation scales per token and 128-column group, fp32).
//
// One wavefront per group of 128 values, two per lane (quant_group_wave): amax = max|x| (NaN
// ignored, as fmaxf does), s = amax/448 (1 for an all-zero group), inv = 1/s, code =
// e4m3(clamp(x*inv, +-448)).  The clamp uses fminf/fmaxf, so a NaN input becomes +448: the
// saturating FP8 conversion that "PR #39593: [Bug]: Fix FlashInfer CUTLASS BF16 + CUDA graphs
// IMA" (Root cause) calls a NaN firewall.  IEEE division (no fast-math), so codes and scales
// are reproducible bit for bit.  The forward quantises x in the router launch instead, with the
// same per-group code.
#include <climits>

#include "launch.hpp"

namespace fmoe {

// rows_hdr, when given, limits the rows to the grouped row count the grouping kernel left in
// the workspace header (the buffer is sized for the worst case).
template <bool BF16_IN>
__global__ __launch_bounds__(256) void k_quant_rows(const void* __restrict__ x, long long ngroups, int cols,
                                                   uint8_t* __restrict__ q, float* __restrict__ s,
                                                   const DevHeader* __restrict__ rows_hdr) {
    const long long g = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (g >= ngroups) return;
    const int lane = lane_id();
    const int G = cols >> 7;
    const long long row = g / G;
    // the row count and the values are loaded together: rows past the count still lie inside
    // the buffer (sized for every assignment), and nothing is stored for them
    const int live_rows = rows_hdr ? rows_hdr->local_rows : INT_MAX;
    const int grp = (int)(g - row * G);
    const size_t base = (size_t)row * cols + (size_t)grp * 128 + lane * 2;
    float a, b;
    if (BF16_IN) {
        const uint32_t two = *(const uint32_t*)((const uint16_t*)x + base);
        a = bf16_to_f32((uint16_t)(two & 0xffffu));
        b = bf16_to_f32((uint16_t)(two >> 16));
    } else {
        const float2 two = *(const float2*)((const float*)x + base);
        a = two.x;
        b = two.y;
    }
    if (row >= live_rows) return;  // the whole wavefront: one row per wavefront
    quant_group_wave(a, b, q + base, s + g);
}

hipError_t launch_quant_rows(const void* x, bool bf16_in, long long rows, int cols, uint8_t* q, float* s,
                             const DevHeader* rows_hdr, hipStream_t st) {
    const long long ngroups = rows * (cols / 128);
    if (ngroups == 0) return hipSuccess;
    const long long blocks = (ngroups + 3) / 4;
    if (bf16_in) k_quant_rows<true><<<(unsigned)blocks, 256, 0, st>>>(x, ngroups, cols, q, s, rows_hdr);
    else k_quant_rows<false><<<(unsigned)blocks, 256, 0, st>>>(x, ngroups, cols, q, s, rows_hdr);
    return hipGetLastError();
}

}  // namespace fmoe

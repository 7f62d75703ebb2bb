// common.hpp -- device-side types and helpers shared by the libfmoe kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fmoe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kE4M3Max = 448.0f;  // largest finite OCP E4M3FN magnitude
constexpr int kMaxKBlocks = 512;    // 128-deep blocks of the reduction dimension (65536 / 128)
constexpr int kLightRows = 32;      // largest row tile of the light GEMM kernel
constexpr int kMaxLightPerExpert = 8;  // light tiles of one expert when heavy tiles are left out
// row tiles of the heavy GEMM kernel: 4 groups of 64 rows, or 5 for an expert of 257..320
// rows in one tile (bf16 only: FP8's activation scales take LDS that a fifth group would need)
constexpr int kHeavyRows = 256;
constexpr int kHeavyRows5 = 320;

// Workspace header written by the grouping kernel and read by later kernels and by
// fmoe_read_stats.  Field order is part of the workspace format of this library only.
struct DevHeader {
    int32_t m_tiles;        // light row tiles (of at most tile_rows rows)
    int32_t local_rows;     // R
    int32_t max_rows;       // largest per-expert count
    int32_t empty_experts;  // local experts with no row
    long long dropped;      // ids outside [0, E)
    int32_t tile_rows;      // largest rows per tile used to cut the experts
    int32_t rows_estimate;  // max(1, ceil(T*top_k/E)) of the host plan
    int32_t m_tiles_heavy;  // heavy row tiles (experts with more than the light limit)
    int32_t heavy_rows;     // largest heavy tile: kHeavyRows, or kHeavyRows5 when used
    int32_t light_rows;     // rows of the light tiles
    int32_t m_tiles_stream; // light tiles of the streaming gate/up kernel (all or none of them)
    int32_t m_tiles_split;  // light tiles of the split-reduction gate/up kernel (the others)
    int32_t pad[3];
};
static_assert(sizeof(DevHeader) == 64, "header size");

// One row tile of a grouped GEMM: local expert, first grouped row, number of rows.
// Heavy tiles also carry, in `group`, their index among the heavy tiles of their expert (low
// 16 bits) and that expert's heavy tile count (high 16 bits, read as unsigned: it reaches
// 32768); light tiles carry 0.
struct MTile {
    int32_t expert, row0, rows, group;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// fp32 -> OCP e4m3 code, round to nearest even with saturation (the gfx950 conversion
// instruction).  Callers clamp to +-448 first.  The GPU quantisation tests compare its codes
// bit for bit with the oracle's own encoder at every rounding midpoint of the format, at both
// fp32 neighbours of each midpoint, and on 2^20 random values spread over every binade.
__device__ __forceinline__ uint32_t f32x2_to_e4m3x2(float a, float b) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// SwiGLU's activation of one feature: SiLU(g) * u = g * u / (1 + e^-g), with e^-g as the hardware
// 2^(-g log2 e) and the hardware reciprocal (each within a few ulp of the correctly rounded
// value, far inside the bf16 rounding of h).  Below g of about -88, e^-g overflows to infinity
// and the result is 0, the limit.  Every GEMM kernel uses this one definition, so the light and
// heavy kernels agree bit for bit.
__device__ __forceinline__ float silu_mul(float g, float u) {
    const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// One group of 128 values quantised by one wavefront, two values per lane (a, b: elements 2l
// and 2l+1 of lane l): amax = max|v| (NaN ignored, as fmaxf does), s = amax/448 (1 for an
// all-zero group), inv = 1/s, code = e4m3(clamp(v*inv, +-448)).  The clamp uses fminf/fmaxf,
// so a NaN value becomes +448.  IEEE division (no fast-math), so codes and scales are
// reproducible bit for bit.  q2: this lane's two code bytes; s: the group's scale.
__device__ __forceinline__ void quant_group_wave(float a, float b, uint8_t* q2, float* s) {
    float am = fmaxf(fmaxf(0.0f, fabsf(a)), fabsf(b));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    const float sc = (am == 0.0f) ? 1.0f : am / kE4M3Max;
    const float inv = 1.0f / sc;
    const float ya = fmaxf(fminf(a * inv, kE4M3Max), -kE4M3Max);
    const float yb = fmaxf(fminf(b * inv, kE4M3Max), -kE4M3Max);
    *(uint16_t*)q2 = (uint16_t)f32x2_to_e4m3x2(ya, yb);
    if (lane_id() == 0) *s = sc;
}

// Group g (row g / (cols/128), column group g % (cols/128)) of a bf16 matrix with `cols`
// columns (a multiple of 128), quantised by one wavefront; its scale goes to s[g].
__device__ __forceinline__ void quant_group_bf16_wave(const uint16_t* __restrict__ x, int cols, long long g,
                                                      uint8_t* __restrict__ q, float* __restrict__ s) {
    const int G = cols >> 7;
    const long long row = g / G;
    const size_t base = (size_t)row * cols + (size_t)(g - row * G) * 128 + lane_id() * 2;
    const uint32_t two = *(const uint32_t*)(x + base);
    quant_group_wave(bf16_to_f32((uint16_t)(two & 0xffffu)), bf16_to_f32((uint16_t)(two >> 16)), q + base, s + g);
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        T w = __shfl_xor(v, o, 64);
        v = v > w ? v : w;
    }
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

}  // namespace fmoe

// launch.hpp -- host-side launchers of the libfmoe kernels (one definition per .hip file).
#pragma once

#include "common.hpp"

namespace fmoe {

struct GemmArgs {
    const void* A;            // [rows, K] bf16, or e4m3 codes
    const float* A_scale;     // FP8: [rows, K/128]
    const int32_t* perm_src;  // gather map (grouped row -> flat assignment) or nullptr
    int topk;
    const void* W0;           // [El, N, K] gate (gated) or down
    const void* W1;           // [El, N, K] up (gated)
    const float* S0;          // FP8: [El, N/128, K/128]
    const float* S1;
    int N, K;
    void* out;                // [R, N] bf16, fp32, or e4m3 codes
    float* out_scale;         // e4m3 output: [R, N/128] scales of the codes (the streaming kernel only)
    const MTile* mtiles;      // this kernel's row-tile list
    const int* tile_count;    // its length (written by the grouping kernel)
};

// FP8 layers: the router launch also quantises x ([T, H] bf16) to e4m3 codes q [T, H] and scales
// s [T, H/128] (the code of launch_quant_rows): extra workgroups of the same launch take one
// 128-column group per wavefront, beside the routing workgroups.
struct XQuant {
    const void* x;
    int H;
    uint8_t* q;
    float* s;
};

hipError_t launch_router_logits(const void* x, const void* w, int T, int H, int E, float* logits, hipStream_t st);
// n_group groups of E/n_group experts, topk_group of them kept (n_group = topk_group = 1: plain top-k)
hipError_t launch_router_topk(const void* logits, bool bf16, int T, int E, int k, int scoring, int renorm,
                              int32_t* ids, float* weights, hipStream_t st, int n_group = 1, int topk_group = 1,
                              const XQuant* xq = nullptr);
size_t group_scratch_bytes(long long n, int El);
// Router top-k (plain) and grouping in one launch, for small T: route_group_fits says when.
bool route_group_fits(int T, int k, int E, int El);
hipError_t launch_route_group(const void* logits, bool bf16, int T, int E, int k, int scoring, int renorm,
                              int32_t* ids, float* weights, int El, int lo, int tile_rows, int light_cap,
                              int heavy5_min, int rows_estimate, int sparse_rows, int32_t* counts, int32_t* offsets,
                              int32_t* perm_src, int32_t* inv_perm, MTile* mtiles, MTile* mtiles_heavy, DevHeader* hdr,
                              hipStream_t st, const XQuant* xq = nullptr);
// light_cap >= tile_rows: experts with up to light_cap rows are cut into light tiles of tile_rows
// rows, heavier ones into heavy tiles.  sparse_rows > 0: the light tiles go to the split-reduction
// gate/up kernel (DevHeader::m_tiles_split) when they hold fewer than sparse_rows rows on
// average, else to the streaming one (m_tiles_stream); 0: always the streaming one.
hipError_t launch_group(const int32_t* ids, int n, int E, int El, int lo, int tile_rows, int light_cap,
                        int heavy5_min, int rows_estimate, int sparse_rows,
                        int32_t* counts, int32_t* offsets, int32_t* perm_src, int32_t* inv_perm, int32_t* rank_buf,
                        int* scratch, MTile* mtiles, MTile* mtiles_heavy, DevHeader* hdr, hipStream_t st);
hipError_t launch_quant_rows(const void* x, bool bf16_in, long long rows, int cols, uint8_t* q, float* s,
                             const DevHeader* rows_hdr, hipStream_t st);
size_t gemm_lds_bytes(bool fp8, int K, int tile_rows);
hipError_t launch_grouped_gemm(bool gated, bool fp8, bool out_f32, const GemmArgs& a, int tile_rows, int wk,
                               int max_tiles, int cus, hipStream_t st);
// Output of the streaming kernel: bf16, fp32, or (gated FP8 only) e4m3 codes with one fp32
// scale per row and 128 features, quantised as launch_quant_rows does.
enum StreamOut { kOutBf16 = 0, kOutF32 = 1, kOutE4M3 = 2 };
hipError_t launch_grouped_gemm_stream(bool gated, bool fp8, int out_mode, const GemmArgs& a, int tile_rows,
                                      int max_tiles, int cus, hipStream_t st);
// heavy row tiles (up to 320 rows, FP8 256) with both operands tiled through LDS
hipError_t launch_grouped_gemm_tiled(bool gated, bool fp8, bool out_f32, const GemmArgs& a, int max_tiles, int cus,
                                     hipStream_t st);
hipError_t launch_combine(const void* Y, const int32_t* inv_perm, const float* w, int T, int k, int H, void* out,
                          hipStream_t st);
// Down GEMM and combine in one launch for small batches (bf16 weights, at most
// kDownCombineMaxRows assignments, I at most kDownCombineMaxInter): h [R, I] grouped bf16 rows,
// the light and heavy tile lists with their counts in hdr, out [T, H] bf16.
constexpr int kDownCombineMaxRows = 64;
constexpr int kDownCombineMaxInter = 1024;
bool down_combine_fits(bool fp8, long long n, int I);
hipError_t launch_down_combine(const void* h, const void* Wd, int H, int I, const MTile* tiles,
                               const MTile* tiles_heavy, const DevHeader* hdr, const int32_t* inv_perm,
                               const float* wts, int T, int k, void* out, hipStream_t st);

}  // namespace fmoe

// down_combine.hip -- down GEMM and routing-weighted combine in one launch, for small batches.
//
// With a handful of tokens every active expert holds a row or two ("vLLM Community Traces H20
// MoE Scheduling Inefficiency to Expert-Load Kernel Selection", paragraph 3: the rows per expert,
// not the token count, decide which kernel fits), so the down GEMM is a stream of weight rows
// each used once or twice: a matrix-vector product bound by the weight bytes.  Written as two
// launches it also pays a second launch and a round trip of y through memory for the combine.
//
// Here one workgroup owns 8 output features of the layer for every token:
//   y[p, f] = sum_i h[p, i] * W_down[l, f, i]    for every grouped row p (local expert l),
//   out[t, f] = sum over j ascending, inv_perm[t*k+j] = p >= 0, of w[t, j] * y[p, f]
// It copies the grouped activation rows h (R rows of I bf16) into LDS once, then walks the row
// tiles (light, then heavy) and multiplies the 8 weight rows of each tile's expert with the
// tile's rows on the matrix cores; y stays in LDS in fp32, and the combine is the workgroup's
// last step: fp32 fused multiply-adds in ascending j, one bf16 rounding, zeros for a token
// without local rows.
//
// Matrix-core layout (v_mfma_f32_16x16x32_bf16): the weight rows are the A operand (rows 0-7 the
// workgroup's features, rows 8-15 zero), 16 tile rows the B operand.  The 4 wavefronts split
// the reduction into 64-deep pairs of steps (wavefront w takes pairs [w*P/4, (w+1)*P/4) of the
// P = I/64); one 16-byte load per lane and pair fetches whole 128-byte lines: lanes of rows 0-7
// take step 2q's piece of their own row, lanes of rows 8-15 step 2q+1's piece of the row 8 below,
// and a rotation by 8 lanes within each 16-lane row (row_ror:8) hands those to rows 0-7 for the
// second step.  The wavefronts' partial sums go to LDS and are added in wavefront order.
//
// The weight pieces of 4 tiles are loaded per step into one of two register sets while the other
// set's tiles are multiplied, so one step's weights are in flight behind the other's arithmetic.
// The loads stay unconditional (and so do the compiler's wait counts): a pair or a tile past the
// end reads through an empty buffer resource, which fetches nothing.
#include "launch.hpp"

namespace fmoe {

namespace {

constexpr int kDcFeat = 8;       // output features per workgroup
constexpr int kDcThreads = 256;  // 4 wavefronts
constexpr int kDcP = 4;          // tiles per step of the weight ring
constexpr int kDcRsrcFlags = 0x00020000;  // buffer resource word 3: 32-bit data, raw (offset) addressing
constexpr int kDcNT = 2;                  // cache policy of the weight loads: non-temporal

// PP: 64-deep pairs of reduction steps per wavefront at most (I <= 256 * PP)
template <int PP>
__global__ __launch_bounds__(kDcThreads) void k_down_combine(const uint16_t* __restrict__ h,
                                                             const uint16_t* __restrict__ Wd, int H, int I,
                                                             const MTile* __restrict__ tiles,
                                                             const MTile* __restrict__ tiles_heavy,
                                                             const DevHeader* __restrict__ hdr,
                                                             const int32_t* __restrict__ inv_perm,
                                                             const float* __restrict__ wts, int T, int k,
                                                             uint16_t* __restrict__ out) {
    // h rows (16-byte pieces, I/8 per row); partial sums [wavefront][row][feature]
    __shared__ i32x4 Hs[kDownCombineMaxRows * 32 * PP];
    __shared__ float Yp[4 * kDownCombineMaxRows * kDcFeat];
    __shared__ int32_t Pl[kDownCombineMaxRows];  // inv_perm and routing weights of the T*k <= 64
    __shared__ float Wl[kDownCombineMaxRows];    // assignments, for the combine

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int r16 = lane & 15, kg = lane >> 4;
    const bool lower = r16 < 8;
    const int f0 = blockIdx.x * kDcFeat;
    const int nq = I >> 3;  // 16-byte pieces per row
    const int npairs = I >> 6;
    const int p_lo = w * npairs / 4, np = (w + 1) * npairs / 4 - p_lo;  // this wavefront's pairs
    const int R = hdr->local_rows;
    const int nl = hdr->m_tiles, nt = nl + hdr->m_tiles_heavy;

    auto tile_at = [&](int i) { return i < nl ? tiles[i] : tiles_heavy[i - nl]; };
    // byte offset of this lane's piece of pair q inside an expert's down matrix (fixed for the
    // launch: each load is a per-tile scalar resource plus one of these)
    uint32_t voff[PP];
#pragma unroll
    for (int q = 0; q < PP; q++) {
        const int pair = p_lo + min(q, max(np - 1, 0));
        voff[q] = (uint32_t)(((size_t)(f0 + (r16 & 7)) * I + (size_t)pair * 64 + (lower ? 0 : 32) + kg * 8) * 2);
    }
    const size_t estride = (size_t)H * I * 2;
    auto load_step = [&](i32x4(&wv)[kDcP][PP], int i0) {
#pragma unroll
        for (int p = 0; p < kDcP; p++) {
            const int e = __builtin_amdgcn_readfirstlane(tile_at(min(i0 + p, nt - 1)).expert);
            const void* base = (const void*)((const char*)Wd + (size_t)e * estride);
            const __amdgpu_buffer_rsrc_t full =
                __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, i0 + p < nt ? (int)estride : 0, kDcRsrcFlags);
            const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, 0, kDcRsrcFlags);
#pragma unroll
            for (int q = 0; q < PP; q++)
                wv[p][q] = __builtin_bit_cast(
                    i32x4, __builtin_amdgcn_raw_buffer_load_b128(q < np ? full : none, (int)voff[q], 0, kDcNT));
        }
        // keep the scheduler from hoisting the previous set's arithmetic (which waits for its
        // loads) above these loads
        __builtin_amdgcn_sched_barrier(0);
    };
    auto compute_step = [&](const i32x4(&wv)[kDcP][PP], int i0) {
#pragma unroll
        for (int p = 0; p < kDcP; p++) {
            if (i0 + p >= nt) break;
            const MTile t = tile_at(i0 + p);
            // A fragments of both steps of each pair: rows 8-15 zero
            bf16x8 a0[PP], a1[PP];
#pragma unroll
            for (int q = 0; q < PP; q++) {
                i32x4 x, y;
#pragma unroll
                for (int d = 0; d < 4; d++) {
                    const int v = wv[p][q][d];
                    const int rot = __builtin_amdgcn_update_dpp(0, v, 0x128, 0xf, 0xf, false);  // row_ror:8
                    x[d] = lower ? v : 0;
                    y[d] = lower ? rot : 0;
                }
                a0[q] = __builtin_bit_cast(bf16x8, x);
                a1[q] = __builtin_bit_cast(bf16x8, y);
            }
            for (int b0 = 0; b0 < t.rows; b0 += 16) {
                const int row = t.row0 + min(b0 + r16, t.rows - 1);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q = 0; q < PP; q++) {
                    if (q >= np) break;
                    const int k0 = (p_lo + q) * 8;  // first piece of the pair
                    const bf16x8 b0v = __builtin_bit_cast(bf16x8, Hs[row * nq + k0 + kg]);
                    const bf16x8 b1v = __builtin_bit_cast(bf16x8, Hs[row * nq + k0 + 4 + kg]);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[q], b0v, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[q], b1v, acc, 0, 0, 0);
                }
                // lane (r16, kg < 2) holds features 4 kg .. 4 kg + 3 of tile row b0 + r16
                if (kg < 2 && b0 + r16 < t.rows) {
                    float* dst = Yp + ((size_t)w * kDownCombineMaxRows + t.row0 + b0 + r16) * kDcFeat + 4 * kg;
                    *(f32x4*)dst = acc;
                }
            }
        }
    };

    // the combine's inputs, loaded first (the oldest loads: they have landed before any wait
    // below is satisfied) and put in LDS at the end
    const int n = T * k;
    int32_t my_p = -1;
    float my_w = 0.0f;
    if (tid < n) {
        my_p = inv_perm[tid];
        my_w = wts[tid];
    }

    if (nt > 0) {
        i32x4 wa[kDcP][PP], wb[kDcP][PP];
        // the grouped activation rows, straight into LDS: wavefront w copies pieces q0 + lane of
        // each 256-piece block (q0 = block + 64 w), the last piece repeated past the end (the
        // buffer holds whole 64-piece runs: R*nq <= 64 * 32*PP)
        const int total = R * nq;
        for (int q0 = w * 64; q0 < total; q0 += kDcThreads)
            __builtin_amdgcn_global_load_lds((const void*)((const i32x4*)h + min(q0 + lane, total - 1)),
                                             (__attribute__((address_space(3))) void*)(Hs + q0), 16, 0, 0);
        // both weight register sets go out behind the copies; loads complete in issue order, so
        // the copies have landed once at most the weight loads are outstanding
        load_step(wa, 0);
        load_step(wb, kDcP);
        constexpr int kAfter = 2 * kDcP * PP;
        static_assert(kAfter <= 63, "vmcnt range");
        // a plain barrier: the fence of __syncthreads would also wait for the weight loads
        __builtin_amdgcn_s_waitcnt((kAfter & 15) | (7 << 4) | (15 << 8) | ((kAfter >> 4) << 14));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        compute_step(wa, 0);
        for (int i0 = kDcP; i0 < nt; i0 += 2 * kDcP) {
            if (i0 + kDcP >= nt) {
                compute_step(wb, i0);
                break;
            }
            load_step(wa, i0 + kDcP);
            compute_step(wb, i0);
            if (i0 + 2 * kDcP >= nt) {
                compute_step(wa, i0 + kDcP);
                break;
            }
            load_step(wb, i0 + 2 * kDcP);
            compute_step(wa, i0 + kDcP);
        }
    }
    if (tid < n) {
        Pl[tid] = my_p;
        Wl[tid] = my_w;
    }
    __syncthreads();

    // combine: thread (token t, feature g) over the token's k assignments in ascending j; y of
    // a row is its four wavefronts' partial sums added in order
    for (int idx = tid; idx < T * kDcFeat; idx += kDcThreads) {
        const int t = idx >> 3, g = idx & 7;
        float acc = 0.0f;
        for (int jj = 0; jj < k; jj++) {
            const int p = Pl[t * k + jj];
            if (p < 0) continue;
            float y = Yp[(size_t)p * kDcFeat + g];
#pragma unroll
            for (int ww = 1; ww < 4; ww++) y += Yp[((size_t)ww * kDownCombineMaxRows + p) * kDcFeat + g];
            acc = __builtin_fmaf(Wl[t * k + jj], y, acc);
        }
        out[(size_t)t * H + f0 + g] = f32_to_bf16(acc);
    }
}

template <int PP>
hipError_t launch_dc(const void* h, const void* Wd, int H, int I, const MTile* tiles, const MTile* tiles_heavy,
                     const DevHeader* hdr, const int32_t* inv_perm, const float* wts, int T, int k, void* out,
                     hipStream_t st) {
    k_down_combine<PP><<<H / kDcFeat, kDcThreads, 0, st>>>((const uint16_t*)h, (const uint16_t*)Wd, H, I, tiles,
                                                          tiles_heavy, hdr, inv_perm, wts, T, k, (uint16_t*)out);
    return hipGetLastError();
}

}  // namespace

bool down_combine_fits(bool fp8, long long n, int I) {
    return !fp8 && n >= 1 && n <= kDownCombineMaxRows && I >= 128 && I <= kDownCombineMaxInter && I % 128 == 0;
}

hipError_t launch_down_combine(const void* h, const void* Wd, int H, int I, const MTile* tiles,
                               const MTile* tiles_heavy, const DevHeader* hdr, const int32_t* inv_perm,
                               const float* wts, int T, int k, void* out, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    switch ((I + 255) / 256) {
        case 1: return launch_dc<1>(h, Wd, H, I, tiles, tiles_heavy, hdr, inv_perm, wts, T, k, out, st);
        case 2: return launch_dc<2>(h, Wd, H, I, tiles, tiles_heavy, hdr, inv_perm, wts, T, k, out, st);
        case 3: return launch_dc<3>(h, Wd, H, I, tiles, tiles_heavy, hdr, inv_perm, wts, T, k, out, st);
        case 4: return launch_dc<4>(h, Wd, H, I, tiles, tiles_heavy, hdr, inv_perm, wts, T, k, out, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fmoe

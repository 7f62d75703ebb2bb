// gemm_stream.hip -- grouped expert GEMMs for light row tiles (up to 32 rows), streaming form.
//
// Same operation as gemm.hip (gate/up with SiLU-and-mul, or down; bf16 or FP8 block-scaled),
// for launches with enough tasks (row tile x 64 or 128 output features) to fill the GPU
// without splitting the reduction.
//
// Decode is bound by the weight stream, so each wavefront is built as one uninterrupted
// stream of weight loads: it walks its workgroup's tasks in order and its ring of D weight
// steps (HBM straight into the MFMA "A" registers, 16 feature rows x 8 consecutive k per lane)
// runs up to D steps ahead across task boundaries, so the stream never drains between tiles.
// The tile's activation rows (the MFMA "B" operand) are the same for all wavefronts of the
// workgroup: they are loaded once per workgroup, a chunk of CS reduction steps at a time,
// through registers into a double-buffered LDS area (each 64-lane fragment is stored in the
// lane order the MFMA reads it, so stores and reads are contiguous 16-byte accesses), with the
// next chunk in flight while the current one is used.  Loading them per wavefront instead
// quadruples the vector-memory instructions of the activations, which then hold back the
// weight stream.  FP8 scales of a chunk (one per 128-deep block and row, and one per
// 128-deep block of the weight rows) are staged with it.
//
// Every step issues the same loads (padding steps past the reduction end re-read the last
// valid step, which hits in cache), so the compiler's static wait counts stay exact.
//
// Outputs are parked in LDS and written to global memory a few tasks at a time (and at the
// end).  A wavefront's memory operations leave its counter in issue order, so a global store
// holds back every weight load issued after it until the store is acknowledged, and the weight
// ring waits for it.  A bf16 down GEMM with its stores left out ran 13% faster (T=256 of the
// 128-expert layer: 73 against 84 us); storing once per OUTQ tasks pays that wait once per
// OUTQ tasks, and not at all for a workgroup with at most OUTQ tasks.  Each wavefront parks and
// stores only its own outputs, so no barrier is involved.
//
// FP8 gate/up may also quantise its output itself (the w8a8 scheme's per-row, per-128-column
// activation scales): a workgroup of 8 wavefronts then holds all 128 features of one scale
// group, the wavefronts combine their row maxima through LDS, and the codes and scales are
// written in place of the fp32 activation, with the arithmetic of the quantisation kernel
// (amax/448, IEEE reciprocal, fminf/fmaxf clamp, saturating conversion).
#include <type_traits>

#include "launch.hpp"

namespace fmoe {

namespace {

// A workgroup of WV wavefronts computes 16 WV output features of a row tile.

template <bool FP8>
struct SCfg {
    using T = bf16x8;
    static constexpr int KSTEP = 32;   // reduction depth of one MFMA
    static constexpr int EB = 2;       // bytes per element
    static constexpr int LANE_B = 16;  // operand bytes per lane per step
    static constexpr int HALVES = 1;   // 16-byte pieces per lane fragment
    static constexpr int CS = 8;       // steps per staged chunk
    static constexpr int PAIR = 2;     // steps per 128-byte weight line of a row
    static constexpr int PART_Y = 64;  // bytes between a lane's two pieces of one line
};
template <>
struct SCfg<true> {
    using T = i32x8;
    static constexpr int KSTEP = 128;
    static constexpr int EB = 1;
    static constexpr int LANE_B = 32;
    static constexpr int HALVES = 2;
    static constexpr int CS = 4;
    static constexpr int PAIR = 1;
    static constexpr int PART_Y = 16;
};

template <bool FP8, int NS, int CS>
struct StreamLds {
    static constexpr int F = NS * CS * SCfg<FP8>::HALVES;  // 1 KB pieces per chunk
    i32x4 x[2][F][64];
    float asc[2][CS][NS * 16];  // FP8: activation scale of each step and tile row
    float wsc[2][2][CS];        // FP8: weight-block scale of each matrix and step
};

// Parked outputs of up to Q tasks per wavefront: each lane's piece of each 16-row sub-block
// (bf16: 4 features, fp32: 4 features, e4m3: 4 codes), the task's first row, rows and this
// wavefront's first feature, and (e4m3, wavefront 0) the scale of each row's 128-feature group.
template <int OUT, int NS, int WV, int Q>
struct StreamParked {
    using T = typename std::conditional<OUT == kOutF32, f32x4,
                                        typename std::conditional<OUT == kOutE4M3, uint32_t, uint2>::type>::type;
    T v[Q][WV][NS][64];
    int meta[Q][WV][3];
    float sc[OUT == kOutE4M3 ? Q : 1][NS][16];
};


// a[i] for a runtime i, as a mask-and-or over the elements.  An indexed read of a register
// array goes through scratch memory, and the compiler may fold a chain of selects over the
// elements back into such a read (it did with 4 and 8 sub-blocks per tile); the masks keep
// the array in registers.
template <int N, typename T>
__device__ __forceinline__ T pick(const T (&a)[N], int i) {
    static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit elements");
    using U = typename std::conditional<sizeof(T) == 4, uint32_t, uint64_t>::type;
    U r = 0;
#pragma unroll
    for (int j = 0; j < N; j++) r |= __builtin_bit_cast(U, a[j]) & (U)0 - (U)(i == j);
    return __builtin_bit_cast(T, r);
}

// Where one task's operands live, for this lane.
template <int NS, int NW>
struct Ctx {
    const uint8_t* w[NW];  // weight rows of this wavefront's 16 features, at this lane's (row, k) slot
    const float* ws[NW];   // FP8: this workgroup's weight-block scale row ([K/128])
    int map[NS];           // gather-map entry of this lane's row in each 16-row sub-block (its
                           // activation row is map / top_k); read only when the task's
                           // activations are staged, well after the load was issued
    int row0, rows;        // grouped rows of the task
    int soff;              // 0, or the step count for a padding context that re-reads the last step
};

template <bool GATED, bool FP8, int OUT, int NS, int D, int WV, int CS, bool LINE>
__global__ __launch_bounds__(64 * WV) void k_grouped_gemm_stream(GemmArgs g) {
    using C = SCfg<FP8>;
    using FT = typename C::T;
    constexpr int NW = GATED ? 2 : 1;
    constexpr int F = StreamLds<FP8, NS, CS>::F;
    constexpr int FPW = F / WV;  // pieces staged per wavefront
    constexpr int FEAT = 16 * WV;
    static_assert(F % WV == 0 && CS % D == 0, "chunk shape");
    static_assert(!FP8 || CS * NS * 16 <= 64 * WV, "one thread per staged activation scale");
    static_assert(OUT != kOutE4M3 || (GATED && FP8 && FEAT == 128), "e4m3 output: one 128-feature group per workgroup");
    __shared__ StreamLds<FP8, NS, CS> L;
    __shared__ float QM[OUT == kOutE4M3 ? NS * WV * 16 : 1];  // row maxima of each wavefront's 16 features
    // tasks parked before a store: 4, or 2 where the staging buffers are large (more than 40 KB),
    // so that two workgroups still fit a CU's LDS
    constexpr int OUTQ = sizeof(StreamLds<FP8, NS, CS>) > 40 * 1024 ? 2 : 4;
    __shared__ StreamParked<OUT, NS, WV, OUTQ> SO;

    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, kg = lane >> 4;
    const int K = g.K;
    const int nsteps = K / C::KSTEP;
    const int nch = (nsteps + CS - 1) / CS;
    const int nkb = K >> 7;
    const int nblocks = g.N / FEAT;
    const int mtc = *g.tile_count;
    // Task order.  Workgroup b runs on XCD b % 8 (the dispatcher deals workgroups to the 8
    // XCDs in turn), and every XCD has its own L2.  With at least 8 row tiles, each tile goes to
    // one XCD and all its feature blocks run there, so the tile's activation rows are fetched
    // into one L2 instead of up to eight; the workgroups of an XCD deal its tasks in turn.  The
    // tiles are dealt to the XCDs in blocks of 8 consecutive tiles (tile m to XCD (m / 8) % 8)
    // as long as every XCD gets a whole block, then one at a time: the light tiles of one
    // expert are consecutive in the list, so an expert cut into several light tiles has them
    // on one XCD, where they run at the same time and share the expert's weights in its L2.
    // With fewer tiles, tasks are dealt over all workgroups in order (spread over the XCDs).
    const int G = (int)gridDim.x, b = (int)blockIdx.x;
    const bool by_xcd = (G % 8 == 0) && mtc >= 8;
    const int xcd = b % 8, slot = b / 8, S = G / 8;
    const int rounds = mtc / 64, rem = mtc - rounds * 64;  // whole rounds of 8 blocks of 8 tiles
    int ntasks;
    if (by_xcd) {
        const int ntx = (rounds * 8 + (rem > xcd ? (rem - xcd + 7) / 8 : 0)) * nblocks;  // tasks of this XCD
        ntasks = ntx > slot ? (ntx - 1 - slot) / S + 1 : 0;
    } else {
        const int total = mtc * nblocks;
        ntasks = total > b ? (total - 1 - b) / G + 1 : 0;
    }
    if (ntasks == 0) return;
    // tile and feature block of this workgroup's task i
    auto task_at = [&](int i, int& mt, int& nb) {
        if (by_xcd) {
            const int j = slot + i * S;
            const int q = j / nblocks;  // this XCD's q-th tile
            mt = q < rounds * 8 ? (q >> 3) * 64 + xcd * 8 + (q & 7) : rounds * 64 + (q - rounds * 8) * 8 + xcd;
            nb = j - q * nblocks;
        } else {
            const int t = b + i * G;
            mt = t / nblocks;
            nb = t - mt * nblocks;
        }
    };
    const size_t rowbytes = (size_t)K * C::EB;
    // Weight loads by whole lines (LINE): a wavefront's 16 rows x 128 bytes (two bf16 steps,
    // or one FP8 step) arrive by two non-temporal loads of 8 full 128-byte lines each, load A
    // rows 0-7 and load B rows 8-15.  The MFMA wants lane (r16, kg) to hold row r16's piece X
    // (step 2p: bytes 16 kg; FP8: the fragment's low half at 32 kg) and piece Y (step 2p+1:
    // 64 + 16 kg; FP8: the high half at 32 kg + 16).  In load A a lower-half lane (r16 < 8)
    // takes piece X of row r16 and an upper-half lane piece Y of row r16 - 8; in load B a
    // lower-half lane takes piece Y of row r16 + 8 and an upper-half lane piece X of row r16.
    // So X is A in the lower and B in the upper half lanes, and Y is the other choice seen 8
    // lanes away (a rotation by 8 within each 16-lane row): the MFMA operands are the bytes a
    // per-step load gives, in the same lanes.  Non-temporal loads (streamed, not kept in the
    // caches) raised a plain read of the weights from 5.7-5.8 to 6.6 TB/s, but only with whole
    // lines per load: with the per-step form (half a line per row and load) the second half
    // was fetched again, and the down GEMM got slower.  The FP8 gate/up GEMM keeps per-step
    // loads: its steps are whole lines already, and the rearrangement measured slower there.
    const bool lower = r16 < 8;
    const size_t lane_w = LINE ? (size_t)(r16 & 7) * rowbytes + kg * C::LANE_B + (lower ? 0 : C::PART_Y)
                               : (size_t)r16 * rowbytes + kg * C::LANE_B;
    const long long lane_ab = 8 * (long long)rowbytes + (lower ? C::PART_Y : -C::PART_Y);

    using CT = Ctx<NS, NW>;
    // task i of this workgroup into slot c; past the last task, a padding context that keeps
    // re-reading the last step of task `prev` (whose addresses are computed, not loaded, so
    // nothing waits on an outstanding load) with activation row 0
    auto load_ctx = [&](CT& c, int i, const CT& prev) {
        if (i >= ntasks) {
#pragma unroll
            for (int h = 0; h < NW; h++) {
                c.w[h] = prev.w[h];
                c.ws[h] = prev.ws[h];
            }
#pragma unroll
            for (int sb = 0; sb < NS; sb++) c.map[sb] = 0;
            c.row0 = prev.row0;
            c.rows = prev.rows;
            c.soff = nsteps;
            return;
        }
        int mt, nb;
        task_at(i, mt, nb);
        // the tile list is read-only here: read it through the constant address space, so the
        // (wavefront-uniform) read is a scalar load that does not wait on the weight stream
        const i32x4 mv = *(const __attribute__((address_space(4))) i32x4*)(g.mtiles + mt);
        const MTile m = {mv[0], mv[1], mv[2], mv[3]};
        const size_t wrow = (size_t)m.expert * g.N + nb * FEAT + w * 16;
        c.w[0] = (const uint8_t*)g.W0 + wrow * rowbytes + lane_w;
        if constexpr (GATED) c.w[NW - 1] = (const uint8_t*)g.W1 + wrow * rowbytes + lane_w;
        if constexpr (FP8) {
            const size_t srow = ((size_t)m.expert * (g.N >> 7) + ((nb * FEAT) >> 7)) * nkb;
            c.ws[0] = g.S0 + srow;
            if constexpr (GATED) c.ws[NW - 1] = g.S1 + srow;
        }
#pragma unroll
        for (int sb = 0; sb < NS; sb++) {
            const int p = m.row0 + min(sb * 16 + r16, m.rows - 1);
            c.map[sb] = g.perm_src ? g.perm_src[p] : p;
        }
        c.row0 = m.row0;
        c.rows = m.rows;
        c.soff = 0;
    };

    // Ring slot s holds step s's weights.  With LINE, bf16 loads a pair of steps into slots
    // (s, s+1) (s even) once both are used, FP8 one step (both loads) into its slot; each
    // arrives as loads A and B and is rearranged into fragments right before its first use.
    constexpr int PAIR = LINE ? C::PAIR : 1;
    static_assert(D % PAIR == 0 && CS % PAIR == 0, "ring and chunk hold whole lines");
    FT bw[D][NW];
    auto issue_w = [&](int slot, const CT& c, int step) {
        if constexpr (!LINE) {
            const size_t o = (size_t)min(step + c.soff, nsteps - 1) * (C::KSTEP * C::EB);
#pragma unroll
            for (int h = 0; h < NW; h++) bw[slot][h] = *(const FT*)(c.w[h] + o);
        } else {
            if (slot % PAIR != PAIR - 1) return;
            const int s0 = step - (PAIR - 1);  // first step of the line; bf16 step counts are even
            const size_t o = (size_t)min(s0 + c.soff, nsteps - PAIR) * (C::KSTEP * C::EB);
#pragma unroll
            for (int h = 0; h < NW; h++) {
                const i32x4 a = __builtin_nontemporal_load((const i32x4*)(c.w[h] + o));
                const i32x4 b = __builtin_nontemporal_load((const i32x4*)(c.w[h] + lane_ab + o));
                if constexpr (FP8) {
                    bw[slot][h] = i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
                } else {
                    bw[slot - 1][h] = __builtin_bit_cast(bf16x8, a);
                    bw[slot][h] = __builtin_bit_cast(bf16x8, b);
                }
            }
        }
    };
    // loads A, B of a line into pieces X, Y: X = lower ? A : B; Y = (lower ? B : A) rotated by 8
    // lanes within each 16-lane row (a row_ror:8 move)
    auto regroup = [&](i32x4& a, i32x4& b) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int x = lower ? a[i] : b[i];
            const int z = lower ? b[i] : a[i];
            a[i] = x;
            b[i] = __builtin_amdgcn_update_dpp(0, z, 0x128, 0xf, 0xf, false);
        }
    };
    auto prepare = [&](int slot) {
#pragma unroll
        for (int h = 0; h < NW && LINE; h++) {
            if constexpr (FP8) {
                i32x4 a = {bw[slot][h][0], bw[slot][h][1], bw[slot][h][2], bw[slot][h][3]};
                i32x4 b = {bw[slot][h][4], bw[slot][h][5], bw[slot][h][6], bw[slot][h][7]};
                regroup(a, b);
                bw[slot][h] = i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
            } else if (slot % 2 == 0) {
                i32x4 a = __builtin_bit_cast(i32x4, bw[slot][h]);
                i32x4 b = __builtin_bit_cast(i32x4, bw[slot + 1][h]);
                regroup(a, b);
                bw[slot][h] = __builtin_bit_cast(bf16x8, a);
                bw[slot + 1][h] = __builtin_bit_cast(bf16x8, b);
            }
        }
    };

    // staging of one chunk: wavefront w loads pieces w*FPW .. w*FPW+FPW-1; piece f is step
    // f / (NS*HALVES), sub-block (f / HALVES) % NS, 16-byte half f % HALVES
    i32x4 xst[FPW];
    float ast = 0.f, wst = 0.f;
    const int topk = g.perm_src ? g.topk : 1;
    auto src_row = [&](const CT& c, int sb) { return c.map[sb] / topk; };
    auto stage_load = [&](const CT& c, int chunk) {
        size_t xoff[NS];
#pragma unroll
        for (int sb = 0; sb < NS; sb++) xoff[sb] = (size_t)src_row(c, sb) * rowbytes + kg * C::LANE_B;
#pragma unroll
        for (int j = 0; j < FPW; j++) {
            const int f = w * FPW + j;
            const int s = f / (NS * C::HALVES), sb = (f / C::HALVES) % NS, half = f % C::HALVES;
            const size_t step = (size_t)min(chunk * CS + s + c.soff, nsteps - 1);
            // sb depends on the wavefront index: picked, not an indexed register array
            xst[j] = *(const i32x4*)((const uint8_t*)g.A + pick(xoff, sb) + step * (C::KSTEP * C::EB) + half * 16);
        }
        if constexpr (FP8) {
            // activation scales: thread t < CS*NS*16 takes step t / (NS*16) of row t % (NS*16),
            // which is this lane's row (r16) of sub-block (t / 16) % NS
            const int t = threadIdx.x % (CS * NS * 16);
            const int s = t / (NS * 16);
            const int kb = min(chunk * CS + s + c.soff, nkb - 1);
            ast = g.A_scale[(size_t)(pick(c.map, (t >> 4) % NS) / topk) * nkb + kb];
            // weight scales: thread t < NW*CS takes matrix t / CS, step t % CS
            const int u = threadIdx.x % (NW * CS);
            const int kw = min(chunk * CS + u % CS + c.soff, nkb - 1);
            wst = pick(c.ws, u / CS)[kw];
        }
    };
    auto stage_store = [&](int buf) {
#pragma unroll
        for (int j = 0; j < FPW; j++) L.x[buf][w * FPW + j][lane] = xst[j];
        if constexpr (FP8) {
            const int t = threadIdx.x;
            if (t < CS * NS * 16) L.asc[buf][t / (NS * 16)][t % (NS * 16)] = ast;
            if (t < NW * CS) L.wsc[buf][t / CS][t % CS] = wst;
        }
    };

    f32x4 acc[NS][NW];
    auto zero_acc = [&]() {
#pragma unroll
        for (int sb = 0; sb < NS; sb++)
#pragma unroll
            for (int h = 0; h < NW; h++) acc[sb][h] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    auto compute = [&](int slot, int buf, int s) {
        prepare(slot);
#pragma unroll
        for (int sb = 0; sb < NS; sb++) {
            FT xb;
            if constexpr (FP8) {
                const i32x4 lo = L.x[buf][(s * NS + sb) * 2][lane];
                const i32x4 hi = L.x[buf][(s * NS + sb) * 2 + 1][lane];
                xb = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                const float sa = L.asc[buf][s][sb * 16 + r16];
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int h = 0; h < NW; h++) {
                    const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bw[slot][h], xb, zero, 0, 0, 0,
                                                                                      0, 0, 0);
                    const float cs = L.wsc[buf][h][s] * sa;
#pragma unroll
                    for (int i = 0; i < 4; i++) acc[sb][h][i] = __builtin_fmaf(p[i], cs, acc[sb][h][i]);
                }
            } else {
                xb = __builtin_bit_cast(bf16x8, L.x[buf][s * NS + sb][lane]);
#pragma unroll
                for (int h = 0; h < NW; h++)
                    acc[sb][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bw[slot][h], xb, acc[sb][h], 0, 0, 0);
            }
        }
    };
    // Parked outputs: nout tasks so far; task j sits in slot j % OUTQ.  flush(n) stores slots
    // 0 .. n-1 of this wavefront (rows past the task's end are not stored).
    int nout = 0;
    auto flush = [&](int n) {
        for (int q = 0; q < n; q++) {
            const int row0 = SO.meta[q][w][0], rows = SO.meta[q][w][1], n0 = SO.meta[q][w][2];
#pragma unroll
            for (int sb = 0; sb < NS; sb++) {
                const int col = sb * 16 + r16;
                if (col >= rows) continue;
                const size_t row = (size_t)(row0 + col);
                const auto v = SO.v[q][w][sb][lane];
                if constexpr (OUT == kOutE4M3) {
                    *(uint32_t*)((uint8_t*)g.out + row * g.N + n0 + kg * 4) = v;
                    if (w == 0 && kg == 0) g.out_scale[row * (g.N >> 7) + (n0 >> 7)] = SO.sc[q][sb][r16];
                } else if constexpr (OUT == kOutF32) {
                    *(f32x4*)((float*)g.out + row * g.N + n0 + kg * 4) = v;
                } else {
                    *(uint2*)((uint16_t*)g.out + row * g.N + n0 + kg * 4) = v;
                }
            }
        }
    };
    // lane holds token column sb*16 + r16 and features n0 + 4*kg + i; the results are parked in
    // this wavefront's next slot, and every OUTQ tasks the slots are stored
    auto epilogue = [&](const CT& c, int n0) {
        const int q = nout % OUTQ;
        if (lane == 0) {
            SO.meta[q][w][0] = c.row0;
            SO.meta[q][w][1] = c.rows;
            SO.meta[q][w][2] = n0;
        }
        if constexpr (OUT == kOutE4M3) {
            // every wavefront of the workgroup runs the same tasks, so all reach this barrier;
            // QM is rewritten only after the next task's chunk barriers
            float r[NS][4], am[NS];
#pragma unroll
            for (int sb = 0; sb < NS; sb++) {
                am[sb] = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    r[sb][i] = silu_mul(acc[sb][0][i], acc[sb][NW - 1][i]);
                    am[sb] = fmaxf(am[sb], fabsf(r[sb][i]));
                }
                am[sb] = fmaxf(am[sb], __shfl_xor(am[sb], 16, 64));
                am[sb] = fmaxf(am[sb], __shfl_xor(am[sb], 32, 64));
                if (kg == 0) QM[(sb * WV + w) * 16 + r16] = am[sb];
            }
            __syncthreads();
#pragma unroll
            for (int sb = 0; sb < NS; sb++) {
                float m = 0.0f;
#pragma unroll
                for (int v = 0; v < WV; v++) m = fmaxf(m, QM[(sb * WV + v) * 16 + r16]);
                const float sc = (m == 0.0f) ? 1.0f : m / kE4M3Max;
                const float inv = 1.0f / sc;
                float y[4];
#pragma unroll
                for (int i = 0; i < 4; i++) y[i] = fmaxf(fminf(r[sb][i] * inv, kE4M3Max), -kE4M3Max);
                SO.v[q][w][sb][lane] = f32x2_to_e4m3x2(y[0], y[1]) | (f32x2_to_e4m3x2(y[2], y[3]) << 16);
                if (w == 0 && kg == 0) SO.sc[q][sb][r16] = sc;
            }
        } else {
#pragma unroll
            for (int sb = 0; sb < NS; sb++) {
                float r[4];
#pragma unroll
                for (int i = 0; i < 4; i++)
                    r[i] = GATED ? silu_mul(acc[sb][0][i], acc[sb][NW - 1][i]) : acc[sb][0][i];
                if constexpr (OUT == kOutF32) {
                    SO.v[q][w][sb][lane] = f32x4{r[0], r[1], r[2], r[3]};
                } else {
                    uint2 pk;
                    pk.x = (uint32_t)f32_to_bf16(r[0]) | ((uint32_t)f32_to_bf16(r[1]) << 16);
                    pk.y = (uint32_t)f32_to_bf16(r[2]) | ((uint32_t)f32_to_bf16(r[3]) << 16);
                    SO.v[q][w][sb][lane] = pk;
                }
            }
        }
        if (++nout % OUTQ == 0) flush(OUTQ);
    };
    auto task_n0 = [&](int i) {
        int mt, nb;
        task_at(i, mt, nb);
        return nb * FEAT + w * 16;
    };

    // Two context slots, used alternately (task i runs from slot i % 2 and reads ahead into
    // the other), so no loaded value is ever copied between registers.
    CT ca, cb;
    load_ctx(ca, 0, ca);
    load_ctx(cb, 1, ca);
#pragma unroll
    for (int d = 0; d < D; d++) issue_w(d, ca, d);
    stage_load(ca, 0);
    stage_store(0);
    __syncthreads();
    if (nch > 1) stage_load(ca, 1);
    else stage_load(cb, 0);
    zero_acc();

    int buf = 0;
    auto run_task = [&](int i, CT& cur, CT& nxt) {
        for (int c = 0; c < nch; c++) {
            const bool last = c == nch - 1;
#pragma unroll
            for (int s = 0; s < CS; s++) {
                if (c * CS + s < nsteps) compute(s % D, buf, s);
                if (!last || s + D < CS) issue_w(s % D, cur, c * CS + s + D);
                else issue_w(s % D, nxt, s + D - CS);
            }
            // publish the staged chunk (the next one of this task, or the first of the next
            // task) and start loading the one after it
            stage_store(buf ^ 1);
            __syncthreads();
            buf ^= 1;
            if (last) {
                epilogue(cur, task_n0(i));
                zero_acc();
                load_ctx(cur, i + 2, nxt);  // this slot now holds the task after the next
                if (nch > 1) stage_load(nxt, 1);
                else stage_load(cur, 0);
            } else if (c + 2 < nch) {
                stage_load(cur, c + 2);
            } else {
                stage_load(nxt, 0);
            }
        }
    };
    for (int i = 0; i < ntasks; i += 2) {
        run_task(i, ca, cb);
        if (i + 1 < ntasks) run_task(i + 1, cb, ca);
    }
    flush(nout % OUTQ);
}

// wavefronts per workgroup: 8 for the down GEMM (its short reduction makes the tile's staged
// activation rows a large share of the traffic: 128 features share them instead of 64) and
// for a gate/up GEMM that quantises its output (one 128-feature scale group per workgroup)
template <bool GATED, int OUT>
constexpr int stream_waves() { return GATED && OUT != kOutE4M3 ? 4 : 8; }

template <bool GATED, bool FP8, int OUT, int NS, int CS, int D>
hipError_t launch_stream(const GemmArgs& a, int max_tiles, int cus, hipStream_t st) {
    constexpr int WV = stream_waves<GATED, OUT>();
    constexpr bool LINE = !(GATED && FP8);
    static int per_cu = 0;
    if (per_cu == 0) {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_grouped_gemm_stream<GATED, FP8, OUT, NS, D, WV, CS, LINE>,
                                                          64 * WV, 0) != hipSuccess || nb < 1)
            nb = 1;
        per_cu = nb;
    }
    long long grid = (long long)max_tiles * (a.N / (16 * WV));
    const long long cap = (long long)cus * per_cu;
    if (grid > cap) grid = cap;
    grid = (grid + 7) / 8 * 8;  // a multiple of 8 for the per-XCD task order (extra workgroups exit)
    k_grouped_gemm_stream<GATED, FP8, OUT, NS, D, WV, CS, LINE><<<(unsigned)grid, 64 * WV, 0, st>>>(a);
    return hipGetLastError();
}

// Chunk length CS and weight ring depth D: bf16 8 and 8, FP8 4 and 4.  An FP8 down GEMM on
// 32-row tiles whose reduction is a multiple of 6 steps but not of 4 (768 deep: 6 steps) takes
// chunks of 2 steps with a ring of 2 instead: no chunk is padded past the reduction end (chunks
// of 4 pad a third of the steps; measured 10% slower), and a task spans several chunks, so the
// next tasks' activations are staged from gather-map entries loaded a task earlier rather than
// right after their load.  Chunks of 2 measured 1-1.5 us faster than one chunk of 6 at 64-256
// tokens of the 128-expert layer; rings of 3 and 6 were no faster than 2.
template <bool GATED, bool FP8, int OUT>
hipError_t launch_stream_rows(const GemmArgs& a, int tile_rows, int max_tiles, int cus, hipStream_t st) {
    constexpr int CS = SCfg<FP8>::CS, D = FP8 ? 4 : 8;
    if (tile_rows == 16) return launch_stream<GATED, FP8, OUT, 1, CS, D>(a, max_tiles, cus, st);
    if (tile_rows == 32) {
        if constexpr (FP8 && !GATED) {
            const int nsteps = a.K / SCfg<FP8>::KSTEP;
            if (nsteps % 6 == 0 && nsteps % CS != 0) return launch_stream<GATED, FP8, OUT, 2, 2, 2>(a, max_tiles, cus, st);
        }
        return launch_stream<GATED, FP8, OUT, 2, CS, D>(a, max_tiles, cus, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_grouped_gemm_stream(bool gated, bool fp8, int out_mode, const GemmArgs& a, int tile_rows,
                                      int max_tiles, int cus, hipStream_t st) {
    if (gated) {
        if (fp8) {
            if (out_mode == kOutE4M3) {
                if (a.N % 128 || !a.out_scale) return hipErrorInvalidValue;
                return launch_stream_rows<true, true, kOutE4M3>(a, tile_rows, max_tiles, cus, st);
            }
            return out_mode == kOutF32 ? launch_stream_rows<true, true, kOutF32>(a, tile_rows, max_tiles, cus, st)
                                       : launch_stream_rows<true, true, kOutBf16>(a, tile_rows, max_tiles, cus, st);
        }
        if (out_mode != kOutBf16) return hipErrorInvalidValue;
        return launch_stream_rows<true, false, kOutBf16>(a, tile_rows, max_tiles, cus, st);
    }
    if (out_mode != kOutBf16) return hipErrorInvalidValue;
    if (fp8) return launch_stream_rows<false, true, kOutBf16>(a, tile_rows, max_tiles, cus, st);
    return launch_stream_rows<false, false, kOutBf16>(a, tile_rows, max_tiles, cus, st);
}

}  // namespace fmoe

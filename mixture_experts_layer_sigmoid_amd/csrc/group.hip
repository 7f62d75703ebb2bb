// group.hip -- per-expert grouping of the routed rows and the row-tile list of the grouped
// GEMMs.
//
// The flat assignments i = t*k + j are cut into chunks of 64, one wavefront each.  Inside a
// chunk the lanes that hold the same local expert find each other with one wavefront ballot
// per bit of the local expert index, so each assignment gets its rank among the earlier
// assignments of its expert in the chunk and each (chunk, expert) its count, without atomics.  A scan per expert over the chunks
// and a scan over the experts then give every (chunk, expert) its first grouped row, and a
// last pass writes every assignment to base + rank.  The result is the stable counting sort
// (experts ascending, flat index ascending inside an expert), identical on every run.
//
// Small batches (at most 64 chunks) run all three phases in one workgroup and one launch;
// larger ones run a counting launch over all chunks, a one-workgroup scan, and a scatter
// launch, so the ballot work spreads over the whole GPU.  Up to 16 tokens the forward routes
// and groups in one launch (k_route_group_small); there, up to 64 assignments (one chunk) are
// grouped by a single wavefront with wavefront scans, without workgroup barriers.
//
// Row tiles: the grouped GEMMs are cut per expert from the real row count, not from the
// token count ("vLLM Community Traces H20 MoE Scheduling Inefficiency to Expert-Load Kernel
// Selection", paragraphs 3-4): an expert with 1..tile_rows rows becomes one tile of the light
// GEMM kernel, a heavier one (a hot expert of a concentrated routing, or any expert of a large
// batch) is cut into tiles of at most 256 rows for the heavy kernel (bf16 in a launch with many
// heavy tasks: an expert of 257..320 rows is one tile), rows spread as evenly as 16-row steps
// allow.  When the host knows that no expert can exceed light_cap rows (a few
// light tiles), experts above tile_rows are cut into several light tiles instead, and the
// heavy-tile launches are left out.
#include "launch.hpp"
#include "router_row.hpp"

namespace fmoe {

constexpr int kScanThreads = 1024;
constexpr int kSmallChunks = 64;  // chunks of the one-workgroup path
constexpr int kSmallPerWave = kSmallChunks / (kScanThreads / 64);  // chunks per wavefront there
// LDS ints of scan_and_tile for El local experts: part sums, three per-expert arrays, a flag
__host__ __device__ constexpr int scan_lds_ints(int El) { return kScanThreads + 3 * El + 1; }

// Phase 1 for one chunk of 64 assignments, by one wavefront.  Writes the chunk's count of
// every local expert to col[e * col_stride] (zeros included) and returns, for this lane, the
// local expert (-1 when not local) and its rank inside the chunk; *bad gets the number of
// ids outside [0, E) in the chunk (same value in every lane).  `mask` is per-wavefront LDS
// scratch of El entries.
// chunk_rank_id takes this lane's id already loaded (valid: the lane holds an assignment).
__device__ void chunk_rank_id(int id, bool valid, int E, int El, int lo, int* col, int col_stride, int* mask,
                              int* out_l, int* out_r, int* bad) {
    const int lane = lane_id();
    for (int e = lane; e < El; e += 64) mask[e] = 0;
    int l = -1, b = 0;
    if (valid) {
        if (id < 0 || id >= E) b = 1;
        else if (id - lo >= 0 && id - lo < El) l = id - lo;
    }
    *bad = __popcll(__ballot(b));
    // lanes with the same local expert: those that agree with this lane on every bit of l (one
    // ballot per bit of El - 1), among the lanes holding a local expert
    const unsigned long long live = __ballot(l >= 0);
    unsigned long long same = live;
    const int nbits = El > 1 ? 32 - __clz(El - 1) : 0;
    for (int bit = 0; bit < nbits; bit++) {
        const bool set = (l >> bit) & 1;
        const unsigned long long m = __ballot(set);
        same &= set ? m : ~m;
    }
    int r = -1;
    if (l >= 0) {
        r = __popcll(same & ((1ull << lane) - 1ull));
        if (r == 0) mask[l] = __popcll(same);  // the first lane of each expert writes its count
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int e = lane; e < El; e += 64) col[e * col_stride] = mask[e];
    *out_l = l;
    *out_r = r;
}

__device__ __forceinline__ void chunk_rank(const int32_t* __restrict__ ids, int n, int E, int El, int lo, int chunk,
                                           int* col, int col_stride, int* mask, int* out_l, int* out_r, int* bad) {
    const int i = chunk * 64 + lane_id();
    chunk_rank_id(i < n ? ids[i] : 0, i < n, E, El, lo, col, col_stride, mask, out_l, out_r, bad);
}

// Which gate/up kernel takes the light tiles: the split-reduction one when sparse_rows > 0 and
// the light tiles hold fewer than sparse_rows rows on average (the cold experts of a
// concentrated batch, one or two rows each), else the streaming one.  Decided here from the real
// counts, so the host launches both and the one without tiles exits at once.
__device__ __forceinline__ void write_light_split(DevHeader* hdr, int n_light, int light_rows, int sparse_rows) {
    const bool split = sparse_rows > 0 && n_light > 0 && (long long)light_rows < (long long)sparse_rows * n_light;
    hdr->light_rows = light_rows;
    hdr->m_tiles_stream = split ? 0 : n_light;
    hdr->m_tiles_split = split ? n_light : 0;
}

// Phase 2 by one workgroup of kScanThreads: turns cnt[c * El + e] (count of expert e in
// chunk c) into the first grouped row of (e, c); writes counts, offsets, the row tiles and
// the header.  Thread t works on expert e = t % El' and part p = t / El' of its chunks
// (El' = El rounded up to a power of two, P = kScanThreads / El' parts), so consecutive
// threads read consecutive experts of a chunk.  The scan over the experts (grouped rows, light
// and heavy tiles before each expert) is one wavefront's: lane j takes experts j*J .. j*J+J-1
// (J = ceil(El/64)) in order, then one wavefront scan adds the lanes' sums.  dropped is read by
// wavefront 0 only.
__device__ void scan_and_tile(int* cnt, int nchunk, int El, int tile_rows, int light_cap, int heavy5_min,
                              int rows_estimate, int sparse_rows, long long dropped,
                              int32_t* __restrict__ counts, int32_t* __restrict__ offsets, MTile* __restrict__ mtiles,
                              MTile* __restrict__ mtiles_heavy, DevHeader* __restrict__ hdr,
                              int* sh /* >= scan_lds_ints(El) ints */) {
    int Ep = 1;
    while (Ep < El) Ep <<= 1;
    const int P = kScanThreads / Ep;  // parts per expert (>= 1 since El <= 1024)
    const int e = threadIdx.x % Ep, part = threadIdx.x / Ep;
    const bool live = e < El;
    const int per = (nchunk + P - 1) / P;
    const int c0 = min(nchunk, part * per), c1 = min(nchunk, c0 + per);
    int s = 0;
    if (live) {
        int c = c0;
        for (; c + 8 <= c1; c += 8) {
            int v[8];
#pragma unroll
            for (int j = 0; j < 8; j++) v[j] = cnt[(c + j) * El + e];
#pragma unroll
            for (int j = 0; j < 8; j++) s += v[j];
        }
        for (; c < c1; c++) s += cnt[c * El + e];
    }
    int* part_sum = sh;               // [kScanThreads]
    int* e_rows = sh + kScanThreads;  // [El]: rows of expert e, then its first grouped row
    int* e_light = e_rows + El;       // [El]: its light tiles, then the light tiles before it
    int* e_heavy = e_light + El;      // [El]: its heavy tiles, then the heavy tiles before it
    int* five = e_heavy + El;         // [1]: experts of 257..320 rows are one tile
    part_sum[threadIdx.x] = s;
    __syncthreads();
    int before = 0, total = 0;  // this part's prefix inside its expert, and the expert total
    for (int q = 0; q < P; q++) {
        const int v = part_sum[q * Ep + e];
        if (q < part) before += v;
        total += v;
    }
    // an expert with 1..light_cap rows is cut into light tiles of tile_rows rows (the last one
    // takes the rest); a heavier one is cut into ceil(total / 256) tiles of equal size rounded up
    // to 16 rows (the last one takes the rest), so the tiles of one expert carry about the same
    // work -- except that an expert of 257..320 rows is one tile of five 64-row groups when
    // the 256-row tiles of all experts number heavy5_min or more (a launch with several tasks
    // per compute unit, where one task in place of two saves the second task's weight copies)
    const bool heavy = total > light_cap;
    const int nlight = (total > 0 && !heavy) ? (total + tile_rows - 1) / tile_rows : 0;
    const bool five_able = heavy && total > kHeavyRows && total <= kHeavyRows5;
    if (live && part == 0) {
        e_rows[e] = total;
        e_light[e] = nlight;
        e_heavy[e] = heavy ? (total + kHeavyRows - 1) / kHeavyRows : 0;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int J = (El + 63) >> 6;
        const int ea = min(El, lane * J), eb = min(El, ea + J);
        int sr = 0, sl = 0, sh_ = 0, lrows = 0, empty = 0, mx = 0, n5 = 0;
        for (int x = ea; x < eb; x++) {
            const int r = e_rows[x], l = e_light[x], h = e_heavy[x];
            sr += r;
            sl += l;
            sh_ += h;
            n5 += h > 0 && r > kHeavyRows && r <= kHeavyRows5;
            lrows += l > 0 ? r : 0;
            empty += r == 0;
            mx = max(mx, r);
        }
        int all256 = sh_;  // heavy tiles of 256 rows, all experts
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) all256 += __shfl_xor(all256, o, 64);
        const bool use5 = all256 >= heavy5_min;
        if (use5 && n5 > 0) {
            sh_ -= n5;  // two tiles become one
            for (int x = ea; x < eb; x++) {
                const int r = e_rows[x];
                if (e_heavy[x] > 0 && r > kHeavyRows && r <= kHeavyRows5) e_heavy[x] = 1;
            }
        }
        if (lane == 0) *five = use5;
        // inclusive scans of the lanes' sums (rows, light tiles, heavy tiles, light rows, empty experts)
        int ir = sr, il = sl, ih = sh_, ilr = lrows, ie = empty;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int yr = __shfl_up(ir, o, 64), yl = __shfl_up(il, o, 64), yh = __shfl_up(ih, o, 64);
            const int ylr = __shfl_up(ilr, o, 64), ye = __shfl_up(ie, o, 64);
            if (lane >= o) {
                ir += yr;
                il += yl;
                ih += yh;
                ilr += ylr;
                ie += ye;
            }
        }
        mx = wave_max(mx);
        int fr = ir - sr, fl = il - sl, fh = ih - sh_;  // before this lane's first expert
        for (int x = ea; x < eb; x++) {
            const int r = e_rows[x], l = e_light[x], h = e_heavy[x];
            e_rows[x] = fr;
            e_light[x] = fl;
            e_heavy[x] = fh;
            fr += r;
            fl += l;
            fh += h;
        }
        if (lane == 63) {
            offsets[El] = ir;
            hdr->m_tiles = il;
            hdr->m_tiles_heavy = ih;
            hdr->local_rows = ir;
            hdr->max_rows = mx;
            hdr->empty_experts = ie;
            hdr->dropped = dropped;
            hdr->tile_rows = tile_rows;
            hdr->heavy_rows = use5 ? kHeavyRows5 : kHeavyRows;
            hdr->rows_estimate = rows_estimate;
            write_light_split(hdr, il, ilr, sparse_rows);
        }
    }
    __syncthreads();
    const int cap = five_able && *five ? kHeavyRows5 : kHeavyRows;
    const int nheavy0 = heavy ? (total + cap - 1) / cap : 0;
    const int hrows = heavy ? min(cap, ((total + nheavy0 - 1) / nheavy0 + 15) / 16 * 16) : 1;
    const int nheavy = heavy ? (total + hrows - 1) / hrows : 0;  // == nheavy0, the count scanned above
    if (live) {
        const int my_first = e_rows[e], my_lfirst = e_light[e], my_hfirst = e_heavy[e];
        int run = my_first + before;
        int c = c0;
        for (; c + 8 <= c1; c += 8) {
            int v[8];
#pragma unroll
            for (int j = 0; j < 8; j++) v[j] = cnt[(c + j) * El + e];
#pragma unroll
            for (int j = 0; j < 8; j++) {
                cnt[(c + j) * El + e] = run;
                run += v[j];
            }
        }
        for (; c < c1; c++) {
            const int v = cnt[c * El + e];
            cnt[c * El + e] = run;
            run += v;
        }
        if (part == 0) {
            counts[e] = total;
            offsets[e] = my_first;
        }
        // row tiles of expert e (split over its P threads)
        for (int j = part; j < nlight; j += P) {
            MTile mt;
            mt.expert = e;
            mt.row0 = my_first + j * tile_rows;
            mt.rows = min(tile_rows, total - j * tile_rows);
            mt.group = 0;
            mtiles[my_lfirst + j] = mt;
        }
        if (heavy) {
            for (int j = part; j < nheavy; j += P) {
                MTile mt;
                mt.expert = e;
                mt.row0 = my_first + j * hrows;
                mt.rows = min(hrows, total - j * hrows);
                // nheavy <= 2^23 / 256 = 32768 (bit 31 when it is 32768: read back unsigned)
                mt.group = (int)((uint32_t)j | ((uint32_t)nheavy << 16));
                mtiles_heavy[my_hfirst + j] = mt;
            }
        }
    }
}

// Phase 3 for one assignment: it goes to base(expert, chunk) + rank.
__device__ __forceinline__ void chunk_scatter(int i, int n, int l, int r, int base, int32_t* __restrict__ perm_src,
                                              int32_t* __restrict__ inv_perm) {
    if (i >= n) return;
    if (l >= 0) {
        const int pos = base + r;
        perm_src[pos] = i;
        inv_perm[i] = pos;
    } else {
        inv_perm[i] = -1;
    }
}

// ---------------------------------------------------------------- one-workgroup path

// All three phases by one workgroup of kScanThreads.  ids may point to global memory or to
// LDS (generic addressing); lds holds small_lds_ints(n, El) ints.
__device__ __forceinline__ void group_small(const int32_t* ids, int n, int E, int El, int lo, int tile_rows,
                                            int light_cap, int heavy5_min, int rows_estimate, int sparse_rows, int32_t* __restrict__ counts,
                                            int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src,
                                            int32_t* __restrict__ inv_perm, MTile* __restrict__ mtiles,
                                            MTile* __restrict__ mtiles_heavy, DevHeader* __restrict__ hdr, int* lds) {
    const int nchunk = (n + 63) / 64;  // <= kSmallChunks
    constexpr int NW = kScanThreads / 64;
    int* cnt = lds;                        // [nchunk][El]
    int* mask = cnt + El * nchunk;         // [NW][El]
    int* bads = mask + NW * El;            // [kSmallChunks]
    int* sh = bads + kSmallChunks;         // scan scratch [scan_lds_ints(El)]
    const int w = threadIdx.x >> 6;
    // wavefront w ranks chunks w, w + NW, ...; the ids of all its chunks are loaded first, so
    // the wavefront waits for memory once rather than once per chunk
    int idv[kSmallPerWave];
#pragma unroll
    for (int j = 0; j < kSmallPerWave; j++) {
        const int i = (w + j * NW) * 64 + lane_id();
        idv[j] = i < n ? ids[i] : 0;
    }
    int l[kSmallPerWave], r[kSmallPerWave];
#pragma unroll
    for (int j = 0; j < kSmallPerWave; j++) {
        const int c = w + j * NW;
        l[j] = r[j] = -1;
        if (c < nchunk) {
            int bad = 0;
            chunk_rank_id(idv[j], c * 64 + lane_id() < n, E, El, lo, cnt + c * El, 1, mask + w * El, &l[j], &r[j],
                          &bad);
            if (lane_id() == 0) bads[c] = bad;
        }
    }
    __syncthreads();
    long long dropped = 0;  // wavefront 0 only (the one that writes the header)
    if (w == 0) {
        int d = 0;
        for (int c = lane_id(); c < nchunk; c += 64) d += bads[c];  // <= 64 per chunk, <= 64 chunks
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) d += __shfl_xor(d, o, 64);
        dropped = d;
    }
    scan_and_tile(cnt, nchunk, El, tile_rows, light_cap, heavy5_min, rows_estimate, sparse_rows, dropped, counts, offsets, mtiles,
                  mtiles_heavy, hdr, sh);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSmallPerWave; j++) {
        const int c = w + j * NW;
        if (c < nchunk)
            chunk_scatter(c * 64 + lane_id(), n, l[j], r[j], l[j] >= 0 ? cnt[c * El + l[j]] : 0, perm_src, inv_perm);
    }
}

static size_t small_lds_ints(int n, int El) {
    const int nchunk = (n + 63) / 64;
    return (size_t)El * nchunk + (size_t)(kScanThreads / 64) * El + kSmallChunks + scan_lds_ints(El);
}

__global__ __launch_bounds__(kScanThreads) void k_group_small(const int32_t* __restrict__ ids, int n, int E, int El,
                                                             int lo, int tile_rows, int light_cap, int heavy5_min,
                                                             int rows_estimate, int sparse_rows,
                                                             int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ perm_src,
                                                             int32_t* __restrict__ inv_perm, MTile* __restrict__ mtiles,
                                                             MTile* __restrict__ mtiles_heavy,
                                                             DevHeader* __restrict__ hdr) {
    extern __shared__ int lds[];
    group_small(ids, n, E, El, lo, tile_rows, light_cap, heavy5_min, rows_estimate, sparse_rows, counts, offsets, perm_src, inv_perm,
                mtiles, mtiles_heavy, hdr, lds);
}

// All three phases by one wavefront, for at most 64 assignments (one chunk) of which no expert
// holds more than tile_rows (so every expert with rows is one light tile).  The results are
// those of group_small: the chunk's counts are the expert totals, the exclusive scans over the
// experts in ascending order give the offsets and the light tile slots, and each assignment
// goes to its expert's offset plus its rank in the chunk.  cnt: El ints of LDS.
__device__ void group_wave(const int32_t* ids, int n, int E, int El, int lo, int tile_rows, int heavy5_min,
                           int rows_estimate, int sparse_rows, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                           int32_t* __restrict__ perm_src, int32_t* __restrict__ inv_perm,
                           MTile* __restrict__ mtiles, DevHeader* __restrict__ hdr, int* cnt) {
    const int lane = lane_id();
    int l, r, bad;
    chunk_rank(ids, n, E, El, lo, 0, cnt, 1, cnt, &l, &r, &bad);  // cnt[e]: rows of expert e
    // lane holds experts lane, lane + 64, ...: one wavefront scan per group of 64 experts
    int run_rows = 0, run_tiles = 0, maxc = 0;
    for (int e0 = 0; e0 < El; e0 += 64) {
        const int e = e0 + lane;
        const int c = e < El ? cnt[e] : 0;  // written by this lane in chunk_rank's copy
        int sr = c, st = c > 0 ? 1 : 0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int yr = __shfl_up(sr, o, 64), yt = __shfl_up(st, o, 64);
            if (lane >= o) {
                sr += yr;
                st += yt;
            }
        }
        const int first = run_rows + sr - c, lfirst = run_tiles + st - (c > 0 ? 1 : 0);
        if (e < El) {
            counts[e] = c;
            offsets[e] = first;
            cnt[e] = first;
            if (c > 0) {
                MTile mt;
                mt.expert = e;
                mt.row0 = first;
                mt.rows = c;
                mt.group = 0;
                mtiles[lfirst] = mt;
            }
        }
        run_rows += __shfl(sr, 63, 64);
        run_tiles += __shfl(st, 63, 64);
        maxc = c > maxc ? c : maxc;
    }
    maxc = wave_max(maxc);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    chunk_scatter(lane, n, l, r, l >= 0 ? cnt[l] : 0, perm_src, inv_perm);
    if (lane == 0) {
        offsets[El] = run_rows;
        hdr->m_tiles = run_tiles;
        hdr->m_tiles_heavy = 0;
        hdr->local_rows = run_rows;
        hdr->max_rows = maxc;
        hdr->empty_experts = El - run_tiles;
        hdr->dropped = bad;
        hdr->tile_rows = tile_rows;
        hdr->heavy_rows = kHeavyRows;
        hdr->rows_estimate = rows_estimate;
        write_light_split(hdr, run_tiles, run_rows, sparse_rows);
    }
}

// Router top-k and grouping in one launch for at most kFusedTokens tokens: wavefront t routes
// token t (plain top-k, the router kernel's row code), writing ids and weights to global memory
// and the ids to LDS as well; after one barrier the workgroup groups the ids from LDS.  No
// expert can exceed a light tile (router ids are distinct per token and every light tile holds
// 16 rows or more), so up to 64 assignments one wavefront groups them alone.  Routing more
// tokens per launch, several per wavefront, measured slower than the two launches (T=32:
// 15.8 us against 12.8 us for router + grouping).
constexpr int kFusedTokens = kScanThreads / 64;
constexpr int kWaveGroupTokens = 16;

template <int SLOTS, bool BF16_IN, bool QX>
__global__ __launch_bounds__(kScanThreads) void k_route_group_small(
    const void* __restrict__ logits, int T, int E, int k, int scoring, int renorm, int32_t* __restrict__ ids,
    float* __restrict__ weights, int El, int lo, int tile_rows, int light_cap, int heavy5_min, int rows_estimate, int sparse_rows,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src,
    int32_t* __restrict__ inv_perm, MTile* __restrict__ mtiles, MTile* __restrict__ mtiles_heavy,
    DevHeader* __restrict__ hdr, XQuant xq) {
    extern __shared__ int lds[];
    const int n = T * k;
    int* ids_lds = lds;  // [n], padded to 4 ints
    const int w = threadIdx.x >> 6;
    if (QX && blockIdx.x > 0) {  // FP8: workgroups 1.. quantise x, one 128-column group per wavefront
        const long long g = (long long)(blockIdx.x - 1) * (kScanThreads / 64) + w;
        if (g < (long long)T * (xq.H >> 7)) quant_group_bf16_wave((const uint16_t*)xq.x, xq.H, g, xq.q, xq.s);
        return;
    }
    if (w < T) topk_row<SLOTS, BF16_IN>(logits, w, E, k, scoring, renorm, 1, 1, ids, weights, ids_lds + w * k);
    __syncthreads();
    if (n <= 64 && T <= kWaveGroupTokens) {
        if (w == 0)
            group_wave(ids_lds, n, E, El, lo, tile_rows, heavy5_min, rows_estimate, sparse_rows, counts, offsets, perm_src,
                       inv_perm, mtiles, hdr, lds + ((n + 3) & ~3));
        return;
    }
    group_small(ids_lds, n, E, El, lo, tile_rows, light_cap, heavy5_min, rows_estimate, sparse_rows, counts, offsets, perm_src,
                inv_perm, mtiles, mtiles_heavy, hdr, lds + ((n + 3) & ~3));
}

// ---------------------------------------------------------------- multi-workgroup path
//
// From kBlockPathChunks chunks on, blocks of kBlockChunks chunks, one workgroup each (one
// wavefront per chunk): the counting launch ranks the block's chunks and sums its counts per
// expert; the one-workgroup scan runs over those block sums (kBlockChunks times fewer than the chunk counts, which one CU would
// otherwise read twice and write once: 14 us of the 23 us grouping at 2^15 assignments); the
// scatter launch turns the block's chunk counts into first grouped rows and places its
// assignments.

constexpr int kBlockChunks = 8;                  // chunks per block
constexpr int kBlockThreads = kBlockChunks * 64;  // one wavefront per chunk
constexpr int kBlockPathChunks = 256;             // from this many chunks on (fewer: the chunk-level
                                                  // path, whose one-workgroup scan is short there)

// Chunk-level path (fewer than kBlockPathChunks chunks).  Phase 1, one wavefront per chunk,
// 4 per workgroup: counts go to cnt[chunk * El + e], ranks to
// rank_buf, the chunk's ids outside [0,E) to bad_buf[chunk].
__global__ __launch_bounds__(256) void k_group_count(const int32_t* __restrict__ ids, int n, int E, int El, int lo,
                                                     int nchunk, int* __restrict__ cnt, int32_t* __restrict__ rank_buf,
                                                     int* __restrict__ bad_buf) {
    extern __shared__ int lds[];
    const int w = threadIdx.x >> 6;
    const int chunk = blockIdx.x * 4 + w;
    if (chunk >= nchunk) return;
    int l, r, bad;
    chunk_rank(ids, n, E, El, lo, chunk, cnt + (size_t)chunk * El, 1, lds + w * El, &l, &r, &bad);
    const int i = chunk * 64 + lane_id();
    if (i < n) rank_buf[i] = r;
    if (lane_id() == 0) bad_buf[chunk] = bad;
}

// Phase 1 for one block: counts to cnt[chunk * El + e], ranks to rank_buf, the chunk's ids
// outside [0,E) to bad_buf[chunk], the block's count of each local expert to
// bsum[block * El + e].
__global__ __launch_bounds__(kBlockThreads) void k_group_count_blocks(const int32_t* __restrict__ ids, int n, int E, int El,
                                                                     int lo, int nchunk, int* __restrict__ cnt,
                                                                     int32_t* __restrict__ rank_buf,
                                                                     int* __restrict__ bad_buf, int* __restrict__ bsum) {
    extern __shared__ int lds[];  // [8][El]: one mask per wavefront
    const int w = threadIdx.x >> 6;
    const int c0 = blockIdx.x * kBlockChunks, c1 = min(nchunk, c0 + kBlockChunks);
    if (c0 + w < c1) {
        const int c = c0 + w;
        int l, r, bad;
        chunk_rank(ids, n, E, El, lo, c, cnt + (size_t)c * El, 1, lds + w * El, &l, &r, &bad);
        const int i = c * 64 + lane_id();
        if (i < n) rank_buf[i] = r;
        if (lane_id() == 0) bad_buf[c] = bad;
    }
    __syncthreads();  // this workgroup's counts are visible to all its threads
    for (int e = threadIdx.x; e < El; e += kBlockThreads) {
        int v[kBlockChunks];
#pragma unroll
        for (int j = 0; j < kBlockChunks; j++) v[j] = c0 + j < c1 ? cnt[(size_t)(c0 + j) * El + e] : 0;
        int sum = 0;
#pragma unroll
        for (int j = 0; j < kBlockChunks; j++) sum += v[j];
        bsum[(size_t)blockIdx.x * El + e] = sum;
    }
}

// Phase 2 over a [nblock][El] count matrix (the chunk counts, or the block sums):
// bsum[block * El + e] becomes the first grouped row of expert e in that chunk or block;
// counts, offsets, tiles and header as in the one-workgroup path.  bad_buf holds nchunk entries.
__global__ __launch_bounds__(kScanThreads) void k_group_scan(int* __restrict__ bsum, int nblock, int nchunk, int El,
                                                            int tile_rows, int light_cap, int heavy5_min, int rows_estimate,
                                                            int sparse_rows, const int* __restrict__ bad_buf,
                                                            int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                            MTile* __restrict__ mtiles, MTile* __restrict__ mtiles_heavy,
                                                            DevHeader* __restrict__ hdr) {
    __shared__ int sh[scan_lds_ints(kScanThreads)];  // El <= kScanThreads (1024 local experts at most)
    __shared__ long long dsum[kScanThreads / 64];
    long long d = 0;
    for (int c = threadIdx.x; c < nchunk; c += kScanThreads) d += bad_buf[c];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) d += __shfl_xor(d, o, 64);
    if (lane_id() == 0) dsum[threadIdx.x >> 6] = d;
    __syncthreads();
    long long dropped = 0;
    for (int q = 0; q < kScanThreads / 64; q++) dropped += dsum[q];
    scan_and_tile(bsum, nblock, El, tile_rows, light_cap, heavy5_min, rows_estimate, sparse_rows, dropped, counts, offsets,
                  mtiles, mtiles_heavy, hdr, sh);
}

// Phase 3 for one block: the first grouped row of each (chunk, expert) is the block's first
// row of the expert plus the counts of the block's earlier chunks; then every assignment goes
// to its chunk's row plus its rank.
__global__ __launch_bounds__(kBlockThreads) void k_group_scatter_blocks(const int32_t* __restrict__ ids, int n, int E, int El,
                                                                       int lo, int nchunk, int* __restrict__ cnt,
                                                                       const int* __restrict__ bsum,
                                                                const int32_t* __restrict__ rank_buf,
                                                                int32_t* __restrict__ perm_src,
                                                                int32_t* __restrict__ inv_perm) {
    const int c0 = blockIdx.x * kBlockChunks, c1 = min(nchunk, c0 + kBlockChunks);
    for (int e = threadIdx.x; e < El; e += kBlockThreads) {
        int v[kBlockChunks];  // all loads first, then the stores
#pragma unroll
        for (int j = 0; j < kBlockChunks; j++) v[j] = c0 + j < c1 ? cnt[(size_t)(c0 + j) * El + e] : 0;
        int run = bsum[(size_t)blockIdx.x * El + e];
#pragma unroll
        for (int j = 0; j < kBlockChunks; j++) {
            if (c0 + j < c1) cnt[(size_t)(c0 + j) * El + e] = run;
            run += v[j];
        }
    }
    __syncthreads();  // this workgroup's first rows are visible to all its threads
    const int i1 = min(n, c1 * 64);
    for (int i = c0 * 64 + (int)threadIdx.x; i < i1; i += kBlockThreads) {
        const int id = ids[i];
        const int l = (id >= 0 && id < E && id - lo >= 0 && id - lo < El) ? id - lo : -1;
        chunk_scatter(i, n, l, rank_buf[i], l >= 0 ? cnt[(size_t)(i / 64) * El + l] : 0, perm_src, inv_perm);
    }
}

// Chunk-level phase 3: every assignment goes to its chunk's first row of its expert plus its rank.
__global__ __launch_bounds__(256) void k_group_scatter(const int32_t* __restrict__ ids, int n, int E, int El, int lo,
                                                       int nchunk, const int* __restrict__ cnt,
                                                       const int32_t* __restrict__ rank_buf,
                                                       int32_t* __restrict__ perm_src, int32_t* __restrict__ inv_perm) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int id = ids[i];
    const int l = (id >= 0 && id < E && id - lo >= 0 && id - lo < El) ? id - lo : -1;
    chunk_scatter(i, n, l, rank_buf[i], l >= 0 ? cnt[(size_t)(i / 64) * El + l] : 0, perm_src, inv_perm);
}

size_t group_scratch_bytes(long long n, int El) {
    const long long nchunk = (n + 63) / 64, nblock = (nchunk + kBlockChunks - 1) / kBlockChunks;
    return (size_t)(nchunk * El + nchunk + nblock * El) * sizeof(int);
}

hipError_t launch_group(const int32_t* ids, int n, int E, int El, int lo, int tile_rows, int light_cap,
                        int heavy5_min, int rows_estimate, int sparse_rows,
                        int32_t* counts, int32_t* offsets, int32_t* perm_src, int32_t* inv_perm, int32_t* rank_buf,
                        int* scratch, MTile* mtiles, MTile* mtiles_heavy, DevHeader* hdr, hipStream_t st) {
    const int nchunk = (n + 63) / 64;
    const size_t lds = small_lds_ints(n, El) * 4;
    if (nchunk <= kSmallChunks && lds <= 65536) {
        k_group_small<<<1, kScanThreads, lds, st>>>(ids, n, E, El, lo, tile_rows, light_cap, heavy5_min, rows_estimate, sparse_rows,
                                                    counts,
                                                    offsets,
                                                    perm_src, inv_perm, mtiles, mtiles_heavy, hdr);
        return hipGetLastError();
    }
    int* cnt = scratch;                    // [nchunk][El]
    int* bad = cnt + (size_t)El * nchunk;  // [nchunk]
    if (nchunk < kBlockPathChunks) {
        k_group_count<<<(nchunk + 3) / 4, 256, (size_t)4 * El * 4, st>>>(ids, n, E, El, lo, nchunk, cnt, rank_buf, bad);
        k_group_scan<<<1, kScanThreads, 0, st>>>(cnt, nchunk, nchunk, El, tile_rows, light_cap, heavy5_min, rows_estimate,
                                                 sparse_rows, bad, counts, offsets, mtiles, mtiles_heavy, hdr);
        k_group_scatter<<<(n + 255) / 256, 256, 0, st>>>(ids, n, E, El, lo, nchunk, cnt, rank_buf, perm_src, inv_perm);
        return hipGetLastError();
    }
    const int nblock = (nchunk + kBlockChunks - 1) / kBlockChunks;
    int* bsum = bad + nchunk;  // [nblock][El]
    k_group_count_blocks<<<nblock, kBlockThreads, (size_t)(kBlockThreads / 64) * El * 4, st>>>(ids, n, E, El, lo, nchunk,
                                                                                                cnt, rank_buf, bad, bsum);
    k_group_scan<<<1, kScanThreads, 0, st>>>(bsum, nblock, nchunk, El, tile_rows, light_cap, heavy5_min, rows_estimate,
                                             sparse_rows, bad, counts, offsets, mtiles, mtiles_heavy, hdr);
    k_group_scatter_blocks<<<nblock, kBlockThreads, 0, st>>>(ids, n, E, El, lo, nchunk, cnt, bsum, rank_buf, perm_src,
                                                            inv_perm);
    return hipGetLastError();
}

static size_t route_group_lds_bytes(int T, int k, int El) {
    const int n = T * k;
    return ((size_t)((n + 3) & ~3) + small_lds_ints(n, El)) * 4;
}

bool route_group_fits(int T, int k, int E, int El) {
    static_assert(kFusedTokens <= kScanThreads / 64 && kWaveGroupTokens <= 16, "one wavefront per token; every "
                  "light tile holds at least 16 rows");
    return T >= 1 && T <= kFusedTokens && (T * k + 63) / 64 <= kSmallChunks && E <= 1024 &&
           route_group_lds_bytes(T, k, El) <= 65536;
}

template <int SLOTS>
static void launch_route_group_slots(const void* logits, bool bf16, int T, int E, int k, int scoring, int renorm,
                                     int32_t* ids, float* weights, int El, int lo, int tile_rows, int light_cap,
                                     int heavy5_min, int rows_estimate, int sparse_rows, int32_t* counts, int32_t* offsets,
                                     int32_t* perm_src, int32_t* inv_perm, MTile* mtiles, MTile* mtiles_heavy,
                                     DevHeader* hdr, hipStream_t st, const XQuant* xq) {
    const size_t lds = route_group_lds_bytes(T, k, El);
    const XQuant none = {nullptr, 0, nullptr, nullptr};
    auto kern = bf16 ? (xq ? k_route_group_small<SLOTS, true, true> : k_route_group_small<SLOTS, true, false>)
                     : (xq ? k_route_group_small<SLOTS, false, true> : k_route_group_small<SLOTS, false, false>);
    // workgroup 0 routes and groups; FP8: one more workgroup per 16 groups of x to quantise
    const unsigned blocks = xq ? 1 + (unsigned)((T * (xq->H / 128) + kScanThreads / 64 - 1) / (kScanThreads / 64)) : 1;
    kern<<<blocks, kScanThreads, lds, st>>>(logits, T, E, k, scoring, renorm, ids, weights, El, lo, tile_rows,
                                            light_cap, heavy5_min, rows_estimate, sparse_rows, counts, offsets, perm_src, inv_perm,
                                            mtiles, mtiles_heavy, hdr, xq ? *xq : none);
}

hipError_t launch_route_group(const void* logits, bool bf16, int T, int E, int k, int scoring, int renorm,
                              int32_t* ids, float* weights, int El, int lo, int tile_rows, int light_cap,
                              int heavy5_min, int rows_estimate, int sparse_rows, int32_t* counts, int32_t* offsets, int32_t* perm_src,
                              int32_t* inv_perm, MTile* mtiles, MTile* mtiles_heavy, DevHeader* hdr, hipStream_t st,
                              const XQuant* xq) {
    if (!route_group_fits(T, k, E, El)) return hipErrorInvalidValue;
    if (xq && (!xq->x || !xq->q || !xq->s || xq->H <= 0 || xq->H % 128)) return hipErrorInvalidValue;
    const int slots = (E + 63) / 64;
#define FMOE_RG(S)                                                                                                  \
    launch_route_group_slots<S>(logits, bf16, T, E, k, scoring, renorm, ids, weights, El, lo, tile_rows, light_cap, \
                                heavy5_min, rows_estimate, sparse_rows, counts, offsets, perm_src, inv_perm, mtiles, mtiles_heavy,   \
                                hdr, st, xq)
    if (slots <= 1) FMOE_RG(1);
    else if (slots <= 2) FMOE_RG(2);
    else if (slots <= 4) FMOE_RG(4);
    else if (slots <= 8) FMOE_RG(8);
    else FMOE_RG(16);
#undef FMOE_RG
    return hipGetLastError();
}

}  // namespace fmoe

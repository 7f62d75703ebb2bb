// group.hip -- per-expert grouping of the routed rows and the row-tile list of the grouped
// GEMMs, in one workgroup.
//
// The flat assignments i = t*k + j are cut into 8 contiguous segments, one per wavefront.
// Phase 1: each wavefront walks its segment 64 assignments at a time, in order; the lanes
// that hold the same local expert find each other with ballots, so every assignment gets
// its rank among the earlier ones of its expert in the segment (a running count per
// (wavefront, expert) in LDS).  Phase 2: a scan per expert over the 8 segments and a scan
// over experts give each (segment, expert) its first grouped row, the counts and offsets,
// and the row tiles.  Phase 3: every assignment is written to its grouped row.  The result
// is the stable counting sort (experts ascending, flat index ascending inside an expert),
// with no atomics, so it is the same on every run.
//
// Row tiles: the grouped GEMMs are cut per expert from the real row count, not from the
// token count ("vLLM Community Traces H20 MoE Scheduling Inefficiency to Expert-Load Kernel
// Selection", paragraphs 3-4): an expert with c rows gets ceil(c / tile_rows) tiles, rows
// spread as evenly as 16-row steps allow.
#include "launch.hpp"

namespace fmoe {

constexpr int kGroupWaves = 8;
constexpr int kGroupThreads = kGroupWaves * 64;
constexpr int kGroupEPT = 2;  // experts per thread in phase 2 (local experts <= 1024)

// Exclusive scan of one int per thread over the workgroup; *total gets the sum.
__device__ int block_exclusive_scan(int v, int* sh, int* total) {
    const int lane = lane_id(), wid = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh[wid] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int w = 0; w < kGroupWaves; w++) {
            int c = sh[w];
            sh[w] = run;
            run += c;
        }
        sh[kGroupWaves] = run;
    }
    __syncthreads();
    int res = x - v + sh[wid];
    *total = sh[kGroupWaves];
    __syncthreads();
    return res;
}

__device__ int block_max(int v, int* sh) {
    const int lane = lane_id(), wid = threadIdx.x >> 6;
    v = wave_max(v);
    if (lane == 0) sh[wid] = v;
    __syncthreads();
    int m = sh[0];
    for (int w = 1; w < kGroupWaves; w++) m = max(m, sh[w]);
    __syncthreads();
    return m;
}

__global__ __launch_bounds__(kGroupThreads) void k_group(const int32_t* __restrict__ ids, int n, int E, int El,
                                                        int lo, int tile_rows, int rows_estimate,
                                                        int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src,
                                                        int32_t* __restrict__ inv_perm, int32_t* __restrict__ rank_buf,
                                                        MTile* __restrict__ mtiles, DevHeader* __restrict__ hdr) {
    extern __shared__ int32_t lds[];
    int* hist = lds;                          // [kGroupWaves][El]
    int* sh = lds + kGroupWaves * El;         // scan scratch [kGroupWaves + 1]
    long long* shl = (long long*)(sh + 16);   // dropped-id partial sums [kGroupWaves]
    const int lane = lane_id(), wid = threadIdx.x >> 6;

    for (int i = threadIdx.x; i < kGroupWaves * El; i += kGroupThreads) hist[i] = 0;
    __syncthreads();

    // ---- phase 1: in-segment ranks
    const int seg = ((n + kGroupWaves * 64 - 1) / (kGroupWaves * 64)) * 64;
    const int begin = wid * seg;
    int* my_hist = hist + wid * El;
    int bad = 0;
    for (int c = 0; c < seg; c += 64) {
        const int i = begin + c + lane;
        int l = -1;
        if (i < n) {
            const int id = ids[i];
            if (id < 0 || id >= E) bad++;
            else if (id - lo >= 0 && id - lo < El) l = id - lo;
        }
        unsigned long long pending = __ballot(l >= 0);
        int r = -1;
        while (pending) {
            const int leader = __ffsll((long long)pending) - 1;
            const int lv = __shfl(l, leader, 64);
            const unsigned long long m = __ballot(l == lv);
            if (l == lv) r = my_hist[lv] + __popcll(m & ((1ull << lane) - 1ull));
            if (lane == leader) my_hist[lv] += __popcll(m);
            pending &= ~m;
        }
        if (i < n) rank_buf[i] = r;
    }
    {
        long long b = bad;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) b += __shfl_xor(b, o, 64);
        if (lane == 0) shl[wid] = b;
    }
    __syncthreads();

    // ---- phase 2: per-expert scans, offsets, tiles
    int cnt[kGroupEPT], run_total = 0;
#pragma unroll
    for (int q = 0; q < kGroupEPT; q++) {
        const int e = threadIdx.x * kGroupEPT + q;
        int run = 0;
        if (e < El) {
            for (int w = 0; w < kGroupWaves; w++) {
                const int c = hist[w * El + e];
                hist[w * El + e] = run;
                run += c;
            }
        }
        cnt[q] = run;
        run_total += run;
    }
    int R;
    const int base = block_exclusive_scan(run_total, sh, &R);
    int ntile[kGroupEPT], nt_total = 0, local_max = 0, local_empty = 0;
    {
        int off = base;
#pragma unroll
        for (int q = 0; q < kGroupEPT; q++) {
            const int e = threadIdx.x * kGroupEPT + q;
            ntile[q] = 0;
            if (e < El) {
                counts[e] = cnt[q];
                offsets[e] = off;
                for (int w = 0; w < kGroupWaves; w++) hist[w * El + e] += off;
                ntile[q] = (cnt[q] + tile_rows - 1) / tile_rows;
                local_max = max(local_max, cnt[q]);
                local_empty += cnt[q] == 0;
            }
            off += cnt[q];
            nt_total += ntile[q];
        }
    }
    int n_mtiles;
    const int tbase = block_exclusive_scan(nt_total, sh, &n_mtiles);
    int empty_total;
    (void)block_exclusive_scan(local_empty, sh, &empty_total);
    const int max_rows = block_max(local_max, sh);
    {
        int tpos = tbase, off = base;
#pragma unroll
        for (int q = 0; q < kGroupEPT; q++) {
            const int e = threadIdx.x * kGroupEPT + q;
            if (e < El && ntile[q] > 0) {
                // rows per tile: even split rounded up to 16, so every tile but the last is full
                const int per = ((cnt[q] + ntile[q] - 1) / ntile[q] + 15) / 16 * 16;
                for (int j = 0; j < ntile[q]; j++) {
                    MTile mt;
                    mt.expert = e;
                    mt.row0 = off + j * per;
                    mt.rows = min(per, cnt[q] - j * per);
                    mt.pad = 0;
                    mtiles[tpos + j] = mt;
                }
            }
            tpos += ntile[q];
            off += cnt[q];
        }
    }
    if (threadIdx.x == 0) {
        offsets[El] = R;
        long long dropped = 0;
        for (int w = 0; w < kGroupWaves; w++) dropped += shl[w];
        hdr->m_tiles = n_mtiles;
        hdr->local_rows = R;
        hdr->max_rows = max_rows;
        hdr->empty_experts = empty_total;
        hdr->dropped = dropped;
        hdr->tile_rows = tile_rows;
        hdr->rows_estimate = rows_estimate;
    }
    __syncthreads();

    // ---- phase 3: scatter
    for (int c = 0; c < seg; c += 64) {
        const int i = begin + c + lane;
        if (i >= n) break;
        const int id = ids[i];
        const int l = id - lo;
        if (id >= 0 && id < E && l >= 0 && l < El) {
            const int pos = my_hist[l] + rank_buf[i];
            perm_src[pos] = i;
            inv_perm[i] = pos;
        } else {
            inv_perm[i] = -1;
        }
    }
}

size_t group_lds_bytes(int El) { return (size_t)(kGroupWaves * El + 16 + 2 * kGroupWaves) * sizeof(int32_t); }

hipError_t launch_group(const int32_t* ids, int n, int E, int El, int lo, int tile_rows, int rows_estimate, int32_t* counts,
                        int32_t* offsets, int32_t* perm_src, int32_t* inv_perm, int32_t* rank_buf, MTile* mtiles,
                        DevHeader* hdr, hipStream_t st) {
    k_group<<<1, kGroupThreads, group_lds_bytes(El), st>>>(ids, n, E, El, lo, tile_rows, rows_estimate, counts, offsets, perm_src,
                                                            inv_perm, rank_buf, mtiles, hdr);
    return hipGetLastError();
}

}  // namespace fmoe

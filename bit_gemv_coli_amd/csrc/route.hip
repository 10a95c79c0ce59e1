// route.hip -- the MoE routing table on the GPU (colibri-strix commit log,
// batched expert-block commit: per-row ragged expert routing; the CPU then did
// the weighted scatter-add -- here the table drives gathers and a
// deterministic combine instead).
//
// Table: counts[e], exclusive offsets[e], and perm = the valid pair indices
// p = s*K+k grouped by ascending expert, ascending p inside an expert (a
// stable counting sort).  Also inv[p] = position of p in perm (-1 if left
// out) and a list of row tiles (expert, first row) for the grouped GEMMs.
//
// One workgroup of 8 wavefronts:
//   1. LDS counters per (wavefront segment, expert);
//   2. exclusive scan over experts, then per-expert running offsets across
//      the segments (segment order = pair order, so the sort is stable);
//   3. each wavefront walks its segment 64 pairs at a time: lanes holding the
//      same expert find each other with ballots over the id bits, take their
//      rank among earlier lanes, and the lowest of them advances the
//      segment's cursor for that expert.
// All counts are integers, so the result is exact and deterministic.
#include "common.h"

namespace coli {

constexpr int RT_WAVES = 8;
constexpr int RT_THREADS = RT_WAVES * 64;
constexpr int RT_EMAX = 4096;

__device__ __forceinline__ int block_exclusive_scan(int v, int *sbuf, int *total) {
    // sbuf: at least RT_WAVES ints.  Returns the exclusive prefix of v over
    // the workgroup in thread order.
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int n = __shfl_up(incl, off, 64);
        if (lane >= off) incl += n;
    }
    if (lane == 63) sbuf[wv] = incl;
    __syncthreads();
    int base = 0, all = 0;
#pragma unroll
    for (int i = 0; i < RT_WAVES; ++i) {
        const int t = sbuf[i];
        if (i < wv) base += t;
        all += t;
    }
    __syncthreads();
    *total = all;
    return base + incl - v;
}

__global__ __launch_bounds__(RT_THREADS) void k_route(const int32_t *__restrict__ ids, int SK, int E,
                                                      int32_t *__restrict__ counts,
                                                      int32_t *__restrict__ offsets,
                                                      int32_t *__restrict__ perm,
                                                      int32_t *__restrict__ n_bad,
                                                      int32_t *__restrict__ inv,
                                                      int32_t *__restrict__ tiles,
                                                      int32_t *__restrict__ n_tiles, int bm,
                                                      int shared_rows,
                                                      int32_t *__restrict__ tiles_s,
                                                      int32_t *__restrict__ n_tiles_s, int bm_s) {
    // seg[w][e]: pairs of segment w routed to e, then that segment's cursor
    __shared__ int seg[RT_WAVES * RT_EMAX];
    __shared__ int sbuf[RT_WAVES];
    __shared__ int bad_s;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int per = (SK + RT_WAVES - 1) / RT_WAVES;
    const int beg = wv * per;
    const int end = min(SK, beg + per);

    for (int i = tid; i < RT_WAVES * E; i += RT_THREADS) seg[i] = 0;
    if (tid == 0) bad_s = 0;
    __syncthreads();

    // 1. per-segment counts
    int mybad = 0;
    for (int p = beg + lane; p < end; p += 64) {
        const int e = ids[p];
        if (e >= 0 && e < E)
            atomicAdd(&seg[wv * E + e], 1);
        else
            ++mybad;
    }
    if (mybad) atomicAdd(&bad_s, mybad);
    __syncthreads();

    // 2. totals, exclusive offsets, per-segment cursors; tile counts
    // (with bm_s > 0, an expert of 1 .. bm_s rows gets one short tile in the
    // second list instead of row tiles of bm in the first)
    int carry = 0, tcarry = 0, scarry = 0;
    for (int e0 = 0; e0 < E; e0 += RT_THREADS) {
        const int e = e0 + tid;
        int c = 0;
        if (e < E)
#pragma unroll
            for (int w = 0; w < RT_WAVES; ++w) c += seg[w * E + e];
        int tot;
        const int ex = block_exclusive_scan(c, sbuf, &tot) + carry;
        const bool small = bm_s > 0 && c >= 1 && c <= bm_s;
        const int nt = (bm > 0 && !small) ? (c + bm - 1) / bm : 0;
        int ttot;
        const int tex = block_exclusive_scan(nt, sbuf, &ttot) + tcarry;
        int stot;
        const int sex = block_exclusive_scan(small ? 1 : 0, sbuf, &stot) + scarry;
        if (tiles_s && small) {
            tiles_s[2 * sex] = e;
            tiles_s[2 * sex + 1] = 0;
        }
        if (e < E) {
            counts[e] = c;
            offsets[e] = ex;
            int run = ex;
#pragma unroll
            for (int w = 0; w < RT_WAVES; ++w) {
                const int cw = seg[w * E + e];
                seg[w * E + e] = run;
                run += cw;
            }
            if (tiles)
                for (int t = 0; t < nt; ++t) {
                    tiles[2 * (tex + t)] = e;
                    tiles[2 * (tex + t) + 1] = t * bm;
                }
        }
        carry += tot;
        tcarry += ttot;
        scarry += stot;
    }
    if (tid == 0) {
        offsets[E] = carry;
        n_bad[0] = bad_s;
        int nt = tcarry;
        if (tiles && shared_rows > 0) {
            // the shared expert (index E) covers rows SK .. SK+shared_rows-1
            for (int m0 = 0; m0 < shared_rows; m0 += bm) {
                tiles[2 * nt] = E;
                tiles[2 * nt + 1] = m0;
                ++nt;
            }
        }
        if (n_tiles) n_tiles[0] = nt;
        if (n_tiles_s) n_tiles_s[0] = scarry;
    }
    __syncthreads();

    // 3. stable placement
    const int idbits = 32 - __clz(E > 1 ? E - 1 : 1);
    for (int b = beg; b < end; b += 64) {
        const int p = b + lane;
        const bool in = p < end;
        const int e = in ? ids[p] : -1;
        const bool valid = in && e >= 0 && e < E;
        // lanes with the same (valid) expert id
        uint64_t same = __ballot(valid);
        if (valid) {
            for (int bit = 0; bit < idbits; ++bit) {
                const uint64_t m = __ballot(((e >> bit) & 1) != 0);
                same &= ((e >> bit) & 1) ? m : ~m;
            }
        } else {
            for (int bit = 0; bit < idbits; ++bit) (void)__ballot(0);
        }
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        if (valid) {
            const int rank = __popcll(same & below);
            const int pos = seg[wv * E + e] + rank;
            perm[pos] = p;
            if (inv) inv[p] = pos;
            if ((same & below) == 0)  // lowest lane of its expert advances the cursor
                seg[wv * E + e] += __popcll(same);
        } else if (in && inv) {
            inv[p] = -1;
        }
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    // unused tail of perm
    for (int i = carry + tid; i < SK; i += RT_THREADS) perm[i] = -1;
}

int launch_route(const int32_t *ids, int S, int K, int E, int32_t *counts, int32_t *offsets,
                 int32_t *perm, int32_t *n_bad, int32_t *inv, int32_t *tiles, int32_t *n_tiles,
                 int bm, int shared_rows, hipStream_t st, int32_t *tiles_s, int32_t *n_tiles_s,
                 int bm_s) {
    if (E < 1 || E > RT_EMAX)
        return decline("route: E=%d outside 1..%d", E, RT_EMAX);
    ProfScope ps("route", st);
    hipLaunchKernelGGL(k_route, dim3(1), dim3(RT_THREADS), 0, st, ids, S * K, E, counts, offsets,
                       perm, n_bad, inv, tiles, n_tiles, bm, shared_rows, tiles_s, n_tiles_s, bm_s);
    return after_launch("route");
}

}  // namespace coli

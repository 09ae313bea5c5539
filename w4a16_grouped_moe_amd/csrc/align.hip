// Sync-free token-to-expert alignment.
//
// Follows the Part 2 blog, "Quantisation alone leaves a sparse execution
// problem" (sort assignments by expert, pad into regular blocks) and "The
// final best W4 MoE kernel" (32-row blocks), and the "dg-w4-kernels" card,
// "Grouped MoE" (alignment without host synchronisation).
//
// One workgroup of 512 threads does the whole job in four phases:
//   1. histogram of expert ids in LDS (integer atomics: order-free result);
//   2. exclusive scan of the block-padded counts over experts (wave scans
//      combined through LDS) -> offsets;
//   3. stable scatter: assignments are taken 512 at a time in ascending flat
//      order; inside a wave, lanes holding the same expert find each other
//      with one ballot per id bit, which gives each lane its rank among
//      earlier lanes; per-wave counts are turned into per-wave starting
//      points by a pass over the 8 waves in order; a running cursor per expert
//      carries across rounds. The result is the ascending-flat-id order
//      inside every expert, independent of timing;
//   4. pad entries and the tile -> expert map, each found by a binary search
//      over the offsets.
// Ids outside [0, E) are skipped everywhere.
#include "dgw4_internal.hpp"

namespace dgw4 {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

__device__ inline int wave_inclusive_scan(int v, int lane)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(v, off, 64);
        if (lane >= off)
            v += u;
    }
    return v;
}

// Largest e in [0, E) with offs[e] <= p (offs is non-decreasing, offs[0] = 0).
__device__ inline int find_expert(const int *offs, int E, int p)
{
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offs[mid] <= p)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

__global__ void __launch_bounds__(kThreads) align_kernel(const int32_t *__restrict__ ids, int A,
                                                        int E, int bm, long long cap,
                                                        int32_t *__restrict__ counts,
                                                        int32_t *__restrict__ offsets,
                                                        int32_t *__restrict__ sorted_ids,
                                                        int32_t *__restrict__ tile_expert,
                                                        int32_t *__restrict__ num_padded)
{
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_off[kMaxExperts + 1];
    __shared__ int s_cur[kMaxExperts];
    __shared__ int s_wave[kWaves][kMaxExperts];
    __shared__ int s_wsum[kWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    for (int e = tid; e < E; e += kThreads) {
        s_cnt[e] = 0;
        s_cur[e] = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            s_wave[w][e] = 0;
    }
    __syncthreads();

    // 1. histogram
    for (int i = tid; i < A; i += kThreads) {
        const int e = ids[i];
        if (e >= 0 && e < E)
            atomicAdd(&s_cnt[e], 1);
    }
    __syncthreads();

    // 2. exclusive scan of padded counts; thread tid owns experts 2tid, 2tid+1
    const int e0 = 2 * tid, e1 = 2 * tid + 1;
    const int p0 = e0 < E ? (s_cnt[e0] + bm - 1) / bm * bm : 0;
    const int p1 = e1 < E ? (s_cnt[e1] + bm - 1) / bm * bm : 0;
    const int incl = wave_inclusive_scan(p0 + p1, lane);
    if (lane == 63)
        s_wsum[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w)
        base += s_wsum[w];
    const int excl = base + incl - (p0 + p1);
    if (e0 < E)
        s_off[e0] = excl;
    if (e1 < E)
        s_off[e1] = excl + p0;
    if (tid == kThreads - 1)
        s_off[E] = base + incl;             // last thread's inclusive total
    __syncthreads();
    for (int e = tid; e < E; e += kThreads) {
        counts[e] = s_cnt[e];
        offsets[e] = s_off[e];
    }
    if (tid == 0) {
        offsets[E] = s_off[E];
        num_padded[0] = s_off[E];
    }

    // 3. stable scatter
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base_i = 0; base_i < A; base_i += kThreads) {
        const int i = base_i + tid;
        const int e = i < A ? ids[i] : -1;
        const bool valid = e >= 0 && e < E;
        unsigned long long mask = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = valid && ((e >> b) & 1);
            const unsigned long long bb = __ballot(bit);
            mask &= bit ? bb : ~bb;
        }
        const int rank = __popcll(mask & below);
        if (valid && rank == 0)
            s_wave[wave][e] = __popcll(mask);
        __syncthreads();
        for (int x = tid; x < E; x += kThreads) {
            int run = s_cur[x];
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const int c = s_wave[w][x];
                if (c)
                    s_wave[w][x] = run;
                run += c;
            }
            s_cur[x] = run;
        }
        __syncthreads();
        if (valid) {
            sorted_ids[s_off[e] + s_wave[wave][e] + rank] = i;
            if (rank == 0)
                s_wave[wave][e] = 0;        // read by every lane of this wave above
        }
    }

    // 4. pads and tile map (disjoint from the positions written above)
    const int total = s_off[E];
    for (long long p = tid; p < cap; p += kThreads) {
        bool pad = true;
        if (p < total) {
            const int e = find_expert(s_off, E, (int)p);
            pad = (int)p - s_off[e] >= s_cnt[e];
        }
        if (pad)
            sorted_ids[p] = A;
    }
    const long long tiles = cap / bm;
    for (long long j = tid; j < tiles; j += kThreads) {
        const long long p = j * bm;
        tile_expert[j] = p < total ? find_expert(s_off, E, (int)p) : -1;
    }
}

}  // namespace

hipError_t launch_align(const int32_t *topk_ids, int A, int E, int block_m, long long cap,
                        int32_t *counts, int32_t *offsets, int32_t *sorted_ids,
                        int32_t *tile_expert, int32_t *num_padded, hipStream_t stream)
{
    align_kernel<<<dim3(1), dim3(kThreads), 0, stream>>>(topk_ids, A, E, block_m, cap, counts,
                                                          offsets, sorted_ids, tile_expert,
                                                          num_padded);
    return hipGetLastError();
}

}  // namespace dgw4

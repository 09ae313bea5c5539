// Sync-free token-to-expert alignment.
//
// Follows the Part 2 blog, "Quantisation alone leaves a sparse execution
// problem" (sort assignments by expert, pad into regular blocks) and "The
// final best W4 MoE kernel" (32-row blocks), and the "dg-w4-kernels" card,
// "Grouped MoE" (alignment without host synchronisation).
//
// One workgroup per expert e, with no communication between workgroups:
//   1. every workgroup builds the full histogram of expert ids with LDS
//      integer atomics (an order-free result), so each knows all counts;
//   2. offset of e = sum of the block-padded counts of the experts below e,
//      total = the sum over all experts (block reductions in a fixed order);
//   3. stable compaction of the flat ids i with ids[i] == e: thread t holds
//      ids c0 + 8t .. c0 + 8t + 7 of an 8192-id chunk, an exclusive block scan
//      of the per-thread match counts gives each thread its first slot, and
//      the matches are written in ascending i;
//   4. e writes its pad entries, counts/offsets and its tile map entries
//      ({expert, rows of the tile that hold assignments} descriptors too);
//      workgroup 0 also writes the totals and fills the buffers past the
//      total (sentinel ids, tiles marked -1).
// The layer kernel at the layer's shape repeats steps 1-3 for its own tile
// inside its workgroups; this kernel serves dgw4_align and the other shapes.
// Ids outside [0, E) are skipped everywhere. The result depends only on the
// ids, never on timing.
#include "dgw4_internal.hpp"

namespace dgw4 {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kPer = 8;                       // ids per thread per chunk
constexpr int kChunk = kThreads * kPer;       // ids per chunk

// inclusive scan of v over the workgroup; also returns the workgroup total
__device__ inline int block_scan_incl(int v, int *s_wsum, int &total)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(v, off, 64);
        if (lane >= off)
            v += u;
    }
    if (lane == 63)
        s_wsum[wave] = v;
    __syncthreads();
    int base = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int s = s_wsum[w];
        base += w < wave ? s : 0;
        total += s;
    }
    __syncthreads();                          // s_wsum is reused by the next scan
    return base + v;
}

__global__ void __launch_bounds__(kThreads) align_kernel(const int32_t *__restrict__ ids, int A,
                                                        int E, int bm, int cap,
                                                        int32_t *__restrict__ counts,
                                                        int32_t *__restrict__ offsets,
                                                        int32_t *__restrict__ sorted_ids,
                                                        int32_t *__restrict__ tile_expert,
                                                        int32_t *__restrict__ num_padded,
                                                        int2 *__restrict__ tile_info)
{
    __shared__ int32_t s_cnt[kMaxExperts];
    __shared__ int32_t s_wsum[kWaves];
    const int tid = threadIdx.x;
    const int e = blockIdx.x;

    for (int x = tid; x < E; x += kThreads)
        s_cnt[x] = 0;
    __syncthreads();

    // ---- 1. histogram (ids of the first chunk stay in registers)
    int v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = tid * kPer + j;
        v[j] = i < A ? ids[i] : -1;
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        if (v[j] >= 0 && v[j] < E)
            atomicAdd(&s_cnt[v[j]], 1);
    for (int c0 = kChunk; c0 < A; c0 += kChunk) {  // later chunks: loads issued together
        int u[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = c0 + j * kThreads + tid;
            u[j] = i < A ? ids[i] : -1;
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (u[j] >= 0 && u[j] < E)
                atomicAdd(&s_cnt[u[j]], 1);
    }
    __syncthreads();

    // ---- 2. offset of e and the total (each sum in a fixed order)
    int below = 0, all = 0;
    for (int x = tid; x < E; x += kThreads) {
        const int padded = (s_cnt[x] + bm - 1) / bm * bm;
        all += padded;
        below += x < e ? padded : 0;
    }
    int total_below, total;
    block_scan_incl(below, s_wsum, total_below);
    block_scan_incl(all, s_wsum, total);
    const int cnt = s_cnt[e];
    const int off = total_below;
    const int padded = (cnt + bm - 1) / bm * bm;

    // ---- 3. stable compaction of this expert's flat ids
    int written = 0;
    for (int c0 = 0; c0 < A; c0 += kChunk) {
        if (c0 > 0) {
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int i = c0 + tid * kPer + j;
                v[j] = i < A ? ids[i] : -1;
            }
        }
        int mine = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            mine += v[j] == e;
        int chunk_total;
        const int incl = block_scan_incl(mine, s_wsum, chunk_total);
        int slot = off + written + incl - mine;
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (v[j] == e)
                sorted_ids[slot++] = c0 + tid * kPer + j;
        written += chunk_total;
    }

    // ---- 4. pads, counts/offsets, tiles of e
    for (int q = off + cnt + tid; q < off + padded; q += kThreads)
        sorted_ids[q] = A;
    for (int t = off / bm + tid; t < (off + padded) / bm; t += kThreads) {
        tile_expert[t] = e;
        if (tile_info)
            tile_info[t] = make_int2(e, min(bm, cnt - (t * bm - off)) | min(padded / bm, 0x7FFF) << 16);
    }
    if (tid == 0) {
        counts[e] = cnt;
        offsets[e] = off;
    }
    if (e == 0) {
        if (tid == 0) {
            offsets[E] = total;
            num_padded[0] = total;
        }
        for (int q = total + tid; q < cap; q += kThreads)
            sorted_ids[q] = A;
        for (int t = total / bm + tid; t < cap / bm; t += kThreads) {
            tile_expert[t] = -1;
            if (tile_info)
                tile_info[t] = make_int2(-1, 0);
        }
    }
}

}  // namespace

hipError_t launch_align(const int32_t *topk_ids, int A, int E, int block_m, long long cap,
                        int32_t *counts, int32_t *offsets, int32_t *sorted_ids,
                        int32_t *tile_expert, int32_t *num_padded, int2 *tile_info,
                        hipStream_t stream)
{
    align_kernel<<<dim3(E), dim3(kThreads), 0, stream>>>(topk_ids, A, E, block_m, (int)cap,
                                                         counts, offsets, sorted_ids, tile_expert,
                                                         num_padded, tile_info);
    return hipGetLastError();
}

}  // namespace dgw4

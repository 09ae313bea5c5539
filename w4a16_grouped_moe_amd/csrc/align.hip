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
//      total = the sum over all experts (one block reduction);
//   3. stable compaction of the flat ids i with ids[i] == e: thread t holds
//      ids c0 + 8t .. c0 + 8t + 7 of an 8192-id chunk, an exclusive block scan
//      of the per-thread match counts gives each thread its first slot, and
//      the matches are written in ascending i;
//   4. e writes its pad entries, counts/offsets and its tile map entries
//      ({expert, rows of the tile that hold assignments} descriptors too);
//      workgroup 0 also writes the totals and fills the buffers past the
//      total (sentinel ids, tiles marked -1);
//   5. optionally each tile's place in the order "most rows first, ties to
//      the lower tile index": a full tile's place is the number of full
//      tiles before it; e's last, partial tile of r rows comes after every
//      full tile and after the partial tiles with more rows or with r rows
//      and a lower expert (three more sums in step 2's reduction).
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

// the workgroup sums of N integers, in every thread (s_w: N * kWaves ints)
template <int N>
__device__ inline void block_sums(int (&v)[N], int *s_w)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
#pragma unroll
        for (int i = 0; i < N; ++i)
            v[i] += __shfl_xor(v[i], off, 64);
    if (lane == 0)
#pragma unroll
        for (int i = 0; i < N; ++i)
            s_w[N * wave + i] = v[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        v[i] = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            v[i] += s_w[N * w + i];
    }
}

__global__ void __launch_bounds__(kThreads) align_kernel(const int32_t *__restrict__ ids, int A,
                                                        int E, int bm, int cap,
                                                        int32_t *__restrict__ counts,
                                                        int32_t *__restrict__ offsets,
                                                        int32_t *__restrict__ sorted_ids,
                                                        int32_t *__restrict__ tile_expert,
                                                        int32_t *__restrict__ num_padded,
                                                        int2 *__restrict__ tile_info,
                                                        int32_t *__restrict__ order)
{
    __shared__ int32_t s_cnt[kMaxExperts];
    __shared__ int32_t s_wsum[kWaves];
    __shared__ int32_t s_w5[5 * kWaves];
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

    // ---- 2. offset of e and the total; with order, the sums step 5 needs:
    // the full tiles below e and in all, and the partial tiles ahead of e's
    const int cnt = s_cnt[e];
    const int part = cnt % bm;                    // rows of e's partial tile, 0: none
    int sums[5] = {0, 0, 0, 0, 0};                // below, all, full below, full, ahead
    for (int x = tid; x < E; x += kThreads) {
        const int cx = s_cnt[x];
        const int padded_x = (cx + bm - 1) / bm * bm;
        sums[1] += padded_x;
        sums[0] += x < e ? padded_x : 0;
        if (order) {
            const int px = cx % bm;
            sums[3] += cx / bm;
            sums[2] += x < e ? cx / bm : 0;
            sums[4] += part > 0 && (px > part || (px == part && x < e));
        }
    }
    block_sums(sums, s_w5);
    const int total = sums[1];
    const int off = sums[0];
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
            if (order)
                order[t] = -1;
        }
    }

    // ---- 5. the tiles' order, most rows first (uniform branch: order is a
    // kernel argument)
    if (order) {
        const int t0 = off / bm, nfull = cnt / bm;
        for (int j = tid; j < nfull; j += kThreads)
            order[sums[2] + j] = t0 + j;
        if (part > 0 && tid == 0)
            order[sums[3] + sums[4]] = t0 + nfull;
    }
}

}  // namespace

hipError_t launch_align(const int32_t *topk_ids, int A, int E, int block_m, long long cap,
                        int32_t *counts, int32_t *offsets, int32_t *sorted_ids,
                        int32_t *tile_expert, int32_t *num_padded, int2 *tile_info,
                        int32_t *order, hipStream_t stream)
{
    align_kernel<<<dim3(E), dim3(kThreads), 0, stream>>>(topk_ids, A, E, block_m, (int)cap,
                                                         counts, offsets, sorted_ids, tile_expert,
                                                         num_padded, tile_info, order);
    return hipGetLastError();
}

}  // namespace dgw4

// Sync-free token-to-expert alignment, plus the forward's activation prep.
//
// Follows the Part 2 blog, "Quantisation alone leaves a sparse execution
// problem" (sort assignments by expert, pad into regular blocks) and "The
// final best W4 MoE kernel" (32-row blocks), and the "dg-w4-kernels" card,
// "Grouped MoE" (alignment without host synchronisation).
//
// Workgroup 0 (1024 threads = 16 waves) aligns, with the ids held in LDS:
//   1. histogram of expert ids with LDS integer atomics (order-free result);
//   2. exclusive scan of the block-padded counts over experts (wave scans
//      combined through LDS) -> offsets;
//   3. stable scatter in rounds of 1024 ids taken in ascending flat order:
//      inside a wave, lanes holding the same expert find each other with one
//      ballot per id bit, which gives each lane its rank among earlier lanes;
//      one thread per expert turns the 16 per-wave counts into per-wave
//      starting points (in wave order) and carries a running cursor across
//      rounds. The result is the ascending-flat-id order inside every expert,
//      independent of timing;
//   4. each expert writes its own pad entries and tile map entries (and, for
//      the forward, the tile descriptors {expert, valid rows}); the tail of
//      the buffers past the total is filled by all threads.
// Ids outside [0, E) are skipped everywhere.
//
// Workgroups 1.. (forward only) copy x into the permuted K order the GEMM
// kernels consume (each 8 fp16 values reordered as [0,4,1,5,2,6,3,7]).
#include "dgw4_internal.hpp"

namespace dgw4 {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// 8 consecutive fp16 values -> the same values in order [0,4,1,5,2,6,3,7].
__device__ inline uint4 permute8(uint4 v)
{
    uint4 o;
    o.x = (v.x & 0xFFFFu) | (v.z << 16);
    o.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
    o.z = (v.y & 0xFFFFu) | (v.w << 16);
    o.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
    return o;
}

template <bool IDS_IN_LDS>
__global__ void __launch_bounds__(kThreads) align_kernel(const int32_t *__restrict__ ids, int A,
                                                        int E, int bm, int cap,
                                                        int32_t *__restrict__ counts,
                                                        int32_t *__restrict__ offsets,
                                                        int32_t *__restrict__ sorted_ids,
                                                        int32_t *__restrict__ tile_expert,
                                                        int32_t *__restrict__ num_padded,
                                                        int2 *__restrict__ tile_info,
                                                        const uint4 *__restrict__ x,
                                                        uint4 *__restrict__ xp, long long x_segs)
{
    const int tid = threadIdx.x;
    if (blockIdx.x > 0) {
        const long long stride = (long long)(gridDim.x - 1) * kThreads;
        for (long long i = (long long)(blockIdx.x - 1) * kThreads + tid; i < x_segs; i += stride)
            xp[i] = permute8(x[i]);
        return;
    }

    extern __shared__ int32_t s_ids[];          // [A] when IDS_IN_LDS
    __shared__ int32_t s_wave[kWaves][kMaxExperts];   // per-round, per-wave counts / starts
    __shared__ int32_t s_cnt[kMaxExperts];
    __shared__ int32_t s_cur[kMaxExperts];
    __shared__ int32_t s_off[kMaxExperts + 1];
    __shared__ int32_t s_wsum[kWaves];
    const int lane = tid & 63;
    const int wave = tid >> 6;

    for (int e = tid; e < E; e += kThreads) {
        s_cnt[e] = 0;
        s_cur[e] = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            s_wave[w][e] = 0;
    }
    if constexpr (IDS_IN_LDS) {
        for (int i = tid; i < A; i += kThreads)
            s_ids[i] = ids[i];
    }
    __syncthreads();
    auto id_at = [&](int i) { return IDS_IN_LDS ? s_ids[i] : ids[i]; };

    // 1. histogram
    for (int i = tid; i < A; i += kThreads) {
        const int e = id_at(i);
        if (e >= 0 && e < E)
            atomicAdd(&s_cnt[e], 1);
    }
    __syncthreads();

    // 2. exclusive scan of padded counts (E <= 1024: one expert per thread)
    const int padded = tid < E ? (s_cnt[tid] + bm - 1) / bm * bm : 0;
    int incl = padded;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(incl, off, 64);
        if (lane >= off)
            incl += u;
    }
    if (lane == 63)
        s_wsum[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w)
        base += s_wsum[w];
    if (tid < E)
        s_off[tid] = base + incl - padded;
    if (tid == kThreads - 1)
        s_off[E] = base + incl;                 // total over all experts
    __syncthreads();
    const int total = s_off[E];
    if (tid < E) {
        counts[tid] = s_cnt[tid];
        offsets[tid] = s_off[tid];
    }
    if (tid == 0) {
        offsets[E] = total;
        num_padded[0] = total;
    }

    // 3. stable scatter, 1024 ids per round
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base_i = 0; base_i < A; base_i += kThreads) {
        const int i = base_i + tid;
        const int e = i < A ? id_at(i) : -1;
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
                s_wave[wave][e] = 0;            // read by every lane of this wave above
        }
        // the next round's first LDS writes (the leaders above) only touch
        // this wave's own row; the expert pass reads all rows after a barrier
    }

    // 4. pads and tile map: per expert, then the tail past the total
    for (int e = tid; e < E; e += kThreads) {
        for (int p = s_off[e] + s_cnt[e]; p < s_off[e + 1]; ++p)
            sorted_ids[p] = A;
        for (int t = s_off[e] / bm; t < s_off[e + 1] / bm; ++t) {
            tile_expert[t] = e;
            if (tile_info)
                tile_info[t] = make_int2(e, min(bm, s_cnt[e] - (t * bm - s_off[e])));
        }
    }
    for (int p = total + tid; p < cap; p += kThreads)
        sorted_ids[p] = A;
    for (int t = total / bm + tid; t < cap / bm; t += kThreads) {
        tile_expert[t] = -1;
        if (tile_info)
            tile_info[t] = make_int2(-1, 0);
    }
}

}  // namespace

// Largest assignment count whose ids are staged in LDS (64 KB).
constexpr int kMaxIdsInLds = 16384;

hipError_t launch_align(const int32_t *topk_ids, int A, int E, int block_m, long long cap,
                        int32_t *counts, int32_t *offsets, int32_t *sorted_ids,
                        int32_t *tile_expert, int32_t *num_padded, hipStream_t stream)
{
    return launch_prep(topk_ids, A, E, block_m, cap, counts, offsets, sorted_ids, tile_expert,
                       num_padded, nullptr, nullptr, nullptr, 0, stream);
}

hipError_t launch_prep(const int32_t *topk_ids, int A, int E, int block_m, long long cap,
                       int32_t *counts, int32_t *offsets, int32_t *sorted_ids,
                       int32_t *tile_expert, int32_t *num_padded, int2 *tile_info,
                       const uint16_t *x, uint16_t *xp, long long x_elems, hipStream_t stream)
{
    const long long segs = x_elems / 8;
    const long long want = (segs + kThreads - 1) / kThreads;
    const int extra = (int)(want < 256 ? want : 256);
    const dim3 grid(1 + extra);
    const uint4 *x4 = reinterpret_cast<const uint4 *>(x);
    uint4 *xp4 = reinterpret_cast<uint4 *>(xp);
    if (A <= kMaxIdsInLds) {
        auto kern = align_kernel<true>;
        const size_t lds = sizeof(int32_t) * (size_t)A;
        static size_t lds_allowed = 64 * 1024;
        if (lds > lds_allowed) {
            hipError_t err = hipFuncSetAttribute((const void *)kern,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
            if (err != hipSuccess)
                return err;
            lds_allowed = lds;
        }
        kern<<<grid, dim3(kThreads), lds, stream>>>(topk_ids, A, E, block_m, (int)cap, counts,
                                                    offsets, sorted_ids, tile_expert, num_padded,
                                                    tile_info, x4, xp4, segs);
    } else {
        align_kernel<false><<<grid, dim3(kThreads), 0, stream>>>(
            topk_ids, A, E, block_m, (int)cap, counts, offsets, sorted_ids, tile_expert,
            num_padded, tile_info, x4, xp4, segs);
    }
    return hipGetLastError();
}

}  // namespace dgw4

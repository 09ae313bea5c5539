// Router: each token's top-k experts and their weights from fp32 router
// logits.
//
// Follows the Part 2 blog, "Quantisation alone leaves a sparse execution
// problem" (a router scores the experts per token; the token picks 8 of 128
// and the chosen experts' outputs are weighted). The experts are the topk
// largest logits, largest first, equal logits ordered by the lower expert
// id: a softmax is monotone, so these are the most probable experts, and the
// choice compares the fp32 logits themselves (no arithmetic decides an id,
// so the ids are exact). The weights are the chosen experts' softmax
// probabilities renormalised to one, i.e. the softmax over the chosen
// logits: w_k = exp(l_k - l_0) / sum_j exp(l_j - l_0), fp32, summed in k
// order.
//
// One wave per token, no sequential rounds: the token's logits go to a slot
// of LDS, every lane ranks the logits it holds against all of them (rank =
// how many logits are larger, or equal at a lower id), and the logit of rank
// k < topk is choice k. The weights' exp terms are laid out in choice order
// and summed in that order by every lane.
#include "dgw4_internal.hpp"

#include <cmath>

namespace dgw4 {
namespace {

constexpr int kRouterWaves = 4;                  // tokens per workgroup

// (v, e) ranks before (v2, e2): the larger value, or the same value at a
// smaller id
__device__ inline bool before(float v, int e, float v2, int e2)
{
    return v > v2 || (v == v2 && e < e2);
}

template <int PER>
__global__ void __launch_bounds__(kRouterWaves * 64) router_kernel(const float *__restrict__ logits,
                                                                  int T, int E, int topk,
                                                                  int32_t *__restrict__ ids,
                                                                  float *__restrict__ w)
{
    __shared__ float s_l[kRouterWaves][PER * 64];    // the token's logits
    __shared__ float s_x[kRouterWaves][64];          // exp terms in choice order
    __shared__ float s_v[kRouterWaves][64];          // chosen logits in choice order
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int t = blockIdx.x * kRouterWaves + wv;
    if (t >= T)
        return;                                      // whole waves: no barrier below
    const float *l = logits + (size_t)t * E;
    float v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = lane + 64 * j;
        v[j] = e < E ? l[e] : 0.0f;
        if (e < E)
            s_l[wv][e] = v[j];
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    int rank[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j)
        rank[j] = 0;
    for (int e2 = 0; e2 < E; ++e2) {                 // the same address for all lanes: a broadcast
        const float v2 = s_l[wv][e2];
#pragma unroll
        for (int j = 0; j < PER; ++j)
            rank[j] += before(v2, e2, v[j], lane + 64 * j);
    }
    // choice k: its id, its logit; the largest logit is choice 0
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = lane + 64 * j;
        if (e < E && rank[j] < topk) {
            ids[(size_t)t * topk + rank[j]] = e;
            s_v[wv][rank[j]] = v[j];
        }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    const float top = s_v[wv][0];
    if (lane < topk)
        s_x[wv][lane] = expf(s_v[wv][lane] - top);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    // w_k = exp(l_k - l_0) / sum_j exp(l_j - l_0), the sum in choice order
    float den = 0.0f;
    for (int k = 0; k < topk; ++k)
        den = __fadd_rn(den, s_x[wv][k]);
    if (lane < topk)
        w[(size_t)t * topk + lane] = __fdiv_rn(s_x[wv][lane], den);
}

}  // namespace

hipError_t launch_router(const float *logits, int T, int E, int topk, int32_t *ids, float *w,
                         hipStream_t stream)
{
    if (T == 0)
        return hipSuccess;
    const dim3 grid((T + kRouterWaves - 1) / kRouterWaves);
    const dim3 block(kRouterWaves * 64);
    if (E <= 128)
        router_kernel<2><<<grid, block, 0, stream>>>(logits, T, E, topk, ids, w);
    else
        router_kernel<kMaxExperts / 64><<<grid, block, 0, stream>>>(logits, T, E, topk, ids, w);
    return hipGetLastError();
}

}  // namespace dgw4

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
// k < topk is choice k. Each comparison is one unsigned 64-bit compare of
// keys (the logit's bits mapped to an order-preserving unsigned integer,
// -0 as +0, above the complement of the id), which orders exactly as
// "larger logit, or equal logit at a lower id" for finite logits. The
// weights' exp terms are laid out in choice order and summed in that order
// by every lane.
#include "dgw4_internal.hpp"

#include <cmath>

namespace dgw4 {
namespace {

constexpr int kRouterWaves = 4;                  // tokens per workgroup

// The ranking key of logit v of expert e: a larger key ranks first. The
// float's bits become an unsigned integer in the floats' order (negative
// values complemented, non-negative ones with the top bit set; -0 as +0),
// the id's complement below it puts equal logits in ascending id order.
__device__ inline uint64_t rank_key(float v, int e)
{
    uint32_t b = __builtin_bit_cast(uint32_t, v);
    if (b == 0x80000000u)
        b = 0u;
    const uint32_t u = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return (uint64_t)u << 32 | (uint32_t)~e;
}

template <int PER>
__global__ void __launch_bounds__(kRouterWaves * 64) router_kernel(const float *__restrict__ logits,
                                                                  int T, int E, int topk,
                                                                  int32_t *__restrict__ ids,
                                                                  float *__restrict__ w)
{
    __shared__ uint64_t s_k[kRouterWaves][PER * 64]; // the token's ranking keys
    __shared__ float s_x[kRouterWaves][64];          // exp terms in choice order
    __shared__ float s_v[kRouterWaves][64];          // chosen logits in choice order
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int t = blockIdx.x * kRouterWaves + wv;
    if (t >= T)
        return;                                      // whole waves: no barrier below
    const float *l = logits + (size_t)t * E;
    float v[PER];
    uint64_t key[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = lane + 64 * j;
        v[j] = e < E ? l[e] : 0.0f;
        key[j] = rank_key(v[j], e);
        if (e < E)
            s_k[wv][e] = key[j];
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    int rank[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j)
        rank[j] = 0;
    for (int e2 = 0; e2 < E; ++e2) {                 // the same address for all lanes: a broadcast
        const uint64_t k2 = s_k[wv][e2];
#pragma unroll
        for (int j = 0; j < PER; ++j)
            rank[j] += k2 > key[j];
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

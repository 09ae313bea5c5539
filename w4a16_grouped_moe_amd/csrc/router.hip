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
// One wave per token: lane i holds logits i, i + 64, ...; each of the topk
// rounds takes the wave's largest untaken logit (ties to the lower id) with
// a butterfly of (value, id) pairs, so every lane ends with the same ordered
// list; lane k writes id k and weight k.
#include "dgw4_internal.hpp"

#include <cmath>

namespace dgw4 {
namespace {

constexpr int kRouterWaves = 4;                  // tokens per workgroup
constexpr int kRouterPer = kMaxExperts / 64;     // logits per lane, at most

// (v, e) beats (v2, e2): the larger value, or the same value at a smaller id
__device__ inline bool beats(float v, int e, float v2, int e2)
{
    return v > v2 || (v == v2 && e < e2);
}

template <int PER>
__global__ void __launch_bounds__(kRouterWaves * 64) router_kernel(const float *__restrict__ logits,
                                                                  int T, int E, int topk,
                                                                  int32_t *__restrict__ ids,
                                                                  float *__restrict__ w)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kRouterWaves + (threadIdx.x >> 6);
    if (t >= T)
        return;
    const float *l = logits + (size_t)t * E;
    float v[PER];
    bool live[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = lane + 64 * j;
        live[j] = e < E;
        v[j] = live[j] ? l[e] : 0.0f;
    }
    float my_v = 0.0f;                               // lane k keeps choice k
    int my_e = 0;
    float top = 0.0f;
    for (int k = 0; k < topk; ++k) {
        // this lane's best untaken logit (ascending id: ties keep the lower)
        float bv = 0.0f;
        int be = -1;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int e = lane + 64 * j;
            if (live[j] && (be < 0 || beats(v[j], e, bv, be))) {
                bv = v[j];
                be = e;
            }
        }
        // the wave's best: a butterfly over (value, id); lanes without an
        // untaken logit carry id -1 and lose to any other
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 64);
            const int oe = __shfl_xor(be, off, 64);
            if (oe >= 0 && (be < 0 || beats(ov, oe, bv, be))) {
                bv = ov;
                be = oe;
            }
        }
        if (k == 0)
            top = bv;
        if (lane == k) {
            my_v = bv;
            my_e = be;
        }
        // the owner lane marks it taken
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if (be == lane + 64 * j)
                live[j] = false;
    }
    // weights: exp(l_k - l_0) / sum_j exp(l_j - l_0), the sum in k order
    float den = 0.0f;
    for (int k = 0; k < topk; ++k)
        den = __fadd_rn(den, expf(__shfl(my_v, k, 64) - top));
    if (lane < topk) {
        ids[(size_t)t * topk + lane] = my_e;
        w[(size_t)t * topk + lane] = __fdiv_rn(expf(my_v - top), den);
    }
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
        router_kernel<kRouterPer><<<grid, block, 0, stream>>>(logits, T, E, topk, ids, w);
    return hipGetLastError();
}

}  // namespace dgw4

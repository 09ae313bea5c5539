// Fixed-order, atomic-free weighted combine.
//
// Follows the Part 2 blog, "Quantisation alone leaves a sparse execution
// problem" (each token's eight expert outputs are reduced in a fixed order,
// never with index_add_ or atomics, because a change in the last bit can flip
// a denoising acceptance decision), and the model card's "What's in here"
// (fixed-order reduction instead of index_add_).
//
// out[t, c] = fp16( sum_{k = 0..topk-1, ascending} w[t, k] * Y[t*topk + k, c] )
// in fp32 (Y holds fp16 expert outputs), skipping k whose expert id is
// outside [0, E). Y comes as one fp16 array or as two partials (the layer
// kernel splits down's contraction in two halves); with two,
// Y = fp32(Y0) + fp32(Y1), rounded once in fp32, before the weighting. Each thread owns four neighbouring columns of one token:
// 8-byte loads of Y, one 8-byte store. Every output element is produced by
// exactly one thread with a fixed sequence of operations, so the result is
// bitwise reproducible.
//
// The kernel is bound by load latency, not bandwidth (11.5 MB of Y spread over
// the whole chip is one round of loads per thread), so for topk = 8 all ids,
// weights and Y loads of a thread are issued before the first addition; a
// token's row of d/4 threads is one workgroup when it fits.
#include "dgw4_internal.hpp"

#pragma clang fp contract(off)

namespace dgw4 {
namespace {

__device__ inline float h2f(uint32_t bits) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits); }

// Four expert-output columns as fp32: one fp16 array, or the sum of two
// fp16 partials (one fp32 rounding).
template <int HALVES>
__device__ inline float4 y4(const uint2 *__restrict__ y, size_t half, size_t at)
{
    const uint2 v = y[at];
    float4 r = make_float4(h2f(v.x & 0xFFFFu), h2f(v.x >> 16), h2f(v.y & 0xFFFFu), h2f(v.y >> 16));
    if constexpr (HALVES == 2) {
        const uint2 u = y[half + at];
        r.x = __fadd_rn(r.x, h2f(u.x & 0xFFFFu));
        r.y = __fadd_rn(r.y, h2f(u.x >> 16));
        r.z = __fadd_rn(r.z, h2f(u.y & 0xFFFFu));
        r.w = __fadd_rn(r.w, h2f(u.y >> 16));
    }
    return r;
}

template <int HALVES>
__global__ void __launch_bounds__(256) combine_kernel(const uint2 *__restrict__ y,
                                                      const int32_t *__restrict__ ids,
                                                      const float *__restrict__ w, int topk,
                                                      int E, int d4, uint2 *__restrict__ out)
{
    const int t = blockIdx.y;
    const int c4 = blockIdx.x * blockDim.x + threadIdx.x;
    if (c4 >= d4)
        return;
    const size_t half = (size_t)gridDim.y * topk * d4;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int k = 0; k < topk; ++k) {
        const int e = ids[(size_t)t * topk + k];
        if (e < 0 || e >= E)
            continue;
        const float wk = w[(size_t)t * topk + k];
        const float4 v = y4<HALVES>(y, half, ((size_t)t * topk + k) * d4 + c4);
        a0 = __fadd_rn(a0, __fmul_rn(wk, v.x));
        a1 = __fadd_rn(a1, __fmul_rn(wk, v.y));
        a2 = __fadd_rn(a2, __fmul_rn(wk, v.z));
        a3 = __fadd_rn(a3, __fmul_rn(wk, v.w));
    }
    const uint32_t h0 = __builtin_bit_cast(uint16_t, (_Float16)a0);   // RN-even
    const uint32_t h1 = __builtin_bit_cast(uint16_t, (_Float16)a1);
    const uint32_t h2 = __builtin_bit_cast(uint16_t, (_Float16)a2);
    const uint32_t h3 = __builtin_bit_cast(uint16_t, (_Float16)a3);
    out[(size_t)t * d4 + c4] = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
}

// topk fixed at compile time: every load is in flight before the first add.
// The Y slot of a skipped k exists (it is simply not written by the GEMMs), so
// it is loaded like the others and left out of the sum.
template <int K, int HALVES>
__global__ void __launch_bounds__(1024) combine_fixed_kernel(const uint2 *__restrict__ y,
                                                             const int32_t *__restrict__ ids,
                                                             const float *__restrict__ w, int E,
                                                             int d4, uint2 *__restrict__ out)
{
    const int t = blockIdx.y;
    const int c4 = blockIdx.x * blockDim.x + threadIdx.x;
    if (c4 >= d4)
        return;
    const size_t half = (size_t)gridDim.y * K * d4;
    int e[K];
    float wk[K];
    uint2 v[HALVES][K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        e[k] = ids[(size_t)t * K + k];
        wk[k] = w[(size_t)t * K + k];
    }
#pragma unroll
    for (int hh = 0; hh < HALVES; ++hh)
#pragma unroll
        for (int k = 0; k < K; ++k)
            v[hh][k] = y[hh * half + ((size_t)t * K + k) * d4 + c4];
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if (e[k] < 0 || e[k] >= E)
            continue;
        float y0 = h2f(v[0][k].x & 0xFFFFu), y1 = h2f(v[0][k].x >> 16);
        float y2 = h2f(v[0][k].y & 0xFFFFu), y3 = h2f(v[0][k].y >> 16);
        if constexpr (HALVES == 2) {
            y0 = __fadd_rn(y0, h2f(v[1][k].x & 0xFFFFu));
            y1 = __fadd_rn(y1, h2f(v[1][k].x >> 16));
            y2 = __fadd_rn(y2, h2f(v[1][k].y & 0xFFFFu));
            y3 = __fadd_rn(y3, h2f(v[1][k].y >> 16));
        }
        a0 = __fadd_rn(a0, __fmul_rn(wk[k], y0));
        a1 = __fadd_rn(a1, __fmul_rn(wk[k], y1));
        a2 = __fadd_rn(a2, __fmul_rn(wk[k], y2));
        a3 = __fadd_rn(a3, __fmul_rn(wk[k], y3));
    }
    const uint32_t h0 = __builtin_bit_cast(uint16_t, (_Float16)a0);
    const uint32_t h1 = __builtin_bit_cast(uint16_t, (_Float16)a1);
    const uint32_t h2 = __builtin_bit_cast(uint16_t, (_Float16)a2);
    const uint32_t h3 = __builtin_bit_cast(uint16_t, (_Float16)a3);
    out[(size_t)t * d4 + c4] = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
}

}  // namespace

hipError_t launch_combine(const uint16_t *y, int halves, const int32_t *topk_ids,
                          const float *topk_w, int T, int topk, int E, int d, uint16_t *out,
                          hipStream_t stream)
{
    if (T == 0)
        return hipSuccess;
    if (halves != 1 && halves != 2)
        return hipErrorInvalidValue;
    const int d4 = d / 4;
    const uint2 *yv = reinterpret_cast<const uint2 *>(y);
    uint2 *ov = reinterpret_cast<uint2 *>(out);
    if (topk == 8) {
        // one workgroup per token row when it fits, whole waves
        const int threads = d4 <= 1024 ? (d4 + 63) / 64 * 64 : 256;
        const dim3 grid((d4 + threads - 1) / threads, T);
        if (halves == 2)
            combine_fixed_kernel<8, 2><<<grid, dim3(threads), 0, stream>>>(yv, topk_ids, topk_w, E, d4, ov);
        else
            combine_fixed_kernel<8, 1><<<grid, dim3(threads), 0, stream>>>(yv, topk_ids, topk_w, E, d4, ov);
        return hipGetLastError();
    }
    const dim3 grid((d4 + 255) / 256, T);
    if (halves == 2)
        combine_kernel<2><<<grid, dim3(256), 0, stream>>>(yv, topk_ids, topk_w, topk, E, d4, ov);
    else
        combine_kernel<1><<<grid, dim3(256), 0, stream>>>(yv, topk_ids, topk_w, topk, E, d4, ov);
    return hipGetLastError();
}

}  // namespace dgw4

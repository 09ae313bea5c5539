// The sampler of a denoising step: entropy, Gumbel-max sample and argmax of
// each row of fp32 logits, in one streaming pass.
//
// Follows the "dg-w4-kernels" card, "Sampler": fused_entropy returns
// Categorical(logits).entropy() in nats from a single pass over the logits
// instead of a chain of kernels; gumbel_argmax_sample draws from the same
// Categorical by Gumbel-max with Philox noise generated inline (no noise
// tensor) and returns the plain argmax from the same reduction. Here both
// come out of one pass: each logit is read once.
//
// Noise: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, SC 2011), one block
// per four consecutive logits of a row: counter {v / 4, row, 0, 0}, key
// {seed low word, seed high word}; the top 23 bits of word v % 4 give the
// uniform U = (floor(w / 512) + 1/2) / 2^23, exact in fp32 and strictly
// inside (0, 1), and G = -log(-log U); the sample is the first v with the
// largest l_v + G_v, all in fp32.
//
// Layout: workgroup (split, row) streams a contiguous slice of the row with
// non-temporal 16-byte loads (each wave instruction covers whole lines) and
// leaves one partial {max, sum exp, sum exp * (l - max), argmax, sample} in
// the workspace; a second kernel merges a row's partials in ascending split
// order. Every reduction has a fixed order, so results are bitwise
// reproducible.
#include "dgw4_internal.hpp"

#include <climits>
#include <mutex>

namespace dgw4 {
namespace {

constexpr int kSmpThreads = 256;
constexpr int kSmpUnroll = 4;                      // float4 loads in flight per thread

struct Partial {
    float m, z, s;                                 // max, sum exp(l - m), sum exp(l - m) * (l - m)
    float av;                                      // argmax value and index
    int ai;
    float sv;                                      // best Gumbel score and index
    int si;
    int pad;
};
static_assert(sizeof(Partial) == 32, "partial layout");

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ inline void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                     uint32_t k1, uint32_t (&out)[4])
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        // each full 64-bit product in one v_mad_u64_u32 (instead of a
        // separate high and low multiply, both quarter rate)
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t h0 = (uint32_t)(p0 >> 32), l0 = (uint32_t)p0;
        const uint32_t h1 = (uint32_t)(p1 >> 32), l1 = (uint32_t)p1;
        const uint32_t n0 = h1 ^ c1 ^ k0, n2 = h0 ^ c3 ^ k1;
        c0 = n0;
        c1 = l1;
        c2 = n2;
        c3 = l0;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

// G = -log(-log U) through the hardware base-2 logarithm (v_log_f32).
// U = (floor(w / 2^9) + 1/2) 2^-23 takes 23 bits so that every value is an
// exact fp32 number: it lies in [2^-24, 1 - 2^-24], never 0 or 1 (24 bits
// would round the top value, 2^24 - 1/2, up to 2^24 and give U = 1, an
// infinite score). -log U is then in [6.0e-8, 16.7], both ends normal, so no
// range handling is needed; the log's error is below one ulp of the score.
__device__ inline float gumbel(uint32_t w)
{
    constexpr float kLn2 = 0.693147180559945309f;
    const float u = ((float)(w >> 9) + 0.5f) * (1.0f / 8388608.0f);
    const float e = -kLn2 * __builtin_amdgcn_logf(u);
    return -kLn2 * __builtin_amdgcn_logf(e);
}

// better(a, b): larger value, or the same value at a smaller index (selects,
// no branches)
__device__ inline void take_best(float &v, int &i, float v2, int i2)
{
    const bool b = (v2 > v) | ((v2 == v) & (i2 < i));
    v = b ? v2 : v;
    i = b ? i2 : i;
}

// merge of two log-sum-exp partials (either may be empty: z == 0)
__device__ inline void merge_lse(float &m, float &z, float &s, float m2, float z2, float s2)
{
    if (z2 == 0.0f)
        return;
    if (z == 0.0f) {
        m = m2;
        z = z2;
        s = s2;
        return;
    }
    const float mm = fmaxf(m, m2);
    const float a = __expf(m - mm), b = __expf(m2 - mm);
    s = a * (s + (m - mm) * z) + b * (s2 + (m2 - mm) * z2);
    z = a * z + b * z2;
    m = mm;
}

__device__ inline void merge_partial(Partial &p, const Partial &q)
{
    merge_lse(p.m, p.z, p.s, q.m, q.z, q.s);
    take_best(p.av, p.ai, q.av, q.ai);
    take_best(p.sv, p.si, q.sv, q.si);
}

template <bool SMP>
__global__ void __launch_bounds__(kSmpThreads) sample_partial_kernel(const f32x4v *__restrict__ logits,
                                                                     int V4, int chunk4, uint32_t k0,
                                                                     uint32_t k1, Partial *__restrict__ part)
{
    const int split = blockIdx.x, r = blockIdx.y;
    const f32x4v *row = logits + (size_t)r * V4;
    const int b = split * chunk4, e = min(V4, b + chunk4);
    Partial p;
    p.z = 0.0f;
    p.s = 0.0f;
    p.av = -INFINITY;
    p.ai = INT_MAX;
    p.sv = -INFINITY;
    p.si = INT_MAX;
    p.m = -INFINITY;
    // one block of four logits (columns 4i .. 4i + 3), branch-free
    auto consume = [&](const f32x4v q, int i) {
        // argmax: the block's first maximum, then against the running best
        float bm = q[0];
        int bj = 0;
#pragma unroll
        for (int j = 1; j < 4; ++j) {
            const bool g = q[j] > bm;
            bm = g ? q[j] : bm;
            bj = g ? j : bj;
        }
        take_best(p.av, p.ai, bm, 4 * i + bj);
        // log-sum-exp against the running maximum nm; a logit of -inf (a
        // masked entry) adds nothing (the limit of p log p at p = 0)
        const float nm = fmaxf(p.m, bm);
        const bool live = nm > -INFINITY;
        const float sc = live ? __expf(p.m - nm) : 1.0f;
        float ez = 0.0f, es = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float d = q[j] - nm;
            const float ex = q[j] > -INFINITY ? __expf(d) : 0.0f;
            ez += ex;
            es += ex > 0.0f ? ex * d : 0.0f;
        }
        const float shift = p.z > 0.0f ? (p.m - nm) * p.z : 0.0f;
        p.s = sc * (p.s + shift) + es;
        p.z = p.z * sc + ez;
        p.m = live ? nm : p.m;
        if constexpr (SMP) {
            uint32_t w[4];
            philox4x32_10((uint32_t)i, (uint32_t)r, 0u, 0u, k0, k1, w);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                take_best(p.sv, p.si, q[j] + gumbel(w[j]), 4 * i + j);
        }
    };
    int i0 = b + (int)threadIdx.x;
    for (; i0 + (kSmpUnroll - 1) * kSmpThreads < e; i0 += kSmpUnroll * kSmpThreads) {
        f32x4v q[kSmpUnroll];
#pragma unroll
        for (int u = 0; u < kSmpUnroll; ++u)
            q[u] = __builtin_nontemporal_load(row + i0 + u * kSmpThreads);
#pragma unroll
        for (int u = 0; u < kSmpUnroll; ++u)
            consume(q[u], i0 + u * kSmpThreads);
    }
    for (; i0 < e; i0 += kSmpThreads)
        consume(__builtin_nontemporal_load(row + i0), i0);
    // the workgroup's partial: butterfly within each wave, then the waves in
    // ascending order (fixed orders: bitwise reproducible)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        Partial q;
        q.m = __shfl_xor(p.m, off, 64);
        q.z = __shfl_xor(p.z, off, 64);
        q.s = __shfl_xor(p.s, off, 64);
        q.av = __shfl_xor(p.av, off, 64);
        q.ai = __shfl_xor(p.ai, off, 64);
        q.sv = __shfl_xor(p.sv, off, 64);
        q.si = __shfl_xor(p.si, off, 64);
        if ((threadIdx.x & off) == 0)
            merge_partial(p, q);
        else {
            merge_partial(q, p);
            p = q;
        }
    }
    __shared__ Partial s_wave[kSmpThreads / 64];
    if ((threadIdx.x & 63) == 0)
        s_wave[threadIdx.x >> 6] = p;
    __syncthreads();
    if (threadIdx.x == 0) {
        Partial t = s_wave[0];
#pragma unroll
        for (int w = 1; w < kSmpThreads / 64; ++w)
            merge_partial(t, s_wave[w]);
        t.pad = 0;
        part[(size_t)r * gridDim.x + split] = t;
    }
}

__global__ void __launch_bounds__(64) sample_merge_kernel(const Partial *__restrict__ part, int R, int S,
                                                          float *__restrict__ entropy,
                                                          int32_t *__restrict__ sample,
                                                          int32_t *__restrict__ argmax)
{
    const int r = blockIdx.x * 64 + (int)threadIdx.x;
    if (r >= R)
        return;
    Partial p = part[(size_t)r * S];
    for (int k = 1; k < S; ++k)
        merge_partial(p, part[(size_t)r * S + k]);
    if (entropy)
        entropy[r] = __logf(p.z) - p.s / p.z;
    if (sample)
        sample[r] = p.si;
    if (argmax)
        argmax[r] = p.ai;
}

}  // namespace

// Partials of dgw4_sample_noalloc: a fixed array that every device the
// library runs on holds for the life of the process. In host code its name
// only stands for the symbol; its device address is looked up once per
// device (sample_scratch) and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[kSampleScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch[kMaxDevices];                      // per device, set on first use
}  // namespace

hipError_t sample_scratch(void **ptr)
{
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return err;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess)
            return err;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

int sample_splits(int R, int V)
{
    // about 2048 workgroups in all, at least 256 float4 per workgroup
    const int V4 = V / 4;
    const int by_rows = R > 0 ? (2048 + R - 1) / R : 1;
    const int by_len = max(1, V4 / kSmpThreads);
    return max(1, min(by_rows, by_len));
}

size_t sample_workspace_bytes(int R, int V)
{
    return (size_t)R * (size_t)sample_splits(R, V) * sizeof(Partial);
}

hipError_t launch_sample(const float *logits, int R, int V, uint64_t seed, float *entropy,
                         int32_t *sample, int32_t *argmax, void *workspace, hipStream_t stream)
{
    if (R == 0)
        return hipSuccess;
    const int S = sample_splits(R, V);
    const int V4 = V / 4;
    const int chunk4 = (V4 + S - 1) / S;
    Partial *part = static_cast<Partial *>(workspace);
    const auto *lg = reinterpret_cast<const f32x4v *>(logits);
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    if (sample)
        sample_partial_kernel<true><<<dim3(S, R), dim3(kSmpThreads), 0, stream>>>(lg, V4, chunk4, k0, k1, part);
    else
        sample_partial_kernel<false><<<dim3(S, R), dim3(kSmpThreads), 0, stream>>>(lg, V4, chunk4, k0, k1, part);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    sample_merge_kernel<<<dim3((R + 63) / 64), dim3(64), 0, stream>>>(part, R, S, entropy, sample, argmax);
    return hipGetLastError();
}

}  // namespace dgw4

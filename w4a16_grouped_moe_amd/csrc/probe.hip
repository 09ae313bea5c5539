// On-box ceilings (measurement aids, not part of the layer): the HBM read
// rate and the dense fp16 MFMA rate.
//
// The layer is a read stream: per forward it reads ~430 MB and writes ~17 MB.
// Its roofline fraction is quoted against MI355X's 8 TB/s; this kernel gives
// the read rate the same box actually sustains, so the benchmark can also
// report the layer as a share of that. Every lane keeps eight 16-byte
// non-temporal loads in flight per iteration over a grid-stride loop, two
// workgroups of 1024 threads per CU: the fastest of the shapes measured on
// MI355X (about 6.5 TB/s; plain loads peak near 5.9 TB/s). A wave instruction
// covers whole 128-byte lines, which is what lets non-temporal loads pay. The
// data are folded into one word that is stored only if it equals a value the
// caller's fill never produces, so the loads cannot be removed.
#include "dgw4_internal.hpp"

namespace dgw4 {
namespace {

constexpr int kProbeThreads = 1024;
constexpr int kProbeBlocksPerCu = 2;
constexpr int kProbeUnroll = 8;
constexpr uint32_t kNever = 0x9E3779B9u;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kProbeThreads) read_probe_kernel(const u32x4 *__restrict__ p,
                                                                   size_t n16,
                                                                   uint32_t *__restrict__ sink)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u)
            v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u)
            acc ^= v[u][0] ^ v[u][3];
    }
    for (; i < n16; i += stride)
        acc ^= __builtin_nontemporal_load(p + i)[0];
    if (acc == kNever)
        sink[0] = acc;
}

// MFMA throughput probe: every wave runs eight independent accumulation
// chains of v_mfma_f32_16x16x32_f16 on operands held in registers (no memory
// traffic), two 512-thread workgroups per CU (four waves per SIMD), so the
// elapsed time gives the dense fp16 matrix rate this machine sustains. The sums
// are folded into one word, stored only if it equals kNever.
constexpr int kMfmaThreads = 512;
constexpr int kMfmaBlocksPerCu = 2;
constexpr int kMfmaChains = 8;

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kMfmaThreads) mfma_probe_kernel(int iters, uint32_t *__restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    f16x8_t a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (_Float16)(float)((lane + j) & 7) * (_Float16)0.0625f;
        b[j] = (_Float16)(float)((lane * 3 + j) & 7) * (_Float16)0.0625f;
    }
    f32x4_t acc[kMfmaChains];
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c)
        acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < kMfmaChains; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c)
        s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    if (__builtin_bit_cast(uint32_t, s) == kNever)
        sink[0] = kNever;
}

}  // namespace

hipError_t launch_mfma_probe(int iters, uint32_t *sink, double *flops, hipStream_t stream)
{
    int dev = 0, cus = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess)
        err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess)
        return err;
    const int blocks = cus * kMfmaBlocksPerCu;
    *flops = (double)blocks * (kMfmaThreads / 64) * (double)iters * kMfmaChains * (2.0 * 16 * 16 * 32);
    mfma_probe_kernel<<<dim3(blocks), dim3(kMfmaThreads), 0, stream>>>(iters, sink);
    return hipGetLastError();
}

hipError_t launch_read_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream)
{
    int dev = 0, cus = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess)
        err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess)
        return err;
    read_probe_kernel<<<dim3(cus * kProbeBlocksPerCu), dim3(kProbeThreads), 0, stream>>>(
        static_cast<const u32x4 *>(buf), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace dgw4

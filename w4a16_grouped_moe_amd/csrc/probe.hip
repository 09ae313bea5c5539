// On-box HBM read ceiling (a measurement aid, not part of the layer).
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

}  // namespace

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

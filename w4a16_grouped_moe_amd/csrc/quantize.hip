// Min/max round-to-nearest uint4 packer (dg-w4a16-v1 layout), and the
// reorder of its output into the GEMMs' tiled load layout.
//
// Follows the "dg-w4-kernels" card, section "W4A16" (quantize_w4 with a group
// size), the model card's "Benchmarks" (round-to-nearest min/max, no
// calibration) and "Checkpoint format" (fp16 scale and zero point per group,
// byte j = q[2j] | q[2j+1] << 4), and the Part 2 blog, "The first constraint
// was capacity" (groups of 128 for gate/up, 64 for down; integer codes).
//
// Per group, in fp32 with round-to-nearest-even and no contraction:
//   s = fp16((hi - lo) / 15), 1 if that is zero
//   z = clamp(rint(-lo / s), -2048, 2048)       (stored as fp16; 0 as +0)
//   q = clamp(rint(w / s) + z, 0, 15)
//
// Mapping: the weight tensor is a sequence of contiguous groups of g floats
// (groups run along K, rows are contiguous). One lane owns two neighbouring
// weights, i.e. one output byte, so a group spans g/2 lanes and a 64-lane wave
// covers 128/g groups. Loads are 8-byte and stores 1-byte per lane, both
// contiguous across the wave.
#include "dgw4_internal.hpp"

#pragma clang fp contract(off)

namespace dgw4 {
namespace {

template <int G>
__global__ void __launch_bounds__(256) quantize_rtn_kernel(const float2 *__restrict__ w,
                                                           long long groups,
                                                           uint8_t *__restrict__ q,
                                                           uint16_t *__restrict__ s,
                                                           uint16_t *__restrict__ z)
{
    constexpr int kLanesPerGroup = G / 2;
    constexpr int kGroupsPerWave = 64 / kLanesPerGroup;
    const int lane = threadIdx.x & 63;
    const long long wave = (long long)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    const long long grp = wave * kGroupsPerWave + lane / kLanesPerGroup;
    const int j = lane % kLanesPerGroup;                 // byte within the group
    const bool live = grp < groups;

    float2 v = make_float2(0.f, 0.f);
    if (live)
        v = w[grp * kLanesPerGroup + j];

    float lo = fminf(v.x, v.y), hi = fmaxf(v.x, v.y);
#pragma unroll
    for (int off = 1; off < kLanesPerGroup; off <<= 1) {
        lo = fminf(lo, __shfl_xor(lo, off, 64));
        hi = fmaxf(hi, __shfl_xor(hi, off, 64));
    }
    if (!live)
        return;

    const float range = __fsub_rn(hi, lo);
    const float s32 = __fdiv_rn(range, 15.0f);
    uint16_t sb = __builtin_bit_cast(uint16_t, (_Float16)s32);   // RN-even
    if ((sb & 0x7FFFu) == 0u)
        sb = 0x3C00u;                                    // 1.0
    const float sf = (float)__builtin_bit_cast(_Float16, sb);
    float zf = rintf(__fdiv_rn(-lo, sf));
    zf = fminf(fmaxf(zf, -2048.0f), 2048.0f);
    const int zi = (int)zf;

    float q0 = __fadd_rn(rintf(__fdiv_rn(v.x, sf)), zf);
    float q1 = __fadd_rn(rintf(__fdiv_rn(v.y, sf)), zf);
    q0 = fminf(fmaxf(q0, 0.0f), 15.0f);
    q1 = fminf(fmaxf(q1, 0.0f), 15.0f);
    q[grp * kLanesPerGroup + j] = (uint8_t)((int)q0 | ((int)q1 << 4));
    if (j == 0) {
        s[grp] = sb;
        z[grp] = __builtin_bit_cast(uint16_t, (_Float16)(float)zi);   // exact, +0 for 0
    }
}

// Canonical -> tiled reorder of packed weights (the GEMMs' load layout): one
// thread per 8-byte unit of the output, written in order; the source unit is
// row 16 t + lrow, byte gi g/2 + quarter g/8 + 8 sub of that row. The tiles of
// all experts follow each other (N is a multiple of 16), so t runs over the
// whole [E N / 16] stack.
template <int G>
__global__ void __launch_bounds__(256) pack_tiled_kernel(const uint2 *__restrict__ q, long long units,
                                                         int K, uint2 *__restrict__ qt)
{
    constexpr int kSub = G / 64;                   // 8-byte units per lane share
    const long long row_units = K / 16;            // 8-byte units per row
    const int groups = K / G;
    for (long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x; u < units;
         u += (long long)gridDim.x * blockDim.x) {
        const long long b = u / G;                 // (tile, group) block of 8 G bytes = G units
        const int w = (int)(u - b * G);
        const int lane = w / kSub, sub = w - lane * kSub;
        const long long t = b / groups;
        const int gi = (int)(b - t * groups);
        const long long row = t * 16 + (lane & 15);
        qt[u] = q[row * row_units + gi * (G / 16) + (lane >> 4) * kSub + sub];
    }
}

}  // namespace

hipError_t launch_pack_tiled(const uint8_t *q, long long rows, int K, int g, uint8_t *qt,
                             hipStream_t stream)
{
    const long long units = rows * (K / 16);
    if (units == 0)
        return hipSuccess;
    const long long want = (units + 255) / 256;
    const unsigned blocks = (unsigned)(want < 8192 ? want : 8192);
    const uint2 *src = reinterpret_cast<const uint2 *>(q);
    uint2 *dst = reinterpret_cast<uint2 *>(qt);
    if (g == 128)
        pack_tiled_kernel<128><<<dim3(blocks), dim3(256), 0, stream>>>(src, units, K, dst);
    else
        pack_tiled_kernel<64><<<dim3(blocks), dim3(256), 0, stream>>>(src, units, K, dst);
    return hipGetLastError();
}

hipError_t launch_quantize_rtn(const float *w, long long groups, int g, uint8_t *q,
                               uint16_t *s, uint16_t *z, hipStream_t stream)
{
    if (groups == 0)
        return hipSuccess;
    const int groups_per_block = 4 * (128 / g);          // 4 waves per block
    const long long blocks = (groups + groups_per_block - 1) / groups_per_block;
    const float2 *w2 = reinterpret_cast<const float2 *>(w);
    if (g == 128)
        quantize_rtn_kernel<128><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(w2, groups, q, s, z);
    else
        quantize_rtn_kernel<64><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(w2, groups, q, s, z);
    return hipGetLastError();
}

}  // namespace dgw4

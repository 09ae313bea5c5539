// Device helpers shared by the GEMM sources (not part of the ABI): buffer
// resources and loads, the packed-weight layouts and fragment loads, the
// nibble dequantisation, and the launch-time LDS allowance.
#pragma once

#include "dgw4_internal.hpp"

namespace dgw4 {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kXcds = 8;                          // accelerator dies (each with its own L2) on MI355X
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;     // a voffset no buffer here reaches

// Raw buffer resource over [base, base + bytes): reads past the end return 0.
__device__ inline rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ inline uint4 load16(rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// 8-byte store at voff; dropped past the end of the buffer.
__device__ inline void store8(rsrc_t r, uint32_t voff, uint2 v)
{
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, voff, 0, 0);
}

template <int G>
struct Frag;                     // one lane's share of one group of one weight row
template <>
struct Frag<128> { uint4 v; };   // 16 bytes = 32 nibbles
template <>
struct Frag<64> { uint2 v; };    // 8 bytes = 16 nibbles

// Packed weights come in one of two layouts (the same bytes, reordered):
//   canonical: q [E, N, K/2], row-major, two nibbles per byte along K;
//   tiled:     per expert, per 16-row block and per quantisation group, the
//              16 rows x g/2 bytes of that group stored in the order in which
//              the MFMA lanes hold them: [E][N/16][K/g][4][16][g/8], i.e.
//              (quarter q, row r) owns bytes q g/8 .. (q + 1) g/8 of row r's
//              group. One wave's load of a group is then 8 g contiguous bytes
//              (whole 128-byte lines), read once and not kept in the caches.
// Lane (quarter, lrow = lane % 16) of a wave that covers the 16 weight rows
// row - lrow .. row - lrow + 15 reads its share of group gi at
// wq_lane_off + wq_group_off(gi) (bytes, from the expert's first byte).
template <int G, bool TL>
__device__ inline uint32_t wq_lane_off(int row, int lane, int K)
{
    if constexpr (TL)
        return (uint32_t)(row - (lane & 15)) * (uint32_t)(K / 2) + (uint32_t)(lane * (G / 8));
    else
        return (uint32_t)row * (uint32_t)(K / 2) + (uint32_t)((lane >> 4) * (G / 8));
}

template <int G, bool TL>
__device__ constexpr uint32_t wq_group_off(int gi)
{
    return (uint32_t)gi * (TL ? 8u * G : G / 2u);
}

// NT: non-temporal (cache policy nt). Only for the tiled layout, whose loads
// cover whole lines, and only where no other workgroup will read the same
// weights (an expert with a single tile): the canonical layout's loads cover
// half or quarter lines whose rest the next group's load reads, and the
// other tiles of a busy expert re-read its weights from the caches.
template <int G, bool NT>
__device__ inline Frag<G> load_frag(rsrc_t r, uint32_t voff, uint32_t soff)
{
    constexpr int kCpol = NT ? 2 : 0;
    Frag<G> f;
    if constexpr (G == 128)
        f.v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCpol));
    else
        f.v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kCpol));
    return f;
}

template <int G>
__device__ inline uint32_t frag_word(const Frag<G> &f, int t)
{
    if constexpr (G == 128)
        return t == 0 ? f.v.x : t == 1 ? f.v.y : t == 2 ? f.v.z : f.v.w;
    else
        return t == 0 ? f.v.x : f.v.y;
}

__device__ inline f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }

// (w & mask) | magic in one v_and_or_b32 (gfx9 VOP3 takes no literal, so the
// compiler would otherwise split it). The result only feeds ordinary VALU
// (the packed subtract below), whose hazards the compiler tracks.
__device__ inline uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(magic));
    return r;
}

// 8 nibbles -> 8 exact fp16 values (q - z) in K order [0,4,1,5,2,6,3,7].
__device__ inline f16x8 dequant8(uint32_t w, f16x2 c1024, f16x2 c64)
{
    const uint32_t w8 = w >> 8;
    const f16x2 a = as_h2(and_or(w, 0x000F000Fu, 0x64006400u)) - c1024;
    const f16x2 b = as_h2(and_or(w, 0x00F000F0u, 0x54005400u)) - c64;
    const f16x2 c = as_h2(and_or(w8, 0x000F000Fu, 0x64006400u)) - c1024;
    const f16x2 d = as_h2(and_or(w8, 0x00F000F0u, 0x54005400u)) - c64;
    f16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

// The same eight nibbles as fp16 weights (q - z) * s in natural K order
// (n0 .. n7). A byte permute puts byte b at bytes 0 and 2, so that one mask
// takes its low nibble to bits 0-3 (fp16 1024 + n) and its high nibble to
// bits 20-23 (fp16 64 + n in the upper half); cmix = (1024 + z, 64 + z).
// q - z is exact, the product with s is rounded once.
__device__ inline f16x8 dequant8_scaled(uint32_t w, f16x2 cmix, f16x2 s2)
{
    const uint32_t u = __builtin_amdgcn_perm(w, w, 0x01000100u);   // bytes 0 1 0 1
    const uint32_t v = __builtin_amdgcn_perm(w, w, 0x03020302u);   // bytes 2 3 2 3
    const f16x2 a = (as_h2(and_or(u, 0x00F0000Fu, 0x54006400u)) - cmix) * s2;        // n0 n1
    const f16x2 b = (as_h2(and_or(u >> 8, 0x00F0000Fu, 0x54006400u)) - cmix) * s2;   // n2 n3
    const f16x2 c = (as_h2(and_or(v, 0x00F0000Fu, 0x54006400u)) - cmix) * s2;        // n4 n5
    const f16x2 d = (as_h2(and_or(v >> 8, 0x00F0000Fu, 0x54006400u)) - cmix) * s2;   // n6 n7
    f16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

// fp16(1024 + z) and fp16(64 + z) as packed pairs; exact for -2033 <= z <= 1024
__device__ inline void zero_point_consts(uint32_t zbits, f16x2 &c1024, f16x2 &c64)
{
    const f16x2 zz = as_h2(zbits | (zbits << 16));
    c1024 = zz + f16x2{(_Float16)1024.0f, (_Float16)1024.0f};
    c64 = zz + f16x2{(_Float16)64.0f, (_Float16)64.0f};
}

// GELU, tanh form: 0.5 v (1 + tanh(u)) with u = sqrt(2/pi) (v + 0.044715 v^3).
// Since 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)), this is v / (1 + exp(-2u)):
// one hardware exp2 and one reciprocal (each within about 1 ulp) instead of a
// library tanh. Both limits hold: exp2 -> +inf gives 0, exp2 -> 0 gives v.
__device__ inline float gelu_tanh(float v)
{
    const float k0 = 0.7978845608028654f;   // sqrt(2/pi)
    const float k1 = 0.044715f;
    const float m2log2e = -2.8853900817779268f;   // -2 log2(e)
    const float u = k0 * (v + k1 * v * v * v);
    return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(m2log2e * u));
}

// 8 consecutive fp16 values (K order 0..7) -> the same values in the
// dequantised weights' order [0,4,1,5,2,6,3,7].
__device__ inline uint4 permute8(uint4 v)
{
    uint4 o;
    o.x = (v.x & 0xFFFFu) | (v.z << 16);
    o.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
    o.z = (v.y & 0xFFFFu) | (v.w << 16);
    o.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
    return o;
}

// Four fp32 values rounded to fp16 (RN-even), packed in 8 bytes.
__device__ inline uint2 pack_f16x4(f32x4 v)
{
    const uint32_t h0 = __builtin_bit_cast(uint16_t, (_Float16)v[0]);
    const uint32_t h1 = __builtin_bit_cast(uint16_t, (_Float16)v[1]);
    const uint32_t h2 = __builtin_bit_cast(uint16_t, (_Float16)v[2]);
    const uint32_t h3 = __builtin_bit_cast(uint16_t, (_Float16)v[3]);
    return make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
}

// Position of column c inside its row when a row is stored permuted per 8
// (the inverse of the K order [0,4,1,5,2,6,3,7]).
__device__ inline int permuted_col(int c)
{
    const int j = c & 7;
    return (c & ~7) | ((j & 3) << 1) | (j >> 2);
}

template <class Kern>
hipError_t allow_lds(Kern kern, size_t lds, size_t &allowed)
{
    if (lds <= allowed)
        return hipSuccess;
    const hipError_t err =
        hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err == hipSuccess)
        allowed = lds;
    return err;
}

}  // namespace
}  // namespace dgw4

// Grouped W4A16 GEMMs of the routed-expert layer: gate_up with the gated
// activation in its epilogue, and down.
//
// Follows the "dg-w4-kernels" card, "Grouped MoE" (one launch covers every
// expert; the activation is folded into the first GEMM's epilogue) and
// "W4A16" (the GEMM reads packed nibbles and dequantises inline); the model
// card, "Checkpoint format" (w = (q - z) * s, one scale/zero per group along
// K, byte j = q[2j] | q[2j+1] << 4); and the Part 2 blog, "Quantisation alone
// leaves a sparse execution problem" and "The final best W4 MoE kernel"
// (assignments sorted by expert and padded to 32-row blocks).
//
// gfx950 design
// -------------
// Both GEMMs stream the packed weights straight from the canonical layout.
// A lane (row = lane % 16, quarter = lane / 16) loads g/8 bytes (16 for
// g = 128, 8 for g = 64) of one weight row per group, so the four quarters
// cover one whole group of 16 rows. Dequantisation builds exact fp16
// integers in registers: for a 32-bit word of nibbles n0..n7,
// (w & 0x000F000F) | 0x64006400 is the fp16 pair (1024 + n0, 1024 + n4) and
// (w & 0x00F000F0) | 0x54005400 is (64 + n1, 64 + n5); the same on w >> 8
// gives n2/n6 and n3/n7, and one packed fp16 subtract of (1024 + z) or
// (64 + z) leaves q - z exactly. The MFMA operand therefore holds K in the
// order [0,4,1,5,2,6,3,7] per 8; the activations are used in the same order
// (gate_up permutes x as it stages it, H is written permuted), which leaves
// the contraction unchanged and needs no weight preshuffle.
// v_mfma_f32_16x16x32_f16 accumulates one group into a fresh fp32 partial and
// the group's scale is applied once per output in fp32 (acc += s * partial),
// so no weight is ever rounded by its scale.
//
// Loads complete in issue order, and the compiler's wait counting is exact
// only in straight-line code without a vector store in flight: a loop back
// edge, or a store issued while loads are pending, turns waits into waits for
// the whole queue. So the step loops are fully unrolled for the layer's
// shapes (K = 2816 and 704; other shapes take a generic loop), every wait is
// for data issued a fixed number of steps earlier, and down keeps its outputs
// in registers until its last tile.
//
// gate_up: workgroup = (32-row tile, 128 output columns), 8 waves, each wave
// one 16-column gate tile and the matching up tile. K is walked in steps of
// one 128-byte line of every weight row (256 K = two g=128 groups); the
// weights and the activation slice of a step are loaded P = 2 steps ahead,
// together, and the slice goes through a double-buffered LDS stage with one
// barrier per step. Epilogue: gelu_tanh(gate) * up in fp32, H in fp16.
//
// down: workgroup = (32-row tile, part of 704 output columns), 4 waves. The
// tile's activations (all of K) and the part's scales/zero points are staged
// in LDS once; each wave then streams its 11 16-row weight tiles (all of K,
// P = 2 tiles ahead) without any barrier. The MFMA takes the weights as its
// row operand, so a lane ends with four consecutive output columns of one
// assignment row: one 16-byte store of fp32 Y per row and tile, at the
// assignment's flat slot t * topk + k.
//
// Both: tiles past the device-side total exit at once (static grid, no host
// readback); the work items of one tile run back to back on one XCD so that
// its activation rows stay in that XCD's L2; tiles with at most 16 valid rows
// run one 16-row MFMA block instead of two.
#include "dgw4_internal.hpp"

namespace dgw4 {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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

template <int G>
struct Frag;                     // one lane's share of one group of one weight row
template <>
struct Frag<128> { uint4 v; };   // 16 bytes = 32 nibbles
template <>
struct Frag<64> { uint2 v; };    // 8 bytes = 16 nibbles

template <int G>
__device__ inline Frag<G> load_frag(rsrc_t r, uint32_t voff, uint32_t soff)
{
    Frag<G> f;
    if constexpr (G == 128)
        f.v = load16(r, voff, soff);
    else
        f.v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
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

// Position of column c inside its row when a row is stored permuted per 8
// (the inverse of the K order [0,4,1,5,2,6,3,7]).
__device__ inline int permuted_col(int c)
{
    const int j = c & 7;
    return (c & ~7) | ((j & 3) << 1) | (j >> 2);
}

// ===========================================================================
// gate_up
//   kWaves  waves per workgroup
//   kTiles  MFMA column tiles (16 weight rows each) per wave: gate and up
//           alternate (tile 2p = gate rows, 2p + 1 = the matching up rows)
//   kAhead  line steps (256 K) in flight per wave
//   kWpe    waves per SIMD the register budget is sized for
template <int W, int T, int P, int WPE>
struct GuShape {
    static constexpr int kWaves = W;
    static constexpr int kTiles = T;
    static constexpr int kAhead = P;
    static constexpr int kWpe = WPE;
};
using GateUpShape = GuShape<8, 2, 2, 4>;
constexpr int kGuSteps = 11;        // line steps of K = 2816, the layer's hidden size
constexpr int kStepSeg = 32;        // 16-byte activation segments per row and step
constexpr int kStepPitch = kStepSeg + 1;   // +16 B per row: 16 rows at one segment hit 16 bank groups

// NSC > 0: the step count is a compile-time constant and the K loop is fully
// unrolled; NSC = 0: a generic loop over ceil(K / 256) steps.
template <int G, class S, int NMS, int NSC>
__device__ __forceinline__ void gate_up_body(const GemmArgs &p, int e, int valid, int row0, int nb)
{
    constexpr int WAVES = S::kWaves;
    constexpr int TPW = S::kTiles;
    constexpr int P = S::kAhead;
    constexpr int kThreads = WAVES * 64;
    constexpr int SG = 256 / G;                   // groups per line step
    constexpr int kWords = G / 32;
    constexpr int kColsPerWave = TPW / 2 * 16;
    constexpr int kColsPerWg = WAVES * kColsPerWave;
    constexpr int kRangeRows = kColsPerWg;        // gate rows (and up rows) of the workgroup
    constexpr int kRows = NMS * 16;               // activation rows staged
    constexpr int XLD = kRows * kStepSeg / kThreads;
    static_assert(kRows * kStepSeg % kThreads == 0 && kThreads % kStepSeg == 0, "activation split");
    static_assert(TPW % 2 == 0, "gate/up tiles come in pairs");
    constexpr int TRIP = NSC > 0 ? NSC : (P % 2 == 0 ? P : 2 * P);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
    const int lrow = lane & 15;
    const int quarter = lane >> 4;
    const int K = p.K;
    const int NG = K / G;
    const int NS = NSC > 0 ? NSC : (K + 255) / 256;
    const int n_out = p.n_out;
    const size_t wexp = (size_t)e * p.n_w;
    // a wave past the last column (n_out is a multiple of 16) loads no
    // weights, skips the math and stores nothing; it still stages activations
    const int col_first = nb * kColsPerWg + wave * kColsPerWave;
    const bool wave_live = col_first < n_out;
    const int range0 = nb * kColsPerWg;           // gate rows; up rows start at n_out + range0

    extern __shared__ uint4 lds[];
    uint4 *lds_x = lds;                                             // [2][32][kStepPitch]
    uint16_t *lds_s = reinterpret_cast<uint16_t *>(lds + 2 * kBlockM * kStepPitch);   // [2 kRangeRows][NG]
    uint16_t *lds_z = lds_s + 2 * kRangeRows * NG;
    __shared__ int s_src[kBlockM];

    // ---- 1. scale/zero loads (two contiguous row ranges), row ids, and the
    // weights of the first P steps. Scale/zero are issued first, so waiting
    // for them does not wait for weights.
    const rsrc_t rs = make_rsrc(p.s + wexp * (size_t)NG, (uint32_t)p.n_w * (uint32_t)NG * 2u);
    const rsrc_t rz = make_rsrc(p.z + wexp * (size_t)NG, (uint32_t)p.n_w * (uint32_t)NG * 2u);
    constexpr int kSzLoads = 2;
    const int range_seg = kRangeRows * NG / 8;     // 16-byte segments per range
    const int sz_total = 2 * range_seg;
    auto sz_off = [&](int x) -> uint32_t {
        if (x >= sz_total)
            return kOutOfRange;
        const int r = x >= range_seg;
        return (uint32_t)(((r ? n_out : 0) + range0) * NG) * 2u + (uint32_t)(x - r * range_seg) * 16u;
    };
    uint4 sv[kSzLoads], zv[kSzLoads];
#pragma unroll
    for (int i = 0; i < kSzLoads; ++i) {
        const uint32_t off = sz_off(i * kThreads + tid);
        sv[i] = load16(rs, off, 0);
        zv[i] = load16(rz, off, 0);
    }
    int fid = 0;
    if (tid < kBlockM)
        fid = p.sorted_ids[row0 + tid];           // row0 + tid < cap: always in the buffer

    const rsrc_t rq = make_rsrc(p.q + wexp * (size_t)(K / 2),
                                wave_live ? (uint32_t)p.n_w * (uint32_t)(K / 2) : 0u);
    uint32_t wvoff[TPW];
    int lds_row[TPW];                              // this lane's row in the scale/zero ranges
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        const int in_range = wave * kColsPerWave + (tt >> 1) * 16 + lrow;
        const int wr = ((tt & 1) ? n_out : 0) + range0 + in_range;
        lds_row[tt] = (tt & 1) * kRangeRows + in_range;
        wvoff[tt] = (uint32_t)wr * (uint32_t)(K / 2) + (uint32_t)(quarter * (G / 8));
    }
    Frag<G> bq[P][TPW][SG];
    auto issue_w = [&](int st, int s) {           // step s into register stage st
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
            for (int h = 0; h < SG; ++h) {
                const int gi = s * SG + h;
                bq[st][tt][h] = load_frag<G>(rq, gi < NG ? wvoff[tt] : kOutOfRange,
                                             (uint32_t)(s * 128 + h * (G / 2)));
            }
    };
#pragma unroll
    for (int s = 0; s < P; ++s)
        issue_w(s, s);
    __builtin_amdgcn_sched_barrier(0);

    // ---- 2. scale/zero and row sources into LDS
    {
        uint4 *ls = reinterpret_cast<uint4 *>(lds_s);
        uint4 *lz = reinterpret_cast<uint4 *>(lds_z);
#pragma unroll
        for (int i = 0; i < kSzLoads; ++i) {
            const int x = i * kThreads + tid;
            if (x < sz_total) {
                ls[x] = sv[i];
                lz[x] = zv[i];
            }
        }
        for (int x = kSzLoads * kThreads + tid; x < sz_total; x += kThreads) {   // large K only
            ls[x] = load16(rs, sz_off(x), 0);
            lz[x] = load16(rz, sz_off(x), 0);
        }
    }
    if (tid < kBlockM)
        s_src[tid] = tid < valid ? fid / p.topk : -1;
    __syncthreads();

    // ---- 3. activation slices: thread -> (row, 16-byte segment) of a step,
    // the segment the same in every row it loads; the first P steps now
    const rsrc_t ra = make_rsrc(p.a_src, (uint32_t)p.a_rows * (uint32_t)K * 2u);
    const int xseg = tid % kStepSeg;
    uint32_t xoff[XLD];
#pragma unroll
    for (int i = 0; i < XLD; ++i) {
        const int src = s_src[(i * kThreads + tid) / kStepSeg];
        xoff[i] = src >= 0 ? (uint32_t)src * (uint32_t)K * 2u + (uint32_t)xseg * 16u : kOutOfRange;
    }
    uint4 xr[P][XLD];
    auto issue_x = [&](int st, int s) {           // rows past `valid` and K past the end read 0
        const bool in_k = s * 256 + xseg * 8 < K;
#pragma unroll
        for (int i = 0; i < XLD; ++i)
            xr[st][i] = load16(ra, in_k && xoff[i] != kOutOfRange ? xoff[i] + (uint32_t)s * 512u
                                                                  : kOutOfRange, 0);
    };
#pragma unroll
    for (int s = 0; s < P; ++s)
        issue_x(s, s);

    f32x4 acc[TPW][NMS];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int ms = 0; ms < NMS; ++ms)
            acc[tt][ms] = f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    // ---- 4. K loop, one line step per iteration: the step's activations
    // into LDS (reordered per 8), one barrier (everyone is done with the step
    // two back, whose buffer this one reuses), the step's groups, then the
    // loads of the step P ahead. Steps past the end read zeros and their
    // groups have scale 0.
    for (int s0 = 0; s0 < NS; s0 += TRIP) {
#pragma unroll
        for (int j = 0; j < TRIP; ++j) {
            const int s = s0 + j;
            const int st = j % P;
            uint4 *xb = lds_x + (j & 1) * kBlockM * kStepPitch;
#pragma unroll
            for (int i = 0; i < XLD; ++i)
                xb[((i * kThreads + tid) / kStepSeg) * kStepPitch + xseg] = permute8(xr[st][i]);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            if (wave_live) {
#pragma unroll
                for (int h = 0; h < SG; ++h) {
                    const int gi = s * SG + h;
                    const int gc = min(gi, NG - 1);
                    float scale[TPW];
                    f16x2 c1024[TPW], c64[TPW];
#pragma unroll
                    for (int tt = 0; tt < TPW; ++tt) {
                        zero_point_consts(lds_z[lds_row[tt] * NG + gc], c1024[tt], c64[tt]);
                        const float sc = (float)__builtin_bit_cast(_Float16, lds_s[lds_row[tt] * NG + gc]);
                        scale[tt] = gi < NG ? sc : 0.0f;
                    }
                    f32x4 part[TPW][NMS];
#pragma unroll
                    for (int t = 0; t < kWords; ++t) {
                        f16x8 bop[TPW];
#pragma unroll
                        for (int tt = 0; tt < TPW; ++tt)
                            bop[tt] = dequant8(frag_word<G>(bq[st][tt][h], t), c1024[tt], c64[tt]);
                        const int seg = h * (G / 8) + quarter * (G / 32) + t;   // this lane's 8 K positions
#pragma unroll
                        for (int ms = 0; ms < NMS; ++ms) {
                            const f16x8 aop = __builtin_bit_cast(f16x8, xb[(ms * 16 + lrow) * kStepPitch + seg]);
#pragma unroll
                            for (int tt = 0; tt < TPW; ++tt)
                                part[tt][ms] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                    aop, bop[tt], t == 0 ? zero4 : part[tt][ms], 0, 0, 0);
                        }
                    }
#pragma unroll
                    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
                        for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                acc[tt][ms][i] += scale[tt] * part[tt][ms][i];
                }
            }
            issue_x(st, s + P);
            issue_w(st, s + P);
        }
    }

    // ---- 5. epilogue: H = gelu_tanh(gate) * up in fp16 at the tile's padded
    // row, permuted per 8 columns. MFMA 16x16 output: lane holds rows
    // 4 * quarter + i, column lrow.
    if (!wave_live)
        return;
    uint16_t *H = static_cast<uint16_t *>(p.out);
#pragma unroll
    for (int ms = 0; ms < NMS; ++ms) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = ms * 16 + quarter * 4 + i;
            if (r >= valid)
                continue;
#pragma unroll
            for (int pp = 0; pp < TPW / 2; ++pp) {
                const int col = col_first + pp * 16 + lrow;
                const float h = gelu_tanh(acc[2 * pp][ms][i]) * acc[2 * pp + 1][ms][i];
                H[(size_t)(row0 + r) * n_out + permuted_col(col)] =
                    __builtin_bit_cast(uint16_t, (_Float16)h);
            }
        }
    }
}

template <int G, class S>
__global__ void __launch_bounds__(S::kWaves * 64)
__attribute__((amdgpu_waves_per_eu(S::kWpe))) gate_up_kernel(GemmArgs p)
{
    // workgroup -> (N-block, tile), XCD-aware: consecutive workgroups go to
    // the XCDs in turn, so XCD x takes tiles x, x + 8, ... and runs all
    // N-blocks of a tile back to back, its activation rows staying in L2
    constexpr int kColsPerWg = S::kWaves * S::kTiles / 2 * 16;
    const int nblocks = (p.n_out + kColsPerWg - 1) / kColsPerWg;
    const int xcd = (int)blockIdx.x % kXcds, slot = (int)blockIdx.x / kXcds;
    const int nb = slot % nblocks;
    const int tile = slot / nblocks * kXcds + xcd;
    if (tile >= p.max_tiles)
        return;
    const int2 info = p.tile_info[tile];           // {expert, valid rows}; -1 past the total
    if (info.x < 0)
        return;
    if ((p.K + 255) / 256 == kGuSteps) {
        if (info.y > 16)
            gate_up_body<G, S, 2, kGuSteps>(p, info.x, info.y, tile * kBlockM, nb);
        else
            gate_up_body<G, S, 1, kGuSteps>(p, info.x, info.y, tile * kBlockM, nb);
    } else {
        if (info.y > 16)
            gate_up_body<G, S, 2, 0>(p, info.x, info.y, tile * kBlockM, nb);
        else
            gate_up_body<G, S, 1, 0>(p, info.x, info.y, tile * kBlockM, nb);
    }
}

template <int G, class S>
size_t gate_up_lds_bytes(int K)
{
    const size_t range_rows = (size_t)S::kWaves * S::kTiles / 2 * 16;
    return sizeof(uint4) * 2 * kBlockM * kStepPitch + 2 * sizeof(uint16_t) * 2 * range_rows * (size_t)(K / G);
}

// ===========================================================================
// down
//   kWaves  waves per workgroup
//   kAhead  weight row tiles (16 rows, all of K) in flight per wave
//   kTiles  row tiles per wave (static: the loop is fully unrolled)
//   kWpe    waves per SIMD the register budget is sized for
template <int W, int P, int RT, int WPE>
struct DnShape {
    static constexpr int kWaves = W;
    static constexpr int kAhead = P;
    static constexpr int kTiles = RT;
    static constexpr int kWpe = WPE;
};
using DownShape = DnShape<4, 2, 11, 2>;
constexpr int kDnGroups = 11;       // K / 64 of the layer's down projection (m = 704)

// NGC: groups per weight tile, known at compile time. Groups past K / G (a
// generic instantiation rounded up) read no weights and have scale 0.
template <int G, class S, int NMS, int NGC>
__device__ __forceinline__ void down_body(const GemmArgs &p, int e, int valid, int row0, int part)
{
    constexpr int WAVES = S::kWaves;
    constexpr int P = S::kAhead;
    constexpr int RT = S::kTiles;
    constexpr int kThreads = WAVES * 64;
    constexpr int kWords = G / 32;
    constexpr int kPartTiles = WAVES * RT;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lrow = lane & 15;
    const int quarter = lane >> 4;
    const int K = p.K;
    const int NG = K / G;
    const int n_out = p.n_out;
    const size_t wexp = (size_t)e * p.n_w;
    // this part's row tiles: [rt0, rt0 + nrt) of the n_out / 16 weight tiles
    const int rt0 = part * kPartTiles;
    const int nrt = min(kPartTiles, n_out / 16 - rt0);
    const int rows_part = nrt * 16;

    extern __shared__ uint4 lds[];
    const int a_pitch = K / 8 + 1;                                  // uint4 per activation row
    uint4 *lds_a = lds;                                             // [32][a_pitch]
    uint16_t *lds_s = reinterpret_cast<uint16_t *>(lds + kBlockM * a_pitch);   // [part rows][NG]
    uint16_t *lds_z = lds_s + kPartTiles * 16 * NG;
    __shared__ int s_dst[kBlockM];

    // ---- 1. scale/zero of the part's rows (one contiguous range each), row
    // ids, the first weight tiles of this wave, then the activation rows
    const rsrc_t rs = make_rsrc(p.s + wexp * (size_t)NG, (uint32_t)p.n_w * (uint32_t)NG * 2u);
    const rsrc_t rz = make_rsrc(p.z + wexp * (size_t)NG, (uint32_t)p.n_w * (uint32_t)NG * 2u);
    const int sz_seg = (rows_part * NG * 2 + 15) / 16;              // 16-byte segments per array
    const uint32_t sz_base = (uint32_t)(rt0 * 16 * NG) * 2u;
    constexpr int kSzLoads = 4;
    uint4 sv[kSzLoads], zv[kSzLoads];
#pragma unroll
    for (int i = 0; i < kSzLoads; ++i) {
        const int x = i * kThreads + tid;
        const uint32_t off = x < sz_seg ? sz_base + (uint32_t)x * 16u : kOutOfRange;
        sv[i] = load16(rs, off, 0);
        zv[i] = load16(rz, off, 0);
    }
    int fid = 0;
    if (tid < kBlockM)
        fid = p.sorted_ids[row0 + tid];

    const rsrc_t rq = make_rsrc(p.q + wexp * (size_t)(K / 2), (uint32_t)p.n_w * (uint32_t)(K / 2));
    // wave w takes row tiles rt0 + w, rt0 + w + WAVES, ...; tiles past the
    // part read no weights and store nothing
    auto tile_live = [&](int j) { return wave + j * WAVES < nrt; };
    auto tile_row = [&](int j) { return (rt0 + wave + j * WAVES) * 16; };   // first weight row
    Frag<G> bq[P][NGC];
    auto issue_w = [&](int st, int j) {
        const uint32_t voff = j < RT && tile_live(j)
                                  ? (uint32_t)(tile_row(j) + lrow) * (uint32_t)(K / 2) +
                                        (uint32_t)(quarter * (G / 8))
                                  : kOutOfRange;
#pragma unroll
        for (int g = 0; g < NGC; ++g)
            bq[st][g] = load_frag<G>(rq, g < NG ? voff : kOutOfRange, (uint32_t)(g * (G / 2)));
    };
#pragma unroll
    for (int j = 0; j < P; ++j)
        issue_w(j, j);

    // activation rows row0 .. row0 + 16 NMS, already in the permuted K order
    // (rows past `valid` read 0)
    const rsrc_t ra = make_rsrc(p.a_src, (uint32_t)p.a_rows * (uint32_t)K * 2u);
    const int seg_row = K / 8;
    const int a_total = 16 * NMS * seg_row;
    for (int x0 = 0; x0 < a_total; x0 += 8 * kThreads) {
        uint4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int x = x0 + i * kThreads + tid;
            const int r = min(x / seg_row, 16 * NMS - 1), sg = x - r * seg_row;
            v[i] = load16(ra, x < a_total && r < valid
                                  ? (uint32_t)(row0 + r) * (uint32_t)K * 2u + (uint32_t)sg * 16u
                                  : kOutOfRange, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int x = x0 + i * kThreads + tid;
            const int r = min(x / seg_row, 16 * NMS - 1), sg = x - r * seg_row;
            if (x < a_total)
                lds_a[r * a_pitch + sg] = v[i];
        }
    }
    {
        uint4 *ls = reinterpret_cast<uint4 *>(lds_s);
        uint4 *lz = reinterpret_cast<uint4 *>(lds_z);
#pragma unroll
        for (int i = 0; i < kSzLoads; ++i) {
            const int x = i * kThreads + tid;
            if (x < sz_seg) {
                ls[x] = sv[i];
                lz[x] = zv[i];
            }
        }
        for (int x = kSzLoads * kThreads + tid; x < sz_seg; x += kThreads) {   // large K only
            ls[x] = load16(rs, sz_base + (uint32_t)x * 16u, 0);
            lz[x] = load16(rz, sz_base + (uint32_t)x * 16u, 0);
        }
    }
    if (tid < kBlockM)
        s_dst[tid] = tid < valid ? fid : -1;
    __syncthreads();

    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    // the MFMAs take the weights as the row operand: a lane ends with four
    // consecutive output columns (weight rows 4 * quarter + i) of assignment
    // row lrow (+16 for the second block)
    int dst[NMS];
#pragma unroll
    for (int ms = 0; ms < NMS; ++ms)
        dst[ms] = s_dst[ms * 16 + lrow];
    f32x4 out[RT][NMS];

    // ---- 2. stream this wave's row tiles, as straight-line code
#pragma unroll
    for (int j = 0; j < RT; ++j) {
        const int st = j % P;
        // the activation reads are the same for every tile: an opaque offset
        // keeps the compiler from holding all of them in registers
        int aoff = 0;
        asm volatile("" : "+v"(aoff));
        const int srow = min(tile_row(j) - rt0 * 16, max(0, rows_part - 16));   // first row in lds_s/lds_z
#pragma unroll
        for (int ms = 0; ms < NMS; ++ms)
            out[j][ms] = zero4;
#pragma unroll
        for (int g = 0; g < NGC; ++g) {
            const int gc = min(g, NG - 1);
            f16x2 c1024, c64;
            zero_point_consts(lds_z[(srow + lrow) * NG + gc], c1024, c64);
            float sc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = (float)__builtin_bit_cast(_Float16, lds_s[(srow + quarter * 4 + i) * NG + gc]);
                sc[i] = g < NG ? v : 0.0f;
            }
            f32x4 prt[NMS];
#pragma unroll
            for (int t = 0; t < kWords; ++t) {
                const f16x8 bop = dequant8(frag_word<G>(bq[st][g], t), c1024, c64);
                const int seg = gc * (G / 8) + quarter * (G / 32) + t;
#pragma unroll
                for (int ms = 0; ms < NMS; ++ms) {
                    const f16x8 aop = __builtin_bit_cast(f16x8, lds_a[aoff + (ms * 16 + lrow) * a_pitch + seg]);
                    prt[ms] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bop, aop, t == 0 ? zero4 : prt[ms], 0, 0, 0);
                }
            }
#pragma unroll
            for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    out[j][ms][i] += sc[i] * prt[ms][i];
            // pin the accumulation here: otherwise the compiler sinks every
            // tile's multiply-adds to the stores and keeps all partials live
#pragma unroll
            for (int ms = 0; ms < NMS; ++ms)
                asm volatile("" : "+v"(out[j][ms]));
        }
        issue_w(st, j + P);
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- 3. outputs: fp32 Y at each assignment's flat slot, one 16-byte
    // store per assignment row and tile
    float *Y = static_cast<float *>(p.out);
#pragma unroll
    for (int j = 0; j < RT; ++j) {
        if (!tile_live(j))
            continue;
        const int col = tile_row(j) + quarter * 4;
#pragma unroll
        for (int ms = 0; ms < NMS; ++ms)
            if (dst[ms] >= 0)
                *reinterpret_cast<f32x4 *>(Y + (size_t)dst[ms] * n_out + col) = out[j][ms];
    }
}

template <int G, class S>
__global__ void __launch_bounds__(S::kWaves * 64)
__attribute__((amdgpu_waves_per_eu(S::kWpe))) down_kernel(GemmArgs p, int parts)
{
    // workgroup -> (part, tile), XCD-aware as in gate_up
    const int xcd = (int)blockIdx.x % kXcds, slot = (int)blockIdx.x / kXcds;
    const int part = slot % parts;
    const int tile = slot / parts * kXcds + xcd;
    if (tile >= p.max_tiles)
        return;
    const int2 info = p.tile_info[tile];
    if (info.x < 0)
        return;
    const int ng = p.K / G;
    // group counts with an instantiation: the layer's (11 groups of 64), else
    // the next of 12 / 24 groups of 64 (6 / 12 of 128) with idle groups masked
    constexpr int kSmall = 768 / G, kLarge = 1536 / G;
    if (G == 64 && ng == kDnGroups) {
        if (info.y > 16)
            down_body<G, S, 2, kDnGroups>(p, info.x, info.y, tile * kBlockM, part);
        else
            down_body<G, S, 1, kDnGroups>(p, info.x, info.y, tile * kBlockM, part);
    } else if (ng <= kSmall) {
        if (info.y > 16)
            down_body<G, S, 2, kSmall>(p, info.x, info.y, tile * kBlockM, part);
        else
            down_body<G, S, 1, kSmall>(p, info.x, info.y, tile * kBlockM, part);
    } else {
        if (info.y > 16)
            down_body<G, S, 2, kLarge>(p, info.x, info.y, tile * kBlockM, part);
        else
            down_body<G, S, 1, kLarge>(p, info.x, info.y, tile * kBlockM, part);
    }
}

template <int G, class S>
size_t down_lds_bytes(int K)
{
    const size_t part_rows = (size_t)S::kWaves * S::kTiles * 16;
    return sizeof(uint4) * kBlockM * ((size_t)K / 8 + 1) +
           2 * sizeof(uint16_t) * part_rows * (size_t)(K / G);
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

template <int G>
hipError_t launch_gate_up_g(const GemmArgs &a, hipStream_t stream)
{
    using S = GateUpShape;
    constexpr int cols_per_wg = S::kWaves * S::kTiles / 2 * 16;
    const int nblocks = (a.n_out + cols_per_wg - 1) / cols_per_wg;
    if (a.max_tiles == 0 || nblocks == 0)
        return hipSuccess;
    auto kern = gate_up_kernel<G, S>;
    static size_t allowed = 64 * 1024;              // raised once per instantiation when needed
    const size_t lds = gate_up_lds_bytes<G, S>(a.K);
    hipError_t err = allow_lds(kern, lds, allowed);
    if (err != hipSuccess)
        return err;
    const int tiles = (a.max_tiles + kXcds - 1) / kXcds * kXcds;
    kern<<<dim3(tiles * nblocks), dim3(S::kWaves * 64), lds, stream>>>(a);
    return hipGetLastError();
}

template <int G>
hipError_t launch_down_g(const GemmArgs &a, hipStream_t stream)
{
    using S = DownShape;
    if (a.max_tiles == 0)
        return hipSuccess;
    const int parts = (a.n_out / 16 + S::kWaves * S::kTiles - 1) / (S::kWaves * S::kTiles);
    auto kern = down_kernel<G, S>;
    static size_t allowed = 64 * 1024;
    const size_t lds = down_lds_bytes<G, S>(a.K);
    hipError_t err = allow_lds(kern, lds, allowed);
    if (err != hipSuccess)
        return err;
    const int tiles = (a.max_tiles + kXcds - 1) / kXcds * kXcds;
    kern<<<dim3(tiles * parts), dim3(S::kWaves * 64), lds, stream>>>(a, parts);
    return hipGetLastError();
}

}  // namespace

size_t gemm_lds_bytes(bool gated, int K, int g)
{
    if (gated)
        return g == 128 ? gate_up_lds_bytes<128, GateUpShape>(K) : gate_up_lds_bytes<64, GateUpShape>(K);
    return g == 128 ? down_lds_bytes<128, DownShape>(K) : down_lds_bytes<64, DownShape>(K);
}

int down_max_k() { return 1536; }

hipError_t launch_gate_up(const GemmArgs &a, int g, hipStream_t stream)
{
    return g == 128 ? launch_gate_up_g<128>(a, stream) : launch_gate_up_g<64>(a, stream);
}

hipError_t launch_down(const GemmArgs &a, int g, hipStream_t stream)
{
    return g == 128 ? launch_down_g<128>(a, stream) : launch_down_g<64>(a, stream);
}

}  // namespace dgw4

// Grouped W4A16 GEMMs of the routed-expert layer: gate_up with the gated
// activation in its epilogue, and down.
//
// Follows the "dg-w4-kernels" card, "Grouped MoE" (one launch covers every
// expert; the activation is folded into the first GEMM's epilogue) and
// "W4A16" (the GEMM reads packed nibbles and dequantises inline); the model
// card, "Checkpoint format" (w = (q - z) * s, one scale/zero per group along
// K, byte j = q[2j] | q[2j+1] << 4; the group size matches the K step so one
// scale and zero serve a whole K chunk); and the Part 2 blog, "Quantisation
// alone leaves a sparse execution problem" and "The final best W4 MoE
// kernel" (assignments sorted by expert and padded to 32-row blocks).
//
// gfx950 design
// -------------
// Work item (N-block, tile): tile = one 32-row block of the padded
// assignment list (one expert), N-block = the output columns of one
// workgroup. Tiles past the device-side total exit at once, so the grid is
// static and the host never reads the routing. Items are laid out so that
// every N-block of a tile runs on the same XCD, back to back.
//
// Each wave streams its 32 weight rows once, straight from the canonical
// packed layout: per group and column tile a lane loads g/8 bytes (16 bytes
// for g=128, 8 for g=64) of one weight row with a buffer load whose group
// offset is scalar; the four lane groups of 16 cover one whole group of that
// row. D groups are in flight per wave; they stay in flight across the
// workgroup barriers (the barrier waits only for LDS traffic).
//
// Dequantisation builds exact fp16 integers in registers: for a 32-bit word
// holding nibbles n0..n7, (w & 0x000F000F) | 0x64006400 is the fp16 pair
// (1024 + n0, 1024 + n4) and (w & 0x00F000F0) | 0x54005400 is (64 + n1,
// 64 + n5); the same on w >> 8 gives n2/n6 and n3/n7. One packed fp16
// subtract of (1024 + z) or (64 + z) leaves the exact integers q - z. The
// MFMA B operand therefore holds K positions in the order [0,4,1,5,2,6,3,7]
// within each 8. A contraction is unchanged by the same permutation on both
// operands, so the activations are consumed in that same order: gate_up
// permutes each 8 values of x as it stages them in LDS, and H is written
// permuted by gate_up's epilogue. No weight preshuffle is needed.
//
// v_mfma_f32_16x16x32_f16 accumulates one group (g/32 MFMAs) into a fresh
// fp32 partial; the group's scale is applied once per output in fp32
// (acc += s * partial). The scale never touches an fp16 weight, so the only
// rounding is the fp32 accumulation.
//
// Activations: the tile's 32 rows are staged through LDS, either in K chunks
// of 512 (double-buffered, loaded into registers one chunk ahead; gate_up)
// or the whole K at once (down, K = m). Scale and zero point of the
// workgroup's rows are copied into LDS once, as contiguous row ranges.
//
// Epilogues: gate_up computes gelu_tanh(gate) * up in fp32 and writes H in
// fp16 at the tile's padded row (permuted per 8 columns, see above); down
// writes fp32 Y at the assignment's flat slot t * topk + k, which the combine
// reads in ascending k.
#include "dgw4_internal.hpp"

#include <type_traits>

namespace dgw4 {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kSingleK = 768;            // largest K staged at once (one loop-free pass)
constexpr int kXcds = 8;                 // accelerator dies (each with its own L2) on MI355X
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;    // a voffset no buffer here reaches

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
// compiler would otherwise split it). The result only feeds ordinary VALU.
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

// Launch shape of one GEMM kernel instantiation.
//   kWaves    waves per workgroup
//   kTiles    MFMA column tiles (16 weight rows each) per wave; gated: gate and
//             up tiles alternate (tile 2p = gate rows, 2p + 1 = the matching
//             up rows), so a wave owns kTiles / 2 * 16 output columns
//   kChunkK   activation K per LDS chunk (0: the whole K staged at once)
//   kAhead    activation chunks of weight groups kept in flight per wave
//   kWpe      waves per SIMD the register budget is sized for
template <int W, int T, int CK, int AH, int WPE>
struct Shape {
    static constexpr int kWaves = W;
    static constexpr int kTiles = T;
    static constexpr int kChunkK = CK;
    static constexpr int kAhead = AH;
    static constexpr int kWpe = WPE;
};

template <int G, bool GATED, class S>
__global__ void __launch_bounds__(S::kWaves * 64)
__attribute__((amdgpu_waves_per_eu(S::kWpe))) moe_gemm_kernel(GemmArgs p)
{
    constexpr int WAVES = S::kWaves;
    constexpr int TPW = S::kTiles;
    constexpr bool SINGLE = S::kChunkK == 0;
    constexpr int kThreads = WAVES * 64;
    constexpr int kWords = G / 32;                 // MFMA K steps per group = words per fragment
    constexpr int kChunkK = SINGLE ? G : S::kChunkK;
    constexpr int kChunkSeg = kChunkK / 8;         // 16-byte segments per row and chunk
    constexpr int kChunkPitch = kChunkSeg + 1;     // +16 B per row: spreads LDS banks
    constexpr int CG = kChunkK / G;                // groups per activation chunk
    // weight groups in flight per wave: all of K when staged at once, else
    // kAhead chunks
    constexpr int D = SINGLE ? kSingleK / G : S::kAhead * CG;
    // chunks per loop trip: register stages and the two LDS buffers both
    // repeat with it, so every index is static inside a trip
    constexpr int TRIP = S::kAhead % 2 == 0 ? S::kAhead : 2 * S::kAhead;
    constexpr int kColsPerWave = GATED ? TPW / 2 * 16 : TPW * 16;
    constexpr int kColsPerWg = WAVES * kColsPerWave;
    constexpr int kRangeRows = WAVES * TPW * 8;    // rows of each scale/zero range
    constexpr int kChunkLoads = kBlockM * kChunkSeg / kThreads;
    static_assert(!GATED || TPW % 2 == 0, "gated tiles come in gate/up pairs");
    // Workgroup -> (N-block, tile), XCD-aware: consecutive workgroups are
    // dispatched to the XCDs in turn, so XCD x takes tiles x, x + 8, ... and
    // runs all N-blocks of a tile back to back; the tile's activation rows
    // then stay in that XCD's L2 while its N-blocks reuse them.
    const int nblocks = (p.n_out + kColsPerWg - 1) / kColsPerWg;
    const int xcd = (int)blockIdx.x % kXcds, slot = (int)blockIdx.x / kXcds;
    const int nb = slot % nblocks;
    const int tile = slot / nblocks * kXcds + xcd;
    if (tile >= p.max_tiles)
        return;
    const int2 info = p.tile_info[tile];           // {expert, valid rows}; -1 past the total
    if (info.x < 0)
        return;
    const int e = info.x;
    const int valid = info.y;
    const int row0 = tile * kBlockM;               // first padded row of this tile

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
    const int lrow = lane & 15;
    const int quarter = lane >> 4;
    const int K = p.K;
    const int NG = K / G;
    const size_t wexp = (size_t)e * p.n_w;

    // columns owned by this wave. A wave past the edge (n_out is a multiple
    // of its width) runs the same code on an empty weight buffer: its loads
    // return zeros without touching memory, and it stores nothing.
    const int col_first = nb * kColsPerWg + wave * kColsPerWave;
    const bool wave_live = col_first < p.n_out;
    // the two scale/zero row ranges of this workgroup (each kRangeRows rows):
    // gated: its gate rows and the matching up rows; down: its rows in two halves
    const int range0 = nb * kColsPerWg;
    const int range1 = GATED ? p.n_out + range0 : range0 + kRangeRows;

    extern __shared__ uint4 lds[];
    // [A buffers][scale][zero]: A is [kBlockM][pitch] uint4, scale/zero are
    // [2 * kRangeRows][NG] fp16
    const int a_pitch = SINGLE ? K / 8 + 1 : kChunkPitch;
    const int a_entries = SINGLE ? kBlockM * a_pitch : 2 * kBlockM * kChunkPitch;
    uint16_t *lds_s = reinterpret_cast<uint16_t *>(lds + a_entries);
    uint16_t *lds_z = lds_s + 2 * kRangeRows * NG;
    __shared__ int s_src[kBlockM];

    // ---- 1. scale/zero of the workgroup's rows (two contiguous ranges of
    // kRangeRows * NG fp16 each, 16-byte aligned) and the tile's row ids.
    // Issued before the weight prefetch so that waiting for them does not
    // wait for weights (loads complete in issue order).
    const rsrc_t rs = make_rsrc(p.s + wexp * (size_t)NG, (uint32_t)p.n_w * (uint32_t)NG * 2u);
    const rsrc_t rz = make_rsrc(p.z + wexp * (size_t)NG, (uint32_t)p.n_w * (uint32_t)NG * 2u);
    constexpr int kSzLoads = 8;                    // 16-byte loads per thread and array
    const int range_seg = kRangeRows * NG / 8;     // 16-byte segments per range
    const int sz_total = 2 * range_seg;
    auto sz_off = [&](int x) -> uint32_t {
        if (x >= sz_total)
            return kOutOfRange;
        const int r = x >= range_seg;
        return (uint32_t)((r ? range1 : range0) * NG) * 2u + (uint32_t)(x - r * range_seg) * 16u;
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
        fid = p.sorted_ids[row0 + tid];            // row0 + tid < cap: always in the buffer

    // ---- 2. weight prefetch, D groups
    const rsrc_t rq = make_rsrc(p.q + wexp * (size_t)(K / 2),
                                wave_live ? (uint32_t)p.n_w * (uint32_t)(K / 2) : 0u);
    uint32_t wvoff[TPW];
    int lds_row[TPW];                              // this lane's row in the scale/zero ranges
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        int wr;
        if constexpr (GATED) {
            const int in_range = wave * kColsPerWave + (tt >> 1) * 16 + lrow;
            wr = ((tt & 1) ? range1 : range0) + in_range;
            lds_row[tt] = (tt & 1) * kRangeRows + in_range;
        } else {
            const int in_range = wave * kColsPerWave + tt * 16 + lrow;
            wr = range0 + in_range;
            lds_row[tt] = in_range;
        }
        wvoff[tt] = (uint32_t)wr * (uint32_t)(K / 2) + (uint32_t)(quarter * (G / 8));
    }
    Frag<G> bq[D][TPW];
    auto prefetch = [&](int s, int gi) {      // group gi (clamped) into stage s
        gi = min(gi, NG - 1);
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
            bq[s][tt] = load_frag<G>(rq, wvoff[tt], (uint32_t)(gi * (G / 2)));
    };
#pragma unroll
    for (int s = 0; s < D; ++s)
        prefetch(s, s);
    __builtin_amdgcn_sched_barrier(0);

    // ---- 3. scale/zero and row sources into LDS
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
        for (int x = kSzLoads * kThreads + tid; x < sz_total; x += kThreads) {   // large NG only
            ls[x] = load16(rs, sz_off(x), 0);
            lz[x] = load16(rz, sz_off(x), 0);
        }
    }
    if (tid < kBlockM)
        s_src[tid] = tid < valid ? (GATED ? fid / p.topk : row0 + tid) : -1;
    __syncthreads();

    // ---- 4. activation staging (sources are already in the permuted K order)
    const rsrc_t ra = make_rsrc(p.a_src, (uint32_t)p.a_rows * (uint32_t)K * 2u);
    uint4 *lds_a = lds;
    f32x4 acc[TPW][2];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
            acc[tt][ms] = f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    const f16x2 k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
    const f16x2 k64 = {(_Float16)64.0f, (_Float16)64.0f};

    // group gi from stage s over NMS 16-row blocks, reading activations at
    // 16-byte segment seg0 (+ lane offsets) of the LDS rows starting at abuf.
    // A group past the last one (gi >= NG, in a padded trip) contributes
    // exactly nothing: its scale is taken as 0 and every index is clamped.
    auto group = [&](int s, const uint4 *abuf, int pitch, int seg0, int gi, auto nms_tag) {
        constexpr int NMS = decltype(nms_tag)::value;
        f16x2 c1024[TPW], c64[TPW];
        float scale[TPW];
        const int gc = min(gi, NG - 1);
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const uint32_t zb = lds_z[lds_row[tt] * NG + gc];
            const f16x2 zz = as_h2(zb | (zb << 16));
            c1024[tt] = zz + k1024;          // fp16(1024 + z), exact for |z| <= 1024
            c64[tt] = zz + k64;
            const float sc = (float)__builtin_bit_cast(_Float16, lds_s[lds_row[tt] * NG + gc]);
            scale[tt] = gi < NG ? sc : 0.0f;
        }
        f32x4 part[TPW][NMS];
#pragma unroll
        for (int t = 0; t < kWords; ++t) {
            f16x8 bop[TPW];
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt)
                bop[tt] = dequant8(frag_word<G>(bq[s][tt], t), c1024[tt], c64[tt]);
            const int seg = seg0 + quarter * (G / 32) + t;   // this lane's 8 K positions
#pragma unroll
            for (int ms = 0; ms < NMS; ++ms) {
                const f16x8 aop = __builtin_bit_cast(f16x8, abuf[(ms * 16 + lrow) * pitch + seg]);
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
    };

    if constexpr (SINGLE) {
        // the whole K of the tile's rows, once; every weight group of the wave
        // is already in flight (D >= NG), so there is no loop at all
        const int seg_row = K / 8;
        const int n = kBlockM * seg_row;
        for (int x0 = 0; x0 < n; x0 += 8 * kThreads) {
            uint4 v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int x = x0 + i * kThreads + tid;
                const int r = min(x / seg_row, kBlockM - 1), sg = x - r * seg_row;
                const int src = x < n ? s_src[r] : -1;
                v[i] = load16(ra, src >= 0 ? (uint32_t)src * (uint32_t)K * 2u + (uint32_t)sg * 16u
                                           : kOutOfRange, 0);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int x = x0 + i * kThreads + tid;
                const int r = min(x / seg_row, kBlockM - 1), sg = x - r * seg_row;
                if (x < n)
                    lds_a[r * a_pitch + sg] = v[i];
            }
        }
        __syncthreads();
        auto run = [&](auto nms_tag) {
            // all loads were issued before this point, so skipping the groups
            // past NG cannot change the wait counts
#pragma unroll
            for (int gi = 0; gi < D; ++gi)
                if (gi < NG)
                    group(gi, lds_a, a_pitch, gi * (G / 8), gi, nms_tag);
        };
        if (valid > 16)
            run(std::integral_constant<int, 2>{});
        else
            run(std::integral_constant<int, 1>{});
    } else {
        const int NC = (K + kChunkK - 1) / kChunkK;
        static_assert(kThreads % kChunkSeg == 0, "a thread keeps one 16-byte column of a chunk");
        constexpr int kRowStep = kThreads / kChunkSeg;
        const int aseg = tid % kChunkSeg;         // this thread's 16-byte column of a chunk
        const int arow0 = tid / kChunkSeg;        // and its rows arow0 + i * kRowStep
        uint4 xr[kChunkLoads];
        auto load_chunk = [&](int c) {            // rows past `valid` and K past the end read 0
            const bool in_k = c * kChunkK + aseg * 8 < K;
            const uint32_t col = (uint32_t)(c * kChunkK + aseg * 8) * 2u;
#pragma unroll
            for (int i = 0; i < kChunkLoads; ++i) {
                const int src = s_src[arow0 + i * kRowStep];
                xr[i] = load16(ra, in_k && src >= 0 ? (uint32_t)src * (uint32_t)K * 2u + col
                                                    : kOutOfRange, 0);
            }
        };
        auto store_chunk = [&](int buf) {
#pragma unroll
            for (int i = 0; i < kChunkLoads; ++i)
                lds_a[buf * kBlockM * kChunkPitch + (arow0 + i * kRowStep) * kChunkPitch + aseg] =
                    GATED ? permute8(xr[i]) : xr[i];
        };
        load_chunk(0);
        store_chunk(0);                           // read only after the loop's first barrier
        // TRIP chunks per trip and no branch inside a trip (chunks past the
        // end read activations as zero and their groups have scale 0), so the
        // wait counts the compiler derives stay exact. Per chunk: load the
        // next activation chunk into registers, one barrier (this chunk is in
        // LDS, the other buffer is free), the chunk's groups each followed by
        // the prefetch of the group kAhead chunks ahead, then store the next
        // chunk.
        auto run = [&](auto nms_tag) {
            for (int c0 = 0; c0 < NC; c0 += TRIP) {
#pragma unroll
                for (int j = 0; j < TRIP; ++j) {
                    const int c = c0 + j;
                    load_chunk(c + 1);
                    __builtin_amdgcn_sched_barrier(0);
                    __syncthreads();
                    const uint4 *abuf = lds_a + (j & 1) * kBlockM * kChunkPitch;
#pragma unroll
                    for (int cs = 0; cs < CG; ++cs) {
                        const int gi = c * CG + cs;
                        group((j * CG + cs) % D, abuf, kChunkPitch, cs * (G / 8), gi, nms_tag);
                        prefetch((j * CG + cs) % D, gi + D);
                    }
                    store_chunk((j & 1) ^ 1);
                }
            }
        };
        if (valid > 16)
            run(std::integral_constant<int, 2>{});
        else
            run(std::integral_constant<int, 1>{});
    }

    if (!wave_live)
        return;
    // ---- epilogue. MFMA 16x16 output: lane holds rows 4*(lane/16)+i, column lane%16.
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = ms * 16 + quarter * 4 + i;
            if (r >= valid)
                continue;
            if constexpr (GATED) {
                uint16_t *H = static_cast<uint16_t *>(p.out);
#pragma unroll
                for (int pp = 0; pp < TPW / 2; ++pp) {
                    const int col = col_first + pp * 16 + lrow;
                    const float h = gelu_tanh(acc[2 * pp][ms][i]) * acc[2 * pp + 1][ms][i];
                    H[(size_t)(row0 + r) * p.n_out + permuted_col(col)] =
                        __builtin_bit_cast(uint16_t, (_Float16)h);
                }
            } else {
                const int f = p.sorted_ids[row0 + r];
                float *Y = static_cast<float *>(p.out);
#pragma unroll
                for (int tt = 0; tt < TPW; ++tt)
                    Y[(size_t)f * p.n_out + col_first + tt * 16 + lrow] = acc[tt][ms][i];
            }
        }
    }
}

// Shapes in use. gate_up streams K = d in chunks; down stages its whole
// K = m once when m <= kSingleK and shares it among 8 waves whose register
// budget (4 waves per SIMD) lets two workgroups share a CU.
using GateUpShape = Shape<4, 4, 128, 2, 2>;
using DownSingleShape = Shape<8, 2, 0, 0, 4>;
using DownChunkShape = Shape<4, 2, 512, 2, 2>;

template <int G, bool GATED, class S>
size_t lds_bytes(int K)
{
    const bool single = S::kChunkK == 0;
    const size_t pitch = single ? (size_t)K / 8 + 1 : (size_t)S::kChunkK / 8 + 1;
    const size_t a = single ? kBlockM * pitch : 2 * kBlockM * pitch;
    const size_t range_rows = (size_t)S::kWaves * S::kTiles * 8;
    return sizeof(uint4) * a + 2 * sizeof(uint16_t) * 2 * range_rows * (size_t)(K / G);
}

template <int G, bool GATED, class S>
hipError_t launch_gemm(const GemmArgs &a, hipStream_t stream)
{
    constexpr int cols_per_wg = S::kWaves * (GATED ? S::kTiles / 2 : S::kTiles) * 16;
    const int nblocks = (a.n_out + cols_per_wg - 1) / cols_per_wg;
    if (a.max_tiles == 0 || nblocks == 0)
        return hipSuccess;
    const size_t lds = lds_bytes<G, GATED, S>(a.K);
    auto kern = moe_gemm_kernel<G, GATED, S>;
    static size_t lds_allowed = 64 * 1024;   // raised once per instantiation when needed
    if (lds > lds_allowed) {
        hipError_t err = hipFuncSetAttribute((const void *)kern,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess)
            return err;
        lds_allowed = lds;
    }
    const int tiles = (a.max_tiles + kXcds - 1) / kXcds * kXcds;
    kern<<<dim3(tiles * nblocks), dim3(S::kWaves * 64), lds, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

size_t gemm_lds_bytes(bool gated, int K, int g)
{
    if (gated)
        return g == 128 ? lds_bytes<128, true, GateUpShape>(K) : lds_bytes<64, true, GateUpShape>(K);
    if (K <= kSingleK)
        return g == 128 ? lds_bytes<128, false, DownSingleShape>(K)
                        : lds_bytes<64, false, DownSingleShape>(K);
    return g == 128 ? lds_bytes<128, false, DownChunkShape>(K)
                    : lds_bytes<64, false, DownChunkShape>(K);
}

hipError_t launch_gate_up(const GemmArgs &a, int g, hipStream_t stream)
{
    return g == 128 ? launch_gemm<128, true, GateUpShape>(a, stream)
                    : launch_gemm<64, true, GateUpShape>(a, stream);
}

hipError_t launch_down(const GemmArgs &a, int g, hipStream_t stream)
{
    if (a.K <= kSingleK)
        return g == 128 ? launch_gemm<128, false, DownSingleShape>(a, stream)
                        : launch_gemm<64, false, DownSingleShape>(a, stream);
    return g == 128 ? launch_gemm<128, false, DownChunkShape>(a, stream)
                    : launch_gemm<64, false, DownChunkShape>(a, stream);
}

}  // namespace dgw4

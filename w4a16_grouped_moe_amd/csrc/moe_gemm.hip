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
// A lane (row = lane % 16, quarter = lane / 16) loads g/8 bytes of one weight
// row per group, so the four quarters cover one group of 16 rows. Weights come
// in either of two layouts of the same bytes (every kernel is instantiated for
// both): the canonical one, where those 16 g/2-byte row pieces are half or
// quarter lines spread over 16 rows, and the tiled one, where they are 8 g
// contiguous bytes. Only the tiled loads cover whole 128-byte lines, which
// lets them bypass the caches (non-temporal): the layer then streams its
// weights about 10% faster. Within a wave the rows' lines are never split with
// another wave (that streams markedly slower).
// Dequantisation builds exact fp16 integers in registers: for a word of
// nibbles n0..n7, (w & 0x000F000F) | 0x64006400 is the fp16 pair (1024 + n0,
// 1024 + n4) and (w & 0x00F000F0) | 0x54005400 is (64 + n1, 64 + n5); the same
// on w >> 8 gives n2/n6 and n3/n7, and one packed fp16 subtract of (1024 + z)
// or (64 + z) leaves q - z exactly. The MFMA operand therefore holds K in the
// order [0,4,1,5,2,6,3,7] per 8; the activations are used in the same order
// (gate_up permutes x as it stages it, H is written permuted), which leaves
// the contraction unchanged; the nibble order inside a byte never changes.
// v_mfma_f32_16x16x32_f16 accumulates one group into a fresh fp32 partial and
// the group's scale is applied once per output in fp32 (acc += s * partial),
// so no weight is ever rounded by its scale.
//
// Loads complete in issue order and the compiler's wait counting is exact only
// in straight-line code, so every K loop is fully unrolled for the layer's
// shapes and every wait is for data issued a fixed number of steps earlier.
// Empty asm statements pin each group's accumulation in place (otherwise the
// compiler sinks the multiply-adds to the epilogue and keeps every partial
// live) and make LDS offsets opaque per step or group (otherwise later reads
// are hoisted and held in registers).
//
// Activation rows re-read from L2 share each CU's vector-memory path with the
// weight stream and measurably lower it, so the layer's shape (d = 2816,
// m = 704, gate_up g = 128, down g = 64) runs as one launch of 11-wave
// workgroups, one per CU, 2 per 32-row tile (256 for the 128 tiles of a
// 256-token canvas), each for one half h of H's 704 columns:
//   alignment: each workgroup finds its tile's expert and rows from the
//     expert ids itself (histogram, fixed-order scan, stable ranks in LDS);
//   gate_up4: H[:, 352 h .. + 352] of the tile; wave w owns pairs 2w and
//     2w + 1 (16 gate columns and the matching up columns each) and walks K
//     in 22 straight-line steps of one group of 128 for all four of its
//     weight tiles. The step's activation slice is staged in LDS once for the
//     11 waves; H stays in LDS;
//   down, split along K: the workgroup's H half times the matching half of
//     every down row gives an fp16 partial of all 2816 outputs, stored per
//     assignment; the waves share out the 176 row tiles through an LDS
//     counter; the combine adds the two partials. No workgroup waits for
//     another.
// down4 (workgroup = (tile, 1408 output columns), the tile's H rows and the
// block's scales/zero points staged in LDS once, wave w streaming row tiles
// w, w + 11, ... two ahead) runs as a launch of its own when gate_up has
// another group size.
// Other shapes take the generic kernels:
//   gate_up_kernel: workgroup = (tile, 64 columns), 4 waves, one pair each.
//   down_kernel: workgroup = (tile, 256 columns), 8 waves, two row tiles each,
//     K in chunks of up to 768.
//
// All kernels: tiles past the device-side total exit at once (static grid, no
// host readback); the workgroups of one tile run on one XCD so that its
// activation rows stay in that XCD's L2; tiles with at most 16 valid rows run
// one 16-row MFMA block instead of two.
#include "dgw4.h"
#include "dgw4_internal.hpp"
#include "gemm_common.hpp"

#include <climits>

namespace dgw4 {
namespace {

// ===========================================================================
// gate_up
//
// Workgroup = (32-row tile, 64 output columns), 4 waves; wave w owns pair w
// (16 gate columns and the matching 16 up columns) over all of K. K is
// walked in line steps of 256 (one 128-byte line of every weight row: the
// wave reads whole lines, which streams markedly faster than splitting a
// line between waves). The step's activation slice is staged once in LDS for
// the four waves. A workgroup needs 45 KB of LDS, so three fit on a CU.
constexpr int kGuWaves = 4;
constexpr int kGuThreads = kGuWaves * 64;
constexpr int kGuCols = kGuWaves * 16;   // output columns per workgroup
constexpr int kGuAhead = 3;         // weight line steps in flight per wave
constexpr int kGuSteps = 11;        // line steps of K = 2816, the layer's hidden size
constexpr int kStepSeg = 32;        // 16-byte activation segments per row and step
constexpr int kStepPitch = kStepSeg + 1;   // +16 B per row: 16 rows at one segment hit distinct banks
constexpr int kGuMaxGroups = 64;    // K / G the scale/zero staging covers (4 loads per thread)

template <int G>
constexpr size_t gate_up_lds_bytes_k(int K)
{
    return sizeof(uint4) * 2 * kBlockM * kStepPitch +                  // activation stages
           2 * sizeof(uint16_t) * 2 * kGuCols * (size_t)(K / G);        // scale, zero of 2 x 64 rows
}

// NSC > 0: K = 256 NSC exactly, a compile-time constant, and the K loop is
// fully unrolled; NSC = 0: a generic loop over ceil(K / 256) steps.
// GATED: each wave computes a gate column tile and the matching up tile and
// stores gelu_tanh(gate) * up as H (permuted per 8); otherwise (the dense
// linear) one column tile, stored as fp16 in natural column order.
template <int G, int NMS, int NSC, bool GATED, bool TL>
__device__ __forceinline__ void gate_up_body(const GemmArgs &p, int e, int valid, int row0, int cb,
                                             const int (&fidr)[4])
{
    constexpr int TT = GATED ? 2 : 1;             // weight row tiles per wave
    constexpr int P = kGuAhead;                   // weights P steps ahead
    constexpr int PX = P - 1;                     // activations P - 1 steps ahead (L2 hits)
    constexpr int SG = 256 / G;                   // groups per line step
    constexpr int kWords = G / 32;                // nibble words per lane and group
    constexpr int kRows = NMS * 16;               // activation rows staged
    constexpr int XLD = kRows * kStepSeg / kGuThreads;
    static_assert(kRows * kStepSeg % kGuThreads == 0 && kGuThreads % kStepSeg == 0, "activation split");
    constexpr int TRIP = NSC > 0 ? NSC : 2 * P * PX;   // multiple of P, PX and 2 (LDS stage parity)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
    const int lrow = lane & 15;
    const int quarter = lane >> 4;
    const int K = NSC > 0 ? NSC * 256 : p.K;
    const int NG = K / G;
    const int NS = NSC > 0 ? NSC : (K + 255) / 256;
    const int n_out = p.n_out;
    const size_t wexp = (size_t)e * p.n_w;
    const int col0 = cb * kGuCols;                // first gate column of the workgroup
    const int pcol = col0 + wave * 16;            // first column of this wave's pair
    // a pair past the last column (n_out is a multiple of 16) loads no
    // weights, skips the math and stores nothing; it still stages activations
    const bool live = pcol < n_out;

    extern __shared__ uint4 lds[];
    uint4 *lds_x = lds;                                             // [2][32][kStepPitch]
    uint16_t *lds_s = reinterpret_cast<uint16_t *>(lds + 2 * kBlockM * kStepPitch);   // [2 x 64 rows][NG]
    uint16_t *lds_z = lds_s + 2 * kGuCols * NG;

    // ---- 1. scale/zero loads (gate rows col0.., up rows n_out + col0..),
    // then the activations and weights of the first steps. Loads complete in
    // issue order: the row ids (issued at kernel entry) come first, then
    // scale/zero, then per step the activations before the weights, so that
    // waiting for a step's activations never waits for later weights.
    const uint32_t sz_bytes = (uint32_t)p.n_w * (uint32_t)NG * 2u;
    const rsrc_t rs = make_rsrc(p.s + wexp * (size_t)NG, sz_bytes);
    const rsrc_t rz = make_rsrc(p.z + wexp * (size_t)NG, sz_bytes);
    constexpr int kSzLoads = 4;                   // covers NG <= kGuMaxGroups
    const int range_seg = kGuCols * NG / 8;       // 16-byte segments per 64-row range
    const int sz_total = TT * range_seg;
    auto sz_off = [&](int x) -> uint32_t {
        if (x >= sz_total)
            return kOutOfRange;
        const int r = x >= range_seg;
        return (uint32_t)(((r ? n_out : 0) + col0) * NG) * 2u + (uint32_t)(x - r * range_seg) * 16u;
    };
    uint4 sv[kSzLoads], zv[kSzLoads];
#pragma unroll
    for (int i = 0; i < kSzLoads; ++i) {
        const uint32_t off = sz_off(i * kGuThreads + tid);
        sv[i] = load16(rs, off, 0);
        zv[i] = load16(rz, off, 0);
    }

    const rsrc_t rq = make_rsrc(p.q + wexp * (size_t)(K / 2),
                                live ? (uint32_t)p.n_w * (uint32_t)(K / 2) : 0u);
    // tile 0 = gate rows pcol + lrow, tile 1 = up rows n_out + pcol + lrow
    uint32_t wvoff[TT];
    int lds_row[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        lds_row[tt] = tt * kGuCols + wave * 16 + lrow;
        wvoff[tt] = wq_lane_off<G, TL>((tt ? n_out : 0) + pcol + lrow, lane, K);
    }
    Frag<G> bq[P][TT][SG];
    auto issue_w = [&](int st, int s) {           // step s into register stage st
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int h = 0; h < SG; ++h) {
                const int gi = s * SG + h;
                bq[st][tt][h] = load_frag<G, false>(rq, gi < NG ? wvoff[tt] : kOutOfRange,
                                                 wq_group_off<G, TL>(gi));
            }
    };
    // activation slices: thread -> (rows tid / 32 + 8 i, 16-byte segment
    // tid % 32) of a step; the row's source token comes from its assignment
    // id (a pad entry, id >= A, reads zeros)
    const rsrc_t ra = make_rsrc(p.a_src, (uint32_t)p.a_rows * (uint32_t)K * 2u);
    const int xseg = tid % kStepSeg;
    uint32_t xoff[XLD];
#pragma unroll
    for (int i = 0; i < XLD; ++i)
        xoff[i] = fidr[i] < p.A ? (uint32_t)(fidr[i] / p.topk) * (uint32_t)K * 2u + (uint32_t)xseg * 16u
                                : kOutOfRange;
    uint4 xr[PX][XLD];
    auto issue_x = [&](int st, int s) {           // rows past `valid` and K past the end read 0
        const bool in_k = s * 256 + xseg * 8 < K;
#pragma unroll
        for (int i = 0; i < XLD; ++i)
            xr[st][i] = load16(ra, in_k && xoff[i] != kOutOfRange ? xoff[i] + (uint32_t)s * 512u
                                                                  : kOutOfRange, 0);
    };
    issue_x(0, 0);
    issue_w(0, 0);
#pragma unroll
    for (int s = 1; s < P; ++s) {
        if (s < PX)
            issue_x(s, s);
        issue_w(s, s);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- 2. scale/zero into LDS (made visible by the first step's barrier)
    {
        uint4 *ls = reinterpret_cast<uint4 *>(lds_s);
        uint4 *lz = reinterpret_cast<uint4 *>(lds_z);
#pragma unroll
        for (int i = 0; i < kSzLoads; ++i) {
            const int x = i * kGuThreads + tid;
            if (x < sz_total) {
                ls[x] = sv[i];
                lz[x] = zv[i];
            }
        }
    }

    f32x4 acc[TT][NMS];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int ms = 0; ms < NMS; ++ms)
            acc[tt][ms] = f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    // ---- 3. K loop, one line step per iteration: the step's activations
    // into LDS (reordered per 8), one barrier (everyone is done with the step
    // two back, whose buffer this one reuses), the step's groups, then the
    // activations PX steps ahead and the weights P steps ahead. Steps past
    // the end read zeros and their groups have scale 0.
    for (int s0 = 0; s0 < NS; s0 += TRIP) {
#pragma unroll
        for (int j = 0; j < TRIP; ++j) {
            const int s = s0 + j;
            const int st = j % P;
            uint4 *xb = lds_x + (j & 1) * kBlockM * kStepPitch;
#pragma unroll
            for (int i = 0; i < XLD; ++i)
                xb[((i * kGuThreads + tid) / kStepSeg) * kStepPitch + xseg] = permute8(xr[j % PX][i]);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            if (live) {
#pragma unroll
                for (int h = 0; h < SG; ++h) {
                    const int gi = s * SG + h;
                    const int gc = min(gi, NG - 1);
                    float scale[TT];
                    f16x2 c1024[TT], c64[TT];
#pragma unroll
                    for (int tt = 0; tt < TT; ++tt) {
                        zero_point_consts(lds_z[lds_row[tt] * NG + gc], c1024[tt], c64[tt]);
                        const float sc = (float)__builtin_bit_cast(_Float16, lds_s[lds_row[tt] * NG + gc]);
                        scale[tt] = gi < NG ? sc : 0.0f;
                    }
                    f32x4 part[TT][NMS];
#pragma unroll
                    for (int t = 0; t < kWords; ++t) {
                        f16x8 bop[TT];
#pragma unroll
                        for (int tt = 0; tt < TT; ++tt)
                            bop[tt] = dequant8(frag_word<G>(bq[st][tt][h], t), c1024[tt], c64[tt]);
                        const int seg = h * (G / 8) + quarter * (G / 32) + t;   // this lane's 8 K positions
#pragma unroll
                        for (int ms = 0; ms < NMS; ++ms) {
                            const f16x8 aop = __builtin_bit_cast(f16x8, xb[(ms * 16 + lrow) * kStepPitch + seg]);
#pragma unroll
                            for (int tt = 0; tt < TT; ++tt)
                                part[tt][ms] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                    aop, bop[tt], t == 0 ? zero4 : part[tt][ms], 0, 0, 0);
                        }
                    }
#pragma unroll
                    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                        for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                acc[tt][ms][i] += scale[tt] * part[tt][ms][i];
                }
            }
            issue_x(j % PX, s + PX);
            issue_w(st, s + P);
        }
    }

    // ---- 4. epilogue: H = gelu_tanh(gate) * up in fp16 at the tile's padded
    // row, permuted per 8 columns (or, ungated, the fp16 output in natural
    // column order). MFMA 16x16 output: lane holds rows 4 * quarter + i,
    // column lrow.
    if (!live)
        return;
    uint16_t *H = static_cast<uint16_t *>(p.out);
    const int col = pcol + lrow;
#pragma unroll
    for (int ms = 0; ms < NMS; ++ms) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = ms * 16 + quarter * 4 + i;
            if (r >= valid)
                continue;
            if constexpr (GATED) {
                const float h = gelu_tanh(acc[0][ms][i]) * acc[TT - 1][ms][i];
                H[(size_t)(row0 + r) * n_out + permuted_col(col)] = __builtin_bit_cast(uint16_t, (_Float16)h);
            } else {
                H[(size_t)(row0 + r) * n_out + col] = __builtin_bit_cast(uint16_t, (_Float16)acc[0][ms][i]);
            }
        }
    }
}

template <int G, bool TL>
__global__ void __launch_bounds__(kGuThreads)
__attribute__((amdgpu_waves_per_eu(3))) gate_up_kernel(GemmArgs p)
{
    // workgroup -> (column block, tile), XCD-aware: consecutive workgroups go
    // to the XCDs in turn, so XCD x takes tiles x, x + 8, ... and runs all
    // column blocks of a tile back to back, its activation rows staying in L2
    const int nblocks = (p.n_out + kGuCols - 1) / kGuCols;
    const int xcd = (int)blockIdx.x % kXcds, slot = (int)blockIdx.x / kXcds;
    const int cb = slot % nblocks;
    const int tile = slot / nblocks * kXcds + xcd;
    if (tile >= p.max_tiles)
        return;
    // the assignment ids of the thread's activation rows (rows tid / 32 and
    // tid / 32 + 8 of each 16-row block) go out together with the tile
    // descriptor, so the activation loads need no further round trip
    const int r0 = (int)threadIdx.x / kStepSeg;
    int fidr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)                   // < cap: always in the buffer
        fidr[i] = p.sorted_ids[tile * kBlockM + r0 + i * (kGuThreads / kStepSeg)];
    const int2 info = p.tile_info[tile];           // {expert, valid rows | tiles << 16}; -1 past the total
    if (info.x < 0)
        return;
    const int valid = tile_valid(info.y);
    if (p.K == kGuSteps * 256) {
        if (valid > 16)
            gate_up_body<G, 2, kGuSteps, true, TL>(p, info.x, valid, tile * kBlockM, cb, fidr);
        else
            gate_up_body<G, 1, kGuSteps, true, TL>(p, info.x, valid, tile * kBlockM, cb, fidr);
    } else {
        if (valid > 16)
            gate_up_body<G, 2, 0, true, TL>(p, info.x, valid, tile * kBlockM, cb, fidr);
        else
            gate_up_body<G, 1, 0, true, TL>(p, info.x, valid, tile * kBlockM, cb, fidr);
    }
}

// Dense W4A16 linear, y = x * deq(W)^T: the ungated body over the rows of x in
// order (32-row tiles, the last one ragged), one weight matrix, no alignment.
// Workgroup -> (column block, row tile), weight-sharing order: XCD x takes
// column blocks x, x + 8, ... and runs all row tiles of a block back to back,
// so the block's weights stream from HBM once and the other row tiles read
// them from that XCD's L2 (x, at most a few MB, stays in every L2).
template <int G, bool TL>
__global__ void __launch_bounds__(kGuThreads)
__attribute__((amdgpu_waves_per_eu(3))) linear_kernel(GemmArgs p)
{
    const int nblocks = (p.n_out + kGuCols - 1) / kGuCols;
    const int xcd = (int)blockIdx.x % kXcds, slot = (int)blockIdx.x / kXcds;
    const int tile = slot % p.max_tiles;
    const int cb = slot / p.max_tiles * kXcds + xcd;
    if (cb >= nblocks)
        return;
    const int r0 = (int)threadIdx.x / kStepSeg;
    int fidr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {                 // rows past the end read zeros
        const int r = tile * kBlockM + r0 + i * (kGuThreads / kStepSeg);
        fidr[i] = r < p.A ? r : p.A;
    }
    const int valid = min(kBlockM, p.A - tile * kBlockM);
    if (p.K == kGuSteps * 256) {
        if (valid > 16)
            gate_up_body<G, 2, kGuSteps, false, TL>(p, 0, valid, tile * kBlockM, cb, fidr);
        else
            gate_up_body<G, 1, kGuSteps, false, TL>(p, 0, valid, tile * kBlockM, cb, fidr);
    } else {
        if (valid > 16)
            gate_up_body<G, 2, 0, false, TL>(p, 0, valid, tile * kBlockM, cb, fidr);
        else
            gate_up_body<G, 1, 0, false, TL>(p, 0, valid, tile * kBlockM, cb, fidr);
    }
}

// ===========================================================================
// down
//
// Workgroup = (32-row tile, 256 output columns = 16 weight row tiles), 8
// waves; wave w owns row tiles w and w + 8 of the block. The tile's
// activations (all of K, already in the permuted K order) and the block's
// scales/zero points (transposed to [group][row]) are staged in LDS once;
// each wave then streams its two weight tiles, K in chunks of CH groups,
// with both tiles' loads in flight from the start. The MFMA takes the
// weights as its row operand, so a lane ends with four consecutive output
// columns of one assignment row: one 16-byte fp32 store per row and tile, at
// the assignment's flat slot t * topk + k, issued after the last chunk.
constexpr int kDnWaves = 8;
constexpr int kDnThreads = kDnWaves * 64;
constexpr int kDnTilesPerWave = 2;
constexpr int kDnRows = kDnWaves * kDnTilesPerWave * 16;   // weight rows (output columns) per block
constexpr int kDnAhead = 2;         // (tile, chunk) units in flight per wave
constexpr int kDnGroups = 11;       // K / 64 of the layer's down projection (m = 704)
constexpr int kALoads = 6;          // activation segments per thread and batch

template <int G>
size_t down_lds_bytes_k(int K)
{
    return sizeof(uint4) * kBlockM * ((size_t)K / 8 + 1) +
           2 * sizeof(uint16_t) * kDnRows * (size_t)(K / G);
}

// Byte offset of 16-byte activation segment x of the tile's 32 rows (all of
// K), or an out-of-range offset past them.
__device__ inline uint32_t down_a_off(const GemmArgs &p, int row0, int x)
{
    const int seg_row = p.K / 8;
    const int r = x / seg_row, sg = x - r * seg_row;
    return x < kBlockM * seg_row ? (uint32_t)(row0 + r) * (uint32_t)p.K * 2u + (uint32_t)sg * 16u
                                 : kOutOfRange;
}

// CH: groups per K chunk; NCH: chunks per weight tile (both compile-time).
// EXACT: K = CH * NCH * G exactly (a compile-time constant); otherwise groups
// past K / G (a rounded-up chunk) read no weights and have scale 0.
template <int G, int NMS, int CH, int NCH, bool EXACT, bool TL>
__device__ __forceinline__ void down_body(const GemmArgs &p, int e, int valid, int row0, int cb,
                                          const uint4 (&av)[kALoads], int fid)
{
    constexpr int P = kDnAhead;
    constexpr int NU = kDnTilesPerWave * NCH;   // units (tile j, chunk c), j-major
    constexpr int kWords = G / 32;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lrow = lane & 15;
    const int quarter = lane >> 4;
    const int K = EXACT ? CH * NCH * G : p.K;
    const int NG = K / G;
    const int n_out = p.n_out;
    const size_t wexp = (size_t)e * p.n_w;
    const int rt0 = cb * (kDnRows / 16);          // first weight row tile of the block
    const int nrt = min(kDnRows / 16, n_out / 16 - rt0);
    const int a_pitch = K / 8 + 1;                // uint4 per activation row

    extern __shared__ uint4 lds[];
    uint4 *lds_a = lds;                                             // [32][a_pitch]
    uint16_t *lds_s = reinterpret_cast<uint16_t *>(lds + kBlockM * a_pitch);   // [NG][kDnRows]
    uint16_t *lds_z = lds_s + kDnRows * NG;
    __shared__ int s_dst[kBlockM];

    // ---- 1. scale/zero of the block's rows (one contiguous range each),
    // then the first weight units of this wave. The activation rows and row
    // ids were issued at kernel entry, so they land first.
    const rsrc_t rs = make_rsrc(p.s + wexp * (size_t)NG, (uint32_t)p.n_w * (uint32_t)NG * 2u);
    const rsrc_t rz = make_rsrc(p.z + wexp * (size_t)NG, (uint32_t)p.n_w * (uint32_t)NG * 2u);
    const int sz_seg = (nrt * 16 * NG * 2 + 15) / 16;             // 16-byte segments per array
    const uint32_t sz_base = (uint32_t)(rt0 * 16 * NG) * 2u;
    constexpr int kSzLoads = 2;                   // 256 rows x NG <= 24 groups
    static_assert(kDnRows * NCH * CH * 2 <= kSzLoads * kDnThreads * 16, "scale/zero loads");
    uint4 sv[kSzLoads], zv[kSzLoads];
#pragma unroll
    for (int i = 0; i < kSzLoads; ++i) {
        const int x = i * kDnThreads + tid;
        const uint32_t off = x < sz_seg ? sz_base + (uint32_t)x * 16u : kOutOfRange;
        sv[i] = load16(rs, off, 0);
        zv[i] = load16(rz, off, 0);
    }
    // activation rows row0 .. row0 + 16 NMS (staged whatever their content: a
    // row past `valid` only feeds output rows that are never stored)
    const rsrc_t ra = make_rsrc(p.a_src, (uint32_t)p.a_rows * (uint32_t)K * 2u);
    const int seg_row = K / 8;
    const int a_total = 16 * NMS * seg_row;
    auto a_put = [&](int x, uint4 v) {
        const int r = min(x / seg_row, 16 * NMS - 1), sg = x - r * seg_row;
        if (x < a_total)
            lds_a[r * a_pitch + sg] = v;
    };

    const rsrc_t rq = make_rsrc(p.q + wexp * (size_t)(K / 2), (uint32_t)p.n_w * (uint32_t)(K / 2));
    auto tile_live = [&](int j) { return wave + j * kDnWaves < nrt; };
    auto tile_row = [&](int j) { return (rt0 + wave + j * kDnWaves) * 16; };   // first weight row
    Frag<G> bq[P][CH];
    auto issue_w = [&](int st, int u) {
        const int j = u / NCH, c = u % NCH;
        const uint32_t voff = u < NU && tile_live(j) ? wq_lane_off<G, TL>(tile_row(j) + lrow, lane, K)
                                                     : kOutOfRange;
#pragma unroll
        for (int g = 0; g < CH; ++g) {
            const int gi = c * CH + g;
            bq[st][g] = load_frag<G, false>(rq, gi < NG ? voff : kOutOfRange, wq_group_off<G, TL>(gi));
        }
    };

    // ---- 2. activations, scale/zero (transposed) and row destinations into
    // LDS. With one chunk (K <= 768) the activations fit one batch and the
    // weights are issued right behind them; a longer K stages its
    // activations in several batches first (the choice is compile-time, so
    // every wait below counts only the loads it needs).
    static_assert(NCH > 1 || 16 * 2 * (CH * G) / 8 <= kALoads * kDnThreads, "one activation batch");
    uint4 avb[kALoads];
    if constexpr (NCH == 1) {
#pragma unroll
        for (int u = 0; u < P; ++u)
            issue_w(u, u);
    }
#pragma unroll
    for (int i = 0; i < kALoads; ++i)
        a_put(i * kDnThreads + tid, av[i]);
    if constexpr (NCH > 1) {
        for (int x0 = kALoads * kDnThreads; x0 < a_total; x0 += kALoads * kDnThreads) {
#pragma unroll
            for (int i = 0; i < kALoads; ++i)
                avb[i] = load16(ra, down_a_off(p, row0, x0 + i * kDnThreads + tid), 0);
#pragma unroll
            for (int i = 0; i < kALoads; ++i)
                a_put(x0 + i * kDnThreads + tid, avb[i]);
        }
    }
    {
        // element x of the block's [rows][NG] range -> lds [g][row]
        auto put8 = [&](uint16_t *dst, int x, uint4 v) {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int el = x * 8 + k;
                const int r = el / NG, g = el - r * NG;
                if (r < nrt * 16)
                    dst[g * kDnRows + r] = (uint16_t)(w[k >> 1] >> (16 * (k & 1)));
            }
        };
#pragma unroll
        for (int i = 0; i < kSzLoads; ++i) {
            const int x = i * kDnThreads + tid;
            if (x < sz_seg) {
                put8(lds_s, x, sv[i]);
                put8(lds_z, x, zv[i]);
            }
        }
    }
    if (tid < kBlockM)
        s_dst[tid] = tid < valid ? fid : -1;
    if constexpr (NCH > 1) {
#pragma unroll
        for (int u = 0; u < P; ++u)
            issue_w(u, u);
    }
    __syncthreads();

    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    // the MFMAs take the weights as the row operand: a lane ends with four
    // consecutive output columns (weight rows 4 * quarter + i) of assignment
    // row lrow (+16 for the second block)
    int dst[NMS];
#pragma unroll
    for (int ms = 0; ms < NMS; ++ms)
        dst[ms] = s_dst[ms * 16 + lrow];
    f32x4 out[kDnTilesPerWave][NMS];
#pragma unroll
    for (int j = 0; j < kDnTilesPerWave; ++j)
#pragma unroll
        for (int ms = 0; ms < NMS; ++ms)
            out[j][ms] = zero4;

    // ---- 3. stream this wave's units, as straight-line code
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int st = u % P;
        const int j = u / NCH, c = u % NCH;
        // the activation reads are the same for every tile: an opaque offset
        // keeps the compiler from holding all of them in registers
        int aoff = 0;
        asm volatile("" : "+v"(aoff));
        const int srow = min(tile_row(j) - rt0 * 16, max(0, nrt * 16 - 16));   // first row in lds_s/lds_z
#pragma unroll
        for (int g = 0; g < CH; ++g) {
            const int gi = c * CH + g;
            const int gc = min(gi, NG - 1);
            f16x2 c1024, c64;
            zero_point_consts(lds_z[gc * kDnRows + srow + lrow], c1024, c64);
            const uint2 s4 = *reinterpret_cast<const uint2 *>(lds_s + gc * kDnRows + srow + quarter * 4);
            float sc[4];
            sc[0] = (float)__builtin_bit_cast(_Float16, (uint16_t)s4.x);
            sc[1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(s4.x >> 16));
            sc[2] = (float)__builtin_bit_cast(_Float16, (uint16_t)s4.y);
            sc[3] = (float)__builtin_bit_cast(_Float16, (uint16_t)(s4.y >> 16));
            if (gi >= NG) {                       // a masked group of a rounded-up chunk
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sc[i] = 0.0f;
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
            // unit's multiply-adds to the stores and keeps all partials live
#pragma unroll
            for (int ms = 0; ms < NMS; ++ms)
                asm volatile("" : "+v"(out[j][ms]));
        }
        issue_w(st, u + P);
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- 4. outputs: fp16 Y at each assignment's flat slot, one 8-byte
    // store per assignment row and tile
    uint16_t *Y = static_cast<uint16_t *>(p.out);
#pragma unroll
    for (int j = 0; j < kDnTilesPerWave; ++j) {
        if (!tile_live(j))
            continue;
        const int col = tile_row(j) + quarter * 4;
#pragma unroll
        for (int ms = 0; ms < NMS; ++ms)
            if (dst[ms] >= 0)
                *reinterpret_cast<uint2 *>(Y + (size_t)dst[ms] * n_out + col) = pack_f16x4(out[j][ms]);
    }
}

// Kernel entry for one (tile, column block): the tile's activation rows and
// assignment ids are requested before its descriptor is known (they depend
// only on the tile index), then the body for its row count runs.
template <int G, int CH, int NCH, bool EXACT, bool TL>
__device__ __forceinline__ void down_entry(const GemmArgs &p, int tile, int cb)
{
    const int tid = threadIdx.x;
    const rsrc_t ra = make_rsrc(p.a_src, (uint32_t)p.a_rows * (uint32_t)p.K * 2u);
    uint4 av[kALoads];
#pragma unroll
    for (int i = 0; i < kALoads; ++i)
        av[i] = load16(ra, down_a_off(p, tile * kBlockM, i * kDnThreads + tid), 0);
    int fid = 0;
    if (tid < kBlockM)
        fid = p.sorted_ids[tile * kBlockM + tid];
    const int2 info = p.tile_info[tile];           // {expert, valid rows | tiles << 16}; -1 past the total
    if (info.x < 0)
        return;
    const int valid = tile_valid(info.y);
    if (valid > 16)
        down_body<G, 2, CH, NCH, EXACT, TL>(p, info.x, valid, tile * kBlockM, cb, av, fid);
    else
        down_body<G, 1, CH, NCH, EXACT, TL>(p, info.x, valid, tile * kBlockM, cb, av, fid);
}

template <int G, bool TL>
__global__ void __launch_bounds__(kDnThreads)
__attribute__((amdgpu_waves_per_eu(4))) down_kernel(GemmArgs p)
{
    // workgroup -> (column block, tile), XCD-aware as in gate_up
    const int nblocks = (p.n_out / 16 + kDnRows / 16 - 1) / (kDnRows / 16);
    const int xcd = (int)blockIdx.x % kXcds, slot = (int)blockIdx.x / kXcds;
    const int cb = slot % nblocks;
    const int tile = slot / nblocks * kXcds + xcd;
    if (tile >= p.max_tiles)
        return;
    const int ng = p.K / G;
    // the layer's 11 groups of 64 as one chunk; otherwise chunks of 768 K
    // (12 groups of 64 or 6 of 128), one or two of them
    constexpr int kCh = 768 / G;
    if constexpr (G == 64) {
        if (ng == kDnGroups) {
            down_entry<G, kDnGroups, 1, true, TL>(p, tile, cb);
            return;
        }
    }
    if (ng <= kCh)
        down_entry<G, kCh, 1, false, TL>(p, tile, cb);
    else
        down_entry<G, kCh, 2, false, TL>(p, tile, cb);
}

// ===========================================================================
// Layer-shape kernel (d = 2816, m = 704, gate_up g = 128, down g = 64): the
// alignment, gate_up with its activation and down in one launch.
//
// Activation rows re-read from L2 share each CU's vector-memory path with the
// weight stream, so the GEMMs cover wide column blocks per workgroup and the
// launch runs one 11-wave workgroup per CU: 2 per 32-row tile (one per half
// h of H's columns), 256 for the 128 tiles of a T = 256 canvas, a single
// round with one prologue.
//
//   1. alignment, per workgroup and sync-free: every workgroup reads all the
//      expert ids (8 KB at T = 256), builds the expert histogram in LDS,
//      finds by a fixed-order scan of the 32-padded counts which expert owns
//      its tile and ranks that expert's ids (ascending flat index) to find
//      the flat ids of its 32 rows. The result is align_kernel's, with no
//      launch, no global buffers and no host readback.
//   2. gate_up: H[:, 352 h .. 352 h + 352] of the tile's rows, kept in LDS.
//   3. down, split along its contraction: the workgroup multiplies its own
//      half of H (K = 352 of 704) into all 2816 outputs and stores the fp16
//      partial at (h, flat id); the combine adds the two halves. No H crosses
//      CUs and no workgroup waits for another. The split falls inside down's
//      group 5 (K 320 .. 383): both halves take that group, each with the
//      lanes that hold the other half's K idle (no load; their activations
//      are zero in LDS), and each applies the group's scale to its part.

constexpr int kL4Waves = 11;
constexpr int kL4Threads = kL4Waves * 64;
constexpr int kGu4Cols = kL4Waves * 32;          // 352
constexpr int kGu4Ahead = 3;                     // weight steps in flight per wave
constexpr int kGu4Rows = 2 * kGu4Cols;           // gate + up weight rows of a workgroup
constexpr int kGu4Groups = kGuSteps * 2;         // 22 groups of 128

constexpr int kGu4XRows = kBlockM + 1;          // row 32 takes the writes of rows past the tile
constexpr int kGu4SzSeg = (kGu4Rows * kGu4Groups * 2 / 16 + kL4Threads - 1) / kL4Threads * kL4Threads;

// The H tile in LDS: 32 rows of the half's 352 columns placed at column
// 32 h of a 384-column frame (the other 32 columns zero), so that local
// down group j (global group j + 5 h) reads its 64 K at column 64 j for
// either half; rows padded by 16 bytes against bank conflicts.
constexpr int kHCols = 384;
constexpr int kHPitch = kHCols + 8;              // fp16 per LDS row

constexpr size_t layer_gate_up_lds_bytes()
{
    return sizeof(uint4) * 2 * kGu4XRows * kStepPitch + 2 * sizeof(uint4) * kGu4SzSeg;
}

constexpr size_t layer_lds_bytes()
{
    return layer_gate_up_lds_bytes() + sizeof(uint16_t) * kBlockM * kHPitch;
}

// ---- 1. alignment inside the kernel, in two parts: which expert owns the
// tile (a histogram of all ids, then a fixed-order scan of the 32-padded
// counts), and, once its weight loads are in flight, the flat ids of its
// rows (stable ranks of that expert's ids).

constexpr int kSetupPer = 4;                     // ids per thread per chunk
constexpr int kSetupChunk = kL4Threads * kSetupPer;

// Exclusive scan of v over the workgroup's threads in thread order (a fixed
// order); *total gets the sum. Every thread must call it.
__device__ inline int l4_scan_excl(int v, int *s_wsum, int &total)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(x, off, 64);
        if (lane >= off)
            x += u;
    }
    if (lane == 63)
        s_wsum[wave] = x;
    __syncthreads();
    int base = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kL4Waves; ++w) {
        const int s = s_wsum[w];
        base += w < wave ? s : 0;
        total += s;
    }
    __syncthreads();                              // s_wsum is reused by the next scan
    return base + x - v;
}

struct TileSetup {
    int v0[kSetupPer];                            // this thread's ids of the first chunk
    int r0;                                       // the tile's first row within its expert
    int valid;                                    // rows holding assignments
    int tiles;                                    // tiles of the expert
};

__device__ inline void load_ids(const int32_t *__restrict__ ids, int A, int c0, int (&v)[kSetupPer])
{
#pragma unroll
    for (int j = 0; j < kSetupPer; ++j) {
        const int i = c0 + (int)threadIdx.x * kSetupPer + j;
        v[j] = i < A ? ids[i] : -1;
    }
}

// The tile's expert, or -1 when the tile lies past the padded total. Ids
// outside [0, E) are skipped. Also sets every s_rows entry to A (pad).
// The tile of the workgroup in slot tslot of XCD xcd: with n tiles in all,
// XCD x takes tiles x ceil(n / 8) .. + ceil(n / 8) - 1, so that the tiles of
// an expert with several (in expert order, consecutive) run on one XCD at
// the same time and read its weights through one L2; -1 past the last.
__device__ inline int layer_tile_of(int xcd, int tslot, int total_rows)
{
    const int ntiles = total_rows / kBlockM;
    const int per = (ntiles + kXcds - 1) / kXcds;
    return tslot < per ? xcd * per + tslot : -1;
}

__device__ int layer_tile_find(const int32_t *__restrict__ ids, int A, int E, int xcd, int tslot,
                               TileSetup &ts, int *s_cnt, int *s_wsum, int *s_rows, int *s_info)
{
    const int tid = threadIdx.x;
    for (int x = tid; x < E; x += kL4Threads)
        s_cnt[x] = 0;
    if (tid < kBlockM)
        s_rows[tid] = A;
    if (tid == 0)
        s_info[0] = -1;
    load_ids(ids, A, 0, ts.v0);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSetupPer; ++j)
        if (ts.v0[j] >= 0 && ts.v0[j] < E)
            atomicAdd(&s_cnt[ts.v0[j]], 1);
    for (int c0 = kSetupChunk; c0 < A; c0 += kSetupChunk) {
        int v[kSetupPer];
        load_ids(ids, A, c0, v);
#pragma unroll
        for (int j = 0; j < kSetupPer; ++j)
            if (v[j] >= 0 && v[j] < E)
                atomicAdd(&s_cnt[v[j]], 1);
    }
    __syncthreads();
    // padded offsets in expert order, all in wave 0 (E <= kL4Threads, see
    // layer_fused: kEPer consecutive experts per lane, then a wave scan, so
    // one barrier publishes the result); the tile follows from the total
    // (see layer_tile_of), and the lane whose expert's rows hold the tile's
    // first row records it
    if (tid < 64) {
        constexpr int kEPer = (kL4Threads + 63) / 64;
        int c[kEPer], sum = 0;
#pragma unroll
        for (int j = 0; j < kEPer; ++j) {
            const int x = tid * kEPer + j;
            c[j] = x < E ? s_cnt[x] : 0;
            sum += (c[j] + kBlockM - 1) / kBlockM * kBlockM;
        }
        int incl = sum;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int u = __shfl_up(incl, d, 64);
            if (tid >= d)
                incl += u;
        }
        const int total = __shfl(incl, 63, 64);
        const int tile = layer_tile_of(xcd, tslot, total);
        const int row = tile < 0 ? INT_MAX : tile * kBlockM;
        int off = incl - sum;
#pragma unroll
        for (int j = 0; j < kEPer; ++j) {
            const int padded = (c[j] + kBlockM - 1) / kBlockM * kBlockM;
            if (off <= row && row < off + padded) {
                s_info[0] = tid * kEPer + j;
                s_info[1] = row - off;                 // the tile's first rank within the expert
                s_info[2] = c[j];
                s_info[3] = padded / kBlockM;
            }
            off += padded;
        }
    }
    __syncthreads();
    // uniform over the workgroup: scalar registers
    const int e = __builtin_amdgcn_readfirstlane(s_info[0]);
    if (e >= 0) {
        ts.r0 = __builtin_amdgcn_readfirstlane(s_info[1]);
        ts.valid = __builtin_amdgcn_readfirstlane(min(kBlockM, s_info[2] - ts.r0));
        ts.tiles = __builtin_amdgcn_readfirstlane(s_info[3]);
    }
    return e;
}

// s_rows[r] = the flat id of the tile's row r: the (r0 + r)-th of expert e's
// ids in ascending flat index. Thread t holds ids c0 + 4 t .. c0 + 4 t + 3
// of each chunk, so thread order is index order.
__device__ void layer_tile_rows(const int32_t *__restrict__ ids, int A, int e, const TileSetup &ts,
                                int *s_wsum, int *s_rows)
{
    const int tid = threadIdx.x;
    int run = 0;
    for (int c0 = 0; c0 < A && run < ts.r0 + kBlockM; c0 += kSetupChunk) {
        int v[kSetupPer];
        if (c0 == 0) {
#pragma unroll
            for (int j = 0; j < kSetupPer; ++j)
                v[j] = ts.v0[j];
        } else {
            load_ids(ids, A, c0, v);
        }
        int mine = 0;
#pragma unroll
        for (int j = 0; j < kSetupPer; ++j)
            mine += v[j] == e;
        int total;
        int rank = run + l4_scan_excl(mine, s_wsum, total);
#pragma unroll
        for (int j = 0; j < kSetupPer; ++j) {
            if (v[j] == e) {
                const int r = rank - ts.r0;
                if (r >= 0 && r < kBlockM)
                    s_rows[r] = c0 + tid * kSetupPer + j;
                ++rank;
            }
        }
        run += total;
    }
    __syncthreads();
}

// ---- 2. gate_up: workgroup = (tile, 352 output columns); wave w owns pairs
// 2w and 2w + 1 (columns col0 + 32 w .. + 32: 16 gate columns and the
// matching 16 up columns each, four weight row tiles) and computes both in
// one pass over K, one group of 128 per step: 22 steps, straight-line, each
// loading 16 bytes per lane of each of the four tiles (4 KB per wave), the
// weights P steps and the activations P - 1 steps ahead. Each step's
// activation slice (the tile's rows, 256 bytes each) is staged in LDS once
// for the 11 waves, so every activation byte is read once per workgroup.
// H = gelu_tanh(gate) * up goes to the LDS frame (see kHPitch). rows() ranks
// the tile's rows into s_rows once the first weight loads are out; after_k
// runs once the last step's weights are consumed, before the epilogue: the
// down phase issues its first loads there.
constexpr int kGu4Seg = 16;                      // 16-byte activation segments per row and step
constexpr int kGu4Pitch = kGu4Seg + 1;           // +16 B per row against bank conflicts

template <int NMS, bool TL, bool NT, class Rows, class AfterK>
__device__ __forceinline__ void gate_up4_body(const GemmArgs &p, int e, int cb, Rows &&rows,
                                              const int *s_rows, AfterK &&after_k)
{
    constexpr int G = 128;
    constexpr int P = 3;                           // weight steps in flight
    constexpr int PX = 2;                          // activation stages, issued P - 1 steps ahead
    constexpr int kWords = 4;
    constexpr int NG = kGu4Groups;                 // 22 steps, one group each
    constexpr int K = kGuSteps * 256;
    constexpr int NT4 = 4;                         // weight row tiles per wave: gate 0, up 0, gate 1, up 1
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lrow = lane & 15;
    const int quarter = lane >> 4;
    const int n_out = p.n_out;
    const size_t wexp = (size_t)e * p.n_w;
    const int col0 = cb * kGu4Cols;

    extern __shared__ uint4 lds[];
    uint4 *lds_x = lds;                                             // [2][33][kGu4Pitch]
    uint16_t *lds_s = reinterpret_cast<uint16_t *>(lds + 2 * kGu4XRows * kStepPitch);   // [704 rows][NG]
    uint16_t *lds_z = lds_s + kGu4SzSeg * 8;
    uint16_t *lds_h = reinterpret_cast<uint16_t *>(reinterpret_cast<char *>(lds) + layer_gate_up_lds_bytes());
    static_assert(kGu4Pitch <= kStepPitch, "activation stage fits its area");

    // ---- 1. scale/zero of the 352 gate and 352 up rows, the weights of the
    // first steps, then (once the rows are known) the activations
    const uint32_t sz_bytes = (uint32_t)p.n_w * (uint32_t)NG * 2u;
    const rsrc_t rs = make_rsrc(p.s + wexp * (size_t)NG, sz_bytes);
    const rsrc_t rz = make_rsrc(p.z + wexp * (size_t)NG, sz_bytes);
    constexpr int kRangeSeg = kGu4Cols * NG / 8;   // 968 segments per 352-row range
    constexpr int kSzLoads = (2 * kRangeSeg + kL4Threads - 1) / kL4Threads;   // 3
    auto sz_off = [&](int x) -> uint32_t {
        if (x >= 2 * kRangeSeg)
            return kOutOfRange;
        const int r = x >= kRangeSeg;
        return (uint32_t)(((r ? n_out : 0) + col0) * NG) * 2u + (uint32_t)(x - r * kRangeSeg) * 16u;
    };
    uint4 sv[kSzLoads], zv[kSzLoads];
#pragma unroll
    for (int i = 0; i < kSzLoads; ++i) {
        const uint32_t off = sz_off(i * kL4Threads + tid);
        sv[i] = load16(rs, off, 0);
        zv[i] = load16(rz, off, 0);
    }

    const rsrc_t rq = make_rsrc(p.q + wexp * (size_t)(K / 2), (uint32_t)p.n_w * (uint32_t)(K / 2));
    // tile u: pair c = u / 2 (columns col0 + 32 wave + 16 c ..), gate (u even) or up
    auto in_range = [&](int c) { return wave * 32 + c * 16 + lrow; };
    auto sz_row = [&](int u) { return (u & 1) * kGu4Cols + in_range(u >> 1); };   // row in lds_s/lds_z
    uint32_t wvoff[NT4];
#pragma unroll
    for (int u = 0; u < NT4; ++u)
        wvoff[u] = wq_lane_off<G, TL>(((u & 1) ? n_out : 0) + col0 + in_range(u >> 1), lane, K);
    Frag<G> bq[P][NT4];
    auto issue_w = [&](int st, int s) {
#pragma unroll
        for (int u = 0; u < NT4; ++u)
            bq[st][u] = load_frag<G, NT>(rq, wvoff[u], wq_group_off<G, TL>(s));
    };
#pragma unroll
    for (int s = 0; s < P; ++s)
        issue_w(s, s);
    __builtin_amdgcn_sched_barrier(0);
    rows();
    // activation slices: thread -> (row tid / 16, 16-byte segment tid % 16)
    // of a step; rows past 16 NMS, pad rows and threads past row 32 read
    // nothing
    const rsrc_t ra = make_rsrc(p.a_src, (uint32_t)p.a_rows * (uint32_t)K * 2u);
    const int xseg = tid % kGu4Seg;
    const int xrow = tid / kGu4Seg;
    const int xfid = s_rows[min(xrow, kBlockM - 1)];
    const uint32_t xoff = xrow < NMS * 16 && xfid < p.A
                              ? (uint32_t)(xfid / p.topk) * (uint32_t)K * 2u + (uint32_t)xseg * 16u
                              : kOutOfRange;
    uint4 xr[PX];
    auto issue_x = [&](int st, int s) {
        xr[st] = load16(ra, xoff != kOutOfRange ? xoff + (uint32_t)s * 256u : kOutOfRange, 0);
    };
    // prologue: w(0) w(1) w(2) (above), x(0) x(1); in step s: x(s + PX) then
    // w(s + P), so waiting for a step's activations never waits for later
    // weights
#pragma unroll
    for (int s = 0; s < PX; ++s)
        issue_x(s, s);
    __builtin_amdgcn_sched_barrier(0);

    // ---- 2. scale/zero into LDS (made visible by the first step's barrier;
    // the segments past the rows land in the area's rounded-up tail)
    {
        uint4 *ls = reinterpret_cast<uint4 *>(lds_s);
        uint4 *lz = reinterpret_cast<uint4 *>(lds_z);
        static_assert(kSzLoads * kL4Threads == kGu4SzSeg, "scale/zero area");
#pragma unroll
        for (int i = 0; i < kSzLoads; ++i) {
            ls[i * kL4Threads + tid] = sv[i];
            lz[i * kL4Threads + tid] = zv[i];
        }
    }
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc[NT4][NMS];
#pragma unroll
    for (int u = 0; u < NT4; ++u)
#pragma unroll
        for (int ms = 0; ms < NMS; ++ms)
            acc[u][ms] = zero4;

    // ---- 3. 22 steps of one group, straight-line
#pragma unroll
    for (int s = 0; s < NG; ++s) {
        const int st = s % P;
        uint4 *xb = lds_x + (s & 1) * kGu4XRows * kStepPitch;
        if (xrow <= kBlockM)                        // row 32 takes the rows past the tile
            xb[xrow * kGu4Pitch + xseg] = permute8(xr[s % PX]);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        // an opaque LDS offset per step keeps the compiler from hoisting
        // later steps' scale/zero and activation reads into registers
        int loff = 0;
        asm volatile("" : "+v"(loff));
#pragma unroll
        for (int c = 0; c < 2; ++c) {              // pair c: its gate and up tiles
            float scale[2];
            f16x2 c1024[2], c64[2];
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const int row = sz_row(2 * c + v);
                zero_point_consts(lds_z[loff + row * NG + s], c1024[v], c64[v]);
                scale[v] = (float)__builtin_bit_cast(_Float16, lds_s[loff + row * NG + s]);
            }
            f32x4 part[2][NMS];
#pragma unroll
            for (int t = 0; t < kWords; ++t) {
                f16x8 bop[2];
#pragma unroll
                for (int v = 0; v < 2; ++v)
                    bop[v] = dequant8(frag_word<G>(bq[st][2 * c + v], t), c1024[v], c64[v]);
                const int seg = quarter * (G / 32) + t;
#pragma unroll
                for (int ms = 0; ms < NMS; ++ms) {
                    const f16x8 aop = __builtin_bit_cast(f16x8, xb[loff + (ms * 16 + lrow) * kGu4Pitch + seg]);
#pragma unroll
                    for (int v = 0; v < 2; ++v)
                        part[v][ms] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            aop, bop[v], t == 0 ? zero4 : part[v][ms], 0, 0, 0);
                }
            }
#pragma unroll
            for (int v = 0; v < 2; ++v)
#pragma unroll
                for (int ms = 0; ms < NMS; ++ms) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[2 * c + v][ms][i] += scale[v] * part[v][ms][i];
                    // pin the accumulation here: otherwise the compiler
                    // sinks it to the epilogue and keeps every partial live
                    asm volatile("" : "+v"(acc[2 * c + v][ms]));
                }
        }
        if (s + PX < NG)
            issue_x(s % PX, s + PX);
        if (s + P < NG)
            issue_w(st, s + P);
    }
    __builtin_amdgcn_sched_barrier(0);
    after_k();
    __builtin_amdgcn_sched_barrier(0);
    // epilogue: H = gelu_tanh(gate) * up in fp16, permuted per 8, into the
    // LDS frame at column 32 cb + local column (each wave owns its columns);
    // rows past the tile's valid rows hold gelu(0) * 0 = 0. The lane's
    // indices are recomputed from an opaque copy of the thread id (kept
    // across the loop they would be spilled, and their reload would wait for
    // every load in flight).
    int etid = threadIdx.x;
    asm volatile("" : "+v"(etid));
    const int equarter = (etid & 63) >> 4;
    const int elrow = etid & 15;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int hcol = kBlockM * cb + permuted_col(wave * 32 + c * 16 + elrow);   // 32 cb: a multiple of 8
#pragma unroll
        for (int ms = 0; ms < NMS; ++ms) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = ms * 16 + equarter * 4 + i;
                const float hv = gelu_tanh(acc[2 * c][ms][i]) * acc[2 * c + 1][ms][i];
                lds_h[r * kHPitch + hcol] = __builtin_bit_cast(uint16_t, (_Float16)hv);
            }
        }
    }
    // the frame's 32 columns outside this half: zero (rows 16 NMS .. 31 are
    // never read)
    if (etid < kBlockM * 4) {
        const int r = etid >> 2, sg = etid & 3;
        const int col = (cb == 0 ? kGu4Cols : 0) + sg * 8;
        *reinterpret_cast<uint4 *>(lds_h + r * kHPitch + col) = make_uint4(0u, 0u, 0u, 0u);
    }
}

// ---- 3. down, the workgroup's half of the contraction into all outputs.
// The 176 row tiles of d = 2816 are shared out at run time: wave w starts
// with tiles w, w + 11 and w + 22, and each time it finishes one it takes the
// next unclaimed tile from a counter in LDS, so waves that the memory path
// serves faster do more tiles and all of them stay busy to the end. A tile
// covers the half's 6 local groups (global groups 5 h .. 5 h + 5). With each
// tile's weights the wave loads the tile's 16 rows of scales and zero points
// (352 contiguous bytes each: lanes 0-21 and 22-43 take 16 bytes apiece) and
// lays them out in a slot of LDS of its own, from which its lanes read what
// they need: no workgroup-wide staging and no barrier. The MFMA takes the
// weights as its row operand, so a lane ends with four consecutive output
// columns of one assignment row and stores them (8 bytes of the fp16
// partial) as soon as the tile is done.
constexpr int kKsRowTiles = 176;                 // row tiles of d = 2816
constexpr int kKsMaxTiles = 20;                  // row tiles one wave may take
static_assert(kL4Waves * kKsMaxTiles >= kKsRowTiles, "the capped waves still take every tile");
constexpr int kKsGroups = 6;                     // local groups per half
constexpr int kKsAhead = 3;                      // row tiles in flight per wave
constexpr int kKsSzLanes = 16 * kDnGroups * 2 / 16;   // 22 lanes of 16 bytes per array
constexpr int kKsSlot = 2 * 16 * kDnGroups * 2;  // bytes of one tile's scales + zeros (704)

static_assert(kL4Waves * kKsAhead * kKsSlot <= layer_gate_up_lds_bytes(),
              "the waves' scale/zero slots fit where gate_up's staging was");

struct DownKsPrefetch {
    Frag<64> bq[kKsAhead][kKsGroups];            // weights of the row tiles in flight
    uint4 sz[kKsAhead];                          // the lane's 16 bytes of their scales/zeros
};

// Lanes of local group j that hold K of the other half: quarters 2, 3 of
// group 5 for h = 0, quarters 0, 1 of group 5 for h = 1.
__device__ inline bool ks_idle(int h, int j, int quarter)
{
    return h == 0 ? (j == kKsGroups - 1 && quarter >= 2) : (j == 0 && quarter < 2);
}

// A lane's part of the down addresses, the same for every row tile: the
// tile enters them as rt * (bytes of a row tile).
struct DownKsLane {
    uint32_t wq;                                 // weight offset in row tile 0
    uint32_t wq_split;                           // the same for the split group (out of range if idle)
    const uint16_t *sz;                          // its 16 bytes of row tile 0's scales or zeros
};

template <bool TL>
__device__ __forceinline__ DownKsLane down_ks_lane(const GemmArgs &p, int e, int h, int lane)
{
    constexpr int K = kDnGroups * 64;
    constexpr int NG = kDnGroups;
    DownKsLane l;
    l.wq = wq_lane_off<64, TL>(lane & 15, lane, K);
    l.wq_split = ks_idle(h, h == 0 ? kKsGroups - 1 : 0, lane >> 4) ? kOutOfRange : l.wq;
    const int sl = lane < 2 * kKsSzLanes ? lane : 0;   // lanes past 43 repeat lane 0's load
    l.sz = (sl < kKsSzLanes ? p.s : p.z) + (size_t)e * p.n_w * NG + (sl % kKsSzLanes) * 8;
    return l;
}

// Loads of row tile rt into prefetch stage st; past the last tile the weight
// loads read nothing and the scale/zero load repeats the last tile's (it is
// issued on every path, so the loads in flight are the same on all of them).
template <bool TL, bool NT>
__device__ __forceinline__ void down_ks_issue(const GemmArgs &p, int e, int h, const DownKsLane &l,
                                              DownKsPrefetch &pf, int st, int rt)
{
    constexpr int K = kDnGroups * 64;
    constexpr int NG = kDnGroups;
    constexpr uint32_t kTileBytes = 16 * K / 2;    // one row tile of the weights
    const rsrc_t rq = make_rsrc(p.q + (size_t)e * p.n_w * (size_t)(K / 2),
                                (uint32_t)p.n_w * (uint32_t)(K / 2));
    const bool live = rt < kKsRowTiles;
    const uint32_t tile_off = (uint32_t)rt * kTileBytes;
    const uint32_t v = live ? l.wq + tile_off : kOutOfRange;
    const uint32_t vs = live && l.wq_split != kOutOfRange ? l.wq_split + tile_off : kOutOfRange;
#pragma unroll
    for (int g = 0; g < kKsGroups; ++g) {
        const bool split = g == (h == 0 ? kKsGroups - 1 : 0);
        pf.bq[st][g] = load_frag<64, NT>(rq, split ? vs : v, wq_group_off<64, TL>(g + 5 * h));
    }
    const int srt = live ? rt : kKsRowTiles - 1;
    pf.sz[st] = *reinterpret_cast<const uint4 *>(l.sz + (size_t)srt * 16 * NG);
}

// The first row tile of prefetch stage j of wave w (the rest are claimed).
__device__ __forceinline__ int ks_first_tile(int wave, int j) { return wave + j * kL4Waves; }

template <bool TL, bool NT>
__device__ __forceinline__ void down_ks_prefetch(const GemmArgs &p, int e, int h, DownKsPrefetch &pf)
{
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const DownKsLane l = down_ks_lane<TL>(p, e, h, tid & 63);
#pragma unroll
    for (int j = 0; j < kKsAhead; ++j)
        down_ks_issue<TL, NT>(p, e, h, l, pf, j, ks_first_tile(wave, j));
}

// s_next: the LDS counter of claimed row tiles, set by this function before
// its first barrier.
template <int NMS, bool TL, bool NT>
__device__ __forceinline__ void down_ks_body(const GemmArgs &p, int e, int h, const int *s_rows,
                                             int valid, DownKsPrefetch &pf, int *s_next)
{
    constexpr int G = 64;
    constexpr int P = kKsAhead;
    constexpr int NG = kDnGroups;
    constexpr int kWords = 2;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));                  // recomputed here, not kept from gate_up
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lrow = lane & 15;
    const int quarter = lane >> 4;
    const int n_out = p.n_out;

    extern __shared__ uint4 lds[];
    char *slots = reinterpret_cast<char *>(lds) + wave * P * kKsSlot;   // this wave's, over gate_up's staging
    const uint16_t *lds_h = reinterpret_cast<const uint16_t *>(reinterpret_cast<const char *>(lds) +
                                                               layer_gate_up_lds_bytes());
    if (tid == 0)
        *s_next = kL4Waves * P;                    // the first P tiles of every wave are fixed
    // H complete; every wave is done with gate_up's staging
    __syncthreads();
    int dst[NMS];                                  // output rows (flat ids) of this lane's MFMA rows
#pragma unroll
    for (int ms = 0; ms < NMS; ++ms)
        dst[ms] = ms * 16 + lrow < valid ? s_rows[ms * 16 + lrow] : -1;

    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    const DownKsLane l = down_ks_lane<TL>(p, e, h, lane);
    // the partial's rows: lane offsets in bytes, out of range (store dropped)
    // for rows past the tile; a row tile adds 32 bytes per tile index
    const rsrc_t ry = make_rsrc(static_cast<uint16_t *>(p.out) + (size_t)h * (size_t)p.A * (size_t)n_out,
                                (uint32_t)p.A * (uint32_t)n_out * 2u);
    uint32_t yoff[NMS];
#pragma unroll
    for (int ms = 0; ms < NMS; ++ms)
        yoff[ms] = dst[ms] >= 0 ? ((uint32_t)dst[ms] * (uint32_t)n_out + (uint32_t)quarter * 4u) * 2u
                                : 0x80000000u;
    int rt[P];                                     // row tile in each prefetch stage (uniform)
#pragma unroll
    for (int st = 0; st < P; ++st)
        rt[st] = ks_first_tile(wave, st);
    // Tile j of the wave comes from stage j % P. Claims only grow and the
    // stages are used in the order they were filled, so the first empty
    // stage ends the wave's work. Straight-line code with forward exits
    // only: the loads in flight are known at every point, so each wait
    // covers just the stage it needs.
#pragma unroll
    for (int j = 0; j < kKsMaxTiles; ++j) {
        const int st = j % P;
        const int cur = rt[st];
        if (cur >= kKsRowTiles)
            break;
        // the tile's scales [16][11] then zero points [16][11] into the
        // slot; the same wave reads them back (its LDS operations run in
        // order)
        char *slot = slots + st * kKsSlot;
        if (lane < 2 * kKsSzLanes)
            *reinterpret_cast<uint4 *>(slot + lane * 16) = pf.sz[st];
        const uint16_t *ls = reinterpret_cast<const uint16_t *>(slot);
        const uint16_t *lz = ls + 16 * NG;
        int aoff = 0;                          // keeps the H reads per tile (see gate_up)
        asm volatile("" : "+v"(aoff));
        f32x4 out[NMS];
#pragma unroll
        for (int ms = 0; ms < NMS; ++ms)
            out[ms] = zero4;
#pragma unroll
        for (int g = 0; g < kKsGroups; ++g) {
            asm volatile("" : "+v"(aoff));     // and per group: no hoisting of later groups' reads
            const int gg = g + 5 * h;          // global group
            f16x2 c1024, c64;
            zero_point_consts(lz[lrow * NG + gg], c1024, c64);
            float sc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sc[i] = (float)__builtin_bit_cast(_Float16, ls[(quarter * 4 + i) * NG + gg]);
            f32x4 prt[NMS];
#pragma unroll
            for (int t = 0; t < kWords; ++t) {
                const f16x8 bop = dequant8(frag_word<G>(pf.bq[st][g], t), c1024, c64);
                const int col = g * G + quarter * (G / 4) + t * 8;   // K in the frame
#pragma unroll
                for (int ms = 0; ms < NMS; ++ms) {
                    const f16x8 aop = *reinterpret_cast<const f16x8 *>(
                        lds_h + aoff + (ms * 16 + lrow) * kHPitch + col);
                    prt[ms] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bop, aop, t == 0 ? zero4 : prt[ms],
                                                                     0, 0, 0);
                }
            }
#pragma unroll
            for (int ms = 0; ms < NMS; ++ms) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    out[ms][i] += sc[i] * prt[ms][i];
                asm volatile("" : "+v"(out[ms]));   // pin the accumulation (see gate_up)
            }
        }
        // claim the wave's next row tile and start its loads in this stage
        // (a wave that has reached its cap claims no more)
        if (j + P < kKsMaxTiles) {
            int next = 0;
            if (lane == 0)
                next = atomicAdd(s_next, 1);
            next = __builtin_amdgcn_readfirstlane(next);
            rt[st] = next;
            down_ks_issue<TL, NT>(p, e, h, l, pf, st, next);
        }
        // output columns cur * 16 + 4 quarter .. + 3 of the lane's rows
#pragma unroll
        for (int ms = 0; ms < NMS; ++ms)
            store8(ry, yoff[ms] + (uint32_t)cur * 32u, pack_f16x4(out[ms]));
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Rows: a callable that ranks the tile's rows into s_rows, run once the
// first weight loads are out.
template <int NMS, bool TL, bool NT, class Rows>
__device__ __forceinline__ void layer_body(const GemmArgs &gu, const GemmArgs &dn, int e, int h,
                                           Rows &&rows, const int *s_rows, int valid, int *s_next)
{
    DownKsPrefetch pf;
    gate_up4_body<NMS, TL, NT>(gu, e, h, rows, s_rows,
                               [&]() { down_ks_prefetch<TL, NT>(dn, e, h, pf); });
    down_ks_body<NMS, TL, NT>(dn, e, h, s_rows, valid, pf, s_next);
}

// Workgroup -> (half, tile): consecutive workgroups go to the 8 XCDs in
// turn, and slot s of XCD x takes half s % 2 of tile layer_tile_of(x, s / 2),
// a contiguous block of tiles per XCD: both halves of a tile share one L2
// (its activation rows), and so do the tiles of an expert with several (its
// weights). Y gets the two fp16 partials [2][A][d] at each assignment's flat
// id.
template <bool TL>
__global__ void __launch_bounds__(kL4Threads) layer_kernel(GemmArgs gu, GemmArgs dn,
                                                           const int32_t *__restrict__ ids, int E)
{
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_wsum[kL4Waves];
    __shared__ int s_rows[kBlockM];
    __shared__ int s_info[4];
    __shared__ int s_next;
    const int xcd = (int)blockIdx.x % kXcds, slot = (int)blockIdx.x / kXcds;
    const int h = slot % 2;
    TileSetup ts;
    const int e = layer_tile_find(ids, gu.A, E, xcd, slot / 2, ts, s_cnt, s_wsum, s_rows, s_info);
    if (e < 0)
        return;
    auto rows = [&]() { layer_tile_rows(ids, gu.A, e, ts, s_wsum, s_rows); };
    const int valid = ts.valid;
    // tiled weights of an expert that no other tile reads stream past the
    // caches; those of an expert with several tiles stay cacheable
    const bool nt = TL && ts.tiles == 1;
    // (the distinct asm statements keep the compiler from hoisting the arms'
    // common prologue above the branch, which spills)
    if (valid > 16) {
        if (nt) {
            asm volatile("; streaming weights");
            layer_body<2, TL, TL>(gu, dn, e, h, rows, s_rows, valid, &s_next);
        } else {
            asm volatile("; cached weights");
            layer_body<2, TL, false>(gu, dn, e, h, rows, s_rows, valid, &s_next);
        }
    } else {
        if (nt) {
            asm volatile("; streaming weights");
            layer_body<1, TL, TL>(gu, dn, e, h, rows, s_rows, valid, &s_next);
        } else {
            asm volatile("; cached weights");
            layer_body<1, TL, false>(gu, dn, e, h, rows, s_rows, valid, &s_next);
        }
    }
}

// ---- down alone (gate_up at another group size, or down's own group size
// 128 at K = 768): workgroup = (tile, 1408 output columns = 88 row tiles);
// wave w streams row tiles w, w + 11, ..., w + 77, P tiles ahead, each
// tile's output stored when done; H from the gate_up launch, the tile's rows
// from the alignment kernel. Instantiated for (g, K/g) = (64, 11) and
// (128, 6): the same body for both group sizes.
constexpr int kDn4Tiles = 8;                     // row tiles per wave
constexpr int kDn4Rows = kL4Waves * kDn4Tiles * 16;   // 1408 weight rows per workgroup
constexpr int kDn4Ahead = 2;
static_assert(kKsRowTiles * 16 == 2 * kDn4Rows, "the layer kernel's down covers all d outputs");

// activation segments per thread: 32 rows x K/8 segments over 704 threads
constexpr int down4_a_loads(int K) { return (kBlockM * (K / 8) + kL4Threads - 1) / kL4Threads; }

template <int G, int NG>
constexpr size_t down4_lds_bytes()
{
    return sizeof(uint4) * kBlockM * (NG * G / 8 + 1) + 2 * sizeof(uint16_t) * kDn4Rows * NG;
}

template <int G, int NG, int NMS, bool TL, bool NT>
__device__ __forceinline__ void down4_body(const GemmArgs &p, int e, int row0, int cb,
                                           const uint4 (&av)[down4_a_loads(NG * G)], int fid)
{
    constexpr int P = kDn4Ahead;
    constexpr int K = NG * G;                      // 704 or 768
    constexpr int kALoads = down4_a_loads(K);
    constexpr int kWords = G / 32;
    constexpr int a_pitch = K / 8 + 1;
    constexpr int seg_row = K / 8;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lrow = lane & 15;
    const int quarter = lane >> 4;
    const int n_out = p.n_out;
    const size_t wexp = (size_t)e * p.n_w;
    const int rt0 = cb * (kDn4Rows / 16);          // first weight row tile of the block

    extern __shared__ uint4 lds[];
    uint4 *lds_a = lds;                                             // [32][a_pitch]
    uint16_t *lds_s = reinterpret_cast<uint16_t *>(lds + kBlockM * a_pitch);   // [NG][1408]
    uint16_t *lds_z = lds_s + kDn4Rows * NG;
    __shared__ int s_dst[kBlockM];

    // ---- 1. scale/zero of the block's rows, then the first weight tiles
    const rsrc_t rs = make_rsrc(p.s + wexp * (size_t)NG, (uint32_t)p.n_w * (uint32_t)NG * 2u);
    const rsrc_t rz = make_rsrc(p.z + wexp * (size_t)NG, (uint32_t)p.n_w * (uint32_t)NG * 2u);
    constexpr int kSzSeg = kDn4Rows * NG * 2 / 16;                  // 1936 or 1056
    constexpr int kSzLoads = (kSzSeg + kL4Threads - 1) / kL4Threads;   // 3 or 2
    const uint32_t sz_base = (uint32_t)(rt0 * 16 * NG) * 2u;
    uint4 sv[kSzLoads], zv[kSzLoads];
#pragma unroll
    for (int i = 0; i < kSzLoads; ++i) {
        const int x = i * kL4Threads + tid;
        const uint32_t off = x < kSzSeg ? sz_base + (uint32_t)x * 16u : kOutOfRange;
        sv[i] = load16(rs, off, 0);
        zv[i] = load16(rz, off, 0);
    }
    const rsrc_t rq = make_rsrc(p.q + wexp * (size_t)(K / 2), (uint32_t)p.n_w * (uint32_t)(K / 2));
    auto tile_row = [&](int j) { return (rt0 + wave + j * kL4Waves) * 16; };   // first weight row
    Frag<G> bq[P][NG];
    auto issue_w = [&](int st, int j) {
        const uint32_t voff = j < kDn4Tiles ? wq_lane_off<G, TL>(tile_row(j) + lrow, lane, K) : kOutOfRange;
#pragma unroll
        for (int g = 0; g < NG; ++g)
            bq[st][g] = load_frag<G, NT>(rq, voff, wq_group_off<G, TL>(g));
    };
#pragma unroll
    for (int j = 0; j < P; ++j)
        issue_w(j, j);
    __builtin_amdgcn_sched_barrier(0);

    // ---- 2. scale/zero (transposed to [g][row]), activations and row
    // destinations into LDS
    {
        auto put8 = [&](uint16_t *dst, int x, uint4 v) {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int el = x * 8 + k;
                const int r = el / NG, g = el - r * NG;
                dst[g * kDn4Rows + r] = (uint16_t)(w[k >> 1] >> (16 * (k & 1)));
            }
        };
#pragma unroll
        for (int i = 0; i < kSzLoads; ++i) {
            const int x = i * kL4Threads + tid;
            if (x < kSzSeg) {
                put8(lds_s, x, sv[i]);
                put8(lds_z, x, zv[i]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kALoads; ++i) {
        const int x = i * kL4Threads + tid;
        const int r = x / seg_row, sg = x - r * seg_row;
        if (r < 16 * NMS)
            lds_a[r * a_pitch + sg] = av[i];
    }
    if (tid < kBlockM)
        s_dst[tid] = fid < p.A ? fid : -1;
    __syncthreads();

    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    int dst[NMS];
#pragma unroll
    for (int ms = 0; ms < NMS; ++ms)
        dst[ms] = s_dst[ms * 16 + lrow];
    uint16_t *Y = static_cast<uint16_t *>(p.out);

    // ---- 3. stream the wave's 8 row tiles, P ahead; each tile's 16 x 32
    // outputs are stored as soon as its NG groups are done
#pragma unroll
    for (int j = 0; j < kDn4Tiles; ++j) {
        const int st = j % P;
        int aoff = 0;                              // keeps the A reads per tile (see gate_up)
        asm volatile("" : "+v"(aoff));
        const int srow = tile_row(j) - rt0 * 16;
        f32x4 out[NMS];
#pragma unroll
        for (int ms = 0; ms < NMS; ++ms)
            out[ms] = zero4;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            asm volatile("" : "+v"(aoff));         // and per group: no hoisting of later groups' reads
            f16x2 c1024, c64;
            zero_point_consts(lds_z[g * kDn4Rows + srow + lrow], c1024, c64);
            const uint2 s4 = *reinterpret_cast<const uint2 *>(lds_s + g * kDn4Rows + srow + quarter * 4);
            float sc[4];
            sc[0] = (float)__builtin_bit_cast(_Float16, (uint16_t)s4.x);
            sc[1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(s4.x >> 16));
            sc[2] = (float)__builtin_bit_cast(_Float16, (uint16_t)s4.y);
            sc[3] = (float)__builtin_bit_cast(_Float16, (uint16_t)(s4.y >> 16));
            f32x4 prt[NMS];
#pragma unroll
            for (int t = 0; t < kWords; ++t) {
                const f16x8 bop = dequant8(frag_word<G>(bq[st][g], t), c1024, c64);
                const int seg = g * (G / 8) + quarter * (G / 32) + t;
#pragma unroll
                for (int ms = 0; ms < NMS; ++ms) {
                    const f16x8 aop = __builtin_bit_cast(f16x8, lds_a[aoff + (ms * 16 + lrow) * a_pitch + seg]);
                    prt[ms] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bop, aop, t == 0 ? zero4 : prt[ms], 0, 0, 0);
                }
            }
#pragma unroll
            for (int ms = 0; ms < NMS; ++ms) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    out[ms][i] += sc[i] * prt[ms][i];
                asm volatile("" : "+v"(out[ms]));   // pin the accumulation (see gate_up)
            }
        }
        issue_w(st, j + P);
        const int col = tile_row(j) + quarter * 4;
#pragma unroll
        for (int ms = 0; ms < NMS; ++ms)
            if (dst[ms] >= 0)
                *reinterpret_cast<uint2 *>(Y + (size_t)dst[ms] * n_out + col) = pack_f16x4(out[ms]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int G, int NG, bool TL>
__global__ void __launch_bounds__(kL4Threads) down4_kernel(GemmArgs p)
{
    constexpr int kALoads = down4_a_loads(NG * G);
    // workgroup -> (column half, tile), both halves of a tile on one XCD; the
    // tile's activation rows and assignment ids are requested before its
    // descriptor is known
    const int xcd = (int)blockIdx.x % kXcds, slot = (int)blockIdx.x / kXcds;
    const int cb = slot % 2;
    const int tile = slot / 2 * kXcds + xcd;
    if (tile >= p.max_tiles)
        return;
    const int tid = threadIdx.x;
    const rsrc_t ra = make_rsrc(p.a_src, (uint32_t)p.a_rows * (uint32_t)p.K * 2u);
    uint4 av[kALoads];
#pragma unroll
    for (int i = 0; i < kALoads; ++i)
        av[i] = load16(ra, down_a_off(p, tile * kBlockM, i * kL4Threads + tid), 0);
    int fid = p.A;
    if (tid < kBlockM)
        fid = p.sorted_ids[tile * kBlockM + tid];
    const int2 info = p.tile_info[tile];
    if (info.x < 0)
        return;
    const bool more = tile_valid(info.y) > 16;
    if (TL && tile_count(info.y) == 1) {
        if (more)
            down4_body<G, NG, 2, TL, TL>(p, info.x, tile * kBlockM, cb, av, fid);
        else
            down4_body<G, NG, 1, TL, TL>(p, info.x, tile * kBlockM, cb, av, fid);
    } else {
        if (more)
            down4_body<G, NG, 2, TL, false>(p, info.x, tile * kBlockM, cb, av, fid);
        else
            down4_body<G, NG, 1, TL, false>(p, info.x, tile * kBlockM, cb, av, fid);
    }
}


// the layer's shape takes the wide-block kernels (gate_up only fused with down)
bool layer_shape_gate_up(const GemmArgs &a, int g)
{
    return g == 128 && a.K == kGuSteps * 256 && a.n_out == 2 * kGu4Cols && a.n_w == 2 * a.n_out;
}

// the wide-block down body: d = 2816 outputs at (g, K) = (64, 704) or (128, 768)
bool layer_shape_down(const GemmArgs &a, int g)
{
    return ((g == 64 && a.K == kDnGroups * 64) || (g == 128 && a.K == 6 * 128)) &&
           a.n_out == 2 * kDn4Rows && a.n_w == a.n_out;
}

template <int G, int NG, bool TL>
hipError_t launch_down4(const GemmArgs &a, hipStream_t stream)
{
    static size_t allowed = 64 * 1024;             // one per instantiation
    hipError_t err = allow_lds(down4_kernel<G, NG, TL>, down4_lds_bytes<G, NG>(), allowed);
    if (err != hipSuccess)
        return err;
    const int tiles = (a.max_tiles + kXcds - 1) / kXcds * kXcds;
    down4_kernel<G, NG, TL><<<dim3(tiles * 2), dim3(kL4Threads), down4_lds_bytes<G, NG>(), stream>>>(a);
    return hipGetLastError();
}

template <bool TL>
hipError_t launch_layer_k(const GemmArgs &gu, const GemmArgs &dn, const int32_t *ids, int E,
                          hipStream_t stream)
{
    static size_t allowed = 64 * 1024;
    hipError_t err = allow_lds(layer_kernel<TL>, layer_lds_bytes(), allowed);
    if (err != hipSuccess)
        return err;
    const int tiles = (gu.max_tiles + kXcds - 1) / kXcds * kXcds;
    layer_kernel<TL><<<dim3(tiles * 2), dim3(kL4Threads), layer_lds_bytes(), stream>>>(gu, dn, ids, E);
    return hipGetLastError();
}

template <int G, bool TL>
hipError_t launch_linear_g(const GemmArgs &a, hipStream_t stream)
{
    const int nblocks = (a.n_out + kGuCols - 1) / kGuCols;
    if (a.max_tiles == 0 || nblocks == 0)
        return hipSuccess;
    auto kern = linear_kernel<G, TL>;
    static size_t allowed = 64 * 1024;              // raised once per instantiation when needed
    const size_t lds = gate_up_lds_bytes_k<G>(a.K);
    hipError_t err = allow_lds(kern, lds, allowed);
    if (err != hipSuccess)
        return err;
    const long long blocks = (long long)(nblocks + kXcds - 1) / kXcds * kXcds * a.max_tiles;
    if (blocks > INT_MAX)
        return hipErrorInvalidValue;
    kern<<<dim3((unsigned)blocks), dim3(kGuThreads), lds, stream>>>(a);
    return hipGetLastError();
}

template <int G, bool TL>
hipError_t launch_gate_up_g(const GemmArgs &a, hipStream_t stream)
{
    const int nblocks = (a.n_out + kGuCols - 1) / kGuCols;
    if (a.max_tiles == 0 || nblocks == 0)
        return hipSuccess;
    auto kern = gate_up_kernel<G, TL>;
    static size_t allowed = 64 * 1024;              // raised once per instantiation when needed
    const size_t lds = gate_up_lds_bytes_k<G>(a.K);
    hipError_t err = allow_lds(kern, lds, allowed);
    if (err != hipSuccess)
        return err;
    const int tiles = (a.max_tiles + kXcds - 1) / kXcds * kXcds;
    kern<<<dim3(tiles * nblocks), dim3(kGuThreads), lds, stream>>>(a);
    return hipGetLastError();
}

template <int G, bool TL>
hipError_t launch_down_g(const GemmArgs &a, hipStream_t stream)
{
    const int nblocks = (a.n_out / 16 + kDnRows / 16 - 1) / (kDnRows / 16);
    if (a.max_tiles == 0 || nblocks == 0)
        return hipSuccess;
    auto kern = down_kernel<G, TL>;
    static size_t allowed = 64 * 1024;
    const size_t lds = down_lds_bytes_k<G>(a.K);
    hipError_t err = allow_lds(kern, lds, allowed);
    if (err != hipSuccess)
        return err;
    const int tiles = (a.max_tiles + kXcds - 1) / kXcds * kXcds;
    kern<<<dim3(tiles * nblocks), dim3(kDnThreads), lds, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

size_t gemm_lds_bytes(bool gated, int K, int g)
{
    if (gated)
        return g == 128 ? gate_up_lds_bytes_k<128>(K) : gate_up_lds_bytes_k<64>(K);
    return g == 128 ? down_lds_bytes_k<128>(K) : down_lds_bytes_k<64>(K);
}

int down_max_k() { return 1536; }

int gate_up_max_groups() { return kGuMaxGroups; }

hipError_t launch_gate_up(const GemmArgs &a, int g, hipStream_t stream)
{
    if (a.max_tiles == 0)
        return hipSuccess;
    if (a.tiled)
        return g == 128 ? launch_gate_up_g<128, true>(a, stream) : launch_gate_up_g<64, true>(a, stream);
    return g == 128 ? launch_gate_up_g<128, false>(a, stream) : launch_gate_up_g<64, false>(a, stream);
}

hipError_t launch_down(const GemmArgs &a, int g, hipStream_t stream)
{
    if (a.max_tiles == 0)
        return hipSuccess;
    if (layer_shape_down(a, g)) {
        if (g == 64)
            return a.tiled ? launch_down4<64, kDnGroups, true>(a, stream)
                           : launch_down4<64, kDnGroups, false>(a, stream);
        return a.tiled ? launch_down4<128, 6, true>(a, stream) : launch_down4<128, 6, false>(a, stream);
    }
    if (a.tiled)
        return g == 128 ? launch_down_g<128, true>(a, stream) : launch_down_g<64, true>(a, stream);
    return g == 128 ? launch_down_g<128, false>(a, stream) : launch_down_g<64, false>(a, stream);
}

// With no choice given, the dense linear takes the many-row kernel from 128
// rows on once T * N >= 2^23, i.e. its 256-row x 256-column workgroups
// would cover 128 CUs at full row blocks. Below that the many-row grid is
// too small to fill the chip: each workgroup runs the whole K (about 65 us
// at K = 2816), so one round of a few workgroups costs as much as a full
// one, while the 32-row tiles spread the same work over many workgroups.
// Measured at K = 2816, g = 128 (us, tiles against many-row): T = 256,
// N = 16384: 47.5 / 68.9; T = 512, N = 16384: 91.3 / 73.0; T = 128,
// N = 32768: 47.7 / 66.9; T = 128, N = 65536: 90.3 / 72.6; the rule picks
// the faster kernel at all 28 points of N = 2^11 .. 2^17 x T = 128 .. 1024.
constexpr int kLinearWideMinRows = 128;
constexpr long long kLinearWideMinWork = 1LL << 23;   // T * N

int linear_row_block(const GemmArgs &a, int g, int rows)
{
    const bool fits = linear_wide_fits(a, g);
    if (rows == DGW4_ROWS_CHUNKS)
        return fits ? kLinearWideRows : -1;
    if (rows == DGW4_ROWS_TILES)
        return kBlockM;
    const bool wide = fits && a.A >= kLinearWideMinRows && (long long)a.A * a.n_out >= kLinearWideMinWork;
    return wide ? kLinearWideRows : kBlockM;
}

hipError_t launch_linear(const GemmArgs &a, int g, int row_block, hipStream_t stream)
{
    if (row_block == kLinearWideRows)
        return launch_linear_wide(a, g, stream);
    if (a.tiled)
        return g == 128 ? launch_linear_g<128, true>(a, stream) : launch_linear_g<64, true>(a, stream);
    return g == 128 ? launch_linear_g<128, false>(a, stream) : launch_linear_g<64, false>(a, stream);
}

bool layer_fused(const GemmArgs &gu, int gu_g, const GemmArgs &dn, int dn_g, int E)
{
    // (the layer kernel stores each Y partial through 32-bit byte offsets
    // below 2^31, and its alignment takes one expert per thread)
    return layer_shape_gate_up(gu, gu_g) && dn_g == 64 && layer_shape_down(dn, dn_g) &&
           gu.tiled == dn.tiled && E <= kL4Threads && (long long)dn.A * dn.n_out * 2 < (1LL << 31);
}

hipError_t launch_layer(const GemmArgs &gu, const GemmArgs &dn, const int32_t *ids, int E,
                        hipStream_t stream)
{
    if (gu.max_tiles == 0)
        return hipSuccess;
    if (gu.tiled != dn.tiled)
        return hipErrorInvalidValue;               // layer_fused() is false for a mixed pair
    return gu.tiled ? launch_layer_k<true>(gu, dn, ids, E, stream)
                    : launch_layer_k<false>(gu, dn, ids, E, stream);
}

}  // namespace dgw4

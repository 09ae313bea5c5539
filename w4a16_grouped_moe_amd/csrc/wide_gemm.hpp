// The many-row W4A16 GEMM body shared by the dense linear over many rows
// (many_rows.hip) and the routed-expert layer's GEMMs over 128-row chunks
// (chunk_gate_up.hip, chunk_down.hip): every weight is formed once per block
// of rows and feeds all of them.
//
// Follows the kernel card's "W4A16" section (w4a16_linear(x, qw, scale,
// zero) equals F.linear(x, dequant(W)), weights dequantised in registers
// into fp16 MFMA fragments) and "Grouped MoE" (one launch covers every
// expert, the gated activation folded into the first GEMM's epilogue); the
// model card's "Checkpoint format" (w = (q - z) * s per group along K); and
// the Part 2 blog's "Quantisation alone leaves a sparse execution problem"
// (assignments sorted by expert and padded to a block size; the block size
// of the chunk GEMMs is 128 rows).
#pragma once

#include "dgw4_internal.hpp"
#include "gemm_common.hpp"

#include <climits>

namespace dgw4 {
namespace {

// ---- The shared body. Workgroup = (block of rows, 256 weight rows), 8
// waves, two per SIMD; wave w takes all the block's rows and two 16-row
// weight tiles (32 of the workgroup's weight rows), so each weight fragment
// it forms feeds one MFMA per 16-row block of rows and each staged
// activation slice serves 256 weight rows. The K loop walks one quantisation
// group per step: each wave loads its tiles' share of the group (16 or 8
// bytes per lane and tile) P steps ahead, and the workgroup stages the
// step's activation slice (the block's rows x G values, as loaded) in a
// double-buffered LDS area from registers loaded ahead of it (the linear: in
// two halves, each half a step ahead; the chunk modes: whole, one or two
// steps ahead), one barrier per step; the slots of a row are XOR-swizzled so
// that the 16 rows one MFMA fragment reads hit distinct banks. The weights are the MFMA's row operand,
// so a lane holds one weight row per tile: it forms that row's fp16 weights
// (q - z) * s for the group (q - z exact, one rounding of the product), in
// natural K order, and the MFMA accumulates all groups in fp32; a lane ends
// with four consecutive output columns of one row. Scales and zero points of
// the workgroup's weight rows are staged in LDS once, transposed to
// [group][weight row].
//
// The three modes differ in the block and its rows:
//   linear: 256 consecutive rows of x, 256 consecutive weight rows (output
//     columns); y stored in natural column order;
//   gate_up: one 128-row chunk (rows of x gathered through the sorted
//     assignment ids), 128 gate rows c0 .. c0 + 127 and the matching up rows
//     m + c0 ..: wave w's tiles are gate rows c0 + 16 w .. and up rows
//     m + c0 + 16 w .., and it stores gelu_tanh(gate) * up as H[chunk row,
//     c0 + 16 w ..] (fp16, natural column order, H rows = the chunk's
//     padded rows);
//   down: one chunk of H's rows, 256 consecutive down rows (output
//     columns); each row's output goes to Y[assignment id] (fp16).
// In the chunk modes only the 16-row blocks that hold assignments run: the
// kernel picks, per wave, the straight-line instance of the body for that
// count (a wave whose tiles lie past the weight rows runs none).
enum : int { kModeLinear = 0, kModeGateUp = 1, kModeDown = 2 };

constexpr int kLwWaves = 8;
constexpr int kLwThreads = kLwWaves * 64;
constexpr int kLwRows = 256;                     // rows per block of the dense linear
constexpr int kLwCols = 256;                     // weight rows per workgroup of the dense linear
constexpr int kChunkWaves = 8;                   // waves per workgroup of the chunk GEMMs
constexpr int kLwNs = 2;                         // 16-row weight tiles per wave

// Waves, threads and weight rows (two 16-row tiles per wave) of a workgroup.
template <int MODE>
constexpr int wide_waves() { return MODE == kModeLinear ? kLwWaves : kChunkWaves; }
template <int MODE>
constexpr int wide_threads() { return wide_waves<MODE>() * 64; }
template <int MODE>
constexpr int wide_cols() { return wide_waves<MODE>() * 16 * kLwNs; }
constexpr int kLwAhead = 2;                      // weight steps in flight (linear)
// The chunk modes run few rows per step (an expert's 16 to 128), too little
// MFMA work to cover a memory latency in one or two steps: gate_up's weights
// go four steps ahead and its activation slices two (a ring of two slices in
// registers, staged whole at the end of a step). down keeps two and one, so
// that it fits 128 VGPRs and two workgroups share a CU.
template <int MODE>
constexpr int chunk_ahead() { return MODE == kModeGateUp ? 4 : 2; }
template <int MODE>
constexpr int chunk_x_ahead() { return MODE == kModeGateUp && kChunkWaves == 8 ? 2 : 1; }
constexpr size_t kMaxWideLds = 160 * 1024;       // a CU's LDS: one workgroup per CU

template <int MODE>
constexpr int wide_rows() { return MODE == kModeLinear ? kLwRows : kChunkM; }

template <int MODE, int G>
constexpr size_t wide_x_bytes() { return sizeof(uint4) * 2 * wide_rows<MODE>() * (G / 8); }

template <int MODE, int G>
size_t wide_lds_bytes(int K)
{
    return wide_x_bytes<MODE, G>() + 2 * sizeof(uint16_t) * (size_t)wide_cols<MODE>() * (size_t)(K / G);
}

// Physical slot of logical 16-byte segment seg of activation row r, an XOR
// swizzle so that a fragment read (16 rows per quarter-wave, the four
// quarters at segments 4 apart) spreads over the banks. With 16 slots per
// row the XOR value is r's low four bits permuted (bit 0 to bit 2): the 16
// rows of a quarter take 16 distinct slots, and rows of opposite parity take
// slots of opposite bit 2, so two quarters served together never meet.
template <int SEGS>
__device__ __forceinline__ int lw_slot(int r, int seg)
{
    if constexpr (SEGS == 16)
        return seg ^ (((r & 1) << 2) | ((r >> 1) & 3) | (r & 8));
    else
        return seg ^ ((r / (16 / SEGS)) % SEGS);
}

// f(S), f(S + 1), ..., f(E - 1) as straight-line code, whatever the body's
// size (a pragma-unrolled loop stops unrolling past a size limit, and its
// stage index would then index registers at run time).
template <int S, int E, class F>
__device__ __forceinline__ void static_steps(F &f)
{
    if constexpr (S < E) {
        f(S);
        static_steps<S + 1, E>(f);
    }
}

// A workgroup's block and a wave's share of it (see wide_block).
struct WideBlock {
    int row0;                // first row of the block (x rows, or chunk rows)
    int col0;                // first weight row of the workgroup's block
    int nvalid;              // rows of the block that hold data
    int wrow;                // first weight row of the wave's tile 0
    int nmb;                 // 16-row blocks the wave runs; -1: the workgroup has no block
    const uint8_t *q;        // the block's weight matrix (the expert's, in the chunk modes)
    const uint16_t *s, *z;
};

template <int MODE>
__device__ __forceinline__ WideBlock wide_block(const GemmArgs &p, int NG)
{
    WideBlock b{};
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lcol = wave * 16 * kLwNs;
    const int xcd = (int)blockIdx.x % kXcds, slot = (int)blockIdx.x / kXcds;
    b.q = p.q;
    b.s = p.s;
    b.z = p.z;
    b.nmb = -1;
    if constexpr (MODE == kModeLinear) {
        // workgroup -> (column block, row block): XCD x takes column blocks
        // x, x + 8, ... and runs a block's row blocks back to back, so those
        // re-read its weights from that XCD's L2
        const int nrb = (p.A + kLwRows - 1) / kLwRows;
        const int rb = slot % nrb;
        const int cb = slot / nrb * kXcds + xcd;
        b.col0 = cb * kLwCols;
        if (b.col0 >= p.n_out)
            return b;
        b.row0 = rb * kLwRows;
        b.nvalid = p.A - b.row0;
        b.wrow = b.col0 + lcol;
        b.nmb = kLwRows / 16;
    } else {
        // workgroup -> (k-th chunk in the alignment's order, most rows
        // first, column block): the column blocks of a chunk run on one XCD,
        // back to back, so its activation rows stay in that XCD's L2; the
        // longest chunks start first, so the last round holds short ones
        constexpr int kBlockCols = MODE == kModeGateUp ? wide_cols<MODE>() / 2 : wide_cols<MODE>();
        const int ncb = (p.n_out + kBlockCols - 1) / kBlockCols;
        const int k = slot / ncb * kXcds + xcd;
        if (k >= p.max_tiles)
            return b;
        const int chunk = p.tile_order ? p.tile_order[k] : k;
        if (chunk < 0 || chunk >= p.max_tiles)
            return b;
        const int2 ti = p.tile_info[chunk];
        if (ti.x < 0)
            return b;
        const size_t e = (size_t)ti.x;
        b.nvalid = tile_valid(ti.y);
        b.row0 = chunk * kChunkM;
        b.col0 = slot % ncb * kBlockCols;
        b.q += e * (size_t)p.n_w * (size_t)(p.K / 2);
        b.s += e * (size_t)p.n_w * (size_t)NG;
        b.z += e * (size_t)p.n_w * (size_t)NG;
        b.wrow = MODE == kModeGateUp ? b.col0 + wave * 16 : b.col0 + lcol;
        // a wave whose tiles lie past the weight rows runs no blocks
        b.nmb = __builtin_amdgcn_readfirstlane(b.wrow < p.n_out ? (b.nvalid + 15) / 16 : 0);
    }
    return b;
}

// NGC > 0: K / G = NGC groups, straight-line code; 0: a loop over K / G.
// NMB: the 16-row blocks the wave runs (the block's, kLwRows / 16, for the
// linear; 0 .. 8 in the chunk modes, the kernel picks the instance), so the
// K loop is straight-line code with no branch around an MFMA.
template <int MODE, int G, int NGC, bool TL, bool NT, int NMB>
__device__ __forceinline__ void wide_body(const GemmArgs &p, const WideBlock &b)
{
    constexpr int P = MODE == kModeLinear ? kLwAhead : chunk_ahead<MODE>();
    constexpr int ROWS = wide_rows<MODE>();
    constexpr int MS = ROWS / 16;                // 16-row MFMA blocks per wave
    constexpr int SEGS = G / 8;                  // 16-byte activation segments per row and step
    constexpr int THREADS = wide_threads<MODE>();
    constexpr int COLS = wide_cols<MODE>();      // weight rows of the workgroup
    constexpr int XLD = ROWS * SEGS / THREADS;   // activation loads per thread and step
    constexpr int kWords = G / 32;               // k-slices of 32 per group
    static_assert(ROWS * SEGS % THREADS == 0 && THREADS % SEGS == 0, "activation split");
    static_assert(MODE == kModeLinear || NGC > 0, "the chunk modes' pipeline needs a static K");
    const int K = p.K;
    const int NG = NGC > 0 ? NGC : K / G;

    static_assert(NMB >= 0 && NMB <= MS, "16-row blocks of the wave");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lrow = lane & 15;
    const int quarter = lane >> 4;
    const int lcol = wave * 16 * kLwNs;          // the wave's first LDS column (weight row)

    const int row0 = b.row0, col0 = b.col0, wrow = b.wrow;
    const uint8_t *qe = b.q;
    const uint16_t *se = b.s, *ze = b.z;
    // rows between the wave's two tiles: the up rows are m below the gate rows
    const int tstride = MODE == kModeGateUp ? p.n_out : 16;
    auto tile_on = [&](int ns) {
        return MODE == kModeGateUp ? wrow < p.n_out : wrow + 16 * ns < p.n_out;
    };

    extern __shared__ uint4 lds[];
    uint4 *lds_x = lds;                                           // [2][ROWS][SEGS], swizzled
    uint16_t *lds_s = reinterpret_cast<uint16_t *>(reinterpret_cast<char *>(lds) + wide_x_bytes<MODE, G>());
    uint16_t *lds_z = lds_s + COLS * NG;                           // [NG][COLS] each

    // ---- scales / zeros of the workgroup's 256 weight rows: [row][group]
    // in memory (512 NG contiguous bytes per array, or two runs of 256 NG for
    // gate_up's gate and up rows), transposed into LDS
    {
        const uint32_t sz_bytes = (uint32_t)p.n_w * (uint32_t)NG * 2u;
        const rsrc_t rs = make_rsrc(se, sz_bytes);
        const rsrc_t rz = make_rsrc(ze, sz_bytes);
        constexpr int kRuns = MODE == kModeGateUp ? 2 : 1;
        constexpr int kRunRows = COLS / kRuns;
        const int per = kRunRows / 8 * NG;       // 16-byte chunks per run
        for (int c = tid; c < kRuns * per; c += THREADS) {
            const int run = kRuns == 2 && c >= per ? 1 : 0;
            const int cc = c - run * per;
            const uint32_t base = (uint32_t)(run * p.n_out + col0) * (uint32_t)NG * 2u;
            const uint4 sv = load16(rs, base + (uint32_t)cc * 16u, 0);
            const uint4 zv = load16(rz, base + (uint32_t)cc * 16u, 0);
            const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
            const uint32_t zw[4] = {zv.x, zv.y, zv.z, zv.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int el = cc * 8 + j;                 // flat [row][group] element of the run
                const int r = el / NG, g = el - r * NG;
                // LDS column: gate_up interleaves the runs per 16 rows, so that
                // wave w's tiles are columns 32 w .. + 15 (gate) and + 16 .. (up)
                const int col = kRuns == 2 ? (r >> 4) * 32 + run * 16 + (r & 15) : r;
                lds_s[g * COLS + col] = (uint16_t)(sw[j >> 1] >> (16 * (j & 1)));
                lds_z[g * COLS + col] = (uint16_t)(zw[j >> 1] >> (16 * (j & 1)));
            }
        }
    }

    // ---- weight loads: tile ns covers weight rows wrow + ns * tstride .. + 15
    const rsrc_t rq = make_rsrc(qe, (uint32_t)p.n_w * (uint32_t)(K / 2));
    // tile ns's lane offset is tile 0's plus ns * tstride rows (scalar);
    // tiles past the weight rows read nothing
    const uint32_t wvoff0 = wq_lane_off<G, TL>(wrow + lrow, lane, K);
    const uint32_t wtile = (uint32_t)tstride * (uint32_t)(K / 2);
    Frag<G> bq[P][kLwNs];
    auto issue_w = [&](int st, int s) {
#pragma unroll
        for (int ns = 0; ns < kLwNs; ++ns)
            bq[st][ns] = load_frag<G, NT>(rq, s < NG && tile_on(ns) ? wvoff0 : kOutOfRange,
                                          wq_group_off<G, TL>(s) + (uint32_t)ns * wtile);
    };
    // ---- activation slices: thread -> (row tid / SEGS + i * rows per pass,
    // segment tid % SEGS); each thread's row offsets, 2^31 (past any source,
    // whatever the step adds) for rows past the block's; the step enters as
    // the scalar offset
    const rsrc_t ra = make_rsrc(p.a_src, (uint32_t)p.a_rows * (uint32_t)K * 2u);
    const int xseg = tid % SEGS;
    constexpr int kRowsPerPass = THREADS / SEGS;
    uint32_t xo[MODE == kModeLinear ? 1 : XLD];
    if constexpr (MODE != kModeLinear) {
#pragma unroll
        for (int i = 0; i < XLD; ++i) {
            const int r = tid / SEGS + i * kRowsPerPass;
            // gate_up: the token of the chunk's r-th assignment; down: H row
            const int src = r >= b.nvalid ? -1
                            : MODE == kModeGateUp ? p.sorted_ids[row0 + r] / p.topk : row0 + r;
            xo[i] = src >= 0 ? (uint32_t)src * (uint32_t)K * 2u + (uint32_t)xseg * 16u : 0x80000000u;
        }
    }
    auto xoff = [&](int i) -> uint32_t {
        if constexpr (MODE == kModeLinear) {
            const int r = row0 + tid / SEGS + i * kRowsPerPass;
            return r < p.A ? (uint32_t)r * (uint32_t)K * 2u + (uint32_t)xseg * 16u : 0x80000000u;
        } else {
            return xo[i];
        }
    };
    // linear: a slice goes in two halves of XLD / 2 loads per thread, each
    // loaded half a step before it is staged
    constexpr int XH = MODE == kModeLinear ? XLD / 2 : 1;
    static_assert(MODE != kModeLinear || XLD % 2 == 0, "activation halves");
    uint4 xr[XH];
    auto issue_x = [&](int s, int half) {
#pragma unroll
        for (int i = 0; i < XH; ++i)
            xr[i] = s < NG ? load16(ra, xoff(half * XH + i), (uint32_t)s * G * 2u) : make_uint4(0u, 0u, 0u, 0u);
    };
    auto stage_x = [&](int buf, int half) {
        uint4 *xb = lds_x + buf * ROWS * SEGS;
#pragma unroll
        for (int i = 0; i < XH; ++i) {
            const int r = tid / SEGS + (half * XH + i) * kRowsPerPass;
            xb[r * SEGS + lw_slot<SEGS>(r, xseg)] = xr[i];
        }
    };

    // chunk modes: slice s in register slot s % XD, loaded whole XD steps
    // before it is staged. Only the rows of the blocks that run are staged
    // (the rest are never read): a thread stages its first XLR rows, which
    // cover rows 0 .. 16 NMB - 1; a wave that runs no block stages all its
    // rows, so that every row the workgroup's other waves read has a stager
    // (the waves of one workgroup run either NMB or no blocks).
    constexpr int XD = MODE == kModeLinear ? 1 : chunk_x_ahead<MODE>();
    constexpr int XLR = MODE == kModeLinear || NMB == 0
                            ? XLD
                            : (NMB * 16 + kRowsPerPass - 1) / kRowsPerPass < XLD
                                  ? (NMB * 16 + kRowsPerPass - 1) / kRowsPerPass
                                  : XLD;
    uint4 xc[XD][MODE == kModeLinear ? 1 : XLR];
    auto issue_xc = [&](int s) {
#pragma unroll
        for (int i = 0; i < XLR; ++i)
            xc[s % XD][i] = s < NG ? load16(ra, xoff(i), (uint32_t)s * G * 2u) : make_uint4(0u, 0u, 0u, 0u);
    };
    auto stage_xc = [&](int s) {
        uint4 *xb = lds_x + (s & 1) * ROWS * SEGS;
#pragma unroll
        for (int i = 0; i < XLR; ++i) {
            const int r = tid / SEGS + i * kRowsPerPass;
            xb[r * SEGS + lw_slot<SEGS>(r, xseg)] = xc[s % XD][i];
        }
    };

#pragma unroll
    for (int s = 0; s < P; ++s)
        issue_w(s, s);
    if constexpr (MODE == kModeLinear) {
        issue_x(0, 0);
        stage_x(0, 0);
        issue_x(0, 1);
        stage_x(0, 1);
        issue_x(1, 0);
    } else {
#pragma unroll
        for (int s = 0; s < XD; ++s)
            issue_xc(s);
        stage_xc(0);
        issue_xc(XD);
    }
    __syncthreads();                             // scales, zeros and slice 0 in LDS

    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc[MS][kLwNs];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int ns = 0; ns < kLwNs; ++ns)
            acc[ms][ns] = zero4;
    // (linear: 16-row blocks past T multiply zeros: a ragged last block costs
    // its MFMAs, the full blocks no branches)

    auto step = [&](int s, int st) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);       // nothing moves between steps
        int loff = 0;                                    // opaque per step: no hoisted reads
        asm volatile("" : "+v"(loff));
        // the slice's buffer as an opaque base, so that the row offsets of the
        // fragment reads stay immediate (the second buffer starts past what
        // an LDS instruction's offset field reaches)
        int xbase = (s & 1) * ROWS * SEGS;
        asm volatile("" : "+v"(xbase));
        const uint4 *xb = lds_x + xbase;
        {
            f16x2 cmix[kLwNs], s2[kLwNs];
#pragma unroll
            for (int ns = 0; ns < kLwNs; ++ns) {
                const int c = loff + s * COLS + lcol + 16 * ns + lrow;   // the lane's weight row
                const uint32_t zb = lds_z[c], sb = lds_s[c];
                cmix[ns] = as_h2(zb | (zb << 16)) + f16x2{(_Float16)1024.0f, (_Float16)64.0f};
                s2[ns] = as_h2(sb | (sb << 16));
            }
            // the step's (k-slice t, 16-row block) pairs in order, each one
            // activation fragment feeding both tiles' MFMAs; fragments are
            // read kAhead pairs before use (LDS latency is several pairs'
            // MFMA time), and between the MFMAs of k-slice t the two tiles'
            // weight fragments of t + 1 are formed
            constexpr int kPairs = kWords * NMB;
            constexpr int kAheadA = MODE == kModeDown ? 3 : 4;   // down: within 128 VGPRs
            // chunk modes: the lane's slot in each k-slice's fragment, one
            // address per k-slice and step (the 16-row block enters as an
            // immediate offset: the swizzle depends on the row's low bits only)
            int aoff[MODE == kModeLinear ? 1 : kWords];
            if constexpr (MODE != kModeLinear) {
#pragma unroll
                for (int t = 0; t < kWords; ++t) {
                    aoff[t] = xbase + lrow * SEGS + lw_slot<SEGS>(lrow, quarter * kWords + t);
                    asm volatile("" : "+v"(aoff[t]));
                }
            }
            auto aread = [&](int i) {
                const int t = i / NMB, ms = i % NMB, r = ms * 16 + lrow;   // row within the block
                if constexpr (MODE == kModeLinear)
                    return __builtin_bit_cast(f16x8, xb[r * SEGS + lw_slot<SEGS>(r, quarter * kWords + t)]);
                else
                    return __builtin_bit_cast(f16x8, lds_x[aoff[t] + ms * 16 * SEGS]);
            };
            // tile ns's fragment of k-slice t + 1 is formed after the MFMAs of
            // block dq_at(ns) of k-slice t
            auto dq_at = [](int ns) {
                const int v = (ns + 1) * NMB / 2 - 1;
                return v > 0 ? v : 0;
            };
            f16x8 bop[kLwNs], bnext[kLwNs];
#pragma unroll
            for (int ns = 0; ns < kLwNs; ++ns)
                bop[ns] = dequant8_scaled(frag_word<G>(bq[st][ns], 0), cmix[ns], s2[ns]);
            f16x8 af[kPairs > 0 ? kPairs : 1];
#pragma unroll
            for (int i = 0; i < kAheadA && i < kPairs; ++i)
                af[i] = aread(i);
#pragma unroll
            for (int i = 0; i < kPairs; ++i) {
                const int t = i / NMB, ms = i % NMB;
                if (MODE == kModeLinear && t == kWords / 2 && ms == 0) {
                    // the first half of the next slice is in: stage it, load the second
                    stage_x((s + 1) & 1, 0);
                    issue_x(s + 1, 1);
                }
                if (i + kAheadA < kPairs)
                    af[i + kAheadA] = aread(i + kAheadA);
#pragma unroll
                for (int ns = 0; ns < kLwNs; ++ns)
                    acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bop[ns], af[i], acc[ms][ns], 0, 0, 0);
#pragma unroll
                for (int ns = 0; ns < kLwNs; ++ns)
                    if (t + 1 < kWords && ms == dq_at(ns))
                        bnext[ns] = dequant8_scaled(frag_word<G>(bq[st][ns], t + 1), cmix[ns], s2[ns]);
                if (t + 1 < kWords && ms == NMB - 1)
#pragma unroll
                    for (int ns = 0; ns < kLwNs; ++ns)
                        bop[ns] = bnext[ns];
                __builtin_amdgcn_sched_barrier(0);   // keep the reads where they are issued
            }
        }
        issue_w(st, s + P);
        if constexpr (MODE == kModeLinear) {
            stage_x((s + 1) & 1, 1);
            issue_x(s + 2, 0);
        } else {
            stage_xc(s + 1);
            issue_xc(s + 1 + XD);
        }
        __syncthreads();
    };
    if constexpr (NGC > 0) {
        auto step_s = [&](int s) __attribute__((always_inline)) { step(s, s % P); };
        static_steps<0, NGC>(step_s);
    } else {
        for (int s0 = 0; s0 < NG; s0 += P)
#pragma unroll
            for (int j = 0; j < P; ++j)
                if (s0 + j < NG)
                    step(s0 + j, j);
    }

    // ---- store: lane (lrow, quarter) has columns 4 quarter .. + 3 of tile
    // ns for row ms * 16 + lrow of the block
    if constexpr (MODE == kModeLinear) {
        // past N the tile stores nothing, past T the buffer drops the store
        const int T = p.A, N = p.n_out;
        const rsrc_t ry = make_rsrc(p.out, (uint32_t)T * (uint32_t)N * 2u);
#pragma unroll
        for (int ns = 0; ns < kLwNs; ++ns) {
            if (!tile_on(ns))
                continue;
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) {
                const int r = row0 + ms * 16 + lrow;
                const uint32_t off = r < T ? ((uint32_t)r * (uint32_t)N + (uint32_t)(wrow + 16 * ns + 4 * quarter)) * 2u
                                           : 0x80000000u;
                store8(ry, off, pack_f16x4(acc[ms][ns]));
            }
        }
    } else if constexpr (MODE == kModeGateUp) {
        // H[row0 + ms * 16 + lrow, wrow + 4 quarter ..] = gelu(gate) * up; the
        // rows of the last block past the chunk's assignments hold zeros
        const int m = p.n_out;
        const rsrc_t rh = make_rsrc(p.out, (uint32_t)p.max_tiles * (uint32_t)ROWS * (uint32_t)m * 2u);
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
            if (ms >= NMB)
                break;
            f32x4 h;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                h[v] = gelu_tanh(acc[ms][0][v]) * acc[ms][1][v];
            const uint32_t off = ((uint32_t)(row0 + ms * 16 + lrow) * (uint32_t)m +
                                  (uint32_t)(wrow + 4 * quarter)) * 2u;
            store8(rh, off, pack_f16x4(h));
        }
    } else {
        // Y[assignment id of the row, wrow + 16 ns + 4 quarter ..]; pad rows
        // (id A) store nothing
        const int d = p.n_out;
        const rsrc_t ry = make_rsrc(p.out, (uint32_t)p.A * (uint32_t)d * 2u);
        int aid[MS];
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
            aid[ms] = ms < NMB ? p.sorted_ids[row0 + ms * 16 + lrow] : p.A;
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
            if (ms >= NMB)
                break;
#pragma unroll
            for (int ns = 0; ns < kLwNs; ++ns) {
                const uint32_t off = aid[ms] < p.A && tile_on(ns)
                                         ? ((uint32_t)aid[ms] * (uint32_t)d +
                                            (uint32_t)(wrow + 16 * ns + 4 * quarter)) * 2u
                                         : 0x80000000u;
                store8(ry, off, pack_f16x4(acc[ms][ns]));
            }
        }
    }
}

template <int MODE, class Kern>
hipError_t launch_wide(Kern kern, size_t lds, size_t &allowed, long long blocks, const GemmArgs &a,
                       hipStream_t stream)
{
    hipError_t err = allow_lds(kern, lds, allowed);
    if (err != hipSuccess)
        return err;
    if (blocks > INT_MAX)
        return hipErrorInvalidValue;
    if (blocks == 0)
        return hipSuccess;
    kern<<<dim3((unsigned)blocks), dim3(wide_threads<MODE>()), lds, stream>>>(a);
    return hipGetLastError();
}

}  // namespace
}  // namespace dgw4

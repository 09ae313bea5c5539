// Dense W4A16 linear over many rows (y = x * deq(W)^T with at least 128
// rows): the many-row kernel, each weight formed once per 256-row block. The
// few-row kernel (32-row tiles) lives with the GEMM bodies it shares.
//
// Follows the kernel card's "W4A16" section: w4a16_linear(x, qw, scale,
// zero) equals F.linear(x, dequant(W)), the weights dequantised in registers
// into fp16 MFMA fragments.
#include "dgw4_internal.hpp"
#include "gemm_common.hpp"

#include <climits>

namespace dgw4 {
namespace {

constexpr int kLinearUnrolledGroups = 22;        // K = 2816 at g = 128: straight-line code

// ---- Dense linear over many rows: every weight dequantised once per
// 256-row block. Workgroup = (256-row block, 256 output columns), 8 waves,
// two per SIMD; wave w takes all 256 rows and columns 32 w .. + 31 of the
// workgroup's (two 16-column weight tiles), so each weight fragment it forms
// feeds sixteen MFMAs and each staged activation slice serves 256 columns of
// weights. The K loop
// walks one quantisation group per step: each wave loads its tiles' share of
// the group (16 or 8 bytes per lane and tile) P steps ahead, and the
// workgroup stages the step's activation slice (256 rows x G values, as
// loaded) in a double-buffered LDS area from registers loaded one step
// ahead, one barrier per step; the slots of a row are XOR-swizzled so that
// the 16 rows one MFMA fragment reads hit distinct banks. The weights are
// the MFMA's row operand, so a lane holds one weight column per tile: it
// forms that column's fp16 weights (q - z) * s for the group (q - z exact,
// one rounding of the product), in natural K order, and the MFMA
// accumulates all groups in fp32; a lane ends with four consecutive output
// columns of one row and stores them (8 bytes). Scales and zero points of
// the workgroup's columns are staged in LDS once, transposed to
// [group][column].
constexpr int kLwWaves = 8;
constexpr int kLwThreads = kLwWaves * 64;
constexpr int kLwRows = 256;                     // rows per block
constexpr int kLwCols = 256;                     // output columns per workgroup
constexpr int kLwMs = 16;                        // 16-row MFMA blocks per wave
constexpr int kLwNs = 2;                         // 16-column weight tiles per wave
constexpr int kLwAhead = 2;                      // weight steps in flight
constexpr size_t kMaxWideLds = 160 * 1024;       // a CU's LDS: one workgroup per CU

template <int G>
constexpr size_t linear_wide_x_bytes() { return sizeof(uint4) * 2 * kLwRows * (G / 8); }

template <int G>
size_t linear_wide_lds_bytes(int K)
{
    return linear_wide_x_bytes<G>() + 2 * sizeof(uint16_t) * (size_t)kLwCols * (size_t)(K / G);
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

// NGC > 0: K / G = NGC groups, straight-line code; 0: a loop over K / G.
template <int G, int NGC, bool TL, bool NT>
__global__ void __launch_bounds__(kLwThreads)
__attribute__((amdgpu_waves_per_eu(2))) linear_wide_kernel(GemmArgs p)
{
    constexpr int P = kLwAhead;
    constexpr int SEGS = G / 8;                  // 16-byte activation segments per row and step
    constexpr int XLD = kLwRows * SEGS / kLwThreads;   // activation loads per thread and step
    constexpr int kWords = G / 32;               // k-slices of 32 per group
    static_assert(kLwRows * SEGS % kLwThreads == 0 && kLwThreads % SEGS == 0, "activation split");
    const int T = p.A, N = p.n_out, K = p.K;
    const int NG = NGC > 0 ? NGC : K / G;
    const int nrb = (T + kLwRows - 1) / kLwRows;
    // workgroup -> (column block, row block): XCD x takes column blocks x,
    // x + 8, ... and runs a block's row blocks back to back, so those re-read
    // its weights from that XCD's L2
    const int xcd = (int)blockIdx.x % kXcds, slot = (int)blockIdx.x / kXcds;
    const int rb = slot % nrb;
    const int cb = slot / nrb * kXcds + xcd;
    const int col0 = cb * kLwCols;
    if (col0 >= N)
        return;
    const int row0 = rb * kLwRows;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lrow = lane & 15;
    const int quarter = lane >> 4;
    const int lcol = wave * 16 * kLwNs;          // the wave's first column in the block
    const int wcol = col0 + lcol;

    extern __shared__ uint4 lds[];
    uint4 *lds_x = lds;                                           // [2][256][SEGS], swizzled
    uint16_t *lds_s = reinterpret_cast<uint16_t *>(reinterpret_cast<char *>(lds) + linear_wide_x_bytes<G>());
    uint16_t *lds_z = lds_s + kLwCols * NG;                        // [NG][256] each

    // ---- scales / zeros of the 256 columns: [col][group] in memory (a
    // contiguous 512 NG bytes per array), transposed into LDS
    {
        const uint32_t sz_bytes = (uint32_t)N * (uint32_t)NG * 2u;
        const rsrc_t rs = make_rsrc(p.s, sz_bytes);
        const rsrc_t rz = make_rsrc(p.z, sz_bytes);
        const uint32_t base = (uint32_t)col0 * (uint32_t)NG * 2u;
        for (int c = tid; c < kLwCols / 8 * NG; c += kLwThreads) {   // 16-byte chunks per array
            const uint4 sv = load16(rs, base + (uint32_t)c * 16u, 0);
            const uint4 zv = load16(rz, base + (uint32_t)c * 16u, 0);
            const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
            const uint32_t zw[4] = {zv.x, zv.y, zv.z, zv.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int el = c * 8 + j;                  // flat [col][group] element
                const int col = el / NG, g = el - col * NG;
                lds_s[g * kLwCols + col] = (uint16_t)(sw[j >> 1] >> (16 * (j & 1)));
                lds_z[g * kLwCols + col] = (uint16_t)(zw[j >> 1] >> (16 * (j & 1)));
            }
        }
    }

    // ---- weight loads: tile ns covers columns wcol + 16 ns .. + 15
    const rsrc_t rq = make_rsrc(p.q, (uint32_t)N * (uint32_t)(K / 2));
    // tile ns's lane offset is tile 0's plus 16 ns rows (scalar); tiles past
    // N (a multiple of 16) read nothing
    const uint32_t wvoff0 = wq_lane_off<G, TL>(wcol + lrow, lane, K);
    const uint32_t wtile = 16u * (uint32_t)(K / 2);
    Frag<G> bq[P][kLwNs];
    auto issue_w = [&](int st, int s) {
#pragma unroll
        for (int ns = 0; ns < kLwNs; ++ns)
            bq[st][ns] = load_frag<G, NT>(rq, s < NG && wcol + 16 * ns < N ? wvoff0 : kOutOfRange,
                                          wq_group_off<G, TL>(s) + (uint32_t)ns * wtile);
    };
    // ---- activation slices: thread -> (row tid / SEGS + i * rows per pass,
    // segment tid % SEGS); each thread's row offsets, 2^31 (past any x,
    // whatever the step adds) for rows past T; the step enters as the
    // scalar offset
    const rsrc_t ra = make_rsrc(p.a_src, (uint32_t)T * (uint32_t)K * 2u);
    const int xseg = tid % SEGS;
    constexpr int kRowsPerPass = kLwThreads / SEGS;
    auto xoff = [&](int i) -> uint32_t {
        const int r = row0 + tid / SEGS + i * kRowsPerPass;
        return r < T ? (uint32_t)r * (uint32_t)K * 2u + (uint32_t)xseg * 16u : 0x80000000u;
    };
    // a slice goes in two halves of XLD / 2 loads per thread, each loaded
    // half a step before it is staged
    constexpr int XH = XLD / 2;
    static_assert(XLD % 2 == 0, "activation halves");
    uint4 xr[XH];
    auto issue_x = [&](int s, int half) {
#pragma unroll
        for (int i = 0; i < XH; ++i)
            xr[i] = s < NG ? load16(ra, xoff(half * XH + i), (uint32_t)s * G * 2u) : make_uint4(0u, 0u, 0u, 0u);
    };
    auto stage_x = [&](int buf, int half) {
        uint4 *xb = lds_x + buf * kLwRows * SEGS;
#pragma unroll
        for (int i = 0; i < XH; ++i) {
            const int r = tid / SEGS + (half * XH + i) * kRowsPerPass;
            xb[r * SEGS + lw_slot<SEGS>(r, xseg)] = xr[i];
        }
    };

#pragma unroll
    for (int s = 0; s < P; ++s)
        issue_w(s, s);
    issue_x(0, 0);
    stage_x(0, 0);
    issue_x(0, 1);
    stage_x(0, 1);
    issue_x(1, 0);
    __syncthreads();                             // scales, zeros and slice 0 in LDS

    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc[kLwMs][kLwNs];
#pragma unroll
    for (int ms = 0; ms < kLwMs; ++ms)
#pragma unroll
        for (int ns = 0; ns < kLwNs; ++ns)
            acc[ms][ns] = zero4;
    // (16-row blocks past T multiply zeros: a ragged last block costs its
    // MFMAs, the full blocks no branches)

    auto step = [&](int s, int st) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);       // nothing moves between steps
        int loff = 0;                                    // opaque per step: no hoisted reads
        asm volatile("" : "+v"(loff));
        // the slice's buffer as an opaque base, so that the row offsets of the
        // fragment reads stay immediate (the second buffer starts past what
        // an LDS instruction's offset field reaches)
        int xbase = (s & 1) * kLwRows * SEGS;
        asm volatile("" : "+v"(xbase));
        const uint4 *xb = lds_x + xbase;
        {
            f16x2 cmix[kLwNs], s2[kLwNs];
#pragma unroll
            for (int ns = 0; ns < kLwNs; ++ns) {
                const int c = loff + s * kLwCols + lcol + 16 * ns + lrow;   // the lane's column
                const uint32_t zb = lds_z[c], sb = lds_s[c];
                cmix[ns] = as_h2(zb | (zb << 16)) + f16x2{(_Float16)1024.0f, (_Float16)64.0f};
                s2[ns] = as_h2(sb | (sb << 16));
            }
            // the step's (k-slice t, 16-row block) pairs in order, each one
            // activation fragment feeding both tiles' MFMAs; fragments are
            // read kAhead pairs before use (LDS latency is several pairs'
            // MFMA time), and between the MFMAs of k-slice t the two tiles'
            // weight fragments of t + 1 are formed
            constexpr int kPairs = kWords * kLwMs;
            constexpr int kAheadA = 4;
            auto aread = [&](int i) {
                const int t = i / kLwMs, r = (i % kLwMs) * 16 + lrow;   // row within the block
                return __builtin_bit_cast(f16x8, xb[r * SEGS + lw_slot<SEGS>(r, quarter * kWords + t)]);
            };
            f16x8 bop[kLwNs], bnext[kLwNs];
#pragma unroll
            for (int ns = 0; ns < kLwNs; ++ns)
                bop[ns] = dequant8_scaled(frag_word<G>(bq[st][ns], 0), cmix[ns], s2[ns]);
            f16x8 af[kPairs];
#pragma unroll
            for (int i = 0; i < kAheadA; ++i)
                af[i] = aread(i);
#pragma unroll
            for (int i = 0; i < kPairs; ++i) {
                const int t = i / kLwMs, ms = i % kLwMs;
                if (t == kWords / 2 && ms == 0) {
                    // the first half of the next slice is in: stage it, load the second
                    stage_x((s + 1) & 1, 0);
                    issue_x(s + 1, 1);
                }
                if (i + kAheadA < kPairs)
                    af[i + kAheadA] = aread(i + kAheadA);
#pragma unroll
                for (int ns = 0; ns < kLwNs; ++ns)
                    acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bop[ns], af[i], acc[ms][ns], 0, 0, 0);
                constexpr int kPer = kLwMs / kLwNs;          // blocks per next fragment
                if (t + 1 < kWords && ms % kPer == kPer - 1) {
                    const int ns = ms / kPer;
                    bnext[ns] = dequant8_scaled(frag_word<G>(bq[st][ns], t + 1), cmix[ns], s2[ns]);
                }
                if (t + 1 < kWords && ms == kLwMs - 1)
#pragma unroll
                    for (int ns = 0; ns < kLwNs; ++ns)
                        bop[ns] = bnext[ns];
                __builtin_amdgcn_sched_barrier(0);   // keep the reads where they are issued
            }
        }
        issue_w(st, s + P);
        stage_x((s + 1) & 1, 1);
        issue_x(s + 2, 0);
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
    // ns for row ms * 16 + lrow; past N the tile stores nothing, past T the
    // buffer drops the store
    const rsrc_t ry = make_rsrc(p.out, (uint32_t)T * (uint32_t)N * 2u);
#pragma unroll
    for (int ns = 0; ns < kLwNs; ++ns) {
        if (wcol + 16 * ns >= N)
            continue;
#pragma unroll
        for (int ms = 0; ms < kLwMs; ++ms) {
            const int r = row0 + ms * 16 + lrow;
            const uint32_t off = r < T ? ((uint32_t)r * (uint32_t)N + (uint32_t)(wcol + 16 * ns + 4 * quarter)) * 2u
                                       : 0x80000000u;
            store8(ry, off, pack_f16x4(acc[ms][ns]));
        }
    }
}

template <int G, int NGC, bool TL, bool NT>
hipError_t launch_linear_wide_k(const GemmArgs &a, size_t lds, hipStream_t stream)
{
    static size_t allowed = 64 * 1024;             // one per instantiation
    auto kern = linear_wide_kernel<G, NGC, TL, NT>;
    hipError_t err = allow_lds(kern, lds, allowed);
    if (err != hipSuccess)
        return err;
    const int nblocks = (a.n_out + kLwCols - 1) / kLwCols;
    const int nrb = (a.A + kLwRows - 1) / kLwRows;
    const long long blocks = (long long)(nblocks + kXcds - 1) / kXcds * kXcds * nrb;
    if (blocks > INT_MAX)
        return hipErrorInvalidValue;
    kern<<<dim3((unsigned)blocks), dim3(kLwThreads), lds, stream>>>(a);
    return hipGetLastError();
}

// The many-row dense linear: rows in blocks of 256, each weight dequantised
// once per block; non-temporal tiled weights when there is one block.
template <int G>
hipError_t launch_linear_wide_g(const GemmArgs &a, size_t lds, hipStream_t stream)
{
    const bool one_block = a.A <= kLwRows;
    if constexpr (G == 128) {
        if (a.K == kLinearUnrolledGroups * 128) {
            if (!a.tiled)
                return launch_linear_wide_k<G, kLinearUnrolledGroups, false, false>(a, lds, stream);
            return one_block ? launch_linear_wide_k<G, kLinearUnrolledGroups, true, true>(a, lds, stream)
                             : launch_linear_wide_k<G, kLinearUnrolledGroups, true, false>(a, lds, stream);
        }
    }
    if (!a.tiled)
        return launch_linear_wide_k<G, 0, false, false>(a, lds, stream);
    return one_block ? launch_linear_wide_k<G, 0, true, true>(a, lds, stream)
                     : launch_linear_wide_k<G, 0, true, false>(a, lds, stream);
}

}  // namespace

bool linear_wide_fits(const GemmArgs &a, int g)
{
    if (reinterpret_cast<uintptr_t>(a.out) % 8 != 0)
        return false;
    const size_t lds = g == 128 ? linear_wide_lds_bytes<128>(a.K) : linear_wide_lds_bytes<64>(a.K);
    return lds <= kMaxWideLds;
}

hipError_t launch_linear_wide(const GemmArgs &a, int g, hipStream_t stream)
{
    if (g == 128)
        return launch_linear_wide_g<128>(a, linear_wide_lds_bytes<128>(a.K), stream);
    return launch_linear_wide_g<64>(a, linear_wide_lds_bytes<64>(a.K), stream);
}

}  // namespace dgw4

// Grouped W4A16 GEMMs of the routed-expert layer: gate_up with the gated
// activation in its epilogue, and down.
//
// Follows the "dg-w4-kernels" card, "Grouped MoE" (one launch covers every
// expert; the activation is folded into the first GEMM's epilogue) and
// "W4A16" (the GEMM reads packed nibbles and dequantises inline); the model
// card, "Checkpoint format" (w = (q - z) * s, one scale/zero per group along
// K, byte j = q[2j] | q[2j+1] << 4; the group size matches the K step so one
// scale and zero load serves a whole K chunk); and the Part 2 blog,
// "Quantisation alone leaves a sparse execution problem" and "The final best
// W4 MoE kernel" (assignments sorted by expert and padded to 32-row blocks).
//
// gfx950 design
// -------------
// Grid (N-block, tile): tile = one 32-row block of the padded assignment list
// (one expert), N-block = 4 waves x 2 MFMA column tiles of 16 weight rows.
// Tiles past the device-side total exit at once, so the grid is static and
// the host never reads the routing.
//
// Each wave streams its 32 weight rows once, straight from the canonical
// packed layout: per group and column tile a lane loads g/8 bytes (a 16-byte
// dwordx4 for g=128, 8 bytes for g=64) of one weight row; the four lane
// groups of 16 cover one whole group of that row. Loads run D groups ahead in
// registers and stay in flight across the workgroup barriers.
//
// Dequantisation builds exact fp16 integers in registers: for a 32-bit word
// holding nibbles n0..n7, (w & 0x000F000F) | 0x64006400 is the fp16 pair
// (1024 + n0, 1024 + n4) and (w & 0x00F000F0) | 0x54005400 is (64 + n1,
// 64 + n5); the same on w >> 8 gives n2/n6 and n3/n7. One packed fp16
// subtract of (1024 + z) or (64 + z) leaves the exact integers q - z. The
// MFMA B operand therefore holds K positions in the order
// [0,4,1,5,2,6,3,7] within each 8; a contraction is unchanged by the same
// permutation on both operands, so the activation rows are stored in LDS
// with that same order and no weight preshuffle is needed.
//
// v_mfma_f32_16x16x32_f16 accumulates one group (g/32 MFMAs) into a fresh
// fp32 partial; the group's scale is applied once per output in fp32
// (acc += s * partial). The scale never touches an fp16 weight, so the only
// rounding is the fp32 accumulation.
//
// Activations: the tile's 32 rows are staged through LDS in K chunks of
// D groups (gathered rows of x for gate_up, rows of H for down), loaded into
// registers one chunk ahead. Scale and zero point of each (row, group) are
// loaded with the weight fragment, D groups ahead.
//
// Epilogues: gate_up computes gelu_tanh(gate) * up in fp32 and writes H in
// fp16 at the tile's padded row; down writes fp32 Y at the assignment's flat
// slot t * topk + k, which the combine reads in ascending k.
#include "dgw4_internal.hpp"

namespace dgw4 {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTilesPerWave = 2;                        // MFMA column tiles per wave
constexpr int kRowsPerWG = kWaves * kTilesPerWave * 16; // weight rows per workgroup
constexpr int kStages = 4;                              // groups in flight per wave

// Activation chunk geometry for group size G: one chunk = kStages groups.
template <int G>
struct Chunk {
    static constexpr int K = kStages * G;                 // activation K per LDS chunk
    static constexpr int Seg = K / 8;                     // 16-byte segments per row
    static constexpr int Pitch = Seg + 1;                 // +16 B per row: spreads banks
    static constexpr int Lds = kBlockM * Pitch;           // uint4 entries
    static constexpr int Loads = kBlockM * Seg / kThreads;  // 16-byte loads per thread
};

template <int G>
struct Frag;                     // one lane's share of one group of one weight row
template <>
struct Frag<128> { uint4 v; };   // 16 bytes = 32 nibbles
template <>
struct Frag<64> { uint2 v; };    // 8 bytes = 16 nibbles

template <int G>
__device__ inline Frag<G> load_frag(const uint8_t *p)
{
    Frag<G> f;
    if constexpr (G == 128)
        f.v = *reinterpret_cast<const uint4 *>(p);
    else
        f.v = *reinterpret_cast<const uint2 *>(p);
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

// 8 nibbles -> 8 exact fp16 values (q - z) in K order [0,4,1,5,2,6,3,7].
__device__ inline f16x8 dequant8(uint32_t w, f16x2 c1024, f16x2 c64)
{
    const uint32_t w8 = w >> 8;
    const f16x2 a = as_h2((w & 0x000F000Fu) | 0x64006400u) - c1024;
    const f16x2 b = as_h2((w & 0x00F000F0u) | 0x54005400u) - c64;
    const f16x2 c = as_h2((w8 & 0x000F000Fu) | 0x64006400u) - c1024;
    const f16x2 d = as_h2((w8 & 0x00F000F0u) | 0x54005400u) - c64;
    f16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

// 8 consecutive fp16 values -> the same values in order [0,4,1,5,2,6,3,7].
__device__ inline uint4 permute8(uint4 v)
{
    uint4 o;
    o.x = (v.x & 0xFFFFu) | (v.z << 16);
    o.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
    o.z = (v.y & 0xFFFFu) | (v.w << 16);
    o.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
    return o;
}

__device__ inline float gelu_tanh(float v)
{
    const float k0 = 0.7978845608028654f;   // sqrt(2/pi)
    const float k1 = 0.044715f;
    return 0.5f * v * (1.0f + tanhf(k0 * (v + k1 * v * v * v)));
}

// Weight row (within the expert) of column tile tt of wave w in N-block nb.
template <bool GATED>
__device__ inline int weight_row(int nb, int w, int tt, int n_out)
{
    if constexpr (GATED)    // tile 0: gate rows, tile 1: the matching up rows
        return nb * (kWaves * 16) + w * 16 + tt * n_out;
    else
        return nb * (kWaves * kTilesPerWave * 16) + w * (kTilesPerWave * 16) + tt * 16;
}

template <int G, bool GATED>
__global__ void __launch_bounds__(kThreads) moe_gemm_kernel(GemmArgs p)
{
    constexpr int D = kStages;
    constexpr int kChunkK = Chunk<G>::K;
    constexpr int kSegPerRow = Chunk<G>::Seg;
    constexpr int kPitch = Chunk<G>::Pitch;
    constexpr int kStageLoads = Chunk<G>::Loads;
    constexpr int kWords = G / 32;          // MFMA K steps per group = words per fragment
    const int nb = blockIdx.x;
    const int tile = blockIdx.y;
    const int total = *p.num_padded;
    if (tile * kBlockM >= total)
        return;
    const int e = p.tile_expert[tile];
    const int row0 = tile * kBlockM;        // first padded row of this tile
    const int valid = min(kBlockM, p.counts[e] - (row0 - p.offsets[e]));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int K = p.K;
    const int NG = K / G;
    const int NC = (K + kChunkK - 1) / kChunkK;

    __shared__ uint4 lds_a[Chunk<G>::Lds];  // [kBlockM][kPitch], K order permuted per 8

    // columns owned by this wave; a wave past the edge only helps with staging
    const int col_first = GATED ? nb * (kWaves * 16) + wave * 16
                                : nb * (kWaves * kTilesPerWave * 16) + wave * (kTilesPerWave * 16);
    const bool wave_live = col_first < p.n_out;

    // ---- activation rows of the tile: source row per tile row, -1 past `valid`
    // gate_up: x row of token sorted_id / topk; down: H row at the padded position
    __shared__ int s_src[kBlockM];
    if (tid < kBlockM) {
        int src = -1;
        if (tid < valid) {
            if constexpr (GATED)
                src = p.sorted_ids[row0 + tid] / p.topk;
            else
                src = row0 + tid;
        }
        s_src[tid] = src;
    }
    __syncthreads();
    // all loads below are unconditional with addresses clamped into the source;
    // rows past `valid` and K past the end become zeros when stored to LDS
    const uint16_t *arow[kStageLoads];
    int aseg[kStageLoads];
    bool arow_ok[kStageLoads];
#pragma unroll
    for (int i = 0; i < kStageLoads; ++i) {
        const int lin = i * kThreads + tid;
        const int src = s_src[lin / kSegPerRow];
        aseg[i] = lin % kSegPerRow;
        arow_ok[i] = src >= 0;
        arow[i] = p.a_src + (size_t)(src >= 0 ? src : 0) * K;
    }
    uint4 xr[kStageLoads];
    auto load_chunk = [&](int c) {
#pragma unroll
        for (int i = 0; i < kStageLoads; ++i) {
            const int k = min(c * kChunkK + aseg[i] * 8, K - 8);
            xr[i] = *reinterpret_cast<const uint4 *>(arow[i] + k);
        }
    };
    auto store_chunk = [&](int c) {
#pragma unroll
        for (int i = 0; i < kStageLoads; ++i) {
            const int lin = i * kThreads + tid;
            // zero by mask, not by a branch, so the load is never sunk into one
            const uint32_t keep =
                (arow_ok[i] && (c * kChunkK + aseg[i] * 8 < K)) ? 0xFFFFFFFFu : 0u;
            uint4 v = permute8(xr[i]);
            v.x &= keep;
            v.y &= keep;
            v.z &= keep;
            v.w &= keep;
            lds_a[(lin / kSegPerRow) * kPitch + aseg[i]] = v;
        }
    };

    // ---- weight fragments: lane -> (row within the column tile, quarter of the group)
    const int lrow = lane & 15;
    const int quarter = lane >> 4;
    const size_t expert_row0 = (size_t)e * p.n_w;
    const uint8_t *wptr[kTilesPerWave];
    const uint16_t *sptr[kTilesPerWave];
    const uint16_t *zptr[kTilesPerWave];
#pragma unroll
    for (int tt = 0; tt < kTilesPerWave; ++tt) {
        int wr = weight_row<GATED>(nb, wave, tt, p.n_out) + lrow;
        if (!wave_live)
            wr = 0;                           // keeps idle waves' pointers in bounds
        wptr[tt] = p.q + (expert_row0 + wr) * (size_t)(K / 2) + quarter * (G / 8);
        sptr[tt] = p.s + (expert_row0 + wr) * (size_t)NG;
        zptr[tt] = p.z + (expert_row0 + wr) * (size_t)NG;
    }
    Frag<G> bq[D][kTilesPerWave];
    uint32_t bs[D][kTilesPerWave], bz[D][kTilesPerWave];
    auto prefetch = [&](int s, int gi) {      // group gi (clamped) into stage s
        gi = min(gi, NG - 1);
#pragma unroll
        for (int tt = 0; tt < kTilesPerWave; ++tt) {
            bq[s][tt] = load_frag<G>(wptr[tt] + gi * (G / 2));
            bs[s][tt] = sptr[tt][gi];
            bz[s][tt] = zptr[tt][gi];
        }
    };

    // activation chunk 0 first, so storing it to LDS waits for these loads only.
    // Idle waves (past the N edge) run the same loads and math on row 0 of the
    // expert and store nothing: no branch separates the loads from their uses.
    load_chunk(0);
    __builtin_amdgcn_sched_barrier(0);        // keep the activation loads first in issue order
#pragma unroll
    for (int s = 0; s < D; ++s)
        prefetch(s, s);
    store_chunk(0);                           // read only after the loop's first barrier

    f32x4 acc[kTilesPerWave][2];
#pragma unroll
    for (int tt = 0; tt < kTilesPerWave; ++tt)
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
            acc[tt][ms] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool two_blocks = valid > 16;       // second 16-row MFMA block has rows
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    // one group from stage s: dequantise, 2 x g/32 MFMAs per row block, scale fold
    auto group = [&](int s) {
        f16x2 c1024[kTilesPerWave], c64[kTilesPerWave];
        float scale[kTilesPerWave];
#pragma unroll
        for (int tt = 0; tt < kTilesPerWave; ++tt) {
            scale[tt] = (float)__builtin_bit_cast(_Float16, (uint16_t)bs[s][tt]);
            const float zf = (float)__builtin_bit_cast(_Float16, (uint16_t)bz[s][tt]);
            const _Float16 a = (_Float16)(1024.0f + zf);
            const _Float16 b = (_Float16)(64.0f + zf);
            c1024[tt] = f16x2{a, a};
            c64[tt] = f16x2{b, b};
        }
        f32x4 part[kTilesPerWave][2];
#pragma unroll
        for (int t = 0; t < kWords; ++t) {
            f16x8 bop[kTilesPerWave];
#pragma unroll
            for (int tt = 0; tt < kTilesPerWave; ++tt)
                bop[tt] = dequant8(frag_word<G>(bq[s][tt], t), c1024[tt], c64[tt]);
            // this lane's 8 K positions inside the chunk
            const int seg = s * (G / 8) + quarter * (G / 32) + t;
#pragma unroll
            for (int ms = 0; ms < 2; ++ms) {
                if (ms == 1 && !two_blocks)
                    continue;
                const f16x8 aop = __builtin_bit_cast(f16x8, lds_a[(ms * 16 + lrow) * kPitch + seg]);
#pragma unroll
                for (int tt = 0; tt < kTilesPerWave; ++tt)
                    part[tt][ms] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        aop, bop[tt], t == 0 ? zero4 : part[tt][ms], 0, 0, 0);
            }
        }
#pragma unroll
        for (int tt = 0; tt < kTilesPerWave; ++tt)
#pragma unroll
            for (int ms = 0; ms < 2; ++ms) {
                if (ms == 1 && !two_blocks)
                    continue;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[tt][ms][i] += scale[tt] * part[tt][ms][i];
            }
    };

    // all chunks but the last: every group exists, prefetch D groups ahead
    for (int c = 0; c + 1 < NC; ++c) {
        load_chunk(c + 1);                    // registers; written to LDS after compute
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();                      // chunk c is in LDS
#pragma unroll
        for (int s = 0; s < D; ++s) {
            group(s);
            prefetch(s, (c + 1) * D + s);
        }
        __syncthreads();                      // everyone is done reading chunk c
        store_chunk(c + 1);
    }
    // last chunk: groups may stop early, nothing left to prefetch
    __syncthreads();
#pragma unroll
    for (int s = 0; s < D; ++s)
        if ((NC - 1) * D + s < NG)
            group(s);

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
                const int col = col_first + lrow;
                const float h = gelu_tanh(acc[0][ms][i]) * acc[1][ms][i];
                uint16_t *H = static_cast<uint16_t *>(p.out);
                H[(size_t)(row0 + r) * p.n_out + col] =
                    __builtin_bit_cast(uint16_t, (_Float16)h);
            } else {
                const int fid = p.sorted_ids[row0 + r];
                float *Y = static_cast<float *>(p.out);
#pragma unroll
                for (int tt = 0; tt < kTilesPerWave; ++tt)
                    Y[(size_t)fid * p.n_out + col_first + tt * 16 + lrow] = acc[tt][ms][i];
            }
        }
    }
}

template <int G, bool GATED>
hipError_t launch_gemm(const GemmArgs &a, hipStream_t stream)
{
    const int cols_per_wg = GATED ? kWaves * 16 : kWaves * kTilesPerWave * 16;
    const int nblocks = (a.n_out + cols_per_wg - 1) / cols_per_wg;
    if (a.max_tiles == 0 || nblocks == 0)
        return hipSuccess;
    moe_gemm_kernel<G, GATED><<<dim3(nblocks, a.max_tiles), dim3(kThreads), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up(const GemmArgs &a, int g, hipStream_t stream)
{
    return g == 128 ? launch_gemm<128, true>(a, stream) : launch_gemm<64, true>(a, stream);
}

hipError_t launch_down(const GemmArgs &a, int g, hipStream_t stream)
{
    return g == 128 ? launch_gemm<128, false>(a, stream) : launch_gemm<64, false>(a, stream);
}

}  // namespace dgw4

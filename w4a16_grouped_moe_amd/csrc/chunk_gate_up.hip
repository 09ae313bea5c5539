// gate_up of the routed-expert layer over 128-row chunks: workgroup =
// (chunk of one expert's sorted assignments, 128 gate rows and the matching
// 128 up rows), the chunk's activation rows gathered through the assignment
// ids; H = gelu_tanh(gate) * up stored per chunk row (the many-row body,
// wide_gemm.hpp). Each expert weight is read once per chunk.
//
// Follows the kernel card's "Grouped MoE" section (one launch for every
// expert, the gated activation in the first GEMM's epilogue) and "W4A16";
// the Part 2 blog's "Quantisation alone leaves a sparse execution problem"
// (assignments sorted by expert and padded to a block size, 128 rows here).
#include "wide_gemm.hpp"

namespace dgw4 {
namespace {

// The chunk GEMMs exist for the layer's shape with tiled weights: gate_up
// K = 22 groups of 128, down K = 11 groups of 64 (straight-line K loops).
constexpr int kChunkGuGroups = 22, kChunkGuG = 128;
constexpr int kChunkDnGroups = 11, kChunkDnG = 64;

// Runs the body instance for the wave's count of 16-row blocks (b.nmb,
// 0 .. kChunkM / 16); the instances share every barrier, so waves of one
// workgroup may take different ones.
template <int MODE, int G, int NGC, int N = 0>
__device__ __forceinline__ void chunk_body(const GemmArgs &p, const WideBlock &b)
{
    if constexpr (N <= kChunkM / 16) {
        if (b.nmb == N)
            wide_body<MODE, G, NGC, true, false, N>(p, b);
        else
            chunk_body<MODE, G, NGC, N + 1>(p, b);
    }
}

// Grid of a chunk GEMM: every possible chunk (max_tiles, rounded up to the
// XCD count) times the column blocks.
long long chunk_grid(const GemmArgs &a, int block_cols)
{
    const long long ncb = (a.n_out + block_cols - 1) / block_cols;
    return (long long)(a.max_tiles + kXcds - 1) / kXcds * kXcds * ncb;
}

__global__ void __launch_bounds__(wide_threads<kModeGateUp>())
__attribute__((amdgpu_waves_per_eu(2))) chunk_gate_up_kernel(GemmArgs p)
{
    const WideBlock b = wide_block<kModeGateUp>(p, kChunkGuGroups);
    if (b.nmb < 0)
        return;
    chunk_body<kModeGateUp, kChunkGuG, kChunkGuGroups>(p, b);
}

}  // namespace

bool chunk_gemms_fit(const GemmArgs &gu, int gu_g, const GemmArgs &dn, int dn_g)
{
    const int m = gu.n_out, d = dn.n_out;
    if (gu_g != kChunkGuG || gu.K != kChunkGuGroups * kChunkGuG || dn_g != kChunkDnG ||
        dn.K != kChunkDnGroups * kChunkDnG || gu.K != d || dn.K != m || !gu.tiled || !dn.tiled)
        return false;
    // 16-row weight tiles; 16-byte runs of scales and zero points (every
    // run starts at a multiple of 128 rows of one expert, the up rows m rows
    // in); 8-byte output stores
    if (m % 16 != 0 || d % 16 != 0 || (long long)m * kChunkGuGroups % 8 != 0 ||
        (long long)d * kChunkDnGroups % 8 != 0)
        return false;
    if (reinterpret_cast<uintptr_t>(gu.out) % 8 != 0 || reinterpret_cast<uintptr_t>(dn.out) % 8 != 0)
        return false;
    // 32-bit offsets into x, H, Y and one expert's weights
    const long long hbytes = (long long)gu.max_tiles * kChunkM * m * 2;
    return (long long)gu.a_rows * d * 2 < (1LL << 31) && hbytes < (1LL << 31) &&
           (long long)dn.A * d * 2 < (1LL << 31) && (long long)gu.n_w * (d / 2) < (1LL << 31) &&
           dn.a_rows >= gu.max_tiles * kChunkM;
}

hipError_t launch_chunk_gate_up(const GemmArgs &gu, hipStream_t stream)
{
    static size_t allowed = 64 * 1024;
    return launch_wide<kModeGateUp>(chunk_gate_up_kernel, wide_lds_bytes<kModeGateUp, kChunkGuG>(gu.K), allowed,
                       chunk_grid(gu, wide_cols<kModeGateUp>() / 2), gu, stream);
}

}  // namespace dgw4

// down of the routed-expert layer over 128-row chunks: workgroup = (chunk of
// one expert's H rows, 256 down rows = output columns); each row's output
// goes to its assignment's row of Y (the many-row body, wide_gemm.hpp).
// Each expert weight is read once per chunk.
//
// Follows the kernel card's "Grouped MoE" and "W4A16" sections and the Part
// 2 blog's "Quantisation alone leaves a sparse execution problem".
#include "wide_gemm.hpp"

namespace dgw4 {
namespace {

constexpr int kChunkDnGroups = 11, kChunkDnG = 64;   // down K = 704 at g = 64

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

__global__ void __launch_bounds__(wide_threads<kModeDown>())
__attribute__((amdgpu_waves_per_eu(2))) chunk_down_kernel(GemmArgs p)
{
    const WideBlock b = wide_block<kModeDown>(p, kChunkDnGroups);
    if (b.nmb < 0)
        return;
    chunk_body<kModeDown, kChunkDnG, kChunkDnGroups>(p, b);
}

}  // namespace

hipError_t launch_chunk_down(const GemmArgs &dn, hipStream_t stream)
{
    static size_t allowed = 64 * 1024;
    return launch_wide<kModeDown>(chunk_down_kernel, wide_lds_bytes<kModeDown, kChunkDnG>(dn.K), allowed,
                       chunk_grid(dn, wide_cols<kModeDown>()), dn, stream);
}

}  // namespace dgw4

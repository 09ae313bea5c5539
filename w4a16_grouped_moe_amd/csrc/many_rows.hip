// Dense W4A16 linear over many rows (y = x * deq(W)^T with at least 128
// rows): 256-row blocks, each weight formed once per block and fed to all
// its rows (the many-row body, wide_gemm.hpp). The few-row kernel (32-row
// tiles) lives with the GEMM bodies it shares.
//
// Follows the kernel card's "W4A16" section: w4a16_linear(x, qw, scale,
// zero) equals F.linear(x, dequant(W)), the weights dequantised in registers
// into fp16 MFMA fragments.
#include "wide_gemm.hpp"

namespace dgw4 {
namespace {

constexpr int kLinearUnrolledGroups = 22;        // K = 2816 at g = 128: straight-line code

template <int G, int NGC, bool TL, bool NT>
__global__ void __launch_bounds__(kLwThreads)
__attribute__((amdgpu_waves_per_eu(2))) linear_wide_kernel(GemmArgs p)
{
    const WideBlock b = wide_block<kModeLinear>(p, NGC > 0 ? NGC : p.K / G);
    if (b.nmb < 0)
        return;
    wide_body<kModeLinear, G, NGC, TL, NT, kLwRows / 16>(p, b);
}

template <int G, int NGC, bool TL, bool NT>
hipError_t launch_linear_wide_k(const GemmArgs &a, size_t lds, hipStream_t stream)
{
    static size_t allowed = 64 * 1024;             // one per instantiation
    const int nblocks = (a.n_out + kLwCols - 1) / kLwCols;
    const int nrb = (a.A + kLwRows - 1) / kLwRows;
    const long long blocks = (long long)(nblocks + kXcds - 1) / kXcds * kXcds * nrb;
    return launch_wide<kModeLinear>(linear_wide_kernel<G, NGC, TL, NT>, lds, allowed, blocks, a, stream);
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
    const size_t lds = g == 128 ? wide_lds_bytes<kModeLinear, 128>(a.K) : wide_lds_bytes<kModeLinear, 64>(a.K);
    return lds <= kMaxWideLds;
}

hipError_t launch_linear_wide(const GemmArgs &a, int g, hipStream_t stream)
{
    if (g == 128)
        return launch_linear_wide_g<128>(a, wide_lds_bytes<kModeLinear, 128>(a.K), stream);
    return launch_linear_wide_g<64>(a, wide_lds_bytes<kModeLinear, 64>(a.K), stream);
}

}  // namespace dgw4

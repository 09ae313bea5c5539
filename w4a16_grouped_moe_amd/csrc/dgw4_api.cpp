// C-ABI entry points of libdgw4 (declared in include/dgw4.h).
//
// Host side only: argument validation, workspace layout and the launch
// sequence. No allocation, no host synchronisation, no state between calls.
#include "dgw4.h"

#include "dgw4_internal.hpp"

#include <limits.h>

namespace {

constexpr size_t kAlign = 256;
// LDS of one CU (160 KB); a GEMM workgroup must fit in it.
constexpr size_t kMaxGemmLds = 160 * 1024;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool group_supported(int g) { return g == 64 || g == 128; }

// Splits a GEMM group-size argument into the group size and the layout flag;
// false for flag bits other than DGW4_WEIGHTS_TILED.
bool split_group(int arg, int &g, int &tiled)
{
    if (arg < 0 || (arg & ~(DGW4_WEIGHTS_TILED | 0xFFFF)) != 0)
        return false;
    g = arg & 0xFFFF;
    tiled = (arg & DGW4_WEIGHTS_TILED) != 0;
    return true;
}

// The layer's row-block choice carried by the gate_up group argument:
// 0 (the library picks), DGW4_ROWS_TILES or DGW4_ROWS_CHUNKS; the bits are
// removed from arg. False for both bits together.
bool split_rows(int &arg, int &rows)
{
    rows = arg & (DGW4_ROWS_TILES | DGW4_ROWS_CHUNKS);
    arg &= ~(DGW4_ROWS_TILES | DGW4_ROWS_CHUNKS);
    return rows != (DGW4_ROWS_TILES | DGW4_ROWS_CHUNKS);
}

// With no choice given, the layer runs on 128-row chunks once the experts
// hold this many assignments each on average (and the chunk GEMMs exist for
// the shape), else on 32-row tiles. Measured at the layer's shape with 128
// experts, top-8: the two are level at 22 (T = 352); below, the tiles are
// faster (99 against 128 us at 16), above, the chunks (139 against 171 us at
// 24, 198 against 263 at 64).
constexpr long long kChunkMinMeanRows = 22;

bool overlap(const void *a, const void *b, size_t bytes)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + bytes && y < x + bytes;
}

thread_local hipError_t g_last_hip = hipSuccess;   // last failed HIP call of this thread

int from_hip(hipError_t e)
{
    if (e == hipSuccess)
        return DGW4_OK;
    g_last_hip = e;
    return DGW4_ERR_HIP;
}

// Workspace of one forward call: alignment buffers (for block_m-row
// blocks), the gated intermediate H (fp16, one row per padded assignment) and
// the per-assignment expert outputs Y (fp16, one row per flat assignment id;
// `halves` such arrays). On 32-row tiles at the layer's shape, the layer
// kernel aligns inside its workgroups, keeps H in LDS and writes two Y
// arrays, the partials of the two halves of down's contraction; on 128-row
// chunks the alignment, H and one Y are used.
struct Layout {
    size_t counts, offsets, num_padded, tile_expert, tile_info, tile_order, sorted_ids, h, y, rids, rw,
        total;
};

Layout layout(long long A, int T, int E, int d, int m, long long cap, int block_m, int halves)
{
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = round_up(off + bytes);
        return at;
    };
    L.counts = take(sizeof(int32_t) * (size_t)E);
    L.offsets = take(sizeof(int32_t) * (size_t)(E + 1));
    L.num_padded = take(sizeof(int32_t));
    L.tile_expert = take(sizeof(int32_t) * (size_t)(cap / block_m));
    L.tile_info = take(sizeof(int2) * (size_t)(cap / block_m));
    L.tile_order = take(sizeof(int32_t) * (size_t)(cap / block_m));
    L.sorted_ids = take(sizeof(int32_t) * (size_t)cap);
    L.h = take(sizeof(uint16_t) * (size_t)cap * (size_t)m);
    L.y = take((size_t)halves * sizeof(uint16_t) * (size_t)A * (size_t)d);
    L.rids = take(sizeof(int32_t) * (size_t)A);       // the router's output (routed forward)
    L.rw = take(sizeof(float) * (size_t)A);
    L.total = off;
    return L;
}

}  // namespace

extern "C" {

const char *dgw4_status_string(int status)
{
    switch (status) {
    case DGW4_OK: return "DGW4_OK";
    case DGW4_ERR_INVALID_ARG: return "DGW4_ERR_INVALID_ARG";
    case DGW4_ERR_UNSUPPORTED: return "DGW4_ERR_UNSUPPORTED";
    case DGW4_ERR_WORKSPACE: return "DGW4_ERR_WORKSPACE";
    case DGW4_ERR_HIP: return "DGW4_ERR_HIP";
    default: return "DGW4_UNKNOWN_STATUS";
    }
}

int dgw4_version(void) { return 100; }   // 0.1.0

const char *dgw4_last_error(void)
{
    return g_last_hip == hipSuccess ? "no HIP error" : hipGetErrorString(g_last_hip);
}

int dgw4_quantize_rtn(const float *w, int E, int N, int K, int g, uint8_t *q, uint16_t *s,
                      uint16_t *z, void *stream)
{
    if (!w || !q || !s || !z)
        return DGW4_ERR_INVALID_ARG;
    if (E < 1 || N < 1 || K < 2 || (K % 2) != 0 || g < 1)
        return DGW4_ERR_INVALID_ARG;
    if (!group_supported(g))
        return DGW4_ERR_UNSUPPORTED;
    if (K % g != 0 || !aligned(w, 8))
        return DGW4_ERR_INVALID_ARG;
    const long long groups = (long long)E * N * (K / g);
    return from_hip(dgw4::launch_quantize_rtn(w, groups, g, q, s, z, (hipStream_t)stream));
}

size_t dgw4_align_capacity(int T, int topk, int E, int block_m)
{
    if (T < 0 || topk < 1 || E < 1 || block_m < 1)
        return 0;
    const long long cap = (long long)T * topk + (long long)E * (block_m - 1);
    return cap > INT_MAX ? 0 : (size_t)cap;
}

int dgw4_align(const int32_t *topk_ids, int T, int topk, int E, int block_m, int32_t *counts,
               int32_t *offsets, int32_t *sorted_ids, int32_t *tile_expert, int32_t *num_padded,
               void *stream)
{
    if (T < 0 || topk < 1 || E < 1 || E > dgw4::kMaxExperts)
        return DGW4_ERR_INVALID_ARG;
    if (block_m != 16 && block_m != 32 && block_m != 64)
        return DGW4_ERR_INVALID_ARG;
    if ((T > 0 && !topk_ids) || !counts || !offsets || !sorted_ids || !tile_expert || !num_padded)
        return DGW4_ERR_INVALID_ARG;
    const size_t cap = dgw4_align_capacity(T, topk, E, block_m);
    if (cap == 0)
        return DGW4_ERR_INVALID_ARG;
    return from_hip(dgw4::launch_align(topk_ids, T * topk, E, block_m, (long long)cap, counts,
                                       offsets, sorted_ids, tile_expert, num_padded, nullptr,
                                       nullptr, (hipStream_t)stream));
}

namespace {

// The row blocks of the layer's expert GEMMs (kBlockM or kChunkM) for the
// GEMMs' shapes (gu, dn without buffers) and the caller's choice; -1 for
// chunks asked for where they do not exist.
int pick_rows(dgw4::GemmArgs gu, int gu_g, dgw4::GemmArgs dn, int dn_g, int rows, int E,
              size_t cap128)
{
    gu.max_tiles = (int)(cap128 / dgw4::kChunkM);
    dn.max_tiles = gu.max_tiles;
    dn.a_rows = (int)cap128;
    const bool chunk_ok = dgw4::chunk_gemms_fit(gu, gu_g, dn, dn_g);
    if (rows == DGW4_ROWS_CHUNKS)
        return chunk_ok ? dgw4::kChunkM : -1;
    const bool chunks = rows == 0 && chunk_ok && (long long)gu.A >= kChunkMinMeanRows * E;
    return chunks ? dgw4::kChunkM : dgw4::kBlockM;
}

// The forward (with_combine) or its expert stages alone; events (5 or null)
// are recorded before the first kernel and after each stage: alignment,
// gate_up, down, combine. At the layer's shape the first three are one
// launch, recorded by marks 1, 2 and 3 together after it.
int moe_forward_impl(const uint16_t *x, const int32_t *topk_ids, const float *topk_w, int T,
                     int topk, int E, int d, int m, const uint8_t *gu_q, const uint16_t *gu_s,
                     const uint16_t *gu_z, int gu_garg, const uint8_t *dn_q, const uint16_t *dn_s,
                     const uint16_t *dn_z, int dn_garg, void *workspace, size_t *ws_bytes,
                     uint16_t *out, void *stream, void *const *events, int n_events,
                     bool with_combine, const float *router_logits = nullptr)
{
    int gu_g = 0, dn_g = 0, gu_tiled = 0, dn_tiled = 0, rows = 0;
    if (!split_rows(gu_garg, rows) || !split_group(gu_garg, gu_g, gu_tiled) ||
        !split_group(dn_garg, dn_g, dn_tiled))
        return DGW4_ERR_INVALID_ARG;
    if (events && n_events != 5)
        return DGW4_ERR_INVALID_ARG;
    if (events)
        for (int i = 0; i < 5; ++i)
            if (!events[i])
                return DGW4_ERR_INVALID_ARG;
    if (!ws_bytes)
        return DGW4_ERR_INVALID_ARG;
    if (T < 0 || E < 1 || E > dgw4::kMaxExperts || topk < 1 || topk > E || d < 1 || m < 1)
        return DGW4_ERR_INVALID_ARG;
    if (gu_g < 1 || dn_g < 1)
        return DGW4_ERR_INVALID_ARG;
    if (!group_supported(gu_g) || !group_supported(dn_g))
        return DGW4_ERR_UNSUPPORTED;
    if (d % gu_g != 0 || m % dn_g != 0)
        return DGW4_ERR_INVALID_ARG;
    const long long A = (long long)T * topk;
    const size_t cap32 = dgw4_align_capacity(T, topk, E, dgw4::kBlockM);
    const size_t cap128 = dgw4_align_capacity(T, topk, E, dgw4::kChunkM);
    if (cap32 == 0 || cap128 == 0 || A > INT_MAX)
        return DGW4_ERR_INVALID_ARG;
    if (dgw4::gemm_lds_bytes(true, d, gu_g) > kMaxGemmLds ||
        dgw4::gemm_lds_bytes(false, m, dn_g) > kMaxGemmLds || m > dgw4::down_max_k() ||
        d / gu_g > dgw4::gate_up_max_groups())
        return DGW4_ERR_UNSUPPORTED;

    // the GEMMs' shapes; the buffers are filled in below
    dgw4::GemmArgs gu{};
    gu.topk = topk;
    gu.A = (int)A;
    dgw4::GemmArgs dn = gu;
    gu.a_rows = T;
    gu.K = d;
    gu.n_w = 2 * m;
    gu.n_out = m;
    gu.tiled = gu_tiled;
    dn.K = m;
    dn.n_w = d;
    dn.n_out = d;
    dn.tiled = dn_tiled;

    // the row blocks: 128-row chunks where asked for or where the experts hold
    // many rows each (and the chunk GEMMs exist for the shape), else 32-row
    // tiles
    const int pick = pick_rows(gu, gu_g, dn, dn_g, rows, E, cap128);
    if (pick < 0)
        return DGW4_ERR_UNSUPPORTED;
    const bool chunks = pick == dgw4::kChunkM;
    const int block_m = chunks ? dgw4::kChunkM : dgw4::kBlockM;
    const size_t cap = chunks ? cap128 : cap32;
    gu.max_tiles = (int)(cap / block_m);
    dn.max_tiles = gu.max_tiles;
    dn.a_rows = (int)cap;
    // the GEMMs address x, H, Y and one expert's packed weights with 32-bit offsets
    if ((long long)T * d * 2 >= (1LL << 31) || (long long)cap * m * 2 >= (1LL << 31) ||
        (long long)2 * m * d / 2 >= (1LL << 31))
        return DGW4_ERR_UNSUPPORTED;
    const bool fused = !chunks && dgw4::layer_fused(gu, gu_g, dn, dn_g, E);
    const Layout L = layout(A, T, E, d, m, (long long)cap, block_m, fused ? 2 : 1);
    if (!workspace) {
        *ws_bytes = L.total;
        return DGW4_OK;
    }
    if (!gu_q || !gu_s || !gu_z || !dn_q || !dn_s || !dn_z)
        return DGW4_ERR_INVALID_ARG;
    if (router_logits && topk > 64)
        return DGW4_ERR_INVALID_ARG;
    if (T > 0 && (!x || (!topk_ids && !router_logits) ||
                  (with_combine && !router_logits && !topk_w) || (with_combine && !out)))
        return DGW4_ERR_INVALID_ARG;
    if (router_logits && !aligned(router_logits, 4))
        return DGW4_ERR_INVALID_ARG;
    if (!aligned(workspace, kAlign) || !aligned(x, 16) || !aligned(gu_q, 16) ||
        !aligned(dn_q, 16) || !aligned(gu_s, 16) || !aligned(gu_z, 16) || !aligned(dn_s, 16) ||
        !aligned(dn_z, 16) || (with_combine && !aligned(out, 8)))
        return DGW4_ERR_INVALID_ARG;
    if (*ws_bytes < L.total)
        return DGW4_ERR_WORKSPACE;
    if (T == 0)
        return DGW4_OK;

    hipStream_t st = (hipStream_t)stream;
    auto mark = [&](int i) {
        return events ? hipEventRecord((hipEvent_t)events[i], st) : hipSuccess;
    };
    char *ws = static_cast<char *>(workspace);
    int32_t *counts = reinterpret_cast<int32_t *>(ws + L.counts);
    int32_t *offsets = reinterpret_cast<int32_t *>(ws + L.offsets);
    int32_t *num_padded = reinterpret_cast<int32_t *>(ws + L.num_padded);
    int32_t *tile_expert = reinterpret_cast<int32_t *>(ws + L.tile_expert);
    int2 *tile_info = reinterpret_cast<int2 *>(ws + L.tile_info);
    int32_t *tile_order = reinterpret_cast<int32_t *>(ws + L.tile_order);
    int32_t *sorted_ids = reinterpret_cast<int32_t *>(ws + L.sorted_ids);
    uint16_t *h = reinterpret_cast<uint16_t *>(ws + L.h);
    uint16_t *y = reinterpret_cast<uint16_t *>(ws + L.y);

    gu.sorted_ids = dn.sorted_ids = sorted_ids;
    gu.tile_info = dn.tile_info = tile_info;
    if (chunks)
        gu.tile_order = dn.tile_order = tile_order;
    gu.a_src = x;
    gu.q = gu_q;
    gu.s = gu_s;
    gu.z = gu_z;
    gu.out = h;
    dn.a_src = h;
    dn.q = dn_q;
    dn.s = dn_s;
    dn.z = dn_z;
    dn.out = y;

    hipError_t err = mark(0);
    if (err != hipSuccess)
        return from_hip(err);
    if (router_logits) {
        // the router's ids and weights into the workspace, then the layer on them
        int32_t *rids = reinterpret_cast<int32_t *>(ws + L.rids);
        float *rw = reinterpret_cast<float *>(ws + L.rw);
        if ((err = dgw4::launch_router(router_logits, T, E, topk, rids, rw, st)) != hipSuccess)
            return from_hip(err);
        topk_ids = rids;
        topk_w = rw;
    }
    if (fused) {
        // alignment, gate_up and down in one launch: marks 1, 2 and 3 all follow it
        if ((err = dgw4::launch_layer(gu, dn, topk_ids, E, st)) != hipSuccess ||
            (err = mark(1)) != hipSuccess || (err = mark(2)) != hipSuccess ||
            (err = mark(3)) != hipSuccess)
            return from_hip(err);
    } else {
        if ((err = dgw4::launch_align(topk_ids, (int)A, E, block_m, (long long)cap, counts,
                                      offsets, sorted_ids, tile_expert, num_padded, tile_info,
                                      chunks ? tile_order : nullptr, st)) != hipSuccess ||
            (err = mark(1)) != hipSuccess)
            return from_hip(err);
        if ((err = chunks ? dgw4::launch_chunk_gate_up(gu, st) : dgw4::launch_gate_up(gu, gu_g, st)) !=
                hipSuccess ||
            (err = mark(2)) != hipSuccess)
            return from_hip(err);
        if ((err = chunks ? dgw4::launch_chunk_down(dn, st) : dgw4::launch_down(dn, dn_g, st)) !=
                hipSuccess ||
            (err = mark(3)) != hipSuccess)
            return from_hip(err);
    }
    if (!with_combine)
        return DGW4_OK;
    if ((err = dgw4::launch_combine(y, fused ? 2 : 1, topk_ids, topk_w, T, topk, E, d, out, st)) !=
            hipSuccess ||
        (err = mark(4)) != hipSuccess)
        return from_hip(err);
    return DGW4_OK;
}

}  // namespace

int dgw4_moe_row_block(int T, int topk, int E, int d, int m, int gu_g, int dn_g)
{
    size_t ws = 0;
    // the forward's own checks (a workspace query launches nothing)
    const int st = moe_forward_impl(nullptr, nullptr, nullptr, T, topk, E, d, m, nullptr, nullptr,
                                    nullptr, gu_g, nullptr, nullptr, nullptr, dn_g, nullptr, &ws,
                                    nullptr, nullptr, nullptr, 0, true);
    if (st != DGW4_OK)
        return -st;
    int gg = 0, rows = 0, g = 0, gt = 0, dgr = 0, dt = 0;
    gg = gu_g;
    split_rows(gg, rows);
    split_group(gg, g, gt);
    split_group(dn_g, dgr, dt);
    dgw4::GemmArgs gu{};
    gu.topk = topk;
    gu.A = T * topk;
    dgw4::GemmArgs dn = gu;
    gu.a_rows = T;
    gu.K = d;
    gu.n_w = 2 * m;
    gu.n_out = m;
    gu.tiled = gt;
    dn.K = m;
    dn.n_w = d;
    dn.n_out = d;
    dn.tiled = dt;
    return pick_rows(gu, g, dn, dgr, rows, E, dgw4_align_capacity(T, topk, E, dgw4::kChunkM));
}

int dgw4_moe_forward_timed(const uint16_t *x, const int32_t *topk_ids, const float *topk_w,
                           int T, int topk, int E, int d, int m, const uint8_t *gu_q,
                           const uint16_t *gu_s, const uint16_t *gu_z, int gu_garg,
                           const uint8_t *dn_q, const uint16_t *dn_s, const uint16_t *dn_z,
                           int dn_garg, void *workspace, size_t *ws_bytes, uint16_t *out,
                           void *stream, void *const *events, int n_events)
{
    return moe_forward_impl(x, topk_ids, topk_w, T, topk, E, d, m, gu_q, gu_s, gu_z, gu_garg, dn_q,
                            dn_s, dn_z, dn_garg, workspace, ws_bytes, out, stream, events, n_events,
                            true);
}

int dgw4_moe_forward(const uint16_t *x, const int32_t *topk_ids, const float *topk_w, int T,
                     int topk, int E, int d, int m, const uint8_t *gu_q, const uint16_t *gu_s,
                     const uint16_t *gu_z, int gu_g, const uint8_t *dn_q, const uint16_t *dn_s,
                     const uint16_t *dn_z, int dn_g, void *workspace, size_t *ws_bytes,
                     uint16_t *out, void *stream)
{
    return moe_forward_impl(x, topk_ids, topk_w, T, topk, E, d, m, gu_q, gu_s, gu_z, gu_g, dn_q,
                            dn_s, dn_z, dn_g, workspace, ws_bytes, out, stream, nullptr, 0, true);
}

int dgw4_moe_forward_routed(const uint16_t *x, const float *router_logits, int T, int topk,
                            int E, int d, int m, const uint8_t *gu_q, const uint16_t *gu_s,
                            const uint16_t *gu_z, int gu_g, const uint8_t *dn_q,
                            const uint16_t *dn_s, const uint16_t *dn_z, int dn_g,
                            void *workspace, size_t *ws_bytes, uint16_t *out, void *stream)
{
    if (workspace && T > 0 && !router_logits)
        return DGW4_ERR_INVALID_ARG;
    return moe_forward_impl(x, nullptr, nullptr, T, topk, E, d, m, gu_q, gu_s, gu_z, gu_g, dn_q,
                            dn_s, dn_z, dn_g, workspace, ws_bytes, out, stream, nullptr, 0, true,
                            router_logits);
}

int dgw4_moe_experts(const uint16_t *x, const int32_t *topk_ids, int T, int topk, int E, int d,
                     int m, const uint8_t *gu_q, const uint16_t *gu_s, const uint16_t *gu_z,
                     int gu_g, const uint8_t *dn_q, const uint16_t *dn_s, const uint16_t *dn_z,
                     int dn_g, void *workspace, size_t *ws_bytes, void *stream)
{
    return moe_forward_impl(x, topk_ids, nullptr, T, topk, E, d, m, gu_q, gu_s, gu_z, gu_g, dn_q,
                            dn_s, dn_z, dn_g, workspace, ws_bytes, nullptr, stream, nullptr, 0,
                            false);
}

int dgw4_router(const float *logits, int T, int E, int topk, int32_t *ids, float *w, void *stream)
{
    if (T < 0 || E < 1 || E > dgw4::kMaxExperts || topk < 1 || topk > E || topk > 64)
        return DGW4_ERR_INVALID_ARG;
    if (T == 0)
        return DGW4_OK;
    if (!logits || !ids || !w || !aligned(logits, 4) || !aligned(ids, 4) || !aligned(w, 4))
        return DGW4_ERR_INVALID_ARG;
    return from_hip(dgw4::launch_router(logits, T, E, topk, ids, w, (hipStream_t)stream));
}

int dgw4_sample_noalloc(const float *logits, int R, int V, uint64_t seed, float *entropy,
                        int32_t *sample, int32_t *argmax, void *stream)
{
    if (R < 0 || V < 4)
        return DGW4_ERR_INVALID_ARG;
    if (V % 4 != 0 || (long long)R * V >= (1LL << 40) || V >= (1 << 30))
        return DGW4_ERR_UNSUPPORTED;
    if (dgw4::sample_workspace_bytes(R, V) > dgw4::kSampleScratchBytes)
        return DGW4_ERR_UNSUPPORTED;
    if (R == 0)
        return DGW4_OK;
    if (!logits || !aligned(logits, 16))
        return DGW4_ERR_INVALID_ARG;
    void *part = nullptr;
    hipError_t err = dgw4::sample_scratch(&part);
    if (err != hipSuccess)
        return from_hip(err);
    return from_hip(dgw4::launch_sample(logits, R, V, seed, entropy, sample, argmax, part,
                                        (hipStream_t)stream));
}

int dgw4_hbm_read_probe(const void *buf, size_t bytes, uint32_t *sink, void *stream)
{
    if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || !aligned(buf, 16))
        return DGW4_ERR_INVALID_ARG;
    return from_hip(dgw4::launch_read_probe(buf, bytes, sink, (hipStream_t)stream));
}

int dgw4_mfma_probe(int iters, uint32_t *sink, double *flops, void *stream)
{
    if (iters < 1 || !sink || !flops)
        return DGW4_ERR_INVALID_ARG;
    return from_hip(dgw4::launch_mfma_probe(iters, sink, flops, (hipStream_t)stream));
}

namespace {

// The dense linear's checks and arguments; query (y unused) leaves the
// kernel's row block in *row_block instead of launching it.
int linear_impl(const uint16_t *x, int T, int K, int N, const uint8_t *q, const uint16_t *s,
                const uint16_t *z, int garg, uint16_t *y, void *stream, int *row_block)
{
    int g = 0, tiled = 0, rows = 0;
    if (!split_rows(garg, rows) || !split_group(garg, g, tiled))
        return DGW4_ERR_INVALID_ARG;
    if (T < 0 || K < 2 || (K % 2) != 0 || N < 1 || g < 1)
        return DGW4_ERR_INVALID_ARG;
    if (!group_supported(g))
        return DGW4_ERR_UNSUPPORTED;
    if (K % g != 0)
        return DGW4_ERR_INVALID_ARG;
    // the kernel covers column blocks of whole 16-column tiles, stages the
    // scales of up to gate_up_max_groups() groups per row in LDS, and
    // addresses x, y and W with 32-bit offsets
    if (N % 16 != 0 || K / g > dgw4::gate_up_max_groups() ||
        (long long)T * K * 2 >= (1LL << 31) || (long long)T * N * 2 >= (1LL << 31) ||
        (long long)N * K / 2 >= (1LL << 31))
        return DGW4_ERR_UNSUPPORTED;
    if (T == 0 && !row_block)
        return DGW4_OK;
    if (!row_block && (!x || !q || !s || !z || !y))
        return DGW4_ERR_INVALID_ARG;
    if (!row_block &&
        (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 16) || !aligned(z, 16) || !aligned(y, 2)))
        return DGW4_ERR_INVALID_ARG;
    dgw4::GemmArgs a{};
    a.a_src = x;
    a.a_rows = T;
    a.q = q;
    a.s = s;
    a.z = z;
    a.K = K;
    a.n_w = N;
    a.n_out = N;
    a.topk = 1;
    a.A = T;
    a.max_tiles = (T + dgw4::kBlockM - 1) / dgw4::kBlockM;
    a.out = y;
    a.tiled = tiled;
    const int rb = dgw4::linear_row_block(a, g, rows);
    if (rb < 0)
        return DGW4_ERR_UNSUPPORTED;
    if (row_block) {
        *row_block = rb;
        return DGW4_OK;
    }
    return from_hip(dgw4::launch_linear(a, g, rb, (hipStream_t)stream));
}

}  // namespace

int dgw4_w4a16_linear(const uint16_t *x, int T, int K, int N, const uint8_t *q,
                      const uint16_t *s, const uint16_t *z, int garg, uint16_t *y, void *stream)
{
    return linear_impl(x, T, K, N, q, s, z, garg, y, stream, nullptr);
}

int dgw4_linear_row_block(int T, int K, int N, int g)
{
    int rb = 0;
    const int st = linear_impl(nullptr, T, K, N, nullptr, nullptr, nullptr, g, nullptr, nullptr, &rb);
    return st == DGW4_OK ? rb : -st;
}

int dgw4_pack_tiled(const uint8_t *q, int E, int N, int K, int g, uint8_t *qt, void *stream)
{
    if (E < 0 || N < 1 || K < 2 || g < 1)
        return DGW4_ERR_INVALID_ARG;
    if (!group_supported(g))
        return DGW4_ERR_UNSUPPORTED;
    if (N % 16 != 0 || K % g != 0)
        return DGW4_ERR_INVALID_ARG;
    if (E == 0)
        return DGW4_OK;
    const size_t bytes = (size_t)E * (size_t)N * (size_t)(K / 2);
    if (!q || !qt || !aligned(q, 8) || !aligned(qt, 8) || overlap(q, qt, bytes))
        return DGW4_ERR_INVALID_ARG;
    return from_hip(dgw4::launch_pack_tiled(q, (long long)E * N, K, g, qt, (hipStream_t)stream));
}

int dgw4_sample(const float *logits, int R, int V, uint64_t seed, float *entropy, int32_t *sample,
                int32_t *argmax, void *workspace, size_t *ws_bytes, void *stream)
{
    if (!ws_bytes || R < 0 || V < 4)
        return DGW4_ERR_INVALID_ARG;
    if (V % 4 != 0 || (long long)R * V >= (1LL << 40) || V >= (1 << 30))
        return DGW4_ERR_UNSUPPORTED;
    const size_t need = dgw4::sample_workspace_bytes(R, V);
    if (!workspace) {
        *ws_bytes = need;
        return DGW4_OK;
    }
    if (*ws_bytes < need)
        return DGW4_ERR_WORKSPACE;
    if (R == 0)
        return DGW4_OK;
    if (!logits || !aligned(logits, 16) || !aligned(workspace, 16))
        return DGW4_ERR_INVALID_ARG;
    return from_hip(dgw4::launch_sample(logits, R, V, seed, entropy, sample, argmax, workspace,
                                        (hipStream_t)stream));
}

}  // extern "C"


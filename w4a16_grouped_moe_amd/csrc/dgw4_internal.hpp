// Internal declarations shared by the dgw4 HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dgw4 {

// Rows of the padded assignment list handled by one GEMM workgroup
// (two 16-row MFMA blocks).
constexpr int kBlockM = 32;

// Rows of one chunk of the many-row expert GEMMs: an expert's sorted
// assignments padded to a multiple of 128 and taken 128 at a time.
constexpr int kChunkM = 128;

// Largest expert count the single-workgroup alignment kernel supports.
constexpr int kMaxExperts = 1024;

// Launchers: plain enqueue on `stream`, no host synchronisation. Shapes are
// validated by the C-ABI layer before these are called.
hipError_t launch_quantize_rtn(const float *w, long long groups, int g, uint8_t *q,
                               uint16_t *s, uint16_t *z, hipStream_t stream);

// Canonical [rows, K/2] packed weights -> the tiled layout of the GEMM loads
// ([rows/16][K/g][4][16][g/8]); rows % 16 == 0, K % g == 0, g 64 or 128.
hipError_t launch_pack_tiled(const uint8_t *q, long long rows, int K, int g, uint8_t *qt,
                             hipStream_t stream);

// A tile descriptor tile_info[j] = {expert or -1, y}: y holds the tile's
// valid rows in bits 0..15 and, in bits 16..30, how many tiles its expert
// has (capped at 0x7FFF; only "one" or "more" is used).
__host__ __device__ constexpr int tile_valid(int y) { return y & 0xFFFF; }
__host__ __device__ constexpr int tile_count(int y) { return y >> 16; }

// Alignment of the flat assignment ids to experts (one workgroup per
// expert). tile_info may be null; otherwise tile_info[j] = {expert, rows of
// the tile that hold assignments | tiles of the expert << 16} for live tiles,
// {-1, 0} past the total. order may be null; otherwise order[k] = the tile
// with the k-th most rows (ties to the lower tile index) for k below the
// tile total, -1 past it: the order in which the chunk GEMMs take tiles.
hipError_t launch_align(const int32_t *topk_ids, int A, int E, int block_m, long long cap,
                        int32_t *counts, int32_t *offsets, int32_t *sorted_ids,
                        int32_t *tile_expert, int32_t *num_padded, int2 *tile_info,
                        int32_t *order, hipStream_t stream);

// Router: ids int32 [T, topk] (the topk largest logits, largest first, ties
// to the lower id) and w fp32 [T, topk] (softmax over the chosen logits) from
// logits fp32 [T, E]; 1 <= topk <= min(E, 64), E <= kMaxExperts.
hipError_t launch_router(const float *logits, int T, int E, int topk, int32_t *ids, float *w,
                         hipStream_t stream);

// LDS one GEMM workgroup needs for contraction width K and group size g.
size_t gemm_lds_bytes(bool gated, int K, int g);

// Largest contraction width (m) the down GEMM supports.
int down_max_k();

// Largest group count along K (d / g) the gate_up GEMM supports.
int gate_up_max_groups();

struct GemmArgs {
    const uint16_t *a_src;      // gate_up: x [T, d] (natural order); down: H [cap, m] (permuted per 8)
    int a_rows;                 // rows of a_src (T or cap)
    const int32_t *sorted_ids;  // [cap]
    const int2 *tile_info;      // [cap / kBlockM]: {expert or -1, valid rows}
    const int32_t *tile_order;  // chunk GEMMs: [max_tiles] tiles, most rows first (-1 past the total)
    const uint8_t *q;           // packed weights [E, n_w, K/2], canonical or tiled (see tiled)
    const uint16_t *s;          // [E, n_w, K/g]
    const uint16_t *z;          // [E, n_w, K/g]
    int K;                      // contraction width (d for gate_up, m for down)
    int n_w;                    // weight rows per expert (2m or d)
    int n_out;                  // output columns (m or d)
    int topk;
    int A;                      // T * topk; also the pad sentinel in sorted_ids
    int max_tiles;              // cap / kBlockM
    void *out;                  // gate_up: H fp16 [cap, m]; down: Y fp16 [A, d]
    int tiled;                  // 1: q in the tiled layout [E][n_w/16][K/g][4][16][g/8]
};

hipError_t launch_gate_up(const GemmArgs &a, int g, hipStream_t stream);

// Dense linear y = x * deq(W)^T over the a.A = a_rows rows of x in order:
// a.sorted_ids / a.tile_info unused, one weight matrix (n_w = n_out = N rows),
// a.out = y fp16 [A, N] in natural column order. linear_row_block gives the
// kernel for the caller's choice rows (0, DGW4_ROWS_TILES or
// DGW4_ROWS_CHUNKS): kBlockM (32-row tiles), kLinearWideRows (the many-row
// kernel) or -1 (the many-row kernel asked for where it does not fit);
// launch_linear runs the one given.
constexpr int kLinearWideRows = 256;
int linear_row_block(const GemmArgs &a, int g, int rows);
hipError_t launch_linear(const GemmArgs &a, int g, int row_block, hipStream_t stream);

// The many-row dense linear (many_rows.hip): whether its LDS and alignment needs
// hold for a, and its launch (a.A rows in 256-row blocks).
bool linear_wide_fits(const GemmArgs &a, int g);
hipError_t launch_linear_wide(const GemmArgs &a, int g, hipStream_t stream);
hipError_t launch_down(const GemmArgs &a, int g, hipStream_t stream);

// The many-row expert GEMMs (many_rows.hip), over 128-row chunks (the
// alignment with block_m = kChunkM: sorted_ids / tile_info per chunk):
// whether they exist for these shapes and buffers, and their launches.
// gate_up writes H fp16 [max_tiles * kChunkM, m] in natural column order
// (dn.a_src, dn.a_rows = max_tiles * kChunkM); down writes Y fp16 [A, d],
// one row per assignment (the combine's halves = 1).
bool chunk_gemms_fit(const GemmArgs &gu, int gu_g, const GemmArgs &dn, int dn_g);
hipError_t launch_chunk_gate_up(const GemmArgs &gu, hipStream_t stream);
hipError_t launch_chunk_down(const GemmArgs &dn, hipStream_t stream);

// Whether alignment and the pair of GEMMs run as one launch (the layer's
// shape), and that launch. It reads the expert ids itself (gu.sorted_ids and
// gu.tile_info are unused) and writes dn.out as two fp16 partials
// [2][A][n_out], one per half of down's contraction, to be added by the
// combine (launch_combine with halves = 2).
bool layer_fused(const GemmArgs &gu, int gu_g, const GemmArgs &dn, int dn_g, int E);
hipError_t launch_layer(const GemmArgs &gu, const GemmArgs &dn, const int32_t *ids, int E,
                        hipStream_t stream);

// Sampler: splits per row, workspace bytes, and the two launches (partials,
// then the per-row merge). V is a multiple of 4; any output may be null
// (sample == null skips the noise).
int sample_splits(int R, int V);
size_t sample_workspace_bytes(int R, int V);
hipError_t launch_sample(const float *logits, int R, int V, uint64_t seed, float *entropy,
                         int32_t *sample, int32_t *argmax, void *workspace, hipStream_t stream);

// The sampler's own partials for callers that cannot allocate: a static
// device array of kSampleScratchBytes per device; sample_scratch gives its
// address on the current device (looked up once per device).
constexpr size_t kSampleScratchBytes = size_t(1) << 20;
hipError_t sample_scratch(void **ptr);

// One read of `bytes` (a multiple of 16) at buf over the whole chip; see
// dgw4_hbm_read_probe.
hipError_t launch_read_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

// The MFMA throughput probe (see dgw4_mfma_probe); *flops gets the launch's
// floating-point operations.
hipError_t launch_mfma_probe(int iters, uint32_t *sink, double *flops, hipStream_t stream);

// y: `halves` (1 or 2) fp16 arrays [T * topk, d] one after the other; each
// assignment's expert output is their sum.
hipError_t launch_combine(const uint16_t *y, int halves, const int32_t *topk_ids,
                          const float *topk_w, int T, int topk, int E, int d, uint16_t *out,
                          hipStream_t stream);

}  // namespace dgw4

/*
 * dgw4 — W4A16 routed-expert (grouped MoE) layer for AMD Instinct MI355X (gfx950).
 *
 * C ABI. Every pointer argument named "device" is device memory owned by the
 * caller; the library allocates nothing, keeps no state between calls and
 * never synchronises the host: each call only enqueues kernels on `stream`
 * (a hipStream_t passed as void*; NULL means the default stream) and returns.
 * Results are ready when the stream reaches that point. Calls are therefore
 * safe to capture in a HIP graph.
 *
 * Errors: every function returns a dgw4_status. Argument checks happen on the
 * host before any HIP call; on an error nothing is launched and no output is
 * written. DGW4_ERR_HIP reports a failed launch (hipGetLastError).
 * Data-dependent preconditions (values inside device buffers) are not checked
 * on the host; where a kernel meets an invalid value the behaviour is stated
 * at the function, and no kernel reads or writes outside the buffers whose
 * sizes are given here.
 *
 * Pages cited (by title and section):
 *   [card]  "DiffusionGemma-26B-A4B W4A16" model card
 *   [kcard] "dg-w4-kernels" kernel card
 *   [blog]  "Inference: Making every denoising pass fast" (Part 2)
 *
 * Packed weight format ([card] "Checkpoint format", dg-w4a16-v1): asymmetric
 * uint4, an fp16 scale s and fp16 zero point z per group of g consecutive
 * weights along the contraction dimension K, two nibbles per byte with
 * byte j of a row = q[2j] | q[2j+1] << 4. A weight is w = (q - z) * s.
 * For a matrix of N rows (outputs) by K (contraction):
 *   q  uint8  [N, K/2]   row-major
 *   s  fp16   [N, K/g]   (passed as uint16 bit patterns)
 *   z  fp16   [N, K/g]   (integer-valued)
 * An expert stack adds a leading [E] dimension to each of the three.
 * gate_up_proj of expert e is [2m, d]: rows 0..m-1 are the gate projection,
 * rows m..2m-1 the up projection. down_proj is [d, m].
 *
 * Tiled weight layout (this library's own, for gfx950; not a checkpoint
 * format): the same bytes of q reordered so that the MFMA lanes' loads of one
 * group of 16 rows are contiguous. With N % 16 == 0 and K % g == 0,
 *   qt [N/16][K/g][4][16][g/8]   (an expert stack: [E] in front)
 * where qt[b][j][p][r][i] = q[16 b + r][j g/2 + p g/8 + i]: block b of 16
 * rows, group j, quarter p of the group's g/2 bytes, row r within the block.
 * s and z keep their layout. dgw4_pack_tiled converts; the GEMM entry points
 * take a matrix in that layout when its group-size argument carries
 * DGW4_WEIGHTS_TILED (g | DGW4_WEIGHTS_TILED). Results are bit-identical to
 * those of the canonical layout on the same kernels; the layer's 128-row
 * chunks (DGW4_ROWS_CHUNKS, the library's choice for tiled weights when the
 * experts hold many rows) take tiled weights only.
 */
#ifndef DGW4_H
#define DGW4_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define DGW4_API __attribute__((visibility("default")))
#else
#define DGW4_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DGW4_OK = 0,
    DGW4_ERR_INVALID_ARG = 1,   /* null pointer, bad shape or size */
    DGW4_ERR_UNSUPPORTED = 2,   /* valid but not implemented (e.g. g not in {64,128}) */
    DGW4_ERR_WORKSPACE = 3,     /* workspace smaller than the queried size */
    DGW4_ERR_HIP = 4            /* a kernel launch failed */
} dgw4_status;

/* Or-ed into a GEMM's group-size argument: that matrix is in the tiled layout. */
#define DGW4_WEIGHTS_TILED 0x10000

/*
 * Or-ed into the layer's gate_up group-size argument (gu_g of
 * dgw4_moe_forward, _timed, _routed and dgw4_moe_experts, the workspace
 * query included): the row blocks the expert GEMMs run on.
 *   DGW4_ROWS_TILES   each expert's sorted assignments padded to 32-row
 *                     tiles; a workgroup per tile (and column block) reads
 *                     the expert's weights, so an expert's weights are read
 *                     once per tile. Fastest when experts hold few rows.
 *   DGW4_ROWS_CHUNKS  padded to 128-row chunks; the weights are formed once
 *                     per chunk and feed all its rows. Fastest when experts
 *                     hold many rows. Exists for d = 2816 at gate_up g = 128
 *                     and m = 704 at down g = 64 (else DGW4_ERR_UNSUPPORTED).
 * Neither (the default): chunks when they exist for the shape and the
 * experts hold at least 22 assignments each on average (T * topk >= 22 E),
 * else tiles. Both bits: DGW4_ERR_INVALID_ARG. The two give the same results
 * up to rounding: tiles apply each group's scale to an fp32 partial, chunks
 * round each dequantised weight (q - z) * s to fp16 once.
 */
#define DGW4_ROWS_TILES 0x20000
#define DGW4_ROWS_CHUNKS 0x40000

/* Human-readable name of a status code (static storage). */
DGW4_API const char *dgw4_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
DGW4_API int dgw4_version(void);

/* Text of the HIP error behind the calling thread's most recent
 * DGW4_ERR_HIP (static storage), or "no HIP error". */
DGW4_API const char *dgw4_last_error(void);

/*
 * dgw4_quantize_rtn — min/max round-to-nearest uint4 packer.
 * ([kcard] "W4A16": quantize_w4(W, group_size); [card] "Benchmarks":
 *  round-to-nearest min/max, no calibration; [blog] "The first constraint was
 *  capacity": per-group integer codes, scale and zero point; groups of 128
 *  for gate/up and 64 for down.)
 *
 * Per row and group G of g weights, in fp32 with IEEE round-to-nearest-even:
 *   lo = min G, hi = max G
 *   s  = fp16((hi - lo) / 15); s = 1 if that rounds to zero
 *   z  = clamp(rint(-lo / s), -2048, 2048)
 *   q  = clamp(rint(w / s) + z, 0, 15)
 * Bit-exact and deterministic.
 *
 *   w       device fp32 [E, N, K], finite, (hi - lo)/15 <= 65504 per group
 *   E, N, K E >= 1, N >= 1, K >= 2 even, K % g == 0
 *   g       64 or 128 (others: DGW4_ERR_UNSUPPORTED)
 *   q       device uint8 [E, N, K/2]        (output)
 *   s, z    device uint16 [E, N, K/g]       (output, fp16 bits)
 */
DGW4_API int dgw4_quantize_rtn(const float *w, int E, int N, int K, int g,
                      uint8_t *q, uint16_t *s, uint16_t *z, void *stream);

/*
 * dgw4_pack_tiled — reorder packed weights from the canonical layout into the
 * tiled layout above (a pure byte permutation, bit-exact).
 *   q       device uint8 [E, N, K/2], canonical, 8-byte aligned
 *   E, N, K E >= 0, N % 16 == 0, K % g == 0
 *   g       64 or 128 (others: DGW4_ERR_UNSUPPORTED), the group size the
 *           matrix was quantised with
 *   qt      device uint8 [E, N, K/2] (output), 8-byte aligned; must not
 *           overlap q (DGW4_ERR_INVALID_ARG)
 * E == 0 is a no-op. Enqueued on `stream`, no host sync.
 */
DGW4_API int dgw4_pack_tiled(const uint8_t *q, int E, int N, int K, int g, uint8_t *qt,
                             void *stream);

/*
 * dgw4_align_capacity — size of the padded assignment list for dgw4_align:
 *   cap = T*topk + E*(block_m - 1); tile_expert holds cap / block_m entries.
 * Returns 0 for invalid arguments.
 */
DGW4_API size_t dgw4_align_capacity(int T, int topk, int E, int block_m);

/*
 * dgw4_align — sync-free token-to-expert alignment.
 * ([blog] "Quantisation alone leaves a sparse execution problem": sort the
 *  assignments by expert and pad into regular blocks; [kcard] "Grouped MoE":
 *  sync-free and graph safe; [blog] "The final best W4 MoE kernel": 32-row
 *  blocks.)
 *
 * Flat assignment id i = t*topk + k, A = T*topk.
 *   counts[e]      number of i with topk_ids[i] == e
 *   offsets[e]     exclusive scan of ceil(counts/block_m)*block_m; offsets[E] = total
 *   sorted_ids[p]  expert e's flat ids in ascending order at [offsets[e], ...);
 *                  every other entry of [0, cap) holds A (pad)
 *   tile_expert[j] expert of the block_m-row tile j < offsets[E]/block_m; -1 after
 *   num_padded[0]  offsets[E]
 * Every output entry is written, so the result does not depend on the
 * buffers' previous contents. Bit-exact and deterministic.
 *
 *   topk_ids    device int32 [T, topk]; an id outside [0, E) is skipped (it
 *               is counted nowhere and never written)
 *   T >= 0, 1 <= topk, 1 <= E <= 1024, block_m in {16, 32, 64}
 *   counts      device int32 [E]                         (output)
 *   offsets     device int32 [E + 1]                     (output)
 *   sorted_ids  device int32 [cap]                       (output)
 *   tile_expert device int32 [cap / block_m]             (output)
 *   num_padded  device int32 [1]                         (output)
 */
DGW4_API int dgw4_align(const int32_t *topk_ids, int T, int topk, int E, int block_m,
               int32_t *counts, int32_t *offsets, int32_t *sorted_ids,
               int32_t *tile_expert, int32_t *num_padded, void *stream);

/*
 * dgw4_router — each token's experts and weights from its router logits
 * ([blog] "Quantisation alone leaves a sparse execution problem": a router
 * scores the experts per token; the token picks 8 of 128 and the chosen
 * experts' outputs are weighted). The pages give no formula; the reading:
 *   ids[t, k]  = the k-th largest of logits[t, :], largest first, equal
 *                logits ordered by the lower expert id (the topk most
 *                probable experts, since a softmax is monotone; the choice
 *                compares the fp32 logits and is exact);
 *   w[t, k]    = exp(l_k - l_0) / sum_j exp(l_j - l_0) over the chosen
 *                logits, fp32 (the chosen softmax probabilities
 *                renormalised to one), the sum taken in k order.
 * ids and w are the topk_ids / topk_w inputs of dgw4_moe_forward.
 *   logits  device fp32 [T, E], finite, 4-byte aligned
 *   ids     device int32 [T, topk] (output); w device fp32 [T, topk] (output)
 *   T >= 0, 1 <= E <= 1024, 1 <= topk <= min(E, 64)
 * Returns DGW4_ERR_INVALID_ARG otherwise (or for null/misaligned pointers
 * with T > 0); T == 0 is a no-op. Enqueued on `stream`, no host sync.
 */
DGW4_API int dgw4_router(const float *logits, int T, int E, int topk, int32_t *ids, float *w,
                         void *stream);

/*
 * dgw4_moe_forward — one routed-expert layer with W4A16 experts.
 * ([kcard] "Grouped MoE": fused_moe_w4_v2(hidden, experts, topk_ids,
 *  topk_weights) with packed gu_q/gu_s/gu_z and dn_q/dn_s/dn_z, one launch for
 *  all experts, activation folded into the first GEMM's epilogue, fixed-order
 *  combine; [blog] "Quantisation alone leaves a sparse execution problem":
 *  each token runs through its routed experts, the outputs are weighted and
 *  added in a fixed order; [card] "Checkpoint format": the packed layout.)
 *
 * For every token t:
 *   out[t] = sum over k = 0..topk-1 (ascending) of
 *            w[t,k] * down_e( gelu_tanh(gate_e(x[t])) * up_e(x[t] ) ),  e = ids[t,k]
 * with expert weights dequantised as w = (q - z) * s. Accumulation is fp32;
 * the gated intermediate and each expert output are rounded to fp16 once
 * (on 32-row tiles at the layer's shape, d = 2816, m = 704, gate_up g = 128,
 * down g = 64, each expert output is kept as two fp16 partials, one per half
 * of down's contraction, added in fp32 by the combine; on 128-row chunks
 * each dequantised weight is rounded to fp16 once, see DGW4_ROWS_CHUNKS),
 * and the combine sums
 * w[t,k] * output in ascending k in fp32 without atomics, then rounds once
 * to fp16. No workgroup waits for another and nothing depends on timing:
 * repeated calls on the same inputs give bit-identical results.
 *
 *   x          device fp16 bits [T, d]
 *   topk_ids   device int32 [T, topk]; ids outside [0, E) contribute nothing
 *   topk_w     device fp32 [T, topk]
 *   T >= 0, 1 <= topk <= E, 1 <= E <= 1024
 *   d, m       d % gu_g == 0, m % dn_g == 0 (so both are multiples of 64)
 *   gu_q/s/z   device, gate_up stack [E, 2m, d] packed with group gu_g
 *   dn_q/s/z   device, down stack [E, d, m] packed with group dn_g
 *              (x, the six pack pointers: 16-byte aligned; out: 8-byte aligned)
 *   gu_g, dn_g 64 or 128 each (others: DGW4_ERR_UNSUPPORTED), each or-ed
 *              with DGW4_WEIGHTS_TILED when that stack's q is in the tiled
 *              layout (same results on the same row blocks; the layer's
 *              shape runs fastest with both tiled, and only then can it take
 *              128-row chunks); gu_g may also carry DGW4_ROWS_TILES or
 *              DGW4_ROWS_CHUNKS. Other bits: DGW4_ERR_INVALID_ARG.
 *   workspace  device scratch of at least *ws_bytes bytes, 256-byte aligned.
 *              If workspace is NULL, the required size is written to
 *              *ws_bytes and nothing is launched. Contents on entry are
 *              irrelevant; the call overwrites what it uses.
 *   ws_bytes   host pointer: in = size of workspace, out (query) = required
 *   out        device fp16 bits [T, d]                   (output)
 * The kernels address x, the gated intermediate (T * topk + E * 31 padded
 * rows x m fp16 on 32-row tiles), the expert outputs and one expert's
 * packed weights through 32-bit byte offsets: a call where any of them
 * would reach 2 GiB returns DGW4_ERR_UNSUPPORTED (the query too), and
 * 128-row chunks are only taken where T * topk * d * 2 < 2 GiB. At d = 2816,
 * m = 704, E = 128, top-8 that is T <= 190154 (T <= 47662 on chunks).
 */
DGW4_API int dgw4_moe_forward(const uint16_t *x, const int32_t *topk_ids, const float *topk_w,
                     int T, int topk, int E, int d, int m,
                     const uint8_t *gu_q, const uint16_t *gu_s, const uint16_t *gu_z, int gu_g,
                     const uint8_t *dn_q, const uint16_t *dn_s, const uint16_t *dn_z, int dn_g,
                     void *workspace, size_t *ws_bytes, uint16_t *out, void *stream);

/*
 * dgw4_moe_row_block — the row blocks dgw4_moe_forward runs its expert GEMMs
 * on for these arguments (gu_g with its DGW4_ROWS_* and DGW4_WEIGHTS_TILED
 * bits, dn_g with its layout bit): 32 (tiles) or 128 (chunks). Host only,
 * launches nothing. Returns the negated status for arguments the forward's
 * workspace query rejects (e.g. -DGW4_ERR_UNSUPPORTED for chunks asked for
 * where they do not exist).
 */
DGW4_API int dgw4_moe_row_block(int T, int topk, int E, int d, int m, int gu_g, int dn_g);

/*
 * dgw4_moe_forward_timed — dgw4_moe_forward with stage events, for per-kernel
 * timing of the same launch sequence (same kernels, same arguments, same
 * results). events is an array of n_events = 5 caller-created hipEvent_t
 * handles (passed as void*); they are recorded on `stream` before the first
 * kernel and after each of the four stages (align, gate_up, down, combine).
 * Elapsed time between consecutive events is the duration of one stage.
 * Where alignment, gate_up and down run as one launch (32-row tiles at the
 * layer's shape: d = 2816, m = 704, gate_up g = 128, down g = 64, both
 * stacks in the same layout, E <= 704), events 1, 2 and 3 are all recorded
 * after that launch, so the first stage brackets it and the next two
 * bracket no kernel. events == NULL
 * behaves exactly like dgw4_moe_forward; any other n_events is
 * DGW4_ERR_INVALID_ARG. A workspace query (workspace == NULL) records
 * nothing.
 */
DGW4_API int dgw4_moe_forward_timed(const uint16_t *x, const int32_t *topk_ids,
                                    const float *topk_w, int T, int topk, int E, int d, int m,
                                    const uint8_t *gu_q, const uint16_t *gu_s,
                                    const uint16_t *gu_z, int gu_g, const uint8_t *dn_q,
                                    const uint16_t *dn_s, const uint16_t *dn_z, int dn_g,
                                    void *workspace, size_t *ws_bytes, uint16_t *out,
                                    void *stream, void *const *events, int n_events);

/*
 * dgw4_moe_forward_routed — dgw4_moe_forward from router logits: the router
 * (dgw4_router) writes each token's ids and weights into the workspace, then
 * the layer runs on them, all on `stream`. router_logits: device fp32
 * [T, E], finite, 4-byte aligned; topk <= 64. Other arguments, checks,
 * workspace (the same size as dgw4_moe_forward's) and results as for
 * dgw4_moe_forward with the router's ids and weights.
 */
DGW4_API int dgw4_moe_forward_routed(const uint16_t *x, const float *router_logits, int T,
                                     int topk, int E, int d, int m, const uint8_t *gu_q,
                                     const uint16_t *gu_s, const uint16_t *gu_z, int gu_g,
                                     const uint8_t *dn_q, const uint16_t *dn_s,
                                     const uint16_t *dn_z, int dn_g, void *workspace,
                                     size_t *ws_bytes, uint16_t *out, void *stream);

/*
 * dgw4_moe_experts — the expert stages of dgw4_moe_forward alone (alignment,
 * gate_up with its activation, down), without the combine: the same kernels
 * with the same arguments, leaving each assignment's expert output in the
 * workspace instead of reducing them into out. A measurement aid (timing the
 * expert kernels back to back without the combine), not a step a layer
 * needs on its own. Arguments, checks and workspace as for dgw4_moe_forward
 * (the same workspace size); topk_w and out are not taken.
 */
DGW4_API int dgw4_moe_experts(const uint16_t *x, const int32_t *topk_ids, int T, int topk, int E,
                              int d, int m, const uint8_t *gu_q, const uint16_t *gu_s,
                              const uint16_t *gu_z, int gu_g, const uint8_t *dn_q,
                              const uint16_t *dn_s, const uint16_t *dn_z, int dn_g,
                              void *workspace, size_t *ws_bytes, void *stream);

/*
 * dgw4_w4a16_linear — the dense W4A16 linear layer: y = x * deq(W)^T
 * ([kcard] "W4A16": w4a16_linear(x, qw, scale, zero) equals F.linear(x,
 * dequant(W)); the same packing and the same GEMM core as the routed-expert
 * layer, one weight matrix, every row of x).
 *   x  fp16 [T, K] row-major, 16-byte aligned;
 *   q  uint8 [N, K/2], s and z fp16 [N, K/g]: one matrix in the layout of
 *      dgw4_quantize_rtn with E = 1 (16-byte aligned);
 *   y  fp16 [T, N] row-major (written, caller-owned).
 * g may carry DGW4_WEIGHTS_TILED (q in the tiled layout; same results) and
 * one of the row-block flags, which pick the kernel:
 *   DGW4_ROWS_TILES   32-row tiles: each output is the fp32 sum over K of x
 *                     times the exact integers (q - z), the group's scale
 *                     applied once per group in fp32;
 *   DGW4_ROWS_CHUNKS  the many-row kernel (256-row blocks): each weight is
 *                     formed once per block as fp16 (q - z) * s (one
 *                     rounding) and the MFMA sums over K in fp32; needs y
 *                     8-byte aligned and K small enough for its LDS staging
 *                     (else DGW4_ERR_UNSUPPORTED);
 *   neither           the many-row kernel where it fits, T >= 128 and
 *                     T * N >= 2^23 (enough 256 x 256 blocks to cover half
 *                     the chip), else the tiles.
 * Either way the result is rounded once to fp16; the two agree up to that
 * rounding of the weights. Returns DGW4_ERR_INVALID_ARG for null pointers
 * (T > 0), negative T, odd K, K % g != 0, unknown flag bits or both row
 * flags in g, or misaligned pointers; DGW4_ERR_UNSUPPORTED for g not in
 * {64, 128}, N not a multiple of 16, more than 64 groups per row, or
 * tensors past 2 GiB. T == 0 is a no-op. Enqueued on `stream`, no host sync.
 */
DGW4_API int dgw4_w4a16_linear(const uint16_t *x, int T, int K, int N, const uint8_t *q,
                               const uint16_t *s, const uint16_t *z, int g, uint16_t *y,
                               void *stream);

/*
 * dgw4_linear_row_block — the row block of the kernel dgw4_w4a16_linear
 * runs for these sizes and g (flags included) with an 8-byte aligned y: 32
 * (the 32-row tiles) or 256 (the many-row kernel); a negative status code
 * (-DGW4_ERR_...) where the call would fail its checks. Launches nothing.
 */
DGW4_API int dgw4_linear_row_block(int T, int K, int N, int g);

/*
 * dgw4_sample — the sampler of a denoising step, in one streaming pass over
 * R rows of V fp32 logits ([kcard] "Sampler": fused_entropy and
 * gumbel_argmax_sample; here one pass gives both):
 *   entropy[r] = -sum_v p_v log p_v, p = softmax(row r), fp32 nats;
 *   argmax[r]  = the first v with the largest logit;
 *   sample[r]  = the first v with the largest l_v + G_v, a draw from
 *                Categorical(p) by Gumbel-max. G_v = -log(-log U_v) in fp32;
 *                U_v = (floor(w / 512) + 1/2) / 2^23, exact in fp32 and
 *                strictly inside (0, 1), with w word v % 4 of the
 *                Philox4x32-10 block with counter {v / 4, r, 0, 0} and key
 *                {seed & 0xffffffff, seed >> 32}. Same seed, same draw.
 * logits: device, row-major [R, V], 16-byte aligned, finite or -inf (masked,
 * probability 0), at least one finite value per row. entropy (fp32 [R]),
 * sample and argmax (int32 [R]): device, each may be NULL to skip it (NULL
 * sample also skips the noise). CUB-style workspace: workspace == NULL
 * writes the size to *ws_bytes and returns DGW4_OK; otherwise at least that
 * many bytes, 16-byte aligned, caller-owned. Every reduction has a fixed
 * order: results are bitwise reproducible.
 * Returns DGW4_ERR_INVALID_ARG (null ws_bytes, R < 0, V < 4, misaligned or
 * null pointers), DGW4_ERR_UNSUPPORTED (V not a multiple of 4, R * V >=
 * 2^40), DGW4_ERR_WORKSPACE (*ws_bytes too small), DGW4_ERR_HIP.
 * Enqueued on `stream`; no host synchronisation.
 */
DGW4_API int dgw4_sample(const float *logits, int R, int V, uint64_t seed, float *entropy,
                         int32_t *sample, int32_t *argmax, void *workspace, size_t *ws_bytes,
                         void *stream);

/*
 * dgw4_sample_noalloc — dgw4_sample for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and results, with the partials in a
 * fixed 1 MiB array that the library holds on each device for the life of
 * the process instead of a caller workspace. It allocates nothing. Shapes
 * whose partials need more (sample_workspace_bytes > 1 MiB: R x splits x 32
 * bytes, which holds for any V up to R = 32768 rows) return
 * DGW4_ERR_UNSUPPORTED before anything is launched; other checks as for
 * dgw4_sample. The array belongs to the device that is current when the call
 * is made, and `stream` must belong to that device. Every call on a device
 * shares its array: calls that overlap on one device (other streams, other
 * host threads) race and must be serialised by the caller; calls in order on
 * one stream are fine. Nothing in the array needs to start at zero (each
 * partial is written before it is read).
 */
DGW4_API int dgw4_sample_noalloc(const float *logits, int R, int V, uint64_t seed,
                                 float *entropy, int32_t *sample, int32_t *argmax,
                                 void *stream);

/*
 * dgw4_hbm_read_probe — a measurement aid, not a step of the layer: reads
 * `bytes` bytes of device memory at `buf` once, with the whole chip
 * (16-byte non-temporal loads, several in flight per lane), so that the elapsed time on
 * `stream` gives the read bandwidth this device sustains. The loads are
 * folded into one word, stored to sink[0] only if it equals 0x9E3779B9
 * (never, for a buffer filled with one repeated byte), which keeps them from
 * being optimised away. buf: device memory, 16-byte aligned; bytes: a
 * positive multiple of 16; sink: device memory of at least 4 bytes.
 * Returns DGW4_ERR_INVALID_ARG otherwise, DGW4_ERR_HIP if the launch fails.
 */
DGW4_API int dgw4_hbm_read_probe(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/*
 * dgw4_mfma_probe — a measurement aid, not a step of the layer: every wave of
 * a whole-chip launch (two 512-thread workgroups per compute unit) runs
 * `iters` rounds of eight independent v_mfma_f32_16x16x32_f16 on operands
 * held in registers, with no memory traffic, so that the elapsed time on
 * `stream` gives the dense fp16 matrix rate this device sustains. *flops
 * (host memory) receives the launch's floating-point operations (2 x 16 x 16
 * x 32 per MFMA). The sums are folded into one word, stored to sink[0] only
 * if it equals 0x9E3779B9, which keeps the work from being optimised away.
 * iters >= 1; sink: device memory of at least 4 bytes. Returns
 * DGW4_ERR_INVALID_ARG otherwise, DGW4_ERR_HIP if the launch fails.
 */
DGW4_API int dgw4_mfma_probe(int iters, uint32_t *sink, double *flops, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DGW4_H */

/*
 * CPU oracle for the W4A16 routed-expert layer (and the sampler that follows
 * it in a denoising step).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may load, link or
 * call this file: it is used by tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py, and by nothing else. It shares no code,
 * header, table or helper with the HIP library.
 *
 * Plain, slow, obviously correct. Each function follows a passage of the
 * pages (cited below by page title and section):
 *
 *   [card]   "DiffusionGemma-26B-A4B W4A16" model card
 *   [kcard]  "dg-w4-kernels" kernel card
 *   [blog]   "Inference: Making every denoising pass fast" (Part 2)
 *
 * Readings where the pages are silent (their quantisation formula was lost in
 * extraction) are listed in the design doc and at each function.
 *
 * Precision: the quantiser takes its integer decisions in fp32 (the precision
 * the GPU packer uses), with the scale rounded to fp16 before use because the
 * stored scale is fp16 ([card] "Checkpoint format"). Everything in the layer
 * forward is fp64: dequantised weights, products, sums, the activation and
 * the combine. Parity of the forward is therefore unpinned by rounding order:
 * the oracle is the (near) exact value.
 *
 * Pins (tests/test_oracle_*.py) hold every function here to something other
 * than itself: numpy's IEEE fp16 cast, the card's packing example, closed
 * forms, numpy bincount/argsort, numpy matmul on dequantised weights, exact
 * GELU via erf, and a dense brute force that runs every token through every
 * expert.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads of the OpenMP loops below (for timing the oracle at a given core
 * count); returns the count now in force. */
int orc_set_threads(int n)
{
    if (n > 0)
        omp_set_num_threads(n);
    return omp_get_max_threads();
}

/* ---------------------------------------------------------------- fp16 ---- */

/* IEEE-754 binary32 -> binary16, round to nearest, ties to even. Written from
 * the format definition: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits; subnormals are multiples of 2^-24. */
uint16_t orc_f32_to_f16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t bexp = (u >> 23) & 0xFFu;
    uint32_t frac = u & 0x7FFFFFu;

    if (bexp == 0xFFu)                       /* inf or NaN */
        return (uint16_t)(sign | 0x7C00u | (frac ? 0x200u : 0u));
    if (bexp == 0u)                          /* fp32 zero or subnormal: < 2^-126 */
        return sign;                          /* far below half of 2^-24 */

    int e = (int)bexp - 127;                  /* value = 1.frac * 2^e */
    uint32_t sig = (1u << 23) | frac;         /* 24-bit significand */

    if (e >= -14) {                           /* normal binary16 range (or overflow) */
        uint32_t keep = sig >> 13;            /* 11 bits incl. the leading one */
        uint32_t rem = sig & 0x1FFFu;
        if (rem > 0x1000u || (rem == 0x1000u && (keep & 1u)))
            keep += 1u;
        int he = e + 15;
        if (keep == 0x800u) {                 /* rounding carried into a new binade */
            keep = 0x400u;
            he += 1;
        }
        if (he >= 31)
            return (uint16_t)(sign | 0x7C00u);  /* overflow -> inf */
        return (uint16_t)(sign | ((uint32_t)he << 10) | (keep & 0x3FFu));
    }
    /* subnormal binary16: count units of 2^-24. value = sig * 2^(e-23)
     * = sig * 2^(e+1) units, e+1 <= -14, so shift right by -(e+1). */
    int sh = -(e + 1);
    if (sh > 25)
        return sign;                          /* < 2^-25: rounds to zero */
    uint32_t units = sig >> sh;
    uint32_t rem = sig & ((1u << sh) - 1u);
    uint32_t half = 1u << (sh - 1);
    if (rem > half || (rem == half && (units & 1u)))
        units += 1u;                          /* may become 0x400 = min normal */
    return (uint16_t)(sign | units);
}

/* binary16 -> binary32, exact. */
float orc_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t he = (h >> 10) & 0x1Fu;
    uint32_t hf = h & 0x3FFu;
    uint32_t u;
    if (he == 0x1Fu) {
        u = sign | 0x7F800000u | (hf << 13);
    } else if (he == 0u) {
        /* subnormal: hf * 2^-24, exact in fp32 */
        float v = (float)hf * 5.9604644775390625e-08f;   /* 2^-24 */
        memcpy(&u, &v, 4);
        u |= sign;
    } else {
        u = sign | ((he - 15u + 127u) << 23) | (hf << 13);
    }
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Element-wise array forms of the two conversions above. */
void orc_f32_to_f16_array(const float *src, long n, uint16_t *dst)
{
    for (long i = 0; i < n; ++i)
        dst[i] = orc_f32_to_f16(src[i]);
}

void orc_f16_to_f32_array(const uint16_t *src, long n, float *dst)
{
    for (long i = 0; i < n; ++i)
        dst[i] = orc_f16_to_f32(src[i]);
}

/* ------------------------------------------------------------ quantiser ---- */

/*
 * Min/max round-to-nearest asymmetric uint4 quantiser ([card] "Benchmarks":
 * round-to-nearest min/max with no calibration; [blog] "The first constraint
 * was capacity": groups of 128 for gate/up, 64 for down, integer q_i with a
 * per-group scale s and zero point z; [kcard] "W4A16": quantize_w4(W,
 * group_size)). The printed formula is lost; the reading used:
 *
 *   lo, hi = min, max of the group          (fp32, exact)
 *   s      = fp16_rn((hi - lo) / 15)         (fp32 subtract and divide)
 *   s      = 1 if s rounds to zero           (degenerate group)
 *   z      = clamp(rint(-lo / s), -2048, 2048)          (integer, stored fp16;
 *            a zero point of 0 is stored as +0)
 *   q_i    = clamp(rint(w_i / s) + z, 0, 15)            (integer add after rint)
 *
 * rint is round-half-to-even. Nibble packing ([card] "Checkpoint format"):
 * along K, byte j of a row holds q[2j] in its low nibble and q[2j+1] in its
 * high nibble.
 *
 * Layout: w fp32 [E, N, K] row-major; q u8 [E, N, K/2]; s, z fp16 bits
 * [E, N, K/g]. Returns 0, or -1 for invalid shapes.
 */
int orc_quantize_rtn(const float *w, int E, int N, int K, int g,
                     uint8_t *q, uint16_t *s, uint16_t *z)
{
    if (E <= 0 || N <= 0 || K <= 0 || g <= 0 || (K % 2) || (K % g) || (g % 2))
        return -1;
    const int ng = K / g;
    const long rows = (long)E * N;
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) {
        const float *wr = w + r * K;
        uint8_t *qr = q + r * (K / 2);
        for (int gi = 0; gi < ng; ++gi) {
            const float *wg = wr + (long)gi * g;
            float lo = wg[0], hi = wg[0];
            for (int i = 1; i < g; ++i) {
                if (wg[i] < lo) lo = wg[i];
                if (wg[i] > hi) hi = wg[i];
            }
            const float range = hi - lo;             /* fp32 subtract */
            const float s32 = range / 15.0f;         /* fp32 divide */
            uint16_t sb = orc_f32_to_f16(s32);
            if ((sb & 0x7FFFu) == 0u)
                sb = 0x3C00u;                        /* 1.0 */
            const float sf = orc_f16_to_f32(sb);
            float zf = rintf(-lo / sf);
            if (zf < -2048.0f) zf = -2048.0f;
            if (zf > 2048.0f) zf = 2048.0f;
            const int zi = (int)zf;                  /* an integer: zero has no sign */
            s[r * ng + gi] = sb;
            z[r * ng + gi] = orc_f32_to_f16((float)zi);   /* exact: |zi| <= 2048 */
            for (int i = 0; i < g; ++i) {
                float v = rintf(wg[i] / sf) + zf;
                if (v < 0.0f) v = 0.0f;
                if (v > 15.0f) v = 15.0f;
                const int k = gi * g + i;
                const uint8_t nib = (uint8_t)v;
                if (k & 1)
                    qr[k >> 1] = (uint8_t)(qr[k >> 1] | (nib << 4));
                else
                    qr[k >> 1] = nib;
            }
        }
    }
    return 0;
}

/* Nibble k of a packed row ([card] "Checkpoint format"). */
static inline int orc_nibble(const uint8_t *row, long k)
{
    return (row[k >> 1] >> (4 * (int)(k & 1))) & 0xF;
}

/* Dequantise one packed row of K weights: w = (q - z) * s ([blog] "The first
 * constraint was capacity": integer q_i with scale s_g and zero point z_g).
 * Exact in fp64 (a small integer times an fp16 value). */
static void orc_deq_row(const uint8_t *qrow, const uint16_t *srow,
                        const uint16_t *zrow, int g, long K, double *dst)
{
    for (long k = 0; k < K; ++k) {
        const long gi = k / g;
        dst[k] = ((double)orc_nibble(qrow, k) - (double)orc_f16_to_f32(zrow[gi])) *
                 (double)orc_f16_to_f32(srow[gi]);
    }
}

/* Rebuild the fp64 matrix [E, N, K] from a packed buffer ([blog] "The first
 * constraint was capacity": a dequantised reference rebuilds the floats). */
int orc_dequant(const uint8_t *q, const uint16_t *s, const uint16_t *z,
                int E, int N, int K, int g, double *out)
{
    if (E <= 0 || N <= 0 || K <= 0 || g <= 0 || (K % 2) || (K % g))
        return -1;
    const int ng = K / g;
    const long rows = (long)E * N;
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r)
        orc_deq_row(q + r * (K / 2), s + r * ng, z + r * ng, g, K, out + r * K);
    return 0;
}

/* ---------------------------------------------------------------- align ---- */

/*
 * Token-to-expert alignment ([blog] "Quantisation alone leaves a sparse
 * execution problem": sort assignments by expert, pad into regular blocks;
 * [kcard] "Grouped MoE": sync-free alignment; [blog] "The final best W4 MoE
 * kernel": 32-row blocks). Flat assignment id i = t*topk + k.
 *
 *   counts[e]      = number of i with ids[i] == e
 *   offsets[0]     = 0, offsets[e+1] = offsets[e] + ceil(counts[e]/bm)*bm
 *   sorted_ids     : expert e's ids in ascending i at [offsets[e], ...),
 *                    every other entry of [0, cap) = T*topk (pad)
 *   tile_expert[j] = e for tiles j in [offsets[e]/bm, offsets[e+1]/bm),
 *                    -1 for the rest of [0, cap/bm)
 *   num_padded     = offsets[E]
 *
 * cap = T*topk + E*(bm-1). Returns 0, or -1 on invalid arguments or an id
 * outside [0, E).
 */
int orc_align(const int32_t *ids, int T, int topk, int E, int bm,
              int32_t *counts, int32_t *offsets, int32_t *sorted_ids,
              int32_t *tile_expert, int32_t *num_padded)
{
    if (T < 0 || topk <= 0 || E <= 0 || bm <= 0)
        return -1;
    const long A = (long)T * topk;
    const long cap = A + (long)E * (bm - 1);
    for (long i = 0; i < A; ++i)
        if (ids[i] < 0 || ids[i] >= E)
            return -1;
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (long i = 0; i < A; ++i)
        counts[ids[i]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) {
        const long tiles = (counts[e] + bm - 1) / bm;
        offsets[e + 1] = (int32_t)(offsets[e] + tiles * bm);
    }
    for (long p = 0; p < cap; ++p)
        sorted_ids[p] = (int32_t)A;
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    if (!cursor)
        return -1;
    for (int e = 0; e < E; ++e)
        cursor[e] = offsets[e];
    for (long i = 0; i < A; ++i)            /* ascending i: stable */
        sorted_ids[cursor[ids[i]]++] = (int32_t)i;
    free(cursor);
    for (long j = 0; j < cap / bm; ++j)
        tile_expert[j] = -1;
    for (int e = 0; e < E; ++e)
        for (long j = offsets[e] / bm; j < offsets[e + 1] / bm; ++j)
            tile_expert[j] = e;
    *num_padded = offsets[E];
    return 0;
}

/* --------------------------------------------------------------- router ---- */

/*
 * Router ([blog] "Quantisation alone leaves a sparse execution problem": a
 * router scores the experts per token, the token picks 8 of 128 and their
 * outputs are weighted). The pages give no formula; the reading used:
 *
 *   the scores are logits l[t, 0..E-1];
 *   the token's experts are its topk largest logits, largest first, equal
 *   logits ordered by the lower expert id (a softmax is monotone, so these
 *   are the topk most probable experts: the choice compares the fp32 inputs
 *   and needs no arithmetic at all);
 *   the weights are the chosen experts' softmax probabilities renormalised
 *   to sum to one, which is the softmax over the chosen logits alone:
 *   w[t, k] = exp(l_k - l_0) / sum_j exp(l_j - l_0), l_0 the largest, in fp64.
 *
 * logits fp32 [T, E] (finite); ids int32 [T, topk]; w fp64 [T, topk].
 * Returns 0, or -1 on invalid arguments.
 */
int orc_router(const float *logits, int T, int E, int topk, int32_t *ids, double *w)
{
    if (T < 0 || E <= 0 || topk <= 0 || topk > E)
        return -1;
    int bad = 0;
#pragma omp parallel for schedule(static)
    for (long t = 0; t < T; ++t) {
        const float *l = logits + t * (long)E;
        unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
        if (!taken) {
            bad = 1;
            continue;
        }
        int32_t *it = ids + t * (long)topk;
        for (int k = 0; k < topk; ++k) {
            int best = -1;
            for (int e = 0; e < E; ++e)        /* ascending e: ties keep the lower id */
                if (!taken[e] && (best < 0 || l[e] > l[best]))
                    best = e;
            taken[best] = 1;
            it[k] = best;
        }
        free(taken);
        const double l0 = (double)l[it[0]];
        double den = 0.0;
        for (int k = 0; k < topk; ++k)
            den += exp((double)l[it[k]] - l0);
        for (int k = 0; k < topk; ++k)
            w[t * (long)topk + k] = exp((double)l[it[k]] - l0) / den;
    }
    return bad ? -1 : 0;
}

/* ----------------------------------------------------------- activation ---- */

/* GELU, tanh form: 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))). The pages
 * say only that the activation sits in the first GEMM's epilogue ([kcard]
 * "Grouped MoE"); gated GELU(tanh) is the reading used. */
double orc_gelu_tanh(double v)
{
    const double c = sqrt(2.0 / M_PI);
    return 0.5 * v * (1.0 + tanh(c * (v + 0.044715 * v * v * v)));
}

/* ---------------------------------------------------------------- linear ---- */

/* w4a16_linear ([kcard] "W4A16": equal to F.linear(x, dequant(W))):
 * out[r, n] = sum_k x[r, k] * deq(W)[n, k], ascending k, fp64.
 * x fp16 bits [M, K]; q u8 [N, K/2]; s, z fp16 bits [N, K/g]; out [M, N]. */
int orc_w4a16_linear(const uint16_t *x, int M, int K, int N,
                     const uint8_t *q, const uint16_t *s, const uint16_t *z, int g,
                     double *out)
{
    if (M < 0 || K <= 0 || N <= 0 || g <= 0 || (K % 2) || (K % g))
        return -1;
    const int ng = K / g;
    int bad = 0;
#pragma omp parallel for schedule(static)
    for (long n = 0; n < N; ++n) {
        double *wrow = (double *)malloc(sizeof(double) * (size_t)K);
        if (!wrow) {
            bad = 1;
            continue;
        }
        orc_deq_row(q + n * (K / 2), s + n * ng, z + n * ng, g, K, wrow);
        for (long r = 0; r < M; ++r) {
            double acc = 0.0;
            for (long k = 0; k < K; ++k)
                acc += (double)orc_f16_to_f32(x[r * K + k]) * wrow[k];
            out[r * N + n] = acc;
        }
        free(wrow);
    }
    return bad ? -1 : 0;
}

/* ---------------------------------------------------------- MoE forward ---- */

/*
 * Routed-expert layer, computed directly from its definition ([blog]
 * "Quantisation alone leaves a sparse execution problem": the router picks 8
 * of 128 experts, the token runs through those eight, the outputs are weighted
 * and added; [kcard] "Grouped MoE": fused_moe_w4_v2(hidden, experts, topk_ids,
 * topk_weights) with packed gu_q/gu_s/gu_z and dn_q/dn_s/dn_z; [blog] same
 * section: each token's eight outputs are reduced in a fixed order).
 *
 * For each listed token t and each k = 0..topk-1 in ascending order,
 * with e = ids[t, k]:
 *   gu[j] = sum_c x[t, c] * deq(gate_up[e])[j, c]          j < 2m, c ascending
 *   h[j]  = gelu_tanh(gu[j]) * gu[m + j]                     j < m
 *           (rows 0..m-1 of gate_up are the gate, m..2m-1 the up projection)
 *   y[c]  = sum_j h[j] * deq(down[e])[c, j]                  c < d, j ascending
 *   out[t, c] += w[t, k] * y[c]
 *
 * Layouts: x fp16 bits [T, d]; ids int32 [T, topk]; w fp32 [T, topk];
 * gate_up: q [E, 2m, d/2], s/z [E, 2m, d/gu_g]; down: q [E, d, m/2],
 * s/z [E, d, m/dn_g]. tokens: list of n_tok token indices (NULL = all T, in
 * order). out fp64 [n_tok, d]; y_out (optional, may be NULL) fp64
 * [n_tok, topk, d] holds each expert's un-weighted output.
 * Returns 0, or -1 on invalid arguments.
 */
int orc_moe_forward(const uint16_t *x, const int32_t *ids, const float *w,
                    int T, int topk, int E, int d, int m,
                    const uint8_t *gu_q, const uint16_t *gu_s, const uint16_t *gu_z, int gu_g,
                    const uint8_t *dn_q, const uint16_t *dn_s, const uint16_t *dn_z, int dn_g,
                    const int32_t *tokens, int n_tok, double *out, double *y_out)
{
    if (T < 0 || topk <= 0 || E <= 0 || d <= 0 || m <= 0 || gu_g <= 0 || dn_g <= 0 ||
        (d % gu_g) || (m % dn_g) || (d % 2) || (m % 2))
        return -1;
    if (!tokens)
        n_tok = T;
    for (int a = 0; a < n_tok; ++a) {
        const int t = tokens ? tokens[a] : a;
        if (t < 0 || t >= T)
            return -1;
        for (int k = 0; k < topk; ++k)
            if (ids[(long)t * topk + k] < 0 || ids[(long)t * topk + k] >= E)
                return -1;
    }
    const int gu_ng = d / gu_g, dn_ng = m / dn_g;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int a = 0; a < n_tok; ++a) {
        const int t = tokens ? tokens[a] : a;
        double *xv = (double *)malloc(sizeof(double) * (size_t)d);
        double *gu = (double *)malloc(sizeof(double) * (size_t)(2 * m));
        double *h = (double *)malloc(sizeof(double) * (size_t)m);
        double *y = (double *)malloc(sizeof(double) * (size_t)d);
        double *wrow = (double *)malloc(sizeof(double) * (size_t)(d > m ? d : m));
        if (!xv || !gu || !h || !y || !wrow) {
            bad = 1;
        } else {
            for (int c = 0; c < d; ++c)
                xv[c] = (double)orc_f16_to_f32(x[(long)t * d + c]);
            double *o = out + (long)a * d;
            for (int c = 0; c < d; ++c)
                o[c] = 0.0;
            for (int k = 0; k < topk; ++k) {
                const long e = ids[(long)t * topk + k];
                /* gate_up projection of expert e */
                for (long j = 0; j < 2L * m; ++j) {
                    const long row = e * 2L * m + j;
                    orc_deq_row(gu_q + row * (d / 2), gu_s + row * gu_ng,
                                gu_z + row * gu_ng, gu_g, d, wrow);
                    double acc = 0.0;
                    for (long c = 0; c < d; ++c)
                        acc += xv[c] * wrow[c];
                    gu[j] = acc;
                }
                /* gated activation */
                for (int j = 0; j < m; ++j)
                    h[j] = orc_gelu_tanh(gu[j]) * gu[m + j];
                /* down projection of expert e */
                for (long c = 0; c < d; ++c) {
                    const long row = e * (long)d + c;
                    orc_deq_row(dn_q + row * (m / 2), dn_s + row * dn_ng,
                                dn_z + row * dn_ng, dn_g, m, wrow);
                    double acc = 0.0;
                    for (long j = 0; j < m; ++j)
                        acc += h[j] * wrow[j];
                    y[c] = acc;
                }
                if (y_out)
                    memcpy(y_out + ((long)a * topk + k) * d, y, sizeof(double) * (size_t)d);
                /* weighted, fixed-order (ascending k) combine */
                const double wk = (double)w[(long)t * topk + k];
                for (int c = 0; c < d; ++c)
                    o[c] += wk * y[c];
            }
        }
        free(xv);
        free(gu);
        free(h);
        free(y);
        free(wrow);
    }
    return bad ? -1 : 0;
}

/* -------------------------------------------------------------- sampler ---- */

/*
 * The sampler of a denoising step ([kcard] "Sampler": fused_entropy computes
 * Categorical(logits).entropy() in one streaming pass; gumbel_argmax_sample
 * returns a Categorical sample by Gumbel-max, with Philox noise generated
 * inline, and the plain argmax from the same pass).
 *
 * Philox4x32-10, written from its published definition (Salmon, Moraes,
 * Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011): a
 * 4 x 32-bit counter c and a 2 x 32-bit key k; each of the 10 rounds forms
 * the 64-bit products c0 * 0xD2511F53 and c2 * 0xCD9E8D57 and sets
 *   c = { hi(c2 * 0xCD9E8D57) ^ c1 ^ k0, lo(c2 * 0xCD9E8D57),
 *         hi(c0 * 0xD2511F53) ^ c3 ^ k1, lo(c0 * 0xD2511F53) },
 * the key being advanced by the Weyl increments (0x9E3779B9, 0xBB67AE85)
 * before every round but the first.
 */
void orc_philox4x32_10(const uint32_t *ctr, const uint32_t *key, uint32_t *out)
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n1 = (uint32_t)p1;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        const uint32_t n3 = (uint32_t)p0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/*
 * Gumbel score of logit l at (row r, column v) under `seed` (reading of the
 * kernel card's "noise comes from Philox inline"; the pages do not fix the
 * stream): the Philox block with counter {v / 4, r, 0, 0} and key
 * {seed low 32 bits, seed high 32 bits}, its word v % 4 as w; the uniform
 * U = (floor(w / 2^9) + 1/2) / 2^23 from the top 23 bits of w, an exact fp32
 * number in [2^-24, 1 - 2^-24] (never 0 or 1, so the score is always
 * finite); the standard Gumbel variate G = -log(-log U); score = l + G.
 * Everything after the integer step is fp32 (the precision the GPU kernel
 * takes the decision in).
 */
float orc_gumbel_uniform(uint32_t w)
{
    return ((float)(w >> 9) + 0.5f) * (1.0f / 8388608.0f);
}

float orc_gumbel_score(float l, int r, int v, uint64_t seed)
{
    const uint32_t ctr[4] = {(uint32_t)v >> 2, (uint32_t)r, 0u, 0u};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    orc_philox4x32_10(ctr, key, w);
    const float u = orc_gumbel_uniform(w[v & 3]);
    const float g = -logf(-logf(u));
    return l + g;
}

/*
 * For each of R rows of V fp32 logits:
 *   entropy[r] = -sum_v p_v log p_v with p = softmax(row), in fp64
 *                (log-sum-exp with the row maximum subtracted);
 *   argmax[r]  = the first v with the largest logit;
 *   sample[r]  = the first v with the largest orc_gumbel_score (a draw from
 *                Categorical(softmax(row)): Gumbel-max);
 *   score[r]   = that largest score (for checking near-ties).
 * Logits are finite or -inf (a masked entry, probability 0); a row needs one
 * finite logit. Any of the outputs may be NULL. Returns 0, or -1 on invalid
 * arguments.
 */
int orc_sample(const float *logits, int R, int V, uint64_t seed, double *entropy,
               int32_t *sample, int32_t *argmax, float *score)
{
    if (R < 0 || V <= 0 || !logits)
        return -1;
#pragma omp parallel for schedule(static)
    for (long r = 0; r < R; ++r) {
        const float *row = logits + r * (long)V;
        int am = 0;
        for (int v = 1; v < V; ++v)
            if (row[v] > row[am])
                am = v;
        if (argmax)
            argmax[r] = am;
        if (entropy) {
            const double m = row[am];
            double z = 0.0, s = 0.0;
            for (int v = 0; v < V; ++v) {
                const double d = (double)row[v] - m;
                const double e = exp(d);
                z += e;
                if (e > 0.0)                 /* a -inf logit adds p log p = 0 */
                    s += e * d;
            }
            entropy[r] = log(z) - s / z;     /* -sum p (d - log z) */
        }
        if (sample || score) {
            int best = 0;
            float bs = orc_gumbel_score(row[0], (int)r, 0, seed);
            for (int v = 1; v < V; ++v) {
                const float sc = orc_gumbel_score(row[v], (int)r, v, seed);
                if (sc > bs) {
                    bs = sc;
                    best = v;
                }
            }
            if (sample)
                sample[r] = best;
            if (score)
                score[r] = bs;
        }
    }
    return 0;
}


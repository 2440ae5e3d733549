/*
 * cgo.c -- CPU oracle of the CacheGen-style KV-cache codec.
 *
 * TEST INFRASTRUCTURE.  Only tests/, the smoke check in __graft_entry__.py and the
 * cpu_baseline leg of bench.py may load this library.  The product path (libcg, HIP)
 * never calls it, and the two share no source, header, table or helper.
 *
 * Plain scalar C99, built with -O2 -ffp-contract=off and no fast-math, so every
 * floating-point operation below is one IEEE binary32 operation in program order and
 * fmaf() is the only fused operation.  Loops follow the steps of the method in the
 * order the pages give them:
 *
 *   1. tokens are cut into chunks, and each chunk into groups of G tokens whose first
 *      token is the anchor ("Guide to CacheGen", Solution pillar 2 and Implementation
 *      Step 2: windows of W tokens, first token kept as the anchor, ceil(S/W) windows,
 *      the last window may be short);
 *   2. every other token is coded as a delta from its anchor (same passage: the delta
 *      equation Delta_t = K_t - K_anchor);
 *   3. deltas are quantized with a per-layer number of levels, finer for early layers
 *      (Solution pillar 1; the gptget.net summary of CacheGen, Methodology), using a
 *      min/max affine grid as in Implementation Step 1 (quantize_tensor /
 *      dequantize_tensor) but taken per channel over the non-anchor deltas;
 *   4. symbols are entropy-coded with an arithmetic-type coder driven by empirical
 *      frequency tables (Solution pillar 3; the summary's Deep Analysis, Methodology:
 *      delta coding combined with arithmetic coding, per layer and channel), here range
 *      asymmetric numeral systems (rANS), one independent stream per (layer, K/V,
 *      channel, chunk) so chunks decode on their own (summary, Methodology: the cache is
 *      cut into chunks that are streamed);
 *   5. decoding inverts 4, then dequantizes and adds the anchor back (Implementation
 *      Step 1 dequantize_tensor, computed in float32; Step 2 decode_sequence).
 *
 * Where the pages leave a step open (the coder, the table precision, the grid, the
 * rounding, the stream layout) the readings written out in the comments below are
 * the ones this project fixed; the same list is kept with the design notes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define CGO_PROB_BITS 8u
#define CGO_PROB_TOTAL (1u << CGO_PROB_BITS) /* frequencies sum to 256 */
#define CGO_MAX_BINS 32u
#define CGO_LANES 64u                       /* channels per interleaved group */
#define CGO_STATE_LOW 0x10000u              /* coder state lives in [2^16, 2^32) */

/* ------------------------------------------------------------------------------ */
/* IEEE-754 binary16 <-> binary32, written from the format definition.             */
/* ------------------------------------------------------------------------------ */

float cgo_half_to_float(uint16_t h)
{
    uint32_t sign = h >> 15, e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -24);                 /* subnormal: m * 2^-24 (exact) */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexpf((float)(m | 0x400u), (int)e - 25); /* (1024 + m) * 2^(e-25) */
    return sign ? -v : v;
}

/* Round-to-nearest-even conversion. */
uint16_t cgo_float_to_half(float f)
{
    uint16_t sign = signbit(f) ? 0x8000u : 0;
    float a = fabsf(f);
    if (isnan(f))
        return (uint16_t)(sign | 0x7E00u);
    if (a >= 65520.0f)                              /* halfway to 2^16 rounds to even = inf */
        return (uint16_t)(sign | 0x7C00u);
    if (a < ldexpf(1.0f, -14)) {                    /* subnormal range: units of 2^-24 */
        float q = rintf(ldexpf(a, 24));             /* default rounding mode: nearest-even */
        return (uint16_t)(sign | (uint16_t)q);      /* q == 1024 encodes the smallest normal */
    }
    int e;
    frexpf(a, &e);                                  /* a = frac * 2^e, frac in [0.5, 1) */
    e -= 1;                                         /* a in [2^e, 2^(e+1)) */
    float m = rintf(ldexpf(a, 10 - e));             /* in [1024, 2048] */
    if (m >= 2048.0f) {
        m = 1024.0f;
        e += 1;
    }
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)((uint32_t)m - 1024u));
}

void cgo_half_to_float_n(const uint16_t *h, float *f, size_t n)
{
    for (size_t i = 0; i < n; i++)
        f[i] = cgo_half_to_float(h[i]);
}

void cgo_float_to_half_n(const float *f, uint16_t *h, size_t n)
{
    for (size_t i = 0; i < n; i++)
        h[i] = cgo_float_to_half(f[i]);
}

static int half_is_finite(uint16_t h) { return ((h >> 10) & 0x1Fu) != 0x1Fu; }

/* ------------------------------------------------------------------------------ */
/* Segmentation: chunks of Tc tokens, groups of G tokens restarting at every chunk. */
/* ------------------------------------------------------------------------------ */

uint32_t cgo_num_chunks(uint32_t S, uint32_t Tc) { return (S + Tc - 1) / Tc; }

uint32_t cgo_chunk_len(uint32_t S, uint32_t Tc, uint32_t k)
{
    uint32_t t0 = k * Tc;
    return (S - t0 < Tc) ? S - t0 : Tc;
}

uint32_t cgo_groups_in(uint32_t len, uint32_t G) { return (len + G - 1) / G; }

int cgo_is_anchor(uint32_t t, uint32_t G, uint32_t Tc) { return ((t % Tc) % G) == 0; }

uint32_t cgo_anchor_of(uint32_t t, uint32_t G, uint32_t Tc)
{
    uint32_t k0 = (t / Tc) * Tc;
    return k0 + ((t - k0) / G) * G;
}

/* ------------------------------------------------------------------------------ */
/* Shapes.                                                                          */
/* ------------------------------------------------------------------------------ */

typedef struct {
    uint32_t L, H, d, S, G, Tc;
    const uint8_t *bins; /* [L][2]: bin count of (layer l, K/V kv) at l * 2 + kv, each in [2, 32] */
} cgo_shape;

static size_t kv_index(const cgo_shape *p, uint32_t l, uint32_t kv, uint32_t t, uint32_t c)
{
    size_t C = (size_t)p->H * p->d;
    return (((size_t)l * 2 + kv) * p->S + t) * C + c;
}

/* ------------------------------------------------------------------------------ */
/* Step 2-3a: per-channel range of the anchor deltas.                               */
/*   Delta = f32(x_t) - f32(x_anchor)    (one binary32 subtraction)                 */
/*   lo, hi = min / max over every non-anchor token of the channel (all chunks)     */
/*   except the first n_sink tokens of the sequence, which are kept in fp16         */
/*   ("Guide to CacheGen", Best Practices: protect the attention sinks);            */
/*   lo = hi = 0 when the channel has no non-anchor token; a zero bound is +0;      */
/*   with the outlier table on (outlier_ppm > 0), [lo, hi] is narrowed to a central */
/*   range first (clip_range below);                                                */
/*   w = (hi - lo) / (N - 1);  r = 1 / w, or 0 when w == 0.                          */
/* Returns -4 if any input element is Inf or NaN, else 0.                           */
/* ------------------------------------------------------------------------------ */

#define CGO_FINE_BINS 256u

/* Grid point j of the fine grid over [lo, hi]: fma(j, wf, lo), wf = (hi - lo) / 256. */
static float fine_point(uint32_t j, float wf, float lo) { return fmaf((float)j, wf, lo); }

/* Fine-grid interval of a delta: the largest j in [0, 255] with fine_point(j) <= delta
 * (0 if none).  The points do not decrease with j, so a binary search finds it. */
static uint32_t fine_index(float delta, float wf, float lo)
{
    uint32_t a = 0, b = CGO_FINE_BINS - 1u;
    while (a < b) {
        uint32_t mid = (a + b + 1u) / 2u;
        if (fine_point(mid, wf, lo) <= delta)
            a = mid;
        else
            b = mid - 1u;
    }
    return a;
}

/* Central range for the sparse outlier table ("Guide to CacheGen", Solution pillar 3:
 * outliers go to a compact sparse table so that they do not distort the regular
 * distribution).  The pages give no rule; the reading taken here: count the row's n
 * deltas in the 256 intervals [p_j, p_j+1) of the fine grid p_j = fma(j, wf, lo) over
 * [lo, hi] (the last interval open above); with the budget b = floor(n * ppm / 10^6),
 * drop whole intervals from the bottom while the dropped count stays <= b, and from the
 * top likewise:
 *   j_lo = the largest j with count(intervals < j) <= b,
 *   j_hi = the smallest j with count(intervals > j) <= b,
 *   lo' = p_{j_lo}, hi' = p_{j_hi + 1} (hi when j_hi = 255), at most hi.
 * Every delta below lo' lies in a dropped interval, and so does every delta above hi',
 * so at most b deltas fall outside each end.  Nothing is narrowed when w is 0 or n is 0. */
static void clip_range(const float *d, size_t n, uint32_t ppm, float *lo_io, float *hi_io)
{
    float lo = *lo_io, hi = *hi_io;
    float wf = (hi - lo) / (float)CGO_FINE_BINS;
    if (n == 0 || ppm == 0 || !(wf > 0.0f))
        return;
    uint64_t cnt[CGO_FINE_BINS];
    memset(cnt, 0, sizeof cnt);
    for (size_t i = 0; i < n; i++)
        cnt[fine_index(d[i], wf, lo)] += 1;
    uint64_t budget = ((uint64_t)n * ppm) / 1000000u;
    uint32_t j_lo = 0, j_hi = CGO_FINE_BINS - 1u;
    uint64_t below = 0;
    for (uint32_t j = 1; j < CGO_FINE_BINS; j++) {
        below += cnt[j - 1];
        if (below > budget)
            break;
        j_lo = j;
    }
    uint64_t above = 0;
    for (uint32_t j = CGO_FINE_BINS - 1u; j > 0; j--) {
        above += cnt[j];
        if (above > budget)
            break;
        j_hi = j - 1u;
    }
    float lo_c = fine_point(j_lo, wf, lo);
    float hi_c = (j_hi == CGO_FINE_BINS - 1u) ? hi : fine_point(j_hi + 1u, wf, lo);
    if (hi_c > hi)
        hi_c = hi;
    *lo_io = lo_c + 0.0f;
    *hi_io = hi_c + 0.0f;
}

int cgo_range(uint32_t L, uint32_t H, uint32_t d, uint32_t S, uint32_t G, uint32_t Tc,
              const uint8_t *bins, const uint16_t *X, float *lo_out, float *w_out, float *r_out,
              uint32_t n_sink, uint32_t outlier_ppm)
{
    cgo_shape p = {L, H, d, S, G, Tc, bins};
    uint32_t C = H * d;
    size_t total = (size_t)L * 2 * S * C;
    for (size_t i = 0; i < total; i++)
        if (!half_is_finite(X[i]))
            return -4;
    float *dl = (float *)malloc(sizeof(float) * (S ? S : 1));
    for (uint32_t l = 0; l < L; l++)
        for (uint32_t kv = 0; kv < 2; kv++)
            for (uint32_t c = 0; c < C; c++) {
                size_t n = 0;
                float lo = 0.0f, hi = 0.0f;
                for (uint32_t t = n_sink; t < S; t++) {
                    if (cgo_is_anchor(t, G, Tc))
                        continue;
                    uint32_t a = cgo_anchor_of(t, G, Tc);
                    float delta = cgo_half_to_float(X[kv_index(&p, l, kv, t, c)]) -
                                  cgo_half_to_float(X[kv_index(&p, l, kv, a, c)]);
                    if (n == 0) {
                        lo = hi = delta;
                    } else {
                        if (delta < lo) lo = delta;
                        if (delta > hi) hi = delta;
                    }
                    dl[n++] = delta;
                }
                size_t row = ((size_t)l * 2 + kv) * C + c;
                /* the sign of a zero bound is not meaningful: +0 + -0 = +0 fixes it */
                lo = lo + 0.0f;
                hi = hi + 0.0f;
                clip_range(dl, n, outlier_ppm, &lo, &hi);
                float w = (hi - lo) / (float)(bins[l * 2 + kv] - 1u);
                lo_out[row] = lo;
                w_out[row] = w;
                r_out[row] = (w > 0.0f) ? 1.0f / w : 0.0f;
            }
    free(dl);
    return 0;
}

/* Step 3b: q = clamp(floor(fma(Delta - lo, r, 0.5)), 0, N - 1): nearest grid point
 * lo + q*w, ties upward.  Anchors carry no symbol (their slot is written as 0). */
static uint8_t quantize_one(float delta, float lo, float r, uint32_t N)
{
    float v = floorf(fmaf(delta - lo, r, 0.5f));
    if (!(v > 0.0f))
        return 0;
    if (v > (float)(N - 1u))
        return (uint8_t)(N - 1u);
    return (uint8_t)v;
}

/* An element is off its grid when the clamp above changes its code: its nearest grid
 * point is more than half a step away (floor(fma(Delta - lo, r, 0.5)) outside [0, N-1]),
 * or the grid has zero width (r = 0: the single point lo) and does not hold it, or
 * Delta is NaN (no grid point holds it; quantize_one codes it 0).  The
 * tables' own cache has no off-grid element except outside a clipped central range; a
 * cache coded with another cache's tables may have more. */
static int off_grid(float delta, float lo, float r, uint32_t N)
{
    if (r == 0.0f)
        return delta != lo;
    float v = floorf(fmaf(delta - lo, r, 0.5f));
    return !(v >= 0.0f && v <= (float)(N - 1u));   /* a NaN Delta: off every grid */
}

void cgo_quantize(uint32_t L, uint32_t H, uint32_t d, uint32_t S, uint32_t G, uint32_t Tc,
                  const uint8_t *bins, const uint16_t *X, const float *lo, const float *r,
                  uint32_t t_begin, uint32_t t_end, uint8_t *sym /* [L][2][S][C] */)
{
    cgo_shape p = {L, H, d, S, G, Tc, bins};
    uint32_t C = H * d;
    for (uint32_t l = 0; l < L; l++)
        for (uint32_t kv = 0; kv < 2; kv++)
            for (uint32_t t = t_begin; t < t_end; t++)
                for (uint32_t c = 0; c < C; c++) {
                    size_t i = kv_index(&p, l, kv, t, c);
                    if (cgo_is_anchor(t, G, Tc)) {
                        sym[i] = 0;
                        continue;
                    }
                    size_t row = ((size_t)l * 2 + kv) * C + c;
                    uint32_t a = cgo_anchor_of(t, G, Tc);
                    float delta = cgo_half_to_float(X[i]) -
                                  cgo_half_to_float(X[kv_index(&p, l, kv, a, c)]);
                    sym[i] = quantize_one(delta, lo[row], r[row], bins[l * 2 + kv]);
                }
}

/* ------------------------------------------------------------------------------ */
/* Step 4a: empirical frequency table per (layer, K/V, channel), shared by all     */
/* chunks of the channel.  Frequencies sum to T = 256 and every symbol gets f >= 1:  */
/*   f[s] = 1 + floor(count[s] * (T - N) / n)     (n = sum of counts; 0 if n == 0)   */
/* and the remainder T - sum(f) goes to the most frequent symbol (lowest index on    */
/* ties).  freqs is [L][2][C][32], entries beyond N are 0.                           */
/* ------------------------------------------------------------------------------ */
void cgo_freqs_from_counts(const uint64_t *count, uint32_t N, uint16_t *f)
{
    uint64_t n = 0;
    for (uint32_t s = 0; s < N; s++)
        n += count[s];
    uint32_t sum = 0, best = 0;
    for (uint32_t s = 0; s < N; s++) {
        uint64_t extra = n ? (count[s] * (uint64_t)(CGO_PROB_TOTAL - N)) / n : 0;
        f[s] = (uint16_t)(1u + extra);
        sum += f[s];
        if (count[s] > count[best])
            best = s;
    }
    f[best] = (uint16_t)(f[best] + (CGO_PROB_TOTAL - sum));
}

/* Symbol counts per channel row over the tokens the range covers (non-anchor tokens
 * from n_sink on). */
void cgo_histograms(uint32_t L, uint32_t H, uint32_t d, uint32_t S, uint32_t G, uint32_t Tc,
                    const uint8_t *bins, const uint8_t *sym, uint64_t *counts /* [L][2][C][32] */,
                    uint32_t n_sink)
{
    cgo_shape p = {L, H, d, S, G, Tc, bins};
    uint32_t C = H * d;
    memset(counts, 0, sizeof(uint64_t) * (size_t)L * 2 * C * CGO_MAX_BINS);
    for (uint32_t l = 0; l < L; l++)
        for (uint32_t kv = 0; kv < 2; kv++)
            for (uint32_t t = n_sink; t < S; t++) {
                if (cgo_is_anchor(t, G, Tc))
                    continue;
                for (uint32_t c = 0; c < C; c++) {
                    size_t row = ((size_t)l * 2 + kv) * C + c;
                    counts[row * CGO_MAX_BINS + sym[kv_index(&p, l, kv, t, c)]] += 1;
                }
            }
}

void cgo_freqs(uint32_t L, uint32_t C, const uint8_t *bins, const uint64_t *counts,
               uint16_t *freqs /* [L][2][C][32] */)
{
    memset(freqs, 0, sizeof(uint16_t) * (size_t)L * 2 * C * CGO_MAX_BINS);
    for (uint32_t l = 0; l < L; l++)
        for (uint32_t kv = 0; kv < 2; kv++)
            for (uint32_t c = 0; c < C; c++) {
                size_t row = ((size_t)l * 2 + kv) * C + c;
                cgo_freqs_from_counts(counts + row * CGO_MAX_BINS, bins[l * 2 + kv],
                                      freqs + row * CGO_MAX_BINS);
            }
}

/* ------------------------------------------------------------------------------ */
/* Step 4b: rANS (J. Duda, "Asymmetric numeral systems", 2009/2013), probabilities   */
/* in units of 1/256, a 32-bit state kept in [2^16, 2^32) and 16-bit output words.    */
/* With cdf[s] = f[0] + ... + f[s-1]:                                                  */
/*   coding step   C(s, x) = floor(x / f[s]) * 256 + (x mod f[s]) + cdf[s]            */
/*   decoding step slot = x mod 256; s = the symbol with cdf[s] <= slot < cdf[s+1];  */
/*                 x = f[s] * floor(x / 256) + slot - cdf[s]     (inverts C exactly)  */
/* The encoder runs over x_{m-1} .. x_0 from x = 2^16; before coding x_i it shifts    */
/* out the low 16 bits of x when x >= f[s] * 2^24, which keeps C(s, x) below 2^32.    */
/* The decoder runs forward from the final encoder state (the stream's first two     */
/* words, high half first) and, after decoding x_i, pulls in a word exactly when x    */
/* fell below 2^16 -- the word the encoder shifted out before coding x_i -- so it     */
/* reads the words in the reverse of the order they were produced and ends in state   */
/* 2^16.  The encoder never shifts before x_{m-1} (x = 2^16 < f * 2^24), so no word   */
/* follows the last symbol.  m == 0 gives an empty stream.                            */
/* Words are returned in read order; steps_out receives the decoder step reading each */
/* word: -1 for the two state words, else i.  Returns the number of words.            */
/* ------------------------------------------------------------------------------ */
static void make_cdf(const uint16_t *f, uint32_t N, uint32_t *cdf)
{
    cdf[0] = 0;
    for (uint32_t s = 0; s < N; s++)
        cdf[s + 1] = cdf[s] + f[s];
}

uint32_t cgo_rans_encode(const uint8_t *x, uint32_t m, const uint16_t *f, uint32_t N,
                         uint16_t *words, int32_t *steps_out)
{
    uint32_t cdf[CGO_MAX_BINS + 1];
    make_cdf(f, N, cdf);
    if (m == 0)
        return 0;
    /* produced[j] / step[j]: words in production order (highest step first) */
    uint16_t *produced = (uint16_t *)malloc(sizeof(uint16_t) * (m + 1));
    int32_t *step = (int32_t *)malloc(sizeof(int32_t) * (m + 1));
    uint32_t np = 0;
    uint32_t state = CGO_STATE_LOW;
    for (uint32_t i = m; i-- > 0;) {
        uint32_t s = x[i], fs = f[s];
        if ((uint64_t)state >= ((uint64_t)fs << 24)) {
            produced[np] = (uint16_t)(state & 0xFFFFu);
            step[np++] = (int32_t)i;
            state >>= 16;
        }
        state = (state / fs) * CGO_PROB_TOTAL + state % fs + cdf[s];
    }
    uint32_t nw = 0;
    words[nw] = (uint16_t)(state >> 16);
    if (steps_out) steps_out[nw] = -1;
    nw++;
    words[nw] = (uint16_t)(state & 0xFFFFu);
    if (steps_out) steps_out[nw] = -1;
    nw++;
    for (uint32_t j = np; j-- > 0;) {
        words[nw] = produced[j];
        if (steps_out) steps_out[nw] = step[j];
        nw++;
    }
    free(produced);
    free(step);
    return nw;
}

/* Decodes m symbols; words past the end of the stream read as 0.  Returns the number
 * of words consumed; *final_state (if given) receives the state after the last symbol
 * (2^16 for an intact stream). */
uint32_t cgo_rans_decode(const uint16_t *words, uint32_t nw, uint32_t m, const uint16_t *f,
                         uint32_t N, uint8_t *x_out, uint32_t *final_state)
{
    uint32_t cdf[CGO_MAX_BINS + 1];
    make_cdf(f, N, cdf);
    if (final_state) *final_state = CGO_STATE_LOW;
    if (m == 0)
        return 0;
    uint32_t pos = 0;
#define NEXTW() (pos < nw ? words[pos++] : (pos++, 0u))
    uint32_t state = NEXTW();
    state = (state << 16) | NEXTW();
    for (uint32_t i = 0; i < m; i++) {
        uint32_t slot = state % CGO_PROB_TOTAL, s = 0;
        for (uint32_t j = 1; j < N; j++)
            if (cdf[j] <= slot)
                s = j;
        state = f[s] * (state / CGO_PROB_TOTAL) + slot - cdf[s];
        x_out[i] = (uint8_t)s;
        if (i + 1 < m && state < CGO_STATE_LOW)
            state = (state << 16) | NEXTW();
    }
#undef NEXTW
    if (final_state) *final_state = state;
    return pos;
}

/* ------------------------------------------------------------------------------ */
/* Container pieces.                                                                */
/*   group  = (chunk k, layer l, K/V kv, block b) with lanes 0..63 <-> channels      */
/*            64b .. 64b+63 (channels >= C absent); groups are numbered in that      */
/*            row-major order over chunks [k_begin, k_end).                          */
/*   A group's word sequence holds the words of all its lanes' streams in the order  */
/*   the 64 decoders read them when they run in lockstep: first words 0 and 1 of     */
/*   lane 0, lane 1, ...; then, for step i = 0 .. m-2, the word each lane reads at   */
/*   step i, lanes in ascending order.                                               */
/*   offsets[g] = first word of group g in the payload, offsets[n_groups] = total.   */
/*   anchors: fp16, for each chunk (ascending) [L][2][groups of the chunk][C].       */
/* ------------------------------------------------------------------------------ */

static uint32_t n_blocks(uint32_t C) { return (C + CGO_LANES - 1) / CGO_LANES; }

uint64_t cgo_num_groups(uint32_t L, uint32_t C, uint32_t k_begin, uint32_t k_end)
{
    return (uint64_t)(k_end - k_begin) * L * 2 * n_blocks(C);
}

uint64_t cgo_anchor_rows(uint32_t L, uint32_t S, uint32_t G, uint32_t Tc, uint32_t k_begin,
                         uint32_t k_end)
{
    uint64_t rows = 0;
    for (uint32_t k = k_begin; k < k_end; k++)
        rows += (uint64_t)L * 2 * cgo_groups_in(cgo_chunk_len(S, Tc, k), G);
    return rows;
}

/* ------------------------------------------------------------------------------ */
/* 8-bit anchors (optional): the anchor token is "quantized and stored with high    */
/* precision" ("Guide to CacheGen", Solution pillar 2), read here as 256 levels on  */
/* a min-offset grid per (layer, K/V, channel) over its anchor tokens (all chunks), */
/* the same grid form as the deltas':                                              */
/*   alo, ahi = min / max of f32(x) over the anchor tokens (+0 for a zero bound);   */
/*   aw = (ahi - alo) / 255; ar = 1 / aw, or 0 when aw == 0;                        */
/*   code = clamp(floor(fma(x - alo, ar, 0.5)), 0, 255);                            */
/*   anchor value = fp16_rne(fma(code, aw, alo)).                                   */
/* The deltas are then taken against the anchor value, so the encoder and decoder   */
/* agree on it and the delta grid's bound is unchanged.                             */
/* ------------------------------------------------------------------------------ */
void cgo_anchor_grid(uint32_t L, uint32_t H, uint32_t d, uint32_t S, uint32_t G, uint32_t Tc,
                     const uint16_t *X, float *alo, float *aw, float *ar)
{
    cgo_shape p = {L, H, d, S, G, Tc, NULL};
    uint32_t C = H * d;
    for (uint32_t l = 0; l < L; l++)
        for (uint32_t kv = 0; kv < 2; kv++)
            for (uint32_t c = 0; c < C; c++) {
                float lo = 0.0f, hi = 0.0f;
                int any = 0;
                for (uint32_t t = 0; t < S; t++) {
                    if (!cgo_is_anchor(t, G, Tc))
                        continue;
                    float x = cgo_half_to_float(X[kv_index(&p, l, kv, t, c)]);
                    if (!any || x < lo) lo = x;
                    if (!any || x > hi) hi = x;
                    any = 1;
                }
                lo = lo + 0.0f;
                hi = hi + 0.0f;
                size_t row = ((size_t)l * 2 + kv) * C + c;
                float w = (hi - lo) / 255.0f;
                alo[row] = lo;
                aw[row] = w;
                ar[row] = (w > 0.0f) ? 1.0f / w : 0.0f;
            }
}

static uint8_t anchor_code(uint16_t x, float alo, float ar)
{
    return quantize_one(cgo_half_to_float(x), alo, ar, 256u);
}

static uint16_t anchor_value(uint8_t code, float alo, float aw)
{
    return cgo_float_to_half(fmaf((float)code, aw, alo));
}

/* X_out = X with every anchor token replaced by its anchor value. */
void cgo_snap_anchors(uint32_t L, uint32_t H, uint32_t d, uint32_t S, uint32_t G, uint32_t Tc,
                      const uint16_t *X, const float *alo, const float *aw, const float *ar,
                      uint16_t *X_out)
{
    cgo_shape p = {L, H, d, S, G, Tc, NULL};
    uint32_t C = H * d;
    memcpy(X_out, X, sizeof(uint16_t) * (size_t)L * 2 * S * C);
    for (uint32_t l = 0; l < L; l++)
        for (uint32_t kv = 0; kv < 2; kv++)
            for (uint32_t t = 0; t < S; t++) {
                if (!cgo_is_anchor(t, G, Tc))
                    continue;
                for (uint32_t c = 0; c < C; c++) {
                    size_t row = ((size_t)l * 2 + kv) * C + c, i = kv_index(&p, l, kv, t, c);
                    X_out[i] = anchor_value(anchor_code(X[i], alo[row], ar[row]), alo[row], aw[row]);
                }
            }
}

/* Anchor codes of chunks [k_begin, k_end) in the anchors section's row order. */
void cgo_anchor_codes(uint32_t L, uint32_t H, uint32_t d, uint32_t S, uint32_t G, uint32_t Tc,
                      const uint16_t *X, const float *alo, const float *ar, uint32_t k_begin,
                      uint32_t k_end, uint8_t *codes_out)
{
    cgo_shape p = {L, H, d, S, G, Tc, NULL};
    uint32_t C = H * d;
    size_t r = 0;
    for (uint32_t k = k_begin; k < k_end; k++) {
        uint32_t ng = cgo_groups_in(cgo_chunk_len(S, Tc, k), G);
        for (uint32_t l = 0; l < L; l++)
            for (uint32_t kv = 0; kv < 2; kv++)
                for (uint32_t g = 0; g < ng; g++, r++)
                    for (uint32_t c = 0; c < C; c++) {
                        size_t row = ((size_t)l * 2 + kv) * C + c;
                        codes_out[r * C + c] =
                            anchor_code(X[kv_index(&p, l, kv, k * Tc + g * G, c)], alo[row], ar[row]);
                    }
    }
}

/* The fp16 anchor values of an anchors section of codes (same row order). */
void cgo_anchors_from_codes(uint32_t L, uint32_t C, uint32_t S, uint32_t G, uint32_t Tc,
                            const uint8_t *codes, const float *alo, const float *aw,
                            uint32_t k_begin, uint32_t k_end, uint16_t *anchors_out)
{
    size_t r = 0;
    for (uint32_t k = k_begin; k < k_end; k++) {
        uint32_t ng = cgo_groups_in(cgo_chunk_len(S, Tc, k), G);
        for (uint32_t l = 0; l < L; l++)
            for (uint32_t kv = 0; kv < 2; kv++)
                for (uint32_t g = 0; g < ng; g++, r++)
                    for (uint32_t c = 0; c < C; c++) {
                        size_t row = ((size_t)l * 2 + kv) * C + c;
                        anchors_out[r * C + c] = anchor_value(codes[r * C + c], alo[row], aw[row]);
                    }
    }
}

/* Copies anchors into anchors_out ([rows][C] fp16). */
void cgo_anchors(uint32_t L, uint32_t H, uint32_t d, uint32_t S, uint32_t G, uint32_t Tc,
                 const uint16_t *X, uint32_t k_begin, uint32_t k_end, uint16_t *anchors_out)
{
    cgo_shape p = {L, H, d, S, G, Tc, NULL};
    uint32_t C = H * d;
    size_t row = 0;
    for (uint32_t k = k_begin; k < k_end; k++) {
        uint32_t len = cgo_chunk_len(S, Tc, k), ng = cgo_groups_in(len, G);
        for (uint32_t l = 0; l < L; l++)
            for (uint32_t kv = 0; kv < 2; kv++)
                for (uint32_t g = 0; g < ng; g++, row++)
                    for (uint32_t c = 0; c < C; c++)
                        anchors_out[row * C + c] = X[kv_index(&p, l, kv, k * Tc + g * G, c)];
    }
}

/* ------------------------------------------------------------------------------ */
/* Sparse outlier table ("Guide to CacheGen", Solution pillar 3).  An entry holds     */
/* one element exactly, in fp16, and is written over the decoded value.  Elements    */
/* taken: every element of the chunks [k_begin, k_end) from token n_sink on that is   */
/* off its grid (off_grid above): a non-anchor token whose delta (against its        */
/* anchor's decoded value) is off the delta grid, or, with 8-bit anchors, an anchor   */
/* token whose code is off the anchor grid.  The stream still codes the clamped       */
/* symbol of such an element, so the streams do not change.                            */
/* Entries are grouped like the payload: for each group (chunk, layer, K/V, block) in */
/* container order, ascending token, then ascending lane, with                        */
/*   key   = (t - k * Tc) << 6 | lane      (token within the chunk, lane in the block) */
/*   value = the element's fp16 bits;                                                  */
/* offsets[g] = first entry of group g, offsets[n_groups] = the total.                 */
/* X is the cache, Xs the same cache with anchor tokens replaced by their decoded     */
/* values (X itself for fp16 anchors); alo / ar are NULL for fp16 anchors.  With      */
/* keys == NULL nothing is stored and the elements are only counted (this is the      */
/* count of clamped elements of a container coded without the table).                 */
/* Returns the number of elements taken.                                               */
/* ------------------------------------------------------------------------------ */
uint64_t cgo_outliers(uint32_t L, uint32_t H, uint32_t d, uint32_t S, uint32_t G, uint32_t Tc,
                      const uint8_t *bins, const uint16_t *X, const uint16_t *Xs,
                      const float *lo, const float *r, const float *alo, const float *ar,
                      uint32_t n_sink, uint32_t k_begin, uint32_t k_end, uint64_t *offsets,
                      uint32_t *keys, uint16_t *values)
{
    cgo_shape p = {L, H, d, S, G, Tc, bins};
    uint32_t C = H * d, NB = n_blocks(C);
    uint64_t n = 0, g = 0;
    for (uint32_t k = k_begin; k < k_end; k++) {
        uint32_t t0 = k * Tc, len = cgo_chunk_len(S, Tc, k);
        for (uint32_t l = 0; l < L; l++)
            for (uint32_t kv = 0; kv < 2; kv++)
                for (uint32_t b = 0; b < NB; b++, g++) {
                    if (offsets) offsets[g] = n;
                    uint32_t lanes = (C - b * CGO_LANES < CGO_LANES) ? C - b * CGO_LANES : CGO_LANES;
                    for (uint32_t t = t0; t < t0 + len; t++) {
                        if (t < n_sink)
                            continue;
                        for (uint32_t lane = 0; lane < lanes; lane++) {
                            uint32_t c = b * CGO_LANES + lane;
                            size_t row = ((size_t)l * 2 + kv) * C + c, i = kv_index(&p, l, kv, t, c);
                            int off;
                            if (cgo_is_anchor(t, G, Tc)) {
                                off = alo ? off_grid(cgo_half_to_float(X[i]), alo[row], ar[row], 256u) : 0;
                            } else {
                                uint32_t a = cgo_anchor_of(t, G, Tc);
                                float delta = cgo_half_to_float(Xs[i]) -
                                              cgo_half_to_float(Xs[kv_index(&p, l, kv, a, c)]);
                                off = off_grid(delta, lo[row], r[row], bins[l * 2 + kv]);
                            }
                            if (!off)
                                continue;
                            if (keys) {
                                keys[n] = ((t - t0) << 6) | lane;
                                values[n] = X[i];
                            }
                            n++;
                        }
                    }
                }
    }
    if (offsets) offsets[g] = n;
    return n;
}

/* Writes the outlier entries of chunks [k_begin, k_end) into out ([L][2][S][C] fp16).
 * Returns 0, or -5 when the offsets or a key do not fit the container's groups. */
int cgo_apply_outliers(uint32_t L, uint32_t H, uint32_t d, uint32_t S, uint32_t Tc,
                       uint32_t k_begin, uint32_t k_end, const uint64_t *offsets,
                       const uint32_t *keys, const uint16_t *values, uint64_t n_entries,
                       uint16_t *out)
{
    cgo_shape p = {L, H, d, S, 1, Tc, NULL};
    uint32_t C = H * d, NB = n_blocks(C);
    uint64_t g = 0;
    for (uint32_t k = k_begin; k < k_end; k++) {
        uint32_t t0 = k * Tc, len = cgo_chunk_len(S, Tc, k);
        for (uint32_t l = 0; l < L; l++)
            for (uint32_t kv = 0; kv < 2; kv++)
                for (uint32_t b = 0; b < NB; b++, g++) {
                    uint64_t beg = offsets[g], end = offsets[g + 1];
                    if (end < beg || end > n_entries)
                        return -5;
                    for (uint64_t e = beg; e < end; e++) {
                        uint32_t u = keys[e] >> 6, lane = keys[e] & 63u;
                        if (u >= len || b * CGO_LANES + lane >= C)
                            return -5;
                        out[kv_index(&p, l, kv, t0 + u, b * CGO_LANES + lane)] = values[e];
                    }
                }
    }
    return 0;
}

/* Encodes chunks [k_begin, k_end).  Writes offsets (n_groups + 1 entries) and the
 * payload; returns the total number of words, or -1 if payload_cap is too small. */
int64_t cgo_encode_payload(uint32_t L, uint32_t H, uint32_t d, uint32_t S, uint32_t G,
                           uint32_t Tc, const uint8_t *bins, const uint8_t *sym,
                           const uint16_t *freqs, uint32_t k_begin, uint32_t k_end,
                           uint64_t *offsets, uint16_t *payload, uint64_t payload_cap)
{
    cgo_shape p = {L, H, d, S, G, Tc, bins};
    uint32_t C = H * d, NB = n_blocks(C);
    uint64_t total = 0, g = 0;
    uint8_t *x = (uint8_t *)malloc(Tc + 1);
    uint16_t *w[CGO_LANES];
    int32_t *st[CGO_LANES];
    uint32_t nw[CGO_LANES], rd[CGO_LANES];
    for (uint32_t i = 0; i < CGO_LANES; i++) {
        w[i] = (uint16_t *)malloc(sizeof(uint16_t) * (Tc + 2));
        st[i] = (int32_t *)malloc(sizeof(int32_t) * (Tc + 2));
    }
    int64_t result = 0;
    for (uint32_t k = k_begin; k < k_end && result == 0; k++) {
        uint32_t t0 = k * Tc, len = cgo_chunk_len(S, Tc, k);
        for (uint32_t l = 0; l < L; l++)
            for (uint32_t kv = 0; kv < 2; kv++)
                for (uint32_t b = 0; b < NB; b++, g++) {
                    offsets[g] = total;
                    uint32_t lanes = (C - b * CGO_LANES < CGO_LANES) ? C - b * CGO_LANES : CGO_LANES;
                    uint32_t m = 0;
                    for (uint32_t lane = 0; lane < lanes; lane++) {
                        uint32_t c = b * CGO_LANES + lane;
                        m = 0;
                        for (uint32_t t = t0; t < t0 + len; t++)
                            if (!cgo_is_anchor(t, G, Tc))
                                x[m++] = sym[kv_index(&p, l, kv, t, c)];
                        size_t row = ((size_t)l * 2 + kv) * C + c;
                        nw[lane] = cgo_rans_encode(x, m, freqs + row * CGO_MAX_BINS, bins[l * 2 + kv],
                                                   w[lane], st[lane]);
                        rd[lane] = 0;
                    }
                    /* merge in the order the lockstep decoders read the words */
                    uint64_t need = 0;
                    for (uint32_t lane = 0; lane < lanes; lane++)
                        need += nw[lane];
                    if (total + need > payload_cap) {
                        result = -1;
                        break;
                    }
                    for (int32_t step = -1; step < (int32_t)m; step++)
                        for (uint32_t lane = 0; lane < lanes; lane++)
                            while (rd[lane] < nw[lane] && st[lane][rd[lane]] == step)
                                payload[total++] = w[lane][rd[lane]++];
                }
    }
    if (result == 0) {
        offsets[g] = total;
        result = (int64_t)total;
    }
    for (uint32_t i = 0; i < CGO_LANES; i++) {
        free(w[i]);
        free(st[i]);
    }
    free(x);
    return result;
}

/* ------------------------------------------------------------------------------ */
/* Step 5: decode chunks [k_begin, k_end) into out ([L][2][S][C] fp16):             */
/*   anchors are copied bit for bit;                                                 */
/*   other tokens: y = fp16_rne(f32(anchor) + fma(f32(q), w, lo)).                   */
/* Lanes of a group run in lockstep so that they read the interleaved words in the   */
/* order they were written.  Reads past the group's end return 0.                    */
/* Returns 0, or -5 when a group's declared extent is inconsistent.                  */
/* ------------------------------------------------------------------------------ */
int cgo_decode(uint32_t L, uint32_t H, uint32_t d, uint32_t S, uint32_t G, uint32_t Tc,
               const uint8_t *bins, const float *lo, const float *w, const uint16_t *freqs,
               uint32_t k_begin, uint32_t k_end, const uint64_t *offsets,
               const uint16_t *payload, uint64_t payload_words, const uint16_t *anchors,
               uint16_t *out)
{
    cgo_shape p = {L, H, d, S, G, Tc, bins};
    uint32_t C = H * d, NB = n_blocks(C);
    uint64_t g = 0, arow_chunk = 0;
    for (uint32_t k = k_begin; k < k_end; k++) {
        uint32_t t0 = k * Tc, len = cgo_chunk_len(S, Tc, k), ng = cgo_groups_in(len, G);
        uint32_t m = len - ng;
        for (uint32_t l = 0; l < L; l++)
            for (uint32_t kv = 0; kv < 2; kv++) {
                const uint16_t *arows = anchors + (arow_chunk + ((uint64_t)l * 2 + kv) * ng) * C;
                /* anchors, bit-exact */
                for (uint32_t gi = 0; gi < ng; gi++)
                    for (uint32_t c = 0; c < C; c++)
                        out[kv_index(&p, l, kv, t0 + gi * G, c)] = arows[(size_t)gi * C + c];
                for (uint32_t b = 0; b < NB; b++, g++) {
                    uint64_t beg = offsets[g], end = offsets[g + 1];
                    if (end < beg || end > payload_words)
                        return -5;
                    uint32_t lanes = (C - b * CGO_LANES < CGO_LANES) ? C - b * CGO_LANES : CGO_LANES;
                    uint32_t state[CGO_LANES], cdf[CGO_LANES][CGO_MAX_BINS + 1];
                    uint64_t cur = beg;
                    if (m == 0)
                        continue;
#define GROUPW() (cur < end ? payload[cur++] : (cur++, 0u))
                    for (uint32_t lane = 0; lane < lanes; lane++) {
                        size_t row = ((size_t)l * 2 + kv) * C + b * CGO_LANES + lane;
                        cdf[lane][0] = 0;
                        for (uint32_t s = 0; s < bins[l * 2 + kv]; s++)
                            cdf[lane][s + 1] = cdf[lane][s] + freqs[row * CGO_MAX_BINS + s];
                        uint32_t hi16 = GROUPW();
                        state[lane] = (hi16 << 16) | GROUPW();
                    }
                    uint32_t i = 0;
                    for (uint32_t t = t0; t < t0 + len; t++) {
                        if (cgo_is_anchor(t, G, Tc))
                            continue;
                        uint32_t a = cgo_anchor_of(t, G, Tc);
                        for (uint32_t lane = 0; lane < lanes; lane++) {
                            uint32_t c = b * CGO_LANES + lane;
                            size_t row = ((size_t)l * 2 + kv) * C + c;
                            uint32_t slot = state[lane] % CGO_PROB_TOTAL, s = 0;
                            for (uint32_t j = 1; j < bins[l * 2 + kv]; j++)
                                if (cdf[lane][j] <= slot)
                                    s = j;
                            state[lane] = (cdf[lane][s + 1] - cdf[lane][s]) *
                                              (state[lane] / CGO_PROB_TOTAL) + slot - cdf[lane][s];
                            float anchor = cgo_half_to_float(out[kv_index(&p, l, kv, a, c)]);
                            float y = anchor + fmaf((float)s, w[row], lo[row]);
                            out[kv_index(&p, l, kv, t, c)] = cgo_float_to_half(y);
                        }
                        if (i + 1 < m)
                            for (uint32_t lane = 0; lane < lanes; lane++)
                                if (state[lane] < CGO_STATE_LOW)
                                    state[lane] = (state[lane] << 16) | GROUPW();
                        i++;
                    }
#undef GROUPW
                }
            }
        arow_chunk += (uint64_t)L * 2 * ng;
    }
    return 0;
}

/* Dequantization of a symbol tensor (the unfused path): same formula as above. */
void cgo_dequantize(uint32_t L, uint32_t H, uint32_t d, uint32_t S, uint32_t G, uint32_t Tc,
                    const float *lo, const float *w, const uint8_t *sym, const uint16_t *X_anchor_src,
                    uint32_t t_begin, uint32_t t_end, uint16_t *out)
{
    cgo_shape p = {L, H, d, S, G, Tc, NULL};
    uint32_t C = H * d;
    for (uint32_t l = 0; l < L; l++)
        for (uint32_t kv = 0; kv < 2; kv++)
            for (uint32_t t = t_begin; t < t_end; t++)
                for (uint32_t c = 0; c < C; c++) {
                    size_t i = kv_index(&p, l, kv, t, c);
                    uint32_t a = cgo_anchor_of(t, G, Tc);
                    uint16_t ah = X_anchor_src[kv_index(&p, l, kv, a, c)];
                    if (a == t) {
                        out[i] = ah;
                        continue;
                    }
                    size_t row = ((size_t)l * 2 + kv) * C + c;
                    float y = cgo_half_to_float(ah) + fmaf((float)sym[i], w[row], lo[row]);
                    out[i] = cgo_float_to_half(y);
                }
}

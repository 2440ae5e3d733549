/*
 * Host driver that runs every entry point of the CPU oracle (oracle/cgo.c) on small
 * seeded caches, for a build with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_oracle_sanitizers.py).  It checks only what needs no second
 * implementation: symbol round trips of the coder, a decode that reproduces every
 * anchor and every outlier entry, and in-bounds decodes of damaged payloads.
 * Inputs come from a 64-bit linear congruential generator (Knuth's MMIX constants).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float cgo_half_to_float(uint16_t h);
uint16_t cgo_float_to_half(float f);
int cgo_range(uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, const uint8_t *,
              const uint16_t *, float *, float *, float *, uint32_t, uint32_t);
void cgo_quantize(uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, const uint8_t *,
                  const uint16_t *, const float *, const float *, uint32_t, uint32_t, uint8_t *);
void cgo_histograms(uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, const uint8_t *,
                    const uint8_t *, uint64_t *, uint32_t);
void cgo_freqs(uint32_t, uint32_t, const uint8_t *, const uint64_t *, uint16_t *);
uint32_t cgo_rans_encode(const uint8_t *, uint32_t, const uint16_t *, uint32_t, uint16_t *, int32_t *);
uint32_t cgo_rans_decode(const uint16_t *, uint32_t, uint32_t, const uint16_t *, uint32_t, uint8_t *,
                         uint32_t *);
uint64_t cgo_num_groups(uint32_t, uint32_t, uint32_t, uint32_t);
uint64_t cgo_anchor_rows(uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t);
void cgo_anchors(uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, const uint16_t *,
                 uint32_t, uint32_t, uint16_t *);
void cgo_anchor_grid(uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, const uint16_t *,
                     float *, float *, float *);
void cgo_snap_anchors(uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, const uint16_t *,
                      const float *, const float *, const float *, uint16_t *);
int64_t cgo_encode_payload(uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t,
                           const uint8_t *, const uint8_t *, const uint16_t *, uint32_t, uint32_t,
                           uint64_t *, uint16_t *, uint64_t);
int cgo_decode(uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, const uint8_t *,
               const float *, const float *, const uint16_t *, uint32_t, uint32_t, const uint64_t *,
               const uint16_t *, uint64_t, const uint16_t *, uint16_t *);
uint64_t cgo_outliers(uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, const uint8_t *,
                      const uint16_t *, const uint16_t *, const float *, const float *,
                      const float *, const float *, uint32_t, uint32_t, uint32_t, uint64_t *,
                      uint32_t *, uint16_t *);
int cgo_apply_outliers(uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t,
                       const uint64_t *, const uint32_t *, const uint16_t *, uint64_t, uint16_t *);
void cgo_dequantize(uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, uint32_t, const float *,
                    const float *, const uint8_t *, const uint16_t *, uint32_t, uint32_t, uint16_t *);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(rng_state >> 33);
}

#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            exit(1);                                                    \
        }                                                               \
    } while (0)

static void run_case(uint32_t L, uint32_t H, uint32_t d, uint32_t S, uint32_t G, uint32_t Tc,
                     uint32_t n_sink, uint32_t ppm, int a8)
{
    const uint32_t C = H * d;
    const size_t n = (size_t)L * 2 * S * C, rows = (size_t)L * 2 * C;
    uint8_t *bins = malloc(2 * L);
    for (uint32_t i = 0; i < 2 * L; i++)
        bins[i] = (uint8_t)(2 + rnd() % 31);
    uint16_t *X = malloc(n * 2), *Xs = malloc(n * 2), *out = calloc(n, 2), *out2 = calloc(n, 2);
    /* a random walk per channel with occasional jumps: locality plus tails */
    for (size_t rc = 0; rc < (size_t)L * 2; rc++)
        for (uint32_t c = 0; c < C; c++) {
            float v = 0.0f;
            for (uint32_t t = 0; t < S; t++) {
                v = 0.9f * v + ((float)(rnd() % 2001) - 1000.0f) / 500.0f;
                if (rnd() % 97 == 0) v += ((float)(rnd() % 200) - 100.0f);
                X[(rc * S + t) * C + c] = cgo_float_to_half(v);
            }
        }
    float *lo = malloc(rows * 4), *w = malloc(rows * 4), *r = malloc(rows * 4);
    float *alo = NULL, *aw = NULL, *ar = NULL;
    memcpy(Xs, X, n * 2);
    if (a8) {
        alo = malloc(rows * 4);
        aw = malloc(rows * 4);
        ar = malloc(rows * 4);
        cgo_anchor_grid(L, H, d, S, G, Tc, X, alo, aw, ar);
        cgo_snap_anchors(L, H, d, S, G, Tc, X, alo, aw, ar, Xs);
    }
    CHECK(cgo_range(L, H, d, S, G, Tc, bins, Xs, lo, w, r, n_sink, ppm) == 0);
    uint8_t *sym = calloc(n, 1);
    cgo_quantize(L, H, d, S, G, Tc, bins, Xs, lo, r, 0, S, sym);
    uint64_t *counts = malloc(rows * 32 * 8);
    uint16_t *freqs = malloc(rows * 32 * 2);
    cgo_histograms(L, H, d, S, G, Tc, bins, sym, counts, n_sink);
    cgo_freqs(L, C, bins, counts, freqs);
    const uint32_t nk = (S + Tc - 1) / Tc;
    const uint64_t ng = cgo_num_groups(L, C, 0, nk), arows = cgo_anchor_rows(L, S, G, Tc, 0, nk);
    uint64_t cap = (uint64_t)L * 2 * C * (S + 2 * nk) + 1;
    uint64_t *offsets = malloc((ng + 1) * 8), *ooff = malloc((ng + 1) * 8);
    uint16_t *payload = malloc(cap * 2 + 2);
    int64_t words = cgo_encode_payload(L, H, d, S, G, Tc, bins, sym, freqs, 0, nk, offsets, payload, cap);
    CHECK(words >= 0);
    uint16_t *anchors = malloc((arows ? arows : 1) * C * 2);
    cgo_anchors(L, H, d, S, G, Tc, Xs, 0, nk, anchors);
    CHECK(cgo_decode(L, H, d, S, G, Tc, bins, lo, w, freqs, 0, nk, offsets, payload, (uint64_t)words,
                     anchors, out) == 0);
    /* every anchor comes back bit for bit; the unfused path gives the same tokens */
    for (uint32_t l = 0; l < L; l++)
        for (uint32_t kv = 0; kv < 2; kv++)
            for (uint32_t t = 0; t < S; t++)
                if ((t % Tc) % G == 0)
                    for (uint32_t c = 0; c < C; c++) {
                        size_t i = (((size_t)l * 2 + kv) * S + t) * C + c;
                        CHECK(out[i] == Xs[i]);
                    }
    cgo_dequantize(L, H, d, S, G, Tc, lo, w, sym, Xs, 0, S, out2);
    CHECK(memcmp(out, out2, n * 2) == 0);
    /* outlier table: entries written over the decode are the cache's own values */
    uint64_t no = cgo_outliers(L, H, d, S, G, Tc, bins, X, Xs, lo, r, alo, ar, n_sink, 0, nk, NULL,
                               NULL, NULL);
    uint32_t *keys = malloc((no ? no : 1) * 4);
    uint16_t *vals = malloc((no ? no : 1) * 2);
    CHECK(cgo_outliers(L, H, d, S, G, Tc, bins, X, Xs, lo, r, alo, ar, n_sink, 0, nk, ooff, keys,
                       vals) == no);
    CHECK(cgo_apply_outliers(L, H, d, S, Tc, 0, nk, ooff, keys, vals, no, out) == 0);
    {
        const uint32_t NB = (C + 63) / 64;
        uint64_t g = 0;
        for (uint32_t k = 0; k < nk; k++)
            for (uint32_t rc = 0; rc < 2 * L; rc++)
                for (uint32_t b = 0; b < NB; b++, g++)
                    for (uint64_t e = ooff[g]; e < ooff[g + 1]; e++) {
                        size_t i = ((size_t)rc * S + k * Tc + (keys[e] >> 6)) * C + b * 64 + (keys[e] & 63u);
                        CHECK(i < n && out[i] == vals[e] && X[i] == vals[e]);
                    }
        CHECK(g == ng && ooff[ng] == no);
    }
    /* damaged payload and offsets still decode inside the buffers */
    for (int k = 0; k < 40 && words > 0; k++)
        payload[rnd() % (uint64_t)words] ^= (uint16_t)rnd();
    CHECK(cgo_decode(L, H, d, S, G, Tc, bins, lo, w, freqs, 0, nk, offsets, payload, (uint64_t)words,
                     anchors, out2) == 0);
    if (ng > 1) {
        offsets[1] = (uint64_t)words + 5;  /* past the end: rejected, not read */
        CHECK(cgo_decode(L, H, d, S, G, Tc, bins, lo, w, freqs, 0, nk, offsets, payload,
                         (uint64_t)words, anchors, out2) == -5);
    }
    if (no) {
        keys[0] = 0xFFFFFFFFu;  /* a key outside its group: rejected */
        CHECK(cgo_apply_outliers(L, H, d, S, Tc, 0, nk, ooff, keys, vals, no, out2) == -5);
    }
    free(bins); free(X); free(Xs); free(out); free(out2); free(lo); free(w); free(r);
    free(alo); free(aw); free(ar); free(sym); free(counts); free(freqs); free(offsets); free(ooff);
    free(payload); free(anchors); free(keys); free(vals);
}

int main(void)
{
    /* coder: random tables and streams, every symbol back, final state 2^16 */
    for (int it = 0; it < 300; it++) {
        uint32_t N = 2 + rnd() % 31, m = rnd() % 400;
        uint16_t f[32];
        uint32_t left = 256 - N;
        for (uint32_t s = 0; s < N; s++) f[s] = 1;
        while (left) { f[rnd() % N]++; left--; }
        uint8_t *x = malloc(m + 1), *y = malloc(m + 1);
        uint16_t *words = malloc((m + 2) * 2);
        int32_t *steps = malloc((m + 2) * 4);
        for (uint32_t i = 0; i < m; i++) x[i] = (uint8_t)(rnd() % N);
        uint32_t nw = cgo_rans_encode(x, m, f, N, words, steps), fin = 0;
        CHECK(cgo_rans_decode(words, nw, m, f, N, y, &fin) <= nw + 2);
        CHECK(m == 0 || (memcmp(x, y, m) == 0 && fin == 0x10000u));
        free(x); free(y); free(words); free(steps);
    }
    run_case(2, 1, 70, 97, 10, 40, 0, 0, 0);
    run_case(2, 1, 70, 97, 7, 30, 5, 20000, 0);
    run_case(1, 2, 36, 61, 5, 61, 3, 100000, 1);
    run_case(1, 1, 8, 5, 10, 3, 9, 250000, 1);
    run_case(1, 1, 64, 40, 1, 16, 0, 5000, 0);
    printf("oracle sanitizer run ok\n");
    return 0;
}

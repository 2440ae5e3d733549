// cg_internal.h -- declarations shared by the kernels and the host side of libcg.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace cgk {

constexpr uint32_t kProbBits = 8;                  // frequencies are in units of 1/256
constexpr uint32_t kProbTotal = 1u << kProbBits;
constexpr uint32_t kMaxBins = 32;
constexpr uint32_t kLanes = 64;                    // channels per group = wavefront width
constexpr uint32_t kStateLow = 1u << 16;           // rANS state in [2^16, 2^32), 16-bit words
constexpr uint32_t kPayloadPadBytes = 1024;        // zero bytes after the payload of a container
// Decode table of one (row, 64-channel block), in 32-bit words: two planes [32 symbols]
// [64 lanes], {f | cdf << 24} then the dequantized delta lo + s * w (fp32 bits), then
// the slot table [256 slots][64 lanes] of bytes: the symbol whose interval [cdf, cdf + f)
// holds the slot.
constexpr uint32_t kTabPlane = kMaxBins * kLanes;
constexpr uint32_t kTabLut = 2 * kTabPlane;
constexpr uint32_t kTabBlock = kTabLut + kProbTotal * kLanes / 4;
// dword 3 of a raw (untyped) buffer resource on gfx9-family GPUs: 32-bit data format
constexpr int kBufferFlags = 0x00020000;

// Geometry of one call.  kb, ke: chunk range being encoded / decoded.
struct Geom {
    uint32_t L, C, S, G, Tc;
    uint32_t NB;   // blocks of 64 channels = ceil(C / 64)
    uint32_t ngF;  // groups in a full chunk = ceil(Tc / G)
    uint32_t kb, ke;
    uint32_t n_sink = 0;  // first tokens of the sequence kept in fp16 (left out of the tables)
    // 8-bit anchors: the anchor grid of every (layer, K/V, channel) row, [L][2][C]; null
    // alo means fp16 anchors
    const float *alo = nullptr, *aw = nullptr, *ar = nullptr;
};

// Paged output (vLLM-style block table): pages fp16 [L][2][num_pages][1 << lp][C]; token t
// of a (layer, K/V) row goes to page bt[t >> lp], row t & ((1 << lp) - 1).
struct Paged {
    uint16_t *pages;
    const int32_t *bt;
    uint32_t lp, num_pages, n_blocks;
};

// Byte offsets of the container sections (and the counts the sections hold).
struct ContainerView {
    uint64_t offsets_off, anchors_off, anchors_bytes, payload_off, payload_words;
    uint64_t sinks_off;            // fp16 [L][2][n_sink][C] from token kb * Tc
    uint32_t n_sink;
    uint64_t out_off, keys_off, vals_off, n_out;  // outlier sections (n_out = 0: none)
    bool outliers;
};

constexpr uint32_t kFineBins = 256;               // fine grid of the outlier clip

// The contiguous and paged value decodes (launch_k3 without symbols, launch_k3_paged)
// write a container's outlier entries themselves, each wavefront those of its chunks;
// for every other decode launch_apply_outliers writes them afterwards.
inline bool outliers_with_rows(const ContainerView &cv) { return cv.outliers && cv.n_out > 0; }

// Chunks decoded by one launch from containers of their own (the streamed decode).  The
// chunks form sets, each of up to 8 chunks that share one set of tables; set j is chunks
// [set_first[j], set_first[j] + set_n[j]) with tables tab[set_tab[j]].  Chunk i is chunk
// k of the cache, read from the container at c (whose first chunk is kb) with the
// payload / offsets / anchors sections at the given byte offsets.
constexpr uint32_t kMaxBatch = 32;        // chunks (and sets) one launch takes
constexpr uint32_t kMaxBatchTables = 4;   // sets of tables one launch takes
constexpr uint32_t kBatchSetChunks = 8;   // chunks of a set: 4 wavefronts x 2 streams
struct BatchTables {
    const uint8_t *bins;
    const uint32_t *dtab;
    const float *lo, *w;
    const float *alo, *aw;   // 8-bit anchor grid, null for fp16 anchors
};
struct BatchChunk {
    const uint8_t *c;
    uint64_t offsets_off, anchors_off, anchors_bytes, payload_off, payload_words;
    uint32_t k, kb;
};
struct ChunkSrcs {
    uint32_t n_sets;
    uint8_t set_first[kMaxBatch], set_n[kMaxBatch], set_tab[kMaxBatch];
    BatchTables tab[kMaxBatchTables];
    BatchChunk ch[kMaxBatch];
};

hipError_t launch_k0(const uint16_t *X, const Geom &g, uint32_t tpt, uint32_t *ord_lo,
                     uint32_t *ord_hi, uint32_t *flag, hipStream_t st);
// lo and hi (zero bounds as +0) from the ordered min / max
hipError_t launch_k0_finalize(const Geom &g, const uint32_t *ord_lo, const uint32_t *ord_hi,
                              float *lo, float *hi, hipStream_t st);
// outlier table: counts of the deltas in the 256 fine intervals over [lo, hi] of every
// channel row, then the central range (lo, hi narrowed in place)
// (partial: fine_parts(g) x [rows][C][256] uint16 counts, every entry written)
uint32_t fine_parts(const Geom &g);
hipError_t launch_fine_hist(const uint16_t *X, const Geom &g, const float *lo, const float *hi,
                            uint16_t *partial, hipStream_t st);
hipError_t launch_clip(const Geom &g, const uint16_t *partial, uint32_t ppm, float *lo,
                       float *hi, hipStream_t st);
// w = (hi - lo) / (N - 1), r = 1 / w (0 when w = 0)
hipError_t launch_width(const Geom &g, const uint8_t *bins, const float *lo, const float *hi,
                        float *w, float *r, hipStream_t st);
hipError_t launch_k1(const uint16_t *X, const Geom &g, const uint8_t *bins, uint32_t max_bins,
                     const float *lo, const float *r, uint32_t *counts, hipStream_t st);
hipError_t launch_k1_freqs(const Geom &g, const uint8_t *bins, const uint32_t *counts,
                           uint16_t *freqs, hipStream_t st);
// the coder tables of every (row, 64-channel block) from the frequencies and grids
hipError_t launch_dtab(const Geom &g, const uint8_t *bins, const uint16_t *freqs,
                       const float *lo, const float *w, uint32_t *dtab, hipStream_t st);
// clamped (if not null) accumulates the number of elements off their grid (tokens from
// n_sink on; with 8-bit anchors, anchors off the anchor grid too)
hipError_t launch_k2(const uint16_t *X, const Geom &g, const uint8_t *bins, const float *lo,
                     const float *r, uint32_t t_lo, uint32_t t_hi, uint32_t tpt, uint8_t *sym,
                     uint32_t sym_t0, uint32_t sym_T, uint16_t *anchors,
                     unsigned long long *clamped, hipStream_t st);
// Outlier entries of the groups of chunks [g.kb, g.ke): with counts set, the number of
// entries of every group; otherwise the entries themselves, group g from offs[g].
hipError_t launch_outliers(const uint16_t *X, const Geom &g, const uint8_t *bins, const float *lo,
                           const float *r, uint64_t *counts, const uint64_t *offs, uint32_t *keys,
                           uint16_t *vals, hipStream_t st);
// Writes a container's outlier entries into the output (contiguous, or pages of pg).
hipError_t launch_apply_outliers(const Geom &g, const uint8_t *container, const ContainerView &cv,
                                 uint16_t *out, const Paged &pg, hipStream_t st);
// Words of one lane's stream for m symbols: at most 2 state words and floor(0.50036 m)
// shifted words (each symbol multiplies the state by at most 256 (1 + 2^-8), each word
// divides it by 2^16, and it starts and ends at or above 2^16).
__host__ __device__ constexpr uint32_t lane_words_max(uint32_t m) { return (m >> 1) + (m >> 11) + 4; }
// Words of the scratch region of one group (worst case over the chunks of g).
uint64_t code_region_words(const Geom &g);
// The fused encoder: for every group of chunks [g.kb, g.ke), its words placed at the end of
// its region, its anchors into `anchors` (the container's anchors section layout), its
// word count and its number of elements off their grid.
hipError_t launch_k5_code(const uint16_t *X, const Geom &g, const uint8_t *bins,
                          const uint32_t *dtab, const float *lo, const float *r,
                          uint16_t *regions, uint8_t *anchors, uint64_t *group_words,
                          uint64_t *group_off_grid, hipStream_t st);
hipError_t launch_scan(const uint64_t *in, uint64_t *out, uint64_t n, hipStream_t st);
// Byte ranges to clear, [r[i][0], r[i][1]) for i < n (each range small: one block).
struct ZeroRanges {
    uint64_t r[8][2];
    uint32_t n;
};
hipError_t launch_zero_ranges(uint8_t *base, const ZeroRanges &zr, hipStream_t st);
hipError_t launch_k5_compact(const uint16_t *regions, uint64_t region_words,
                             const uint64_t *group_words, const uint64_t *group_off,
                             uint64_t n_groups, uint16_t *payload, hipStream_t st);
hipError_t launch_k3(const Geom &g, const uint8_t *bins, const uint32_t *dtab, const float *lo,
                     const float *w, const uint8_t *container, const ContainerView &cv,
                     uint16_t *out, uint8_t *sym_out, hipStream_t st);
// Decodes the chunk sets of srcs (g gives the cache shape; its tables fields are unused).
// Every set's tables have 8-bit anchors, or none has.
hipError_t launch_k3_multi(const Geom &g, const ChunkSrcs &srcs, uint16_t *out, hipStream_t st);
hipError_t launch_k3_paged(const Geom &g, const uint8_t *bins, const uint32_t *dtab,
                           const float *lo, const float *w, const uint8_t *container,
                           const ContainerView &cv, const Paged &pg, hipStream_t st);
// The 8-bit anchor grid of every (layer, K/V, channel) row over its anchor tokens.
hipError_t launch_anchor_grid(const uint16_t *X, const Geom &g, float *alo, float *aw, float *ar,
                              hipStream_t st);
// Writes the fp16 sink rows sinks [L][2][n_tok][C] (tokens t0 .. t0 + n_tok) into the
// output: the contiguous [L][2][S][C] out, or the pages of pg when pg.pages is set.

hipError_t launch_sinks(const Geom &g, const uint16_t *sinks, uint32_t n_tok, uint32_t t0,
                        uint16_t *out, const Paged &pg, hipStream_t st);
hipError_t launch_k4(const Geom &g, const float *lo, const float *w, const uint8_t *sym,
                     const uint8_t *container, const ContainerView &cv, uint32_t t_lo,
                     uint32_t t_hi, uint32_t tpt, uint16_t *out, hipStream_t st);

}  // namespace cgk

/*
 * cg.h -- C ABI of libcg, a CacheGen-style KV-cache codec for AMD MI355X (gfx950).
 *
 * The codec compresses an fp16 KV cache [L][2][S][C] (C = H_kv * d channels; index 1
 * is K = 0 / V = 1) into independent bitstreams and decodes it back:
 *   - tokens are cut into chunks of `chunk` tokens and each chunk into groups of
 *     `group` tokens whose first token (the anchor) is kept in fp16 ("Guide to
 *     CacheGen", Solution pillar 2 and Implementation Step 2);
 *   - every other token is coded as its delta from the anchor, quantized to the
 *     layer's number of levels, finer for early layers (same page, pillar 1; the
 *     gptget.net summary of CacheGen, Methodology);
 *   - the symbols are entropy-coded (rANS, an arithmetic-type coder) with empirical
 *     frequency tables per (layer, K/V, channel), one stream per (layer, K/V, channel,
 *     chunk) (pillar 3; the summary's Deep Analysis, Methodology);
 *   - decoding inverts the coder, dequantizes in float32 and adds the anchor back
 *     (Implementation Step 1 dequantize_tensor, Step 2 decode_sequence).
 * The problem statement these calls follow is the pages' KV-size formula
 * 2 * L * H_kv * d * S * sizeof(dtype) ("Guide to CacheGen", Problem) and the
 * encode-into-compact-bitstreams / stream-chunks / GPU-decode pipeline (summary,
 * Methodology).
 *
 * Conventions for every call:
 *   - pointers named *_dev are device pointers on the current HIP device; the caller
 *     owns them and the streams.  `hip_stream` is a hipStream_t (NULL = null stream).
 *   - handles (cg_tables, cg_blob) are owned by the library, immutable after creation
 *     and released with cg_free().  Concurrent cg_decode calls with the same handles on
 *     different streams are allowed.
 *   - return value: CG_OK or a negative CG_E_* code; cg_last_error() gives a message
 *     (thread-local).  No call throws or aborts.
 *   - limits: 1 <= L, H_kv, d, S; C = H_kv * d a multiple of 8; 1 <= group;
 *     1 <= chunk <= 16384; 2 <= bins[l] <= 32 (and bins_v[l]); L * 2 * S * C < 2^40; S * C < 2^32;
 *     chunk * C * 2 < 2^32 (32-bit offsets within one row of symbols and one chunk).
 */
#ifndef CG_H
#define CG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CG_OK 0
#define CG_E_INVAL (-1)     /* bad argument: null pointer, out-of-range size or chunk range */
#define CG_E_NOMEM (-2)     /* device or host allocation failed */
#define CG_E_HIP (-3)       /* HIP runtime error; cg_last_error() holds its text */
#define CG_E_NONFINITE (-4) /* the KV input holds Inf or NaN */
#define CG_E_CORRUPT (-5)   /* container and tables do not describe the same cache */

#define CG_MAX_BINS 32
#define CG_MAX_CHUNK 16384
#define CG_LANES 64         /* channels per interleaved group of streams */
#define CG_CONTAINER_MAGIC 0x31474B43u /* "CKG1" */

/* Shape and coding parameters.  `bins` points to L bin counts (host memory, copied);
 * `bins_v`, if not NULL, to L bin counts for the V rows, `bins` then giving those of the
 * K rows (keys kept finer than values: "Guide to CacheGen", Solution pillar 1). */
typedef struct cg_params {
    uint32_t L, H_kv, d, S;
    uint32_t group;          /* anchor interval G */
    uint32_t chunk;          /* tokens per chunk (one stream per (layer, K/V, channel, chunk)) */
    const uint8_t *bins;     /* [L], bins[l] = number of quantization levels of layer l */
    const uint8_t *bins_v;   /* [L] or NULL: levels of the V rows of layer l (NULL: bins[l]) */
    uint32_t n_sink;         /* first n_sink tokens of the sequence (attention sinks, "Guide to
                                CacheGen", Best Practices) kept in fp16: left out of ranges
                                and histograms, stored by cg_encode in every container that
                                holds them and written back exactly by every decode; 0 = none;
                                values above S act as S */
    uint32_t anchor_bits;    /* 0 or 16: anchors stored as fp16.  8: each anchor stored as a
                                code on a 256-level grid of its (layer, K/V, channel) row
                                ("Guide to CacheGen", Solution pillar 2: anchors quantized
                                with high precision), min to max of the row's anchor tokens;
                                the decoded anchor is the fp16 grid value and the deltas are
                                taken against it */
    uint32_t outlier_ppm;    /* 0: no outlier table.  1 .. 250000: sparse outlier table
                                ("Guide to CacheGen", Solution pillar 3: outliers kept in a
                                compact sparse table so that they do not distort the regular
                                distribution).  Each channel row's grid spans a central range
                                that leaves at most floor(n * outlier_ppm / 10^6) of its n
                                deltas out at each end (chosen on 256 equal intervals of the
                                full range), and every element off its grid is stored
                                exactly in fp16 in the container */
} cg_params;

typedef struct cg_tables cg_tables; /* per-channel ranges and frequency tables (device) */
typedef struct cg_blob cg_blob;     /* one encoded container (device) */

/*
 * Container (version 3): one buffer, little endian, every section 256-byte aligned
 * relative to the first byte, the bytes between sections zero:
 *   header     cg_container_header (160 bytes)
 *   offsets    uint64[n_groups + 1]: first payload word of every group, then the total.
 *              Groups are (chunk, layer, K/V, block) in row-major order over chunks
 *              [chunk_begin, chunk_end); block b holds channels 64b .. 64b+63.
 *   anchors    fp16 (uint8 grid codes with 8-bit anchors), for each chunk:
 *              [L][2][ceil(len_k / group)][C]
 *   sinks      fp16 [L][2][n_sink][C]: tokens chunk_begin * chunk .. + n_sink, the
 *              attention sinks among the container's tokens, copied from the encoded cache
 *   outliers   (outlier_ppm > 0 only) uint64[n_groups + 1] first entry of every group,
 *              then the total; then uint32 keys [n_outliers] (token within the chunk << 6
 *              | lane), then uint16 fp16 values [n_outliers] (each its own section).
 *              A group's entries are in ascending key order.
 *   payload    uint16 words, then 1 KiB of zeros.  A group's words are the words of its
 *              (up to) 64 rANS streams in the order 64 decoders running in lockstep read
 *              them: the two state words of every lane in lane order, then after each
 *              symbol step the next word of every lane whose state fell below 2^16, in
 *              lane order.
 * Every section offset follows from the fields before it: offsets at 256, then each
 * section at the next multiple of 256 after the previous one's end; the outlier sections
 * are empty (all three offsets equal) when outlier_ppm is 0.  total_bytes =
 * payload_offset + 2 * payload_words + 1024.
 * Tables are stored separately (cg_tables_serialize); the compression ratio counts both.
 */
typedef struct cg_container_header {
    uint32_t magic, version;          /* CG_CONTAINER_MAGIC, CG_CONTAINER_VERSION */
    uint32_t L, H_kv, d, S, group, chunk;
    uint32_t chunk_begin, chunk_end;
    uint32_t n_blocks;                /* ceil(H_kv * d / 64) */
    uint32_t anchor_bits;             /* 16: fp16 anchors, 8: grid codes */
    uint32_t n_sink;                  /* sink tokens stored in this container */
    uint32_t outlier_ppm;             /* the tables' setting; 0: no outlier sections */
    uint64_t n_groups;
    uint64_t offsets_offset;
    uint64_t anchors_offset, anchors_bytes;
    uint64_t sinks_offset;
    uint64_t outliers_offset, outlier_keys_offset, outlier_values_offset, n_outliers;
    uint64_t clamped;                 /* elements off their grid coded clamped (no outlier
                                         table): 0 for the cache the tables were built from */
    uint64_t payload_offset, payload_words;
    uint64_t total_bytes;
} cg_container_header;

#define CG_CONTAINER_VERSION 3u
#define CG_TABLES_MAGIC 0x31544743u  /* "CGT1" */
#define CG_TABLES_VERSION 1u

/*
 * Stored tables (cg_tables_serialize / cg_tables_import), little endian, no padding
 * except after bins:
 *   header   cg_tables_header (56 bytes)
 *   bins     uint8 [L][2] (level count of every (layer, K/V) row), zero-padded to 4 bytes
 *   lo, w    float [L][2][C] each: the grid of every channel row
 *   alo, aw  float [L][2][C] each, with 8-bit anchors only: the anchor grid
 *   freqs    uint16: for each (layer, K/V) row and channel, its N frequencies (sum 256)
 * The reciprocals r = 1/w (and 1/aw) are recomputed on import, 0 where the width is 0.
 */
typedef struct cg_tables_header {
    uint32_t magic, version;          /* CG_TABLES_MAGIC, CG_TABLES_VERSION */
    uint32_t L, H_kv, d, S, group, chunk;
    uint32_t n_sink, anchor_bits, outlier_ppm, reserved;
    uint64_t total_bytes;
} cg_tables_header;

typedef struct cg_blob_info {
    const void *data;             /* device pointer to the container */
    cg_container_header header;   /* host copy of its header */
} cg_blob_info;

typedef struct cg_tables_info {
    uint32_t L, H_kv, d, S, group, chunk;
    uint64_t stored_bytes;        /* size of the stored tables (cg_tables_serialize) */
} cg_tables_info;

/*
 * Builds the per-(layer, K/V, channel) tables from the whole cache ("Guide to CacheGen",
 * Solution pillar 3: tables of empirical symbol frequencies from calibration profiling,
 * kept per layer and channel as in the gptget.net summary's Deep Analysis): the range of
 * the anchor deltas (narrowed to a central range with the outlier table), the bin width
 * from the layer's level count (pillar 1), and a frequency table of the quantized deltas
 * over all chunks (T = 256, every symbol >= 1).
 *   params: shape and coding parameters, read during the call only.
 *   kv_dev: fp16 [L][2][S][C] on the current device, read only.
 *   *out:   receives a new handle on success, untouched on error.
 * Synchronises `hip_stream` once (to report CG_E_NONFINITE).
 * Errors: CG_E_INVAL (null pointer, a zero dimension, a limit exceeded, bins outside
 * [2, 32], anchor_bits not 0 / 8 / 16, outlier_ppm > 250000), CG_E_NOMEM, CG_E_HIP,
 * CG_E_NONFINITE.
 */
int cg_build_cdf(const cg_params *params, const void *kv_dev, void *hip_stream,
                 cg_tables **out);

/*
 * Encodes chunks [chunk_begin, chunk_end) of kv_dev into a new container: the anchors,
 * the sink rows among those tokens, the entropy-coded delta symbols ("Guide to CacheGen",
 * Solution pillars 2-3 and Implementation Step 2; the summary's Methodology: the cache is
 * encoded into compact bitstreams, chunk by chunk) and, with the outlier table, the
 * entries of every element off its grid.
 *   kv_dev: fp16 [L][2][S][C], read only: the cache the tables were built from, or
 *           another cache of the same shape coded with these tables (calibration
 *           tables).  Elements of another cache that the tables' grids do not hold
 *           within half a step are stored exactly with the outlier table; without it
 *           they are coded clamped and counted in the header's `clamped`.
 * Synchronises `hip_stream` (the payload size is data dependent); the container is
 * complete when the call returns.
 * Errors: CG_E_INVAL (null pointer, bad chunk range), CG_E_NOMEM, CG_E_HIP.
 */
int cg_encode(const cg_tables *tables, const void *kv_dev, uint32_t chunk_begin,
              uint32_t chunk_end, void *hip_stream, cg_blob **out);

/*
 * Decodes a container into kv_out_dev (fp16 [L][2][S][C]) ("Guide to CacheGen",
 * Implementation Step 1 dequantize_tensor and Step 2 decode_sequence; the summary's
 * Methodology: GPU decoding of the received bitstreams).  Writes exactly the tokens of
 * chunks [chunk_begin, chunk_end) and leaves every other token untouched: the decoded
 * rows, then, on the same stream, the container's sink rows and outlier entries.
 *   container_dev: NULL to decode the blob's own copy, or a device buffer holding the
 *                  same container bytes (e.g. staged from pinned host memory).  Its
 *                  payload, offsets and outlier entries are not trusted: damaged bytes
 *                  decode to wrong values but every read and write stays in bounds.
 * Fully asynchronous on hip_stream.  Errors: CG_E_INVAL, CG_E_CORRUPT (blob and
 * tables disagree on the shape or settings), CG_E_HIP.
 */
int cg_decode(const cg_tables *tables, const cg_blob *blob, const void *container_dev,
              void *kv_out_dev, void *hip_stream);

/*
 * Decodes into a paged KV cache (vLLM-style block table) instead of a contiguous one:
 * the decompressor writes straight into the serving engine's KV blocks ("Guide to
 * CacheGen", Best Practices: inject into paged buffers).
 *   pages_dev:       fp16 [L][2][num_pages][page_tokens][H_kv * d], device, caller-owned;
 *                    one pool of num_pages pages per (layer, K/V).
 *   block_table_dev: int32 [ceil(S / page_tokens)], device: token t of every (layer, K/V)
 *                    goes to page block_table[t / page_tokens], row t % page_tokens.
 *   page_tokens:     a power of two; (num_pages + 1) * page_tokens * H_kv * d * 2 <= 2^32.
 * Writes the tokens of the blob's chunks (sink rows and outlier entries as in
 * cg_decode); a block whose page id is negative or >= num_pages is skipped (none of its
 * rows is written), other pages are untouched.
 * container_dev as in cg_decode.  Fully asynchronous on hip_stream.  Errors:
 * CG_E_INVAL, CG_E_CORRUPT, CG_E_HIP.
 */
int cg_decode_paged(const cg_tables *tables, const cg_blob *blob, const void *container_dev,
                    void *pages_dev, const int32_t *block_table_dev, uint32_t page_tokens,
                    uint32_t num_pages, void *hip_stream);

/* Releases a cg_tables* or cg_blob* and its device memory ("Guide to CacheGen",
 * Implementation: the compressor / decompressor objects own their buffers).  NULL is a
 * no-op; any other pointer must be a live handle of this library. */
void cg_free(void *handle);

/*
 * cg_encode for callers that cannot allocate memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same kernels and the same container
 * bytes, written into a caller-owned buffer, with the scratch taken from a fixed 64 MiB
 * array in the library's device memory (one per device, held until the process ends).
 * No hipMalloc, hipFree or other allocating call is made.
 *   container_dev: device buffer of `capacity` bytes, 256-byte aligned.
 *   header_out:    receives the container's header (host), also when the capacity is too
 *                  small (then its total_bytes is the size needed and nothing is written).
 * Encodes whose scratch (about (2 + m / 2 + m / 2048 + 2) * 128 bytes per 64-channel
 * group of a chunk with m coded tokens, plus the anchors section) exceeds 64 MiB are
 * refused with CG_E_INVAL before any device work.  All calls on one device share the
 * array: the library serialises them (a call holds it from its first launch to its last
 * wait); the array keeps the last call's contents and needs no clearing.  Synchronises
 * hip_stream twice.  Errors: CG_E_INVAL, CG_E_HIP.
 */
int cg_encode_noalloc(const cg_tables *tables, const void *kv_dev, uint32_t chunk_begin,
                      uint32_t chunk_end, void *container_dev, uint64_t capacity,
                      void *hip_stream, cg_container_header *header_out);

/* ----------------------------------------------------------------------------------
 * Stored form.  Tables and containers are written to host memory, kept or sent
 * elsewhere, and imported by a receiver that decodes them ("Guide to CacheGen", Problem:
 * caches offloaded to RAM, SSD or remote storage; the gptget.net summary, Methodology:
 * encoded bitstreams streamed over the network to the serving GPU).
 * ---------------------------------------------------------------------------------- */

/* Writes the stored tables (layout above) to host_dst if capacity allows; *size_out
 * (if not NULL) receives their size either way.  Synchronous.
 * Errors: CG_E_INVAL (null tables, host_dst NULL or capacity too small with a non-NULL
 * host_dst), CG_E_HIP. */
int cg_tables_serialize(const cg_tables *tables, void *host_dst, uint64_t capacity,
                        uint64_t *size_out);

/* Checks stored tables in host memory without touching a device: header, sizes, level
 * counts, finite grids with widths >= 0, every frequency table >= 1 per symbol and
 * summing to 256.  *header_out (if not NULL) receives the header.  Returns CG_OK or
 * CG_E_CORRUPT (CG_E_INVAL for null bytes). */
int cg_tables_check(const void *host_bytes, uint64_t nbytes, cg_tables_header *header_out);

/* Checks, then builds a tables handle on the current device from stored tables.
 * Synchronous.  Errors: CG_E_INVAL, CG_E_CORRUPT, CG_E_NOMEM, CG_E_HIP. */
int cg_tables_import(const void *host_bytes, uint64_t nbytes, cg_tables **out);

/* Checks a container in host memory without touching a device: magic, version, shape
 * limits, every section offset against the layout, group offsets starting at 0,
 * non-decreasing and ending at payload_words, outlier offsets likewise and every key
 * inside its group's chunk and block.  *header_out (if not NULL) receives the header.
 * Returns CG_OK or CG_E_CORRUPT (CG_E_INVAL for null bytes). */
int cg_container_check(const void *host_bytes, uint64_t nbytes, cg_container_header *header_out);

/* Checks a container against itself (cg_container_check) and against the tables (shape,
 * anchor width, outlier setting, sink count), then copies it to the tables' device as a
 * new blob.  Synchronous on hip_stream.  Errors: CG_E_INVAL, CG_E_CORRUPT, CG_E_NOMEM,
 * CG_E_HIP. */
int cg_blob_import(const cg_tables *tables, const void *host_bytes, uint64_t nbytes,
                   void *hip_stream, cg_blob **out);

/* ----------------------------------------------------------------------------------
 * Streamed decode.  Chunk containers arrive from host memory while earlier chunks
 * decode, and each chunk may come at its own compression level ("Guide to CacheGen",
 * section 4, Overlapped Streaming Decoder Pipeline: chunk i decodes while chunk i+1 is
 * in transit; gptget summary of arXiv 2310.07240, Methodology: the compression level
 * follows the available bandwidth and GPU decoding keeps pace with transmission).
 * ---------------------------------------------------------------------------------- */

/* One container to stream: the tables of the level it was coded at, its handle (for
 * the layout only; the handle's device copy is not read) and the same container bytes
 * (cg_blob_read of the whole container) in host memory.  Pinned host memory (hipHostMalloc)
 * lets the copy overlap decoding; pageable memory works but serialises. */
typedef struct cg_stream_item {
    const cg_tables *tables;
    const cg_blob *blob;
    const void *host_container;
} cg_stream_item;

/* Timings of a streamed decode from HIP events, milliseconds. */
typedef struct cg_stream_stats {
    float total_ms;        /* first copy started -> last decode finished */
    float copy_ms;         /* sum over items of the host-to-device copy */
    float decode_ms;       /* sum over windows of the decode (see cg_stream_decode) */
    uint64_t copied_bytes; /* sum over items of the container size */
} cg_stream_stats;

/*
 * Decodes items[0 .. n_items) in order into kv_out_dev (fp16 [L][2][S][C]).  Item i is
 * copied into staging slot i % n_slots (slot j starts at staging_dev + j * slot_bytes)
 * on copy_stream and decoded from there on decode_stream (sink tokens and outliers as in
 * cg_decode); a slot is refilled only after the decode that read it has finished.  The
 * items are decoded in windows of min(32, max(1, n_slots / 2)) consecutive items: once a
 * window's copies have landed, one launch decodes every chunk of the window (more than
 * one if the window holds over 32 chunks or 4 sets of tables, or fp16 and 8-bit anchors),
 * while the next window is copied into other slots.
 *   staging_dev:   caller-owned device memory, n_slots * slot_bytes bytes; the address
 *                  and slot_bytes are multiples of 256.
 *   copy_stream, decode_stream: two different streams of the tables' device.
 *   stats:         NULL to return once everything is queued (kv_out_dev, the staging
 *                  memory and the host containers stay in use until decode_stream and
 *                  copy_stream have drained); otherwise waits for both and fills *stats.
 * Every item's tables must be on one device and describe the same cache shape, and its
 * container must fit a slot; all of this is checked before anything is queued.
 * Errors: CG_E_INVAL, CG_E_CORRUPT, CG_E_NOMEM, CG_E_HIP (after waiting for both
 * streams if work had been queued).
 */
int cg_stream_decode(const cg_stream_item *items, uint32_t n_items, void *staging_dev,
                     uint64_t slot_bytes, uint32_t n_slots, void *kv_out_dev,
                     void *copy_stream, void *decode_stream, cg_stream_stats *stats);

/* ----------------------------------------------------------------------------------
 * Inspection and the unfused path.  Same conventions as above.
 * ---------------------------------------------------------------------------------- */

/* Thread-local text of the last error (empty string if none). */
const char *cg_last_error(void);

/* Host copies of the tables.  lo, w, r: float [L][2][C]; freqs: uint16 [L][2][C][32]
 * (entries >= the bin count of the (layer, K/V) row are 0).  Any pointer may be NULL.
 * Synchronous. */
int cg_tables_export(const cg_tables *tables, float *lo, float *w, float *r, uint16_t *freqs);
int cg_tables_get_info(const cg_tables *tables, cg_tables_info *info);
int cg_blob_get_info(const cg_blob *blob, cg_blob_info *info);

/* Copies bytes [offset, offset + nbytes) of the container to host memory (synchronous).
 * CG_E_INVAL if the range leaves the container. */
int cg_blob_read(const cg_blob *blob, uint64_t offset, uint64_t nbytes, void *host_dst);

/* The quantizer alone: uint8 symbols [L][2][S][C] for tokens of chunks
 * [chunk_begin, chunk_end) (anchor slots are written 0, other tokens untouched).
 * Asynchronous. */
int cg_quantize(const cg_tables *tables, const void *kv_dev, uint32_t chunk_begin,
                uint32_t chunk_end, void *sym_dev, void *hip_stream);

/* The entropy decoder alone: writes uint8 symbols [L][2][S][C] for the container's
 * tokens (anchor slots written 0).  Asynchronous. */
int cg_decode_symbols(const cg_tables *tables, const cg_blob *blob, const void *container_dev,
                      void *sym_dev, void *hip_stream);

/* Dequantize + anchor-add alone: symbols [L][2][S][C] and the container's anchors to
 * fp16 [L][2][S][C] for the container's tokens, then its sink rows and outlier entries
 * as in cg_decode.  Asynchronous. */
int cg_dequantize(const cg_tables *tables, const cg_blob *blob, const void *container_dev,
                  const void *sym_dev, void *kv_out_dev, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* CG_H */

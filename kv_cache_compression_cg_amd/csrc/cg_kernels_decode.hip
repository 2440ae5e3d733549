// cg_kernels_decode.hip -- gfx950 kernels of cg_decode: the rANS decoder fused with
// dequantize + anchor-add (K3), and the unfused dequantize + anchor-add (K4).

#include "cg_device.h"

namespace cgk {

// ------------------------------------------------------------------------------ K3 (+K4)
// rANS decoder fused with dequantize + anchor-add.  Block = 4 wavefronts, each decoding
// two chunks of the same (row, block) in lockstep, all sharing the block's decode table
// in LDS (f and cdf of up to 32 symbols per lane as bytes, and the 256-slot table of
// symbol bytes laid out one LDS bank per lane).  Everything
// that is the same for the 64 lanes (chunk, token, group, stream cursor, row addresses)
// is kept in scalar registers; only the coder state and the table address are per lane.

// Per-wavefront LDS ring of payload words, refilled with
// 4-byte-per-lane loads.  Ring slots [0, 64) are mirrored at [R, R + 64), so the up-to-
// 64 words one step reads are contiguous in LDS.
// Cache policy of the decoder's own memory traffic: nt (non-temporal, streaming) for the
// row stores and for the container reads (payload words, anchor rows), each touched once.
// On the 70B-shaped cache this took the decode from 3.56 to 3.33 ms (stores 3.50, payload
// words 3.36, anchors 3.33); sc0 did not help.
constexpr int kNT = 2;
constexpr uint32_t kRingWords = 256;
constexpr uint32_t kRingAlloc = kRingWords + 64;
constexpr uint32_t kFetchWords = 128;
constexpr uint32_t kWavesPerBlock = 4;
constexpr uint32_t kStreamsPerWave = 2;   // chunks one wavefront decodes in lockstep
// Groups of this many decode steps (anchor interval 10) run fully unrolled with their
// outputs held in registers; any other group length takes the generic loop.
constexpr int kUnrolledSteps = 9;

// A 32-bit view of ring words that the compiler must treat as aliasing the 16-bit
// reads (a word read back after a refill is reloaded, not forwarded from before it).
typedef uint32_t __attribute__((may_alias)) ring_pair_t;

// Stores the 2 words at stream position pos (even) into the ring.
__device__ __forceinline__ void ring_put(uint16_t *ring, uint32_t pos, uint32_t v)
{
    const uint32_t slot = pos & (kRingWords - 1);
    *reinterpret_cast<ring_pair_t *>(ring + slot) = v;
    if (slot < 64) *reinterpret_cast<ring_pair_t *>(ring + slot + kRingWords) = v;
}

// The block's table in LDS.  Tables of more than 16 symbols: f of symbol s for this lane
// at byte 64 s + lane, cdf of s 2 KiB further.  Tables of at most 16: the entry
// {f | cdf << 24} of s for this lane as the dword 64 s + lane (one read per symbol, and
// the 64 lanes of a read hit 64 banks), in the same 4 KiB.  Then the slot table at byte
// 256 (slot / 4) + 4 lane + slot mod 4 (20 KiB in all).  The dequantized delta lo + s * w
// is recomputed (one conversion and one fma, as the table builder does) rather than
// staged.
constexpr uint32_t kLdsCdf = kMaxBins * kLanes;
constexpr uint32_t kLdsLut = 2 * kMaxBins * kLanes;
constexpr uint32_t kLdsWords = (kLdsLut + kProbTotal * kLanes) / 4;

struct WaveDecoder {
    uint32_t x;        // rANS state, in [2^16, 2^32) between symbols
    float dlo, dw24;   // the lane's channel: lo, and the bin width times 2^24
    uint64_t pmask;    // lanes with a channel (wave-uniform)
    uint32_t cur, re;  // next unread word; words [re - R, re) are in the ring
    uint32_t i, m;     // symbols decoded so far / in the chunk
    uint16_t *ring;
    __amdgpu_buffer_rsrc_t wrs;
    bool present;

    // Decoding a symbol: the low 8 bits of the state name a slot, the slot table names
    // the symbol, and x = f * (x >> 8) + slot - cdf.  In two halves, so that the slot
    // table reads of a wavefront's two streams are both in flight before either is used.
    __device__ __forceinline__ uint32_t slot_symbol(const uint8_t *tab, uint32_t lane,
                                                    uint32_t &slot) const
    {
        slot = x & (kProbTotal - 1u);
        // byte of (slot, lane): 256 (slot / 4) + 4 lane + slot mod 4 (one bank per lane),
        // formed as ((x & 0xFC) << 6) | ((x & 3) | 4 lane) in one shift-or
        uint32_t a;
        asm("v_lshl_or_b32 %0, %1, 6, %2" : "=v"(a) : "v"(x & 0xFCu), "v"((x & 3u) | (lane << 2)));
        return tab[kLdsLut + a];
    }

    template <bool DW = false>
    __device__ __forceinline__ void update(const uint8_t *tab, uint32_t lane, uint32_t slot,
                                           uint32_t s, float &dq)
    {
        const uint32_t p = s * kLanes + lane;
        // fma(s, w, lo) with s taken as the fp16 subnormal s * 2^-24 and w pre-scaled by
        // 2^24: both scalings are exact and the fma's product is the same real number,
        // so the result is bit-identical, and the hardware reads s straight from the
        // byte without a conversion instruction
        dq = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)s), dw24, dlo);
        if constexpr (DW) {
            // the entry {f | cdf << 24} as one dword (tables of at most 16 symbols): f is
            // its low 24 bits, slot - cdf one subtraction of byte 0 of x and byte 3
            const uint32_t e = reinterpret_cast<const uint32_t *>(tab)[p];
            uint32_t d;
            asm("v_sub_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0 src1_sel:BYTE_3"
                : "=v"(d) : "v"(x), "v"(e));
            x = __umul24(e, x >> kProbBits) + d;
        } else {
            const uint32_t f = tab[p], cdf = tab[kLdsCdf + p];
            x = __umul24(f, x >> kProbBits) + slot - cdf;
        }
    }

    // Returns the symbol.
    template <bool DW = false>
    __device__ __forceinline__ uint32_t symbol(const uint8_t *tab, uint32_t lane, float &dq)
    {
        uint32_t slot;
        uint32_t s = slot_symbol(tab, lane, slot);
        // (an opaque 32-bit value from here: the byte read already zero-extends, and
        // without this the compiler masks it again)
        asm volatile("" : "+v"(s));
        update<DW>(tab, lane, slot, s, dq);
        return s;
    }

    // Loads ring chunks until the words [cur, cur + cnt) are present (rare path).
    __device__ __forceinline__ void refill_now(uint32_t cnt, uint32_t lane)
    {
        while (cur + cnt > re) {
            ring_put(ring, re + 2 * lane, __builtin_amdgcn_raw_buffer_load_b32(wrs, 2 * (re + 2 * lane), 0, kNT));
            re += kFetchWords;
        }
    }

    // Renormalisation after a symbol that is not the chunk's last, in two halves so that
    // the two streams of a wavefront can share one refill branch and overlap their ring
    // reads.  First: which lanes read a word, and how many words that takes.
    __device__ __forceinline__ uint64_t renorm_mask() const
    {
        // the compare's own lane mask (a ballot of a combined condition would first be
        // materialised as a 0/1 vector and compared again)
        return __builtin_amdgcn_uicmp(x, kStateLow, 36 /* unsigned less-than */) & pmask;
    }

    // Then: every lane reads the ring at its rank among the reading lanes (lanes that do
    // not read take a neighbour's word, in bounds), and the reading lanes shift it in.
    // No branch: some lane reads at almost every step.
    __device__ __forceinline__ void renorm_take(uint64_t mask)
    {
        const uint32_t at = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, cur & (kRingWords - 1)));
        const uint32_t w = ring[at];
        const bool need = present && (x < kStateLow);
        x = need ? (x << 16) | w : x;
        cur += (uint32_t)__builtin_popcountll(mask);
    }

    __device__ __forceinline__ void renorm(uint32_t lane)
    {
        const uint64_t mask = renorm_mask();
        const uint32_t cnt = (uint32_t)__builtin_popcountll(mask);
        if (__builtin_expect(cur + cnt > re, 0)) refill_now(cnt, lane);
        renorm_take(mask);
    }
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <bool SYMBOLS>
__device__ __forceinline__ void put_out(const __amdgpu_buffer_rsrc_t &ors, uint32_t olane,
                                        uint32_t orow, uint32_t v)
{
    if (SYMBOLS)
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)v, ors, olane, orow, kNT);
    else
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)v, ors, olane, orow, kNT);
}

// Writes the rows held for one unrolled group: fp16 values are converted two rows per
// instruction (round to nearest even), symbols are stored as they are.
template <bool SYMBOLS>
__device__ __forceinline__ void flush_rows(const __amdgpu_buffer_rsrc_t &ors, uint32_t olane,
                                           uint32_t orow, uint32_t ostride, const float *yf,
                                           const uint32_t *ys)
{
#pragma unroll
    for (int u = 0; u < kUnrolledSteps; u += 2) {
        if (SYMBOLS) {
            put_out<true>(ors, olane, orow + u * ostride, ys[u]);
            if (u + 1 < kUnrolledSteps) put_out<true>(ors, olane, orow + (u + 1) * ostride, ys[u + 1]);
        } else if (u + 1 < kUnrolledSteps) {
            const f32x2 v = {yf[u], yf[u + 1]};
            const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
            put_out<false>(ors, olane, orow + u * ostride, h & 0xFFFFu);
            put_out<false>(ors, olane, orow + (u + 1) * ostride, h >> 16);
        } else {
            put_out<false>(ors, olane, orow + u * ostride, f2h(yf[u]));
        }
    }
}

// The page pool of one (row, channel block) of a paged output, shared by the streams of
// a wavefront: pool is the row's pool from channel b * 64 on; page p starts p << lp token
// rows into it.  (Every decoded token is below S, so its block is below the table's
// ceil(S / 2^lp) entries.)
struct PageMap {
    __amdgpu_buffer_rsrc_t pool;
    const int32_t *bt;
    uint32_t lp, num_pages;
};

// The page map of (row, b) for a paged decode (an unused one otherwise).
template <bool PAGED>
__device__ __forceinline__ PageMap page_map(const Geom &g, const Paged &pg, uint32_t row, uint32_t b)
{
    if constexpr (!PAGED) return PageMap{make_rsrc(nullptr, 0u), nullptr, 0u, 0u};
    const uint64_t elems = ((uint64_t)pg.num_pages << pg.lp) * g.C;
    return PageMap{make_rsrc(pg.pages + (uint64_t)row * elems + b * kLanes,
                             (uint32_t)(2 * elems - 2 * (uint64_t)b * kLanes)),
                   pg.bt, pg.lp, pg.num_pages};
}

// The outlier entries of group gidx = (chunk k, row, channel block b), one per lane, over
// the decoded rows.  The container is not trusted: offsets are clamped to the entry count
// and an entry whose token or channel lies outside its group is skipped.
template <bool PAGED>
__device__ __forceinline__ void apply_group_outliers(const Geom &g, const uint8_t *container,
                                                     const ContainerView &cv, uint64_t gidx,
                                                     uint32_t k, uint32_t row, uint32_t b,
                                                     uint32_t lane, uint16_t *out, const Paged &pg)
{
    const uint64_t *offs = reinterpret_cast<const uint64_t *>(container + cv.out_off);
    const uint64_t beg = min(offs[gidx], cv.n_out);
    const uint64_t end = max(beg, min(offs[gidx + 1], cv.n_out));
    const uint32_t t0 = k * g.Tc, len = chunk_len(g, k);
    const uint32_t *keys = reinterpret_cast<const uint32_t *>(container + cv.keys_off);
    const uint16_t *vals = reinterpret_cast<const uint16_t *>(container + cv.vals_off);
    for (uint64_t e = beg + lane; e < end; e += kLanes) {
        const uint32_t key = keys[e];
        const uint32_t u = key >> 6, c = b * kLanes + (key & 63u);
        if (u >= len || c >= g.C) continue;
        const uint32_t t = t0 + u;
        uint16_t *dst;
        if constexpr (PAGED) {
            const uint32_t blk = t >> pg.lp;
            if (blk >= pg.n_blocks) continue;
            const uint32_t id = (uint32_t)pg.bt[blk];
            if (id >= pg.num_pages) continue;  // negative ids too
            const uint64_t pool = ((uint64_t)pg.num_pages << pg.lp) * g.C;
            dst = pg.pages + row * pool + (((uint64_t)id << pg.lp) + (t & ((1u << pg.lp) - 1u))) * g.C + c;
        } else {
            dst = out + ((uint64_t)row * g.S + t) * g.C + c;
        }
        *dst = vals[e];
    }
}

// One decoder stream: chunk k of (row, channel block b), one channel per lane, with its
// anchor rows, output rows and payload words.  Vector memory is only touched at anchor
// boundaries: at a group's start the next anchor row and the next chunk of words are
// requested and the previous group's outputs (held in registers) are written; the
// requested data is consumed at the group's end.  Waits for it therefore never wait for
// a store issued during the group.
template <bool SYMBOLS, bool PAGED = false, bool A8 = false, bool DW = false>
struct Stream {
    WaveDecoder dec;
    __amdgpu_buffer_rsrc_t ars, ors;
    uint32_t ng, len;           // groups / tokens in the chunk
    uint32_t astride, ostride, olane;
    uint32_t a16;               // anchor row of the current group (fp16 bits)
    float galo, gaw;            // 8-bit anchors (A8): ars holds codes on this lane's grid
    float af;
    uint32_t orow;              // byte offset of the current anchor row (paged: its token)
    uint32_t orow_held;         // byte offset of the first row held in yf / ys (paged: token)
    bool held;                  // yf / ys hold the outputs of the previous group
    uint32_t a_next, pf, pf_at; // requests of the current group
    bool fetch;
    float yf[kUnrolledSteps];
    uint32_t ys[kUnrolledSteps];
    // paged output only: the block whose page is current, and the lane's byte offset of
    // that page in the pool (for an invalid page id, the pool's end)
    uint32_t pblk, pvo;

    static constexpr uint32_t kNoBlock = 0xFFFFFFFFu;

    // Byte offset of token t in its page, after making pvo that page's offset.  A page id
    // that is not a page of the pool selects the pool's end: the store is still issued
    // (so every row store of a group stays unconditional) and the buffer range check
    // discards it.  (The pool and one page more fit 32 bits, so no offset wraps.)
    __device__ __forceinline__ uint32_t page_row(const PageMap &pm, uint32_t t)
    {
        const uint32_t blk = t >> pm.lp;
        if (blk != pblk) {
            pblk = blk;
            // a scalar load (the table is read-only and the same for the whole wavefront),
            // waited for in the same block
            uint32_t pg;
            const int32_t *p = pm.bt + blk;
            asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)"
                         : "=s"(pg) : "s"(p) : "memory");
            pvo = olane + ((pg < pm.num_pages ? pg : pm.num_pages) << pm.lp) * ostride;
        }
        return (t & ((1u << pm.lp) - 1u)) * ostride;
    }

    // stores value v as the row at orow value r (paged: token r)
    __device__ __forceinline__ void store_row(const PageMap &pm, uint32_t r, uint32_t v)
    {
        if constexpr (PAGED) {
            const uint32_t o = page_row(pm, r);
            put_out<SYMBOLS>(pm.pool, pvo, o, v);
        } else {
            put_out<SYMBOLS>(ors, olane, r, v);
        }
    }

    // step of orow per token row: bytes in the linear output, one token when paged
    __device__ __forceinline__ uint32_t rstep() const { return PAGED ? 1u : ostride; }

    // the rows held for one unrolled group
    __device__ __forceinline__ void flush(const PageMap &pm)
    {
        if constexpr (!PAGED) {
            flush_rows<SYMBOLS>(ors, olane, orow_held, ostride, yf, ys);
        } else if ((1u << pm.lp) - (orow_held & ((1u << pm.lp) - 1u)) >= (uint32_t)kUnrolledSteps) {
            // the group's rows lie in one page: stored as the linear output stores them
            const uint32_t o = page_row(pm, orow_held);
            flush_rows<SYMBOLS>(pm.pool, pvo, o, ostride, yf, ys);
        } else {
            flush_paged_rows(pm);
        }
    }

    // the held rows one by one, each through its own page
    __device__ __forceinline__ void flush_paged_rows(const PageMap &pm)
    {
#pragma unroll
        for (int u = 0; u < kUnrolledSteps; u += 2) {
            if (u + 1 < kUnrolledSteps) {
                const f32x2 v = {yf[u], yf[u + 1]};
                const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
                store_row(pm, orow_held + u, h & 0xFFFFu);
                store_row(pm, orow_held + u + 1, h >> 16);
            } else {
                store_row(pm, orow_held + u, f2h(yf[u]));
            }
        }
    }

    __device__ __forceinline__ void init(const Geom &g, uint16_t *ring,
                                         const float *__restrict__ lo,
                                         const float *__restrict__ w,
                                         const uint8_t *__restrict__ container,
                                         const ContainerView &cv, uint32_t k, uint32_t row,
                                         uint32_t b, uint32_t lane, bool present,
                                         uint16_t *__restrict__ out, uint8_t *__restrict__ sym_out)
    {
        const uint32_t nl = min(kLanes, g.C - b * kLanes);
        const uint32_t t0_chunk = k * g.Tc;
        len = chunk_len(g, k);
        ng = (len + g.G - 1) / g.G;
        dec.present = present;
        dec.m = len - ng;
        dec.i = 0;
        dec.ring = ring;
        const uint64_t gidx = ((uint64_t)(k - g.kb) * 2 * g.L + row) * g.NB + b;
        const uint64_t *offs = reinterpret_cast<const uint64_t *>(container + cv.offsets_off);
        const uint64_t end = min(offs[gidx + 1], cv.payload_words);
        const uint64_t beg = min(offs[gidx], end);
        // words from the group's first word to the end of the zero-padded payload; the
        // hardware range check returns 0 for anything past it
        const uint64_t avail = 2 * (cv.payload_words - beg) + kPayloadPadBytes;
        dec.wrs = make_rsrc(container + cv.payload_off + 2 * beg,
                            (uint32_t)min(avail, (uint64_t)0xFFFFFFFFu));
        // anchor rows of this chunk: row gi at byte 2 * (gi * C + lane); reads beyond the
        // anchors section return 0
        const uint64_t aoff = anchor_row(g, k, row, 0) * g.C + b * kLanes;
        const uint64_t aesz = A8 ? 1u : 2u;  // bytes per anchor element
        ars = make_rsrc(container + cv.anchors_off + aesz * aoff,
                        (uint32_t)min(cv.anchors_bytes - min(aesz * aoff, cv.anchors_bytes),
                                      (uint64_t)0xFFFFFFFFu));
        astride = (uint32_t)aesz * g.C;
        galo = 0.0f;
        gaw = 0.0f;
        if (A8 && present) {
            galo = g.alo[(uint64_t)row * g.C + b * kLanes + lane];
            gaw = g.aw[(uint64_t)row * g.C + b * kLanes + lane];
        }
        const uint64_t obase = ((uint64_t)row * g.S + t0_chunk) * g.C + b * kLanes;
        ors = SYMBOLS ? make_rsrc(sym_out + obase, 0xFFFFFFFFu) : make_rsrc(out + obase, 0xFFFFFFFFu);
        ostride = g.C * (SYMBOLS ? 1u : 2u);  // bytes between token rows
        olane = lane * (SYMBOLS ? 1u : 2u);
        if constexpr (PAGED) {
            pblk = kNoBlock;
            pvo = olane;
        }

        dec.x = kStateLow;
        dec.dlo = present ? lo[(uint64_t)row * g.C + b * kLanes + lane] : 0.0f;
        dec.dw24 = present ? w[(uint64_t)row * g.C + b * kLanes + lane] * 16777216.0f : 0.0f;
        dec.pmask = __builtin_amdgcn_ballot_w64(present);
        dec.re = 0;
        if (dec.m > 0) {
            dec.cur = 0;
            dec.refill_now(kRingWords, lane);
            if (present) dec.x = ((uint32_t)ring[2 * lane] << 16) | ring[2 * lane + 1];
        }
        dec.cur = 2 * nl;
        held = false;
        orow = PAGED ? t0_chunk : 0u;
        orow_held = orow;
    }

    // first anchor row; the empty asm pins the wait for it here
    __device__ __forceinline__ void first_anchor(uint32_t lane)
    {
        uint32_t v = A8 ? __builtin_amdgcn_raw_buffer_load_b8(ars, lane, 0, kNT)
                        : __builtin_amdgcn_raw_buffer_load_b16(ars, 2 * lane, 0, kNT);
        asm volatile("" : "+v"(v));
        set_anchor(v);
    }

    // the anchor row from its loaded value: fp16 bits, or an 8-bit code on the grid
    __device__ __forceinline__ void set_anchor(uint32_t v)
    {
        a16 = A8 ? f2h_fma((float)v, gaw, galo) : v;
        af = h2f(a16);
    }

    // decode steps in group gi (tokens less the anchor), wave-uniform
    __device__ __forceinline__ uint32_t steps(const Geom &g, uint32_t gi) const
    {
        return __builtin_amdgcn_readfirstlane(min(g.G, len - gi * g.G) - 1);
    }

    // a full group that does not hold the chunk's last symbol
    __device__ __forceinline__ bool unrollable(uint32_t nsteps) const
    {
        return nsteps == (uint32_t)kUnrolledSteps && dec.i + kUnrolledSteps < dec.m;
    }

    // the next anchor row, and the next chunk of words if the ring has room for it (with
    // non-temporal loads a request that would be dropped is not worth a fetch: its words
    // would be fetched again, not found in the cache)
    __device__ __forceinline__ void request(uint32_t gi, uint32_t lane)
    {
        a_next = A8 ? __builtin_amdgcn_raw_buffer_load_b8(ars, lane, (gi + 1) * astride, kNT)
                    : __builtin_amdgcn_raw_buffer_load_b16(ars, 2 * lane, (gi + 1) * astride, kNT);
        fetch = dec.m > 0 && dec.re + kFetchWords - dec.cur <= kRingWords;
        pf_at = dec.re;
        pf = 0;
        if (fetch) pf = __builtin_amdgcn_raw_buffer_load_b32(dec.wrs, 2 * (pf_at + 2 * lane), 0, kNT);
    }

    // write_rows for a stream holding rows with every lane present
    __device__ __forceinline__ void write_held_rows(const PageMap &pm)
    {
        flush(pm);
        held = false;
        store_row(pm, orow, SYMBOLS ? 0u : a16);
        orow += rstep();
    }

    // the previous group's outputs, then this group's anchor row
    __device__ __forceinline__ void write_rows(const PageMap &pm)
    {
        if (held) {
            if (dec.present) flush(pm);
            held = false;
        }
        if (dec.present) store_row(pm, orow, SYMBOLS ? 0u : a16);
        orow += rstep();
    }

    // takes in the requests; the ring chunk is dropped if a refill inside the group
    // already loaded those words.  (The empty asm pins where the loaded values are first
    // needed, so the wait for them is placed here.)
    __device__ __forceinline__ void consume(uint32_t lane)
    {
        uint32_t an = a_next, pv = pf;
        asm volatile("" : "+v"(an), "+v"(pv));
        set_anchor(an);
        if (fetch && dec.re == pf_at) {
            ring_put(dec.ring, pf_at + 2 * lane, pv);
            dec.re = pf_at + kFetchWords;
        }
    }

    // step u of an unrolled group: the output stays in a register
    __device__ __forceinline__ void hold(int u, uint32_t s, float dq)
    {
        if (SYMBOLS)
            ys[u] = s;
        else
            yf[u] = af + dq;
    }

    __device__ __forceinline__ void step_held(const uint8_t *tab, uint32_t lane, int u)
    {
        float dq;
        const uint32_t s = dec.symbol<DW>(tab, lane, dq);
        hold(u, s, dq);
    }

    __device__ __forceinline__ void finish_unrolled()
    {
        dec.i += kUnrolledSteps;
        held = true;
        orow_held = orow;
        orow += kUnrolledSteps * rstep();
    }

    __device__ __forceinline__ void unrolled(const uint8_t *tab, uint32_t lane)
    {
#pragma unroll
        for (int u = 0; u < kUnrolledSteps; ++u) {
            step_held(tab, lane, u);
            // the state update is computed here, next to its table reads
            asm volatile("" : "+v"(dec.x));
            dec.renorm(lane);
        }
        finish_unrolled();
    }

    // any other group: one store per step
    __device__ __forceinline__ void generic(const PageMap &pm, const uint8_t *tab, uint32_t lane,
                                            uint32_t nsteps)
    {
        for (uint32_t u = nsteps; u != 0; --u) {
            float dq;
            const uint32_t sym = dec.symbol<DW>(tab, lane, dq);
            if (dec.present)
                store_row(pm, orow, SYMBOLS ? sym : f2h(af + dq));
            orow += rstep();
            if (++dec.i < dec.m) dec.renorm(lane);
        }
    }

    __device__ __forceinline__ void final_flush(const PageMap &pm)
    {
        if (held && dec.present) flush(pm);
    }
};

// An unrolled group of both streams of a wavefront in lockstep.
template <bool SYMBOLS, bool PAGED, bool A8, bool DW, int NS>
__device__ __forceinline__ void paired_steps(Stream<SYMBOLS, PAGED, A8, DW> (&st)[NS], const uint8_t *tab,
                                             uint32_t lane)
{
#pragma unroll
    for (int u = 0; u < kUnrolledSteps; ++u) {
        uint32_t slot[NS], sym[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) sym[s] = st[s].dec.slot_symbol(tab, lane, slot[s]);
        // (opaque 32-bit values: see WaveDecoder::symbol)
        asm volatile("" : "+v"(sym[0]), "+v"(sym[NS - 1]));
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            float dq;
            st[s].dec.template update<DW>(tab, lane, slot[s], sym[s], dq);
            st[s].hold(u, sym[s], dq);
        }
        // both state updates are computed here, next to their table reads
        asm volatile("" : "+v"(st[0].dec.x), "+v"(st[NS - 1].dec.x));
        // Renormalisation.  Each lane reads the ring at its rank among the reading lanes
        // (lanes that do not read take a neighbour's word, in bounds) before the check
        // that the ring holds those words, so the reads do not wait for the check; in
        // the rare case that a refill is due they are repeated after it.
        bool need[NS];
        uint32_t at[NS], wv[NS], curn[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            WaveDecoder &d = st[s].dec;
            need[s] = d.present && d.x < kStateLow;
            const uint64_t mask = __builtin_amdgcn_ballot_w64(need[s]);
            at[s] = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)mask, d.cur & (kRingWords - 1)));
            wv[s] = d.ring[at[s]];
            curn[s] = d.cur + (uint32_t)__builtin_popcountll(mask);
        }
        int32_t room = (int32_t)(st[0].dec.re - curn[0]);
        if (NS == 2) room |= (int32_t)(st[NS - 1].dec.re - curn[NS - 1]);
        if (__builtin_expect(room < 0, 0)) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                st[s].dec.refill_now(curn[s] - st[s].dec.cur, lane);
                wv[s] = st[s].dec.ring[at[s]];
            }
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            WaveDecoder &d = st[s].dec;
            d.x = need[s] ? (d.x << 16) | wv[s] : d.x;
            d.cur = curn[s];
        }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) st[s].finish_unrolled();
}

// One wavefront decodes NS chunks of the same (row, channel block) in lockstep, sharing
// the block's LDS table.  With two, the symbol decodes of both streams sit in one
// basic block, so the dependent LDS reads of one overlap the arithmetic of the other.
// With MULTI, k0 and k1 index srcs->ch: the chunk and the container it is read from.
template <bool SYMBOLS, bool FULL, int NS, bool PAGED, bool A8, bool MULTI = false, bool OUTL = false,
          bool DW = false>
__device__ __forceinline__ void decode_chunks(const Geom &g, const uint8_t *__restrict__ tab,
                                              uint16_t *__restrict__ ring,
                                              const float *__restrict__ lo,
                                              const float *__restrict__ w,
                                              const uint8_t *__restrict__ container,
                                              const ContainerView &cv, uint32_t k0, uint32_t k1,
                                              uint32_t row, uint32_t b, uint32_t lane,
                                              uint16_t *__restrict__ out,
                                              uint8_t *__restrict__ sym_out, const Paged &pg,
                                              const ChunkSrcs *srcs = nullptr)
{
    const bool present = FULL || lane < min(kLanes, g.C - b * kLanes);
    const PageMap pm = page_map<PAGED>(g, pg, row, b);
    Stream<SYMBOLS, PAGED, A8, DW> st[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const uint32_t i = s == 0 ? k0 : k1;
        if constexpr (MULTI) {
            const BatchChunk &ch = srcs->ch[i];
            Geom gk = g;
            gk.kb = ch.kb;
            gk.ke = ch.k + 1;
            ContainerView cvk{};
            cvk.offsets_off = ch.offsets_off;
            cvk.anchors_off = ch.anchors_off;
            cvk.anchors_bytes = ch.anchors_bytes;
            cvk.payload_off = ch.payload_off;
            cvk.payload_words = ch.payload_words;
            st[s].init(gk, ring + s * kRingAlloc, lo, w, ch.c, cvk, ch.k, row, b, lane, present,
                       out, sym_out);
        } else {
            st[s].init(g, ring + s * kRingAlloc, lo, w, container, cv, i, row, b, lane, present,
                       out, sym_out);
        }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) st[s].first_anchor(lane);
    uint32_t ngmax = st[0].ng;
    if (NS == 2) ngmax = max(ngmax, st[NS - 1].ng);

    for (uint32_t gi = 0; gi < ngmax; ++gi) {
        bool act[NS];
        uint32_t nsteps[NS];
        bool unr[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            act[s] = gi < st[s].ng;
            nsteps[s] = act[s] ? st[s].steps(g, gi) : 0u;
            unr[s] = act[s] && st[s].unrollable(nsteps[s]);
        }
        if (FULL && NS == 2 && unr[0] && unr[NS - 1] && st[0].held && st[NS - 1].held) {
            // The common group.  Every memory operation in it is unconditional, so the
            // wait at its end (the counter retires in issue order) covers the requests
            // but not the 20 row stores issued after them.
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < NS; ++s) st[s].request(gi, lane);
#pragma unroll
            for (int s = 0; s < NS; ++s) st[s].write_held_rows(pm);
            __builtin_amdgcn_sched_barrier(0);
            paired_steps(st, tab, lane);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < NS; ++s) st[s].consume(lane);
            continue;
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < NS; ++s)
            if (act[s]) st[s].request(gi, lane);
#pragma unroll
        for (int s = 0; s < NS; ++s)
            if (act[s]) st[s].write_rows(pm);
        __builtin_amdgcn_sched_barrier(0);
        if (NS == 2 && unr[0] && unr[NS - 1]) {
            paired_steps(st, tab, lane);
        } else {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                if (unr[s])
                    st[s].unrolled(tab, lane);
                else if (act[s])
                    st[s].generic(pm, tab, lane, nsteps[s]);
            }
        }

        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < NS; ++s)
            if (act[s]) st[s].consume(lane);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) st[s].final_flush(pm);
    if constexpr (OUTL) {
        // The chunks' outlier entries over their rows.  An entry's element was stored by
        // another lane of this wavefront: the release fence orders those row stores
        // before the entries' stores.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const uint32_t k = s == 0 ? k0 : k1;
            const uint64_t gidx = ((uint64_t)(k - g.kb) * 2 * g.L + row) * g.NB + b;
            apply_group_outliers<PAGED>(g, container, cv, gidx, k, row, b, lane, out, pg);
        }
    }
}

// Block = WPB wavefronts over the chunks [kb + 2 WPB set, kb + 2 WPB (set + 1)) of one
// (row, channel block); wavefront w takes chunks base + w and base + w + WPB.  Launches
// over many chunks use 4 wavefronts per block, sharing the staged table; launches over
// a few chunks (a streamed chunk) use 1, so that more blocks are resident.
//
// Block order: the channel block varies fastest, then the chunk set, then the row, so
// that the blocks dispatched together cover every 128-byte column of the same token rows
// (whole 2 KiB rows for C = 1024 are written at about the same time).  Blocks are dealt
// to the 8 XCDs in turn (block index mod 8), so the channel block is also rotated by the
// row: otherwise an XCD would hold only the columns b with one residue mod 8, and its
// writes and anchor reads would queue on the few L2 / memory channels those addresses
// map to.
template <bool SYMBOLS, uint32_t WPB, bool PAGED, bool A8, bool MULTI, bool OUTL = false>
__device__ __forceinline__ void decode_block(Geom g, const uint8_t *__restrict__ bins,
                                             const uint32_t *__restrict__ dtab,
                                             const float *__restrict__ lo,
                                             const float *__restrict__ w,
                                             const uint8_t *__restrict__ container,
                                             const ContainerView &cv, uint32_t n_sets,
                                             uint16_t *__restrict__ out,
                                             uint8_t *__restrict__ sym_out, const Paged &pg,
                                             const ChunkSrcs *srcs)
{
    __shared__ uint32_t tab[kLdsWords];
    __shared__ uint16_t rings[WPB * kStreamsPerWave * kRingAlloc];
    const uint32_t tmp = blockIdx.x / g.NB;
    const uint32_t set = tmp % n_sets;
    const uint32_t row = tmp / n_sets;
    const uint32_t b = (blockIdx.x % g.NB + row) % g.NB;
    // chunks (indices into srcs->ch with MULTI) of this wavefront: k0, and k1 if below ke
    uint32_t k0 = g.kb + set * WPB * kStreamsPerWave;
    if constexpr (MULTI) {
        const BatchTables &t = srcs->tab[srcs->set_tab[set]];
        bins = t.bins;
        dtab = t.dtab;
        lo = t.lo;
        w = t.w;
        g.alo = t.alo;
        g.aw = t.aw;
        k0 = srcs->set_first[set];
        g.ke = k0 + srcs->set_n[set];
    }
    const uint32_t N = bins[row];
    // stage f and cdf of the N used entries as bytes, and the slot table
    const uint32_t *src = dtab + (uint64_t)(row * g.NB + b) * kTabBlock;
    uint8_t *tb8 = reinterpret_cast<uint8_t *>(tab);
    // tables of at most 16 symbols: their entries as dwords (one read per symbol and no
    // bank conflicts, in the same 4 KiB); larger ones as the f and cdf byte planes
    const bool dw = N <= 16;
    if (dw) {
        for (uint32_t j = threadIdx.x; j < N * kLanes; j += blockDim.x) tab[j] = src[j];
    } else {
        for (uint32_t j = threadIdx.x; j < N * kLanes; j += blockDim.x) {
            const uint32_t e = src[j];
            tb8[j] = (uint8_t)e;
            tb8[kLdsCdf + j] = (uint8_t)(e >> 24);
        }
    }
    const uint4 *lsrc = reinterpret_cast<const uint4 *>(src + kTabLut);
    uint4 *ldst = reinterpret_cast<uint4 *>(tb8 + kLdsLut);
    for (uint32_t j = threadIdx.x; j < kProbTotal * kLanes / 16; j += blockDim.x)
        ldst[j] = lsrc[j];
    __syncthreads();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
    const uint32_t lane = threadIdx.x % kLanes;
    k0 += wave;
    const uint32_t k1 = k0 + WPB;
    if (k0 >= g.ke) return;
    const uint8_t *tb = reinterpret_cast<const uint8_t *>(tab);
    uint16_t *ring = rings + wave * kStreamsPerWave * kRingAlloc;
    const bool pair = k1 < g.ke;
    const bool full = g.C - b * kLanes >= kLanes;
    if (dw) {
        if (full && pair)
            decode_chunks<SYMBOLS, true, 2, PAGED, A8, MULTI, OUTL, true>(g, tb, ring, lo, w, container, cv, k0, k1, row, b, lane, out, sym_out, pg, srcs);
        else if (full)
            decode_chunks<SYMBOLS, true, 1, PAGED, A8, MULTI, OUTL, true>(g, tb, ring, lo, w, container, cv, k0, k1, row, b, lane, out, sym_out, pg, srcs);
        else if (pair)
            decode_chunks<SYMBOLS, false, 2, PAGED, A8, MULTI, OUTL, true>(g, tb, ring, lo, w, container, cv, k0, k1, row, b, lane, out, sym_out, pg, srcs);
        else
            decode_chunks<SYMBOLS, false, 1, PAGED, A8, MULTI, OUTL, true>(g, tb, ring, lo, w, container, cv, k0, k1, row, b, lane, out, sym_out, pg, srcs);
    } else {
        if (full && pair)
            decode_chunks<SYMBOLS, true, 2, PAGED, A8, MULTI, OUTL>(g, tb, ring, lo, w, container, cv, k0, k1, row, b, lane, out, sym_out, pg, srcs);
        else if (full)
            decode_chunks<SYMBOLS, true, 1, PAGED, A8, MULTI, OUTL>(g, tb, ring, lo, w, container, cv, k0, k1, row, b, lane, out, sym_out, pg, srcs);
        else if (pair)
            decode_chunks<SYMBOLS, false, 2, PAGED, A8, MULTI, OUTL>(g, tb, ring, lo, w, container, cv, k0, k1, row, b, lane, out, sym_out, pg, srcs);
        else
            decode_chunks<SYMBOLS, false, 1, PAGED, A8, MULTI, OUTL>(g, tb, ring, lo, w, container, cv, k0, k1, row, b, lane, out, sym_out, pg, srcs);
    }
}

template <bool SYMBOLS, uint32_t WPB, bool PAGED = false, bool A8 = false, bool OUTL = false>
__global__ __launch_bounds__(WPB * 64) void k3_decode(Geom g, const uint8_t *__restrict__ bins,
                                                  const uint32_t *__restrict__ dtab,
                                                  const float *__restrict__ lo,
                                                  const float *__restrict__ w,
                                                  const uint8_t *__restrict__ container,
                                                  ContainerView cv, uint32_t n_sets,
                                                  uint16_t *__restrict__ out,
                                                  uint8_t *__restrict__ sym_out, Paged pg)
{
    decode_block<SYMBOLS, WPB, PAGED, A8, false, OUTL>(g, bins, dtab, lo, w, container, cv, n_sets,
                                                       out, sym_out, pg, nullptr);
}

// The streamed decode's form: chunks from containers of their own, in sets that share
// tables (see ChunkSrcs); blocks and wavefronts as above, a block per (row, channel
// block, set).
template <uint32_t WPB, bool A8>
__global__ __launch_bounds__(WPB * 64) void k3_decode_multi(Geom g, uint16_t *__restrict__ out,
                                                        ChunkSrcs srcs)
{
    decode_block<false, WPB, false, A8, true>(g, nullptr, nullptr, nullptr, nullptr, nullptr,
                                              ContainerView{}, srcs.n_sets, out, nullptr,
                                              Paged{}, &srcs);
}

// ------------------------------------------------------------------------------ K4
// Dequantize + anchor-add for a symbol tensor [L][2][S][C] (the unfused path):
// y = fp16_rne(f32(anchor) + fma(f32(q), w, lo)); anchors copied from the container.
__global__ __launch_bounds__(256) void k4_dequant(Geom g, const float *__restrict__ lo,
                                                   const float *__restrict__ w,
                                                   const uint8_t *__restrict__ sym,
                                                   const uint8_t *__restrict__ container,
                                                   ContainerView cv, uint32_t t_lo,
                                                   uint32_t t_hi, uint32_t tpt, uint32_t ntb,
                                                   uint16_t *__restrict__ out)
{
    const uint32_t O = g.C / 8;
    uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (uint64_t)g.L * 2 * ntb * O) return;
    uint32_t o = (uint32_t)(i % O);
    uint64_t tmp = i / O;
    uint32_t tb = (uint32_t)(tmp % ntb);
    uint32_t row = (uint32_t)(tmp / ntb);
    uint32_t t_begin = t_lo + tb * tpt;
    if (t_begin >= t_hi) return;
    uint32_t t_end = min(t_hi, t_begin + tpt);
    const uint16_t *anc = reinterpret_cast<const uint16_t *>(container + cv.anchors_off) + o * 8;
    const uint8_t *anc8 = container + cv.anchors_off + o * 8;
    float lo8[8], w8[8], af[8];
    uint64_t r0 = (uint64_t)row * g.C + o * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        lo8[j] = lo[r0 + j];
        w8[j] = w[r0 + j];
    }
    // an anchor row: fp16 bits, or 8-bit codes mapped to their grid values
    auto load_anchor = [&](uint64_t arow) -> uint4 {
        if (!g.alo) return *reinterpret_cast<const uint4 *>(anc + arow * g.C);
        const uint2 c = *reinterpret_cast<const uint2 *>(anc8 + arow * g.C);
        uint32_t h[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            h[j] = f2h_fma((float)(((j < 4 ? c.x : c.y) >> (8 * (j & 3))) & 0xFFu), g.aw[r0 + j],
                           g.alo[r0 + j]);
        return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                          h[6] | (h[7] << 16));
    };
    TokenWalk tw;
    tw.init(g, t_begin);
    if (tw.gp != 0) {
        uint4 a = load_anchor(anchor_row(g, tw.k, row, tw.gi));
        unpack8(a, af);
    }
    const uint64_t ob = (uint64_t)row * g.S * g.C + o * 8;
    for (; tw.t < t_end; tw.next(g)) {
        uint4 res;
        if (tw.gp == 0) {
            res = load_anchor(anchor_row(g, tw.k, row, tw.gi));
            unpack8(res, af);
        } else {
            uint2 s8 = *reinterpret_cast<const uint2 *>(sym + ob + (uint64_t)tw.t * g.C);
            uint32_t h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                uint32_t q = ((j < 4 ? s8.x : s8.y) >> (8 * (j & 3))) & 0xFFu;
                h[j] = f2h(af[j] + fmaf((float)q, w8[j], lo8[j]));
            }
            res = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                             h[6] | (h[7] << 16));
        }
        *reinterpret_cast<uint4 *>(out + ob + (uint64_t)tw.t * g.C) = res;
    }
}

// ------------------------------------------------------------------------------ launchers
// The value decode (fp16 or 8-bit anchors, contiguous or paged, the outlier entries
// written by the decoding wavefronts or not).
template <bool PAGED, bool OUTL>
void launch_values(const Geom &g, bool wide, dim3 grid, dim3 block, const uint8_t *bins,
                   const uint32_t *dtab, const float *lo, const float *w, const uint8_t *container,
                   const ContainerView &cv, uint32_t n_sets, uint16_t *out, const Paged &pg,
                   hipStream_t st)
{
    if (g.alo && wide)
        hipLaunchKernelGGL((k3_decode<false, kWavesPerBlock, PAGED, true, OUTL>), grid, block, 0, st,
                           g, bins, dtab, lo, w, container, cv, n_sets, out, nullptr, pg);
    else if (g.alo)
        hipLaunchKernelGGL((k3_decode<false, 1, PAGED, true, OUTL>), grid, block, 0, st, g, bins,
                           dtab, lo, w, container, cv, n_sets, out, nullptr, pg);
    else if (wide)
        hipLaunchKernelGGL((k3_decode<false, kWavesPerBlock, PAGED, false, OUTL>), grid, block, 0, st,
                           g, bins, dtab, lo, w, container, cv, n_sets, out, nullptr, pg);
    else
        hipLaunchKernelGGL((k3_decode<false, 1, PAGED, false, OUTL>), grid, block, 0, st, g, bins,
                           dtab, lo, w, container, cv, n_sets, out, nullptr, pg);
}

hipError_t launch_k3(const Geom &g, const uint8_t *bins, const uint32_t *dtab, const float *lo,
                     const float *w, const uint8_t *container, const ContainerView &cv,
                     uint16_t *out, uint8_t *sym_out, hipStream_t st)
{
    const uint32_t nk = g.ke - g.kb;
    // fewer than 8 chunks: one wavefront per block (see k3_decode)
    const bool wide = nk >= kWavesPerBlock * kStreamsPerWave;
    const uint32_t wpb = wide ? kWavesPerBlock : 1u;
    const uint32_t per_block = wpb * kStreamsPerWave;
    const uint32_t n_sets = (g.ke - g.kb + per_block - 1) / per_block;
    const uint64_t blocks = (uint64_t)g.L * 2 * g.NB * n_sets;
    const dim3 grid((uint32_t)blocks), block(wpb * kLanes);
    const Paged none{};
    // symbols do not depend on the anchors: the symbol decoder reads an 8-bit anchors
    // section as fp16 rows, in bounds (the resource ends with the section), and ignores it
    if (sym_out) {
        if (wide)
            hipLaunchKernelGGL((k3_decode<true, kWavesPerBlock>), grid, block, 0, st, g, bins,
                               dtab, lo, w, container, cv, n_sets, out, sym_out, none);
        else
            hipLaunchKernelGGL((k3_decode<true, 1>), grid, block, 0, st, g, bins, dtab,
                               lo, w, container, cv, n_sets, out, sym_out, none);
    } else if (outliers_with_rows(cv)) {
        launch_values<false, true>(g, wide, grid, block, bins, dtab, lo, w, container, cv, n_sets,
                                   out, none, st);
    } else {
        launch_values<false, false>(g, wide, grid, block, bins, dtab, lo, w, container, cv, n_sets,
                                    out, none, st);
    }
    return hipGetLastError();
}

// Attention sinks ("Guide to CacheGen", Best Practices): the container's fp16 rows of
// the sink tokens among its chunks, [L][2][n_tok][C] for tokens t0 .., written into the
// output, one thread per 8 channels of one token of one (layer, K/V) row.
__global__ __launch_bounds__(256) void k_sinks(Geom g, const uint16_t *__restrict__ sinks,
                                               uint32_t n_tok, uint32_t t0,
                                               uint16_t *__restrict__ out, Paged pg)
{
    const uint32_t O = g.C / 8;
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (uint64_t)g.L * 2 * n_tok * O) return;
    const uint32_t o = (uint32_t)(i % O);
    const uint64_t tmp = i / O;
    const uint32_t ti = (uint32_t)(tmp % n_tok);
    const uint32_t row = (uint32_t)(tmp / n_tok);
    const uint32_t t = t0 + ti;
    const uint4 v = *reinterpret_cast<const uint4 *>(sinks + ((uint64_t)row * n_tok + ti) * g.C + o * 8);
    uint16_t *dst;
    if (pg.pages) {
        const uint32_t blk = t >> pg.lp;
        if (blk >= pg.n_blocks) return;
        const uint32_t id = (uint32_t)pg.bt[blk];
        if (id >= pg.num_pages) return;  // negative ids too
        const uint64_t pool = ((uint64_t)pg.num_pages << pg.lp) * g.C;
        dst = pg.pages + row * pool + (((uint64_t)id << pg.lp) + (t & ((1u << pg.lp) - 1u))) * g.C;
    } else {
        dst = out + ((uint64_t)row * g.S + t) * g.C;
    }
    *reinterpret_cast<uint4 *>(dst + o * 8) = v;
}

hipError_t launch_sinks(const Geom &g, const uint16_t *sinks, uint32_t n_tok, uint32_t t0,
                        uint16_t *out, const Paged &pg, hipStream_t st)
{
    if (!n_tok) return hipSuccess;
    const uint64_t n = (uint64_t)g.L * 2 * n_tok * (g.C / 8);
    hipLaunchKernelGGL(k_sinks, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, st, g, sinks,
                       n_tok, t0, out, pg);
    return hipGetLastError();
}

// Sparse outlier table ("Guide to CacheGen", Solution pillar 3): the entries of one group
// (chunk, row, channel block b) per wavefront, written over the decoded rows.  The
// container is not trusted: offsets are clamped to the entry count and an entry whose
// token or channel lies outside its group is skipped.
template <bool PAGED>
__global__ __launch_bounds__(256) void k_apply_outliers(Geom g, const uint8_t *__restrict__ container,
                                                         ContainerView cv, uint64_t n_groups,
                                                         uint16_t *__restrict__ out, Paged pg)
{
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
    const uint64_t gidx = (uint64_t)blockIdx.x * (blockDim.x / kLanes) + wave;
    if (gidx >= n_groups) return;
    const uint32_t b = (uint32_t)(gidx % g.NB);
    const uint64_t tmp = gidx / g.NB;
    const uint32_t row = (uint32_t)(tmp % (2 * g.L));
    const uint32_t k = g.kb + (uint32_t)(tmp / (2 * g.L));
    apply_group_outliers<PAGED>(g, container, cv, gidx, k, row, b, threadIdx.x % kLanes, out, pg);
}

hipError_t launch_apply_outliers(const Geom &g, const uint8_t *container, const ContainerView &cv,
                                 uint16_t *out, const Paged &pg, hipStream_t st)
{
    if (!cv.outliers || !cv.n_out) return hipSuccess;
    const uint64_t n_groups = (uint64_t)(g.ke - g.kb) * g.L * 2 * g.NB;
    const uint32_t blocks = (uint32_t)((n_groups + 3) / 4);
    if (pg.pages)
        hipLaunchKernelGGL(k_apply_outliers<true>, dim3(blocks), dim3(256), 0, st, g, container, cv,
                           n_groups, out, pg);
    else
        hipLaunchKernelGGL(k_apply_outliers<false>, dim3(blocks), dim3(256), 0, st, g, container, cv,
                           n_groups, out, pg);
    return hipGetLastError();
}

hipError_t launch_k3_multi(const Geom &g, const ChunkSrcs &srcs, uint16_t *out, hipStream_t st)
{
    if (srcs.n_sets == 0) return hipSuccess;
    if (srcs.n_sets > kMaxBatch) return hipErrorInvalidValue;
    uint32_t most = 0;
    for (uint32_t j = 0; j < srcs.n_sets; ++j) {
        if (srcs.set_n[j] == 0 || srcs.set_n[j] > kBatchSetChunks ||
            srcs.set_first[j] + srcs.set_n[j] > kMaxBatch || srcs.set_tab[j] >= kMaxBatchTables)
            return hipErrorInvalidValue;
        most = std::max<uint32_t>(most, srcs.set_n[j]);
    }
    const bool a8 = srcs.tab[srcs.set_tab[0]].alo != nullptr;
    // sets of at most 2 chunks: one wavefront per block (see k3_decode)
    const bool wide = most > kStreamsPerWave;
    const uint64_t blocks = (uint64_t)g.L * 2 * g.NB * srcs.n_sets;
    const dim3 grid((uint32_t)blocks), block((wide ? kWavesPerBlock : 1u) * kLanes);
    if (a8 && wide)
        hipLaunchKernelGGL((k3_decode_multi<kWavesPerBlock, true>), grid, block, 0, st, g, out, srcs);
    else if (a8)
        hipLaunchKernelGGL((k3_decode_multi<1, true>), grid, block, 0, st, g, out, srcs);
    else if (wide)
        hipLaunchKernelGGL((k3_decode_multi<kWavesPerBlock, false>), grid, block, 0, st, g, out, srcs);
    else
        hipLaunchKernelGGL((k3_decode_multi<1, false>), grid, block, 0, st, g, out, srcs);
    return hipGetLastError();
}

hipError_t launch_k3_paged(const Geom &g, const uint8_t *bins, const uint32_t *dtab,
                           const float *lo, const float *w, const uint8_t *container,
                           const ContainerView &cv, const Paged &pg, hipStream_t st)
{
    const uint32_t nk = g.ke - g.kb;
    const bool wide = nk >= kWavesPerBlock * kStreamsPerWave;
    const uint32_t wpb = wide ? kWavesPerBlock : 1u;
    const uint32_t per_block = wpb * kStreamsPerWave;
    const uint32_t n_sets = (g.ke - g.kb + per_block - 1) / per_block;
    const uint64_t blocks = (uint64_t)g.L * 2 * g.NB * n_sets;
    const dim3 grid((uint32_t)blocks), block(wpb * kLanes);
    if (outliers_with_rows(cv))
        launch_values<true, true>(g, wide, grid, block, bins, dtab, lo, w, container, cv, n_sets,
                                  nullptr, pg, st);
    else
        launch_values<true, false>(g, wide, grid, block, bins, dtab, lo, w, container, cv, n_sets,
                                   nullptr, pg, st);
    return hipGetLastError();
}

hipError_t launch_k4(const Geom &g, const float *lo, const float *w, const uint8_t *sym,
                     const uint8_t *container, const ContainerView &cv, uint32_t t_lo,
                     uint32_t t_hi, uint32_t tpt, uint16_t *out, hipStream_t st)
{
    uint32_t ntb = (t_hi - t_lo + tpt - 1) / tpt;
    uint64_t threads = (uint64_t)g.L * 2 * ntb * (g.C / 8);
    hipLaunchKernelGGL(k4_dequant, dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0, st, g,
                       lo, w, sym, container, cv, t_lo, t_hi, tpt, ntb, out);
    return hipGetLastError();
}

}  // namespace cgk

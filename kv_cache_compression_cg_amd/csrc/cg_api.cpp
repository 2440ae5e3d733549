// cg_api.cpp -- host side of libcg: validation, handle ownership, allocation and the
// launch sequence of every entry point declared in include/cg.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "cg.h"
#include "cg_internal.h"

using namespace cgk;

namespace {

constexpr uint32_t kTablesMagic = 0x54424743u;  // "CGBT"
constexpr uint32_t kBlobMagic = 0x42424743u;    // "CGBB"

thread_local std::string g_error;

int fail(int code, const std::string &msg)
{
    g_error = msg;
    return code;
}

int hip_fail(hipError_t e, const char *what)
{
    if (e == hipErrorOutOfMemory)
        return fail(CG_E_NOMEM, std::string(what) + ": out of device memory");
    return fail(CG_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define CG_HIP(call, what)                       \
    do {                                         \
        hipError_t e_ = (call);                  \
        if (e_ != hipSuccess) return hip_fail(e_, what); \
    } while (0)

// Device buffer released on scope exit unless detached.
struct DevBuf {
    void *p = nullptr;
    DevBuf() = default;
    DevBuf(const DevBuf &) = delete;
    DevBuf &operator=(const DevBuf &) = delete;
    ~DevBuf()
    {
        if (p) (void)hipFree(p);
    }
    hipError_t alloc(size_t n)
    {
        return hipMalloc(&p, n ? n : 16);
    }
    void *detach()
    {
        void *q = p;
        p = nullptr;
        return q;
    }
    template <class T> T *as() const { return static_cast<T *>(p); }
};

// Makes `dev` current for the scope of a call and restores the caller's device.
struct DeviceScope {
    int prev = -1;
    bool changed = false;
    hipError_t enter(int dev)
    {
        hipError_t e = hipGetDevice(&prev);
        if (e != hipSuccess) return e;
        if (prev != dev) {
            changed = true;
            return hipSetDevice(dev);
        }
        return hipSuccess;
    }
    ~DeviceScope()
    {
        if (changed) (void)hipSetDevice(prev);
    }
};

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

uint32_t ceil_div(uint32_t a, uint32_t b) { return (a + b - 1) / b; }

}  // namespace

struct cg_tables {
    uint32_t magic;
    int device;
    uint32_t L, H, d, S, G, Tc, C, NB;
    uint32_t max_bins;
    std::vector<uint8_t> bins;    // per (layer, K/V) row, l * 2 + kv
    uint8_t *d_bins;
    float *d_lo, *d_w, *d_r;
    uint16_t *d_freqs;
    uint32_t *d_dtab;
    uint32_t n_sink;              // min(params n_sink, S)
    uint16_t *d_sinks;            // fp16 [L][2][n_sink][C], or null
    float *d_alo, *d_aw, *d_ar;   // 8-bit anchor grid [L][2][C], or null (fp16 anchors)
};

struct cg_blob {
    uint32_t magic;
    int device;
    cg_container_header hdr;
    uint8_t *d_data;
};

namespace {

Geom make_geom(const cg_tables *t, uint32_t kb, uint32_t ke)
{
    Geom g;
    g.L = t->L;
    g.C = t->C;
    g.S = t->S;
    g.G = t->G;
    g.Tc = t->Tc;
    g.NB = t->NB;
    g.ngF = ceil_div(t->Tc, t->G);
    g.kb = kb;
    g.ke = ke;
    g.n_sink = t->n_sink;
    g.alo = t->d_alo;
    g.aw = t->d_aw;
    g.ar = t->d_ar;
    return g;
}

// Writes the sink rows among the tokens of chunks [kb, ke) into a contiguous output or,
// when pg.pages is set, into pages.
hipError_t put_sinks(const cg_tables *t, uint32_t kb, uint32_t ke, uint16_t *out, const Paged &pg,
                     hipStream_t st)
{
    if (!t->n_sink) return hipSuccess;
    const uint64_t a = (uint64_t)kb * t->Tc, b = std::min<uint64_t>((uint64_t)ke * t->Tc, t->n_sink);
    if (a >= b) return hipSuccess;
    return launch_sinks(make_geom(t, kb, ke), t->d_sinks, t->n_sink, (uint32_t)a, (uint32_t)b, out, pg, st);
}

// Tokens per thread for the streaming kernels: about two million threads in flight.
uint32_t pick_tpt(const cg_tables *t, uint64_t tokens)
{
    uint64_t work = (uint64_t)t->L * 2 * tokens * (t->C / 8);
    uint64_t tpt = (work + (1u << 21) - 1) >> 21;
    if (tpt < 8) tpt = 8;
    if (tpt > 4096) tpt = 4096;
    return (uint32_t)tpt;
}

int check_tables(const cg_tables *t)
{
    if (!t || t->magic != kTablesMagic) return fail(CG_E_INVAL, "invalid cg_tables handle");
    return CG_OK;
}

int check_blob(const cg_tables *t, const cg_blob *b)
{
    if (!b || b->magic != kBlobMagic) return fail(CG_E_INVAL, "invalid cg_blob handle");
    const cg_container_header &h = b->hdr;
    if (h.L != t->L || h.H_kv != t->H || h.d != t->d || h.S != t->S || h.group != t->G ||
        h.chunk != t->Tc || h.reserved != (t->d_alo ? 8u : 0u))
        return fail(CG_E_CORRUPT, "container and tables describe different caches");
    return CG_OK;
}

ContainerView view_of(const cg_blob *b)
{
    ContainerView v;
    v.offsets_off = b->hdr.offsets_offset;
    v.anchors_off = b->hdr.anchors_offset;
    v.anchors_bytes = b->hdr.anchors_bytes;
    v.payload_off = b->hdr.payload_offset;
    v.payload_words = b->hdr.payload_words;
    return v;
}

uint64_t anchor_rows(const cg_tables *t, uint32_t kb, uint32_t ke)
{
    uint64_t rows = 0;
    for (uint32_t k = kb; k < ke; ++k) {
        uint32_t t0 = k * t->Tc;
        uint32_t len = (t->S - t0 < t->Tc) ? t->S - t0 : t->Tc;
        rows += (uint64_t)t->L * 2 * ceil_div(len, t->G);
    }
    return rows;
}

}  // namespace

extern "C" {

const char *cg_last_error(void) { return g_error.c_str(); }

int cg_build_cdf(const cg_params *params, const void *kv_dev, void *hip_stream, cg_tables **out)
{
    g_error.clear();
    if (!params || !kv_dev || !out || !params->bins)
        return fail(CG_E_INVAL, "null argument");
    const cg_params &p = *params;
    if (!p.L || !p.H_kv || !p.d || !p.S || !p.group || !p.chunk)
        return fail(CG_E_INVAL, "zero dimension");
    if (p.chunk > CG_MAX_CHUNK) return fail(CG_E_INVAL, "chunk > 16384");
    if (p.anchor_bits != 0 && p.anchor_bits != 8 && p.anchor_bits != 16)
        return fail(CG_E_INVAL, "anchor_bits must be 0, 8 or 16");
    uint64_t C = (uint64_t)p.H_kv * p.d;
    if (C % 8 != 0) return fail(CG_E_INVAL, "H_kv * d must be a multiple of 8");
    // 32-bit offsets inside one (layer, K/V) row of symbols and inside one chunk's rows
    if (C >= (1u << 24) || p.S >= (1u << 31) || (uint64_t)p.L * 2 * C >= (1ull << 31) ||
        (uint64_t)p.L * 2 * p.S * C >= (1ull << 40) || (uint64_t)p.S * C >= (1ull << 32) ||
        (uint64_t)p.chunk * C * 2 >= (1ull << 32))
        return fail(CG_E_INVAL, "cache too large");
    uint32_t max_bins = 0;
    for (uint32_t l = 0; l < p.L; ++l)
        for (uint32_t kv = 0; kv < 2; ++kv) {
            const uint8_t n = (kv && p.bins_v) ? p.bins_v[l] : p.bins[l];
            if (n < 2 || n > CG_MAX_BINS) return fail(CG_E_INVAL, "bins outside [2, 32]");
            if (n > max_bins) max_bins = n;
        }
    hipStream_t st = (hipStream_t)hip_stream;

    cg_tables *t = new (std::nothrow) cg_tables();
    if (!t) return fail(CG_E_NOMEM, "host allocation");
    t->magic = 0;
    CG_HIP(hipGetDevice(&t->device), "hipGetDevice");
    t->L = p.L;
    t->H = p.H_kv;
    t->d = p.d;
    t->S = p.S;
    t->G = p.group;
    t->Tc = p.chunk;
    t->C = (uint32_t)C;
    t->NB = ceil_div(t->C, kLanes);
    t->max_bins = max_bins;
    t->n_sink = std::min(p.n_sink, p.S);
    t->d_sinks = nullptr;
    t->d_alo = t->d_aw = t->d_ar = nullptr;
    t->bins.resize((size_t)2 * p.L);  // per (layer, K/V) row: l * 2 + kv
    for (uint32_t l = 0; l < p.L; ++l) {
        t->bins[2 * l] = p.bins[l];
        t->bins[2 * l + 1] = p.bins_v ? p.bins_v[l] : p.bins[l];
    }

    struct Owner {  // frees the half-built handle on every error path
        cg_tables *t;
        ~Owner()
        {
            if (t) cg_free(t);
        }
    } owner{t};
    t->magic = kTablesMagic;  // cg_free may now release it

    const uint64_t rows = (uint64_t)t->L * 2 * t->C;
    DevBuf bins_d, lo_d, w_d, r_d, fr_d, dt_d;
    CG_HIP(bins_d.alloc((uint64_t)2 * t->L), "hipMalloc");
    CG_HIP(lo_d.alloc(rows * 4), "hipMalloc");
    CG_HIP(w_d.alloc(rows * 4), "hipMalloc");
    CG_HIP(r_d.alloc(rows * 4), "hipMalloc");
    CG_HIP(fr_d.alloc(rows * kMaxBins * 2), "hipMalloc");
    const uint64_t dtab_bytes = (uint64_t)t->L * 2 * t->NB * kTabBlock * sizeof(uint32_t);
    CG_HIP(dt_d.alloc(dtab_bytes), "hipMalloc");
    t->d_bins = bins_d.as<uint8_t>();
    t->d_lo = lo_d.as<float>();
    t->d_w = w_d.as<float>();
    t->d_r = r_d.as<float>();
    t->d_freqs = fr_d.as<uint16_t>();
    t->d_dtab = dt_d.as<uint32_t>();
    if (p.anchor_bits == 8) {
        DevBuf alo_d, aw_d, ar_d;
        CG_HIP(alo_d.alloc(rows * 4), "hipMalloc");
        CG_HIP(aw_d.alloc(rows * 4), "hipMalloc");
        CG_HIP(ar_d.alloc(rows * 4), "hipMalloc");
        t->d_alo = alo_d.as<float>();
        t->d_aw = aw_d.as<float>();
        t->d_ar = ar_d.as<float>();
        alo_d.detach();
        aw_d.detach();
        ar_d.detach();
    }
    const uint64_t sink_row = (uint64_t)t->n_sink * t->C * 2;  // bytes per (layer, K/V)
    if (sink_row) {
        DevBuf sk_d;
        CG_HIP(sk_d.alloc(2 * t->L * sink_row), "hipMalloc");
        t->d_sinks = sk_d.as<uint16_t>();
        sk_d.detach();
        CG_HIP(hipMemcpy2DAsync(t->d_sinks, sink_row, kv_dev, (uint64_t)t->S * t->C * 2, sink_row,
                                2 * t->L, hipMemcpyDeviceToDevice, st),
               "copy sink rows");
    }
    bins_d.detach();
    lo_d.detach();
    w_d.detach();
    r_d.detach();
    fr_d.detach();
    dt_d.detach();

    DevBuf ordlo, ordhi, counts, flag;
    CG_HIP(ordlo.alloc(rows * 4), "hipMalloc");
    CG_HIP(ordhi.alloc(rows * 4), "hipMalloc");
    CG_HIP(counts.alloc(rows * kMaxBins * 4), "hipMalloc");
    CG_HIP(flag.alloc(4), "hipMalloc");

    CG_HIP(hipMemcpyAsync(t->d_bins, t->bins.data(), (size_t)2 * t->L, hipMemcpyHostToDevice, st),
           "copy bins");
    CG_HIP(hipMemsetAsync(ordlo.p, 0xFF, rows * 4, st), "memset");
    CG_HIP(hipMemsetAsync(ordhi.p, 0x00, rows * 4, st), "memset");
    CG_HIP(hipMemsetAsync(counts.p, 0, rows * kMaxBins * 4, st), "memset");
    CG_HIP(hipMemsetAsync(flag.p, 0, 4, st), "memset");
    CG_HIP(hipMemsetAsync(t->d_dtab, 0, dtab_bytes, st), "memset");

    Geom g = make_geom(t, 0, ceil_div(t->S, t->Tc));
    if (t->d_alo)
        CG_HIP(launch_anchor_grid(static_cast<const uint16_t *>(kv_dev), g, t->d_alo, t->d_aw,
                                  t->d_ar, st),
               "k_anchor_grid");
    CG_HIP(launch_k0(static_cast<const uint16_t *>(kv_dev), g, pick_tpt(t, t->S),
                     ordlo.as<uint32_t>(), ordhi.as<uint32_t>(), flag.as<uint32_t>(), st),
           "k0_minmax");
    CG_HIP(launch_k0_finalize(g, t->d_bins, ordlo.as<uint32_t>(), ordhi.as<uint32_t>(), t->d_lo,
                              t->d_w, t->d_r, st),
           "k0_finalize");
    CG_HIP(launch_k1(static_cast<const uint16_t *>(kv_dev), g, t->d_bins, max_bins, t->d_lo,
                     t->d_r, counts.as<uint32_t>(), st),
           "k1_hist");
    CG_HIP(launch_k1_freqs(g, t->d_bins, counts.as<uint32_t>(), t->d_lo, t->d_w, t->d_freqs,
                           t->d_dtab, st),
           "k1_freqs");
    uint32_t h_flag = 0;
    CG_HIP(hipMemcpyAsync(&h_flag, flag.p, 4, hipMemcpyDeviceToHost, st), "copy flag");
    CG_HIP(hipStreamSynchronize(st), "hipStreamSynchronize");
    if (h_flag) return fail(CG_E_NONFINITE, "KV input holds Inf or NaN");
    owner.t = nullptr;
    *out = t;
    return CG_OK;
}

int cg_encode(const cg_tables *t, const void *kv_dev, uint32_t kb, uint32_t ke, void *hip_stream,
              cg_blob **out)
{
    g_error.clear();
    if (int rc = check_tables(t)) return rc;
    if (!kv_dev || !out) return fail(CG_E_INVAL, "null argument");
    const uint32_t nchunks = ceil_div(t->S, t->Tc);
    if (kb >= ke || ke > nchunks) return fail(CG_E_INVAL, "chunk range out of bounds");
    DeviceScope ds;
    CG_HIP(ds.enter(t->device), "hipSetDevice");
    hipStream_t st = (hipStream_t)hip_stream;
    Geom g = make_geom(t, kb, ke);
    const uint32_t t_lo = kb * t->Tc;
    const uint32_t t_hi = (ke * (uint64_t)t->Tc < t->S) ? ke * t->Tc : t->S;
    const uint32_t T_r = t_hi - t_lo;
    const uint64_t n_groups = (uint64_t)(ke - kb) * t->L * 2 * t->NB;
    const uint64_t arows = anchor_rows(t, kb, ke);

    // word-read ballots of every step of every group, 64 steps per row chunk
    const uint32_t full = t->Tc < t->S ? t->Tc : t->S;
    const uint32_t mstride = (full - ceil_div(full, t->G) + 63) / 64 * 64;
    DevBuf sym, anc, lane_words, group_words, group_off, masks;
    CG_HIP(sym.alloc((uint64_t)t->L * 2 * T_r * t->C), "hipMalloc symbols");
    CG_HIP(anc.alloc(arows * t->C * 2), "hipMalloc anchors");
    CG_HIP(lane_words.alloc(n_groups * kLanes * 4), "hipMalloc");
    CG_HIP(group_words.alloc(n_groups * 8), "hipMalloc");
    CG_HIP(group_off.alloc((n_groups + 1) * 8), "hipMalloc");
    CG_HIP(masks.alloc(n_groups * (mstride ? mstride : 1) * 8), "hipMalloc ballots");

    CG_HIP(launch_k2(static_cast<const uint16_t *>(kv_dev), g, t->d_bins, t->d_lo, t->d_r, t_lo,
                     t_hi, pick_tpt(t, T_r), sym.as<uint8_t>(), t_lo, T_r, anc.as<uint16_t>(), st),
           "k2_delta_quant");
    CG_HIP(launch_k5_plan(sym.as<uint8_t>(), t_lo, T_r, g, t->d_bins, t->d_dtab,
                          lane_words.as<uint32_t>(), group_words.as<uint64_t>(),
                          masks.as<uint64_t>(), mstride, st),
           "k5_plan");
    CG_HIP(launch_scan(group_words.as<uint64_t>(), group_off.as<uint64_t>(), n_groups, st),
           "scan");
    uint64_t total_words = 0;
    CG_HIP(hipMemcpyAsync(&total_words, group_off.as<uint64_t>() + n_groups, 8,
                          hipMemcpyDeviceToHost, st),
           "copy size");
    CG_HIP(hipStreamSynchronize(st), "hipStreamSynchronize");

    cg_container_header h;
    std::memset(&h, 0, sizeof h);
    h.magic = CG_CONTAINER_MAGIC;
    h.version = 2;  // rANS with 8-bit frequencies
    h.L = t->L;
    h.H_kv = t->H;
    h.d = t->d;
    h.S = t->S;
    h.group = t->G;
    h.chunk = t->Tc;
    h.chunk_begin = kb;
    h.chunk_end = ke;
    h.n_blocks = t->NB;
    h.n_groups = n_groups;
    h.offsets_offset = align256(sizeof(cg_container_header));
    h.anchors_offset = align256(h.offsets_offset + (n_groups + 1) * 8);
    h.anchors_bytes = arows * t->C * (t->d_alo ? 1 : 2);
    h.reserved = t->d_alo ? 8u : 0u;  // bits per stored anchor element (0: fp16)
    h.payload_offset = align256(h.anchors_offset + h.anchors_bytes);
    h.payload_words = total_words;
    h.total_bytes = h.payload_offset + total_words * 2 + kPayloadPadBytes;

    cg_blob *b = new (std::nothrow) cg_blob();
    if (!b) return fail(CG_E_NOMEM, "host allocation");
    b->magic = 0;
    b->device = t->device;
    b->hdr = h;
    DevBuf data, scratch;
    hipError_t e = data.alloc(align256(h.total_bytes));
    if (e != hipSuccess) {
        delete b;
        return hip_fail(e, "hipMalloc container");
    }
    e = scratch.alloc(total_words * 2);
    if (e != hipSuccess) {
        delete b;
        return hip_fail(e, "hipMalloc scratch");
    }
    uint8_t *base = data.as<uint8_t>();
#define CG_HIP_B(call, what)                 \
    do {                                     \
        hipError_t e2_ = (call);             \
        if (e2_ != hipSuccess) {             \
            delete b;                        \
            return hip_fail(e2_, what);      \
        }                                    \
    } while (0)
    CG_HIP_B(hipMemcpyAsync(base, &h, sizeof h, hipMemcpyHostToDevice, st), "copy header");
    CG_HIP_B(hipMemsetAsync(base + h.payload_offset + total_words * 2, 0, kPayloadPadBytes, st),
             "clear padding");
    CG_HIP_B(hipMemcpyAsync(base + h.offsets_offset, group_off.p, (n_groups + 1) * 8,
                            hipMemcpyDeviceToDevice, st),
             "copy offsets");
    CG_HIP_B(hipMemcpyAsync(base + h.anchors_offset, anc.p, h.anchors_bytes,
                            hipMemcpyDeviceToDevice, st),
             "copy anchors");
    CG_HIP_B(launch_k5_encode(sym.as<uint8_t>(), t_lo, T_r, g, t->d_bins, t->d_dtab,
                              lane_words.as<uint32_t>(), group_off.as<uint64_t>(),
                              scratch.as<uint16_t>(), st),
             "k5_encode");
    CG_HIP_B(launch_k5_interleave(g, lane_words.as<uint32_t>(), group_off.as<uint64_t>(),
                                  masks.as<uint64_t>(), mstride, scratch.as<uint16_t>(),
                                  reinterpret_cast<uint16_t *>(base + h.payload_offset), st),
             "k5_interleave");
    CG_HIP_B(hipStreamSynchronize(st), "hipStreamSynchronize");
#undef CG_HIP_B
    b->d_data = static_cast<uint8_t *>(data.detach());
    b->magic = kBlobMagic;
    *out = b;
    return CG_OK;
}

int cg_decode_paged(const cg_tables *t, const cg_blob *b, const void *container_dev,
                    void *pages_dev, const int32_t *block_table_dev, uint32_t page_tokens,
                    uint32_t num_pages, void *hip_stream)
{
    g_error.clear();
    if (int rc = check_tables(t)) return rc;
    if (int rc = check_blob(t, b)) return rc;
    if (!pages_dev || !block_table_dev) return fail(CG_E_INVAL, "null pages or block table");
    if (!page_tokens || (page_tokens & (page_tokens - 1)))
        return fail(CG_E_INVAL, "page_tokens must be a power of two");
    if (!num_pages) return fail(CG_E_INVAL, "no pages");
    if ((uint64_t)num_pages * page_tokens * t->C * 2 >= (1ull << 32))
        return fail(CG_E_INVAL, "page pool too large for 32-bit offsets");
    DeviceScope ds;
    CG_HIP(ds.enter(t->device), "hipSetDevice");
    const uint8_t *cont = container_dev ? static_cast<const uint8_t *>(container_dev) : b->d_data;
    Geom g = make_geom(t, b->hdr.chunk_begin, b->hdr.chunk_end);
    Paged pg;
    pg.pages = static_cast<uint16_t *>(pages_dev);
    pg.bt = block_table_dev;
    pg.lp = 0;
    while ((1u << pg.lp) < page_tokens) ++pg.lp;
    pg.num_pages = num_pages;
    pg.n_blocks = ceil_div(t->S, page_tokens);
    CG_HIP(launch_k3_paged(g, t->d_bins, t->d_dtab, t->d_lo, t->d_w, cont, view_of(b), pg,
                           (hipStream_t)hip_stream),
           "k3_decode (paged)");
    CG_HIP(put_sinks(t, g.kb, g.ke, nullptr, pg, (hipStream_t)hip_stream), "k_sinks (paged)");
    return CG_OK;
}

int cg_decode(const cg_tables *t, const cg_blob *b, const void *container_dev, void *kv_out_dev,
              void *hip_stream)
{
    g_error.clear();
    if (int rc = check_tables(t)) return rc;
    if (int rc = check_blob(t, b)) return rc;
    if (!kv_out_dev) return fail(CG_E_INVAL, "null output");
    DeviceScope ds;
    CG_HIP(ds.enter(t->device), "hipSetDevice");
    const uint8_t *cont = container_dev ? static_cast<const uint8_t *>(container_dev) : b->d_data;
    Geom g = make_geom(t, b->hdr.chunk_begin, b->hdr.chunk_end);
    CG_HIP(launch_k3(g, t->d_bins, t->d_dtab, t->d_lo, t->d_w, cont, view_of(b), static_cast<uint16_t *>(kv_out_dev),
                     nullptr, (hipStream_t)hip_stream),
           "k3_decode");
    CG_HIP(put_sinks(t, g.kb, g.ke, static_cast<uint16_t *>(kv_out_dev), Paged{}, (hipStream_t)hip_stream),
           "k_sinks");
    return CG_OK;
}

namespace {

// Events of one streamed decode, destroyed on scope exit (HIP releases an event that is
// still pending once it completes).
struct EventSet {
    std::vector<hipEvent_t> ev;
    ~EventSet()
    {
        for (hipEvent_t e : ev)
            if (e) (void)hipEventDestroy(e);
    }
    hipError_t make(size_t n, bool timing)
    {
        ev.assign(n, nullptr);
        for (size_t i = 0; i < n; ++i) {
            hipError_t e = timing ? hipEventCreate(&ev[i])
                                  : hipEventCreateWithFlags(&ev[i], hipEventDisableTiming);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
};

bool same_shape(const cg_tables *a, const cg_tables *b)
{
    return a->L == b->L && a->H == b->H && a->d == b->d && a->S == b->S && a->G == b->G &&
           a->Tc == b->Tc;
}

}  // namespace

int cg_stream_decode(const cg_stream_item *items, uint32_t n_items, void *staging_dev,
                     uint64_t slot_bytes, uint32_t n_slots, void *kv_out_dev,
                     void *copy_stream, void *decode_stream, cg_stream_stats *stats)
{
    g_error.clear();
    if (!items || !staging_dev || !kv_out_dev || !n_slots || !slot_bytes)
        return fail(CG_E_INVAL, "null argument");
    if (copy_stream == decode_stream)
        return fail(CG_E_INVAL, "copy and decode streams must differ");
    if (slot_bytes > UINT64_MAX / n_slots) return fail(CG_E_INVAL, "staging size overflows");
    // container sections are 256-byte aligned relative to the container's first byte
    if (reinterpret_cast<uintptr_t>(staging_dev) % 256 != 0 || slot_bytes % 256 != 0)
        return fail(CG_E_INVAL, "staging memory and slot size must be 256-byte aligned");
    if (n_items == 0) {
        if (stats) *stats = cg_stream_stats{};
        return CG_OK;
    }
    const cg_tables *t0 = items[0].tables;
    if (int rc = check_tables(t0)) return rc;
    for (uint32_t i = 0; i < n_items; ++i) {
        const cg_stream_item &it = items[i];
        if (int rc = check_tables(it.tables)) return rc;
        if (int rc = check_blob(it.tables, it.blob)) return rc;
        if (!it.host_container) return fail(CG_E_INVAL, "null host container");
        if (it.tables->device != t0->device || !same_shape(it.tables, t0))
            return fail(CG_E_INVAL, "items describe different caches or devices");
        if (it.blob->hdr.total_bytes > slot_bytes)
            return fail(CG_E_INVAL, "a container does not fit a staging slot");
    }
    DeviceScope ds;
    CG_HIP(ds.enter(t0->device), "hipSetDevice");
    hipStream_t cs = (hipStream_t)copy_stream, dec = (hipStream_t)decode_stream;

    // per slot: copied (decode may start) and freed (the slot may be refilled); with
    // stats, per item: copy start/end and decode start/end
    EventSet slot_ev, item_ev;
    CG_HIP(slot_ev.make(2 * (size_t)n_slots, false), "hipEventCreate");
    if (stats) CG_HIP(item_ev.make(4 * (size_t)n_items, true), "hipEventCreate");
    hipEvent_t *copied = slot_ev.ev.data(), *freed = copied + n_slots;

    hipError_t err = hipSuccess;
    const char *what = "";
    uint64_t bytes = 0;
    const uint32_t batch = n_slots > 1 ? n_slots / 2 : 1;
    for (uint32_t i = 0; i < n_items && err == hipSuccess; ++i) {
        const cg_stream_item &it = items[i];
        const uint32_t j = i % n_slots;
        uint8_t *slot = static_cast<uint8_t *>(staging_dev) + (uint64_t)j * slot_bytes;
        const uint64_t nb = it.blob->hdr.total_bytes;
        hipEvent_t *ie = stats ? item_ev.ev.data() + 4 * (size_t)i : nullptr;
        // slot reuse: one wait per `batch` items, on the decode of the last item whose
        // slot the next `batch` items take (decodes finish in order, so that event covers
        // the earlier ones).  A wait per copy leaves the copy engine idle between copies.
        if (i >= n_slots && (i - n_slots) % batch == 0) {
            const uint32_t last = i - n_slots + batch - 1;
            if ((err = hipStreamWaitEvent(cs, freed[last % n_slots], 0)) != hipSuccess) {
                what = "hipStreamWaitEvent";
                break;
            }
        }
        if (ie && (err = hipEventRecord(ie[0], cs)) != hipSuccess) { what = "hipEventRecord"; break; }
        if ((err = hipMemcpyAsync(slot, it.host_container, nb, hipMemcpyHostToDevice, cs)) !=
            hipSuccess) {
            what = "hipMemcpyAsync";
            break;
        }
        if (ie && (err = hipEventRecord(ie[1], cs)) != hipSuccess) { what = "hipEventRecord"; break; }
        if ((err = hipEventRecord(copied[j], cs)) != hipSuccess ||
            (err = hipStreamWaitEvent(dec, copied[j], 0)) != hipSuccess) {
            what = "copy -> decode event";
            break;
        }
        if (ie && (err = hipEventRecord(ie[2], dec)) != hipSuccess) { what = "hipEventRecord"; break; }
        const cg_blob *b = it.blob;
        Geom g = make_geom(it.tables, b->hdr.chunk_begin, b->hdr.chunk_end);
        if ((err = launch_k3(g, it.tables->d_bins, it.tables->d_dtab, it.tables->d_lo, it.tables->d_w, slot, view_of(b),
                             static_cast<uint16_t *>(kv_out_dev), nullptr, dec)) != hipSuccess) {
            what = "k3_decode";
            break;
        }
        if ((err = put_sinks(it.tables, g.kb, g.ke, static_cast<uint16_t *>(kv_out_dev), Paged{}, dec)) !=
            hipSuccess) {
            what = "k_sinks";
            break;
        }
        if (ie && (err = hipEventRecord(ie[3], dec)) != hipSuccess) { what = "hipEventRecord"; break; }
        if ((err = hipEventRecord(freed[j], dec)) != hipSuccess) { what = "hipEventRecord"; break; }
        bytes += nb;
    }
    if (err != hipSuccess) {
        (void)hipStreamSynchronize(cs);
        (void)hipStreamSynchronize(dec);
        return hip_fail(err, what);
    }
    if (!stats) return CG_OK;

    CG_HIP(hipStreamSynchronize(cs), "hipStreamSynchronize");
    CG_HIP(hipStreamSynchronize(dec), "hipStreamSynchronize");
    cg_stream_stats st{};
    const hipEvent_t *ie = item_ev.ev.data();
    for (uint32_t i = 0; i < n_items; ++i) {
        float c = 0.f, d = 0.f;
        CG_HIP(hipEventElapsedTime(&c, ie[4 * i], ie[4 * i + 1]), "hipEventElapsedTime");
        CG_HIP(hipEventElapsedTime(&d, ie[4 * i + 2], ie[4 * i + 3]), "hipEventElapsedTime");
        st.copy_ms += c;
        st.decode_ms += d;
    }
    CG_HIP(hipEventElapsedTime(&st.total_ms, ie[0], ie[4 * ((size_t)n_items - 1) + 3]),
           "hipEventElapsedTime");
    st.copied_bytes = bytes;
    *stats = st;
    return CG_OK;
}

int cg_decode_symbols(const cg_tables *t, const cg_blob *b, const void *container_dev,
                      void *sym_dev, void *hip_stream)
{
    g_error.clear();
    if (int rc = check_tables(t)) return rc;
    if (int rc = check_blob(t, b)) return rc;
    if (!sym_dev) return fail(CG_E_INVAL, "null output");
    DeviceScope ds;
    CG_HIP(ds.enter(t->device), "hipSetDevice");
    const uint8_t *cont = container_dev ? static_cast<const uint8_t *>(container_dev) : b->d_data;
    Geom g = make_geom(t, b->hdr.chunk_begin, b->hdr.chunk_end);
    CG_HIP(launch_k3(g, t->d_bins, t->d_dtab, t->d_lo, t->d_w, cont, view_of(b), nullptr,
                     static_cast<uint8_t *>(sym_dev), (hipStream_t)hip_stream),
           "k3_decode_symbols");
    return CG_OK;
}

int cg_dequantize(const cg_tables *t, const cg_blob *b, const void *container_dev,
                  const void *sym_dev, void *kv_out_dev, void *hip_stream)
{
    g_error.clear();
    if (int rc = check_tables(t)) return rc;
    if (int rc = check_blob(t, b)) return rc;
    if (!sym_dev || !kv_out_dev) return fail(CG_E_INVAL, "null argument");
    DeviceScope ds;
    CG_HIP(ds.enter(t->device), "hipSetDevice");
    const uint8_t *cont = container_dev ? static_cast<const uint8_t *>(container_dev) : b->d_data;
    Geom g = make_geom(t, b->hdr.chunk_begin, b->hdr.chunk_end);
    const uint32_t t_lo = g.kb * t->Tc;
    const uint32_t t_hi = (g.ke * (uint64_t)t->Tc < t->S) ? g.ke * t->Tc : t->S;
    CG_HIP(launch_k4(g, t->d_lo, t->d_w, static_cast<const uint8_t *>(sym_dev), cont, view_of(b),
                     t_lo, t_hi, pick_tpt(t, t_hi - t_lo), static_cast<uint16_t *>(kv_out_dev),
                     (hipStream_t)hip_stream),
           "k4_dequant");
    CG_HIP(put_sinks(t, g.kb, g.ke, static_cast<uint16_t *>(kv_out_dev), Paged{}, (hipStream_t)hip_stream),
           "k_sinks");
    return CG_OK;
}

int cg_quantize(const cg_tables *t, const void *kv_dev, uint32_t kb, uint32_t ke, void *sym_dev,
                void *hip_stream)
{
    g_error.clear();
    if (int rc = check_tables(t)) return rc;
    if (!kv_dev || !sym_dev) return fail(CG_E_INVAL, "null argument");
    const uint32_t nchunks = ceil_div(t->S, t->Tc);
    if (kb >= ke || ke > nchunks) return fail(CG_E_INVAL, "chunk range out of bounds");
    DeviceScope ds;
    CG_HIP(ds.enter(t->device), "hipSetDevice");
    Geom g = make_geom(t, kb, ke);
    const uint32_t t_lo = kb * t->Tc;
    const uint32_t t_hi = (ke * (uint64_t)t->Tc < t->S) ? ke * t->Tc : t->S;
    CG_HIP(launch_k2(static_cast<const uint16_t *>(kv_dev), g, t->d_bins, t->d_lo, t->d_r, t_lo,
                     t_hi, pick_tpt(t, t_hi - t_lo), static_cast<uint8_t *>(sym_dev), 0, t->S,
                     nullptr, (hipStream_t)hip_stream),
           "k2_delta_quant");
    return CG_OK;
}

int cg_tables_export(const cg_tables *t, float *lo, float *w, float *r, uint16_t *freqs)
{
    g_error.clear();
    if (int rc = check_tables(t)) return rc;
    DeviceScope ds;
    CG_HIP(ds.enter(t->device), "hipSetDevice");
    const uint64_t rows = (uint64_t)t->L * 2 * t->C;
    if (lo) CG_HIP(hipMemcpy(lo, t->d_lo, rows * 4, hipMemcpyDeviceToHost), "copy lo");
    if (w) CG_HIP(hipMemcpy(w, t->d_w, rows * 4, hipMemcpyDeviceToHost), "copy w");
    if (r) CG_HIP(hipMemcpy(r, t->d_r, rows * 4, hipMemcpyDeviceToHost), "copy r");
    if (freqs)
        CG_HIP(hipMemcpy(freqs, t->d_freqs, rows * kMaxBins * 2, hipMemcpyDeviceToHost),
               "copy freqs");
    return CG_OK;
}

int cg_tables_get_info(const cg_tables *t, cg_tables_info *info)
{
    g_error.clear();
    if (int rc = check_tables(t)) return rc;
    if (!info) return fail(CG_E_INVAL, "null argument");
    info->L = t->L;
    info->H_kv = t->H;
    info->d = t->d;
    info->S = t->S;
    info->group = t->G;
    info->chunk = t->Tc;
    uint64_t bytes = (uint64_t)t->L * 2 * t->C * 8 + (uint64_t)2 * t->L;
    for (uint32_t r = 0; r < 2 * t->L; ++r) bytes += (uint64_t)t->C * t->bins[r] * 2;
    bytes += (uint64_t)2 * t->L * t->n_sink * t->C * 2;
    if (t->d_alo) bytes += (uint64_t)t->L * 2 * t->C * 8;
    info->stored_bytes = bytes;
    return CG_OK;
}

int cg_blob_get_info(const cg_blob *b, cg_blob_info *info)
{
    g_error.clear();
    if (!b || b->magic != kBlobMagic) return fail(CG_E_INVAL, "invalid cg_blob handle");
    if (!info) return fail(CG_E_INVAL, "null argument");
    info->data = b->d_data;
    info->header = b->hdr;
    return CG_OK;
}

int cg_blob_read(const cg_blob *b, uint64_t offset, uint64_t nbytes, void *host_dst)
{
    g_error.clear();
    if (!b || b->magic != kBlobMagic) return fail(CG_E_INVAL, "invalid cg_blob handle");
    if (!host_dst && nbytes) return fail(CG_E_INVAL, "null argument");
    if (offset > b->hdr.total_bytes || nbytes > b->hdr.total_bytes - offset)
        return fail(CG_E_INVAL, "range outside the container");
    if (!nbytes) return CG_OK;
    DeviceScope ds;
    CG_HIP(ds.enter(b->device), "hipSetDevice");
    CG_HIP(hipMemcpy(host_dst, b->d_data + offset, nbytes, hipMemcpyDeviceToHost), "copy container");
    return CG_OK;
}

void cg_free(void *handle)
{
    if (!handle) return;
    uint32_t magic;
    std::memcpy(&magic, handle, sizeof magic);
    if (magic == kTablesMagic) {
        cg_tables *t = static_cast<cg_tables *>(handle);
        t->magic = 0;
        void *ptrs[] = {t->d_bins, t->d_lo, t->d_w, t->d_r, t->d_freqs, t->d_dtab, t->d_sinks,
                        t->d_alo, t->d_aw, t->d_ar};
        for (void *p : ptrs)
            if (p) (void)hipFree(p);
        delete t;
    } else if (magic == kBlobMagic) {
        cg_blob *b = static_cast<cg_blob *>(handle);
        b->magic = 0;
        if (b->d_data) (void)hipFree(b->d_data);
        delete b;
    }
}

}  // extern "C"

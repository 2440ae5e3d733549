// cg_api.cpp -- host side of libcg: validation, handle ownership, allocation and the
// launch sequence of every entry point declared in include/cg.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "cg.h"
#include "cg_internal.h"

using namespace cgk;

namespace {

constexpr uint32_t kTablesMagic = 0x54424743u;  // "CGBT" (live handle)
constexpr uint32_t kBlobMagic = 0x42424743u;    // "CGBB" (live handle)
constexpr uint64_t kHeaderBytes = sizeof(cg_container_header);
constexpr uint32_t kMaxOutlierPpm = 250000;
static_assert(sizeof(cg_container_header) == 160, "container header is 160 bytes");
static_assert(sizeof(cg_tables_header) == 56, "tables header is 56 bytes");

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

// The shape limits of include/cg.h; returns an error text or nullptr.
const char *shape_error(uint32_t L, uint32_t H, uint32_t d, uint32_t S, uint32_t G, uint32_t Tc)
{
    if (!L || !H || !d || !S || !G || !Tc) return "zero dimension";
    if (Tc > CG_MAX_CHUNK) return "chunk > 16384";
    const uint64_t C = (uint64_t)H * d;
    if (C % 8 != 0) return "H_kv * d must be a multiple of 8";
    // 32-bit offsets inside one (layer, K/V) row of symbols and inside one chunk's rows
    if (C >= (1u << 24) || S >= (1u << 31) || (uint64_t)L * 2 * C >= (1ull << 31) ||
        (uint64_t)L * 2 * S * C >= (1ull << 40) || (uint64_t)S * C >= (1ull << 32) ||
        (uint64_t)Tc * C * 2 >= (1ull << 32))
        return "cache too large";
    return nullptr;
}

// Scratch kept between calls, one area per device (grown when a call needs more).
// Calls that use it hold the lock from their first launch to their last wait, so a
// kernel never runs on an area another call is about to replace.
struct Arena {
    int device;
    void *p;
    uint64_t bytes;
    uint64_t *host;   // 256 pinned host bytes: values a call reads back, a header it writes
};
std::mutex g_arena_mu;
std::vector<Arena> g_arenas;

// Scratch of at least `bytes` on `device`, and the device's pinned read-back words (the
// caller holds g_arena_mu).
hipError_t arena_get(int device, uint64_t bytes, uint8_t **out, uint64_t **host = nullptr)
{
    Arena *a = nullptr;
    for (Arena &x : g_arenas)
        if (x.device == device) a = &x;
    if (!a) {
        g_arenas.push_back(Arena{device, nullptr, 0, nullptr});
        a = &g_arenas.back();
    }
    if (!a->host) {
        void *h = nullptr;
        hipError_t e = hipHostMalloc(&h, 256, hipHostMallocDefault);
        if (e != hipSuccess) return e;
        a->host = static_cast<uint64_t *>(h);
    }
    if (a->bytes < bytes) {
        if (a->p) {
            hipError_t e = hipFree(a->p);
            a->p = nullptr;
            a->bytes = 0;
            if (e != hipSuccess) return e;
        }
        const uint64_t want = (bytes + (bytes >> 4) + 0xFFFFF) & ~uint64_t(0xFFFFF);  // +1/16
        hipError_t e = hipMalloc(&a->p, want);
        if (e != hipSuccess) {
            a->p = nullptr;
            return e;
        }
        a->bytes = want;
    }
    *out = static_cast<uint8_t *>(a->p);
    if (host) *host = a->host;
    return hipSuccess;
}

// Consecutive 256-byte aligned pieces of one scratch area.
struct Carve {
    uint64_t used = 0;
    uint64_t take(uint64_t bytes)
    {
        const uint64_t at = used;
        used += (bytes + 255) & ~uint64_t(255);
        return at;
    }
};

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
    uint32_t anchor_bits;         // 16 or 8
    uint32_t outlier_ppm;
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

// Tokens per thread for the streaming kernels: about two million threads in flight.
uint32_t pick_tpt(const cg_tables *t, uint64_t tokens)
{
    uint64_t work = (uint64_t)t->L * 2 * tokens * (t->C / 8);
    uint64_t tpt = (work + (1u << 21) - 1) >> 21;
    if (tpt < 8) tpt = 8;
    if (tpt > 4096) tpt = 4096;
    return (uint32_t)tpt;
}

// Sink tokens stored in a container of chunks [kb, ke): tokens kb * Tc .. + count.
uint32_t sinks_in(const cg_tables *t, uint32_t kb, uint32_t ke)
{
    const uint64_t a = (uint64_t)kb * t->Tc;
    const uint64_t b = std::min<uint64_t>(std::min<uint64_t>((uint64_t)ke * t->Tc, t->S), t->n_sink);
    return b > a ? (uint32_t)(b - a) : 0u;
}

// Anchor rows of chunks [kb, ke) in closed form: only the cache's last chunk is short.
uint64_t anchor_rows(uint32_t L, uint32_t S, uint32_t G, uint32_t Tc, uint32_t kb, uint32_t ke)
{
    const uint32_t nk = ceil_div(S, Tc);
    const uint32_t last = S - (nk - 1) * Tc;
    uint64_t per_chunk = ceil_div(Tc, G);
    uint64_t rows = (uint64_t)(ke - kb) * per_chunk;
    if (ke == nk && last != Tc) rows = rows - per_chunk + ceil_div(last, G);
    return rows * L * 2;
}

// Every section offset of a container header from its shape, chunk range, anchor width,
// sink count, outlier setting and entry count, and payload size (include/cg.h layout).
void fill_layout(cg_container_header &h)
{
    const uint64_t C = (uint64_t)h.H_kv * h.d;
    h.n_blocks = (uint32_t)((C + kLanes - 1) / kLanes);
    h.n_groups = (uint64_t)(h.chunk_end - h.chunk_begin) * h.L * 2 * h.n_blocks;
    h.offsets_offset = align256(kHeaderBytes);
    h.anchors_offset = align256(h.offsets_offset + (h.n_groups + 1) * 8);
    h.anchors_bytes = anchor_rows(h.L, h.S, h.group, h.chunk, h.chunk_begin, h.chunk_end) * C *
                      (h.anchor_bits == 8 ? 1u : 2u);
    h.sinks_offset = align256(h.anchors_offset + h.anchors_bytes);
    uint64_t end = h.sinks_offset + (uint64_t)2 * h.L * h.n_sink * C * 2;
    h.outliers_offset = align256(end);
    if (h.outlier_ppm) {
        h.outlier_keys_offset = align256(h.outliers_offset + (h.n_groups + 1) * 8);
        h.outlier_values_offset = align256(h.outlier_keys_offset + h.n_outliers * 4);
        end = h.outlier_values_offset + h.n_outliers * 2;
    } else {
        h.outlier_keys_offset = h.outlier_values_offset = h.outliers_offset;
    }
    h.payload_offset = align256(end);
    h.total_bytes = h.payload_offset + h.payload_words * 2 + kPayloadPadBytes;
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
        h.chunk != t->Tc || h.anchor_bits != t->anchor_bits || h.outlier_ppm != t->outlier_ppm ||
        h.n_sink != sinks_in(t, h.chunk_begin, h.chunk_end))
        return fail(CG_E_CORRUPT, "container and tables describe different caches or settings");
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
    v.sinks_off = b->hdr.sinks_offset;
    v.n_sink = b->hdr.n_sink;
    v.out_off = b->hdr.outliers_offset;
    v.keys_off = b->hdr.outlier_keys_offset;
    v.vals_off = b->hdr.outlier_values_offset;
    v.n_out = b->hdr.n_outliers;
    v.outliers = b->hdr.outlier_ppm != 0;
    return v;
}

// After the decoded rows: the container's sink rows, then its outlier entries (unless the
// value decode wrote them: values_decode).
hipError_t put_extras(const cg_tables *t, const cg_blob *b, const uint8_t *cont, uint16_t *out,
                      const Paged &pg, hipStream_t st, bool values_decode = false)
{
    const Geom g = make_geom(t, b->hdr.chunk_begin, b->hdr.chunk_end);
    const ContainerView cv = view_of(b);
    hipError_t e = launch_sinks(g, reinterpret_cast<const uint16_t *>(cont + cv.sinks_off), cv.n_sink,
                                b->hdr.chunk_begin * t->Tc, out, pg, st);
    if (e != hipSuccess || (values_decode && outliers_with_rows(cv))) return e;
    return launch_apply_outliers(g, cont, cv, out, pg, st);
}

// Frees a half-built handle on every error path.
struct TablesOwner {
    cg_tables *t;
    ~TablesOwner();
};

// A tables handle with its shape set and its device arrays allocated (decode tables
// zeroed), or an error.  `bins` holds the level count of every (layer, K/V) row.
int new_tables(uint32_t L, uint32_t H, uint32_t d, uint32_t S, uint32_t G, uint32_t Tc,
               const std::vector<uint8_t> &bins, uint32_t n_sink, uint32_t anchor_bits,
               uint32_t ppm, hipStream_t st, cg_tables **out)
{
    cg_tables *t = new (std::nothrow) cg_tables();
    if (!t) return fail(CG_E_NOMEM, "host allocation");
    t->magic = kTablesMagic;  // cg_free may release it from here on
    TablesOwner owner{t};
    CG_HIP(hipGetDevice(&t->device), "hipGetDevice");
    t->L = L;
    t->H = H;
    t->d = d;
    t->S = S;
    t->G = G;
    t->Tc = Tc;
    t->C = H * d;
    t->NB = ceil_div(t->C, kLanes);
    t->bins = bins;
    t->max_bins = 0;
    for (uint8_t n : bins) t->max_bins = std::max<uint32_t>(t->max_bins, n);
    t->n_sink = std::min(n_sink, S);
    t->anchor_bits = anchor_bits == 8 ? 8u : 16u;
    t->outlier_ppm = ppm;
    const uint64_t rows = (uint64_t)t->L * 2 * t->C;
    DevBuf bins_d, lo_d, w_d, r_d, fr_d, dt_d;
    CG_HIP(bins_d.alloc((uint64_t)2 * t->L), "hipMalloc");
    CG_HIP(lo_d.alloc(rows * 4), "hipMalloc");
    CG_HIP(w_d.alloc(rows * 4), "hipMalloc");
    CG_HIP(r_d.alloc(rows * 4), "hipMalloc");
    CG_HIP(fr_d.alloc(rows * kMaxBins * 2), "hipMalloc");
    const uint64_t dtab_bytes = (uint64_t)t->L * 2 * t->NB * kTabBlock * sizeof(uint32_t);
    CG_HIP(dt_d.alloc(dtab_bytes), "hipMalloc");
    if (t->anchor_bits == 8) {
        DevBuf alo_d, aw_d, ar_d;
        CG_HIP(alo_d.alloc(rows * 4), "hipMalloc");
        CG_HIP(aw_d.alloc(rows * 4), "hipMalloc");
        CG_HIP(ar_d.alloc(rows * 4), "hipMalloc");
        t->d_alo = static_cast<float *>(alo_d.detach());
        t->d_aw = static_cast<float *>(aw_d.detach());
        t->d_ar = static_cast<float *>(ar_d.detach());
    }
    t->d_bins = static_cast<uint8_t *>(bins_d.detach());
    t->d_lo = static_cast<float *>(lo_d.detach());
    t->d_w = static_cast<float *>(w_d.detach());
    t->d_r = static_cast<float *>(r_d.detach());
    t->d_freqs = static_cast<uint16_t *>(fr_d.detach());
    t->d_dtab = static_cast<uint32_t *>(dt_d.detach());
    CG_HIP(hipMemcpyAsync(t->d_bins, t->bins.data(), (size_t)2 * t->L, hipMemcpyHostToDevice, st),
           "copy bins");
    CG_HIP(hipMemsetAsync(t->d_freqs, 0, rows * kMaxBins * 2, st), "memset");
    CG_HIP(hipMemsetAsync(t->d_dtab, 0, dtab_bytes, st), "memset");
    owner.t = nullptr;
    *out = t;
    return CG_OK;
}

// Size of the stored tables.
uint64_t tables_stored_bytes(const cg_tables *t)
{
    const uint64_t rows = (uint64_t)t->L * 2 * t->C;
    uint64_t bytes = sizeof(cg_tables_header) + (((uint64_t)2 * t->L + 3) & ~uint64_t(3));
    bytes += rows * 8 * (t->anchor_bits == 8 ? 2 : 1);
    for (uint32_t r = 0; r < 2 * t->L; ++r) bytes += (uint64_t)t->C * t->bins[r] * 2;
    return bytes;
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
    if (const char *err = shape_error(p.L, p.H_kv, p.d, p.S, p.group, p.chunk))
        return fail(CG_E_INVAL, err);
    if (p.anchor_bits != 0 && p.anchor_bits != 8 && p.anchor_bits != 16)
        return fail(CG_E_INVAL, "anchor_bits must be 0, 8 or 16");
    if (p.outlier_ppm > kMaxOutlierPpm) return fail(CG_E_INVAL, "outlier_ppm > 250000");
    std::vector<uint8_t> bins((size_t)2 * p.L);  // per (layer, K/V) row: l * 2 + kv
    for (uint32_t l = 0; l < p.L; ++l)
        for (uint32_t kv = 0; kv < 2; ++kv) {
            const uint8_t n = (kv && p.bins_v) ? p.bins_v[l] : p.bins[l];
            if (n < 2 || n > CG_MAX_BINS) return fail(CG_E_INVAL, "bins outside [2, 32]");
            bins[2 * l + kv] = n;
        }
    hipStream_t st = (hipStream_t)hip_stream;
    cg_tables *t = nullptr;
    if (int rc = new_tables(p.L, p.H_kv, p.d, p.S, p.group, p.chunk, bins, p.n_sink,
                            p.anchor_bits, p.outlier_ppm, st, &t))
        return rc;
    TablesOwner owner{t};

    const uint64_t rows = (uint64_t)t->L * 2 * t->C;
    Carve cv;
    const uint64_t o_lo = cv.take(rows * 4), o_hi = cv.take(rows * 4), o_h = cv.take(rows * 4);
    const uint64_t o_cnt = cv.take(rows * kMaxBins * 4), o_flag = cv.take(4);
    const uint64_t o_fine = t->outlier_ppm
                                ? cv.take((uint64_t)fine_parts(make_geom(t, 0, 1)) * rows * kFineBins * 2)
                                : 0;
    std::lock_guard<std::mutex> lock(g_arena_mu);
    uint8_t *sc = nullptr;
    uint64_t *hw = nullptr;
    CG_HIP(arena_get(t->device, cv.used, &sc, &hw), "scratch");
    uint32_t *ordlo = reinterpret_cast<uint32_t *>(sc + o_lo), *ordhi = reinterpret_cast<uint32_t *>(sc + o_hi);
    float *hi = reinterpret_cast<float *>(sc + o_h);
    uint32_t *counts = reinterpret_cast<uint32_t *>(sc + o_cnt), *flag = reinterpret_cast<uint32_t *>(sc + o_flag);
    uint16_t *fine = reinterpret_cast<uint16_t *>(sc + o_fine);
    CG_HIP(hipMemsetAsync(ordlo, 0xFF, rows * 4, st), "memset");
    CG_HIP(hipMemsetAsync(ordhi, 0x00, rows * 4, st), "memset");
    CG_HIP(hipMemsetAsync(counts, 0, rows * kMaxBins * 4, st), "memset");
    CG_HIP(hipMemsetAsync(flag, 0, 4, st), "memset");

    const uint16_t *X = static_cast<const uint16_t *>(kv_dev);
    Geom g = make_geom(t, 0, ceil_div(t->S, t->Tc));
    if (t->d_alo)
        CG_HIP(launch_anchor_grid(X, g, t->d_alo, t->d_aw, t->d_ar, st), "k_anchor_grid");
    CG_HIP(launch_k0(X, g, pick_tpt(t, t->S), ordlo, ordhi, flag, st), "k0_minmax");
    CG_HIP(launch_k0_finalize(g, ordlo, ordhi, t->d_lo, hi, st), "k0_finalize");
    if (t->outlier_ppm) {
        CG_HIP(launch_fine_hist(X, g, t->d_lo, hi, fine, st), "k_fine_hist");
        CG_HIP(launch_clip(g, fine, t->outlier_ppm, t->d_lo, hi, st), "k_clip");
    }
    CG_HIP(launch_width(g, t->d_bins, t->d_lo, hi, t->d_w, t->d_r, st), "k_width");
    CG_HIP(launch_k1(X, g, t->d_bins, t->max_bins, t->d_lo, t->d_r, counts, st), "k1_hist");
    CG_HIP(launch_k1_freqs(g, t->d_bins, counts, t->d_freqs, st), "k1_freqs");
    CG_HIP(launch_dtab(g, t->d_bins, t->d_freqs, t->d_lo, t->d_w, t->d_dtab, st), "k_dtab");
    CG_HIP(hipMemcpyAsync(hw, flag, 4, hipMemcpyDeviceToHost, st), "copy flag");
    CG_HIP(hipStreamSynchronize(st), "hipStreamSynchronize");
    if (*reinterpret_cast<volatile uint32_t *>(hw)) return fail(CG_E_NONFINITE, "KV input holds Inf or NaN");
    owner.t = nullptr;
    *out = t;
    return CG_OK;
}

}  // extern "C"

namespace {

// Scratch of an encode of chunks [kb, ke): the groups' word regions, the anchors section,
// per-group word and off-grid counts and their scans.
struct EncPlan {
    uint64_t n_groups, region_words, anchor_bytes;
    uint64_t o_reg, o_anc, o_gw, o_go, o_ow, o_oo, bytes;
};

EncPlan enc_plan(const cg_tables *t, uint32_t kb, uint32_t ke)
{
    EncPlan p;
    const Geom g = make_geom(t, kb, ke);
    p.n_groups = (uint64_t)(ke - kb) * t->L * 2 * t->NB;
    p.region_words = code_region_words(g);
    p.anchor_bytes = anchor_rows(t->L, t->S, t->G, t->Tc, kb, ke) * t->C * (t->anchor_bits == 8 ? 1u : 2u);
    Carve cv;
    p.o_reg = cv.take(p.n_groups * p.region_words * 2);
    p.o_anc = cv.take(p.anchor_bytes);
    p.o_gw = cv.take(p.n_groups * 8);
    p.o_go = cv.take((p.n_groups + 1) * 8);
    p.o_ow = cv.take(p.n_groups * 8);
    p.o_oo = cv.take((p.n_groups + 1) * 8);
    p.bytes = cv.used;
    return p;
}

// The coding pass and the scans; back on the host (after a wait): the payload words and
// the elements off their grid.  `rb` receives them (pinned memory, or a host variable).
hipError_t enc_code(const cg_tables *t, const uint16_t *X, uint32_t kb, uint32_t ke, uint8_t *sc,
                    const EncPlan &p, hipStream_t st, uint64_t *rb, const char **what)
{
    const Geom g = make_geom(t, kb, ke);
    uint64_t *gw = reinterpret_cast<uint64_t *>(sc + p.o_gw), *go = reinterpret_cast<uint64_t *>(sc + p.o_go);
    uint64_t *ow = reinterpret_cast<uint64_t *>(sc + p.o_ow), *oo = reinterpret_cast<uint64_t *>(sc + p.o_oo);
    hipError_t e;
    *what = "k5_code";
    if ((e = launch_k5_code(X, g, t->d_bins, t->d_dtab, t->d_lo, t->d_r,
                            reinterpret_cast<uint16_t *>(sc + p.o_reg), sc + p.o_anc, gw, ow, st)) != hipSuccess)
        return e;
    *what = "scan";
    if ((e = launch_scan(gw, go, p.n_groups, st)) != hipSuccess) return e;
    if ((e = launch_scan(ow, oo, p.n_groups, st)) != hipSuccess) return e;
    *what = "read back sizes";
    if ((e = hipMemcpyAsync(rb, go + p.n_groups, 8, hipMemcpyDeviceToHost, st)) != hipSuccess) return e;
    if ((e = hipMemcpyAsync(rb + 1, oo + p.n_groups, 8, hipMemcpyDeviceToHost, st)) != hipSuccess) return e;
    return hipStreamSynchronize(st);
}

cg_container_header enc_header(const cg_tables *t, uint32_t kb, uint32_t ke, uint64_t words, uint64_t n_off)
{
    cg_container_header h;
    std::memset(&h, 0, sizeof h);
    h.magic = CG_CONTAINER_MAGIC;
    h.version = CG_CONTAINER_VERSION;
    h.L = t->L;
    h.H_kv = t->H;
    h.d = t->d;
    h.S = t->S;
    h.group = t->G;
    h.chunk = t->Tc;
    h.chunk_begin = kb;
    h.chunk_end = ke;
    h.anchor_bits = t->anchor_bits;
    h.n_sink = sinks_in(t, kb, ke);
    h.outlier_ppm = t->outlier_ppm;
    h.n_outliers = t->outlier_ppm ? n_off : 0;
    h.clamped = t->outlier_ppm ? 0 : n_off;
    h.payload_words = words;
    fill_layout(h);
    return h;
}

// Writes the container described by h at `base` (device, h.total_bytes): padding, the
// header (copied from `hsrc`, which must stay valid until the stream has run), offsets,
// anchors, sink rows, outlier sections and the packed payload.  Asynchronous.
hipError_t enc_write(const cg_tables *t, const uint16_t *X, uint32_t kb, uint32_t ke, uint8_t *sc,
                     const EncPlan &p, const cg_container_header &h, const void *hsrc, uint8_t *base,
                     hipStream_t st, const char **what)
{
    const Geom g = make_geom(t, kb, ke);
    const uint64_t C = t->C, ng = p.n_groups;
    uint64_t *gw = reinterpret_cast<uint64_t *>(sc + p.o_gw), *go = reinterpret_cast<uint64_t *>(sc + p.o_go);
    uint64_t *oo = reinterpret_cast<uint64_t *>(sc + p.o_oo);
    // zero bytes between sections and after the payload
    const uint64_t ends[][2] = {
        {kHeaderBytes, h.offsets_offset},
        {h.offsets_offset + (ng + 1) * 8, h.anchors_offset},
        {h.anchors_offset + h.anchors_bytes, h.sinks_offset},
        {h.sinks_offset + (uint64_t)2 * t->L * h.n_sink * C * 2, h.outliers_offset},
        {h.outlier_ppm ? h.outliers_offset + (ng + 1) * 8 : h.outliers_offset, h.outlier_keys_offset},
        {h.outlier_keys_offset + h.n_outliers * 4, h.outlier_values_offset},
        {h.outlier_values_offset + (h.outlier_ppm ? h.n_outliers * 2 : 0), h.payload_offset},
        {h.payload_offset + h.payload_words * 2, h.total_bytes}};
    ZeroRanges zr;
    zr.n = 0;
    for (const auto &z : ends)
        if (z[1] > z[0]) {
            zr.r[zr.n][0] = z[0];
            zr.r[zr.n][1] = z[1];
            ++zr.n;
        }
    hipError_t e;
    *what = "clear padding";
    if ((e = launch_zero_ranges(base, zr, st)) != hipSuccess) return e;
    *what = "copy header";
    if ((e = hipMemcpyAsync(base, hsrc, sizeof h, hipMemcpyHostToDevice, st)) != hipSuccess) return e;
    *what = "copy offsets";
    if ((e = hipMemcpyAsync(base + h.offsets_offset, go, (ng + 1) * 8, hipMemcpyDeviceToDevice, st)) != hipSuccess)
        return e;
    *what = "copy anchors";
    if ((e = hipMemcpyAsync(base + h.anchors_offset, sc + p.o_anc, h.anchors_bytes, hipMemcpyDeviceToDevice,
                            st)) != hipSuccess)
        return e;
    if (h.n_sink) {
        // the sink rows of the encoded cache: 2L rows of n_sink tokens from the first token
        const uint64_t w = (uint64_t)h.n_sink * C * 2;
        *what = "copy sink rows";
        if ((e = hipMemcpy2DAsync(base + h.sinks_offset, w, X + (uint64_t)kb * t->Tc * C,
                                  (uint64_t)t->S * C * 2, w, 2 * t->L, hipMemcpyDeviceToDevice, st)) != hipSuccess)
            return e;
    }
    if (t->outlier_ppm) {
        *what = "copy outlier offsets";
        if ((e = hipMemcpyAsync(base + h.outliers_offset, oo, (ng + 1) * 8, hipMemcpyDeviceToDevice, st)) !=
            hipSuccess)
            return e;
        *what = "k_outliers";
        if (h.n_outliers &&
            (e = launch_outliers(X, g, t->d_bins, t->d_lo, t->d_r, nullptr, oo,
                                 reinterpret_cast<uint32_t *>(base + h.outlier_keys_offset),
                                 reinterpret_cast<uint16_t *>(base + h.outlier_values_offset), st)) != hipSuccess)
            return e;
    }
    *what = "k5_compact";
    return launch_k5_compact(reinterpret_cast<const uint16_t *>(sc + p.o_reg), p.region_words, gw, go, ng,
                             reinterpret_cast<uint16_t *>(base + h.payload_offset), st);
}

// Scratch for cg_encode_noalloc: a fixed array in each device's memory, its address
// looked up once per device.  Calls hold g_static_mu from the first launch to the last
// wait, so calls do not overlap on it.
constexpr uint64_t kStaticScratch = 64ull << 20;
constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
uint8_t *g_static_ptr[kMaxDevices];

}  // namespace

static __device__ __align__(256) uint8_t scratch[kStaticScratch];

namespace {
hipError_t static_scratch(int device, uint8_t **out)
{
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    if (!g_static_ptr[device]) {
        void *p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_static_ptr[device] = static_cast<uint8_t *>(p);
    }
    *out = g_static_ptr[device];
    return hipSuccess;
}
}  // namespace

extern "C" {

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
    const uint16_t *X = static_cast<const uint16_t *>(kv_dev);
    const EncPlan p = enc_plan(t, kb, ke);
    std::lock_guard<std::mutex> lock(g_arena_mu);
    uint8_t *sc = nullptr;
    uint64_t *hw = nullptr;
    CG_HIP(arena_get(t->device, p.bytes, &sc, &hw), "scratch");
    const char *what = "";
    hipError_t e = enc_code(t, X, kb, ke, sc, p, st, hw, &what);
    if (e != hipSuccess) return hip_fail(e, what);
    const cg_container_header h = enc_header(t, kb, ke, hw[0], hw[1]);

    cg_blob *b = new (std::nothrow) cg_blob();
    if (!b) return fail(CG_E_NOMEM, "host allocation");
    b->magic = 0;
    b->device = t->device;
    b->hdr = h;
    DevBuf data;
    e = data.alloc(align256(h.total_bytes));
    if (e != hipSuccess) {
        delete b;
        return hip_fail(e, "hipMalloc container");
    }
    std::memcpy(hw + 8, &h, sizeof h);  // staged in pinned memory (waited for below)
    e = enc_write(t, X, kb, ke, sc, p, h, hw + 8, data.as<uint8_t>(), st, &what);
    if (e == hipSuccess) {
        what = "hipStreamSynchronize";
        e = hipStreamSynchronize(st);
    }
    if (e != hipSuccess) {
        delete b;
        return hip_fail(e, what);
    }
    b->d_data = static_cast<uint8_t *>(data.detach());
    b->magic = kBlobMagic;
    *out = b;
    return CG_OK;
}

int cg_encode_noalloc(const cg_tables *t, const void *kv_dev, uint32_t kb, uint32_t ke,
                      void *container_dev, uint64_t capacity, void *hip_stream,
                      cg_container_header *header_out)
{
    g_error.clear();
    if (int rc = check_tables(t)) return rc;
    if (!kv_dev || !container_dev || !header_out) return fail(CG_E_INVAL, "null argument");
    if (reinterpret_cast<uintptr_t>(container_dev) % 256 != 0)
        return fail(CG_E_INVAL, "container buffer must be 256-byte aligned");
    const uint32_t nchunks = ceil_div(t->S, t->Tc);
    if (kb >= ke || ke > nchunks) return fail(CG_E_INVAL, "chunk range out of bounds");
    const EncPlan p = enc_plan(t, kb, ke);
    if (p.bytes > kStaticScratch)
        return fail(CG_E_INVAL, "encode needs " + std::to_string(p.bytes) +
                                    " bytes of scratch, more than the 64 MiB of cg_encode_noalloc");
    DeviceScope ds;
    CG_HIP(ds.enter(t->device), "hipSetDevice");
    hipStream_t st = (hipStream_t)hip_stream;
    const uint16_t *X = static_cast<const uint16_t *>(kv_dev);
    std::lock_guard<std::mutex> lock(g_static_mu);
    uint8_t *sc = nullptr;
    CG_HIP(static_scratch(t->device, &sc), "hipGetSymbolAddress");
    uint64_t rb[2] = {0, 0};
    const char *what = "";
    hipError_t e = enc_code(t, X, kb, ke, sc, p, st, rb, &what);
    if (e != hipSuccess) return hip_fail(e, what);
    const cg_container_header h = enc_header(t, kb, ke, rb[0], rb[1]);
    *header_out = h;
    if (h.total_bytes > capacity)
        return fail(CG_E_INVAL, "container needs " + std::to_string(h.total_bytes) +
                                    " bytes, more than the capacity given (header_out holds its size)");
    e = enc_write(t, X, kb, ke, sc, p, h, &h, static_cast<uint8_t *>(container_dev), st, &what);
    if (e == hipSuccess) {
        what = "hipStreamSynchronize";
        e = hipStreamSynchronize(st);  // (the header is copied from this frame)
    }
    if (e != hipSuccess) return hip_fail(e, what);
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
    // (the decoder sends the rows of a skipped block to the page after the pool)
    if ((uint64_t)(num_pages + 1ull) * page_tokens * t->C * 2 > (1ull << 32))
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
    CG_HIP(put_extras(t, b, cont, nullptr, pg, (hipStream_t)hip_stream, true),
           "sinks / outliers (paged)");
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
    uint16_t *out = static_cast<uint16_t *>(kv_out_dev);
    CG_HIP(launch_k3(g, t->d_bins, t->d_dtab, t->d_lo, t->d_w, cont, view_of(b), out, nullptr,
                     (hipStream_t)hip_stream),
           "k3_decode");
    CG_HIP(put_extras(t, b, cont, out, Paged{}, (hipStream_t)hip_stream, true), "sinks / outliers");
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

// Decodes every chunk of items[0 .. n) (container i staged at slot[i]) with as few
// multi-container launches as the launch limits allow: the chunks are grouped by their
// tables (first appearance order), each group cut into sets of up to 8 chunks, and the
// sets packed into launches of up to kMaxBatch chunks and kMaxBatchTables tables, with
// fp16 and 8-bit anchors in launches of their own.
hipError_t decode_window(const cg_stream_item *items, uint32_t n, uint8_t *const *slot,
                         uint16_t *out, hipStream_t st)
{
    const Geom g = make_geom(items[0].tables, 0, 1);
    std::vector<const cg_tables *> order;
    for (uint32_t i = 0; i < n; ++i)
        if (std::find(order.begin(), order.end(), items[i].tables) == order.end())
            order.push_back(items[i].tables);
    for (int a8 = 0; a8 < 2; ++a8) {
        ChunkSrcs srcs{};
        uint32_t n_ch = 0, n_tab = 0;
        auto flush = [&]() -> hipError_t {
            hipError_t e = launch_k3_multi(g, srcs, out, st);
            srcs = ChunkSrcs{};
            n_ch = n_tab = 0;
            return e;
        };
        for (const cg_tables *t : order) {
            if ((t->d_alo != nullptr) != (a8 == 1)) continue;
            // this group's chunks in item order
            std::vector<BatchChunk> chunks;
            for (uint32_t i = 0; i < n; ++i) {
                if (items[i].tables != t) continue;
                const cg_blob *b = items[i].blob;
                const ContainerView cv = view_of(b);
                for (uint32_t k = b->hdr.chunk_begin; k < b->hdr.chunk_end; ++k)
                    chunks.push_back(BatchChunk{slot[i], cv.offsets_off, cv.anchors_off,
                                                cv.anchors_bytes, cv.payload_off,
                                                cv.payload_words, k, b->hdr.chunk_begin});
            }
            for (size_t c0 = 0; c0 < chunks.size();) {
                const uint32_t m =
                    (uint32_t)std::min<size_t>(kBatchSetChunks, chunks.size() - c0);
                if (n_ch + m > kMaxBatch || srcs.n_sets == kMaxBatch ||
                    (n_tab == kMaxBatchTables && !(srcs.tab[n_tab - 1].dtab == t->d_dtab))) {
                    if (hipError_t e = flush()) return e;
                }
                if (n_tab == 0 || srcs.tab[n_tab - 1].dtab != t->d_dtab)
                    srcs.tab[n_tab++] = BatchTables{t->d_bins, t->d_dtab, t->d_lo, t->d_w,
                                                    t->d_alo, t->d_aw};
                const uint32_t j = srcs.n_sets++;
                srcs.set_first[j] = (uint8_t)n_ch;
                srcs.set_n[j] = (uint8_t)m;
                srcs.set_tab[j] = (uint8_t)(n_tab - 1);
                for (uint32_t q = 0; q < m; ++q) srcs.ch[n_ch++] = chunks[c0 + q];
                c0 += m;
            }
        }
        if (srcs.n_sets)
            if (hipError_t e = flush()) return e;
    }
    return hipSuccess;
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

    // Items are decoded in windows of up to `batch` (half the slots, at most 32): the
    // window's copies go out back to back, and once the last has landed a multi-container
    // decode takes every chunk of the window, whatever its tables (a lone chunk per launch
    // fills too little of the GPU, and a launch per level leaves it idle between
    // launches).  Meanwhile the next window copies into other slots.  The last windows
    // shrink (batch / 2, batch / 4, batch / 8 items, at least 1) so that little decoding
    // is left once the last copy has landed; the first window takes what does not divide.
    // Per window: copied (its decode may start) and decoded (its slots may be refilled);
    // with stats, per item: copy start/end, and per window: decode start/end.
    const uint32_t batch = std::min(kMaxBatch, n_slots > 1 ? n_slots / 2 : 1u);
    std::vector<uint32_t> wbeg;   // window starts, then n_items
    {
        std::vector<uint32_t> sizes;   // from the last window back
        uint32_t left = n_items, m = std::max(1u, batch / 8);
        while (left) {
            sizes.push_back(std::min(left, m));
            left -= sizes.back();
            m = std::min(batch, 2 * m);
        }
        wbeg.push_back(0);
        for (size_t j = sizes.size(); j-- > 0;) wbeg.push_back(wbeg.back() + sizes[j]);
    }
    const uint32_t n_windows = (uint32_t)wbeg.size() - 1;
    std::vector<uint32_t> win_of(n_items);
    for (uint32_t wi = 0; wi < n_windows; ++wi)
        for (uint32_t i = wbeg[wi]; i < wbeg[wi + 1]; ++i) win_of[i] = wi;
    EventSet slot_ev, item_ev, win_ev;
    CG_HIP(slot_ev.make(2 * (size_t)n_windows, false), "hipEventCreate");
    if (stats) {
        CG_HIP(item_ev.make(2 * (size_t)n_items, true), "hipEventCreate");
        CG_HIP(win_ev.make(2 * (size_t)n_windows, true), "hipEventCreate");
    }
    hipEvent_t *copied = slot_ev.ev.data(), *decoded = copied + n_windows;

    hipError_t err = hipSuccess;
    const char *what = "";
    uint64_t bytes = 0;
    uint16_t *out = static_cast<uint16_t *>(kv_out_dev);
    auto slot_of = [&](uint32_t i) {
        return static_cast<uint8_t *>(staging_dev) + (uint64_t)(i % n_slots) * slot_bytes;
    };
    uint32_t waited = 0;   // windows [0, waited) known decoded on the copy stream
    for (uint32_t wi = 0; wi < n_windows && err == hipSuccess; ++wi) {
        const uint32_t ib = wbeg[wi], ie_ = wbeg[wi + 1];
        for (uint32_t i = ib; i < ie_; ++i) {
            const cg_stream_item &it = items[i];
            hipEvent_t *ie = stats ? item_ev.ev.data() + 2 * (size_t)i : nullptr;
            // slot reuse: item i - n_slots, which held this slot, must have been decoded.
            // Its window is an earlier one (windows hold at most n_slots / 2 items),
            // already queued; one wait per window, as a wait per copy leaves the copy
            // engine idle between copies.
            if (i >= n_slots && win_of[i - n_slots] >= waited) {
                const uint32_t w = win_of[i - n_slots];
                if ((err = hipStreamWaitEvent(cs, decoded[w], 0)) != hipSuccess) {
                    what = "hipStreamWaitEvent";
                    break;
                }
                waited = w + 1;
            }
            if (ie && (err = hipEventRecord(ie[0], cs)) != hipSuccess) { what = "hipEventRecord"; break; }
            if ((err = hipMemcpyAsync(slot_of(i), it.host_container, it.blob->hdr.total_bytes,
                                      hipMemcpyHostToDevice, cs)) != hipSuccess) {
                what = "hipMemcpyAsync";
                break;
            }
            if (ie && (err = hipEventRecord(ie[1], cs)) != hipSuccess) { what = "hipEventRecord"; break; }
            bytes += it.blob->hdr.total_bytes;
        }
        if (err != hipSuccess) break;
        if ((err = hipEventRecord(copied[wi], cs)) != hipSuccess ||
            (err = hipStreamWaitEvent(dec, copied[wi], 0)) != hipSuccess) {
            what = "copy -> decode event";
            break;
        }
        hipEvent_t *we = stats ? win_ev.ev.data() + 2 * (size_t)wi : nullptr;
        if (we && (err = hipEventRecord(we[0], dec)) != hipSuccess) { what = "hipEventRecord"; break; }
        std::vector<uint8_t *> slots(ie_ - ib);
        for (uint32_t i = ib; i < ie_; ++i) slots[i - ib] = slot_of(i);
        if ((err = decode_window(items + ib, ie_ - ib, slots.data(), out, dec)) != hipSuccess) {
            what = "k3_decode_multi";
            break;
        }
        // sinks and outliers after the decodes that wrote those rows
        for (uint32_t i = ib; i < ie_ && err == hipSuccess; ++i)
            if ((err = put_extras(items[i].tables, items[i].blob, slot_of(i), out, Paged{}, dec)) !=
                hipSuccess)
                what = "sinks / outliers";
        if (err != hipSuccess) break;
        if (we && (err = hipEventRecord(we[1], dec)) != hipSuccess) { what = "hipEventRecord"; break; }
        if ((err = hipEventRecord(decoded[wi], dec)) != hipSuccess) {
            what = "hipEventRecord";
            break;
        }
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
    const hipEvent_t *ie = item_ev.ev.data(), *we = win_ev.ev.data();
    for (uint32_t i = 0; i < n_items; ++i) {
        float c = 0.f;
        CG_HIP(hipEventElapsedTime(&c, ie[2 * i], ie[2 * i + 1]), "hipEventElapsedTime");
        st.copy_ms += c;
    }
    for (uint32_t wi = 0; wi < n_windows; ++wi) {
        float d = 0.f;
        CG_HIP(hipEventElapsedTime(&d, we[2 * wi], we[2 * wi + 1]), "hipEventElapsedTime");
        st.decode_ms += d;
    }
    CG_HIP(hipEventElapsedTime(&st.total_ms, ie[0], we[2 * ((size_t)n_windows - 1) + 1]),
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
    uint16_t *out = static_cast<uint16_t *>(kv_out_dev);
    CG_HIP(launch_k4(g, t->d_lo, t->d_w, static_cast<const uint8_t *>(sym_dev), cont, view_of(b),
                     t_lo, t_hi, pick_tpt(t, t_hi - t_lo), out, (hipStream_t)hip_stream),
           "k4_dequant");
    CG_HIP(put_extras(t, b, cont, out, Paged{}, (hipStream_t)hip_stream), "sinks / outliers");
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
                     nullptr, nullptr, (hipStream_t)hip_stream),
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
    info->stored_bytes = tables_stored_bytes(t);
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

// ------------------------------------------------------------------------------ stored form
int cg_tables_serialize(const cg_tables *t, void *host_dst, uint64_t capacity, uint64_t *size_out)
{
    g_error.clear();
    if (int rc = check_tables(t)) return rc;
    const uint64_t size = tables_stored_bytes(t);
    if (size_out) *size_out = size;
    if (!host_dst) return size_out ? CG_OK : fail(CG_E_INVAL, "null destination");
    if (capacity < size) return fail(CG_E_INVAL, "destination smaller than the stored tables");
    DeviceScope ds;
    CG_HIP(ds.enter(t->device), "hipSetDevice");
    const uint64_t rows = (uint64_t)t->L * 2 * t->C;
    std::vector<float> lo(rows), w(rows), alo, aw;
    std::vector<uint16_t> fr(rows * kMaxBins);
    CG_HIP(hipMemcpy(lo.data(), t->d_lo, rows * 4, hipMemcpyDeviceToHost), "copy lo");
    CG_HIP(hipMemcpy(w.data(), t->d_w, rows * 4, hipMemcpyDeviceToHost), "copy w");
    CG_HIP(hipMemcpy(fr.data(), t->d_freqs, rows * kMaxBins * 2, hipMemcpyDeviceToHost), "copy freqs");
    if (t->anchor_bits == 8) {
        alo.resize(rows);
        aw.resize(rows);
        CG_HIP(hipMemcpy(alo.data(), t->d_alo, rows * 4, hipMemcpyDeviceToHost), "copy alo");
        CG_HIP(hipMemcpy(aw.data(), t->d_aw, rows * 4, hipMemcpyDeviceToHost), "copy aw");
    }
    uint8_t *p = static_cast<uint8_t *>(host_dst);
    cg_tables_header h;
    std::memset(&h, 0, sizeof h);
    h.magic = CG_TABLES_MAGIC;
    h.version = CG_TABLES_VERSION;
    h.L = t->L;
    h.H_kv = t->H;
    h.d = t->d;
    h.S = t->S;
    h.group = t->G;
    h.chunk = t->Tc;
    h.n_sink = t->n_sink;
    h.anchor_bits = t->anchor_bits;
    h.outlier_ppm = t->outlier_ppm;
    h.total_bytes = size;
    std::memcpy(p, &h, sizeof h);
    p += sizeof h;
    const uint64_t bins_pad = ((uint64_t)2 * t->L + 3) & ~uint64_t(3);
    std::memset(p, 0, bins_pad);
    std::memcpy(p, t->bins.data(), (size_t)2 * t->L);
    p += bins_pad;
    std::memcpy(p, lo.data(), rows * 4);
    p += rows * 4;
    std::memcpy(p, w.data(), rows * 4);
    p += rows * 4;
    if (t->anchor_bits == 8) {
        std::memcpy(p, alo.data(), rows * 4);
        p += rows * 4;
        std::memcpy(p, aw.data(), rows * 4);
        p += rows * 4;
    }
    for (uint64_t i = 0; i < rows; ++i) {
        const uint32_t n = t->bins[i / t->C];
        std::memcpy(p, fr.data() + i * kMaxBins, (size_t)n * 2);
        p += (size_t)n * 2;
    }
    return CG_OK;
}

int cg_tables_check(const void *host_bytes, uint64_t nbytes, cg_tables_header *header_out)
{
    g_error.clear();
    if (!host_bytes) return fail(CG_E_INVAL, "null bytes");
    if (nbytes < sizeof(cg_tables_header)) return fail(CG_E_CORRUPT, "shorter than a tables header");
    cg_tables_header h;
    std::memcpy(&h, host_bytes, sizeof h);
    if (h.magic != CG_TABLES_MAGIC) return fail(CG_E_CORRUPT, "not stored tables (magic)");
    if (h.version != CG_TABLES_VERSION) return fail(CG_E_CORRUPT, "unknown tables version");
    if (const char *err = shape_error(h.L, h.H_kv, h.d, h.S, h.group, h.chunk))
        return fail(CG_E_CORRUPT, std::string("tables shape: ") + err);
    if (h.anchor_bits != 8 && h.anchor_bits != 16) return fail(CG_E_CORRUPT, "anchor_bits");
    if (h.outlier_ppm > kMaxOutlierPpm) return fail(CG_E_CORRUPT, "outlier_ppm");
    if (h.n_sink > h.S) return fail(CG_E_CORRUPT, "n_sink above S");
    const uint64_t C = (uint64_t)h.H_kv * h.d, rows = (uint64_t)h.L * 2 * C;
    const uint64_t bins_pad = ((uint64_t)2 * h.L + 3) & ~uint64_t(3);
    const uint64_t fixed = sizeof h + bins_pad + rows * 8 * (h.anchor_bits == 8 ? 2 : 1);
    if (nbytes < fixed) return fail(CG_E_CORRUPT, "truncated tables");
    const uint8_t *p = static_cast<const uint8_t *>(host_bytes);
    const uint8_t *bins = p + sizeof h;
    uint64_t size = fixed;
    for (uint32_t r = 0; r < 2 * h.L; ++r) {
        if (bins[r] < 2 || bins[r] > CG_MAX_BINS) return fail(CG_E_CORRUPT, "bins outside [2, 32]");
        size += C * bins[r] * 2;
    }
    for (uint64_t j = 2 * h.L; j < bins_pad; ++j)
        if (bins[j]) return fail(CG_E_CORRUPT, "padding after bins is not zero");
    if (h.total_bytes != size || nbytes < size) return fail(CG_E_CORRUPT, "tables size");
    const uint8_t *q = p + sizeof h + bins_pad;
    const uint64_t n_grid = rows * (h.anchor_bits == 8 ? 4 : 2);  // lo, w (, alo, aw)
    for (uint64_t i = 0; i < n_grid; ++i) {
        float v;
        std::memcpy(&v, q + 4 * i, 4);
        const uint64_t which = i / rows;  // 0 lo, 1 w, 2 alo, 3 aw
        if (!std::isfinite(v) || ((which == 1 || which == 3) && !(v >= 0.0f)))
            return fail(CG_E_CORRUPT, "grid values must be finite, widths >= 0");
    }
    const uint8_t *f = q + 4 * n_grid;
    for (uint64_t i = 0; i < rows; ++i) {
        const uint32_t n = bins[i / C];
        uint32_t sum = 0;
        for (uint32_t s = 0; s < n; ++s) {
            uint16_t v;
            std::memcpy(&v, f, 2);
            f += 2;
            if (v == 0) return fail(CG_E_CORRUPT, "a frequency of 0");
            sum += v;
        }
        if (sum != kProbTotal) return fail(CG_E_CORRUPT, "frequencies do not sum to 256");
    }
    if (header_out) *header_out = h;
    return CG_OK;
}

int cg_tables_import(const void *host_bytes, uint64_t nbytes, cg_tables **out)
{
    g_error.clear();
    if (!out) return fail(CG_E_INVAL, "null argument");
    cg_tables_header h;
    if (int rc = cg_tables_check(host_bytes, nbytes, &h)) return rc;
    const uint8_t *p = static_cast<const uint8_t *>(host_bytes);
    std::vector<uint8_t> bins(p + sizeof h, p + sizeof h + (size_t)2 * h.L);
    cg_tables *t = nullptr;
    if (int rc = new_tables(h.L, h.H_kv, h.d, h.S, h.group, h.chunk, bins, h.n_sink, h.anchor_bits,
                            h.outlier_ppm, nullptr, &t))
        return rc;
    TablesOwner owner{t};
    const uint64_t rows = (uint64_t)t->L * 2 * t->C;
    const uint8_t *q = p + sizeof h + ((((uint64_t)2 * h.L) + 3) & ~uint64_t(3));
    std::vector<float> lo(rows), w(rows), r(rows);
    std::memcpy(lo.data(), q, rows * 4);
    std::memcpy(w.data(), q + rows * 4, rows * 4);
    q += rows * 8;
    for (uint64_t i = 0; i < rows; ++i) r[i] = w[i] > 0.0f ? 1.0f / w[i] : 0.0f;
    CG_HIP(hipMemcpy(t->d_lo, lo.data(), rows * 4, hipMemcpyHostToDevice), "copy lo");
    CG_HIP(hipMemcpy(t->d_w, w.data(), rows * 4, hipMemcpyHostToDevice), "copy w");
    CG_HIP(hipMemcpy(t->d_r, r.data(), rows * 4, hipMemcpyHostToDevice), "copy r");
    if (t->anchor_bits == 8) {
        std::vector<float> alo(rows), aw(rows), ar(rows);
        std::memcpy(alo.data(), q, rows * 4);
        std::memcpy(aw.data(), q + rows * 4, rows * 4);
        q += rows * 8;
        for (uint64_t i = 0; i < rows; ++i) ar[i] = aw[i] > 0.0f ? 1.0f / aw[i] : 0.0f;
        CG_HIP(hipMemcpy(t->d_alo, alo.data(), rows * 4, hipMemcpyHostToDevice), "copy alo");
        CG_HIP(hipMemcpy(t->d_aw, aw.data(), rows * 4, hipMemcpyHostToDevice), "copy aw");
        CG_HIP(hipMemcpy(t->d_ar, ar.data(), rows * 4, hipMemcpyHostToDevice), "copy ar");
    }
    std::vector<uint16_t> fr(rows * kMaxBins, 0);
    for (uint64_t i = 0; i < rows; ++i) {
        const uint32_t n = t->bins[i / t->C];
        std::memcpy(fr.data() + i * kMaxBins, q, (size_t)n * 2);
        q += (size_t)n * 2;
    }
    CG_HIP(hipMemcpy(t->d_freqs, fr.data(), rows * kMaxBins * 2, hipMemcpyHostToDevice), "copy freqs");
    CG_HIP(launch_dtab(make_geom(t, 0, 1), t->d_bins, t->d_freqs, t->d_lo, t->d_w, t->d_dtab, nullptr),
           "k_dtab");
    CG_HIP(hipStreamSynchronize(nullptr), "hipStreamSynchronize");
    owner.t = nullptr;
    *out = t;
    return CG_OK;
}

int cg_container_check(const void *host_bytes, uint64_t nbytes, cg_container_header *header_out)
{
    g_error.clear();
    if (!host_bytes) return fail(CG_E_INVAL, "null bytes");
    if (nbytes < kHeaderBytes) return fail(CG_E_CORRUPT, "shorter than a container header");
    cg_container_header h;
    std::memcpy(&h, host_bytes, sizeof h);
    if (h.magic != CG_CONTAINER_MAGIC) return fail(CG_E_CORRUPT, "not a container (magic)");
    if (h.version != CG_CONTAINER_VERSION) return fail(CG_E_CORRUPT, "unknown container version");
    if (const char *err = shape_error(h.L, h.H_kv, h.d, h.S, h.group, h.chunk))
        return fail(CG_E_CORRUPT, std::string("container shape: ") + err);
    const uint32_t nk = ceil_div(h.S, h.chunk);
    if (h.chunk_begin >= h.chunk_end || h.chunk_end > nk) return fail(CG_E_CORRUPT, "chunk range");
    if (h.anchor_bits != 8 && h.anchor_bits != 16) return fail(CG_E_CORRUPT, "anchor_bits");
    if (h.outlier_ppm > kMaxOutlierPpm) return fail(CG_E_CORRUPT, "outlier_ppm");
    if (!h.outlier_ppm && h.n_outliers) return fail(CG_E_CORRUPT, "outlier entries without the table");
    const uint64_t t_lo = (uint64_t)h.chunk_begin * h.chunk;
    const uint64_t t_hi = std::min<uint64_t>((uint64_t)h.chunk_end * h.chunk, h.S);
    if (h.n_sink > t_hi - t_lo) return fail(CG_E_CORRUPT, "more sink tokens than tokens");
    const uint64_t C = (uint64_t)h.H_kv * h.d;
    const uint64_t elems = (uint64_t)h.L * 2 * (t_hi - t_lo) * C;
    if (h.n_outliers > elems || h.clamped > elems || h.payload_words > (1ull << 46))
        return fail(CG_E_CORRUPT, "counts larger than the container's elements");
    cg_container_header e = h;
    fill_layout(e);
    if (std::memcmp(&e, &h, sizeof h) != 0)
        return fail(CG_E_CORRUPT, "section offsets do not follow the layout");
    if (h.total_bytes > nbytes) return fail(CG_E_CORRUPT, "container truncated");
    const uint8_t *p = static_cast<const uint8_t *>(host_bytes);
    // group word offsets: 0 first, non-decreasing, the payload size last
    const uint64_t ng = h.n_groups;
    uint64_t prev = 0;
    for (uint64_t g = 0; g <= ng; ++g) {
        uint64_t v;
        std::memcpy(&v, p + h.offsets_offset + 8 * g, 8);
        if ((g == 0 && v != 0) || v < prev || v > h.payload_words)
            return fail(CG_E_CORRUPT, "group offsets out of order or past the payload");
        prev = v;
    }
    if (prev != h.payload_words) return fail(CG_E_CORRUPT, "group offsets do not end at the payload size");
    if (h.outlier_ppm) {
        const uint32_t NB = h.n_blocks, last_len = h.S - (nk - 1) * h.chunk;
        prev = 0;
        for (uint64_t g = 0; g <= ng; ++g) {
            uint64_t v;
            std::memcpy(&v, p + h.outliers_offset + 8 * g, 8);
            if ((g == 0 && v != 0) || v < prev || v > h.n_outliers)
                return fail(CG_E_CORRUPT, "outlier offsets out of order or past the entries");
            if (g > 0) {
                const uint64_t gi = g - 1;
                const uint32_t b = (uint32_t)(gi % NB);
                const uint32_t k = h.chunk_begin + (uint32_t)(gi / NB / (2 * (uint64_t)h.L));
                const uint32_t len = (k == nk - 1) ? last_len : h.chunk;
                const uint64_t lanes = std::min<uint64_t>(kLanes, C - (uint64_t)b * kLanes);
                for (uint64_t i = prev; i < v; ++i) {
                    uint32_t key;
                    std::memcpy(&key, p + h.outlier_keys_offset + 4 * i, 4);
                    if ((key >> 6) >= len || (key & 63u) >= lanes)
                        return fail(CG_E_CORRUPT, "an outlier key outside its group");
                }
            }
            prev = v;
        }
        if (prev != h.n_outliers) return fail(CG_E_CORRUPT, "outlier offsets do not end at the entry count");
    }
    if (header_out) *header_out = h;
    return CG_OK;
}

int cg_blob_import(const cg_tables *t, const void *host_bytes, uint64_t nbytes, void *hip_stream,
                   cg_blob **out)
{
    g_error.clear();
    if (int rc = check_tables(t)) return rc;
    if (!out) return fail(CG_E_INVAL, "null argument");
    cg_container_header h;
    if (int rc = cg_container_check(host_bytes, nbytes, &h)) return rc;
    if (h.L != t->L || h.H_kv != t->H || h.d != t->d || h.S != t->S || h.group != t->G ||
        h.chunk != t->Tc || h.anchor_bits != t->anchor_bits || h.outlier_ppm != t->outlier_ppm ||
        h.n_sink != sinks_in(t, h.chunk_begin, h.chunk_end))
        return fail(CG_E_CORRUPT, "container and tables describe different caches or settings");
    DeviceScope ds;
    CG_HIP(ds.enter(t->device), "hipSetDevice");
    hipStream_t st = (hipStream_t)hip_stream;
    cg_blob *b = new (std::nothrow) cg_blob();
    if (!b) return fail(CG_E_NOMEM, "host allocation");
    b->magic = 0;
    b->device = t->device;
    b->hdr = h;
    DevBuf data;
    hipError_t e = data.alloc(align256(h.total_bytes));
    if (e == hipSuccess)
        e = hipMemcpyAsync(data.p, host_bytes, h.total_bytes - kPayloadPadBytes, hipMemcpyHostToDevice, st);
    if (e == hipSuccess)
        e = hipMemsetAsync(data.as<uint8_t>() + h.total_bytes - kPayloadPadBytes, 0, kPayloadPadBytes, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
        delete b;
        return hip_fail(e, "import container");
    }
    b->d_data = static_cast<uint8_t *>(data.detach());
    b->magic = kBlobMagic;
    *out = b;
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
        void *ptrs[] = {t->d_bins, t->d_lo, t->d_w, t->d_r, t->d_freqs, t->d_dtab,
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

namespace {
TablesOwner::~TablesOwner()
{
    if (t) cg_free(t);
}
}  // namespace

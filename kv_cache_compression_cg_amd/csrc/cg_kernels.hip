// cg_kernels.hip -- gfx950 kernels of the KV-cache codec (see include/cg.h).
//
// Layout conventions shared by every kernel:
//   * KV caches are fp16 [L][2][S][C]; "row" means (layer, K/V) = l * 2 + kv.
//   * A "group" is (chunk, row, block b) with its 64 lanes = channels 64b .. 64b+63.
//     One wavefront decodes one group: lane i owns the stream of channel 64b + i,
//     all lanes step through the same token at the same time, so every output row
//     is written as one contiguous 128-byte store and the interleaved words of the
//     group are read from a contiguous, advancing window.
//   * Decode table entry (8 bytes) of symbol s for a lane: {f[s] | cdf[s] << 16,
//     dequantized delta lo + s * w as fp32 bits}, two planes [32][64 lanes] per
//     (row, block), so that all 64 lanes reading entry s of their own channel hit
//     64 different LDS banks whatever s each lane holds.
//
// Float rules (bit-exact with the CPU oracle): -ffp-contract=off, fp32 division and
// reciprocal correctly rounded (HIP default), fmaf only where written, fp16 output
// converted round-to-nearest-even.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cstdint>

#include "cg_internal.h"

namespace cgk {

// ------------------------------------------------------------------------------ helpers
__device__ __forceinline__ float h2f(uint32_t h) { return __half2float(__ushort_as_half((unsigned short)h)); }
__device__ __forceinline__ uint32_t f2h(float f) { return __half_as_ushort(__float2half_rn(f)); }

// unsigned image of a float that orders like the float (for atomic min / max)
__device__ __forceinline__ uint32_t f2ord(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord2f(uint32_t o)
{
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ bool any_nonfinite(uint4 v)
{
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        bad |= (w[i] & 0x7C00u) == 0x7C00u;
        bad |= (w[i] & 0x7C000000u) == 0x7C000000u;
    }
    return bad;
}

__device__ __forceinline__ void unpack8(uint4 v, float f[8])
{
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = h2f(w[i] & 0xFFFFu);
        f[2 * i + 1] = h2f(w[i] >> 16);
    }
}

// q = clamp(floor(fma(delta - lo, r, 0.5)), 0, N - 1)
__device__ __forceinline__ uint32_t quantize1(float delta, float lo, float r, uint32_t N)
{
    float v = floorf(fmaf(delta - lo, r, 0.5f));
    if (!(v > 0.0f)) return 0;
    if (v > (float)(N - 1u)) return N - 1u;
    return (uint32_t)v;
}

__device__ __forceinline__ uint32_t chunk_len(const Geom &g, uint32_t k)
{
    uint32_t t0 = k * g.Tc;
    return (g.S - t0 < g.Tc) ? g.S - t0 : g.Tc;
}

// Walks tokens [t, t_end) keeping the chunk / group position without divisions.
struct TokenWalk {
    uint32_t t, u, gp, gi, k;  // token, offset in chunk, offset in group, group in chunk, chunk
    __device__ void init(const Geom &g, uint32_t t_start)
    {
        t = t_start;
        k = t / g.Tc;
        u = t - k * g.Tc;
        gi = u / g.G;
        gp = u - gi * g.G;
    }
    __device__ void next(const Geom &g)
    {
        ++t;
        ++u;
        if (u == g.Tc) {
            u = 0;
            gp = 0;
            gi = 0;
            ++k;
        } else if (++gp == g.G) {
            gp = 0;
            ++gi;
        }
    }
};

// Row of the anchors section holding (chunk k, row, group gi); chunks before k in the
// range are full (only the last chunk of a cache can be short).
__device__ __forceinline__ uint64_t anchor_row(const Geom &g, uint32_t k, uint32_t row, uint32_t gi)
{
    uint32_t len = chunk_len(g, k);
    uint32_t ng = (len + g.G - 1) / g.G;
    return (uint64_t)(k - g.kb) * g.L * 2 * g.ngF + (uint64_t)row * ng + gi;
}

// ------------------------------------------------------------------------------ K0
// Per-channel min / max of the anchor deltas, and the non-finite flag.
// Thread = (row, token block, 8 channels); 16-byte loads, one row of C channels is
// read by C/8 consecutive threads.
__global__ __launch_bounds__(256) void k0_minmax(const uint16_t *__restrict__ X, Geom g,
                                                  uint32_t tpt, uint32_t ntb,
                                                  uint32_t *__restrict__ ord_lo,
                                                  uint32_t *__restrict__ ord_hi,
                                                  uint32_t *__restrict__ flag)
{
    const uint32_t O = g.C / 8;
    uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (uint64_t)g.L * 2 * ntb * O) return;
    uint32_t o = (uint32_t)(i % O);
    uint64_t tmp = i / O;
    uint32_t tb = (uint32_t)(tmp % ntb);
    uint32_t row = (uint32_t)(tmp / ntb);
    uint32_t t_begin = tb * tpt;
    if (t_begin >= g.S) return;
    uint32_t t_end = min(g.S, t_begin + tpt);
    const uint16_t *base = X + (uint64_t)row * g.S * g.C + o * 8;

    TokenWalk w;
    w.init(g, t_begin);
    float af[8], mn[8], mx[8];
    bool any = false, bad = false;
    if (w.gp != 0) {
        uint4 a = *reinterpret_cast<const uint4 *>(base + (uint64_t)(t_begin - w.gp) * g.C);
        unpack8(a, af);
    }
    for (; w.t < t_end; w.next(g)) {
        uint4 v = *reinterpret_cast<const uint4 *>(base + (uint64_t)w.t * g.C);
        bad |= any_nonfinite(v);
        float xf[8];
        unpack8(v, xf);
        if (w.gp == 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j) af[j] = xf[j];
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float dl = xf[j] - af[j];
                if (!any) {
                    mn[j] = dl;
                    mx[j] = dl;
                } else {
                    mn[j] = (dl < mn[j]) ? dl : mn[j];
                    mx[j] = (dl > mx[j]) ? dl : mx[j];
                }
            }
            any = true;
        }
    }
    if (any) {
        uint64_t r0 = (uint64_t)row * g.C + o * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            atomicMin(&ord_lo[r0 + j], f2ord(mn[j]));
            atomicMax(&ord_hi[r0 + j], f2ord(mx[j]));
        }
    }
    if (bad) atomicOr(flag, 1u);
}

// lo, w = (hi - lo) / (N - 1), r = 1 / w per (row, channel).
__global__ __launch_bounds__(256) void k0_finalize(Geom g, const uint8_t *__restrict__ bins,
                                                    const uint32_t *__restrict__ ord_lo,
                                                    const uint32_t *__restrict__ ord_hi,
                                                    float *__restrict__ lo, float *__restrict__ w,
                                                    float *__restrict__ r)
{
    uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= g.L * 2 * g.C) return;
    uint32_t l = i / (2 * g.C);
    float a = 0.0f, b = 0.0f;
    if (ord_lo[i] != 0xFFFFFFFFu) {
        a = ord2f(ord_lo[i]);
        b = ord2f(ord_hi[i]);
    }
    a = a + 0.0f;  // a zero bound is +0
    b = b + 0.0f;
    float ww = (b - a) / (float)(bins[l] - 1u);
    lo[i] = a;
    w[i] = ww;
    r[i] = (ww > 0.0f) ? 1.0f / ww : 0.0f;
}

// ------------------------------------------------------------------------------ K1
// Fused delta -> quantize -> histogram.  Block = (row, tile of 8*OCT channels, token
// block); its SUB x OCT threads each own 8 channels of a token sub-range.  Counts go
// to an LDS histogram [N][8][OCT] (consecutive lanes -> consecutive banks), then the
// non-zero bins are added to the global u32 counts.
__global__ __launch_bounds__(256) void k1_hist(const uint16_t *__restrict__ X, Geom g,
                                                const uint8_t *__restrict__ bins,
                                                const float *__restrict__ lo,
                                                const float *__restrict__ r, uint32_t OCT,
                                                uint32_t SUB, uint32_t tpt, uint32_t ntiles,
                                                uint32_t ntb, uint32_t *__restrict__ counts)
{
    extern __shared__ uint32_t hist[];
    uint32_t tbb = blockIdx.x % ntb;
    uint32_t tmp = blockIdx.x / ntb;
    uint32_t ct = tmp % ntiles;
    uint32_t row = tmp / ntiles;
    uint32_t N = bins[row >> 1];
    uint32_t nh = N * 8 * OCT;
    for (uint32_t j = threadIdx.x; j < nh; j += blockDim.x) hist[j] = 0;
    __syncthreads();

    const uint32_t O = g.C / 8;
    uint32_t ol = threadIdx.x % OCT, sub = threadIdx.x / OCT;
    uint32_t o = ct * OCT + ol;
    uint32_t t_begin = (tbb * SUB + sub) * tpt;
    if (sub < SUB && o < O && t_begin < g.S) {
        uint32_t t_end = min(g.S, t_begin + tpt);
        const uint16_t *base = X + (uint64_t)row * g.S * g.C + o * 8;
        float lo8[8], r8[8], af[8];
        uint64_t r0 = (uint64_t)row * g.C + o * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            lo8[j] = lo[r0 + j];
            r8[j] = r[r0 + j];
        }
        TokenWalk w;
        w.init(g, t_begin);
        if (w.gp != 0) {
            uint4 a = *reinterpret_cast<const uint4 *>(base + (uint64_t)(t_begin - w.gp) * g.C);
            unpack8(a, af);
        }
        for (; w.t < t_end; w.next(g)) {
            uint4 v = *reinterpret_cast<const uint4 *>(base + (uint64_t)w.t * g.C);
            float xf[8];
            unpack8(v, xf);
            if (w.gp == 0) {
#pragma unroll
                for (int j = 0; j < 8; ++j) af[j] = xf[j];
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    uint32_t q = quantize1(xf[j] - af[j], lo8[j], r8[j], N);
                    atomicAdd(&hist[(q * 8 + j) * OCT + ol], 1u);
                }
            }
        }
    }
    __syncthreads();
    for (uint32_t j = threadIdx.x; j < nh; j += blockDim.x) {
        uint32_t v = hist[j];
        if (!v) continue;
        uint32_t s = j / (8 * OCT), rem = j - s * 8 * OCT;
        uint32_t jj = rem / OCT, oo = ct * OCT + rem % OCT;
        if (oo >= O) continue;
        atomicAdd(&counts[((uint64_t)row * g.C + oo * 8 + jj) * kMaxBins + s], v);
    }
}

// Frequencies (T = 4096, f >= 1, remainder to the most frequent symbol) and the decode
// table of one (row, channel).
__global__ __launch_bounds__(256) void k1_freqs(Geom g, const uint8_t *__restrict__ bins,
                                                 const uint32_t *__restrict__ counts,
                                                 const float *__restrict__ lo,
                                                 const float *__restrict__ w,
                                                 uint16_t *__restrict__ freqs,
                                                 uint32_t *__restrict__ dtab)
{
    uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= g.L * 2 * g.C) return;
    uint32_t row = i / g.C, c = i - row * g.C;
    uint32_t N = bins[row >> 1];
    const uint32_t *cnt = counts + (uint64_t)i * kMaxBins;
    uint64_t n = 0;
    for (uint32_t s = 0; s < N; ++s) n += cnt[s];
    uint32_t f[kMaxBins];
    uint32_t sum = 0, best = 0;
    for (uint32_t s = 0; s < N; ++s) {
        uint64_t extra = n ? ((uint64_t)cnt[s] * (kProbTotal - N)) / n : 0;
        f[s] = 1u + (uint32_t)extra;
        sum += f[s];
        if (cnt[s] > cnt[best]) best = s;
    }
    f[best] += kProbTotal - sum;
    uint32_t P = 1;
    while (P < N) P <<= 1;
    float lo1 = lo[i], w1 = w[i];
    uint32_t *tb = dtab + (uint64_t)(row * g.NB + c / kLanes) * kTabBlock + (c % kLanes);
    uint32_t cdf = 0;
    for (uint32_t s = 0; s < kMaxBins; ++s) {
        uint32_t fs = (s < N) ? f[s] : 0;
        freqs[(uint64_t)i * kMaxBins + s] = (uint16_t)fs;
        uint32_t cf, dq;
        if (s < N) {
            cf = fs | (cdf << 16);
            dq = __float_as_uint(fmaf((float)s, w1, lo1));
        } else {
            // padding up to a power of two: cdf = T is never <= code for a valid stream
            cf = kProbTotal << 16;
            dq = __float_as_uint(fmaf((float)(N - 1u), w1, lo1));
        }
        tb[(uint64_t)s * kLanes] = cf;
        tb[kTabPlane + (uint64_t)s * kLanes] = dq;
        cdf += fs;
    }
}

// ------------------------------------------------------------------------------ K2
// Fused anchor-delta + quantize over tokens [t_lo, t_hi): 16-byte fp16 loads, 8-byte
// symbol stores, anchors copied to the container layout.  sym is [L][2][sym_T][C]
// holding tokens from sym_t0.
__global__ __launch_bounds__(256) void k2_delta_quant(const uint16_t *__restrict__ X, Geom g,
                                                       const uint8_t *__restrict__ bins,
                                                       const float *__restrict__ lo,
                                                       const float *__restrict__ r,
                                                       uint32_t t_lo, uint32_t t_hi,
                                                       uint32_t tpt, uint32_t ntb,
                                                       uint8_t *__restrict__ sym,
                                                       uint32_t sym_t0, uint32_t sym_T,
                                                       uint16_t *__restrict__ anchors)
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
    uint32_t N = bins[row >> 1];
    const uint16_t *base = X + (uint64_t)row * g.S * g.C + o * 8;
    uint8_t *sbase = sym + (uint64_t)row * sym_T * g.C + o * 8;
    float lo8[8], r8[8], af[8];
    uint64_t r0 = (uint64_t)row * g.C + o * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        lo8[j] = lo[r0 + j];
        r8[j] = r[r0 + j];
    }
    TokenWalk w;
    w.init(g, t_begin);
    if (w.gp != 0) {
        uint4 a = *reinterpret_cast<const uint4 *>(base + (uint64_t)(t_begin - w.gp) * g.C);
        unpack8(a, af);
    }
    for (; w.t < t_end; w.next(g)) {
        uint4 v = *reinterpret_cast<const uint4 *>(base + (uint64_t)w.t * g.C);
        uint2 packed = make_uint2(0, 0);
        float xf[8];
        unpack8(v, xf);
        if (w.gp == 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j) af[j] = xf[j];
            if (anchors) {
                uint64_t ar = anchor_row(g, w.k, row, w.gi);
                *reinterpret_cast<uint4 *>(anchors + ar * g.C + o * 8) = v;
            }
        } else {
            uint32_t q[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) q[j] = quantize1(xf[j] - af[j], lo8[j], r8[j], N);
            packed.x = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
            packed.y = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
        }
        *reinterpret_cast<uint2 *>(sbase + (uint64_t)(w.t - sym_t0) * g.C) = packed;
    }
}

// ------------------------------------------------------------------------------ shared
// Buffer resource over `bytes` bytes at p: loads at or past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             kBufferFlags);
}

// bytes between the table entries of consecutive symbols of one lane (32 symbols x 64
// lanes x 4 bytes per plane)
constexpr uint32_t kSymStride = kLanes * 4;              // bytes between symbols

// ------------------------------------------------------------------------------ K5
// Range encoder, three passes over the groups (chunk, row, channel block b); a block
// holds 4 wavefronts = 4 chunks of one (row, b), sharing that pair's {f | cdf << 16}
// table plane in LDS, and lane i codes the stream of channel 64b + i.  Symbols are loaded
// eight steps ahead of their use.
//   plan        replays the range evolution: counts each lane's words and records the
//               wavefront's renormalisation ballot of every step;
//   encode      codes each lane's stream into a lane-major scratch (exact size), carries
//               rippled back into the words already written;
//   interleave  moves every word to the position the lockstep decoders read it from,
//               following the recorded ballots (no second replay of the coder).
constexpr uint32_t kSymAhead = 8;
constexpr uint32_t kEncWaves = 4;

struct GroupCtx {
    uint32_t k, row, b, lane, c, nl, t0, len, ng, m;
    bool present;
};

__device__ __forceinline__ GroupCtx group_ctx(const Geom &g, uint64_t gidx, uint32_t lane)
{
    GroupCtx x;
    x.b = (uint32_t)(gidx % g.NB);
    uint64_t tmp = gidx / g.NB;
    x.row = (uint32_t)(tmp % (2 * g.L));
    x.k = g.kb + (uint32_t)(tmp / (2 * g.L));
    x.lane = lane;
    x.c = x.b * kLanes + lane;
    x.nl = min(kLanes, g.C - x.b * kLanes);
    x.present = x.c < g.C;
    x.t0 = x.k * g.Tc;
    x.len = chunk_len(g, x.k);
    x.ng = (x.len + g.G - 1) / g.G;
    x.m = x.len - x.ng;
    return x;
}

__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v, uint32_t lane)
{
    uint32_t x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t y = __shfl_up(x, d, 64);
        if (lane >= (uint32_t)d) x += y;
    }
    return x - v;
}

__device__ __forceinline__ uint32_t mbcnt64(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Symbol i of a lane's stream sits at token t0 + 1 + i + i / (G - 1): anchors are
// skipped.  Loads go through a buffer resource over the symbol rows of one (layer, K/V),
// the lane's channel as vector offset and the token row as scalar offset; reads past
// the rows return 0.
struct SymFeed {
    __amdgpu_buffer_rsrc_t rs;
    uint32_t voff, C, G1, rel, pos;

    __device__ __forceinline__ void init(const uint8_t *rows, uint32_t bytes, uint32_t c,
                                         uint32_t C_, uint32_t G, uint32_t t_rel)
    {
        rs = make_rsrc(rows, bytes);
        voff = c;
        C = C_;
        G1 = G - 1;
        rel = t_rel + 1;
        pos = 0;
    }
    // issues the load of the next symbol
    __device__ __forceinline__ uint32_t next()
    {
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b8(rs, voff, rel * C, 0);
        rel += 1;
        if (++pos == G1) {
            pos = 0;
            rel += 1;
        }
        return v;
    }
};

// Block set-up shared by the encoder passes: (row, b, set) from the block index, the
// P = 2^logp used entries of the table plane staged into LDS.  Returns the chunk of
// this wavefront.
__device__ __forceinline__ uint32_t enc_block(const Geom &g, const uint8_t *__restrict__ bins,
                                              const uint32_t *__restrict__ dtab,
                                              uint32_t n_sets, uint32_t *tab, uint32_t &row,
                                              uint32_t &b)
{
    const uint32_t set = blockIdx.x % n_sets;
    const uint32_t tmp = blockIdx.x / n_sets;
    b = tmp % g.NB;
    row = tmp / g.NB;
    const uint32_t N = bins[row >> 1];
    uint32_t P = 1;
    while (P < N) P <<= 1;
    const uint4 *src = reinterpret_cast<const uint4 *>(dtab + (uint64_t)(row * g.NB + b) * kTabBlock);
    uint4 *dst = reinterpret_cast<uint4 *>(tab);
    for (uint32_t j = threadIdx.x; j < P * kLanes / 4; j += blockDim.x) dst[j] = src[j];
    __syncthreads();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
    return g.kb + set * kEncWaves + wave;
}

__global__ __launch_bounds__(256) void k5_plan(const uint8_t *__restrict__ sym, uint32_t sym_t0,
                                                uint32_t sym_T, Geom g,
                                                const uint8_t *__restrict__ bins,
                                                const uint32_t *__restrict__ dtab,
                                                uint32_t n_sets, uint32_t *__restrict__ lane_words,
                                                uint64_t *__restrict__ group_words,
                                                uint64_t *__restrict__ masks, uint32_t mstride)
{
    __shared__ uint32_t tab[kTabPlane];
    uint32_t row, b;
    const uint32_t k = enc_block(g, bins, dtab, n_sets, tab, row, b);
    if (k >= g.ke) return;
    const uint32_t lane = threadIdx.x % kLanes;
    const uint64_t gidx = ((uint64_t)(k - g.kb) * 2 * g.L + row) * g.NB + b;
    const GroupCtx x = group_ctx(g, gidx, lane);
    uint32_t words = 0;
    if (x.m > 0) {  // uniform
        SymFeed sf;
        sf.init(sym + (uint64_t)row * sym_T * g.C, sym_T * g.C, x.present ? x.c : 0, g.C, g.G,
                x.t0 - sym_t0);
        const uint8_t *tb = reinterpret_cast<const uint8_t *>(tab) + lane * 4;
        uint64_t *mrow = masks + gidx * mstride;
        uint32_t range = kRangeInit, ev = 0, mlo = 0, mhi = 0;
        // one step: the ballot of step i is kept in lane i % 64 and written every 64 steps
        auto step = [&](uint32_t i, uint32_t s) __attribute__((always_inline)) {
            const uint32_t f = *reinterpret_cast<const uint16_t *>(tb + s * kSymStride);
            range = (range >> kProbBits) * f;
            const bool need = x.present && i + 1 < x.m && range < kRenormBelow;
            const uint64_t mask = __builtin_amdgcn_ballot_w64(need);
            if (need) {
                range <<= 16;
                ++ev;
            }
            const uint32_t j = i % kLanes;
            if (lane == j) {
                mlo = (uint32_t)mask;
                mhi = (uint32_t)(mask >> 32);
            }
            if (j == kLanes - 1 || i + 1 == x.m) {
                if (lane <= j) {
                    uint2 v;
                    v.x = mlo;
                    v.y = mhi;
                    *reinterpret_cast<uint2 *>(mrow + (i - j) + lane) = v;
                }
            }
        };
        uint32_t sr[kSymAhead];
#pragma unroll
        for (uint32_t r = 0; r < kSymAhead; ++r) sr[r] = sf.next();
        uint32_t i = 0;
        for (; i + kSymAhead <= x.m; i += kSymAhead) {
#pragma unroll
            for (uint32_t r = 0; r < kSymAhead; ++r) {
                const uint32_t s_ = sr[r];
                sr[r] = sf.next();
                step(i + r, s_);
            }
        }
#pragma unroll
        for (uint32_t r = 0; r < kSymAhead; ++r)
            if (i + r < x.m) step(i + r, sr[r]);
        if (x.present) words = 2 + ev;
    }
    lane_words[gidx * kLanes + lane] = words;
    uint32_t tot = words;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) tot += __shfl_xor(tot, d, 64);
    if (lane == 0) group_words[gidx] = tot;
}

// Exclusive prefix sum of n values in one block; out[n] = total.
__global__ __launch_bounds__(1024) void k_scan(const uint64_t *__restrict__ in,
                                                uint64_t *__restrict__ out, uint64_t n)
{
    __shared__ uint64_t part[1024];
    uint32_t tid = threadIdx.x;
    uint64_t per = (n + 1023) / 1024;
    uint64_t beg = min(n, (uint64_t)tid * per), end = min(n, beg + per);
    uint64_t s = 0;
    for (uint64_t j = beg; j < end; ++j) s += in[j];
    part[tid] = s;
    __syncthreads();
    for (uint32_t d = 1; d < 1024; d <<= 1) {
        uint64_t y = (tid >= d) ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += y;
        __syncthreads();
    }
    uint64_t run = part[tid] - s;
    for (uint64_t j = beg; j < end; ++j) {
        out[j] = run;
        run += in[j];
    }
    if (tid == 1023) out[n] = part[1023];
}

__global__ __launch_bounds__(256) void k5_encode(const uint8_t *__restrict__ sym, uint32_t sym_t0,
                                                  uint32_t sym_T, Geom g,
                                                  const uint8_t *__restrict__ bins,
                                                  const uint32_t *__restrict__ dtab,
                                                  uint32_t n_sets,
                                                  const uint32_t *__restrict__ lane_words,
                                                  const uint64_t *__restrict__ group_off,
                                                  uint16_t *__restrict__ scratch)
{
    __shared__ uint32_t tab[kTabPlane];
    uint32_t row, b;
    const uint32_t k = enc_block(g, bins, dtab, n_sets, tab, row, b);
    if (k >= g.ke) return;
    const uint32_t lane = threadIdx.x % kLanes;
    const uint64_t gidx = ((uint64_t)(k - g.kb) * 2 * g.L + row) * g.NB + b;
    const GroupCtx x = group_ctx(g, gidx, lane);
    const uint32_t nwords = lane_words[gidx * kLanes + lane];
    const uint32_t lane_off = wave_excl_scan(nwords, lane);
    if (x.m == 0) return;  // uniform
    uint16_t *out = scratch + group_off[gidx] + lane_off;
    SymFeed sf;
    sf.init(sym + (uint64_t)row * sym_T * g.C, sym_T * g.C, x.present ? x.c : 0, g.C, g.G,
            x.t0 - sym_t0);
    const uint8_t *tb = reinterpret_cast<const uint8_t *>(tab) + lane * 4;
    uint64_t low = 0;
    uint32_t range = kRangeInit, nw = 0;
    auto step = [&](uint32_t i, uint32_t s) __attribute__((always_inline)) {
        const uint32_t e = *reinterpret_cast<const uint32_t *>(tb + s * kSymStride);
        const uint32_t q = range >> kProbBits;
        low += (uint64_t)q * (e >> 16);
        range = q * (e & 0xFFFFu);
        if (low >> 32) {  // carry into the words already written
            low &= 0xFFFFFFFFull;
            uint32_t j = nw;
            uint16_t v;
            do {
                --j;
                v = (uint16_t)(out[j] + 1u);
                out[j] = v;
            } while (v == 0 && j > 0);
        }
        if (i + 1 < x.m && range < kRenormBelow) {
            out[nw++] = (uint16_t)(low >> 16);
            low = (low & 0xFFFFull) << 16;
            range <<= 16;
        }
    };
    uint32_t sr[kSymAhead];
#pragma unroll
    for (uint32_t r = 0; r < kSymAhead; ++r) sr[r] = sf.next();
    uint32_t i = 0;
    if (x.present) {
        for (; i + kSymAhead <= x.m; i += kSymAhead) {
#pragma unroll
            for (uint32_t r = 0; r < kSymAhead; ++r) {
                const uint32_t s_ = sr[r];
                sr[r] = sf.next();
                step(i + r, s_);
            }
        }
#pragma unroll
        for (uint32_t r = 0; r < kSymAhead; ++r)
            if (i + r < x.m) step(i + r, sr[r]);
        out[nw++] = (uint16_t)(low >> 16);
        out[nw++] = (uint16_t)(low & 0xFFFFu);
    }
}

__global__ __launch_bounds__(256) void k5_interleave(Geom g, uint32_t n_sets,
                                                      const uint32_t *__restrict__ lane_words,
                                                      const uint64_t *__restrict__ group_off,
                                                      const uint64_t *__restrict__ masks,
                                                      uint32_t mstride,
                                                      const uint16_t *__restrict__ scratch,
                                                      uint16_t *__restrict__ payload)
{
    const uint32_t set = blockIdx.x % n_sets;
    const uint32_t tmp = blockIdx.x / n_sets;
    const uint32_t b = tmp % g.NB;
    const uint32_t row = tmp / g.NB;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
    const uint32_t k = g.kb + set * kEncWaves + wave;
    if (k >= g.ke) return;
    const uint32_t lane = threadIdx.x % kLanes;
    const uint64_t gidx = ((uint64_t)(k - g.kb) * 2 * g.L + row) * g.NB + b;
    const GroupCtx x = group_ctx(g, gidx, lane);
    const uint32_t nwords = lane_words[gidx * kLanes + lane];
    const uint32_t lane_off = wave_excl_scan(nwords, lane);
    if (x.m == 0) return;  // uniform
    const uint16_t *src = scratch + group_off[gidx] + lane_off;
    uint16_t *dst = payload + group_off[gidx];
    uint32_t e = 2, w_next = 0;
    if (x.present) {
        dst[2 * lane] = src[0];
        dst[2 * lane + 1] = src[1];
        if (nwords > 2) w_next = src[2];
    }
    const uint64_t *mrow = masks + gidx * mstride;
    uint32_t cursor = 2 * x.nl;
    for (uint32_t base = 0; base < x.m; base += kLanes) {
        // the ballots of steps base .. base + 63, one per lane
        uint2 mm = make_uint2(0, 0);
        if (base + lane < x.m) mm = *reinterpret_cast<const uint2 *>(mrow + base + lane);
        const uint32_t n = min(kLanes, x.m - base);
        for (uint32_t j = 0; j < n; ++j) {
            // (readlane returns a signed int: go through uint32_t, no sign extension)
            const uint32_t mlo = (uint32_t)__builtin_amdgcn_readlane(mm.x, j);
            const uint32_t mhi = (uint32_t)__builtin_amdgcn_readlane(mm.y, j);
            const uint64_t mask = ((uint64_t)mhi << 32) | mlo;
            if (mask) {
                if ((mask >> lane) & 1u) {
                    dst[cursor + mbcnt64(mask)] = (uint16_t)w_next;
                    ++e;
                    if (e < nwords) w_next = src[e];
                }
                cursor += (uint32_t)__builtin_popcountll(mask);
            }
        }
    }
}


// ------------------------------------------------------------------------------ K3 (+K4)
// Range decoder fused with dequantize + anchor-add.  Block = 4 wavefronts, each decoding
// two chunks of the same (row, block) in lockstep, all sharing the block's decode table
// in LDS (P <= 32 entries x 64 lanes x 8 bytes).  Everything that is the same for the
// 64 lanes (chunk, token, group, stream cursor, row addresses) is kept in scalar
// registers; only the coder state and the table address are per lane.

// Per-wavefront LDS ring of payload words (stored inverted, see below), refilled with
// 4-byte-per-lane loads.  Ring slots [0, 64) are mirrored at [R, R + 64), so the up-to-
// 64 words one step reads are contiguous in LDS.
constexpr uint32_t kRingWords = 256;
constexpr uint32_t kRingAlloc = kRingWords + 64;
constexpr uint32_t kFetchWords = 128;
constexpr uint32_t kWavesPerBlock = 4;
constexpr uint32_t kStreamsPerWave = 2;   // chunks one wavefront decodes in lockstep
// Groups of this many decode steps (anchor interval 10) run fully unrolled with their
// outputs held in registers; any other group length takes the generic loop.
constexpr int kUnrolledSteps = 9;

// Stores the 2 words at stream position pos (even) into the ring, inverted.
__device__ __forceinline__ void ring_put(uint16_t *ring, uint32_t pos, uint32_t v)
{
    const uint32_t slot = pos & (kRingWords - 1);
    *reinterpret_cast<uint32_t *>(ring + slot) = ~v;
    if (slot < 64) *reinterpret_cast<uint32_t *>(ring + slot + kRingWords) = ~v;
}

// State of one wavefront's decoder.  The coder state is kept as ncode = ~code, which
// turns both the symbol search and the state update into one multiply-add each:
//   q*cdf <= code  <=>  (int)(q*cdf + ncode) < 0    (all values < 2^31)
//   ~(code - q*cdf) = q*cdf + ncode.
// Renormalisation shifts in inverted words, which is why the ring holds ~word.
// The LDS table holds, per symbol s and lane, {f | cdf << 16} at byte 256*s + 4*lane
// (cdf in the upper half, read zero-extended by the search) and the dequantized delta
// 8 KiB further: a lane's probe never conflicts with
// another lane's, whatever symbols the lanes are at.
constexpr uint32_t kDqOffset = kTabPlane * 4;            // byte offset of the delta plane

// p + (d < 0 ? STEP : 0) for a power-of-two STEP, as a shift and a shift-add.  (Written
// out because the compiler otherwise folds the last level into an and + add pair.)
template <uint32_t STEP>
__device__ __forceinline__ uint32_t take_upper(uint32_t d, uint32_t p)
{
    static_assert((STEP & (STEP - 1)) == 0 && STEP >= 4 && STEP <= (1u << 15), "step");
    constexpr uint32_t kShift = __builtin_ctz(STEP);
    uint32_t r;
    asm("v_lshrrev_b32 %0, 31, %1\n\tv_lshl_add_u32 %0, %0, %2, %3"
        : "=&v"(r)
        : "v"(d), "n"(kShift), "v"(p));
    return r;
}

struct WaveDecoder {
    uint32_t ncode, range;
    uint32_t cur, re;  // next unread word; words [re - R, re) are in the ring
    uint32_t i, m;     // symbols decoded so far / in the chunk
    uint16_t *ring;
    __amdgpu_buffer_rsrc_t wrs;
    bool present;

    // Binary search over the lane's cdf column, levels LEVEL .. 0: the largest symbol
    // s with q*cdf[s] <= code, as the byte offset of its entry.
    template <int LEVEL>
    __device__ __forceinline__ uint32_t search(const uint8_t *tab, uint32_t p, uint32_t q) const
    {
        if constexpr (LEVEL < 0) {
            return p;
        } else {
            constexpr uint32_t kStep = (1u << LEVEL) * kSymStride;
            const uint32_t cdf = *reinterpret_cast<const uint16_t *>(tab + p + kStep + 2);
            return search<LEVEL - 1>(tab, take_upper<kStep>(__umul24(q, cdf) + ncode, p), q);
        }
    }

    // Decodes one symbol; returns the byte offset of its table entry.  ctop is the
    // lane's cdf at the first probe (symbol P/2), the same for every step.
    template <int LOGP>
    __device__ __forceinline__ uint32_t symbol(const uint8_t *tab, uint32_t lb, uint32_t ctop,
                                               float &dq)
    {
        constexpr uint32_t kTop = (1u << (LOGP - 1)) * kSymStride;
        const uint32_t q = range >> kProbBits;
        const uint32_t p = search<LOGP - 2>(tab, take_upper<kTop>(__umul24(q, ctop) + ncode, lb), q);
        // cdf as a zero-extending 16-bit read of the upper half, f from the low half of
        // the whole entry (a word-select operand of the multiply): no masking needed
        const uint32_t cdf = *reinterpret_cast<const uint16_t *>(tab + p + 2);
        const uint32_t e = *reinterpret_cast<const uint32_t *>(tab + p);
        dq = *reinterpret_cast<const float *>(tab + p + kDqOffset);
        ncode = __umul24(q, cdf) + ncode;
        range = __umul24(q, e & 0xFFFFu);
        return p;
    }

    // Loads ring chunks until the words [cur, cur + cnt) are present (rare path).
    __device__ __forceinline__ void refill_now(uint32_t cnt, uint32_t lane)
    {
        while (cur + cnt > re) {
            ring_put(ring, re + 2 * lane, __builtin_amdgcn_raw_buffer_load_b32(wrs, 2 * (re + 2 * lane), 0, 0));
            re += kFetchWords;
        }
    }

    // Renormalisation after a symbol that is not the chunk's last.
    __device__ __forceinline__ void renorm(uint32_t lane)
    {
        // (the ballot takes the comparison itself, so the lane mask is not materialised
        // in a vector register; with no lane renormalising the body does nothing)
        const bool need = present && (range < kRenormBelow);
        const uint64_t mask = __builtin_amdgcn_ballot_w64(need);
        const uint32_t cnt = (uint32_t)__builtin_popcountll(mask);
        if (__builtin_expect(cur + cnt > re, 0)) refill_now(cnt, lane);
        if (need) {
            const uint16_t *rp = ring + (cur & (kRingWords - 1));
            ncode = (ncode << 16) | rp[mbcnt64(mask)];
            range <<= 16;
        }
        cur += cnt;
    }
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <bool SYMBOLS>
__device__ __forceinline__ void put_out(const __amdgpu_buffer_rsrc_t &ors, uint32_t olane,
                                        uint32_t orow, uint32_t v)
{
    if (SYMBOLS)
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)v, ors, olane, orow, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)v, ors, olane, orow, 0);
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

// One decoder stream: chunk k of (row, channel block b), one channel per lane, with its
// anchor rows, output rows and payload words.  Vector memory is only touched at anchor
// boundaries: at a group's start the next anchor row and the next chunk of words are
// requested and the previous group's outputs (held in registers) are written; the
// requested data is consumed at the group's end.  Waits for it therefore never wait for
// a store issued during the group.
template <bool SYMBOLS>
struct Stream {
    WaveDecoder dec;
    __amdgpu_buffer_rsrc_t ars, ors;
    uint32_t ng, len;           // groups / tokens in the chunk
    uint32_t astride, ostride, olane;
    uint32_t a16;               // anchor row of the current group (fp16 bits)
    float af;
    uint32_t orow;              // byte offset of the current anchor row
    uint32_t orow_held;         // byte offset of the first row held in yf / ys
    bool held;                  // yf / ys hold the outputs of the previous group
    uint32_t a_next, pf, pf_at; // requests of the current group
    bool fetch;
    float yf[kUnrolledSteps];
    uint32_t ys[kUnrolledSteps];

    __device__ __forceinline__ void init(const Geom &g, uint16_t *ring,
                                         const uint8_t *__restrict__ container,
                                         const ContainerView &cv, uint32_t k, uint32_t row,
                                         uint32_t b, uint32_t lane, bool present,
                                         uint16_t *__restrict__ out, uint8_t *__restrict__ sym_out)
    {
        const uint32_t nl = min(kLanes, g.C - b * kLanes);
        const uint32_t t0 = k * g.Tc;
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
        ars = make_rsrc(container + cv.anchors_off + 2 * aoff,
                        (uint32_t)min(cv.anchors_bytes - min(2 * aoff, cv.anchors_bytes),
                                      (uint64_t)0xFFFFFFFFu));
        astride = 2 * g.C;
        const uint64_t obase = ((uint64_t)row * g.S + t0) * g.C + b * kLanes;
        ors = SYMBOLS ? make_rsrc(sym_out + obase, 0xFFFFFFFFu) : make_rsrc(out + obase, 0xFFFFFFFFu);
        ostride = g.C * (SYMBOLS ? 1u : 2u);  // bytes between token rows
        olane = lane * (SYMBOLS ? 1u : 2u);

        dec.ncode = 0xFFFFFFFFu;
        dec.range = kRangeInit;
        dec.re = 0;
        if (dec.m > 0) {
            dec.cur = 0;
            dec.refill_now(kRingWords, lane);
            if (present) dec.ncode = ((uint32_t)ring[2 * lane] << 16) | ring[2 * lane + 1];
        }
        dec.cur = 2 * nl;
        held = false;
        orow = 0;
        orow_held = 0;
    }

    // first anchor row; the empty asm pins the wait for it here
    __device__ __forceinline__ void first_anchor(uint32_t lane)
    {
        uint32_t v = __builtin_amdgcn_raw_buffer_load_b16(ars, 2 * lane, 0, 0);
        asm volatile("" : "+v"(v));
        a16 = v;
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

    // the next anchor row and the next chunk of words (kept only if the ring has room)
    __device__ __forceinline__ void request(uint32_t gi, uint32_t lane)
    {
        a_next = __builtin_amdgcn_raw_buffer_load_b16(ars, 2 * lane, (gi + 1) * astride, 0);
        fetch = dec.m > 0 && dec.re + kFetchWords - dec.cur <= kRingWords;
        pf_at = dec.re;
        pf = __builtin_amdgcn_raw_buffer_load_b32(dec.wrs, 2 * (pf_at + 2 * lane), 0, 0);
    }

    // the previous group's outputs, then this group's anchor row
    __device__ __forceinline__ void write_rows()
    {
        if (held) {
            if (dec.present) flush_rows<SYMBOLS>(ors, olane, orow_held, ostride, yf, ys);
            held = false;
        }
        if (dec.present) put_out<SYMBOLS>(ors, olane, orow, SYMBOLS ? 0u : a16);
        orow += ostride;
    }

    // takes in the requests; the ring chunk is dropped if a refill inside the group
    // already loaded those words.  (The empty asm pins where the loaded values are first
    // needed, so the wait for them is placed here.)
    __device__ __forceinline__ void consume(uint32_t lane)
    {
        uint32_t an = a_next, pv = pf;
        asm volatile("" : "+v"(an), "+v"(pv));
        a16 = an;
        af = h2f(a16);
        if (fetch && dec.re == pf_at) {
            ring_put(dec.ring, pf_at + 2 * lane, pv);
            dec.re = pf_at + kFetchWords;
        }
    }

    // step u of an unrolled group: the output stays in a register
    template <int LOGP>
    __device__ __forceinline__ void step_held(const uint8_t *tab, uint32_t lb, uint32_t ctop, int u)
    {
        float dq;
        const uint32_t p = dec.template symbol<LOGP>(tab, lb, ctop, dq);
        if (SYMBOLS)
            ys[u] = p / kSymStride;
        else
            yf[u] = af + dq;
    }

    __device__ __forceinline__ void finish_unrolled()
    {
        dec.i += kUnrolledSteps;
        held = true;
        orow_held = orow;
        orow += kUnrolledSteps * ostride;
    }

    template <int LOGP>
    __device__ __forceinline__ void unrolled(const uint8_t *tab, uint32_t lb, uint32_t ctop,
                                             uint32_t lane)
    {
#pragma unroll
        for (int u = 0; u < kUnrolledSteps; ++u) {
            step_held<LOGP>(tab, lb, ctop, u);
            // the state update is computed here, next to its table read
            asm volatile("" : "+v"(dec.ncode));
            dec.renorm(lane);
        }
        finish_unrolled();
    }

    // any other group: one store per step
    template <int LOGP>
    __device__ __forceinline__ void generic(const uint8_t *tab, uint32_t lb, uint32_t ctop,
                                            uint32_t nsteps, uint32_t lane)
    {
        for (uint32_t u = nsteps; u != 0; --u) {
            float dq;
            const uint32_t p = dec.template symbol<LOGP>(tab, lb, ctop, dq);
            if (dec.present)
                put_out<SYMBOLS>(ors, olane, orow, SYMBOLS ? p / kSymStride : f2h(af + dq));
            orow += ostride;
            if (++dec.i < dec.m) dec.renorm(lane);
        }
    }

    __device__ __forceinline__ void final_flush()
    {
        if (held && dec.present) flush_rows<SYMBOLS>(ors, olane, orow_held, ostride, yf, ys);
    }
};

// One wavefront decodes NS chunks of the same (row, channel block) in lockstep, sharing
// the block's LDS table.  With two, the symbol searches of both streams sit in one
// basic block, so the dependent LDS reads of one overlap the arithmetic of the other.
template <int LOGP, bool SYMBOLS, bool FULL, int NS>
__device__ __forceinline__ void decode_chunks(const Geom &g, const uint8_t *__restrict__ tab,
                                              uint16_t *__restrict__ ring,
                                              const uint8_t *__restrict__ container,
                                              const ContainerView &cv, uint32_t k0, uint32_t k1,
                                              uint32_t row, uint32_t b, uint32_t lane,
                                              uint16_t *__restrict__ out,
                                              uint8_t *__restrict__ sym_out)
{
    const bool present = FULL || lane < min(kLanes, g.C - b * kLanes);
    const uint32_t lb = lane * 4;  // entry (symbol 0, this lane)
    const uint32_t ctop =
        *reinterpret_cast<const uint16_t *>(tab + lb + (1u << (LOGP - 1)) * kSymStride + 2);
    Stream<SYMBOLS> st[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s)
        st[s].init(g, ring + s * kRingAlloc, container, cv, s == 0 ? k0 : k1, row, b, lane,
                   present, out, sym_out);
#pragma unroll
    for (int s = 0; s < NS; ++s) st[s].first_anchor(lane);
    uint32_t ngmax = st[0].ng;
    if (NS == 2) ngmax = max(ngmax, st[NS - 1].ng);

    for (uint32_t gi = 0; gi < ngmax; ++gi) {
        bool act[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) act[s] = gi < st[s].ng;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < NS; ++s)
            if (act[s]) st[s].request(gi, lane);
#pragma unroll
        for (int s = 0; s < NS; ++s)
            if (act[s]) st[s].write_rows();
        __builtin_amdgcn_sched_barrier(0);

        uint32_t nsteps[NS];
        bool unr[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            nsteps[s] = act[s] ? st[s].steps(g, gi) : 0u;
            unr[s] = act[s] && st[s].unrollable(nsteps[s]);
        }
        if (NS == 2 && unr[0] && unr[NS - 1]) {
#pragma unroll
            for (int u = 0; u < kUnrolledSteps; ++u) {
#pragma unroll
                for (int s = 0; s < NS; ++s) st[s].template step_held<LOGP>(tab, lb, ctop, u);
                // both state updates are computed here, next to their table reads
                asm volatile("" : "+v"(st[0].dec.ncode), "+v"(st[NS - 1].dec.ncode));
#pragma unroll
                for (int s = 0; s < NS; ++s) st[s].dec.renorm(lane);
            }
#pragma unroll
            for (int s = 0; s < NS; ++s) st[s].finish_unrolled();
        } else {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                if (unr[s])
                    st[s].template unrolled<LOGP>(tab, lb, ctop, lane);
                else if (act[s])
                    st[s].template generic<LOGP>(tab, lb, ctop, nsteps[s], lane);
            }
        }

        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < NS; ++s)
            if (act[s]) st[s].consume(lane);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) st[s].final_flush();
}

template <bool SYMBOLS, bool FULL>
__device__ __forceinline__ void decode_dispatch(uint32_t logp, bool pair, const Geom &g,
                                                const uint8_t *tab, uint16_t *ring,
                                                const uint8_t *container, const ContainerView &cv,
                                                uint32_t k0, uint32_t k1, uint32_t row, uint32_t b,
                                                uint32_t lane, uint16_t *out, uint8_t *sym_out)
{
#define CG_DECODE_CASE(LP)                                                                        \
    case LP:                                                                                      \
        if (pair)                                                                                 \
            decode_chunks<LP, SYMBOLS, FULL, 2>(g, tab, ring, container, cv, k0, k1, row, b,      \
                                                lane, out, sym_out);                              \
        else                                                                                      \
            decode_chunks<LP, SYMBOLS, FULL, 1>(g, tab, ring, container, cv, k0, k1, row, b,      \
                                                lane, out, sym_out);                              \
        break;
    switch (logp) {
        CG_DECODE_CASE(1)
        CG_DECODE_CASE(2)
        CG_DECODE_CASE(3)
        CG_DECODE_CASE(4)
    default:
        CG_DECODE_CASE(5)
    }
#undef CG_DECODE_CASE
}

// Block = WPB wavefronts over the chunks [kb + 2 WPB set, kb + 2 WPB (set + 1)) of one
// (row, channel block); wavefront w takes chunks base + w and base + w + WPB.  Launches
// over many chunks use 4 wavefronts per block, sharing the staged table; launches over
// a few chunks (a streamed chunk) use 1, so that more blocks are resident.
template <bool SYMBOLS, uint32_t WPB>
__global__ __launch_bounds__(WPB * 64) void k3_decode(Geom g, const uint8_t *__restrict__ bins,
                                                  const uint32_t *__restrict__ dtab,
                                                  const uint8_t *__restrict__ container,
                                                  ContainerView cv, uint32_t n_sets,
                                                  uint16_t *__restrict__ out,
                                                  uint8_t *__restrict__ sym_out)
{
    __shared__ uint32_t tab[kTabBlock];
    __shared__ uint16_t rings[WPB * kStreamsPerWave * kRingAlloc];
    const uint32_t set = blockIdx.x % n_sets;
    const uint32_t tmp = blockIdx.x / n_sets;
    const uint32_t b = tmp % g.NB;
    const uint32_t row = tmp / g.NB;
    const uint32_t N = bins[row >> 1];
    uint32_t logp = 0;
    while ((1u << logp) < N) ++logp;
    // stage the P = 2^logp used entries of both planes
    const uint32_t n16 = ((1u << logp) * kLanes) / 4;  // 16-byte pieces per plane
    const uint4 *src = reinterpret_cast<const uint4 *>(dtab + (uint64_t)(row * g.NB + b) * kTabBlock);
    uint4 *dst = reinterpret_cast<uint4 *>(tab);
    for (uint32_t j = threadIdx.x; j < n16; j += blockDim.x) {
        dst[j] = src[j];
        dst[kTabPlane / 4 + j] = src[kTabPlane / 4 + j];
    }
    __syncthreads();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
    const uint32_t lane = threadIdx.x % kLanes;
    const uint32_t k0 = g.kb + set * WPB * kStreamsPerWave + wave;
    const uint32_t k1 = k0 + WPB;
    if (k0 >= g.ke) return;
    const uint8_t *tb = reinterpret_cast<const uint8_t *>(tab);
    uint16_t *ring = rings + wave * kStreamsPerWave * kRingAlloc;
    const bool pair = k1 < g.ke;
    if (g.C - b * kLanes >= kLanes)
        decode_dispatch<SYMBOLS, true>(logp, pair, g, tb, ring, container, cv, k0, k1, row, b,
                                       lane, out, sym_out);
    else
        decode_dispatch<SYMBOLS, false>(logp, pair, g, tb, ring, container, cv, k0, k1, row, b,
                                        lane, out, sym_out);
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
    float lo8[8], w8[8], af[8];
    uint64_t r0 = (uint64_t)row * g.C + o * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        lo8[j] = lo[r0 + j];
        w8[j] = w[r0 + j];
    }
    TokenWalk tw;
    tw.init(g, t_begin);
    if (tw.gp != 0) {
        uint4 a = *reinterpret_cast<const uint4 *>(anc + anchor_row(g, tw.k, row, tw.gi) * g.C);
        unpack8(a, af);
    }
    const uint64_t ob = (uint64_t)row * g.S * g.C + o * 8;
    for (; tw.t < t_end; tw.next(g)) {
        uint4 res;
        if (tw.gp == 0) {
            res = *reinterpret_cast<const uint4 *>(anc + anchor_row(g, tw.k, row, tw.gi) * g.C);
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
hipError_t launch_k0(const uint16_t *X, const Geom &g, uint32_t tpt, uint32_t *ord_lo,
                     uint32_t *ord_hi, uint32_t *flag, hipStream_t st)
{
    uint32_t ntb = (g.S + tpt - 1) / tpt;
    uint64_t threads = (uint64_t)g.L * 2 * ntb * (g.C / 8);
    hipLaunchKernelGGL(k0_minmax, dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0, st, X, g,
                       tpt, ntb, ord_lo, ord_hi, flag);
    return hipGetLastError();
}

hipError_t launch_k0_finalize(const Geom &g, const uint8_t *bins, const uint32_t *ord_lo,
                              const uint32_t *ord_hi, float *lo, float *w, float *r, hipStream_t st)
{
    uint32_t n = g.L * 2 * g.C;
    hipLaunchKernelGGL(k0_finalize, dim3((n + 255) / 256), dim3(256), 0, st, g, bins, ord_lo,
                       ord_hi, lo, w, r);
    return hipGetLastError();
}

hipError_t launch_k1(const uint16_t *X, const Geom &g, const uint8_t *bins, uint32_t max_bins,
                     const float *lo, const float *r, uint32_t *counts, hipStream_t st)
{
    const uint32_t O = g.C / 8;
    const uint32_t OCT = O < 32 ? O : 32;
    const uint32_t SUB = 256 / OCT;
    const uint32_t ntiles = (O + OCT - 1) / OCT;
    const uint64_t rows = (uint64_t)g.L * 2;
    uint64_t ntb_target = (8192 + rows * ntiles - 1) / (rows * ntiles);
    uint64_t tpt = (g.S + ntb_target * SUB - 1) / (ntb_target * SUB);
    if (tpt < 16) tpt = 16;
    uint32_t ntb = (uint32_t)((g.S + tpt * SUB - 1) / (tpt * SUB));
    size_t lds = (size_t)max_bins * 8 * OCT * sizeof(uint32_t);
    hipLaunchKernelGGL(k1_hist, dim3((uint32_t)(rows * ntiles * ntb)), dim3(256), lds, st, X, g,
                       bins, lo, r, OCT, SUB, (uint32_t)tpt, ntiles, ntb, counts);
    return hipGetLastError();
}

hipError_t launch_k1_freqs(const Geom &g, const uint8_t *bins, const uint32_t *counts,
                           const float *lo, const float *w, uint16_t *freqs, uint32_t *dtab,
                           hipStream_t st)
{
    uint32_t n = g.L * 2 * g.C;
    hipLaunchKernelGGL(k1_freqs, dim3((n + 255) / 256), dim3(256), 0, st, g, bins, counts, lo, w,
                       freqs, dtab);
    return hipGetLastError();
}

hipError_t launch_k2(const uint16_t *X, const Geom &g, const uint8_t *bins, const float *lo,
                     const float *r, uint32_t t_lo, uint32_t t_hi, uint32_t tpt, uint8_t *sym,
                     uint32_t sym_t0, uint32_t sym_T, uint16_t *anchors, hipStream_t st)
{
    uint32_t ntb = (t_hi - t_lo + tpt - 1) / tpt;
    uint64_t threads = (uint64_t)g.L * 2 * ntb * (g.C / 8);
    hipLaunchKernelGGL(k2_delta_quant, dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0, st,
                       X, g, bins, lo, r, t_lo, t_hi, tpt, ntb, sym, sym_t0, sym_T, anchors);
    return hipGetLastError();
}

static uint32_t enc_sets(const Geom &g) { return (g.ke - g.kb + kEncWaves - 1) / kEncWaves; }

hipError_t launch_k5_plan(const uint8_t *sym, uint32_t sym_t0, uint32_t sym_T, const Geom &g,
                          const uint8_t *bins, const uint32_t *dtab, uint32_t *lane_words,
                          uint64_t *group_words, uint64_t *masks, uint32_t mstride,
                          hipStream_t st)
{
    const uint32_t n_sets = enc_sets(g);
    const uint64_t blocks = (uint64_t)g.L * 2 * g.NB * n_sets;
    hipLaunchKernelGGL(k5_plan, dim3((uint32_t)blocks), dim3(256), 0, st, sym, sym_t0, sym_T, g,
                       bins, dtab, n_sets, lane_words, group_words, masks, mstride);
    return hipGetLastError();
}

hipError_t launch_scan(const uint64_t *in, uint64_t *out, uint64_t n, hipStream_t st)
{
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, st, in, out, n);
    return hipGetLastError();
}

hipError_t launch_k5_encode(const uint8_t *sym, uint32_t sym_t0, uint32_t sym_T, const Geom &g,
                            const uint8_t *bins, const uint32_t *dtab,
                            const uint32_t *lane_words, const uint64_t *group_off,
                            uint16_t *scratch, hipStream_t st)
{
    const uint32_t n_sets = enc_sets(g);
    const uint64_t blocks = (uint64_t)g.L * 2 * g.NB * n_sets;
    hipLaunchKernelGGL(k5_encode, dim3((uint32_t)blocks), dim3(256), 0, st, sym, sym_t0, sym_T, g,
                       bins, dtab, n_sets, lane_words, group_off, scratch);
    return hipGetLastError();
}

hipError_t launch_k5_interleave(const Geom &g, const uint32_t *lane_words,
                                const uint64_t *group_off, const uint64_t *masks,
                                uint32_t mstride, const uint16_t *scratch, uint16_t *payload,
                                hipStream_t st)
{
    const uint32_t n_sets = enc_sets(g);
    const uint64_t blocks = (uint64_t)g.L * 2 * g.NB * n_sets;
    hipLaunchKernelGGL(k5_interleave, dim3((uint32_t)blocks), dim3(256), 0, st, g, n_sets,
                       lane_words, group_off, masks, mstride, scratch, payload);
    return hipGetLastError();
}

hipError_t launch_k3(const Geom &g, const uint8_t *bins, const uint32_t *dtab,
                     const uint8_t *container, const ContainerView &cv, uint16_t *out,
                     uint8_t *sym_out, hipStream_t st)
{
    // fewer than 8 chunks: one wavefront per block (see k3_decode)
    const bool wide = g.ke - g.kb >= kWavesPerBlock * kStreamsPerWave;
    const uint32_t wpb = wide ? kWavesPerBlock : 1u;
    const uint32_t per_block = wpb * kStreamsPerWave;
    const uint32_t n_sets = (g.ke - g.kb + per_block - 1) / per_block;
    const uint64_t blocks = (uint64_t)g.L * 2 * g.NB * n_sets;
    const dim3 grid((uint32_t)blocks), block(wpb * kLanes);
    if (sym_out) {
        if (wide)
            hipLaunchKernelGGL((k3_decode<true, kWavesPerBlock>), grid, block, 0, st, g, bins,
                               dtab, container, cv, n_sets, out, sym_out);
        else
            hipLaunchKernelGGL((k3_decode<true, 1>), grid, block, 0, st, g, bins, dtab,
                               container, cv, n_sets, out, sym_out);
    } else {
        if (wide)
            hipLaunchKernelGGL((k3_decode<false, kWavesPerBlock>), grid, block, 0, st, g, bins,
                               dtab, container, cv, n_sets, out, sym_out);
        else
            hipLaunchKernelGGL((k3_decode<false, 1>), grid, block, 0, st, g, bins, dtab,
                               container, cv, n_sets, out, sym_out);
    }
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

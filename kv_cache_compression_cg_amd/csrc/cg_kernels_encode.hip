// cg_kernels_encode.hip -- gfx950 kernels of cg_build_cdf and cg_encode: range and
// non-finite check (K0), histogram and frequency / decode tables (K1), anchor delta +
// quantize (K2) and the rANS encoder (K5).

#include "cg_device.h"

#include <type_traits>

namespace cgk {
constexpr int kNT16 = 2;  // aux bits of a buffer load: non-temporal (single-use stream)
// Non-temporal (streaming) accesses for the encoder's single-use streams: the KV rows it
// reads once per pass, the symbols and anchors it writes once.  (On the 70B-shaped cache
// the encode went from 36.1 to 34.4 ms with them.)
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int nt_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ntload16(const void *p)
{
    const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void ntstore16(void *p, uint4 v)
{
    const nt_u32x4 t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<nt_u32x4 *>(p));
}
__device__ __forceinline__ void ntstore8(void *p, uint2 v)
{
    const nt_u32x2 t = {v.x, v.y};
    __builtin_nontemporal_store(t, reinterpret_cast<nt_u32x2 *>(p));
}


// x - a for the fp16 bits h of x, as one mixed-precision fma x * one + (-a) that reads h
// directly (one = 1.0 held in a register the compiler cannot see through, so the fma is
// not folded back into a conversion and a subtraction).  The product is exact, so the
// single rounding gives the fp32 difference bit for bit, signed zeros included.
__device__ __forceinline__ float delta_mix(uint32_t h, float one, float a)
{
    return fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)h), one, -a);
}
// 1.0f, opaque to the compiler
__device__ __forceinline__ float opaque_one()
{
    float one = 1.0f;
    asm volatile("" : "+v"(one));
    return one;
}

// ------------------------------------------------------------------------------ K0
// Per-channel min / max of the anchor deltas, and the non-finite flag; 16-byte loads,
// one row of C channels read by C/8 consecutive threads.
//
// A delta is the fp32 difference x - a of a token and its group's anchor, and rounding is
// monotone, so over the tokens of one group min(x - a) = min(x) - a (likewise max): the
// group's tokens are reduced as fp16 pairs (one packed min and one packed max per two
// channels) and only the group's extremes are converted and differenced.  That is exact
// for finite inputs; an input with an Inf or NaN is rejected through the flag, which
// collects x * 0 + acc per half (0 for every finite x, NaN from the first Inf or NaN on).
// Signed zeros may come out in another order than element by element; a zero bound is
// stored as +0 in any case.
__device__ __forceinline__ uint32_t pk_min_f16(uint32_t a, uint32_t b)
{
    uint32_t r;
    asm("v_pk_min_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ uint32_t pk_max_f16(uint32_t a, uint32_t b)
{
    uint32_t r;
    asm("v_pk_max_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
// acc + x * 0 per half: stays 0 while x is finite, NaN from the first Inf or NaN on
__device__ __forceinline__ uint32_t pk_nonfinite_acc(uint32_t acc, uint32_t x)
{
    uint32_t r;
    asm("v_pk_fma_f16 %0, %1, 0, %2" : "=v"(r) : "v"(x), "v"(acc));
    return r;
}

// Thread = (row, token stream tb, 8 channels): the thread takes the row's groups tb,
// tb + ntb, tb + 2 ntb, ... (group slots in chunk order, ngF per chunk), so the threads of a
// row read neighbouring groups at the same time (a window of ntb groups moving through the
// row) rather than each its own distant token range.
__global__ __launch_bounds__(256) void k0_minmax(const uint16_t *__restrict__ X, Geom g,
                                                  uint32_t ntb, uint32_t *__restrict__ ord_lo,
                                                  uint32_t *__restrict__ ord_hi,
                                                  uint32_t *__restrict__ flag)
{
    const uint32_t O = g.C / 8;
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (uint64_t)g.L * 2 * ntb * O) return;
    const uint32_t o = (uint32_t)(i % O);
    const uint64_t tmp = i / O;
    const uint32_t tb = (uint32_t)(tmp % ntb);
    const uint32_t row = (uint32_t)(tmp / ntb);
    const uint16_t *base = X + (uint64_t)row * g.S * g.C + o * 8;
    const uint64_t r0 = (uint64_t)row * g.C + o * 8;
    const uint32_t slots = (g.S + g.Tc - 1) / g.Tc * g.ngF;

    constexpr uint32_t kPosInf2 = 0x7C007C00u, kNegInf2 = 0xFC00FC00u;
    constexpr uint32_t kBatch = 9;   // tokens loaded together after a group's anchor
    float mn[8], mx[8];
    uint32_t nf[4] = {0u, 0u, 0u, 0u};  // the non-finite sums
    bool any = false;
    for (uint32_t j = tb; j < slots; j += ntb) {
        const uint32_t k = j / g.ngF, gi = j - k * g.ngF;
        const uint32_t cl = chunk_len(g, k);
        if (gi * g.G >= cl) continue;  // past the last group of a short last chunk
        const uint32_t t0 = k * g.Tc + gi * g.G, gl = min(g.G, cl - gi * g.G);
        const uint4 a = ntload16(base + (uint64_t)t0 * g.C);
        nf[0] = pk_nonfinite_acc(nf[0], a.x);
        nf[1] = pk_nonfinite_acc(nf[1], a.y);
        nf[2] = pk_nonfinite_acc(nf[2], a.z);
        nf[3] = pk_nonfinite_acc(nf[3], a.w);
        float af[8];
        unpack8(a, af);
        snap8(g, r0, af);
        uint32_t gmn[4], gmx[4];  // the group's fp16 min / max pairs
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            gmn[q] = kPosInf2;
            gmx[q] = kNegInf2;
        }
        bool gany = false;
        // the other tokens, kBatch at a time; loads past the group's end repeat its last
        // token, which changes neither the min / max nor the non-finite sums
        for (uint32_t u0 = 1; u0 < gl; u0 += kBatch) {
            uint4 v[kBatch];
#pragma unroll
            for (uint32_t b = 0; b < kBatch; ++b)
                v[b] = ntload16(base + (uint64_t)(t0 + min(u0 + b, gl - 1)) * g.C);
            const bool all_coded = t0 + u0 >= g.n_sink;  // else: sink tokens in the batch
#pragma unroll
            for (uint32_t b = 0; b < kBatch; ++b) {
                const uint32_t x[4] = {v[b].x, v[b].y, v[b].z, v[b].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) nf[q] = pk_nonfinite_acc(nf[q], x[q]);
                if (all_coded || t0 + min(u0 + b, gl - 1) >= g.n_sink) {  // sinks stay out
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        gmn[q] = pk_min_f16(gmn[q], x[q]);
                        gmx[q] = pk_max_f16(gmx[q], x[q]);
                    }
                    gany = true;
                }
            }
        }
        if (gany) {
            // the group's extremes into the fp32 range of deltas
            float hmn[8], hmx[8];
            unpack8(make_uint4(gmn[0], gmn[1], gmn[2], gmn[3]), hmn);
            unpack8(make_uint4(gmx[0], gmx[1], gmx[2], gmx[3]), hmx);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float dmn = hmn[q] - af[q], dmx = hmx[q] - af[q];
                mn[q] = (!any || dmn < mn[q]) ? dmn : mn[q];
                mx[q] = (!any || dmx > mx[q]) ? dmx : mx[q];
            }
            any = true;
        }
    }
    if (any) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            atomicMin(&ord_lo[r0 + q], f2ord(mn[q]));
            atomicMax(&ord_hi[r0 + q], f2ord(mx[q]));
        }
    }
    if (((nf[0] | nf[1] | nf[2] | nf[3]) & 0x7FFF7FFFu) != 0) atomicOr(flag, 1u);
}

// lo and hi per (row, channel) from the ordered min / max; a row with no coded token
// gets lo = hi = 0, and a zero bound is stored as +0.
__global__ __launch_bounds__(256) void k0_finalize(Geom g, const uint32_t *__restrict__ ord_lo,
                                                    const uint32_t *__restrict__ ord_hi,
                                                    float *__restrict__ lo, float *__restrict__ hi)
{
    uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= g.L * 2 * g.C) return;
    float a = 0.0f, b = 0.0f;
    if (ord_lo[i] != 0xFFFFFFFFu) {
        a = ord2f(ord_lo[i]);
        b = ord2f(ord_hi[i]);
    }
    lo[i] = a + 0.0f;  // a zero bound is +0
    hi[i] = b + 0.0f;
}

// w = (hi - lo) / (N - 1), r = 1 / w per (row, channel).
__global__ __launch_bounds__(256) void k_width(Geom g, const uint8_t *__restrict__ bins,
                                                const float *__restrict__ lo,
                                                const float *__restrict__ hi,
                                                float *__restrict__ w, float *__restrict__ r)
{
    uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= g.L * 2 * g.C) return;
    const uint32_t row = i / g.C;   // (layer, K/V) row
    const float ww = (hi[i] - lo[i]) / (float)(bins[row] - 1u);
    w[i] = ww;
    r[i] = (ww > 0.0f) ? 1.0f / ww : 0.0f;
}

// ------------------------------------------------------------------------------ outlier clip
// Sparse outlier table ("Guide to CacheGen", Solution pillar 3): each channel row's grid
// spans a central range chosen on the fine grid p_j = fma(j, wf, lo), wf = (hi - lo) / 256.
// The fine interval of a delta is the largest j in [0, 255] with p_j <= delta (0 if
// none): estimated from (delta - lo) / wf, then moved until exact (the points do not
// decrease with j).
__device__ __forceinline__ uint32_t fine_index(float dl, float lo, float wf, float rf)
{
    float e = floorf((dl - lo) * rf);
    e = fminf(fmaxf(e, 0.0f), (float)(kFineBins - 1u));
    uint32_t j = (uint32_t)e;
    while (j < kFineBins - 1u && fmaf((float)(j + 1u), wf, lo) <= dl) ++j;
    while (j > 0u && fmaf((float)j, wf, lo) > dl) --j;
    return j;
}

// Counts of the coded deltas in the fine intervals.  Block = 8 wavefronts over one
// (row, 64-channel block b, token part p); lane = channel; each wavefront takes an eighth
// of the part's tokens with 2-byte loads of its channel, kFineAhead rows in flight.  The
// LDS histogram holds two 16-bit counters per word, word (bin / 2, lane) at
// (bin / 2) * 65 + lane: one column per lane, so no two lanes of a wavefront update the
// same word, and a padding column puts a lane's word in bank (bin / 2 + lane) mod 64.
// 33 KiB per block lets 4 blocks (32 wavefronts) share a CU, enough 128-byte loads in
// flight to stream the cache.  A part holds at most 65535 tokens, so no counter
// overflows.  The block writes its counts to partial[p][row][c][256] (uint16, every bin);
// k_clip sums the parts.
constexpr uint32_t kFineCols = kLanes + 1;
constexpr uint32_t kFineWaves = 8;
constexpr int kFineAhead = 8;

template <bool A8>
__global__ __launch_bounds__(kFineWaves * 64) void k_fine_hist(const uint16_t *__restrict__ X, Geom g,
                                                                const float *__restrict__ lo,
                                                                const float *__restrict__ hi,
                                                                uint32_t parts,
                                                                uint16_t *__restrict__ partial)
{
    __shared__ uint32_t hist[kFineBins / 2 * kFineCols];
    const uint32_t p = blockIdx.x % parts;
    const uint32_t tmp = blockIdx.x / parts;
    const uint32_t b = tmp % g.NB;
    const uint32_t row = tmp / g.NB;
    for (uint32_t j = threadIdx.x; j < kFineBins / 2 * kFineCols; j += blockDim.x) hist[j] = 0;
    __syncthreads();

    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
    const uint32_t lane = threadIdx.x % kLanes;
    const uint32_t c = b * kLanes + lane;
    const bool present = c < g.C;
    const uint32_t per_part = (g.S + parts - 1) / parts;
    const uint32_t p0 = min(g.S, p * per_part), p1 = min(g.S, p0 + per_part);
    const uint32_t per_wave = (p1 - p0 + kFineWaves - 1) / kFineWaves;
    const uint32_t t_begin = min(p1, p0 + wave * per_wave), t_end = min(p1, t_begin + per_wave);
    const uint64_t ri = (uint64_t)row * g.C + (present ? c : 0u);
    if (t_begin < t_end) {
        const float l0 = lo[ri];
        const float wf = (hi[ri] - l0) / (float)kFineBins;
        const float rf = wf > 0.0f ? 1.0f / wf : 0.0f;
        // lanes without a channel or with a zero-width row count nothing (and take no
        // step in fine_index: a delta of -inf stays at interval 0)
        const bool counts = present && wf > 0.0f;
        float alo = 0.0f, aw = 0.0f, ar = 0.0f;
        if constexpr (A8) {
            alo = g.alo[ri];
            aw = g.aw[ri];
            ar = g.ar[ri];
        }
        const uint16_t *col = X + (uint64_t)row * g.S * g.C + (present ? c : 0u);
        auto load = [&](uint32_t t) __attribute__((always_inline)) {
            return __builtin_nontemporal_load(col + (uint64_t)t * g.C);
        };
        // position of token t: u in its chunk, gp in its group (wave-uniform), advanced
        // with selects rather than branches
        uint32_t t = t_begin, u = t_begin % g.Tc, gp = u % g.G;
        float af = 0.0f;
        if (gp != 0) {
            const float x = h2f(load(t_begin - gp));
            af = A8 ? anchor_snap(x, alo, aw, ar) : x;
        }
        uint16_t buf[kFineAhead];
#pragma unroll
        for (int k = 0; k < kFineAhead; ++k) buf[k] = load(min(t_begin + k, t_end - 1));
        // A batch of kFineAhead rows (all below t_end when `full`): the fine interval of
        // each delta from the estimate floor((delta - lo) / wf), which is exact when
        // p_e <= delta < p_(e+1) (at the ends: e = 0 or e = 255); otherwise, rarely, the
        // batch takes the stepping search.  Lanes that count nothing carry -inf.
        auto batch = [&](bool full) __attribute__((always_inline)) {
            float dl[kFineAhead];
            bool cnt[kFineAhead];
            uint32_t q[kFineAhead];
            uint64_t bad = 0;
#pragma unroll
            for (int k = 0; k < kFineAhead; ++k) {
                const bool in = full || t < t_end;
                const uint16_t v = buf[k];
                if (full) buf[k] = load(min(t + kFineAhead, t_end - 1));
                const float x = h2f(v);
                const bool anc = in && gp == 0;
                if constexpr (A8) {
                    if (anc) af = anchor_snap(x, alo, aw, ar);
                } else {
                    af = anc ? x : af;
                }
                cnt[k] = counts & in & !anc & (t >= g.n_sink);   // (no short circuit: no branch)
                float d = x - af;
                asm volatile("" : "+v"(d));
                dl[k] = cnt[k] ? d : -__builtin_inff();
                const float e = fminf(fmaxf(floorf((dl[k] - l0) * rf), 0.0f), (float)(kFineBins - 1u));
                const float p_e = fmaf(e, wf, l0), p_n = fmaf(e + 1.0f, wf, l0);
                const bool ok = ((e == 0.0f) | (p_e <= dl[k])) &
                                ((e == (float)(kFineBins - 1u)) | (p_n > dl[k]));
                bad |= __builtin_amdgcn_ballot_w64(!ok);
                q[k] = (uint32_t)e;
                if (in) {
                    ++t;
                    const bool wrap = ++u == g.Tc;
                    u = wrap ? 0u : u;
                    gp = (wrap || gp + 1u == g.G) ? 0u : gp + 1u;
                }
            }
            if (bad) {
#pragma unroll
                for (int k = 0; k < kFineAhead; ++k) q[k] = fine_index(dl[k], l0, wf, rf);
            }
#pragma unroll
            for (int k = 0; k < kFineAhead; ++k)
                atomicAdd(&hist[(q[k] >> 1) * kFineCols + lane], cnt[k] ? 1u << ((q[k] & 1u) * 16u) : 0u);
        };
        for (uint32_t n = (t_end - t_begin) / kFineAhead; n > 0; --n) batch(true);
        if (t < t_end) batch(false);
    }
    __syncthreads();
    // thread -> (one of two channels, bin): consecutive threads write consecutive bins
    const uint32_t nl = min(kLanes, g.C - b * kLanes);
    uint16_t *dst = partial + (((uint64_t)p * g.L * 2 + row) * g.C + b * kLanes) * kFineBins;
    const uint32_t bin = threadIdx.x % kFineBins;
    for (uint32_t ch = threadIdx.x / kFineBins; ch < nl; ch += blockDim.x / kFineBins)
        dst[(uint64_t)ch * kFineBins + bin] =
            (uint16_t)(hist[(bin >> 1) * kFineCols + ch] >> ((bin & 1u) * 16u));
}

// The central range of one channel row: with n coded deltas and the budget
// b = floor(n * ppm / 10^6), whole fine intervals are dropped from the bottom while the
// dropped count stays <= b, and from the top likewise; lo' = p_{j_lo},
// hi' = p_{j_hi + 1} (hi when j_hi = 255), at most hi.  lo and hi are narrowed in place.
// One wavefront per row element, lane i holding bins 4i .. 4i + 3 summed over the parts:
// with pre(j) = the count below interval j (non-decreasing in j), j_lo is the number of
// j in [1, 255] with pre(j) <= b, and 255 - j_hi the number with n - pre(j) <= b.
__global__ __launch_bounds__(256) void k_clip(Geom g, const uint16_t *__restrict__ partial,
                                               uint32_t parts, uint32_t ppm,
                                               float *__restrict__ lo, float *__restrict__ hi)
{
    const uint64_t rows = (uint64_t)g.L * 2 * g.C;
    const uint64_t i = (uint64_t)blockIdx.x * (blockDim.x / kLanes) + threadIdx.x / kLanes;
    const uint32_t lane = threadIdx.x % kLanes;
    if (i >= rows) return;
    const float l0 = lo[i], h0 = hi[i];
    const float wf = (h0 - l0) / (float)kFineBins;
    if (!(wf > 0.0f) || ppm == 0) return;
    uint32_t cnt[4] = {0u, 0u, 0u, 0u};
    for (uint32_t p = 0; p < parts; ++p) {
        const uint2 v = *reinterpret_cast<const uint2 *>(partial + ((uint64_t)p * rows + i) * kFineBins + 4 * lane);
        cnt[0] += v.x & 0xFFFFu;
        cnt[1] += v.x >> 16;
        cnt[2] += v.y & 0xFFFFu;
        cnt[3] += v.y >> 16;
    }
    const uint32_t mine = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    // inclusive scan of the lane sums
    uint32_t incl = mine;
#pragma unroll
    for (uint32_t d = 1; d < kLanes; d <<= 1) {
        const uint32_t y = __shfl_up(incl, d, kLanes);
        if (lane >= d) incl += y;
    }
    const uint32_t n = __shfl(incl, kLanes - 1, kLanes);
    if (n == 0) return;
    const uint64_t budget = ((uint64_t)n * ppm) / 1000000u;
    uint32_t pre = incl - mine, n_lo = 0, n_hi = 0;
#pragma unroll
    for (uint32_t k = 0; k < 4; ++k) {
        if (4 * lane + k >= 1) {
            n_lo += pre <= budget ? 1u : 0u;
            n_hi += (uint64_t)(n - pre) <= budget ? 1u : 0u;
        }
        pre += cnt[k];
    }
#pragma unroll
    for (uint32_t d = kLanes / 2; d >= 1; d >>= 1) {
        n_lo += __shfl_xor(n_lo, d, kLanes);
        n_hi += __shfl_xor(n_hi, d, kLanes);
    }
    if (lane != 0) return;
    const uint32_t j_lo = n_lo, j_hi = kFineBins - 1u - n_hi;
    const float lo_c = fmaf((float)j_lo, wf, l0);
    float hi_c = (j_hi == kFineBins - 1u) ? h0 : fmaf((float)(j_hi + 1u), wf, l0);
    if (hi_c > h0) hi_c = h0;
    lo[i] = lo_c + 0.0f;
    hi[i] = hi_c + 0.0f;
}

// ------------------------------------------------------------------------------ K1
// Fused delta -> quantize -> histogram.  Block = (row, tile of 8*OCT channels, set of
// SUB token streams); its SUB x OCT threads each own 8 channels of one stream, which takes
// every NS-th group of the row (NS = streams per row), so that a row's blocks read
// neighbouring groups at the same time.  Counts go to an LDS histogram [N/2][8][OCT] of
// 16-bit counter pairs (bins 2m and 2m + 1 in one word; consecutive lanes -> consecutive
// banks; half the LDS of 32-bit counters, so more blocks are resident), then the non-zero
// bins are added to the global u32 counts.
__global__ __launch_bounds__(256) void k1_hist(const uint16_t *__restrict__ X, Geom g,
                                                const uint8_t *__restrict__ bins,
                                                const float *__restrict__ lo,
                                                const float *__restrict__ r, uint32_t OCT,
                                                uint32_t SUB, uint32_t ntiles,
                                                uint32_t ntb, uint32_t *__restrict__ counts)
{
    extern __shared__ uint32_t hist[];
    uint32_t tbb = blockIdx.x % ntb;
    uint32_t tmp = blockIdx.x / ntb;
    uint32_t ct = tmp % ntiles;
    uint32_t row = tmp / ntiles;
    uint32_t N = bins[row];
    const float nm1 = (float)(N - 1u);
    // counters of bins 2m and 2m + 1 share a word (16 bits each: a block counts fewer
    // than 2^16 tokens per channel)
    uint32_t nh = (N + 1) / 2 * 8 * OCT;
    for (uint32_t j = threadIdx.x; j < nh; j += blockDim.x) hist[j] = 0;
    __syncthreads();

    const uint32_t O = g.C / 8;
    uint32_t ol = threadIdx.x % OCT, sub = threadIdx.x / OCT;
    uint32_t o = ct * OCT + ol;
    if (sub < SUB && o < O) {
        const uint16_t *base = X + (uint64_t)row * g.S * g.C + o * 8;
        float lo8[8], r8[8], af[8];
        uint64_t r0 = (uint64_t)row * g.C + o * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            lo8[j] = lo[r0 + j];
            r8[j] = r[r0 + j];
        }
        // byte offset of the counter word of (bin pair m, channel j):
        // 4 (m * 8 OCT + j OCT + ol), with 4 m * 8 OCT = (q & ~1) * 16 OCT for q = 2m or 2m + 1
        const uint32_t pair_bytes = 16 * OCT;
        uint32_t hb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) hb[j] = 4 * (j * OCT + ol);
        const float one = opaque_one();
        // the stream's groups: slots st, st + NS, st + 2 NS, ... of the row (as in the range
        // pass, so that the blocks of a row read neighbouring groups at the same time)
        const uint32_t NS = ntb * SUB, st = tbb * SUB + sub;
        const uint32_t slots = (g.S + g.Tc - 1) / g.Tc * g.ngF;
        constexpr uint32_t kBatch = 9;   // tokens loaded together after a group's anchor
        for (uint32_t j = st; j < slots; j += NS) {
            const uint32_t k = j / g.ngF, gi = j - k * g.ngF;
            const uint32_t cl = chunk_len(g, k);
            if (gi * g.G >= cl) continue;  // past the last group of a short last chunk
            const uint32_t t0 = k * g.Tc + gi * g.G, gl = min(g.G, cl - gi * g.G);
            unpack8(ntload16(base + (uint64_t)t0 * g.C), af);
            snap8(g, r0, af);
            for (uint32_t u0 = 1; u0 < gl; u0 += kBatch) {
                uint4 v[kBatch];
#pragma unroll
                for (uint32_t b = 0; b < kBatch; ++b)
                    v[b] = ntload16(base + (uint64_t)(t0 + min(u0 + b, gl - 1)) * g.C);
#pragma unroll
                for (uint32_t b = 0; b < kBatch; ++b) {
                    // tokens of the group only, and from n_sink on (sinks stay out)
                    if (u0 + b >= gl || t0 + u0 + b < g.n_sink) continue;
                    const uint32_t x[4] = {v[b].x, v[b].y, v[b].z, v[b].w};
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        const uint32_t h = (c & 1) ? x[c / 2] >> 16 : x[c / 2] & 0xFFFFu;
                        const uint32_t q = quantize_bf(delta_mix(h, one, af[c]), lo8[c], r8[c], nm1);
                        uint32_t *cw = reinterpret_cast<uint32_t *>(
                            reinterpret_cast<char *>(hist) + __umul24(q & ~1u, pair_bytes) + hb[c]);
                        atomicAdd(cw, 1u << (16 * (q & 1u)));
                    }
                }
            }
        }
    }
    __syncthreads();
    for (uint32_t j = threadIdx.x; j < nh; j += blockDim.x) {
        uint32_t v = hist[j];
        if (!v) continue;
        uint32_t m = j / (8 * OCT), rem = j - m * 8 * OCT;
        uint32_t jj = rem / OCT, oo = ct * OCT + rem % OCT;
        if (oo >= O) continue;
        uint32_t *cnt = &counts[((uint64_t)row * g.C + oo * 8 + jj) * kMaxBins + 2 * m];
        if (v & 0xFFFFu) atomicAdd(cnt, v & 0xFFFFu);
        if (v >> 16) atomicAdd(cnt + 1, v >> 16);
    }
}

// Frequencies of one (row, channel): T = 256, f[s] = 1 + floor(count[s] * (T - N) / n),
// the remainder to the most frequent symbol (lowest index among equals).
__global__ __launch_bounds__(256) void k1_freqs(Geom g, const uint8_t *__restrict__ bins,
                                                 const uint32_t *__restrict__ counts,
                                                 uint16_t *__restrict__ freqs)
{
    uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= g.L * 2 * g.C) return;
    uint32_t row = i / g.C;
    uint32_t N = bins[row];
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
    for (uint32_t s = 0; s < kMaxBins; ++s)
        freqs[(uint64_t)i * kMaxBins + s] = (uint16_t)((s < N) ? f[s] : 0u);
}

// The coder tables of one (row, channel) from its frequencies (each >= 1, sum 256) and
// grid: the {f | cdf << 24} plane, the dequantized deltas fma(s, w, lo), and the slot
// table.
__global__ __launch_bounds__(256) void k_dtab(Geom g, const uint8_t *__restrict__ bins,
                                               const uint16_t *__restrict__ freqs,
                                               const float *__restrict__ lo,
                                               const float *__restrict__ w,
                                               uint32_t *__restrict__ dtab)
{
    uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= g.L * 2 * g.C) return;
    uint32_t row = i / g.C, c = i - row * g.C;
    uint32_t N = bins[row];
    uint32_t f[kMaxBins];
    for (uint32_t s = 0; s < kMaxBins; ++s) f[s] = (s < N) ? freqs[(uint64_t)i * kMaxBins + s] : 0u;
    float lo1 = lo[i], w1 = w[i];
    uint32_t *tb = dtab + (uint64_t)(row * g.NB + c / kLanes) * kTabBlock + (c % kLanes);
    uint32_t cdf = 0;
    for (uint32_t s = 0; s < kMaxBins; ++s) {
        // (f <= 255 and cdf <= 255 since N >= 2; symbols >= N are never looked up)
        tb[(uint64_t)s * kLanes] = (s < N) ? f[s] | (cdf << 24) : 0u;
        tb[kTabPlane + (uint64_t)s * kLanes] =
            __float_as_uint(fmaf((float)min(s, N - 1u), w1, lo1));
        cdf += f[s];
    }
    // slot table: every slot in [cdf[s], cdf[s] + f[s]) names s; the byte of (slot, lane)
    // is at 256 (slot / 4) + 4 lane + slot mod 4, so each lane's slots share its own
    // 4-byte column and 64 lanes reading any slots hit 64 different dwords of one row
    // each in its own bank
    uint8_t *lut = reinterpret_cast<uint8_t *>(dtab + (uint64_t)(row * g.NB + c / kLanes) * kTabBlock +
                                               kTabLut) + 4 * (c % kLanes);
    uint32_t s = 0, end = f[0];
    for (uint32_t slot = 0; slot < kProbTotal; ++slot) {
        while (slot >= end && s + 1 < kMaxBins) end += f[++s];
        lut[(slot >> 2) * (4 * kLanes) + (slot & 3u)] = (uint8_t)s;
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
                                                       uint16_t *__restrict__ anchors,
                                                       unsigned long long *__restrict__ clamped)
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
    uint32_t N = bins[row];
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
        snap8(g, (uint64_t)row * g.C + o * 8, af);
    }
    uint32_t n_off = 0;  // elements off their grid (counted from token n_sink on)
    for (; w.t < t_end; w.next(g)) {
        uint4 v = ntload16(base + (uint64_t)w.t * g.C);
        uint2 packed = make_uint2(0, 0);
        float xf[8];
        unpack8(v, xf);
        const bool coded = w.t >= g.n_sink;
        if (w.gp == 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j) af[j] = xf[j];
            if (g.alo) {
                // 8-bit anchors: the codes go to the container, their grid values anchor
                // the deltas
                const uint64_t r0 = (uint64_t)row * g.C + o * 8;
                uint32_t cd[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    n_off += (coded && off_grid(af[j], g.alo[r0 + j], g.ar[r0 + j], 256u)) ? 1u : 0u;
                    cd[j] = quantize1(af[j], g.alo[r0 + j], g.ar[r0 + j], 256u);
                    af[j] = h2f(f2h_fma((float)cd[j], g.aw[r0 + j], g.alo[r0 + j]));
                }
                if (anchors) {
                    uint8_t *a8 = reinterpret_cast<uint8_t *>(anchors);
                    const uint2 pk = make_uint2(cd[0] | (cd[1] << 8) | (cd[2] << 16) | (cd[3] << 24),
                                                cd[4] | (cd[5] << 8) | (cd[6] << 16) | (cd[7] << 24));
                    ntstore8(a8 + anchor_row(g, w.k, row, w.gi) * g.C + o * 8, pk);
                }
            } else if (anchors) {
                uint64_t ar = anchor_row(g, w.k, row, w.gi);
                ntstore16(anchors + ar * g.C + o * 8, v);
            }
        } else {
            uint32_t q[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                q[j] = quantize1(xf[j] - af[j], lo8[j], r8[j], N);
                n_off += (coded && off_grid(xf[j] - af[j], lo8[j], r8[j], N)) ? 1u : 0u;
            }
            packed.x = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
            packed.y = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
        }
        ntstore8(sbase + (uint64_t)(w.t - sym_t0) * g.C, packed);
    }
    if (clamped && n_off) atomicAdd(clamped, (unsigned long long)n_off);
}

// ------------------------------------------------------------------------------ outliers
// The outlier entries of one group (chunk, row, channel block b) per wavefront, lane =
// channel: tokens in ascending order, from n_sink on, each element tested against its
// grid as the quantizer sees it (the delta against the anchor's decoded value; with
// 8-bit anchors the anchor's own code against the anchor grid).  Counting pass: the
// group's number of entries.  Writing pass: entry e of the group at offs[gidx] + e,
// key (token within the chunk) << 6 | lane, value the element's fp16 bits; a token's
// entries are placed in lane order by a ballot.  Rows are loaded kOutAhead ahead and
// tested without branches (the quantizer's clamp changed floor(fma(delta - lo, r, 0.5)),
// or a zero-width grid misses delta); only a row with an entry takes the writing branch.
constexpr int kOutAhead = 8;
template <bool B> struct BoolTag {
    static constexpr bool value = B;
};

template <bool WRITE, bool A8>
__global__ __launch_bounds__(256) void k_outliers(const uint16_t *__restrict__ X, Geom g,
                                                   const uint8_t *__restrict__ bins,
                                                   const float *__restrict__ lo,
                                                   const float *__restrict__ r,
                                                   uint64_t n_groups, uint64_t *__restrict__ counts,
                                                   const uint64_t *__restrict__ offs,
                                                   uint32_t *__restrict__ keys,
                                                   uint16_t *__restrict__ vals)
{
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
    const uint64_t gidx = (uint64_t)blockIdx.x * (blockDim.x / kLanes) + wave;
    if (gidx >= n_groups) return;
    const uint32_t lane = threadIdx.x % kLanes;
    const uint32_t b = (uint32_t)(gidx % g.NB);
    const uint64_t tmp = gidx / g.NB;
    const uint32_t row = (uint32_t)(tmp % (2 * g.L));
    const uint32_t k = g.kb + (uint32_t)(tmp / (2 * g.L));
    const uint32_t c = b * kLanes + lane;
    const bool present = c < g.C;
    const uint32_t t0 = k * g.Tc, len = chunk_len(g, k);
    const float nm1 = (float)(bins[row] - 1u);
    const uint64_t ri = (uint64_t)row * g.C + (present ? c : 0u);
    const float lo1 = lo[ri], r1 = r[ri];
    float alo = 0.0f, aw = 0.0f, ar = 0.0f;
    if constexpr (A8) {
        alo = g.alo[ri];
        aw = g.aw[ri];
        ar = g.ar[ri];
    }
    // the row parameters are waited for here: a wait at their first use inside the row
    // loop would also drain the rows loaded ahead, every iteration
    asm volatile("" ::"v"(lo1), "v"(r1), "v"(alo), "v"(aw), "v"(ar));
    const uint64_t pmask = __builtin_amdgcn_ballot_w64(present);
    const uint64_t zmask = __builtin_amdgcn_ballot_w64(r1 == 0.0f);   // zero-width grids
    const uint64_t azmask = __builtin_amdgcn_ballot_w64(ar == 0.0f);  // (8-bit anchors)
    // Each lane loads the aligned 4 bytes holding its channel (channel pairs share them)
    // and shifts its half down: 16-bit values would be packed or masked at the end of
    // every batch, which waits for the rows loaded ahead.  The rows come through a
    // buffer resource over the chunk: the row offset advances in a scalar register and
    // rows past the chunk read 0.
    const __amdgpu_buffer_rsrc_t xs =
        make_rsrc(X + ((uint64_t)row * g.S + t0) * g.C, (uint32_t)((uint64_t)len * g.C * 2));
    const uint32_t voff = 2 * ((present ? c : 0u) & ~1u);
    const uint32_t rstride = 2 * g.C;
    const uint32_t half = 16u * (lane & 1u);
    auto load = [&](uint32_t soff) __attribute__((always_inline)) {
        return __builtin_amdgcn_raw_buffer_load_b32(xs, voff, soff, kNT16);
    };
    // lanes off the grid l + q / rr (q in [0, n]) for x
    auto off_mask = [&](float x, float l, float rr, float n, uint64_t zm) __attribute__((always_inline)) {
        const float v = floorf(fmaf(x - l, rr, 0.5f));
        const float vc = __builtin_amdgcn_fmed3f(v, 0.0f, n);
        return __builtin_amdgcn_fcmpf(v, vc, 14 /* unordered or not equal */) |
               (zm & __builtin_amdgcn_fcmpf(x, l, 14));
    };
    // rows from u_sink on are coded (the sinks before it are not)
    const uint32_t u_sink = g.n_sink > t0 ? min(g.n_sink - t0, len) : 0u;
    uint64_t run = WRITE ? offs[gidx] : 0;
    float af = 0.0f;
    uint32_t u = 0, gp = 0, soff = 0;
    uint32_t buf[kOutAhead];
#pragma unroll
    for (int j = 0; j < kOutAhead; ++j) buf[j] = load(j * rstride);
    // a batch of kOutAhead rows (all inside the chunk when FULL); ZW: some lane's grid has
    // zero width
    auto batch = [&](auto full_tag, auto zw_tag) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full_tag)::value, ZW = decltype(zw_tag)::value;
        uint64_t m[kOutAhead];
        uint32_t x[kOutAhead];
        uint32_t uu[kOutAhead];
        uint64_t any = 0;
#pragma unroll
        for (int j = 0; j < kOutAhead; ++j) {
            const bool in = FULL || u < len;
            x[j] = buf[j] >> half;
            if (FULL) buf[j] = load(soff + kOutAhead * rstride);
            const float xf = h2f(x[j] & 0xFFFFu);
            const bool anc = gp == 0;
            uint64_t ma = 0;   // an anchor: off its own grid (8-bit anchors only)
            if constexpr (A8) {
                ma = off_mask(xf, alo, ar, 255.0f, azmask);
                if (anc) af = anchor_snap(xf, alo, aw, ar);
            } else {
                af = anc ? xf : af;
            }
            float d = xf - af;
            asm volatile("" : "+v"(d));
            const float v = floorf(fmaf(d - lo1, r1, 0.5f));
            const float vc = __builtin_amdgcn_fmed3f(v, 0.0f, nm1);
            uint64_t mn = __builtin_amdgcn_fcmpf(v, vc, 14 /* unordered or not equal */);
            if constexpr (ZW) mn |= zmask & __builtin_amdgcn_fcmpf(d, lo1, 14);
            m[j] = (in & (u >= u_sink)) ? (anc ? ma : mn) & pmask : 0;
            uu[j] = u;
            any |= m[j];
            if (in) {
                ++u;
                soff += rstride;
                gp = gp + 1u == g.G ? 0u : gp + 1u;
            }
        }
        // only a batch with an entry moves the group's entry count
        if (any) {
#pragma unroll
            for (int j = 0; j < kOutAhead; ++j) {
                if (WRITE && ((m[j] >> lane) & 1u)) {
                    const uint64_t e = run + mbcnt64(m[j]);
                    keys[e] = (uu[j] << 6) | lane;
                    vals[e] = (uint16_t)x[j];
                }
                run += (uint64_t)__builtin_popcountll(m[j]);
            }
        }
    };
    auto rows = [&](auto zw_tag) __attribute__((always_inline)) {
        for (uint32_t n = len / kOutAhead; n > 0; --n) batch(BoolTag<true>{}, zw_tag);
        if (u < len) batch(BoolTag<false>{}, zw_tag);
    };
    if (zmask)
        rows(BoolTag<true>{});
    else
        rows(BoolTag<false>{});
    if (!WRITE && lane == 0) counts[gidx] = run;
}

// 8-bit anchor grid ("Guide to CacheGen", Solution pillar 2: the anchor is quantized with
// high precision): per (layer, K/V, channel) row, min / max of its anchor tokens over all
// chunks, width (max - min) / 255, zero bounds as +0.  Block = 16 wavefronts over one
// (row, 64-channel block), lane = channel; wavefront p takes anchors p, p + 16, ... (anchor
// a is token (a / ngF) Tc + (a % ngF) G: every chunk but the last is full), 8 loads in
// flight; the 16 partial ranges meet in LDS.
constexpr uint32_t kGridWaves = 16;

__global__ __launch_bounds__(kGridWaves * 64) void k_anchor_grid(const uint16_t *__restrict__ X, Geom g,
                                                                  float *__restrict__ alo,
                                                                  float *__restrict__ aw,
                                                                  float *__restrict__ ar)
{
    __shared__ float plo[kGridWaves][kLanes], phi[kGridWaves][kLanes];
    const uint32_t b = blockIdx.x % g.NB, row = blockIdx.x / g.NB;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
    const uint32_t lane = threadIdx.x % kLanes;
    const uint32_t c = b * kLanes + lane;
    const bool present = c < g.C;
    const uint16_t *base = X + (uint64_t)row * g.S * g.C + (present ? c : 0u);
    const uint32_t nk = (g.S + g.Tc - 1) / g.Tc;
    const uint32_t n_anchor = (nk - 1) * g.ngF + (g.S - (nk - 1) * g.Tc + g.G - 1) / g.G;
    auto token = [&](uint32_t a) __attribute__((always_inline)) {
        return (a / g.ngF) * g.Tc + (a % g.ngF) * g.G;
    };
    float lo = __builtin_inff(), hi = -__builtin_inff();
    constexpr uint32_t A = 8;
    uint32_t a = wave;
    for (; a + (A - 1) * kGridWaves < n_anchor; a += A * kGridWaves) {
        uint16_t v[A];
#pragma unroll
        for (uint32_t j = 0; j < A; ++j) v[j] = base[(uint64_t)token(a + j * kGridWaves) * g.C];
#pragma unroll
        for (uint32_t j = 0; j < A; ++j) {
            const float x = h2f(v[j]);
            lo = x < lo ? x : lo;
            hi = x > hi ? x : hi;
        }
    }
    for (; a < n_anchor; a += kGridWaves) {
        const float x = h2f(base[(uint64_t)token(a) * g.C]);
        lo = x < lo ? x : lo;
        hi = x > hi ? x : hi;
    }
    plo[wave][lane] = lo;
    phi[wave][lane] = hi;
    __syncthreads();
    if (wave != 0 || !present) return;
#pragma unroll
    for (uint32_t p = 1; p < kGridWaves; ++p) {
        lo = plo[p][lane] < lo ? plo[p][lane] : lo;
        hi = phi[p][lane] > hi ? phi[p][lane] : hi;
    }
    lo = lo + 0.0f;
    hi = hi + 0.0f;
    const float w = (hi - lo) / 255.0f;
    const uint64_t i = (uint64_t)row * g.C + c;
    alo[i] = lo;
    aw[i] = w;
    ar[i] = (w > 0.0f) ? 1.0f / w : 0.0f;
}

hipError_t launch_anchor_grid(const uint16_t *X, const Geom &g, float *alo, float *aw, float *ar,
                              hipStream_t st)
{
    const uint64_t blocks = (uint64_t)g.L * 2 * g.NB;
    hipLaunchKernelGGL(k_anchor_grid, dim3((uint32_t)blocks), dim3(kGridWaves * 64), 0, st, X, g,
                       alo, aw, ar);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------ K5
// rANS encoder fused with anchor delta + quantize, one pass over the cache.  Block = 8
// wavefronts = 8 chunks of one (row, channel block b) sharing the block's coding table in
// LDS; wavefront = group (chunk, row, b), lane i codes the stream of channel 64b + i.
//
// The coder runs from a chunk's last symbol to its first, and the lockstep decoders read
// the words in the order "state words, then after each symbol the words of the lanes that
// renormalise, in lane order".  So the words of symbol i are the ones closest to the end
// of the group's word sequence among those not yet placed: every word is placed at its
// distance D from the end, D = (words of later symbols) + (words of symbol i) - rank of
// the lane among the shifting lanes, and the state words last.  The words go to a
// per-wavefront LDS ring indexed by -D and leave it 256 at a time (one 8-byte store per
// lane) into a region of the group's worst-case size, counted back from the region's end;
// a compaction copy then packs the regions into the container's payload.  Lanes that do
// not shift write a parking slot of their own, so the step has no branch.
//
// Coding step on symbol s with f = f[s], cdf = cdf[s] (state x in [2^16, 2^32)):
//   if x >= f * 2^24, the low 16 bits of x leave as a word and x >>= 16 (now x < f * 2^24);
//   q = floor(x / f); x = q * 256 + (x - q f) + cdf = x + q (256 - f) + cdf.
// q is taken as trunc(double(x) * rcp) with rcp = (1/f)(1 + 2^-40) rounded to double:
// the product exceeds x/f by a relative 2^-40 - 4 * 2^-53 > 0, so it is at least q, and by
// less than x/f * 2^-39 < 1/f (x < 2^39), so it stays below q + 1 - 1/f + 1/f.
//
// The chunk's tokens are visited group by group from the last group to the first; in a
// group the anchor first (it anchors the group's deltas, and goes to the anchors section),
// then the other tokens from the last to the first.  Groups of 10 tokens (the usual
// anchor interval) are unrolled: their 9 symbols and table reads are independent of the
// state and come first, the state chain follows, and the next group's rows are loaded
// meanwhile; other lengths go one token at a time.
constexpr uint32_t kEncWaves = 8;
constexpr uint32_t kWordRing = 1024;    // words per wavefront ring (power of two)
constexpr uint32_t kRingAlloc = kWordRing + kLanes;  // + one parking slot per lane
constexpr uint32_t kFlushWords = 256;   // words per flush: 4 per lane
constexpr uint32_t kUG = 10;            // group length of the unrolled path

typedef uint64_t __attribute__((may_alias)) ring_u64_t;

struct EncEntry {
    double rcp;        // (1/f)(1 + 2^-40)
    uint32_t f24;      // f << 24: renormalisation threshold
    uint32_t pk;       // (256 - f) | cdf << 24
};

// State of one wavefront's coder: the lane's channel parameters, the rANS state, and the
// placement of words (all counts wave-uniform).
struct Coder {
    const EncEntry *tab;
    uint16_t *ring;
    uint16_t *rend;         // end of the group's region
    float lo, r, nmax, af;  // grid, the largest float below N, the current anchor value
    bool zero_w;            // the grid is the single point lo
    bool present;           // this lane has a channel
    uint64_t pmask;         // lanes with a channel
    uint64_t zmask;         // lanes whose grid is the single point lo
    uint32_t lane, x, E, flushed, n_off;

    // q = clamp(floor(fma(delta - lo, r, 0.5)), 0, N - 1) without branches (a median and a
    // truncating conversion give quantize1's result); off: the clamp changed v,
    // or a zero-width grid misses delta (tested only with ZW: some lane of the wavefront
    // has a zero-width grid).  `coded`: the token is from n_sink on.  The off-grid lanes
    // come straight from the compares' lane masks (a ballot of a combined bool would
    // first be materialised as 0 / 1 and compared again).
    template <bool ZW>
    __device__ __forceinline__ uint32_t symbol(float dl, bool coded)
    {
        uint64_t om;
        const uint32_t q = symbol_mask<ZW>(dl, om);
        n_off += coded ? (uint32_t)__builtin_popcountll(om & pmask) : 0u;
        return q;
    }

    // The same, with the off-grid lanes returned in om rather than counted.
    template <bool ZW>
    __device__ __forceinline__ uint32_t symbol_mask(float dl, uint64_t &om) const
    {
        // v before its floor: floor(v) lies in [0, N - 1] exactly when v lies in
        // [0, nmax], so the clamp to [0, nmax] changes v exactly when floor(v) is off the
        // grid, and the truncating conversion of the clamped value is floor(v) clamped
        const float v = fmaf(dl - lo, r, 0.5f);
        const float vc = __builtin_amdgcn_fmed3f(v, 0.0f, nmax);
        om = __builtin_amdgcn_fcmpf(v, vc, 14 /* unordered or not equal */);
        if constexpr (ZW) om |= zmask & __builtin_amdgcn_fcmpf(dl, lo, 14);
        return (uint32_t)vc;
    }

    __device__ __forceinline__ EncEntry entry(uint32_t q) const { return tab[q * kLanes + lane]; }

    // One coding step with the table entry of the symbol; the shifted-out word (if any)
    // goes to the ring at its distance from the end, other lanes write their parking slot.
    // The ring index is computed for every lane and then selected (kept opaque so that the
    // select is not turned into a branch around the lane-count arithmetic).
    __device__ __forceinline__ void step(const EncEntry &en)
    {
        const uint64_t mask = __builtin_amdgcn_uicmp(x, en.f24, 35 /* unsigned >= */) & pmask;
        E += (uint32_t)__builtin_popcountll(mask);
        // distance from the end D = E - rank; the ring is indexed by -D
        uint32_t at = (mbcnt64(mask) - E) & (kWordRing - 1);
        asm volatile("" : "+v"(at));
        const bool mine = (x >= en.f24) & present;
        ring[mine ? at : kWordRing + lane] = (uint16_t)x;
        x = mine ? x >> 16 : x;
        const uint32_t qq = (uint32_t)((double)x * en.rcp);
        // x + q (256 - f) in one 24-bit multiply-add, then + cdf taken as byte 3 of pk
        const uint32_t t = __umul24(qq, en.pk) + x;
        asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
            "src1_sel:BYTE_3"
            : "=v"(x)
            : "v"(t), "v"(en.pk));
    }

    // writes out whole 256-word blocks of placed words (distances flushed + 1 ..): region
    // words [end - flushed - 256, end - flushed), 4 per lane
    __device__ __forceinline__ void flush()
    {
        while (E - flushed >= kFlushWords) {
            const uint32_t s0 = (0u - (flushed + kFlushWords) + 4 * lane) & (kWordRing - 1);
            const uint64_t w4 = *reinterpret_cast<const ring_u64_t *>(ring + s0);
            *reinterpret_cast<uint64_t *>(rend - flushed - kFlushWords + 4 * lane) = w4;
            flushed += kFlushWords;
        }
    }
};

template <uint32_t GU>
__global__ __launch_bounds__(kEncWaves * 64) void k5_code(const uint16_t *__restrict__ X, Geom g,
                                                         const uint8_t *__restrict__ bins,
                                                         const uint32_t *__restrict__ dtab,
                                                         const float *__restrict__ lo,
                                                         const float *__restrict__ r,
                                                         uint32_t n_sets, uint64_t region_words,
                                                         uint16_t *__restrict__ regions,
                                                         uint8_t *__restrict__ anchors,
                                                         uint64_t *__restrict__ group_words,
                                                         uint64_t *__restrict__ group_off_grid)
{
    __shared__ EncEntry tab[kMaxBins * kLanes];
    __shared__ __attribute__((aligned(16))) uint16_t rings[kEncWaves * kRingAlloc];
    // block order as in the decoder: channel block fastest, rotated by the row
    const uint32_t tmp = blockIdx.x / g.NB;
    const uint32_t set = tmp % n_sets;
    const uint32_t row = tmp / n_sets;
    const uint32_t b = (blockIdx.x % g.NB + row) % g.NB;
    const uint32_t N = bins[row];
    {
        const uint32_t *src = dtab + (uint64_t)(row * g.NB + b) * kTabBlock;
        for (uint32_t j = threadIdx.x; j < N * kLanes; j += blockDim.x) {
            const uint32_t e = src[j];
            const uint32_t f = max(e & 0xFFu, 1u), cdf = e >> 24;  // (absent lanes: f = 1)
            EncEntry en;
            en.rcp = (1.0 / (double)f) * (1.0 + 0x1p-40);
            en.f24 = f << 24;
            en.pk = (kProbTotal - f) | (cdf << 24);
            tab[j] = en;
        }
    }
    __syncthreads();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
    const uint32_t k = g.kb + set * kEncWaves + wave;
    if (k >= g.ke) return;
    const uint32_t lane = threadIdx.x % kLanes;
    const uint64_t gidx = ((uint64_t)(k - g.kb) * 2 * g.L + row) * g.NB + b;
    const uint32_t c = b * kLanes + lane;
    const uint32_t nl = min(kLanes, g.C - b * kLanes);
    const bool present = lane < nl;
    const uint32_t t0 = k * g.Tc, len = chunk_len(g, k);
    const uint32_t G = GU ? GU : g.G;
    const uint32_t ng = (len + G - 1) / G, m = len - ng;
    const uint64_t ri = (uint64_t)row * g.C + (present ? c : 0u);
    const bool a8 = g.alo != nullptr;
    float alo = 0.0f, aw = 0.0f, ar = 0.0f;
    if (a8) {
        alo = g.alo[ri];
        aw = g.aw[ri];
        ar = g.ar[ri];
    }
    Coder cd;
    cd.tab = tab;
    cd.ring = rings + wave * kRingAlloc;
    cd.rend = regions + (gidx + 1) * region_words;
    cd.lo = lo[ri];
    cd.r = r[ri];
    cd.nmax = __uint_as_float(__float_as_uint((float)N) - 1u);
    cd.zero_w = cd.r == 0.0f;
    cd.af = 0.0f;
    cd.present = present;
    cd.pmask = __builtin_amdgcn_ballot_w64(present);
    cd.zmask = __builtin_amdgcn_ballot_w64(cd.zero_w);
    cd.lane = lane;
    cd.x = kStateLow;
    cd.E = cd.flushed = cd.n_off = 0;

    // the chunk's rows of this (layer, K/V): token u at byte u * 2C, channel at 2c
    const __amdgpu_buffer_rsrc_t xs = make_rsrc(X + ((uint64_t)row * g.S + t0) * g.C,
                                                (uint32_t)((uint64_t)len * g.C * 2));
    const float one = opaque_one();
    const uint32_t voff = 2 * (present ? c : 0u);
    const uint32_t rstride = 2 * g.C;
    const uint64_t arow0 = anchor_row(g, k, row, 0);   // anchor row of group gi: arow0 + gi
    auto load = [&](uint32_t u) __attribute__((always_inline)) {
        return __builtin_amdgcn_raw_buffer_load_b16(xs, voff, u * rstride, kNT16);
    };
    // an anchor: its decoded value anchors the group; its fp16 bits or grid code go to
    // the anchors section
    auto anchor = [&](uint32_t v, uint32_t gi) __attribute__((always_inline)) {
        const float xa = h2f(v);
        const uint64_t ai = (arow0 + gi) * g.C + c;
        if (a8) {
            const uint32_t code = quantize1(xa, alo, ar, 256u);
            const bool off = off_grid(xa, alo, ar, 256u);
            const uint64_t om = __builtin_amdgcn_ballot_w64(off) & cd.pmask;
            cd.n_off += (t0 + gi * G >= g.n_sink) ? (uint32_t)__builtin_popcountll(om) : 0u;
            cd.af = h2f(f2h_fma((float)code, aw, alo));
            if (present) anchors[ai] = (uint8_t)code;
        } else {
            cd.af = xa;
            if (present) reinterpret_cast<uint16_t *>(anchors)[ai] = (uint16_t)v;
        }
    };
    // The coding loop, compiled twice: with the zero-width grid test (some lane's grid is
    // the single point lo) and without it, so the usual case takes no per-symbol branch.
    auto code_chunk = [&](auto zw) __attribute__((always_inline)) {
        constexpr bool ZW = decltype(zw)::value;
        // any group, one token at a time (its last token first)
        auto group_generic = [&](uint32_t gi) __attribute__((always_inline)) {
            const uint32_t u0 = gi * G, gl = min(G, len - u0);
            anchor(load(u0), gi);
            for (uint32_t j = gl - 1; j >= 1; --j) {
                const uint32_t q = cd.template symbol<ZW>(delta_mix(load(u0 + j), one, cd.af),
                                                          t0 + u0 + j >= g.n_sink);
                cd.step(cd.entry(q));
                cd.flush();
            }
        };

        uint32_t gi = ng;  // groups left, processed from the last to the first
        if constexpr (GU > 0) {
            // the chunk's last group may be short: one token at a time; then full groups,
            // unrolled, the next group's rows loaded while this one is coded
            const uint32_t last = len - (ng - 1) * G;
            if (last != G) group_generic(--gi);
            if (gi > 0) {
                uint32_t cur[GU], nxt[GU];
                --gi;
#pragma unroll
                for (uint32_t j = 0; j < GU; ++j) cur[j] = load(gi * G + j);
                while (true) {
                    const uint32_t ugi = gi;
                    const bool more = ugi > 0;
                    const uint32_t nb = more ? (ugi - 1) * G : ugi * G;  // in bounds either way
#pragma unroll
                    for (uint32_t j = 0; j < GU; ++j) nxt[j] = load(nb + j);
                    anchor(cur[0], ugi);
                    const bool coded = t0 + ugi * G + 1 >= g.n_sink;
                    // The group's symbols; their off-grid lanes are only gathered, and
                    // counted token by token when some lane is off its grid (rare).
                    uint32_t q[GU];
                    uint64_t anyoff = 0;
#pragma unroll
                    for (uint32_t j = GU - 1; j >= 1; --j) {
                        uint64_t om;
                        q[j] = cd.template symbol_mask<ZW>(delta_mix(cur[j], one, cd.af), om);
                        anyoff |= om;
                    }
                    if (anyoff & cd.pmask) {
#pragma unroll
                        for (uint32_t j = GU - 1; j >= 1; --j)
                            cd.template symbol<ZW>(delta_mix(cur[j], one, cd.af),
                                                   coded || t0 + ugi * G + j >= g.n_sink);
                    }
                    EncEntry en[GU];
#pragma unroll
                    for (uint32_t j = GU - 1; j >= 1; --j) en[j] = cd.entry(q[j]);
#pragma unroll
                    for (uint32_t j = GU - 1; j >= 1; --j) cd.step(en[j]);
                    cd.flush();
                    if (!more) break;
                    --gi;
#pragma unroll
                    for (uint32_t j = 0; j < GU; ++j) cur[j] = nxt[j];
                }
            }
        } else {
            while (gi > 0) group_generic(--gi);
        }
    };
    if (cd.zmask)
        code_chunk(std::true_type{});
    else
        code_chunk(std::false_type{});

    // the state words come first in read order: lane i's two words at positions 2i, 2i+1
    uint32_t total = 0;
    if (m > 0) {
        total = cd.E + 2 * nl;
        if (present) {
            cd.ring[(0u - (total - 2 * lane)) & (kWordRing - 1)] = (uint16_t)(cd.x >> 16);
            cd.ring[(0u - (total - 2 * lane - 1)) & (kWordRing - 1)] = (uint16_t)cd.x;
        }
    }
    for (uint32_t i = lane; i < total - cd.flushed; i += kLanes) {
        const uint32_t D = cd.flushed + 1 + i;
        *(cd.rend - D) = cd.ring[(0u - D) & (kWordRing - 1)];
    }
    if (lane == 0) {
        group_words[gidx] = total;
        group_off_grid[gidx] = cd.n_off;
    }
}

// Exclusive prefix sum of n values in one block of 1024 threads; out[n] = total.  Tiles
// of 4096 values: each thread loads 4 consecutive ones, the 1024 sums are scanned in the
// wavefronts (shuffles) and across them (LDS), and a carry runs over the tiles.
__global__ __launch_bounds__(1024) void k_scan(const uint64_t *__restrict__ in,
                                                uint64_t *__restrict__ out, uint64_t n)
{
    __shared__ uint64_t wsum[16];
    const uint32_t tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    uint64_t carry = 0;
    for (uint64_t base = 0; base < n; base += 4096) {
        const uint64_t i0 = base + 4 * (uint64_t)tid;
        uint64_t v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = (i0 + k < n) ? in[i0 + k] : 0;
        const uint64_t tsum = v[0] + v[1] + v[2] + v[3];
        uint64_t incl = tsum;  // inclusive scan of the thread sums in the wavefront
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint64_t y = __shfl_up(incl, d, 64);
            if (lane >= (uint32_t)d) incl += y;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        uint64_t before = carry;
        for (uint32_t w = 0; w < wave; ++w) before += wsum[w];
        uint64_t tile = 0;
        for (uint32_t w = 0; w < 16; ++w) tile += wsum[w];
        uint64_t run = before + incl - tsum;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (i0 + k < n) out[i0 + k] = run;
            run += v[k];
        }
        carry += tile;
        __syncthreads();
    }
    if (tid == 0) out[n] = carry;
}

// Packs the groups' words from the ends of their regions into the payload; wavefront =
// group.  The payload side is written in 16-byte pieces: the words before the first
// 16-byte boundary and after the last one go one per lane, the rest 8 per lane, each
// piece cut out of the two aligned 16-byte source pieces it straddles (the source is off
// by the same number of words m for the whole group).
__device__ __forceinline__ uint4 words_at(uint4 A, uint4 B, uint32_t m)
{
    const uint32_t w[8] = {A.x, A.y, A.z, A.w, B.x, B.y, B.z, B.w};
    const uint32_t sh = (m & 1u) * 16u;
    uint32_t o[4];
    switch (m >> 1) {  // wave-uniform
    case 0:
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = __builtin_amdgcn_alignbit(w[i + 1], w[i], sh);
        break;
    case 1:
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = __builtin_amdgcn_alignbit(w[i + 2], w[i + 1], sh);
        break;
    case 2:
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = __builtin_amdgcn_alignbit(w[i + 3], w[i + 2], sh);
        break;
    default:
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = __builtin_amdgcn_alignbit(i + 4 < 8 ? w[i + 4] : 0u, w[i + 3], sh);
        break;
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

__global__ __launch_bounds__(256) void k5_compact(const uint16_t *__restrict__ regions,
                                                   uint64_t region_words,
                                                   const uint64_t *__restrict__ group_words,
                                                   const uint64_t *__restrict__ group_off,
                                                   uint64_t n_groups,
                                                   uint16_t *__restrict__ payload)
{
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
    const uint64_t gidx = (uint64_t)blockIdx.x * (blockDim.x / kLanes) + wave;
    if (gidx >= n_groups) return;
    const uint32_t lane = threadIdx.x % kLanes;
    const uint64_t n = group_words[gidx];
    const uint64_t s0 = (gidx + 1) * region_words - n;   // first source word
    const uint64_t d0 = group_off[gidx];                  // first payload word
    const uint64_t head = min(n, (8 - (d0 & 7)) & 7);
    for (uint64_t i = lane; i < head; i += kLanes) payload[d0 + i] = regions[s0 + i];
    const uint64_t body = (n - head) & ~uint64_t(7);
    const uint64_t sa = s0 + head, da = d0 + head;       // da is a multiple of 8
    const uint32_t m = (uint32_t)(sa & 7);
    const uint4 *src = reinterpret_cast<const uint4 *>(regions + (sa - m));
    uint4 *dst = reinterpret_cast<uint4 *>(payload + da);
    for (uint64_t p = lane; p < body / 8; p += kLanes) {
        const uint4 A = src[p];
        const uint4 B = m ? src[p + 1] : A;
        dst[p] = m ? words_at(A, B, m) : A;
    }
    for (uint64_t i = head + body + lane; i < n; i += kLanes) payload[d0 + i] = regions[s0 + i];
}


// ------------------------------------------------------------------------------ launchers
hipError_t launch_k0(const uint16_t *X, const Geom &g, uint32_t tpt, uint32_t *ord_lo,
                     uint32_t *ord_hi, uint32_t *flag, hipStream_t st)
{
    // token streams per row: one per 2 tpt tokens, at most one per group slot (~52 on the
    // 70B-shaped cache: fewer streams merge fewer partial results at the end, more read
    // more in parallel; 26, 52, 104, 416 and 1664 took 1.83, 1.79, 1.89, 3.7 and 14.5 ms)
    const uint32_t slots = (g.S + g.Tc - 1) / g.Tc * g.ngF;
    const uint32_t ntb = std::max(1u, std::min((g.S + 2 * tpt - 1) / (2 * tpt), slots));
    uint64_t threads = (uint64_t)g.L * 2 * ntb * (g.C / 8);
    hipLaunchKernelGGL(k0_minmax, dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0, st, X, g,
                       ntb, ord_lo, ord_hi, flag);
    return hipGetLastError();
}

hipError_t launch_k0_finalize(const Geom &g, const uint32_t *ord_lo, const uint32_t *ord_hi,
                              float *lo, float *hi, hipStream_t st)
{
    uint32_t n = g.L * 2 * g.C;
    hipLaunchKernelGGL(k0_finalize, dim3((n + 255) / 256), dim3(256), 0, st, g, ord_lo, ord_hi, lo, hi);
    return hipGetLastError();
}

hipError_t launch_width(const Geom &g, const uint8_t *bins, const float *lo, const float *hi,
                        float *w, float *r, hipStream_t st)
{
    uint32_t n = g.L * 2 * g.C;
    hipLaunchKernelGGL(k_width, dim3((n + 255) / 256), dim3(256), 0, st, g, bins, lo, hi, w, r);
    return hipGetLastError();
}

uint32_t fine_parts(const Geom &g)
{
    // token parts per (row, channel block): at most 65535 tokens each (16-bit counters),
    // and up to 4 of about 16K tokens for enough blocks
    return std::max((g.S + 65534u) / 65535u, std::min(4u, (g.S + 16383u) / 16384u));
}

hipError_t launch_fine_hist(const uint16_t *X, const Geom &g, const float *lo, const float *hi,
                            uint16_t *partial, hipStream_t st)
{
    const uint32_t parts = fine_parts(g);
    const uint64_t blocks = (uint64_t)g.L * 2 * g.NB * parts;
    if (g.alo)
        hipLaunchKernelGGL(k_fine_hist<true>, dim3((uint32_t)blocks), dim3(kFineWaves * 64), 0, st, X,
                           g, lo, hi, parts, partial);
    else
        hipLaunchKernelGGL(k_fine_hist<false>, dim3((uint32_t)blocks), dim3(kFineWaves * 64), 0, st, X,
                           g, lo, hi, parts, partial);
    return hipGetLastError();
}

hipError_t launch_clip(const Geom &g, const uint16_t *partial, uint32_t ppm, float *lo,
                       float *hi, hipStream_t st)
{
    const uint64_t n = (uint64_t)g.L * 2 * g.C;
    hipLaunchKernelGGL(k_clip, dim3((uint32_t)((n + 3) / 4)), dim3(256), 0, st, g, partial,
                       fine_parts(g), ppm, lo, hi);
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
    // 16-bit counters: a block's SUB streams take at most ceil(slots / (ntb SUB)) groups of
    // at most G tokens each
    const uint64_t slots = (uint64_t)((g.S + g.Tc - 1) / g.Tc) * g.ngF;
    while ((uint64_t)SUB * ((slots + (uint64_t)ntb * SUB - 1) / ((uint64_t)ntb * SUB)) * g.G > 0xFFFFu) ++ntb;
    size_t lds = (size_t)(max_bins + 1) / 2 * 8 * OCT * sizeof(uint32_t);
    hipLaunchKernelGGL(k1_hist, dim3((uint32_t)(rows * ntiles * ntb)), dim3(256), lds, st, X, g,
                       bins, lo, r, OCT, SUB, ntiles, ntb, counts);
    return hipGetLastError();
}

hipError_t launch_k1_freqs(const Geom &g, const uint8_t *bins, const uint32_t *counts,
                           uint16_t *freqs, hipStream_t st)
{
    uint32_t n = g.L * 2 * g.C;
    hipLaunchKernelGGL(k1_freqs, dim3((n + 255) / 256), dim3(256), 0, st, g, bins, counts, freqs);
    return hipGetLastError();
}

hipError_t launch_dtab(const Geom &g, const uint8_t *bins, const uint16_t *freqs,
                       const float *lo, const float *w, uint32_t *dtab, hipStream_t st)
{
    uint32_t n = g.L * 2 * g.C;
    hipLaunchKernelGGL(k_dtab, dim3((n + 255) / 256), dim3(256), 0, st, g, bins, freqs, lo, w, dtab);
    return hipGetLastError();
}

hipError_t launch_k2(const uint16_t *X, const Geom &g, const uint8_t *bins, const float *lo,
                     const float *r, uint32_t t_lo, uint32_t t_hi, uint32_t tpt, uint8_t *sym,
                     uint32_t sym_t0, uint32_t sym_T, uint16_t *anchors,
                     unsigned long long *clamped, hipStream_t st)
{
    uint32_t ntb = (t_hi - t_lo + tpt - 1) / tpt;
    uint64_t threads = (uint64_t)g.L * 2 * ntb * (g.C / 8);
    hipLaunchKernelGGL(k2_delta_quant, dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0, st,
                       X, g, bins, lo, r, t_lo, t_hi, tpt, ntb, sym, sym_t0, sym_T, anchors,
                       clamped);
    return hipGetLastError();
}

hipError_t launch_outliers(const uint16_t *X, const Geom &g, const uint8_t *bins, const float *lo,
                           const float *r, uint64_t *counts, const uint64_t *offs, uint32_t *keys,
                           uint16_t *vals, hipStream_t st)
{
    const uint64_t n_groups = (uint64_t)(g.ke - g.kb) * g.L * 2 * g.NB;
    const uint32_t blocks = (uint32_t)((n_groups + 3) / 4);
    if (counts && g.alo)
        hipLaunchKernelGGL((k_outliers<false, true>), dim3(blocks), dim3(256), 0, st, X, g, bins, lo,
                           r, n_groups, counts, offs, keys, vals);
    else if (counts)
        hipLaunchKernelGGL((k_outliers<false, false>), dim3(blocks), dim3(256), 0, st, X, g, bins, lo,
                           r, n_groups, counts, offs, keys, vals);
    else if (g.alo)
        hipLaunchKernelGGL((k_outliers<true, true>), dim3(blocks), dim3(256), 0, st, X, g, bins, lo,
                           r, n_groups, counts, offs, keys, vals);
    else
        hipLaunchKernelGGL((k_outliers<true, false>), dim3(blocks), dim3(256), 0, st, X, g, bins, lo,
                           r, n_groups, counts, offs, keys, vals);
    return hipGetLastError();
}

static uint32_t enc_sets(const Geom &g) { return (g.ke - g.kb + kEncWaves - 1) / kEncWaves; }

uint64_t code_region_words(const Geom &g)
{
    const uint32_t full = g.Tc < g.S ? g.Tc : g.S;
    const uint32_t m = full - (full + g.G - 1) / g.G;
    return ((uint64_t)kLanes * lane_words_max(m) + 3) & ~uint64_t(3);
}

hipError_t launch_k5_code(const uint16_t *X, const Geom &g, const uint8_t *bins,
                          const uint32_t *dtab, const float *lo, const float *r,
                          uint16_t *regions, uint8_t *anchors, uint64_t *group_words,
                          uint64_t *group_off_grid, hipStream_t st)
{
    const uint32_t n_sets = enc_sets(g);
    const uint64_t blocks = (uint64_t)g.L * 2 * g.NB * n_sets;
    if (g.G == kUG)
        hipLaunchKernelGGL(k5_code<kUG>, dim3((uint32_t)blocks), dim3(kEncWaves * 64), 0, st, X, g,
                           bins, dtab, lo, r, n_sets, code_region_words(g), regions, anchors,
                           group_words, group_off_grid);
    else
        hipLaunchKernelGGL(k5_code<0>, dim3((uint32_t)blocks), dim3(kEncWaves * 64), 0, st, X, g,
                           bins, dtab, lo, r, n_sets, code_region_words(g), regions, anchors,
                           group_words, group_off_grid);
    return hipGetLastError();
}

// Clears the byte ranges [r[i][0], r[i][1]) of a buffer (the padding between container
// sections): one launch instead of a fill per range.
__global__ __launch_bounds__(256) void k_zero_ranges(uint8_t *__restrict__ base, ZeroRanges zr)
{
    for (uint32_t i = 0; i < zr.n; ++i)
        for (uint64_t a = zr.r[i][0] + threadIdx.x; a < zr.r[i][1]; a += blockDim.x) base[a] = 0;
}

hipError_t launch_zero_ranges(uint8_t *base, const ZeroRanges &zr, hipStream_t st)
{
    hipLaunchKernelGGL(k_zero_ranges, dim3(1), dim3(256), 0, st, base, zr);
    return hipGetLastError();
}

hipError_t launch_scan(const uint64_t *in, uint64_t *out, uint64_t n, hipStream_t st)
{
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, st, in, out, n);
    return hipGetLastError();
}

hipError_t launch_k5_compact(const uint16_t *regions, uint64_t region_words,
                             const uint64_t *group_words, const uint64_t *group_off,
                             uint64_t n_groups, uint16_t *payload, hipStream_t st)
{
    if (!n_groups) return hipSuccess;
    hipLaunchKernelGGL(k5_compact, dim3((uint32_t)((n_groups + 3) / 4)), dim3(256), 0, st, regions,
                       region_words, group_words, group_off, n_groups, payload);
    return hipGetLastError();
}


}  // namespace cgk

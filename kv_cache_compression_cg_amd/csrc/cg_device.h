// cg_device.h -- device helpers and layout conventions shared by the encoder and decoder
// kernels of the KV-cache codec (see include/cg.h).
////
// Layout conventions shared by every kernel:
//   * KV caches are fp16 [L][2][S][C]; "row" means (layer, K/V) = l * 2 + kv.
//   * A "group" is (chunk, row, block b) with its 64 lanes = channels 64b .. 64b+63.
//     One wavefront decodes one group: lane i owns the stream of channel 64b + i,
//     all lanes step through the same token at the same time, so every output row
//     is written as one contiguous 128-byte store and the interleaved words of the
//     group are read from a contiguous, advancing window.
//   * Coder tables of one (row, block) (kTabBlock words, see cg_internal.h): a plane
//     [32 symbols][64 lanes] of {f | cdf << 24}, a plane of the dequantized deltas
//     lo + s * w (fp32 bits), then the 256-slot symbol table; a lane's entries sit in
//     its own 4-byte column, so 64 lanes reading any entries hit 64 different LDS banks.
//
// Float rules (bit-exact with the CPU oracle): -ffp-contract=off, fp32 division and
// reciprocal correctly rounded (HIP default), fmaf only where written, fp16 output
// converted round-to-nearest-even.

#pragma once

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

// quantize1 without branches, for finite delta, lo and r: the clamp to [0, N - 1] as the
// median of (v, 0, N - 1) gives the same integer (v <= 0, -0 included, -> 0;
// v > N - 1 -> N - 1).  nm1 = (float)(N - 1).
__device__ __forceinline__ uint32_t quantize_bf(float delta, float lo, float r, float nm1)
{
    return (uint32_t)__builtin_amdgcn_fmed3f(floorf(fmaf(delta - lo, r, 0.5f)), 0.0f, nm1);
}

// Whether quantize1 had to clamp: the nearest grid point is more than half a step away
// (floor(fma(delta - lo, r, 0.5)) outside [0, N - 1]), or the grid has zero width (r = 0,
// the single point lo) and delta is not on it, or delta is NaN (no grid point holds it).
__device__ __forceinline__ bool off_grid(float delta, float lo, float r, uint32_t N)
{
    if (r == 0.0f) return delta != lo;
    const float v = floorf(fmaf(delta - lo, r, 0.5f));
    return !(v >= 0.0f && v <= (float)(N - 1u));
}

// fp16_rne of fp32 fma(a, b, c), the fma rounded to fp32 first.  (The empty asm keeps
// the compiler from fusing the fma and the conversion into one mixed-precision fma,
// which rounds once and differs from the two roundings in rare cases.)
__device__ __forceinline__ uint32_t f2h_fma(float a, float b, float c)
{
    float v = fmaf(a, b, c);
    asm volatile("" : "+v"(v));
    return f2h(v);
}

// 8-bit anchors: the anchor value of x on its row's grid, fp16_rne(fma(code, aw, alo))
// with code = quantize1(x, alo, ar, 256), as a float.
__device__ __forceinline__ float anchor_snap(float x, float alo, float aw, float ar)
{
    return h2f(f2h_fma((float)quantize1(x, alo, ar, 256u), aw, alo));
}

// Applies anchor_snap to the 8 channels of an anchor read by an encoder thread whose
// channels start at row element r0 (no-op for fp16 anchors).
__device__ __forceinline__ void snap8(const Geom &g, uint64_t r0, float af[8])
{
    if (!g.alo) return;
#pragma unroll
    for (int j = 0; j < 8; ++j) af[j] = anchor_snap(af[j], g.alo[r0 + j], g.aw[r0 + j], g.ar[r0 + j]);
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

// rank of this lane among the set bits of a wave-wide mask
__device__ __forceinline__ uint32_t mbcnt64(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

}  // namespace cgk

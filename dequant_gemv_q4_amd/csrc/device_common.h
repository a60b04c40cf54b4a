// device_common.h -- device helpers shared by the gfx950 kernels of libqgemv: chunk decode,
// block-offset folding, staging of x into LDS, scale decode, lane reductions.
#pragma once

#include <hip/hip_runtime.h>

#include "qgemv_internal.h"

namespace qg {

// ------------------------------------------------------------------------------------ helpers

__device__ __forceinline__ float h2f(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ float ub0(uint32_t v) { return (float)(v & 0xffu); }
__device__ __forceinline__ float ub1(uint32_t v) { return (float)((v >> 8) & 0xffu); }
__device__ __forceinline__ float ub2(uint32_t v) { return (float)((v >> 16) & 0xffu); }
__device__ __forceinline__ float ub3(uint32_t v) { return (float)(v >> 24); }

__device__ __forceinline__ int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }

__device__ __forceinline__ uint32_t ucomp(const uint4 &v, int k)
{
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

__device__ __forceinline__ float4 f4scale(float4 v, float s, float4 g)
{
    return make_float4(v.x * s * g.x, v.y * s * g.y, v.z * s * g.z, v.w * s * g.w);
}

// Per-format compile-time facts of the chunk (16 bytes of quants) a lane processes.
template <int FMT> struct Fc {
    static constexpr int XF4 = fmt_facts(FMT).xf4, CE = fmt_facts(FMT).ce, NS = fmt_facts(FMT).ns;
};

// Element (within a K tile) of float4 j of chunk i.
template <int FMT>
__device__ __forceinline__ int chunk_elem(int i, int j)
{
    if constexpr (FMT == FQ4_0 || FMT == FQ5_0 || fmt_generic(FMT)) {
        return 32 * i + 4 * j;             // 32 consecutive weights per chunk
    } else if constexpr (FMT == FQ8_0) {
        return 16 * i + 4 * j;             // half a block per chunk
    } else if constexpr (FMT == FQ6_K) {
        // Q6_K: chunk i is ql bytes 16t..16t+15 of super-block s (t = i % 8, n = t / 4,
        // u = t % 4); its low nibbles are elements 128n + 16u + 0..15, its high nibbles
        // elements 128n + 64 + 16u + 0..15.
        const int s = i >> 3, t = i & 7, n = t >> 2, u = t & 3;
        const int base = 256 * s + 128 * n + 16 * u;
        return j < 4 ? base + 4 * j : base + 64 + 4 * (j - 4);
    } else {
        // Q4_K: chunk i is bytes 16q..16q+15 of super-block s's nibbles (q = i % 8).  Its low
        // nibbles are elements 64c + 16h + 0..15 (sub-block 2c), its high nibbles elements
        // 64c + 32 + 16h + 0..15 (sub-block 2c + 1), with c = q / 2, h = q % 2.
        const int s = i >> 3, q = i & 7, c = q >> 1, h = q & 1;
        const int base = 256 * s + 64 * c + 16 * h;
        return j < 4 ? base + 4 * j : base + 32 + 4 * (j - 4);
    }
}

// ------------------------------------------------------------------------------------ staging

// Stage K-tile t of NB x rows into LDS.  Row r comes from xrow[r] (nullptr = a zero row).  With
// NRM every element is multiplied by inv[r] and gamma.  Then the per-chunk sums S are formed in
// exactly the order the dot products consume the elements.
template <int FMT, int NB, bool NRM>
__device__ void stage_tile(const float *const *xrow, const float *gamma, const float *inv, int t,
                           int kt, float4 *X4, float *S)
{
    constexpr int XF4 = Fc<FMT>::XF4, CE = Fc<FMT>::CE;
    const int ct = kt / CE;
    const int total = NB * ct * XF4;
    for (int f = threadIdx.x; f < total; f += blockDim.x) {
        const int j = f % XF4;
        const int i = (f / XF4) % ct;
        const int r = f / (XF4 * ct);
        const int e = t * kt + chunk_elem<FMT>(i, j);
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (xrow[r]) {
            v = *reinterpret_cast<const float4 *>(xrow[r] + e);
            if constexpr (NRM)
                v = f4scale(v, inv[r], *reinterpret_cast<const float4 *>(gamma + e));
        }
        X4[(r * XF4 + j) * ct + i] = v;
    }
    __syncthreads();
    for (int f = threadIdx.x; f < NB * ct; f += blockDim.x) {
        const int r = f / ct, i = f % ct;
        const float4 *xc = X4 + (size_t)r * XF4 * ct + i;
        if constexpr (FMT == FQ4_0 || FMT == FQ5_0 || fmt_generic(FMT)) {
            // dot order: for each dword k, its low nibbles (elements 4k..4k+3) then its high
            // nibbles (elements 16+4k..16+4k+3) (the affine format's sum: any fixed order)
            float s = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float4 a = xc[k * ct], b = xc[(4 + k) * ct];
                s += a.x; s += a.y; s += a.z; s += a.w;
                s += b.x; s += b.y; s += b.z; s += b.w;
            }
            S[f] = s;
        } else if constexpr (FMT == FQ8_0) {
            float s = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float4 a = xc[k * ct];
                s += a.x; s += a.y; s += a.z; s += a.w;
            }
            S[f] = s;
        } else {
            float sa = 0.f, sb = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float4 a = xc[k * ct], b = xc[(4 + k) * ct];
                sa += a.x; sa += a.y; sa += a.z; sa += a.w;
                sb += b.x; sb += b.y; sb += b.z; sb += b.w;
            }
            S[2 * f] = sa;
            S[2 * f + 1] = sb;
        }
    }
    __syncthreads();
}

// 1 / sqrt(mean(x_r^2) + eps) for the NB rows, computed by the whole workgroup in a fixed order.
template <int NB>
__device__ void row_inv_rms(const float *const *xrow, int64_t K, float eps, float *inv_out,
                            float *red /* LDS, NB * 4 floats */)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int r = 0; r < NB; ++r) {
        float ss = 0.f;
        if (xrow[r]) {
            for (int64_t e = 4 * threadIdx.x; e < K; e += 4 * blockDim.x) {
                const float4 v = *reinterpret_cast<const float4 *>(xrow[r] + e);
                ss = fmaf(v.x, v.x, ss); ss = fmaf(v.y, v.y, ss);
                ss = fmaf(v.z, v.z, ss); ss = fmaf(v.w, v.w, ss);
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            ss += __shfl_xor(ss, off);
        if (lane == 0)
            red[r * 4 + wave] = ss;
    }
    __syncthreads();
    if (threadIdx.x < NB) {
        const int r = threadIdx.x;
        const float ss = ((red[r * 4 + 0] + red[r * 4 + 1]) + red[r * 4 + 2]) + red[r * 4 + 3];
        inv_out[r] = 1.0f / sqrtf(ss / (float)K + eps);
    }
    __syncthreads();
}

// ------------------------------------------------------------------------------------ compute

struct MatPtr {
    const uint8_t *qs, *sc, *hb, *dd;   // quant, scale, high-bit and (Q6_K) d planes
    uint4 cbt;                          // IQ4 formats: the 16 signed codebook bytes
};

// Codebook lookup of four 4-bit indices (one per byte of idx, bits 4-7 clear) in the 16-entry
// byte table T (entry e = byte e % 4 of T[e / 4]): v_perm_b32 picks bytes out of eight, so
// entries 0-7 and 8-15 are looked up separately and a third permute takes, per byte, the one
// that bit 3 of the index names (selector i, or i + 4 for the second lookup).  The first two
// permutes see the index with bit 3 still set and return a constant for it, which the third
// drops.
__device__ __forceinline__ uint32_t cb_lookup(const uint4 &T, uint32_t idx)
{
    const uint32_t lo = __builtin_amdgcn_perm(T.y, T.x, idx);
    const uint32_t hi = __builtin_amdgcn_perm(T.w, T.z, idx & 0x07070707u);
    const uint32_t sel = ((idx >> 1) & 0x04040404u) | 0x03020100u;
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Row strides of the four planes.
struct RowBytes {
    int64_t qs, sc, hb, d;
};

// Scale terms of one chunk of one row: Q4_0/Q8_0 use a (the block scale); Q4_K uses
// aA, bA (sub-block of the low nibbles) and aB, bB (high nibbles).
struct ChunkScale {
    float a, b, a2, b2;
};

template <int FMT>
__device__ __forceinline__ ChunkScale chunk_scale(const uint4 &s, int q /* chunk in super-block */)
{
    ChunkScale cs;
    if constexpr (FMT == FIQ4_XS) {
        // s.x: f16 d, then the 16-bit word of high scale bits (sub-block q at bits 2q, 2q + 1);
        // s.y: the low 4-bit scale of sub-block q at bits 4q..4q+3; scale d (ls - 32)
        const uint32_t ls = ((s.y >> (4 * q)) & 15u) | (((s.x >> (16 + 2 * q)) & 3u) << 4);
        cs.a = h2f(s.x & 0xffffu) * (float)((int)ls - 32);
        cs.b = cs.a2 = cs.b2 = 0.f;
    } else if constexpr (FMT == FAQ4) {
        // f16 scale s and f16 bias c: w = s q + c, held as a q - b with b = -c
        cs.a = h2f(s.x & 0xffffu);
        cs.b = -h2f(s.x >> 16);
        cs.a2 = cs.b2 = 0.f;
    } else if constexpr (FMT == FQ6_K) {
        // s.x, s.y: the eight signed scales of the chunk's half of the super-block (bytes 8n..8n+7,
        // n = q / 4); the chunk (u = q % 4) takes scale u (low nibbles) and u + 4 (high);
        // s.z: the super-block's f16 d
        const float d = h2f(s.z & 0xffffu);
        const int u = q & 3;
        cs.a = d * (float)(int8_t)((s.x >> (8 * u)) & 0xffu);
        cs.a2 = d * (float)(int8_t)((s.y >> (8 * u)) & 0xffu);
        cs.b = cs.b2 = 0.f;
    } else if constexpr (fmt_min(FMT)) {
        // sub-blocks 2c, 2c + 1 of the 12 scale bytes (s.y: bytes 0-3, s.z: 4-7, s.w: 8-11):
        // sub-block j < 4 keeps its scale in the low 6 bits of byte j and its min in byte j + 4;
        // j >= 4 keeps 4 low bits of each in byte j + 4 (scale low nibble, min high nibble) and
        // the 2 high bits in the top bits of bytes j - 4 and j.  Both cases as one set of bit-field
        // extracts whose source word and widths depend on c (the lanes of a wave hold different
        // chunks of their super-blocks, so a branch on c would run both sides)
        const float d = h2f(s.x & 0xffffu), dmin = h2f(s.x >> 16);
        const int c = q >> 1;
        const bool up = c >= 2;
        const uint32_t sA = 16u * (uint32_t)(c & 1), sB = sA + 8u;
        const uint32_t lsc = up ? s.w : s.y, lm = up ? s.w : s.z;
        const uint32_t wl = up ? 4u : 6u, om = up ? 4u : 0u, hm = up ? 3u : 0u;
        const uint32_t scA = __builtin_amdgcn_ubfe(lsc, sA, wl) |
                             ((__builtin_amdgcn_ubfe(s.y, sA + 6u, 2u) & hm) << 4);
        const uint32_t mA = __builtin_amdgcn_ubfe(lm, sA + om, wl) |
                            ((__builtin_amdgcn_ubfe(s.z, sA + 6u, 2u) & hm) << 4);
        const uint32_t scB = __builtin_amdgcn_ubfe(lsc, sB, wl) |
                             ((__builtin_amdgcn_ubfe(s.y, sB + 6u, 2u) & hm) << 4);
        const uint32_t mB = __builtin_amdgcn_ubfe(lm, sB + om, wl) |
                            ((__builtin_amdgcn_ubfe(s.z, sB + 6u, 2u) & hm) << 4);
        cs.a = d * (float)scA;
        cs.b = dmin * (float)mA;
        cs.a2 = d * (float)scB;
        cs.b2 = dmin * (float)mB;
    } else {
        cs.a = h2f(s.x & 0xffffu);
        cs.b = cs.a2 = cs.b2 = 0.f;
    }
    return cs;
}

// Q4_K sub-block centre.  With a = d sc and b = dmin m the weights are w = a n - b =
// a (n - c) + (a c - b) for any integer c; c = the integer nearest b / a, kept in [0, 63], makes
// a |n - c| at most about 2 |w| for every n != c and |a c - b| at most about |w| for every weight,
// so a dot over (n - c) and the term (a c - b) sum x carry no cancellation: their rounding is
// relative to sum |w x| (for b / a outside [0, 63] every |w| is already at least 48 a).  a = 0 or
// NaN ratios give c = 0 (any c is exact there).
__device__ __forceinline__ float k_center(float a, float b)
{
    return fminf(fmaxf(rintf(b * __builtin_amdgcn_rcpf(a)), 0.f), 63.f);
}

// The affine format's centre: w = s q + c = s (q - c') + (s c' + c) with c' the point of
// {0, ..., 15} nearest t = -c / s.  Every weight has |q - t| >= |c' - t| (c' is the nearest of
// the values q takes), so |s c' + c| = |s| |c' - t| <= |w| and |s (q - c')| <= 2 |w| for every
// weight of the block: the dot over q - c' and the term (s c' + c) sum x round relative to
// sum |w x|.  s = 0 (t infinite or NaN) gives 0 or 15, exact there (every w is c).
__device__ __forceinline__ float aq_center(float a, float b)
{
    return fminf(fmaxf(rintf(b * __builtin_amdgcn_rcpf(a)), 0.f), 15.f);
}

// Decode the 16-byte chunk into the per-element factors the dot multiplies, exact in f32 and in
// dot order: Q4_0 the signed q - 8, Q5_0 q - 16, Q8_0 the signed byte, Q6_K q - 32, Q4_K and Q5_K
// the unsigned q (centred per sub-block in chunk_dot).  h: the chunk's high-bit words (the
// layout k_pack writes: low nibble of byte 4k + m at bit 8m + k, high nibble at 8m + 4 + k; Q6_K
// two bits each, at 8m + 2k of h.x (low) and h.y (high)).
template <int FMT>
__device__ __forceinline__ void decode_chunk(const uint4 &q, const uint2 &h, const uint4 &cbt,
                                             float *w)
{
    if constexpr (fmt_codebook(FMT)) {
        // codebook entries in Q4_0's nibble order: w[8k + m] element 4k + m (low nibble of byte
        // 4k + m), w[8k + 4 + m] element 16 + 4k + m (its high nibble)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t v = ucomp(q, k);
            const uint32_t lo = cb_lookup(cbt, v & 0x0f0f0f0fu);
            const uint32_t hi = cb_lookup(cbt, (v >> 4) & 0x0f0f0f0fu);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                w[8 * k + m] = (float)(int8_t)((lo >> (8 * m)) & 0xffu);
                w[8 * k + 4 + m] = (float)(int8_t)((hi >> (8 * m)) & 0xffu);
            }
        }
        return;
    }
    if constexpr (FMT == FQ1_0) {
        // natural order: w[e] = +1 if bit e of the chunk's word is set, else -1
#pragma unroll
        for (int e = 0; e < 32; ++e)
            w[e] = ((q.x >> e) & 1u) ? 1.0f : -1.0f;
        return;
    }
    if constexpr (FMT == FAQ4) {
        // natural order: element 2i the low nibble of byte i, 2i + 1 its high nibble
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t b = (ucomp(q, i >> 2) >> (8 * (i & 3))) & 0xffu;
            w[2 * i] = (float)(b & 15u);
            w[2 * i + 1] = (float)(b >> 4);
        }
        return;
    }
    if constexpr (fmt_hbits(FMT)) {
        const float off = FMT == FQ5_0 ? 16.0f : FMT == FQ6_K ? 32.0f : 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t v = ucomp(q, k);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint32_t lo = (v >> (8 * m)) & 15u, hi = (v >> (8 * m + 4)) & 15u;
                uint32_t bl, bh;
                if constexpr (FMT == FQ6_K) {
                    bl = (h.x >> (8 * m + 2 * k)) & 3u;
                    bh = (h.y >> (8 * m + 2 * k)) & 3u;
                } else {
                    bl = (h.x >> (8 * m + k)) & 1u;
                    bh = (h.x >> (8 * m + 4 + k)) & 1u;
                }
                w[8 * k + m] = (float)(lo | (bl << 4)) - off;
                w[8 * k + 4 + m] = (float)(hi | (bh << 4)) - off;
            }
        }
        return;
    }
    if constexpr (FMT == FQ8_0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t v = ucomp(q, k);
            w[4 * k + 0] = (float)(int8_t)(v & 0xffu);
            w[4 * k + 1] = (float)(int8_t)((v >> 8) & 0xffu);
            w[4 * k + 2] = (float)(int8_t)((v >> 16) & 0xffu);
            w[4 * k + 3] = (float)(int8_t)(v >> 24);
        }
    } else {
        const float off = FMT == FQ4_0 ? 8.0f : 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t v = ucomp(q, k);
            const uint32_t lo = v & 0x0f0f0f0fu, hi = (v >> 4) & 0x0f0f0f0fu;
            w[8 * k + 0] = ub0(lo) - off; w[8 * k + 1] = ub1(lo) - off;
            w[8 * k + 2] = ub2(lo) - off; w[8 * k + 3] = ub3(lo) - off;
            w[8 * k + 4] = ub0(hi) - off; w[8 * k + 5] = ub1(hi) - off;
            w[8 * k + 6] = ub2(hi) - off; w[8 * k + 7] = ub3(hi) - off;
        }
    }
}

// Accumulate one decoded chunk against one staged x chunk (xv: XF4 float4s, Sv: NS sums).
template <int FMT>
__device__ __forceinline__ float chunk_dot(const float *w, const float4 *xv, const float *Sv,
                                           const ChunkScale &cs, float acc)
{
    if constexpr (FMT == FQ1_0 || FMT == FAQ4) {
        // natural order; the affine format centred (aq_center), its (s c' + c) term times the
        // chunk's x sum
        const float c = FMT == FAQ4 ? aq_center(cs.a, cs.b) : 0.f;
        float dot = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            dot = fmaf(w[4 * j + 0] - c, xv[j].x, dot);
            dot = fmaf(w[4 * j + 1] - c, xv[j].y, dot);
            dot = fmaf(w[4 * j + 2] - c, xv[j].z, dot);
            dot = fmaf(w[4 * j + 3] - c, xv[j].w, dot);
        }
        acc = fmaf(cs.a, dot, acc);
        if constexpr (FMT == FAQ4)
            acc = fmaf(fmaf(cs.a, c, -cs.b), Sv[0], acc);
        return acc;
    } else if constexpr (FMT == FQ4_0 || FMT == FQ5_0 || fmt_codebook(FMT)) {
        float dot = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            dot = fmaf(w[8 * k + 0], xv[k].x, dot);
            dot = fmaf(w[8 * k + 1], xv[k].y, dot);
            dot = fmaf(w[8 * k + 2], xv[k].z, dot);
            dot = fmaf(w[8 * k + 3], xv[k].w, dot);
            dot = fmaf(w[8 * k + 4], xv[4 + k].x, dot);
            dot = fmaf(w[8 * k + 5], xv[4 + k].y, dot);
            dot = fmaf(w[8 * k + 6], xv[4 + k].z, dot);
            dot = fmaf(w[8 * k + 7], xv[4 + k].w, dot);
        }
        return fmaf(cs.a, dot, acc);
    } else if constexpr (FMT == FQ8_0) {
        float dot = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            dot = fmaf(w[4 * k + 0], xv[k].x, dot);
            dot = fmaf(w[4 * k + 1], xv[k].y, dot);
            dot = fmaf(w[4 * k + 2], xv[k].z, dot);
            dot = fmaf(w[4 * k + 3], xv[k].w, dot);
        }
        return fmaf(cs.a, dot, acc);
    } else if constexpr (FMT == FQ6_K) {
        float da = 0.f, db = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            da = fmaf(w[8 * k + 0], xv[k].x, da);
            da = fmaf(w[8 * k + 1], xv[k].y, da);
            da = fmaf(w[8 * k + 2], xv[k].z, da);
            da = fmaf(w[8 * k + 3], xv[k].w, da);
            db = fmaf(w[8 * k + 4], xv[4 + k].x, db);
            db = fmaf(w[8 * k + 5], xv[4 + k].y, db);
            db = fmaf(w[8 * k + 6], xv[4 + k].z, db);
            db = fmaf(w[8 * k + 7], xv[4 + k].w, db);
        }
        return fmaf(cs.a2, db, fmaf(cs.a, da, acc));
    } else {
        // centred sub-blocks (k_center): dots over n - c, then the (a c - b) sum x terms
        const float cA = k_center(cs.a, cs.b), cB = k_center(cs.a2, cs.b2);
        float da = 0.f, db = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            da = fmaf(w[8 * k + 0] - cA, xv[k].x, da);
            da = fmaf(w[8 * k + 1] - cA, xv[k].y, da);
            da = fmaf(w[8 * k + 2] - cA, xv[k].z, da);
            da = fmaf(w[8 * k + 3] - cA, xv[k].w, da);
            db = fmaf(w[8 * k + 4] - cB, xv[4 + k].x, db);
            db = fmaf(w[8 * k + 5] - cB, xv[4 + k].y, db);
            db = fmaf(w[8 * k + 6] - cB, xv[4 + k].z, db);
            db = fmaf(w[8 * k + 7] - cB, xv[4 + k].w, db);
        }
        acc = fmaf(cs.a, da, acc);
        acc = fmaf(fmaf(cs.a, cA, -cs.b), Sv[0], acc);
        acc = fmaf(cs.a2, db, acc);
        acc = fmaf(fmaf(cs.a2, cB, -cs.b2), Sv[1], acc);
        return acc;
    }
}

template <int FMT>
__device__ __forceinline__ void load_chunk(const MatPtr &m, const RowBytes &rb, int64_t n,
                                           int64_t ci, uint4 &q, uint4 &s, uint2 &h)
{
    if constexpr (FMT == FQ1_0)
        q = make_uint4(*reinterpret_cast<const uint32_t *>(m.qs + n * rb.qs + ci * 4), 0u, 0u, 0u);
    else
        q = *reinterpret_cast<const uint4 *>(m.qs + n * rb.qs + ci * 16);
    h = make_uint2(0u, 0u);
    if constexpr (FMT == FIQ4_XS) {
        const uint2 w = *reinterpret_cast<const uint2 *>(m.sc + n * rb.sc + (ci >> 3) * 8);
        s = make_uint4(w.x, w.y, 0u, 0u);
    } else if constexpr (FMT == FQ1_0) {
        s = make_uint4(*reinterpret_cast<const uint16_t *>(m.sc + n * rb.sc + (ci >> 2) * 2), 0u,
                       0u, 0u);
    } else if constexpr (FMT == FAQ4) {
        s = make_uint4(*reinterpret_cast<const uint32_t *>(m.sc + n * rb.sc + ci * 4), 0u, 0u, 0u);
    } else if constexpr (FMT == FQ4_0 || FMT == FQ5_0 || FMT == FIQ4_NL) {
        s = make_uint4(*reinterpret_cast<const uint16_t *>(m.sc + n * rb.sc + ci * 2), 0u, 0u, 0u);
    } else if constexpr (FMT == FQ8_0) {
        s = make_uint4(*reinterpret_cast<const uint16_t *>(m.sc + n * rb.sc + (ci >> 1) * 2), 0u,
                       0u, 0u);
    } else if constexpr (FMT == FQ6_K) {
        const uint2 w = *reinterpret_cast<const uint2 *>(m.sc + n * rb.sc + (ci >> 3) * 16 +
                                                         ((ci & 7) >> 2) * 8);
        s = make_uint4(w.x, w.y,
                       *reinterpret_cast<const uint16_t *>(m.dd + n * rb.d + (ci >> 3) * 2), 0u);
    } else {
        s = *reinterpret_cast<const uint4 *>(m.sc + n * rb.sc + (ci >> 3) * 16);
    }
    if constexpr (FMT == FQ6_K)
        h = *reinterpret_cast<const uint2 *>(m.hb + n * rb.hb + ci * 8);
    else if constexpr (fmt_hbits(FMT))
        h.x = *reinterpret_cast<const uint32_t *>(m.hb + n * rb.hb + ci * 4);
}

// One K tile of one wave step: rows row0 + u*G + slot (u < U) of each of MATS matrices against
// the NB staged x rows.  Lane lir of its LPR-lane group takes chunks lir, lir + lpr, ...
template <int FMT, int NB, int U, int MATS>
__device__ __forceinline__ void tile_compute(const MatPtr (&mat)[MATS], const RowBytes &rb,
                                             int64_t row0, int64_t N, int G,
                                             int slot, int lir, int lpr, int t, int ct,
                                             const float4 *X4, const float *S,
                                             float (&acc)[MATS][U][NB])
{
    constexpr int XF4 = Fc<FMT>::XF4, CE = Fc<FMT>::CE, NS = Fc<FMT>::NS;
    for (int i = lir; i < ct; i += lpr) {
        const int64_t ci = (int64_t)t * ct + i;
        uint4 q[MATS][U], s[MATS][U];
        uint2 h[MATS][U];
#pragma unroll
        for (int m = 0; m < MATS; ++m)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t n = row0 + (int64_t)u * G + slot;
                if (n < N) {
                    load_chunk<FMT>(mat[m], rb, n, ci, q[m][u], s[m][u], h[m][u]);
                } else {
                    q[m][u] = make_uint4(0u, 0u, 0u, 0u);
                    s[m][u] = make_uint4(0u, 0u, 0u, 0u);
                    h[m][u] = make_uint2(0u, 0u);
                }
            }
        const int qpos = (int)(ci & 7);
        if constexpr (NB == 1) {
            float4 xv[XF4];
#pragma unroll
            for (int j = 0; j < XF4; ++j)
                xv[j] = X4[j * ct + i];
            float Sv[NS];
#pragma unroll
            for (int k = 0; k < NS; ++k)
                Sv[k] = S[i * NS + k];
#pragma unroll
            for (int m = 0; m < MATS; ++m)
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float w[CE];
                    decode_chunk<FMT>(q[m][u], h[m][u], mat[m].cbt, w);
                    const ChunkScale cs = chunk_scale<FMT>(s[m][u], qpos);
                    acc[m][u][0] = chunk_dot<FMT>(w, xv, Sv, cs, acc[m][u][0]);
                }
        } else {
            float w[MATS][U][CE];
            ChunkScale cs[MATS][U];
#pragma unroll
            for (int m = 0; m < MATS; ++m)
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    decode_chunk<FMT>(q[m][u], h[m][u], mat[m].cbt, w[m][u]);
                    cs[m][u] = chunk_scale<FMT>(s[m][u], qpos);
                }
#pragma unroll
            for (int r = 0; r < NB; ++r) {
                float4 xv[XF4];
#pragma unroll
                for (int j = 0; j < XF4; ++j)
                    xv[j] = X4[(r * XF4 + j) * ct + i];
                float Sv[NS];
#pragma unroll
                for (int k = 0; k < NS; ++k)
                    Sv[k] = S[(r * ct + i) * NS + k];
#pragma unroll
                for (int m = 0; m < MATS; ++m)
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        acc[m][u][r] = chunk_dot<FMT>(w[m][u], xv, Sv, cs[m][u], acc[m][u][r]);
            }
        }
    }
}

__device__ __forceinline__ float group_sum(float v, int lpr)
{
    for (int off = lpr >> 1; off > 0; off >>= 1)
        v += __shfl_xor(v, off);
    return v;
}

// act(g) u of the gated product: silu(g) = g / (1 + e^-g) ("honeycrisp mod.rs",
// fused_norm_swiglu_down), or the tanh form of GELU, 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3)))
// (the GeluTanh variant of the gate/up + norm pipeline, "honeycrisp mod.rs",
// pipe_q8_large4_gus_nrm_gelu).  act is uniform across the launch.
__device__ __forceinline__ float gated(float g, float u, int act)
{
    if (act == A_GELU_TANH) {
        const float k0 = 0.7978845608028654f;   // sqrt(2 / pi)
        const float t = tanhf(k0 * fmaf(0.044715f * g, g * g, g));
        return 0.5f * g * (1.0f + t) * u;
    }
    return g / (1.0f + expf(-g)) * u;
}

// Order-preserving key: larger value -> larger key; equal values -> the lower index wins.
__device__ __forceinline__ unsigned long long argmax_key(float v, int64_t n)
{
    const uint32_t b = __float_as_uint(v + 0.0f);   // -0 -> +0
    const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((unsigned long long)ord << 32) | (unsigned long long)(0xffffffffu - (uint32_t)n);
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int off)
{
    const uint32_t lo = __shfl_xor((uint32_t)v, off), hi = __shfl_xor((uint32_t)(v >> 32), off);
    return ((unsigned long long)hi << 32) | lo;
}


}  // namespace qg

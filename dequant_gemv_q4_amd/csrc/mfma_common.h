// mfma_common.h -- operand helpers of the gfx950 matrix-core dequant kernels (mfma_kernels.hip,
// gemm_kernels.hip): exact f16 weights from quant bytes in the order the 16x16x32 f16 operands
// take them, and the 4 x 4 dword transpose across the 16-lane rows of a wave.
//
// Operand layouts (CDNA4 v_mfma_f32_16x16x32_f16): lane l holds A[l % 16][8 (l / 16) + 0..7] and
// B[8 (l / 16) + 0..7][l % 16], and D[4 (l / 16) + 0..3][l % 16].  A k position may be any block
// element as long as A and B agree, so the eight halves a lane holds for one block are the eight
// elements of one dword of quant bytes (Q4_0: bytes 4j..4j+3, their low and high nibbles; Q8_0:
// bytes 4j..4j+3 of both 16-byte halves of the block; Q4_K: the low (or high) nibbles of bytes
// 4j..4j+3 of the sub-block's two 16-byte chunks), and x is laid out to match (mf_slot).
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"

namespace qg {

typedef _Float16 mh2 __attribute__((ext_vector_type(2)));
typedef _Float16 mh8 __attribute__((ext_vector_type(8)));
typedef _Float16 mh4 __attribute__((ext_vector_type(4)));
typedef float mf4 __attribute__((ext_vector_type(4)));

constexpr int MF_WAVES = 16;             // waves per workgroup: one per batch row in the prologue
constexpr int MF_THREADS = 64 * MF_WAVES;
constexpr int MF_KMAX = 4096;            // longest row the staged x fits (x2 K classes)

__device__ __forceinline__ uint32_t mf_and_or(uint32_t v, uint32_t m, uint32_t c)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "v"(m), "v"(c));
    return r;
}

__device__ __forceinline__ uint32_t mf_hadd(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(mh2, a) + __builtin_bit_cast(mh2, b));
}

struct MfConst {
    uint32_t m_lo, m_hi, c, off_lo, off_hi;
    uint32_t m_b, m_nb, m_sel, c_id, c64;   // byte mask, nibble mask, codebook lookup constants
    uint32_t c1;                            // f16 pair (1.0, 1.0): Q1_0's sign pairs
};

template <int FMT>
__device__ __forceinline__ MfConst mf_const()
{
    MfConst k;
    k.m_lo = FMT == FQ8_0 ? 0x00FF00FFu : 0x000F000Fu;
    k.m_hi = 0x00F000F0u;
    k.c = 0x64006400u;
    k.off_lo = FMT == FQ8_0 ? 0xE480E480u : 0xE408E408u;   // -1152 (Q8_0) / -1032 (n - 8)
    k.off_hi = 0xE480E480u;                                // -1152: 16 n - 128
    k.m_b = 0x00FF00FFu;
    k.m_nb = 0x0F0F0F0Fu;
    k.m_sel = 0x04040404u;
    k.c_id = 0x03020100u;
    k.c64 = 0x64646464u;
    k.c1 = 0x3C003C00u;
    asm volatile("" : "+v"(k.m_lo), "+v"(k.m_hi), "+v"(k.c), "+v"(k.off_lo), "+v"(k.off_hi));
    if constexpr (FMT == FQ5_0 || FMT == FQ5_K || FMT == FQ6_K)
        asm volatile("" : "+v"(k.m_b), "+v"(k.m_nb));
    if constexpr (FMT == FQ1_0)
        asm volatile("" : "+v"(k.c1));
    if constexpr (fmt_codebook(FMT))
        asm volatile("" : "+v"(k.m_sel), "+v"(k.c_id), "+v"(k.c64));
    return k;
}

// B operand (eight exact f16 weights) of one block from the lane's dword(s).
template <int FMT>
__device__ __forceinline__ mh8 mf_bop(uint32_t q0, uint32_t q1, const MfConst &k)
{
    uint32_t w[4];
    if constexpr (FMT == FQ8_0) {
        const uint32_t u0 = q0 ^ 0x80808080u, u1 = q1 ^ 0x80808080u;
        w[0] = mf_hadd(mf_and_or(u0, k.m_lo, k.c), k.off_lo);          // bytes 0, 2 (half 0)
        w[1] = mf_hadd(mf_and_or(u0 >> 8, k.m_lo, k.c), k.off_lo);     // bytes 1, 3
        w[2] = mf_hadd(mf_and_or(u1, k.m_lo, k.c), k.off_lo);          // bytes 0, 2 (half 1)
        w[3] = mf_hadd(mf_and_or(u1 >> 8, k.m_lo, k.c), k.off_lo);     // bytes 1, 3
    } else {
        const uint32_t t = q0 >> 8;
        w[0] = mf_hadd(mf_and_or(q0, k.m_lo, k.c), k.off_lo);   // low nibbles of bytes 0, 2
        w[1] = mf_hadd(mf_and_or(q0, k.m_hi, k.c), k.off_hi);   // high nibbles of bytes 0, 2 (x16)
        w[2] = mf_hadd(mf_and_or(t, k.m_lo, k.c), k.off_lo);    // low nibbles of bytes 1, 3
        w[3] = mf_hadd(mf_and_or(t, k.m_hi, k.c), k.off_hi);    // high nibbles of bytes 1, 3 (x16)
    }
    struct W4 {
        uint32_t v[4];
    } p = {{w[0], w[1], w[2], w[3]}};
    return __builtin_bit_cast(mh8, p);
}

// Position (dword j of the block, half h of the lane's eight) of block element eb (0..31), and
// whether it carries the 1/16 of a high nibble.
template <int FMT>
__device__ __forceinline__ void mf_slot(int eb, int &j, int &h, bool &hi)
{
    if constexpr (FMT == FAQ4) {
        // dword j holds elements 8j..8j+7, element 8j + 2m + u in nibble u of byte m; halves:
        // [lo b0, lo b2, hi b0, hi b2, lo b1, lo b3, hi b1, hi b3] (high nibbles held x16)
        const int r = eb & 7, m = r >> 1, u = r & 1;
        j = eb >> 3;
        h = (m & 1) * 4 + u * 2 + (m >> 1);
        hi = u != 0;
        return;
    }
    if constexpr (FMT == FQ1_0) {
        // lane column j takes elements 4j + t and 4j + t + 16 as the pair t (halves 2t, 2t + 1)
        j = (eb & 15) >> 2;
        h = 2 * (eb & 3) + (eb >> 4);
        hi = false;
        return;
    }
    const int second = eb >= 16, e = eb & 15, t = e & 3;
    j = e >> 2;
    if constexpr (FMT == FQ4_0) {
        // halves: [lo b0, lo b2, hi b0, hi b2, lo b1, lo b3, hi b1, hi b3]
        h = (t & 1) * 4 + second * 2 + (t >> 1);
        hi = second;
    } else {
        // byte-like formats (Q8_0; nibbles joined with high bits, codebook entries, K-quant
        // sub-blocks over two chunks): halves [b0, b2, b1, b3] of the first 16 elements'
        // dword, then of the second 16's
        h = 4 * second + (t == 0 ? 0 : t == 2 ? 1 : t == 1 ? 2 : 3);
        hi = false;
    }
}

// Q4_K B operand of one 32-weight sub-block: the low nibbles of dwords q0 and q1 (the sub-block's
// two 16-byte chunks; a high-nibble sub-block passes q >> 4) as the exact centred weights n - c,
// with off the f16 pair -(1024 + c) (mf_splat_off).  Halves: [b0, b2, b1, b3] of q0, then of q1.
__device__ __forceinline__ mh8 mf_bop_k(uint32_t q0, uint32_t q1, uint32_t off, const MfConst &k)
{
    struct W4 {
        uint32_t v[4];
    } p = {{mf_hadd(mf_and_or(q0, k.m_lo, k.c), off), mf_hadd(mf_and_or(q0 >> 8, k.m_lo, k.c), off),
            mf_hadd(mf_and_or(q1, k.m_lo, k.c), off), mf_hadd(mf_and_or(q1 >> 8, k.m_lo, k.c), off)}};
    return __builtin_bit_cast(mh8, p);
}

// The f16 pair -(1024 + c), c an integer in [0, 1023] (exact).
__device__ __forceinline__ uint32_t mf_splat_off(float c)
{
    const uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)(-1024.0f - c));
    return h | (h << 16);
}

// All-ones B operand (sums of the A operand's k values).
__device__ __forceinline__ mh8 kc_ones()
{
    const _Float16 o = (_Float16)1.0f;
    return mh8{o, o, o, o, o, o, o, o};
}

// The affine format's sum operand: 1 at low-nibble positions, 16 at high-nibble ones (whose x
// the A operand holds / 16), so the product is the plain sum of the block's x.
__device__ __forceinline__ mh8 mf_ones_q4()
{
    const _Float16 o = (_Float16)1.0f, s = (_Float16)16.0f;
    return mh8{o, o, s, s, o, o, s, s};
}

// B operand of four weight bytes per half: bytes 0, 2 and 1, 3 of u0, then of u1, each in the
// mantissa of 1024.0 and moved by the f16 pair off (exact).
__device__ __forceinline__ mh8 mf_bop_bytes(uint32_t u0, uint32_t u1, uint32_t off, const MfConst &k)
{
    struct W4 {
        uint32_t v[4];
    } p = {{mf_hadd(mf_and_or(u0, k.m_b, k.c), off), mf_hadd(mf_and_or(u0 >> 8, k.m_b, k.c), off),
            mf_hadd(mf_and_or(u1, k.m_b, k.c), off), mf_hadd(mf_and_or(u1 >> 8, k.m_b, k.c), off)}};
    return __builtin_bit_cast(mh8, p);
}

// Q5 formats: dword j of a chunk's nibbles joined with their fifth bits (h: the chunk's high-bit
// word as packed, the bit of the low nibble of byte 4k + m at bit 8m + k, of the high nibble at
// 8m + 4 + k) into four bytes: the low nibbles (mf_join5_lo) or the high ones (mf_join5_hi).
__device__ __forceinline__ uint32_t mf_join5_lo(uint32_t q, uint32_t h, int j)
{
    return mf_and_or(q, 0x0F0F0F0Fu, (h << (4 - j)) & 0x10101010u);
}
__device__ __forceinline__ uint32_t mf_join5_hi(uint32_t q, uint32_t h, int j)
{
    return mf_and_or(q >> 4, 0x0F0F0F0Fu, (h >> j) & 0x10101010u);
}

// IQ4 formats: the codebook entries of four indices (bits 0-2 in idx7, bit 3 at bit 2 of each
// byte of b3) from the table T (entries + 128), as the two f16 pairs (bytes 0, 2) and (1, 3),
// exact signed entries: entries 0-7 and 8-15 by one permute each, a third picks per byte, two
// more place the bytes under 0x64 (f16 1024 + u), one packed add each removes 1152.
__device__ __forceinline__ void mf_cb_pairs(uint32_t idx7, uint32_t b3, const uint4 &T,
                                            const MfConst &k, uint32_t &w02, uint32_t &w13)
{
    const uint32_t lo = __builtin_amdgcn_perm(T.y, T.x, idx7);
    const uint32_t hi = __builtin_amdgcn_perm(T.w, T.z, idx7);
    const uint32_t r = __builtin_amdgcn_perm(hi, lo, mf_and_or(b3, k.m_sel, k.c_id));
    w02 = mf_hadd(__builtin_amdgcn_perm(k.c64, r, 0x04020400u), 0xE480E480u);
    w13 = mf_hadd(__builtin_amdgcn_perm(k.c64, r, 0x04030401u), 0xE480E480u);
}

// B operand of an IQ4 block from dword j of its chunk: entries of the low nibbles (elements
// 4j..4j+3), then of the high nibbles (16 + 4j..): the byte-like half order.
__device__ __forceinline__ mh8 mf_bop_cb(uint32_t q, const uint4 &T, const MfConst &k)
{
    struct W4 {
        uint32_t v[4];
    } p;
    mf_cb_pairs(q & 0x07070707u, q >> 1, T, k, p.v[0], p.v[1]);
    mf_cb_pairs((q >> 4) & 0x07070707u, q >> 5, T, k, p.v[2], p.v[3]);
    return __builtin_bit_cast(mh8, p);
}

// Affine Q4 B operand of dword j (elements 8j..8j+7): Q4_0's pair order with the centring offsets
// off_lo = -(1024 + c), off_hi = -(1024 + 16 c): exact q - c and 16 (q - c).
__device__ __forceinline__ mh8 mf_bop_aq(uint32_t q, uint32_t off_lo, uint32_t off_hi,
                                         const MfConst &k)
{
    const uint32_t t = q >> 8;
    struct W4 {
        uint32_t v[4];
    } p = {{mf_hadd(mf_and_or(q, k.m_lo, k.c), off_lo), mf_hadd(mf_and_or(q, k.m_hi, k.c), off_hi),
            mf_hadd(mf_and_or(t, k.m_lo, k.c), off_lo), mf_hadd(mf_and_or(t, k.m_hi, k.c), off_hi)}};
    return __builtin_bit_cast(mh8, p);
}

// 4 x 4 transpose of dwords across the four 16-lane rows: register r of lane row c holds dword
// c of row r's chunk afterwards.
__device__ __forceinline__ void mf_xpose(uint32_t (&v)[4])
{
    auto s0 = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
    auto s1 = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
    auto t0 = __builtin_amdgcn_permlane16_swap(s0[0], s1[0], false, false);
    auto t1 = __builtin_amdgcn_permlane16_swap(s0[1], s1[1], false, false);
    v[0] = t0[0];
    v[1] = t0[1];
    v[2] = t1[0];
    v[3] = t1[1];
}


// Block element (0..31) at half h of dword j of the A / B operands (the inverse of mf_slot), and
// whether it carries the 1/16 of a high nibble.
template <int FMT>
__device__ __forceinline__ int mf_elem(int j, int h, bool &hi)
{
    static_assert(FMT != FAQ4 && FMT != FQ6_K, "no inverse layout here");
    if constexpr (FMT == FQ1_0) {
        // pair t = h / 2 of lane column j: elements 4j + t (low half) and 4j + t + 16 (high)
        hi = false;
        return 4 * j + (h >> 1) + 16 * (h & 1);
    } else if constexpr (FMT != FQ4_0) {
        // halves: [b0, b2, b1, b3] of half 0, then of half 1
        const int second = h >> 2, t4 = h & 3;
        const int t = t4 == 0 ? 0 : t4 == 1 ? 2 : t4 == 2 ? 1 : 3;
        hi = false;
        return 16 * second + 4 * j + t;
    } else {
        // halves: [lo b0, lo b2, hi b0, hi b2, lo b1, lo b3, hi b1, hi b3]
        const int second = (h >> 1) & 1, t = ((h >> 2) & 1) | ((h & 1) << 1);
        hi = second != 0;
        return 16 * second + 4 * j + t;
    }
}

}  // namespace qg

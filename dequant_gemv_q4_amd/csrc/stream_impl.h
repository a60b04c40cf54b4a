// stream_impl.h -- the streaming dequant-GEMV kernel templates of libqgemv for gfx950 (included by
// stream_kernels.hip and stream_kernels_x.hip, which instantiate them per format).
//
// One wave64 owns whole rows: lane l takes the 16-byte quant chunk l (and l + 64, ... when a
// row is split over several waves) of R rows at a time, so every weight load instruction reads
// 1 KB contiguous.  Each wave keeps PD row groups in flight: the quants and scales of its next
// groups stream in while it decodes the current one.  x (or x * gamma for the norm prologue) is
// staged once per workgroup in LDS; each lane turns its own chunk of x into f16 pairs once.
// R x NB partial sums leave the wave through a transposed butterfly (each exchange halves the
// number of values a lane carries), and one lane per (row, batch row) runs the epilogue.
//
// Decode: a Q4_0 byte holds element j in its low nibble and element j + 16 in its high nibble
// (GGUF order).  Nibbles become exact f16 weights by an and-or into the mantissa of 1024.0, two
// per instruction, then one packed f16 add removes the 1024 mantissa offset together with the
// format's own offset (Q4_0's -8, "Crate inferencelayer" docs, q4_0_to_q8_0n: q8 = nib - 8), so
// the dot operands are the exact signed weights; they meet x through v_dot2_f32_f16 (two f16
// products, exact in f32, added to an f32 accumulator).  No offset is cancelled in the sums.
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "qgemv.h"

namespace qg {

// ------------------------------------------------------------------------------------ helpers

// Value of lane (l ^ OFF), every partner exact: OFF 1 and 2 by DPP quad permutes, 8 by DPP
// row rotation, 4 and 16 by ds_swizzle (bit mode, xor mask), 32 by ds_bpermute (bp32 holds
// ((l ^ 32) << 2), computed once).
template <int OFF>
__device__ __forceinline__ float xor_lane(float v, int bp32)
{
    const int iv = __float_as_int(v);
    int r;
    if constexpr (OFF == 1)
        r = __builtin_amdgcn_update_dpp(0, iv, 0xB1, 0xF, 0xF, true);    // quad_perm [1,0,3,2]
    else if constexpr (OFF == 2)
        r = __builtin_amdgcn_update_dpp(0, iv, 0x4E, 0xF, 0xF, true);    // quad_perm [2,3,0,1]
    else if constexpr (OFF == 8)
        r = __builtin_amdgcn_update_dpp(0, iv, 0x128, 0xF, 0xF, true);   // row_ror:8
    else if constexpr (OFF == 4)
        r = __builtin_amdgcn_ds_swizzle(iv, (4 << 10) | 0x1F);
    else if constexpr (OFF == 16)
        r = __builtin_amdgcn_ds_swizzle(iv, (16 << 10) | 0x1F);
    else
        r = __builtin_amdgcn_ds_bpermute(bp32, iv);
    return __int_as_float(r);
}

// One butterfly stage at offset OFF.  Transposed (H > 0): the lane keeps items [0, H) or
// [H, 2H) (by its OFF bit), sends the other half to its partner and adds what it receives.
template <int OFF, int IP, int P>
__device__ __forceinline__ void bfly_stage(float (&v)[IP][P], int lane, int bp32, int H)
{
    const bool up = (lane & OFF) != 0;
#pragma unroll
    for (int i = 0; i < IP; ++i)
        if (i < (H > 0 ? H : 1))
#pragma unroll
            for (int p = 0; p < P; ++p) {
                if (H > 0) {
                    const float keep = up ? v[H + i][p] : v[i][p];
                    const float send = up ? v[i][p] : v[H + i][p];
                    v[i][p] = keep + xor_lane<OFF>(send, bp32);
                } else {
                    v[i][p] += xor_lane<OFF>(v[i][p], bp32);
                }
            }
}

// Butterfly that leaves, in lane l, the 64-lane total of item (l >> (6 - log2 IP)) in v[0][*].
// The first log2 IP stages are transposed (each halves the items a lane carries), the rest
// plain.  Every stage pairs lane l with l ^ off, off = 32, 16, ..., 1 in that order, so an
// item's sum has the same association whatever IP is.
template <int IP, int P>
__device__ __forceinline__ void xpose_reduce(float (&v)[IP][P], int lane, int bp32)
{
    constexpr int L = IP == 1 ? 0 : IP == 2 ? 1 : IP == 4 ? 2 : IP == 8 ? 3 : IP == 16 ? 4 : 5;
    static_assert((1 << L) == IP, "item count must be a power of two <= 32");
    bfly_stage<32>(v, lane, bp32, L > 0 ? IP >> 1 : 0);
    bfly_stage<16>(v, lane, bp32, L > 1 ? IP >> 2 : 0);
    bfly_stage<8>(v, lane, bp32, L > 2 ? IP >> 3 : 0);
    bfly_stage<4>(v, lane, bp32, L > 3 ? IP >> 4 : 0);
    bfly_stage<2>(v, lane, bp32, L > 4 ? IP >> 5 : 0);
    bfly_stage<1>(v, lane, bp32, 0);
}

constexpr int pow2_ceil(int v) { return v <= 1 ? 1 : 2 * pow2_ceil((v + 1) / 2); }

// Compile-time shape of the streaming kernels.  KS: waves that share one row.
template <int FMT, int NB, int CPL, int MATS, int KS = 1>
struct SP {
    static constexpr int R = stream_rows_fmt(FMT, NB, CPL, MATS);
    static constexpr int XF4 = Fc<FMT>::XF4, CE = Fc<FMT>::CE, NS = Fc<FMT>::NS;
    // waves per SIMD the register budget must allow (at most 512 / WPE VGPRs per lane): a row
    // batch of 2..4 on one matrix with one wave per row holds its x pairs in about 120 VGPRs,
    // so three waves fit (more waves to hide the longer decode of several batch rows); rows
    // split over several waves are short, and fewer, smaller workgroups start sooner there
    // (the super-block, high-bit and codebook formats hold more per chunk: two waves per SIMD)
    static constexpr int WPE = (NB == 1 && CPL == 1 && !fmt_super(FMT) && !fmt_hbits(FMT))
                                   ? QG_WPE_NB1
                             : (NB > 1 && KS == 1 && MATS == 1 && !fmt_super(FMT) &&
                                !fmt_hbits(FMT) && !fmt_codebook(FMT)) ? 3 : 2;
    static constexpr int ITEMS = R * NB;
    static constexpr int IP = pow2_ceil(ITEMS);
    // GEMV family: one workgroup fills a CU (WPE waves on each of its 4 SIMDs)
    static constexpr int WV = 4 * WPE, NT = 64 * WV;
};

// Raw scale bytes as loaded: one f16 (kept 16-bit, so nothing has to mask a load's result before
// it is used), the 16-byte Q4_K / Q5_K header, or Q6_K's eight scales of the chunk's half
// super-block (x, y) and its f16 d (z).
template <int FMT>
struct ScaleT {
    using T = uint16_t;
};
template <>
struct ScaleT<FQ4_K> {
    using T = uint4;
};
template <>
struct ScaleT<FQ5_K> {
    using T = uint4;
};
template <>
struct ScaleT<FQ6_K> {
    using T = uint4;
};
template <>
struct ScaleT<FIQ4_XS> {   // f16 d and the 16-bit word of high scale bits; the low 4-bit scales
    using T = uint2;
};
template <>
struct ScaleT<FAQ4> {      // f16 scale and f16 bias
    using T = uint32_t;
};

// Loads of one row group: for each matrix, row and chunk slot, 16 bytes of quants, the scale and
// (high-bit formats) the chunk's high-bit words.
template <int FMT, int CPL, int MATS, int R>
struct GroupBuf {
    static constexpr int HW = fmt_hwords(FMT) > 0 ? fmt_hwords(FMT) : 1;
    uint4 q[MATS][R][CPL];
    typename ScaleT<FMT>::T s[MATS][R][CPL];
    uint32_t h[MATS][R][CPL][HW];
    uint32_t sw;   // one-load scales: dword `lane` of the group's scale bytes, as loaded
};

// A packed matrix seen through buffer resources (quant plane, scale plane, and for the high-bit
// formats the high-bit plane and Q6_K's d plane).  A lane's chunk offset is a constant VGPR.
// A load whose (vector) offset is at or past the plane's size returns zeros without a memory
// request: q_end / s_end / h_end / d_end (the sizes) are added to the offsets of loads that must
// move no data.  Row offsets go in the vector offset too, so that every load is range-checked.
struct BufMat {
    __amdgpu_buffer_rsrc_t q, s, h, d;
    uint32_t q_end, s_end, h_end, d_end;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t plane_rsrc(const uint8_t *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ BufMat buf_mat(const uint8_t *qs, const uint8_t *sc, uint32_t q_bytes,
                                          uint32_t s_bytes, const uint8_t *hb = nullptr,
                                          uint32_t h_bytes = 0, const uint8_t *dd = nullptr,
                                          uint32_t d_bytes = 0)
{
    BufMat m;
    m.q_end = q_bytes;
    m.s_end = s_bytes;
    m.h_end = h_bytes;
    m.d_end = d_bytes;
    m.q = plane_rsrc(qs, q_bytes);
    m.s = plane_rsrc(sc, s_bytes);
    m.h = plane_rsrc(hb ? hb : qs, h_bytes);
    m.d = plane_rsrc(dd ? dd : qs, d_bytes);
    return m;
}

// Bytes per row of each plane (as the 32-bit offsets the loads take).
struct RowB {
    uint32_t q, s, h, d;
};

// Byte offsets of a lane's chunk slots inside a row.  A slot past the row's C chunks reads the
// row's last chunk and gets a zero scale, so it adds exactly nothing.
template <int CPL>
struct LaneOff {
    uint32_t q[CPL], s[CPL], h[CPL], d[CPL];
    uint32_t w4;   // 4 * lane: the lane's dword of a group's scale bytes (one-load scales)
    bool ok[CPL];
};

template <int FMT, int CPL>
__device__ __forceinline__ LaneOff<CPL> lane_offsets(int lane, int C)
{
    LaneOff<CPL> o;
    o.w4 = 4u * (uint32_t)(lane & 63);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        o.ok[i] = c < C;
        const uint32_t cx = (uint32_t)(c < C ? c : C - 1);
        o.q[i] = cx * (uint32_t)fmt_chunk_bytes(FMT);
        o.s[i] = (FMT == FQ4_0 || FMT == FQ5_0 || FMT == FIQ4_NL) ? cx * 2u
               : FMT == FQ8_0 ? (cx >> 1) * 2u
               : FMT == FQ1_0 ? (cx >> 2) * 2u
               : FMT == FAQ4 ? cx * 4u
               : FMT == FIQ4_XS ? (cx >> 3) * 8u
               : FMT == FQ6_K ? (cx >> 3) * 16u + ((cx & 7u) >> 2) * 8u
                              : (cx >> 3) * 16u;
        o.h[i] = cx * 4u * (uint32_t)(fmt_hwords(FMT) > 0 ? fmt_hwords(FMT) : 1);
        o.d[i] = (cx >> 3) * 2u;
    }
    return o;
}

// Loads of one row group, unconditional so the compiler can count them exactly in its
// s_waitcnt.  A row outside [0, N) (a group index < 0 marks a group with no result) is loaded
// out of range: zeros, no memory traffic; its results are dropped by the epilogue.
// SCW (one-load scales; one matrix, rows of at most 64 chunks): the scale bytes of all R rows of
// the group are contiguous and at most 256, so each lane loads one dword of them and the block
// scales reach their lanes by a cross-lane permute when the group is decoded (one load
// instruction instead of R two-byte loads).
template <int FMT, int CPL, int MATS, int R, bool SCW = false>
__device__ __forceinline__ void load_group(GroupBuf<FMT, CPL, MATS, R> &b, const BufMat (&mat)[MATS],
                                           const RowB &rw, int64_t N, const LaneOff<CPL> &lo,
                                           int64_t g)
{
    const uint32_t qs_row = rw.q, sc_row = rw.s;
    static_assert(!SCW || (MATS == 1 && CPL == 1), "one-load scales: one matrix, one chunk slot");
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int64_t nr = g * R + u;   // wave-uniform
        const bool in = nr >= 0 && nr < N;
        const uint32_t n = (uint32_t)(in ? nr : 0);
#pragma unroll
        for (int m = 0; m < MATS; ++m)
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const uint32_t roq = in ? n * qs_row : mat[m].q_end;
                const uint32_t ros = in ? n * sc_row : mat[m].s_end;
                if constexpr (FMT == FQ1_0) {
                    b.q[m][u][i] = make_uint4(__builtin_amdgcn_raw_buffer_load_b32(
                                                  mat[m].q, (int)(lo.q[i] + roq), 0, QG_WCPOL_STREAM),
                                              0u, 0u, 0u);
                } else {
                    const auto v = __builtin_amdgcn_raw_buffer_load_b128(
                        mat[m].q, (int)(lo.q[i] + roq), 0, QG_WCPOL_STREAM);
                    b.q[m][u][i] = make_uint4(v[0], v[1], v[2], v[3]);
                }
                // raw scale bytes: the lane mask is applied where they are used, so that no
                // instruction touches a load's result before its group is decoded
                if constexpr (SCW) {
                    (void)ros;
                } else if constexpr (fmt_min(FMT)) {
                    const auto w = __builtin_amdgcn_raw_buffer_load_b128(
                        mat[m].s, (int)(lo.s[i] + ros), 0, QG_WCPOL_STREAM);
                    b.s[m][u][i] = make_uint4(w[0], w[1], w[2], w[3]);
                } else if constexpr (FMT == FIQ4_XS) {
                    const auto w = __builtin_amdgcn_raw_buffer_load_b64(
                        mat[m].s, (int)(lo.s[i] + ros), 0, QG_WCPOL_STREAM);
                    b.s[m][u][i] = make_uint2(w[0], w[1]);
                } else if constexpr (FMT == FAQ4) {
                    b.s[m][u][i] = __builtin_amdgcn_raw_buffer_load_b32(
                        mat[m].s, (int)(lo.s[i] + ros), 0, QG_WCPOL_STREAM);
                } else if constexpr (FMT == FQ6_K) {
                    const auto w = __builtin_amdgcn_raw_buffer_load_b64(
                        mat[m].s, (int)(lo.s[i] + ros), 0, QG_WCPOL_STREAM);
                    const uint32_t rod = in ? n * rw.d : mat[m].d_end;
                    const uint32_t dv = __builtin_amdgcn_raw_buffer_load_b16(
                        mat[m].d, (int)(lo.d[i] + rod), 0, QG_WCPOL_STREAM);
                    b.s[m][u][i] = make_uint4(w[0], w[1], dv, 0u);
                } else {
                    b.s[m][u][i] = __builtin_amdgcn_raw_buffer_load_b16(
                        mat[m].s, (int)(lo.s[i] + ros), 0, QG_WCPOL_STREAM);
                }
                if constexpr (fmt_hwords(FMT) == 1) {
                    const uint32_t roh = in ? n * rw.h : mat[m].h_end;
                    b.h[m][u][i][0] = __builtin_amdgcn_raw_buffer_load_b32(
                        mat[m].h, (int)(lo.h[i] + roh), 0, QG_WCPOL_STREAM);
                } else if constexpr (fmt_hwords(FMT) == 2) {
                    const uint32_t roh = in ? n * rw.h : mat[m].h_end;
                    const auto hv = __builtin_amdgcn_raw_buffer_load_b64(
                        mat[m].h, (int)(lo.h[i] + roh), 0, QG_WCPOL_STREAM);
                    b.h[m][u][i][0] = hv[0];
                    b.h[m][u][i][1] = hv[1];
                }
            }
    }
    if constexpr (SCW) {
        const bool gin = g >= 0 && g * R < N;
        const uint32_t so = gin ? (uint32_t)(g * R) * sc_row + lo.w4 : mat[0].s_end;
        b.sw = __builtin_amdgcn_raw_buffer_load_b32(mat[0].s, (int)so, 0, QG_WCPOL_STREAM);
    }
}

template <int FMT>
__device__ __forceinline__ ChunkScale scale_of(uint16_t s, int) { ChunkScale cs; cs.a = (float)__builtin_bit_cast(_Float16, s); cs.b = cs.a2 = cs.b2 = 0.f; return cs; }
template <int FMT>
__device__ __forceinline__ ChunkScale scale_of(const uint4 &s, int qpos) { return chunk_scale<FMT>(s, qpos); }
template <int FMT>
__device__ __forceinline__ ChunkScale scale_of(const uint2 &s, int qpos) { return chunk_scale<FMT>(make_uint4(s.x, s.y, 0u, 0u), qpos); }
template <int FMT>
__device__ __forceinline__ ChunkScale scale_of(uint32_t s, int qpos) { return chunk_scale<FMT>(make_uint4(s, 0u, 0u, 0u), qpos); }

// Workgroup-shared x.  A few loader waves each load float4s base + stride * i of the NB rows
// (and of gamma) and write them to LDS (natural [row][K] order).  With NRM the stored value is
// x * gamma, and beside it the sum of squares of each float4 of raw x, so every wave can form a
// row's norm in a fixed order; every float4 also gets its largest |value| (the row scale).
template <int NB, bool NRM, int XPT>
struct XStage {
    float4 v[XPT];
    float4 g[NRM ? XPT : 1];
};

template <int NB, bool NRM, int XPT>
__device__ __forceinline__ void xstage_issue(XStage<NB, NRM, XPT> &st, const float *x,
                                             const float *gamma, int K4, int base, int stride)
{
    const int tot = NB * K4;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int f = base + stride * i;
        const int fc = f < tot ? f : tot - 1;
        st.v[i] = reinterpret_cast<const float4 *>(x)[fc];
        if constexpr (NRM)
            st.g[i] = reinterpret_cast<const float4 *>(gamma)[NB == 1 ? fc : fc % K4];
    }
}

// Threads past the end store at the last index the value loaded for it (the same value as the
// thread that owns it), so the stores, and the loads before them, are unconditional: a load
// used only under a branch would be sunk below the weight loads.
template <int NB, bool NRM, int XPT>
__device__ __forceinline__ void xstage_store(const XStage<NB, NRM, XPT> &st, int K4, int base,
                                             int stride, float4 *X4, float *SS)
{
    const int tot = NB * K4;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int f = base + stride * i;
        const int fc = f < tot ? f : tot - 1;
        float4 v = st.v[i];
        if constexpr (NRM) {
            float q = v.x * v.x;
            q = fmaf(v.y, v.y, q);
            q = fmaf(v.z, v.z, q);
            q = fmaf(v.w, v.w, q);
            SS[fc] = q;
            const float4 g = st.g[i];
            v = make_float4(v.x * g.x, v.y * g.y, v.z * g.z, v.w * g.w);
        }
        X4[fc] = v;
    }
}

// ------------------------------------------------------------------------------------ f16 pairs
//
// The streaming GEMV forms its dot products with v_dot2_f32_f16: two f16 products (exact in
// f32) added to an f32 accumulator.  Weights: a nibble n placed in the mantissa of the f16
// 0x6400 (1024.0) reads as 1024 + n, and a nibble in mantissa bits 4..7 as 1024 + 16 n, so one
// and-or per dword yields two weights (exact); the x operand of a high-nibble pair carries a
// factor 1/16.  x: the values of each chunk (the 16 or 32 x elements one 16-byte quant chunk
// multiplies) are scaled by a power of two that puts their largest |value| in [2^14, 2^15), then
// rounded to f16 (relative error at most 2^-11, far inside the stated 1e-3 * sum|w x| bound); the
// scale is undone, exactly, on the chunk's partial sums.  The 1024 mantissa offset, and Q4_0's
// -8 and Q8_0's +128 bias, are removed from every weight pair by one exact packed f16 add before
// the dot, so a dot sums exact products of the true weights: its rounding error is relative to
// sum |w x|, whatever the weights (a weight pattern of mostly-zero weights cancels nothing).
typedef _Float16 qg_h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(qg_h2, w), __builtin_bit_cast(qg_h2, x), c,
                                  false);
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b)
{
    const _Float16 ha = (_Float16)a, hb = (_Float16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, ha) |
           ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// x of a lane's CPL chunk slots for every batch row, as f16 pairs in dot order, and the offset
// sums of each slot.
template <int FMT, int NB, int CPL = 1>
struct XH {
    static constexpr int NP = FMT == FQ8_0 ? 8 : 16;   // pairs per 16-byte chunk
    static constexpr int NZ = fmt_min(FMT) ? 2 : 1;
    uint32_t p[NB][CPL][NP];
    float z[NB][CPL][NZ];   // Q4_K / Q5_K: S_A, S_B, the x sums of the two sub-blocks (others: unused)
};

// (v & m) | c in one instruction.  A three-operand instruction of this target takes no literal
// and one scalar operand at most, so the masks and the constant live in VGPRs (set once).
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t m, uint32_t c)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "v"(m), "v"(c));
    return r;
}

// Loop-invariant operands of w_pairs, kept in VGPRs: the masks, the 1024.0 pair, and the f16
// pairs added to remove the offsets (low nibble / byte, high nibble held x16).
struct WConst {
    uint32_t m_lo, m_hi, c, off_lo, off_hi, m_nb, m_hb;
    uint4 cb[2];   // IQ4 formats: the codebooks of the (up to two) matrices, each byte + 128
};

template <int FMT>
__device__ __forceinline__ WConst w_const()
{
    WConst k;
    // byte formats (Q8_0, the high-bit formats, whose nibbles and high bits are first joined into
    // bytes, and the codebook formats, whose looked-up entries are bytes) take bytes 0 / 2 of a
    // dword; the Q4 formats take nibbles; Q1_0 takes the sign bits of a pair (its c: 1.0, 1.0)
    k.m_lo = (FMT == FQ8_0 || fmt_hbits(FMT) || fmt_codebook(FMT)) ? 0x00FF00FFu
           : FMT == FQ1_0 ? 0x80008000u : 0x000F000Fu;
    k.m_hi = 0x00F000F0u;
    k.c = FMT == FQ1_0 ? 0x3C003C00u : 0x64006400u;
    // Q4_0: -1032 (1024 + n -> n - 8), -1152 (1024 + 16 n -> 16 (n - 8)); Q8_0: -1152
    // (1024 + q + 128 -> q); Q5_0: -1040 (1024 + q -> q - 16); Q6_K: -1056 (1024 + q -> q - 32);
    // Q4_K / Q5_K: set per sub-block from its centre (see compute_group_h)
    k.off_lo = FMT == FQ4_0 ? 0xE408E408u : (FMT == FQ8_0 || fmt_codebook(FMT)) ? 0xE480E480u
             : FMT == FQ5_0 ? 0xE410E410u : FMT == FQ6_K ? 0xE420E420u : 0xE400E400u;
    k.off_hi = FMT == FQ4_0 ? 0xE480E480u : fmt_hbits(FMT) ? k.off_lo : 0xE400E400u;
    k.m_nb = 0x0F0F0F0Fu;                                  // the nibbles of four bytes
    k.m_hb = FMT == FQ6_K ? 0x30303030u : 0x10101010u;     // their high bits' places
    if constexpr (fmt_codebook(FMT)) {
        // codebook lookups (cb_pairs): bit 2 of each byte, the identity byte selectors, and the
        // high byte of f16 1024 + u in every byte
        k.m_hi = 0x04040404u;
        k.c = 0x03020100u;
        k.m_nb = 0x64646464u;
    }
    k.cb[0] = k.cb[1] = make_uint4(0u, 0u, 0u, 0u);
    asm volatile("" : "+v"(k.m_lo), "+v"(k.m_hi), "+v"(k.c), "+v"(k.off_lo), "+v"(k.off_hi),
                 "+v"(k.m_nb), "+v"(k.m_hb));
    return k;
}

// Exact packed f16 sum of two pairs (every result here is a small integer times a power of two).
__device__ __forceinline__ uint32_t h2_add(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(qg_h2, a) + __builtin_bit_cast(qg_h2, b));
}

// The f16 value v (exact: an integer below 2048 in magnitude) in both halves of a pair.
__device__ __forceinline__ uint32_t h2_splat(float v)
{
    const uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)v);
    return h | (h << 16);
}

// Exact signed weight pairs of one dword of a 16-byte chunk, in dot order.
template <int FMT>
__device__ __forceinline__ void w_pairs(uint32_t q, const WConst &k, uint32_t *w)
{
    if constexpr (FMT == FQ8_0) {
        const uint32_t u = q ^ 0x80808080u;                          // q + 128 as unsigned bytes
        w[0] = h2_add(and_or(u, k.m_lo, k.c), k.off_lo);             // bytes 0, 2
        w[1] = h2_add(and_or(u >> 8, k.m_lo, k.c), k.off_lo);        // bytes 1, 3
    } else {
        const uint32_t t = q >> 8;
        w[0] = h2_add(and_or(q, k.m_lo, k.c), k.off_lo);   // low nibbles of bytes 0, 2
        w[1] = h2_add(and_or(q, k.m_hi, k.c), k.off_hi);   // high nibbles of bytes 0, 2 (x16)
        w[2] = h2_add(and_or(t, k.m_lo, k.c), k.off_lo);   // low nibbles of bytes 1, 3
        w[3] = h2_add(and_or(t, k.m_hi, k.c), k.off_hi);   // high nibbles of bytes 1, 3 (x16)
    }
}

// Exact signed weight pairs of dword K of a chunk of a high-bit format, in dot order (as w_pairs:
// low-nibble bytes 0, 2; high-nibble bytes 0, 2; low 1, 3; high 1, 3).  h0 / h1: the chunk's
// high-bit words as k_pack lays them out (Q5: bit 8m + K of h0 is the fifth bit of the low nibble
// of byte m, bit 8m + 4 + K that of its high nibble; Q6_K: bits 8m + 2K, +1 of h0 / h1 the two
// high bits of the low / high nibble).  One shift and one and-or put them at bit 4 (4-5) of each
// byte beside its nibble, and the bytes become pairs as Q8_0's do.
template <int FMT, int K>
__device__ __forceinline__ void w_pairs_hb(uint32_t q, uint32_t h0, uint32_t h1, const WConst &k,
                                           uint32_t *w)
{
    uint32_t hl, hh;
    if constexpr (FMT == FQ6_K) {
        hl = K <= 2 ? h0 << (4 - 2 * K) : h0 >> (2 * K - 4);
        hh = K <= 2 ? h1 << (4 - 2 * K) : h1 >> (2 * K - 4);
    } else {
        (void)h1;
        hl = h0 << (4 - K);
        hh = h0 >> K;
    }
    const uint32_t lo = and_or(q, k.m_nb, hl & k.m_hb);          // low nibbles + high bits
    const uint32_t hi = and_or(q >> 4, k.m_nb, hh & k.m_hb);     // high nibbles + high bits
    w[0] = h2_add(and_or(lo, k.m_lo, k.c), k.off_lo);
    w[1] = h2_add(and_or(hi, k.m_lo, k.c), k.off_hi);
    w[2] = h2_add(and_or(lo >> 8, k.m_lo, k.c), k.off_lo);
    w[3] = h2_add(and_or(hi >> 8, k.m_lo, k.c), k.off_hi);
}

// Codebook formats: the pairs of dword q of a chunk in Q4_0's pair order (low-nibble entries of
// bytes 0, 2; high-nibble entries of bytes 0, 2; low 1, 3; high 1, 3).  T holds every entry
// + 128 as an unsigned byte; four indices are looked up as in cb_lookup (entries 0-7 and 8-15 by
// one permute each, with bit 3 of the index dropped, then a per-byte choice by bit 3, taken from
// q itself), and two permutes then place bytes 0, 2 and 1, 3 of the result under the byte 0x64:
// f16 1024 + entry + 128, from which the exact signed entry is one packed add away (-1152).
__device__ __forceinline__ void cb_pairs(uint32_t idx7, uint32_t b3, const WConst &k,
                                         const uint4 &T, uint32_t &w02, uint32_t &w13)
{
    const uint32_t lo = __builtin_amdgcn_perm(T.y, T.x, idx7);
    const uint32_t hi = __builtin_amdgcn_perm(T.w, T.z, idx7);
    const uint32_t r = __builtin_amdgcn_perm(hi, lo, and_or(b3, k.m_hi, k.c));
    w02 = h2_add(__builtin_amdgcn_perm(k.m_nb, r, 0x04020400u), k.off_lo);
    w13 = h2_add(__builtin_amdgcn_perm(k.m_nb, r, 0x04030401u), k.off_lo);
}

__device__ __forceinline__ void w_pairs_cb(uint32_t q, const WConst &k, const uint4 &T, uint32_t *w)
{
    // bit 3 of each low nibble moved to bit 2 of its byte (q >> 1), of each high nibble (q >> 5)
    cb_pairs(q & 0x07070707u, q >> 1, k, T, w[0], w[2]);
    cb_pairs((q >> 4) & 0x07070707u, q >> 5, k, T, w[1], w[3]);
}

// Q1_0: pair p (p < 16) of the chunk's 32 sign bits is (element p, element p + 16) as f16 +-1:
// the inverted bits p and p + 16 shifted to bits 15 and 31 (the f16 sign bits) over 1.0, 1.0.
__device__ __forceinline__ void w_pairs_q1(uint32_t q, const WConst &k, uint32_t *w)
{
    const uint32_t v = ~q;
#pragma unroll
    for (int p = 0; p < 16; ++p)
        w[p] = and_or(v << (15 - p), k.m_lo, k.c);
}

// Dot chains of one chunk for one batch row: d[0] (two-sub-block formats: low-nibble chain d[0],
// high d[1]).
template <int FMT>
__device__ __forceinline__ void chunk_chains(const uint32_t (&w)[FMT == FQ8_0 ? 8 : 16],
                                             const uint32_t *x, float *d)
{
    if constexpr (FMT == FQ8_0) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            a = dot2(w[i], x[i], a);
        d[0] = a;
    } else if constexpr (!fmt_two_sub(FMT)) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            a = dot2(w[i], x[i], a);
        d[0] = a;
    } else {
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a = dot2(w[4 * i + 0], x[4 * i + 0], a);
            b = dot2(w[4 * i + 1], x[4 * i + 1], b);
            a = dot2(w[4 * i + 2], x[4 * i + 2], a);
            b = dot2(w[4 * i + 3], x[4 * i + 3], b);
        }
        d[0] = a;
        d[1] = b;
    }
}

// x pairs of one chunk (its float4s xv in chunk_elem order), scaled by sc; the min formats also
// the sums of the two sub-blocks' rounded, scaled x (the (a c - b) terms multiply them).  The Q4
// formats' high-nibble pairs carry 1/16 (their weights are held x16); the high-bit formats
// decode every weight from a whole byte and take x as it is.
template <int FMT>
__device__ __forceinline__ void x_pairs(const float4 *xv, float sc, uint32_t *p, float *z)
{
    if constexpr (FMT == FQ1_0) {
        // pair p: elements p and p + 16
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[4 * i + 0] = pack_h2(xv[i].x * sc, xv[4 + i].x * sc);
            p[4 * i + 1] = pack_h2(xv[i].y * sc, xv[4 + i].y * sc);
            p[4 * i + 2] = pack_h2(xv[i].z * sc, xv[4 + i].z * sc);
            p[4 * i + 3] = pack_h2(xv[i].w * sc, xv[4 + i].w * sc);
        }
        z[0] = 0.f;
    } else if constexpr (FMT == FAQ4) {
        // dword k holds elements 8k..8k+7, element 2i in the low nibble of byte i: pairs
        // (8k, 8k+4), (8k+1, 8k+5) / 16, (8k+2, 8k+6), (8k+3, 8k+7) / 16, the high-nibble pairs
        // carrying 1/16 as the Q4 formats' do; z[0] the sum of the rounded, scaled x
        const float sh = sc * 0.0625f;
        float sa = 0.f, sb = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 a = xv[2 * k], b = xv[2 * k + 1];
            p[4 * k + 0] = pack_h2(a.x * sc, b.x * sc);
            p[4 * k + 1] = pack_h2(a.y * sh, b.y * sh);
            p[4 * k + 2] = pack_h2(a.z * sc, b.z * sc);
            p[4 * k + 3] = pack_h2(a.w * sh, b.w * sh);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const qg_h2 h = __builtin_bit_cast(qg_h2, p[4 * k + j]);
                if (j & 1) {
                    sb += (float)h.x; sb += (float)h.y;
                } else {
                    sa += (float)h.x; sa += (float)h.y;
                }
            }
        }
        z[0] = fmaf(sb, 16.0f, sa);
    } else if constexpr (FMT == FQ8_0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[2 * i + 0] = pack_h2(xv[i].x * sc, xv[i].z * sc);
            p[2 * i + 1] = pack_h2(xv[i].y * sc, xv[i].w * sc);
        }
        z[0] = 0.f;
    } else {
        const float sh = fmt_q4(FMT) ? sc * 0.0625f : sc;    // Q4 high-nibble pairs carry 1/16
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[4 * i + 0] = pack_h2(xv[i].x * sc, xv[i].z * sc);
            p[4 * i + 1] = pack_h2(xv[4 + i].x * sh, xv[4 + i].z * sh);
            p[4 * i + 2] = pack_h2(xv[i].y * sc, xv[i].w * sc);
            p[4 * i + 3] = pack_h2(xv[4 + i].y * sh, xv[4 + i].w * sh);
        }
        if constexpr (!fmt_min(FMT)) {
            z[0] = 0.f;
        } else {
            // S_A, S_B: the sums of the (rounded, scaled) x of the two sub-blocks
            float sa = 0.f, sb = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const qg_h2 a0 = __builtin_bit_cast(qg_h2, p[4 * i + 0]);
                const qg_h2 a1 = __builtin_bit_cast(qg_h2, p[4 * i + 2]);
                const qg_h2 b0 = __builtin_bit_cast(qg_h2, p[4 * i + 1]);
                const qg_h2 b1 = __builtin_bit_cast(qg_h2, p[4 * i + 3]);
                sa += (float)a0.x; sa += (float)a0.y; sa += (float)a1.x; sa += (float)a1.y;
                sb += (float)b0.x; sb += (float)b0.y; sb += (float)b1.x; sb += (float)b1.y;
            }
            z[0] = sa;
            z[1] = fmt_q4(FMT) ? sb * 16.0f : sb;
        }
    }
}

// The lane's chunk c of every batch row as f16 pairs, each chunk scaled by the power of two that
// puts its largest |value| in [2^14, 2^15), and the factor that undoes that scale (un[r], exact).
// The scale depends on the chunk's own 16 or 32 values only, so no wave waits for a reduction
// over the row before its first dot product.
template <int FMT, int NB>
__device__ __forceinline__ void xh_from_lds(XH<FMT, NB> &xh, float (&un)[NB], const float4 *X4,
                                            int K4, int C, int c)
{
    constexpr int XF4 = Fc<FMT>::XF4;
    const int cx = c < C ? c : C - 1;
#pragma unroll
    for (int r = 0; r < NB; ++r) {
        float4 xv[XF4];
#pragma unroll
        for (int j = 0; j < XF4; ++j)
            xv[j] = X4[(size_t)r * K4 + chunk_elem<FMT>(cx, j) / 4];
        float mx = 0.f;
#pragma unroll
        for (int j = 0; j < XF4; ++j)
            mx = fmaxf(mx, fmaxf(fmaxf(fabsf(xv[j].x), fabsf(xv[j].y)),
                                 fmaxf(fabsf(xv[j].z), fabsf(xv[j].w))));
        int e2 = 0;
        frexpf(mx, &e2);                                    // max |x| = f 2^e2, f in [0.5, 1)
        const int sk = 15 - e2 < 127 ? 15 - e2 : 127;       // 2^sk stays a finite f32
        un[r] = ldexpf(1.0f, -sk);
        x_pairs<FMT>(xv, ldexpf(1.0f, sk), xh.p[r][0], xh.z[r][0]);
    }
}

// 1 / sqrt(mean x^2 + eps) of each batch row, from the staged per-float4 squares: lane-strided
// partial sums, then a butterfly, so the order is the same whatever the batch size and every wave
// gets the same value.
template <int NB>
__device__ __forceinline__ void row_inv_rms(float (&inv)[NB], const float *SS, float eps, int K4,
                                            int lane, int bp32)
{
#pragma unroll
    for (int r = 0; r < NB; ++r) {
        float ss = 0.f;
#pragma unroll 4
        for (int e = lane; e < K4; e += 64)
            ss += SS[r * K4 + e];
        ss += xor_lane<32>(ss, bp32);
        ss += xor_lane<16>(ss, bp32);
        ss += xor_lane<8>(ss, bp32);
        ss += xor_lane<4>(ss, bp32);
        ss += xor_lane<2>(ss, bp32);
        ss += xor_lane<1>(ss, bp32);
        inv[r] = 1.0f / sqrtf(ss / (float)(4 * K4) + eps);
    }
}

// Decode + dot of one row group with f16 pairs for the first NB of the NBX batch rows xh holds;
// acc[item][m] with item = u * NBX + r, in the scaled domain of each batch row.
template <int FMT, int NB, int CPL, int MATS, int R, int IP, int NBX = NB>
__device__ __forceinline__ void compute_group_h(const GroupBuf<FMT, CPL, MATS, R> &b,
                                                const XH<FMT, NBX, CPL> &xh, const WConst &k,
                                                int C, int c0, float (&acc)[IP][MATS])
{
    static_assert(NB <= NBX && R * NBX <= IP, "rows and items must fit");
    constexpr int NP = XH<FMT, NBX, CPL>::NP;
#pragma unroll
    for (int it = 0; it < IP; ++it)
#pragma unroll
        for (int m = 0; m < MATS; ++m)
            acc[it][m] = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
    if (i > 0)
        __builtin_amdgcn_sched_barrier(0);   // one chunk slot's pairs and decode live at a time
    const int c = c0 + 64 * i;
    const int cx = c < C ? c : C - 1;   // a slot past the row's chunks gets zero scales
    const int qpos = cx & 7;
#pragma unroll
    for (int m = 0; m < MATS; ++m)
#pragma unroll
        for (int u = 0; u < R; ++u) {
            ChunkScale cs = scale_of<FMT>(b.s[m][u][i], qpos);
            if (c >= C)
                cs.a = cs.b = cs.a2 = cs.b2 = 0.f;
            uint32_t w[NP];
            const uint4 q = b.q[m][u][i];
            WConst kk = k;
            float resA = 0.f, resB = 0.f;
            if constexpr (fmt_min(FMT)) {
                // centred sub-blocks (k_center): the pairs hold q - c (Q4_K's high nibbles
                // 16 (q - c)) exactly, and (a c - b) multiplies the sub-block's x sum
                const float cA = k_center(cs.a, cs.b), cB = k_center(cs.a2, cs.b2);
                kk.off_lo = h2_splat(-1024.0f - cA);
                kk.off_hi = h2_splat(-1024.0f - (fmt_q4(FMT) ? 16.0f : 1.0f) * cB);
                resA = fmaf(cs.a, cA, -cs.b);
                resB = fmaf(cs.a2, cB, -cs.b2);
            } else if constexpr (FMT == FAQ4) {
                // centred block (aq_center): pairs q - c' (high nibbles 16 (q - c')), and
                // (s c' + c) times the chunk's x sum
                const float cA = aq_center(cs.a, cs.b);
                kk.off_lo = h2_splat(-1024.0f - cA);
                kk.off_hi = h2_splat(-1024.0f - 16.0f * cA);
                resA = fmaf(cs.a, cA, -cs.b);
            }
            if constexpr (fmt_hbits(FMT)) {
                const uint32_t h0 = b.h[m][u][i][0];
                const uint32_t h1 = b.h[m][u][i][fmt_hwords(FMT) - 1];
                w_pairs_hb<FMT, 0>(q.x, h0, h1, kk, w + 0);
                w_pairs_hb<FMT, 1>(q.y, h0, h1, kk, w + 4);
                w_pairs_hb<FMT, 2>(q.z, h0, h1, kk, w + 8);
                w_pairs_hb<FMT, 3>(q.w, h0, h1, kk, w + 12);
            } else if constexpr (fmt_codebook(FMT)) {
                w_pairs_cb(q.x, kk, kk.cb[m], w + 0);
                w_pairs_cb(q.y, kk, kk.cb[m], w + 4);
                w_pairs_cb(q.z, kk, kk.cb[m], w + 8);
                w_pairs_cb(q.w, kk, kk.cb[m], w + 12);
            } else if constexpr (FMT == FQ1_0) {
                w_pairs_q1(q.x, kk, w);
            } else {
                w_pairs<FMT>(q.x, kk, w + 0 * (NP / 4));
                w_pairs<FMT>(q.y, kk, w + 1 * (NP / 4));
                w_pairs<FMT>(q.z, kk, w + 2 * (NP / 4));
                w_pairs<FMT>(q.w, kk, w + 3 * (NP / 4));
            }
#pragma unroll
            for (int r = 0; r < NB; ++r) {
                float d[2];
                chunk_chains<FMT>(w, xh.p[r][i], d);
                float &a = acc[u * NBX + r][m];
                if constexpr (fmt_min(FMT)) {
                    a = fmaf(cs.a, d[0], a);
                    a = fmaf(resA, xh.z[r][i][0], a);
                    a = fmaf(cs.a2, d[1], a);
                    a = fmaf(resB, xh.z[r][i][1], a);
                } else if constexpr (FMT == FQ6_K) {
                    a = fmaf(cs.a, d[0], a);
                    a = fmaf(cs.a2, d[1], a);
                } else if constexpr (FMT == FAQ4) {
                    a = fmaf(cs.a, d[0], a);
                    a = fmaf(resA, xh.z[r][i][0], a);
                } else {
                    a = fmaf(cs.a, d[0], a);
                }
            }
        }
    }
}

// ------------------------------------------------------------------------------------ GEMV family

// Workgroup b streams a pool of row groups: the tiles (TG consecutive groups) b, b + grid,
// b + 2 grid, ... so that at any time the grid reads one dense window of the matrix (pools of
// contiguous rows would put hundreds of streams a power-of-two stride apart, on the same memory
// channels).  Each wave keeps PD groups in flight in PD register buffers: group g is decoded while
// the next PD - 1 stream in.  With KS = 1 a wave takes a whole row group (one 16-byte chunk per
// lane) and, after its first PD groups, claims the next group of the pool from an LDS counter,
// so that waves whose loads the memory system serves early take more groups and all waves of
// the CU finish together.  With KS > 1 a row's C chunks are split over KS waves (a team) that
// walk the pool in a fixed order and combine their row sums in LDS (slices added in order).
// Results wait in LDS and leave in one coalesced pass at the end, so the loop holds no stores
// (one counter tracks loads and stores on this target: a store among the in-flight loads would
// make the compiler wait for all of them).  x is staged in LDS once per workgroup.
template <int FMT, int NB, int KS, int EPI, bool NRM, int PD>
__global__ __launch_bounds__((SP<FMT, NB, 1, EPI == E_GUS ? 2 : 1, KS>::NT))
__attribute__((amdgpu_waves_per_eu(SP<FMT, NB, 1, EPI == E_GUS ? 2 : 1, KS>::WPE)))
void k_stream(GemvArgs a)
{
    constexpr int MATS = EPI == E_GUS ? 2 : 1;
    using P = SP<FMT, NB, 1, MATS, KS>;
    constexpr int R = P::R, IP = P::IP, WV = P::WV, NT = P::NT, ITEMS = P::ITEMS;
    constexpr int LG = IP == 1 ? 0 : IP == 2 ? 1 : IP == 4 ? 2 : IP == 8 ? 3 : IP == 16 ? 4 : 5;
    constexpr int TEAMS = WV / KS;
    // float4s of x each loader lane fetches: at least 2 (more loader waves, each with fewer loads,
    // publish x sooner; measured against 1, 4 and 8), and enough for the workgroup's waves to
    // cover the longest row of this K class
    constexpr int XPL0 = (NB * KS * Fc<FMT>::XF4 + WV - 1) / WV;
    constexpr int XPL = XPL0 > 2 ? XPL0 : 2;

    extern __shared__ float4 lds4[];
    __shared__ unsigned long long s_key[NB * WV];
    __shared__ float s_comb[KS > 1 ? 2 : 1][WV][IP][MATS];
    __shared__ int s_next;
    __shared__ int s_xcnt;
    // norm: bits of 1 / rms of each batch row with the sign bit flipped, published by the last
    // loader wave; 0 = not yet (1 / sqrt(y) is never -0.0, so the value is its own ready flag)
    __shared__ unsigned s_inv[NB];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ks = wave % KS, team = wave / KS;
    const int C = (int)(a.qs_row / fmt_chunk_bytes(FMT));
    const int K4 = (int)(a.K / 4);
    float4 *X4 = lds4;                                              // x (norm: x * gamma)
    float *SS = reinterpret_cast<float *>(lds4 + (size_t)NB * K4);  // norm: float4 squares
    float *s_out = SS + (NRM ? NB * K4 : 0);                        // [pool][ITEMS] results

    // the scale plane's range rounded up to whole dwords (one-load scales read dwords; the packed
    // layout pads each plane to 256 bytes)
    const uint32_t qbytes = (uint32_t)(a.N * a.qs_row),
                   sbytes = ((uint32_t)(a.N * a.sc_row) + 3u) & ~3u;
    const uint32_t hbytes = (uint32_t)(a.N * a.hb_row), dbytes = (uint32_t)(a.N * a.d_row);
    BufMat mat[MATS];
    mat[0] = buf_mat(a.qs0, a.sc0, qbytes, sbytes, a.hb0, hbytes, a.dd0, dbytes);
    if constexpr (MATS == 2)
        mat[MATS - 1] = buf_mat(a.qs1, a.sc1, qbytes, sbytes, a.hb1, hbytes, a.dd1, dbytes);
    const LaneOff<1> lo = lane_offsets<FMT, 1>(ks * 64 + lane, C);
    const uint32_t srow = (uint32_t)a.sc_row;
    const RowB rw{(uint32_t)a.qs_row, srow, (uint32_t)a.hb_row, (uint32_t)a.d_row};
    // one-load scales (see load_group): this lane's block scale of row u of a group is half
    // ssh[u] / 16 of the dword that lane sbp[u] / 4 loaded
    constexpr bool SCW = KS == 1 && MATS == 1 &&
                         (((FMT == FQ4_0 || FMT == FQ8_0 || FMT == FIQ4_NL) && R == 2) ||
                          (FMT == FQ1_0 && R == 8));
    uint32_t sbp[R], ssh[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const uint32_t cx = (uint32_t)(lane < C ? lane : C - 1);
        const uint32_t byte =
            u * srow + 2u * (FMT == FQ8_0 ? cx >> 1 : FMT == FQ1_0 ? cx >> 2 : cx);
        sbp[u] = byte & ~3u;
        ssh[u] = (byte & 2u) * 8u;
    }

    // this workgroup's pool of row groups: pool-local index c is group gmap(c); indices at or
    // past `pool` (and groups past T in the last tile) carry no result
    const int tgl = a.tg_log2, TG = 1 << tgl;    // groups per tile (1..8, set by the host)
    const int64_t T = (a.N + R - 1) / R;
    const int n_tiles = (int)((T + TG - 1) >> tgl);
    const int pool = (int)(((uint32_t)(n_tiles - (int)blockIdx.x) + gridDim.x - 1u) / gridDim.x) << tgl;
    auto gmap = [&](int c) -> int64_t {
        return ((int64_t)((c >> tgl) * (int)gridDim.x + (int)blockIdx.x) << tgl) + (c & (TG - 1));
    };
    // the group of pool index c, or -1 (loaded out of range: no traffic, no result)
    auto gclamp = [&](int c) -> int64_t {
        if (c >= pool)
            return -1;
        const int64_t g = gmap(c);
        return g < T ? g : -1;
    };

    // residual operand of the (row, batch row) this lane reports, fetched with its group
    const int my_item = lane >> (6 - LG);
    const bool writer = (lane & ((64 >> LG) - 1)) == 0 && my_item < ITEMS;
    const int my_u = my_item / NB, my_r = my_item % NB;
    auto load_res = [&](int gl) -> float {
        if constexpr (EPI == E_RES) {
            const int64_t g = gclamp(gl), nr = (g < 0 ? 0 : g) * R + my_u;
            return a.res[(int64_t)my_r * a.res_rstride + (nr < a.N ? nr : a.N - 1)];
        } else {
            return 0.f;
        }
    };

    const int cme = ks * 64 + lane;   // this lane's chunk of the row
    const int bp32 = (lane ^ 32) << 2;
    // First group of each buffer: KS = 1, wave w takes p * WV + w; KS > 1, team t takes
    // t + p * TEAMS (its steps are t + k * TEAMS).
    auto first_group = [&](int p) -> int { return KS == 1 ? p * WV + wave : team + p * TEAMS; };

    // x: the first xw waves fetch it (XPL float4s per lane) and publish it in LDS, counting
    // themselves in s_xcnt; the other waves issue their weight loads at once and only then wait
    // for the count, so the x latency runs under the weight latency.  (A workgroup barrier here
    // would hold every wave until the slowest one had issued its weight loads.)
    const int xw = (NB * K4 + 64 * XPL - 1) / (64 * XPL);
    const bool xloader = wave < xw;
    if (threadIdx.x == 0) {
        s_next = PD * WV;
        s_xcnt = 0;
#pragma unroll
        for (int r = 0; r < NB; ++r)
            s_inv[r] = 0u;
    }
    __syncthreads();   // the counters are set (no memory wait: nothing is in flight yet)
    GroupBuf<FMT, 1, MATS, R> buf[PD];
    float resv[PD];
    int gcur[PD];
    // issued group by group, in the order the loop re-issues them, so that the wait counts the
    // compiler derives at the loop head hold on the first round too
    auto issue_first = [&]() {
#pragma unroll
        for (int p = 0; p < PD; ++p) {
            gcur[p] = first_group(p);
            load_group<FMT, 1, MATS, R, SCW>(buf[p], mat, rw, a.N, lo, gclamp(gcur[p]));
            resv[p] = load_res(gcur[p]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Each path issues its own weight loads, so that no path inherits pending x loads from the
    // other (the compiler's wait counts merge paths conservatively).
    if (!xloader)
        issue_first();
    if (xloader) {
        XStage<NB, NRM, XPL> xs;
        xstage_issue<NB, NRM, XPL>(xs, a.x, a.gamma, K4, lane + 64 * wave, 64 * xw);
        xstage_store<NB, NRM, XPL>(xs, K4, lane + 64 * wave, 64 * xw, X4, SS);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        int seen = 0;
        if (lane == 0)
            seen = __hip_atomic_fetch_add(&s_xcnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        seen = __builtin_amdgcn_readfirstlane(seen);
        issue_first();
        if constexpr (NRM) {
            // The last loader to count forms every row's 1 / rms once, after its weight loads are
            // out; the other waves need it only at their first epilogue.  Every other loader
            // finished its stores before counting, and LDS accesses complete in order.
            if (seen == xw - 1) {
                asm volatile("" ::: "memory");
                float inv[NB];
                row_inv_rms<NB>(inv, SS, a.eps, K4, lane, bp32);
                if (lane == 0)
#pragma unroll
                    for (int r = 0; r < NB; ++r)
                        __hip_atomic_store(&s_inv[r], __float_as_uint(inv[r]) ^ 0x80000000u,
                                           __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
    }
    // wait for x: relaxed polling (an acquire would also wait for this wave's weight loads); LDS
    // accesses of a wave complete in order, and every loader finished its stores before counting
    while (__hip_atomic_load(&s_xcnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < xw)
        __builtin_amdgcn_s_sleep(1);
    asm volatile("" ::: "memory");
    XH<FMT, NB> xh;
    WConst wk = w_const<FMT>();
    if constexpr (fmt_codebook(FMT)) {
        const uint4 t0 = *reinterpret_cast<const uint4 *>(a.cb0);
        wk.cb[0] = make_uint4(t0.x ^ 0x80808080u, t0.y ^ 0x80808080u, t0.z ^ 0x80808080u,
                              t0.w ^ 0x80808080u);
        if constexpr (MATS == 2) {
            const uint4 t1 = *reinterpret_cast<const uint4 *>(a.cb1);
            wk.cb[1] = make_uint4(t1.x ^ 0x80808080u, t1.y ^ 0x80808080u, t1.z ^ 0x80808080u,
                                  t1.w ^ 0x80808080u);
        }
    }
    float un[NB];   // factor undoing the scale of this lane's x chunk, per batch row
    xh_from_lds<FMT, NB>(xh, un, X4, K4, C, cme);
    // the row factor this lane's reported item takes: 1 / rms of its batch row with the norm,
    // read at the first epilogue (my_inv_ready)
    float my_inv = 1.0f;
    bool my_inv_ready = !NRM;

    unsigned long long best = 0ull;
    // the value this lane's item contributes to y (residual, gated product), argmax bookkeeping
    auto epilogue = [&](const float (&v)[MATS], int gl, float res) {
        float out;
        if constexpr (EPI == E_RES) {
            out = v[0] + res;
        } else if constexpr (EPI == E_GUS) {
            out = gated(v[0], v[MATS - 1], a.act);
        } else {
            out = v[0];
        }
        if (writer) {
            s_out[gl * ITEMS + my_item] = out;
            if constexpr (EPI == E_ARGMAX) {
                const int64_t n = gmap(gl) * R + my_u;
                if (n < a.N) {
                    const unsigned long long k = argmax_key(out, n);
                    best = k > best ? k : best;
                }
            }
        }
    };
    // reduce one computed group (gl in the pool); with KS > 1 combine the slices through LDS
    auto finish = [&](float (&acc)[IP][MATS], int gl, int par, float res) {
        // undo the chunk scales (exact: powers of two), then sum over the lanes
#pragma unroll
        for (int u = 0; u < R; ++u)
#pragma unroll
            for (int r = 0; r < NB; ++r)
#pragma unroll
                for (int m = 0; m < MATS; ++m)
                    acc[u * NB + r][m] *= un[r];
        xpose_reduce<IP, MATS>(acc, lane, bp32);
        if constexpr (NRM) {
            if (!my_inv_ready) {   // wave-uniform
                unsigned bits[NB];
#pragma unroll
                for (int r = 0; r < NB; ++r)
                    while ((bits[r] = __hip_atomic_load(&s_inv[r], __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_WORKGROUP)) == 0u)
                        __builtin_amdgcn_s_sleep(1);
                my_inv = __uint_as_float(bits[0] ^ 0x80000000u);
#pragma unroll
                for (int r = 1; r < NB; ++r)
                    my_inv = my_r == r ? __uint_as_float(bits[r] ^ 0x80000000u) : my_inv;
                my_inv_ready = true;
            }
#pragma unroll
            for (int m = 0; m < MATS; ++m)
                acc[0][m] *= my_inv;
        }
        if constexpr (KS == 1) {
            epilogue(acc[0], gl, res);
        } else {
            if (writer)
#pragma unroll
                for (int m = 0; m < MATS; ++m)
                    s_comb[par][wave][my_item][m] = acc[0][m];
            __syncthreads();
            if (ks == 0 && gl < pool) {
                float v[MATS];
#pragma unroll
                for (int m = 0; m < MATS; ++m) {
                    v[m] = 0.f;
                    if (writer)
                        for (int q = 0; q < KS; ++q)
                            v[m] += s_comb[par][wave + q][my_item][m];
                }
                epilogue(v, gl, res);
            }
        }
    };

    if constexpr (KS == 1) {
        // Rounds of PD groups; the loop has one exit, at the end of a round (an exit edge back
        // through the loop head would make the compiler's wait counts there assume the newest
        // buffer is the next one).  Claims are increasing, so once the first claim of a round
        // is past the pool every buffer is.  A buffer past the pool is re-loaded (clamped, no
        // result) so that every round issues the same loads.
        if (gcur[0] < pool) {
            for (;;) {
#pragma unroll
                for (int p = 0; p < PD; ++p) {
                    const int gl = gcur[p];
                    float acc[IP][MATS];
                    if (gl < pool) {
                        if constexpr (SCW)
#pragma unroll
                            for (int u = 0; u < R; ++u)
                                buf[p].s[0][u][0] = (uint16_t)(
                                    (uint32_t)__builtin_amdgcn_ds_bpermute((int)sbp[u], (int)buf[p].sw) >>
                                    ssh[u]);
                        compute_group_h<FMT, NB, 1, MATS, R, IP>(buf[p], xh, wk, C, cme, acc);
                    }
                    int nx = 0;
                    if (lane == 0)
                        nx = atomicAdd(&s_next, 1);
                    nx = __builtin_amdgcn_readfirstlane(nx);
                    const float res = resv[p];
                    load_group<FMT, 1, MATS, R, SCW>(buf[p], mat, rw, a.N, lo, gclamp(nx));
                    resv[p] = load_res(nx);
                    if (gl < pool)
                        finish(acc, gl, 0, res);
                    gcur[p] = nx;
                }
                if (gcur[0] >= pool)
                    break;
            }
        }
    } else {
        // the team's steps t + k * TEAMS, k < steps (the same count for every wave: the combine
        // has barriers); whole rounds of PD, then the last steps % PD with no further loads
        const int steps = (pool + TEAMS - 1) / TEAMS;
        const int rounds = steps / PD, rem = steps - rounds * PD;
        int k = 0, par = 0;
        for (int rd = 0; rd < rounds; ++rd) {
#pragma unroll
            for (int p = 0; p < PD; ++p) {
                const int gl = team + k * TEAMS;
                float acc[IP][MATS];
                compute_group_h<FMT, NB, 1, MATS, R, IP>(buf[p], xh, wk, C, cme, acc);
                const float res = resv[p];
                const int gn = gl + PD * TEAMS;
                load_group(buf[p], mat, rw, a.N, lo, gclamp(gn));
                resv[p] = load_res(gn);
                finish(acc, gl, par, res);
                par ^= 1;
                ++k;
            }
        }
#pragma unroll
        for (int p = 0; p < PD - 1; ++p) {
            if (p < rem) {
                const int gl = team + k * TEAMS;
                float acc[IP][MATS];
                compute_group_h<FMT, NB, 1, MATS, R, IP>(buf[p], xh, wk, C, cme, acc);
                finish(acc, gl, par, resv[p]);
                par ^= 1;
                ++k;
            }
        }
    }

    // all results of the pool are in LDS: write them out, row-contiguous within each tile
    __syncthreads();
    const int prow = pool * R;
    for (int i = threadIdx.x; i < NB * prow; i += NT) {
        const int r = i / prow, nl = i - r * prow;
        const int64_t n = gmap(nl / R) * R + nl % R;
        if (n < a.N)
            a.y[(int64_t)r * a.N + n] = s_out[(nl / R) * ITEMS + (nl % R) * NB + r];
    }

    if constexpr (EPI == E_ARGMAX) {
        // per batch row: wave max over the writer lanes of that row, then the workgroup's
        // partial key; k_argmax_fold reduces the partials after this kernel
#pragma unroll
        for (int r = 0; r < NB; ++r) {
            unsigned long long k = (writer && my_r == r) ? best : 0ull;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                const unsigned long long o = shfl_xor_u64(k, off);
                k = o > k ? o : k;
            }
            if (lane == 0)
                s_key[r * WV + wave] = k;
        }
        __syncthreads();
        if (threadIdx.x < NB) {
            const int r = threadIdx.x;
            unsigned long long k = s_key[r * WV];
            for (int w = 1; w < WV; ++w)
                k = s_key[r * WV + w] > k ? s_key[r * WV + w] : k;
            a.keys[(int64_t)blockIdx.x * NB + r] = k;
        }
    }
}

// ------------------------------------------------------------------------------------ launchers

template <int FMT, int NB, int EPI, int KS>
constexpr int stream_threads() { return SP<FMT, NB, 1, EPI == E_GUS ? 2 : 1, KS>::NT; }

// Kernel of one streaming variant, and its workgroup size.
struct StreamFn {
    const void *fn;
    int threads;
};

template <int FMT, int NB, int KS, int EPI, bool NRM>
inline StreamFn stream_fn_pd(int pd)
{
    constexpr int T = stream_threads<FMT, NB, EPI, KS>();
    switch (pd) {
    case 1: return {reinterpret_cast<const void *>(&k_stream<FMT, NB, KS, EPI, NRM, 1>), T};
    case 2: return {reinterpret_cast<const void *>(&k_stream<FMT, NB, KS, EPI, NRM, 2>), T};
    case 4:
        if constexpr (NB == 1)
            return {reinterpret_cast<const void *>(&k_stream<FMT, NB, KS, EPI, NRM, 4>), T};
        return {nullptr, 0};
    default: return {nullptr, 0};
    }
}

template <int FMT, int KS, int EPI, bool NRM>
inline StreamFn stream_fn_nb(int nb, int pd)
{
    switch (nb) {
    case 1: return stream_fn_pd<FMT, 1, KS, EPI, NRM>(pd);
    case 2: return stream_fn_pd<FMT, 2, KS, EPI, NRM>(pd);
    case 3: return stream_fn_pd<FMT, 3, KS, EPI, NRM>(pd);
    case 4: return stream_fn_pd<FMT, 4, KS, EPI, NRM>(pd);
    default: return {nullptr, 0};
    }
}

template <int FMT, int EPI, bool NRM>
inline StreamFn stream_fn_ks(int ks, int nb, int pd)
{
    return ks == 1 ? stream_fn_nb<FMT, 1, EPI, NRM>(nb, pd)
         : ks == 2 ? stream_fn_nb<FMT, 2, EPI, NRM>(nb, pd)
         : ks == 4 ? stream_fn_nb<FMT, 4, EPI, NRM>(nb, pd) : StreamFn{nullptr, 0};
}

template <int FMT>
inline StreamFn stream_fn_fmt(int epi, bool nrm, int ks, int nb, int pd)
{
    switch (epi) {
    case E_STORE:
        return nrm ? stream_fn_ks<FMT, E_STORE, true>(ks, nb, pd)
                   : stream_fn_ks<FMT, E_STORE, false>(ks, nb, pd);
    case E_RES:
        return nrm ? stream_fn_ks<FMT, E_RES, true>(ks, nb, pd)
                   : stream_fn_ks<FMT, E_RES, false>(ks, nb, pd);
    case E_GUS: return stream_fn_ks<FMT, E_GUS, true>(ks, nb, pd);
    case E_ARGMAX: return stream_fn_ks<FMT, E_ARGMAX, false>(ks, nb, pd);
    default: return {nullptr, 0};
    }
}

}  // namespace qg

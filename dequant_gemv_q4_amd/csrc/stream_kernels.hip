// stream_kernels.hip -- the streaming dequant-GEMV kernels of libqgemv for gfx950.
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
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "qgemv.h"

#include <mutex>
#include <vector>

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
    static constexpr int R = stream_rows(NB, CPL, MATS);
    static constexpr int XF4 = Fc<FMT>::XF4, CE = Fc<FMT>::CE, NS = Fc<FMT>::NS;
    // waves per SIMD the register budget must allow (at most 512 / WPE VGPRs per lane): a row
    // batch of 2..4 on one matrix with one wave per row holds its x pairs in about 120 VGPRs,
    // so three waves fit (more waves to hide the longer decode of several batch rows); rows
    // split over several waves are short, and fewer, smaller workgroups start sooner there
    static constexpr int WPE = (NB == 1 && CPL == 1 && FMT != FQ4_K) ? QG_WPE_NB1
                             : (NB > 1 && KS == 1 && MATS == 1 && FMT != FQ4_K) ? 3 : 2;
    static constexpr int ITEMS = R * NB;
    static constexpr int IP = pow2_ceil(ITEMS);
    // GEMV family: one workgroup fills a CU (WPE waves on each of its 4 SIMDs)
    static constexpr int WV = 4 * WPE, NT = 64 * WV;
};

// Raw scale bytes as loaded: one f16 (kept 16-bit, so nothing has to mask a load's result before
// it is used), or the 16-byte Q4_K header.
template <int FMT>
struct ScaleT {
    using T = uint16_t;
};
template <>
struct ScaleT<FQ4_K> {
    using T = uint4;
};

// Loads of one row group: for each matrix, row and chunk slot, 16 bytes of quants and the scale.
template <int FMT, int CPL, int MATS, int R>
struct GroupBuf {
    uint4 q[MATS][R][CPL];
    typename ScaleT<FMT>::T s[MATS][R][CPL];
    uint32_t sw;   // one-load scales: dword `lane` of the group's scale bytes, as loaded
};

// A packed matrix seen through two buffer resources (quant plane, scale plane).  Row offsets
// are wave-uniform and go in the scalar offset; a lane's chunk offset is a constant VGPR.
// A load whose (vector) offset is at or past the plane's size returns zeros without a memory
// request: q_end / s_end (the sizes) are added to the offsets of loads that must move no data.
// Row offsets go in the vector offset too, so that every load is range-checked.
struct BufMat {
    __amdgpu_buffer_rsrc_t q, s;
    uint32_t q_end, s_end;
};

__device__ __forceinline__ BufMat buf_mat(const uint8_t *qs, const uint8_t *sc, uint32_t q_bytes,
                                          uint32_t s_bytes)
{
    BufMat m;
    m.q_end = q_bytes;
    m.s_end = s_bytes;
    m.q = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(qs), (short)0, (int)q_bytes,
                                            0x00020000);
    m.s = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(sc), (short)0, (int)s_bytes,
                                            0x00020000);
    return m;
}

// Byte offsets of a lane's chunk slots inside a row.  A slot past the row's C chunks reads the
// row's last chunk and gets a zero scale, so it adds exactly nothing.
template <int CPL>
struct LaneOff {
    uint32_t q[CPL], s[CPL];
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
        o.q[i] = cx * 16u;
        o.s[i] = FMT == FQ4_0 ? cx * 2u : FMT == FQ8_0 ? (cx >> 1) * 2u : (cx >> 3) * 16u;
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
                                           uint32_t qs_row, uint32_t sc_row, int64_t N,
                                           const LaneOff<CPL> &lo, int64_t g)
{
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
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(mat[m].q,
                                                                     (int)(lo.q[i] + roq), 0, QG_WCPOL_STREAM);
                b.q[m][u][i] = make_uint4(v[0], v[1], v[2], v[3]);
                // raw scale bytes: the lane mask is applied where they are used, so that no
                // instruction touches a load's result before its group is decoded
                if constexpr (SCW) {
                    (void)ros;
                } else if constexpr (FMT == FQ4_K) {
                    const auto w = __builtin_amdgcn_raw_buffer_load_b128(
                        mat[m].s, (int)(lo.s[i] + ros), 0, QG_WCPOL_STREAM);
                    b.s[m][u][i] = make_uint4(w[0], w[1], w[2], w[3]);
                } else {
                    b.s[m][u][i] = __builtin_amdgcn_raw_buffer_load_b16(
                        mat[m].s, (int)(lo.s[i] + ros), 0, QG_WCPOL_STREAM);
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
    static constexpr int NZ = FMT == FQ4_K ? 2 : 1;
    uint32_t p[NB][CPL][NP];
    float z[NB][CPL][NZ];   // Q4_K: S_A, S_B, the x sums of the two sub-blocks (others: unused)
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
    uint32_t m_lo, m_hi, c, off_lo, off_hi;
};

template <int FMT>
__device__ __forceinline__ WConst w_const()
{
    WConst k;
    k.m_lo = FMT == FQ8_0 ? 0x00FF00FFu : 0x000F000Fu;
    k.m_hi = 0x00F000F0u;
    k.c = 0x64006400u;
    // Q4_0: -1032 (1024 + n -> n - 8), -1152 (1024 + 16 n -> 16 (n - 8)); Q8_0: -1152
    // (1024 + q + 128 -> q); Q4_K: set per sub-block from its centre (see compute_group_h)
    k.off_lo = FMT == FQ4_0 ? 0xE408E408u : FMT == FQ8_0 ? 0xE480E480u : 0xE400E400u;
    k.off_hi = FMT == FQ4_0 ? 0xE480E480u : 0xE400E400u;
    asm volatile("" : "+v"(k.m_lo), "+v"(k.m_hi), "+v"(k.c), "+v"(k.off_lo), "+v"(k.off_hi));
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

// Dot chains of one chunk for one batch row: d[0] (Q4_K: low-nibble chain d[0], high d[1]).
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
    } else if constexpr (FMT == FQ4_0) {
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

// x pairs of one chunk (its float4s xv in chunk_elem order), scaled by sc; Q4_K also the sums of
// the two sub-blocks' rounded, scaled x (the -dmin m terms multiply them).
template <int FMT>
__device__ __forceinline__ void x_pairs(const float4 *xv, float sc, uint32_t *p, float *z)
{
    if constexpr (FMT == FQ8_0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[2 * i + 0] = pack_h2(xv[i].x * sc, xv[i].z * sc);
            p[2 * i + 1] = pack_h2(xv[i].y * sc, xv[i].w * sc);
        }
        z[0] = 0.f;
    } else {
        const float sh = sc * 0.0625f;                       // high-nibble pairs carry 1/16
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[4 * i + 0] = pack_h2(xv[i].x * sc, xv[i].z * sc);
            p[4 * i + 1] = pack_h2(xv[4 + i].x * sh, xv[4 + i].z * sh);
            p[4 * i + 2] = pack_h2(xv[i].y * sc, xv[i].w * sc);
            p[4 * i + 3] = pack_h2(xv[4 + i].y * sh, xv[4 + i].w * sh);
        }
        if constexpr (FMT == FQ4_0) {
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
            z[1] = sb * 16.0f;
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
            if constexpr (FMT == FQ4_K) {
                // centred sub-blocks (k_center): the pairs hold n - c (16 (n - c) for the high
                // nibbles) exactly, and (a c - b) multiplies the sub-block's x sum
                const float cA = k_center(cs.a, cs.b), cB = k_center(cs.a2, cs.b2);
                kk.off_lo = h2_splat(-1024.0f - cA);
                kk.off_hi = h2_splat(-1024.0f - 16.0f * cB);
                resA = fmaf(cs.a, cA, -cs.b);
                resB = fmaf(cs.a2, cB, -cs.b2);
            }
            w_pairs<FMT>(q.x, kk, w + 0 * (NP / 4));
            w_pairs<FMT>(q.y, kk, w + 1 * (NP / 4));
            w_pairs<FMT>(q.z, kk, w + 2 * (NP / 4));
            w_pairs<FMT>(q.w, kk, w + 3 * (NP / 4));
#pragma unroll
            for (int r = 0; r < NB; ++r) {
                float d[2];
                chunk_chains<FMT>(w, xh.p[r][i], d);
                float &a = acc[u * NBX + r][m];
                if constexpr (FMT == FQ4_K) {
                    a = fmaf(cs.a, d[0], a);
                    a = fmaf(resA, xh.z[r][i][0], a);
                    a = fmaf(cs.a2, d[1], a);
                    a = fmaf(resB, xh.z[r][i][1], a);
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
    const int C = (int)(a.qs_row / 16);
    const int K4 = (int)(a.K / 4);
    float4 *X4 = lds4;                                              // x (norm: x * gamma)
    float *SS = reinterpret_cast<float *>(lds4 + (size_t)NB * K4);  // norm: float4 squares
    float *s_out = SS + (NRM ? NB * K4 : 0);                        // [pool][ITEMS] results

    // the scale plane's range rounded up to whole dwords (one-load scales read dwords; the packed
    // layout pads each plane to 256 bytes)
    const uint32_t qbytes = (uint32_t)(a.N * a.qs_row),
                   sbytes = ((uint32_t)(a.N * a.sc_row) + 3u) & ~3u;
    BufMat mat[MATS];
    mat[0] = buf_mat(a.qs0, a.sc0, qbytes, sbytes);
    if constexpr (MATS == 2)
        mat[MATS - 1] = buf_mat(a.qs1, a.sc1, qbytes, sbytes);
    const LaneOff<1> lo = lane_offsets<FMT, 1>(ks * 64 + lane, C);
    const uint32_t qrow = (uint32_t)a.qs_row, srow = (uint32_t)a.sc_row;
    // one-load scales (see load_group): this lane's block scale of row u of a group is half
    // ssh[u] / 16 of the dword that lane sbp[u] / 4 loaded
    constexpr bool SCW = KS == 1 && MATS == 1 && R == 2 && (FMT == FQ4_0 || FMT == FQ8_0);
    uint32_t sbp[R], ssh[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const uint32_t cx = (uint32_t)(lane < C ? lane : C - 1);
        const uint32_t byte = u * srow + 2u * (FMT == FQ8_0 ? cx >> 1 : cx);
        sbp[u] = byte & ~3u;
        ssh[u] = (byte & 2u) * 8u;
    }

    // this workgroup's pool of row groups: pool-local index c is group gmap(c); indices at or
    // past `pool` (and groups past T in the last tile) carry no result
    const int tgl = a.tg_log2, TG = 1 << tgl;    // groups per tile (1..8, set by the host)
    const int64_t T = (a.N + R - 1) / R;
    const int n_tiles = (int)((T + TG - 1) >> tgl);
    const int pool = (int)blockIdx.x < n_tiles
                         ? ((n_tiles - 1 - (int)blockIdx.x) / (int)gridDim.x + 1) << tgl : 0;
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
            load_group<FMT, 1, MATS, R, SCW>(buf[p], mat, qrow, srow, a.N, lo, gclamp(gcur[p]));
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
    const WConst wk = w_const<FMT>();
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
                    load_group<FMT, 1, MATS, R, SCW>(buf[p], mat, qrow, srow, a.N, lo, gclamp(nx));
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
                load_group(buf[p], mat, qrow, srow, a.N, lo, gclamp(gn));
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

// idx[r] from the per-workgroup partial keys [n_part][nb] of an argmax launch (one workgroup of
// 16 waves, one batch row per wave).  A lane's keys are loaded eight at a time, all issued before
// the first compare, so a row of up to 512 partial keys costs one memory latency.
__global__ __launch_bounds__(1024) void k_argmax_fold(const unsigned long long *part, int n_part,
                                                      int nb, int32_t *idx)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int r = wave; r < nb; r += 16) {
        unsigned long long k = 0ull;
        for (int b0 = lane; b0 < n_part; b0 += 64 * 8) {
            unsigned long long o[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int b = b0 + 64 * u;
                o[u] = b < n_part ? part[(int64_t)b * nb + r] : 0ull;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                k = o[u] > k ? o[u] : k;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const unsigned long long o = shfl_xor_u64(k, off);
            k = o > k ? o : k;
        }
        if (lane == 0)
            idx[r] = (int32_t)(0xffffffffu - (uint32_t)(k & 0xffffffffull));
    }
}

// ------------------------------------------------------------------------------------ experts

// Routed experts.  The (row, slot) pairs of the routing table are grouped by expert (ascending
// id; pairs in (row, slot) order) into sets of at most NBX pairs; set s multiplies the N x K
// matrix of its expert e_s by the x rows of its pairs.  The row groups of all sets, laid end to
// end (set s owns virtual groups [s GS, (s + 1) GS)), are cut into equal contiguous ranges, one
// per workgroup, so that every workgroup streams the same number of weight bytes whatever the
// routing.  The host launches at least as many workgroups as there are pairs, so a range
// touches at most two sets; their x rows are staged in LDS by loader waves while the other
// waves issue their first weight loads.  Waves then claim the range's groups from an LDS
// counter (as in the GEMV kernels) and keep the x pairs of the set they are in, reloading them
// when a claim crosses into the second set.  Results collect in LDS and leave in one pass to
// part[pair][n]; k_moe_combine then forms y[r][n] = sum_t wts[r][t] part[r][t][n], t ascending.
template <int FMT, int CPL, int PD>
__global__ __launch_bounds__(moe_threads(FMT, CPL, PD))
__attribute__((amdgpu_waves_per_eu(moe_threads(FMT, CPL, PD) / 256)))
void k_moe(MoeArgs a)
{
    constexpr int NBX = 4 / CPL;                  // x rows a wave holds in registers
    constexpr int R = stream_rows(NBX, CPL, 1);
    constexpr int ITX = R * NBX, IPX = pow2_ceil(ITX);
    constexpr int LG = IPX == 1 ? 0 : IPX == 2 ? 1 : IPX == 4 ? 2 : IPX == 8 ? 3 : 4;
    constexpr int NT = moe_threads(FMT, CPL, PD), WV = NT / 64;
    constexpr int XPL = 8;   // float4s in flight per loader lane while a row is copied
    extern __shared__ float4 lds4[];
    __shared__ int s_pair[QG_PAIRS_MAX][NBX];
    __shared__ int s_e[QG_PAIRS_MAX], s_nb[QG_PAIRS_MAX];
    __shared__ int s_wsum[WV];
    __shared__ float s_rs[2 * NBX];   // factor undoing each staged row's scale
    __shared__ int s_next, s_xcnt;

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int P = a.nb * a.topk;
    const int C = (int)(a.qs_row / 16), K4 = (int)(a.K / 4);
    const int N = (int)a.N, E = (int)a.n_exp;
    // [E][4] per-expert masks of the pairs (bit t of the 128), then [E] set bases and counts
    uint32_t *pmask = reinterpret_cast<uint32_t *>(lds4);
    int *hist = reinterpret_cast<int *>(pmask + 4 * E);

    // 1. the sets.  Every workgroup builds the same sets: each expert's pairs are marked in a
    // bit mask (the order of the atomic ors does not matter), a pair's rank among its expert's
    // pairs is the number of lower pair indices in the mask, an exclusive scan over the experts
    // of ceil(count / NBX) places each expert's sets, and every pair goes into its set in rank
    // order.
    for (int e = t; e < 4 * E; e += NT)
        pmask[e] = 0u;
    if (t == 0) {
        s_next = PD * WV;
        s_xcnt = 0;
    }
    __syncthreads();
    int id = -1;
    if (t < P) {
        id = a.ids[t];
        if (id < 0 || id >= E) {
            if (blockIdx.x == 0)
                atomicOr(a.err, 1u);
            id = -1;
        } else {
            atomicOr(&pmask[4 * id + (t >> 5)], 1u << (t & 31));
        }
    }
    __syncthreads();
    int cnt[4], csum = 0;   // thread t scans experts [4t, 4t + 4)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int e = 4 * t + k;
        cnt[k] = 0;
        if (e < E) {
            const uint4 m = reinterpret_cast<const uint4 *>(pmask)[e];
            cnt[k] = __popc(m.x) + __popc(m.y) + __popc(m.z) + __popc(m.w);
        }
        csum += (cnt[k] + NBX - 1) / NBX;
    }
    int inc = csum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(inc, off);
        inc += lane >= off ? v : 0;
    }
    if (lane == 63)
        s_wsum[wave] = inc;
    __syncthreads();
    int run = inc - csum, n_sets = 0;
    for (int w = 0; w < WV; ++w) {
        run += w < wave ? s_wsum[w] : 0;
        n_sets += s_wsum[w];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int e = 4 * t + k;
        if (e < E)
            hist[e] = (run << 8) | cnt[k];   // first set of expert e, its pair count (<= 128)
        run += (cnt[k] + NBX - 1) / NBX;
    }
    __syncthreads();
    if (id >= 0) {
        int rank = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t m = pmask[4 * id + w];
            const int lo = t - 32 * w;   // pairs below t in this word
            rank += lo >= 32 ? __popc(m) : lo > 0 ? __popc(m & ((1u << lo) - 1u)) : 0;
        }
        const int h = hist[id];
        const int set = (h >> 8) + rank / NBX, pos = rank % NBX;
        s_pair[set][pos] = t;
        if (pos == 0) {
            s_e[set] = id;
            s_nb[set] = (h & 255) - rank < NBX ? (h & 255) - rank : NBX;
        }
    }
    __syncthreads();

    // Every value below is the same in all lanes; divisions and LDS reads produce it in vector
    // registers, and readfirstlane makes it scalar again, so that the branches on it stay scalar
    // and the buffer resources built from it need no per-lane loop.  V < 2^31 (checked by the host).
    auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
    const int GS = (N + R - 1) / R;
    const int64_t V = (int64_t)uni(n_sets) * GS;
    const int v0 = uni((int)(V * blockIdx.x / gridDim.x));
    const int v1 = uni((int)(V * (blockIdx.x + 1) / gridDim.x));
    int L = v1 - v0;
    const int s0 = L > 0 ? uni(v0 / GS) : 0;
    const int s1 = L > 0 ? uni((v1 - 1) / GS) : 0;
    if (L > a.pool_max || s1 > s0 + 1) {   // outside the launch's contract: flag, do nothing
        if (t == 0)
            atomicOr(a.err, 2u);
        L = 0;
    }
    L = uni(L);
    const int nb0 = L > 0 ? uni(s_nb[s0]) : 0;
    const int nb1 = L > 0 && s1 > s0 ? uni(s_nb[s1]) : 0;
    const int j0 = v0 - s0 * GS;                    // group of set s0 at local index 0
    const int b1 = GS - j0;                         // local index where set s0 + 1 starts
    // local group gl: set (0 or 1, -1 past the range) and group within the set
    auto locate = [&](int gl, int &ls, int &j) {
        ls = gl >= L ? -1 : gl < b1 ? 0 : 1;
        j = ls < 0 ? -1 : ls == 0 ? gl + j0 : gl - b1;
    };

    // Staged x: staged row q = ls * NBX + r is row r of set s0 + ls.  Loader wave q copies its
    // row to LDS (raw, in X4[q]), takes the row's largest |value| on the way, and converts the
    // chunk slots of each lane to f16 pairs and offset sums once, in XP[q][slot][k][lane]
    // (uint4 k < NP / 4: pairs; k = NP / 4: the sums); the waves entering a set then only read
    // them.  The results pool reuses the raw rows' space (no result is written before every
    // loader has finished).
    constexpr int NP = XH<FMT, NBX, CPL>::NP, NZ = XH<FMT, NBX, CPL>::NZ, NQ4 = NP / 4 + 1;
    static_assert(2 * NBX <= WV, "one loader wave per staged row");
    uint4 *XP = reinterpret_cast<uint4 *>(lds4 + E + (E + 3) / 4);
    float4 *X4 = reinterpret_cast<float4 *>(XP + (size_t)2 * NBX * CPL * NQ4 * 64);
    float *s_out = reinterpret_cast<float *>(X4);   // [pool][ITX] results, item r * R + u
    const int xw = nb0 + nb1;
    const bool xloader = wave < xw;

    // the two experts' matrices (one buffer resource each: every plane is under 2 GiB)
    const int64_t eqb = a.N * a.qs_row, esb = a.N * a.sc_row;
    const int64_t e0 = L > 0 ? uni(s_e[s0]) : 0;
    const int64_t e1 = L > 0 && s1 > s0 ? uni(s_e[s1]) : e0;
    const LaneOff<CPL> lo = lane_offsets<FMT, CPL>(lane, C);
    const uint32_t qrow = (uint32_t)a.qs_row, srow = (uint32_t)a.sc_row;
    const int bp32 = (lane ^ 32) << 2;

    GroupBuf<FMT, CPL, 1, R> buf[PD];
    int gcur[PD];
    auto load = [&](int p, int gl) {
        int ls, j;
        locate(gl, ls, j);
        const int64_t e = uni((int)(ls == 1 ? e1 : e0));
        const BufMat m[1] = {buf_mat(a.qs + e * eqb, a.sc + e * esb, (uint32_t)eqb, (uint32_t)esb)};
        load_group(buf[p], m, qrow, srow, a.N, lo, j);
    };
    auto issue_first = [&]() {
#pragma unroll
        for (int p = 0; p < PD; ++p) {
            gcur[p] = p * WV + wave;
            load(p, gcur[p]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (!xloader)
        issue_first();
    if (xloader) {
        const int ls = wave < nb0 ? 0 : 1, r = ls ? wave - nb0 : wave, q = ls * NBX + r;
        const float4 *xs = reinterpret_cast<const float4 *>(a.x) +
                           (int64_t)(s_pair[s0 + ls][r] / a.topk) * K4;
        float4 *xq = X4 + (size_t)q * K4;
        float mx = 0.f;
        for (int e0 = 0; e0 < K4; e0 += 64 * XPL) {
            float4 v[XPL];
#pragma unroll
            for (int i = 0; i < XPL; ++i) {
                const int e = e0 + 64 * i + lane;
                v[i] = xs[e < K4 ? e : K4 - 1];
            }
#pragma unroll
            for (int i = 0; i < XPL; ++i) {
                const int e = e0 + 64 * i + lane;
                if (e < K4)
                    xq[e] = v[i];
                mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)),
                                     fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
            }
        }
        mx = fmaxf(mx, xor_lane<32>(mx, bp32));
        mx = fmaxf(mx, xor_lane<16>(mx, bp32));
        mx = fmaxf(mx, xor_lane<8>(mx, bp32));
        mx = fmaxf(mx, xor_lane<4>(mx, bp32));
        mx = fmaxf(mx, xor_lane<2>(mx, bp32));
        mx = fmaxf(mx, xor_lane<1>(mx, bp32));
        int e2 = 0;
        frexpf(mx, &e2);                                // max |x| = f 2^e2, f in [0.5, 1)
        const int sk = 15 - e2 < 127 ? 15 - e2 : 127;   // 2^sk stays a finite f32
        const float sc = ldexpf(1.0f, sk);
        if (lane == 0)
            s_rs[q] = ldexpf(1.0f, -sk);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            const int cx = c < C ? c : C - 1;
            float4 xv[Fc<FMT>::XF4];
#pragma unroll
            for (int j = 0; j < Fc<FMT>::XF4; ++j)
                xv[j] = xq[chunk_elem<FMT>(cx, j) / 4];
            uint32_t pp[NP];
            float zz[NZ];
            x_pairs<FMT>(xv, sc, pp, zz);
            uint4 *dst = XP + (size_t)(q * CPL + i) * NQ4 * 64 + lane;
#pragma unroll
            for (int k = 0; k < NP / 4; ++k)
                dst[k * 64] = make_uint4(pp[4 * k], pp[4 * k + 1], pp[4 * k + 2], pp[4 * k + 3]);
            uint4 zq = make_uint4(0u, 0u, 0u, 0u);
            zq.x = __float_as_uint(zz[0]);
            if constexpr (NZ == 2)
                zq.y = __float_as_uint(zz[1]);
            dst[(NP / 4) * 64] = zq;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        if (lane == 0)
            __hip_atomic_fetch_add(&s_xcnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        issue_first();
    }
    while (__hip_atomic_load(&s_xcnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < xw)
        __builtin_amdgcn_s_sleep(1);
    asm volatile("" ::: "memory");

    XH<FMT, NBX, CPL> xh;
    const WConst wk = w_const<FMT>();
    int cur = -1, nbc = 0;
    float my_rs = 1.f;
    const int my_item = lane >> (6 - LG);
    const int my_u = my_item / NBX, my_r = my_item % NBX;
    const bool writer = (lane & ((64 >> LG) - 1)) == 0 && my_item < ITX;

    if (gcur[0] < L) {
        for (;;) {
#pragma unroll
            for (int p = 0; p < PD; ++p) {
                const int gl = gcur[p];
                float acc[IPX][1];
                if (gl < L) {
                    int ls, j;
                    locate(gl, ls, j);
                    if (ls != cur) {   // entering a set: its x pairs and row scales
                        cur = uni(ls);
                        nbc = uni(ls == 0 ? nb0 : nb1);
#pragma unroll
                        for (int r = 0; r < NBX; ++r)
                            if (r < nbc)
#pragma unroll
                                for (int i = 0; i < CPL; ++i) {
                                    const uint4 *src =
                                        XP + (size_t)((ls * NBX + r) * CPL + i) * NQ4 * 64 + lane;
#pragma unroll
                                    for (int k = 0; k < NP / 4; ++k) {
                                        const uint4 v = src[k * 64];
                                        xh.p[r][i][4 * k] = v.x;
                                        xh.p[r][i][4 * k + 1] = v.y;
                                        xh.p[r][i][4 * k + 2] = v.z;
                                        xh.p[r][i][4 * k + 3] = v.w;
                                    }
                                    const uint4 zq = src[(NP / 4) * 64];
                                    xh.z[r][i][0] = __uint_as_float(zq.x);
                                    if constexpr (NZ == 2)
                                        xh.z[r][i][1] = __uint_as_float(zq.y);
                                }
                        my_rs = s_rs[ls * NBX + (my_r < nbc ? my_r : 0)];
                    }
                    if (nbc == 1) {
                        compute_group_h<FMT, 1, CPL, 1, R, IPX, NBX>(buf[p], xh, wk, C, lane, acc);
                    } else if constexpr (NBX >= 2) {
                        if (nbc == 2)
                            compute_group_h<FMT, 2, CPL, 1, R, IPX, NBX>(buf[p], xh, wk, C, lane, acc);
                        else if constexpr (NBX >= 4) {
                            if (nbc == 3)
                                compute_group_h<FMT, 3, CPL, 1, R, IPX, NBX>(buf[p], xh, wk, C, lane, acc);
                            else
                                compute_group_h<FMT, 4, CPL, 1, R, IPX, NBX>(buf[p], xh, wk, C, lane, acc);
                        }
                    }
                }
                int nx = 0;
                if (lane == 0)
                    nx = atomicAdd(&s_next, 1);
                nx = __builtin_amdgcn_readfirstlane(nx);
                load(p, nx);
                if (gl < L) {
                    xpose_reduce<IPX, 1>(acc, lane, bp32);
                    if (writer && my_r < nbc)
                        s_out[gl * ITX + my_r * R + my_u] = acc[0][0] * my_rs;
                }
                gcur[p] = nx;
            }
            if (gcur[0] >= L)
                break;
        }
    }

    // 3. results to part[pair][n], contiguous in n for each (set, row) run
    __syncthreads();
    const int LR = L * R;
    for (int i = t; i < NBX * LR; i += NT) {
        const int r = i / LR, rem = i - r * LR;
        const int gl = rem / R, u = rem - gl * R;
        int ls, j;
        locate(gl, ls, j);
        const int n = j * R + u;
        if (r < (ls == 0 ? nb0 : nb1) && n < N) {
            const int pair = s_pair[s0 + ls][r];
            a.part[(int64_t)pair * N + n] = s_out[gl * ITX + r * R + u];
        }
    }
}

// y[r][n] = sum_t wts[r][t] part[r][t][n], t ascending, skipping out-of-range expert ids.  A
// thread forms four consecutive n of one row; every part load is issued before the first add
// (a load under the id test would wait for the one before it).
__global__ __launch_bounds__(256) void k_moe_combine(const float *part, const int32_t *ids,
                                                     const float *wts, int nb, int topk,
                                                     int64_t n_exp, int64_t N, float *y)
{
    const int64_t N4 = (N + 3) / 4;
    const int64_t f = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (f >= (int64_t)nb * N4)
        return;
    const int r = (int)(f / N4);
    const int64_t n0 = (f - r * N4) * 4;
    float4 v[QG_MAX_TOPK];
    bool ok[QG_MAX_TOPK];
    float w[QG_MAX_TOPK];
#pragma unroll
    for (int t = 0; t < QG_MAX_TOPK; ++t) {
        const int tt = t < topk ? t : 0;
        const int32_t id = ids[r * topk + tt];
        ok[t] = t < topk && id >= 0 && id < n_exp;
        w[t] = wts[r * topk + tt];
        const float *pr = part + ((int64_t)r * topk + tt) * N;
        if (n0 + 3 < N && (N & 3) == 0) {
            v[t] = *reinterpret_cast<const float4 *>(pr + n0);
        } else {
            v[t].x = pr[n0];
            v[t].y = pr[n0 + 1 < N ? n0 + 1 : n0];
            v[t].z = pr[n0 + 2 < N ? n0 + 2 : n0];
            v[t].w = pr[n0 + 3 < N ? n0 + 3 : n0];
        }
    }
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int t = 0; t < QG_MAX_TOPK; ++t) {
        if (ok[t]) {
            acc.x = fmaf(w[t], v[t].x, acc.x);
            acc.y = fmaf(w[t], v[t].y, acc.y);
            acc.z = fmaf(w[t], v[t].z, acc.z);
            acc.w = fmaf(w[t], v[t].w, acc.w);
        }
    }
    float *yr = y + (int64_t)r * N;
    if (n0 + 3 < N && (N & 3) == 0) {
        *reinterpret_cast<float4 *>(yr + n0) = acc;
    } else {
        yr[n0] = acc.x;
        if (n0 + 1 < N) yr[n0 + 1] = acc.y;
        if (n0 + 2 < N) yr[n0 + 2] = acc.z;
        if (n0 + 3 < N) yr[n0 + 3] = acc.w;
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
static StreamFn stream_fn_pd(int pd)
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
static StreamFn stream_fn_nb(int nb, int pd)
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
static StreamFn stream_fn_ks(int ks, int nb, int pd)
{
    return ks == 1 ? stream_fn_nb<FMT, 1, EPI, NRM>(nb, pd)
         : ks == 2 ? stream_fn_nb<FMT, 2, EPI, NRM>(nb, pd)
         : ks == 4 ? stream_fn_nb<FMT, 4, EPI, NRM>(nb, pd) : StreamFn{nullptr, 0};
}

template <int FMT>
static StreamFn stream_fn_fmt(int epi, bool nrm, int ks, int nb, int pd)
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

static StreamFn stream_fn(int fmt, int epi, bool nrm, int ks, int nb, int pd)
{
    return fmt == FQ4_0 ? stream_fn_fmt<FQ4_0>(epi, nrm, ks, nb, pd)
         : fmt == FQ8_0 ? stream_fn_fmt<FQ8_0>(epi, nrm, ks, nb, pd)
         : fmt == FQ4_K ? stream_fn_fmt<FQ4_K>(epi, nrm, ks, nb, pd) : StreamFn{nullptr, 0};
}

int launch_stream(int fmt, int epi, bool nrm, int cpl, int pd, const GemvArgs &a, int grid,
                  size_t lds_bytes, void *stream)
{
    const StreamFn f = stream_fn(fmt, epi, nrm, cpl, a.nb, pd);
    if (!f.fn)
        return (int)hipErrorInvalidValue;
    void *args[] = {const_cast<GemvArgs *>(&a)};
    return (int)hipLaunchKernel(f.fn, dim3(grid), dim3(f.threads), args, lds_bytes,
                                static_cast<hipStream_t>(stream));
}

template <int FMT>
static const void *moe_fn_fmt(int cpl, int pd)
{
    switch (cpl * 8 + pd) {
    case 1 * 8 + 2: return reinterpret_cast<const void *>(&k_moe<FMT, 1, 2>);
    case 1 * 8 + 4: return reinterpret_cast<const void *>(&k_moe<FMT, 1, 4>);
    case 2 * 8 + 2: return reinterpret_cast<const void *>(&k_moe<FMT, 2, 2>);
    case 2 * 8 + 4: return reinterpret_cast<const void *>(&k_moe<FMT, 2, 4>);
    case 4 * 8 + 2: return reinterpret_cast<const void *>(&k_moe<FMT, 4, 2>);
    case 4 * 8 + 4:   // Q4_K would spill
        if constexpr (FMT != FQ4_K)
            return reinterpret_cast<const void *>(&k_moe<FMT, 4, 4>);
        return nullptr;
    default: return nullptr;
    }
}

static const void *moe_fn(int fmt, int cpl, int pd)
{
    return fmt == FQ4_0 ? moe_fn_fmt<FQ4_0>(cpl, pd)
         : fmt == FQ8_0 ? moe_fn_fmt<FQ8_0>(cpl, pd)
         : fmt == FQ4_K ? moe_fn_fmt<FQ4_K>(cpl, pd) : nullptr;
}

int launch_moe(int fmt, int cpl, int pd, const MoeArgs &a, int grid, size_t lds_bytes,
               void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    const void *fn = moe_fn(fmt, cpl, pd);
    if (!fn)
        return (int)hipErrorInvalidValue;
    void *args[] = {const_cast<MoeArgs *>(&a)};
    const hipError_t err = hipLaunchKernel(fn, dim3(grid), dim3(moe_threads(fmt, cpl, pd)), args,
                                           lds_bytes, s);
    if (err != hipSuccess)
        return (int)err;
    const int64_t quads = (int64_t)a.nb * ((a.N + 3) / 4);
    hipLaunchKernelGGL(k_moe_combine, dim3((int)((quads + 255) / 256)), dim3(256), 0, s, a.part,
                       a.ids, a.wts, a.nb, a.topk, a.n_exp, a.N, a.y);
    return (int)hipGetLastError();
}

// The fixed scratch of the no-allocation argmax entry point: one partial key per workgroup and
// batch row at the largest grid and batch an argmax launch may have (512 KiB per device, held
// until the process ends).  Host code never passes the array's name to a kernel: on the host it
// is a stand-in, not a device address; noalloc_scratch looks the device address up once per
// device and every launch takes that pointer.
static __device__ __align__(256) unsigned long long scratch[QG_ARGMAX_MAX_GRID * QG_MAX_NB];

int noalloc_scratch(void **ptr, size_t *bytes)
{
    constexpr int kMaxDev = 64;
    static std::mutex mu;
    static void *dev_ptr[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev)
        return -1;
    std::lock_guard<std::mutex> lk(mu);
    if (!dev_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return -1;
        dev_ptr[dev] = p;
    }
    *ptr = dev_ptr[dev];
    *bytes = sizeof(scratch);
    return 0;
}

int launch_argmax_fold(const unsigned long long *part, int n_part, int nb, int32_t *idx,
                       void *stream)
{
    hipLaunchKernelGGL(k_argmax_fold, dim3(1), dim3(1024), 0, static_cast<hipStream_t>(stream),
                       part, n_part, nb, idx);
    return (int)hipGetLastError();
}

// ------------------------------------------------------------------------------------ occupancy

// Workgroups of this streaming variant that fit on the device at once with lds_bytes of dynamic
// LDS (0 if it does not fit at all or the query fails), and its waves per workgroup.  Cached per
// device and variant.
// Workgroups of kernel fn (threads per workgroup, dynamic LDS bytes) resident at once on the
// current device, cached per (kernel, device, LDS size); 0 if the query fails or LDS is too big.
static int resident_wgs(const void *fn, int threads, size_t lds_bytes)
{
    int dev = 0;
    if (!fn || hipGetDevice(&dev) != hipSuccess)
        return 0;
    struct Entry {
        const void *fn;
        int dev;
        size_t lds;
        int resident;
    };
    static std::mutex mu;
    static std::vector<Entry> cache;
    {
        std::lock_guard<std::mutex> lk(mu);
        for (const Entry &e : cache)
            if (e.fn == fn && e.dev == dev && e.lds == lds_bytes)
                return e.resident;
    }
    int cus = 0, per_cu = 0, max_lds = 0;
    hipFuncAttributes attr;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess ||
        hipFuncGetAttributes(&attr, fn) != hipSuccess)
        return 0;
    int resident = 0;
    if (attr.sharedSizeBytes + lds_bytes <= (size_t)max_lds &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds_bytes) ==
            hipSuccess)
        resident = cus * per_cu;
    std::lock_guard<std::mutex> lk(mu);
    cache.push_back({fn, dev, lds_bytes, resident});
    return resident;
}

int stream_resident_wgs(int fmt, int epi, bool nrm, int cpl, int nb, int pd, size_t lds_bytes,
                        int *waves)
{
    const StreamFn f = stream_fn(fmt, epi, nrm, cpl, nb, pd);
    if (!f.fn)
        return 0;
    *waves = f.threads / 64;
    return resident_wgs(f.fn, f.threads, lds_bytes);
}

int moe_resident_wgs(int fmt, int cpl, int pd, size_t lds_bytes)
{
    return resident_wgs(moe_fn(fmt, cpl, pd), moe_threads(fmt, cpl, pd), lds_bytes);
}

}  // namespace qg

// stream_kernels.hip -- the streaming dequant-GEMV kernels of libqgemv for gfx950.
//
// One wave64 owns whole rows: lane l takes the 16-byte chunks l, l + 64, ... (CPL per row) of
// R rows at a time, so every global load instruction reads 1 KB contiguous.  Each wave
// double-buffers its loads: the quants and scales of its next row group are in flight while
// it decodes and FMAs the current one.  x (or rmsnorm(x)) is staged once per workgroup in
// LDS and, when small enough, held in registers for the whole kernel.  R x NB partial sums
// leave the wave through a transposed butterfly (each exchange halves the number of values a
// lane carries), and one lane per (row, batch row) runs the epilogue.
//
// Q4_0 decode: byte b_j of a block holds element j (low nibble lo_j) and element j + 16 (high
// nibble hi_j).  Since hi_j = (b_j - lo_j) / 16,
//     lo_j x_j + hi_j x_{j+16} = lo_j u_j + b_j v_j,  u_j = x_j - x_{j+16}/16,  v_j = x_{j+16}/16,
// so a dword of nibbles costs one mask and eight byte converts (v_cvt_f32_ubyteN) before its
// eight FMAs.  x is staged as (u, v).  The -8 offset of Q4_0 ("Crate inferencelayer" docs,
// q4_0_to_q8_0n: q8 = nib - 8) is folded into S' = sum_j (u_j + 17 v_j), accumulated in the
// dot's own order, so eight-valued nibbles (b = 0x88) give exactly 0.
#include <hip/hip_runtime.h>

#include "device_common.h"

namespace qg {

// ------------------------------------------------------------------------------------ helpers

// v & m as an opaque instruction, so the compiler keeps the byte structure and converts each
// byte with v_cvt_f32_ubyteN instead of re-extracting single nibbles.
__device__ __forceinline__ uint32_t and_opaque(uint32_t v, uint32_t m)
{
    uint32_t r;
    asm("v_and_b32 %0, %1, %2" : "=v"(r) : "s"(m), "v"(v));
    return r;
}

template <int FMT>
__device__ __forceinline__ void decode_stream(const uint4 &q, float *w)
{
    if constexpr (FMT == FQ4_0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t v = ucomp(q, k);
            const uint32_t lo = and_opaque(v, 0x0f0f0f0fu);
            w[8 * k + 0] = ub0(lo); w[8 * k + 1] = ub1(lo);
            w[8 * k + 2] = ub2(lo); w[8 * k + 3] = ub3(lo);
            w[8 * k + 4] = ub0(v); w[8 * k + 5] = ub1(v);
            w[8 * k + 6] = ub2(v); w[8 * k + 7] = ub3(v);
        }
    } else if constexpr (FMT == FQ4_K) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t v = ucomp(q, k);
            const uint32_t lo = and_opaque(v, 0x0f0f0f0fu);
            const uint32_t hi = and_opaque(v >> 4, 0x0f0f0f0fu);
            w[8 * k + 0] = ub0(lo); w[8 * k + 1] = ub1(lo);
            w[8 * k + 2] = ub2(lo); w[8 * k + 3] = ub3(lo);
            w[8 * k + 4] = ub0(hi); w[8 * k + 5] = ub1(hi);
            w[8 * k + 6] = ub2(hi); w[8 * k + 7] = ub3(hi);
        }
    } else {
        decode_chunk<FMT>(q, w);
    }
}

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

// Compile-time shape of the streaming kernels.
template <int FMT, int NB, int CPL, int MATS>
struct SP {
    static constexpr int R = stream_rows(NB, CPL, MATS);
    static constexpr int XF4 = Fc<FMT>::XF4, CE = Fc<FMT>::CE, NS = Fc<FMT>::NS;
    // waves per SIMD the register budget must allow (at most 512 / WPE VGPRs per lane)
    static constexpr int WPE = (NB == 1 && CPL == 1 && FMT != FQ4_K) ? QG_WPE_NB1 : 2;
    static constexpr int ITEMS = R * NB;
    static constexpr int IP = pow2_ceil(ITEMS);
};

template <int FMT>
struct ScaleT {
    using T = uint32_t;
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
};

// A packed matrix seen through two buffer resources (quant plane, scale plane).  Row offsets
// are wave-uniform and go in the scalar offset; a lane's chunk offset is a constant VGPR.
struct BufMat {
    __amdgpu_buffer_rsrc_t q, s;
};

__device__ __forceinline__ BufMat buf_mat(const uint8_t *qs, const uint8_t *sc, uint32_t q_bytes,
                                          uint32_t s_bytes)
{
    BufMat m;
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
    bool ok[CPL];
};

template <int FMT, int CPL>
__device__ __forceinline__ LaneOff<CPL> lane_offsets(int lane, int C)
{
    LaneOff<CPL> o;
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
// s_waitcnt: rows past N reload row N - 1 (their results are dropped by the epilogue).
template <int FMT, int CPL, int MATS, int R>
__device__ __forceinline__ void load_group(GroupBuf<FMT, CPL, MATS, R> &b, const BufMat (&mat)[MATS],
                                           uint32_t qs_row, uint32_t sc_row, int64_t N,
                                           const LaneOff<CPL> &lo, int64_t g)
{
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int64_t nr = g * R + u;   // wave-uniform
        const uint32_t n = (uint32_t)(nr < N ? nr : N - 1);
        const uint32_t soq = n * qs_row, sos = n * sc_row;
#pragma unroll
        for (int m = 0; m < MATS; ++m)
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(mat[m].q, (int)lo.q[i],
                                                                     (int)soq, 0);
                b.q[m][u][i] = make_uint4(v[0], v[1], v[2], v[3]);
                // raw scale bytes: the lane mask is applied where they are used, so that no
                // instruction touches a load's result before its group is decoded
                if constexpr (FMT == FQ4_K) {
                    const auto w = __builtin_amdgcn_raw_buffer_load_b128(mat[m].s, (int)lo.s[i],
                                                                         (int)sos, 0);
                    b.s[m][u][i] = make_uint4(w[0], w[1], w[2], w[3]);
                } else {
                    b.s[m][u][i] = __builtin_amdgcn_raw_buffer_load_b16(mat[m].s, (int)lo.s[i],
                                                                         (int)sos, 0);
                }
            }
    }
}

template <int FMT>
__device__ __forceinline__ ChunkScale scale_of(uint32_t s, int) { ChunkScale cs; cs.a = h2f(s & 0xffffu); cs.b = cs.a2 = cs.b2 = 0.f; return cs; }
template <int FMT>
__device__ __forceinline__ ChunkScale scale_of(const uint4 &s, int qpos) { return chunk_scale<FMT>(s, qpos); }

// x of the lane's chunk slots (i) of every batch row (r), in registers, with the block sums.
template <int FMT, int NB, int CPL>
struct XCache {
    float4 xv[NB][CPL][Fc<FMT>::XF4];
    float sv[NB][CPL][Fc<FMT>::NS];
};

// Decode + FMA of one row group; acc[item][m] with item = u * NB + r.
template <int FMT, int NB, int CPL, int MATS, int R, int IP>
__device__ __forceinline__ void compute_group(const GroupBuf<FMT, CPL, MATS, R> &b,
                                              const XCache<FMT, NB, CPL> &xc, int C, int lane,
                                              float (&acc)[IP][MATS])
{
    // a slot past the row's C chunks re-reads the last chunk; a zero scale cancels it
    constexpr int XF4 = Fc<FMT>::XF4, CE = Fc<FMT>::CE, NS = Fc<FMT>::NS;
#pragma unroll
    for (int it = 0; it < IP; ++it)
#pragma unroll
        for (int m = 0; m < MATS; ++m)
            acc[it][m] = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        if (i > 0)
            __builtin_amdgcn_sched_barrier(0);   // one chunk slot's x and decode live at a time
        const int c = lane + 64 * i;
        const int cx = c < C ? c : C - 1;   // slots past the row hold zero weights and scales
        const int qpos = cx & 7;
#pragma unroll
        for (int m = 0; m < MATS; ++m)
#pragma unroll
            for (int u = 0; u < R; ++u) {
                float w[CE];
                decode_stream<FMT>(b.q[m][u][i], w);
                ChunkScale cs = scale_of<FMT>(b.s[m][u][i], qpos);
                if (c >= C)
                    cs.a = cs.b = cs.a2 = cs.b2 = 0.f;
#pragma unroll
                for (int r = 0; r < NB; ++r)
                    acc[u * NB + r][m] = chunk_dot<FMT>(w, xc.xv[r][i], xc.sv[r][i], cs,
                                                        acc[u * NB + r][m]);
            }
    }
}

// In-register form of one chunk's x as the dot consumes it (Q4_0: u, v), and its block sums in
// the dot's own order.
template <int FMT>
__device__ __forceinline__ void x_chunk_transform(float4 *xv, float *sv)
{
    if constexpr (FMT == FQ4_0) {
        float sum = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 hv = make_float4(xv[4 + k].x * 0.0625f, xv[4 + k].y * 0.0625f,
                                          xv[4 + k].z * 0.0625f, xv[4 + k].w * 0.0625f);
            const float4 u = make_float4(xv[k].x - hv.x, xv[k].y - hv.y, xv[k].z - hv.z,
                                         xv[k].w - hv.w);
            xv[k] = u;
            xv[4 + k] = hv;
            sum += u.x; sum += u.y; sum += u.z; sum += u.w;
            sum = fmaf(17.0f, hv.x, sum); sum = fmaf(17.0f, hv.y, sum);
            sum = fmaf(17.0f, hv.z, sum); sum = fmaf(17.0f, hv.w, sum);
        }
        sv[0] = sum;
    } else if constexpr (FMT == FQ8_0) {
        float sum = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            sum += xv[k].x; sum += xv[k].y; sum += xv[k].z; sum += xv[k].w;
        }
        sv[0] = sum;
    } else {
        float sa = 0.f, sb = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            sa += xv[k].x; sa += xv[k].y; sa += xv[k].z; sa += xv[k].w;
            sb += xv[4 + k].x; sb += xv[4 + k].y; sb += xv[4 + k].z; sb += xv[4 + k].w;
        }
        sv[0] = sa;
        sv[1] = sb;
    }
}

// x for this lane's chunk c of every batch row, read straight from global memory into
// registers (x is a few KB: L1/L2 resident after the first wave), so no LDS staging or
// workgroup barrier precedes the first row.  With NRM each wave forms 1/sqrt(mean x^2 + eps)
// itself: its 64 lanes cover the KS chunks of the whole row.  Q4_0 is kept as (u, v) and every
// block sum is formed in the dot's own order, as in the staging it replaces.
template <int FMT, int NB, int KS, bool NRM>
__device__ __forceinline__ void load_x_direct(XCache<FMT, NB, 1> &xc, const float *x,
                                              const float *gamma, float eps, int64_t K, int C,
                                              int c, int lane, int bp32)
{
    constexpr int XF4 = Fc<FMT>::XF4;
    const int cx = c < C ? c : C - 1;
#pragma unroll
    for (int r = 0; r < NB; ++r)
#pragma unroll
        for (int j = 0; j < XF4; ++j)
            xc.xv[r][0][j] = *reinterpret_cast<const float4 *>(x + r * K + chunk_elem<FMT>(cx, j));
    if constexpr (NRM) {
        float4 gv[XF4];
#pragma unroll
        for (int j = 0; j < XF4; ++j)
            gv[j] = *reinterpret_cast<const float4 *>(gamma + chunk_elem<FMT>(cx, j));
#pragma unroll
        for (int r = 0; r < NB; ++r) {
            float ss = 0.f;
#pragma unroll
            for (int q = 0; q < KS; ++q) {
                const int cq = q * 64 + lane;
                if (cq < C) {
#pragma unroll
                    for (int j = 0; j < XF4; ++j) {
                        const float4 v = q * 64 == c - lane
                                             ? xc.xv[r][0][j]
                                             : *reinterpret_cast<const float4 *>(
                                                   x + r * K + chunk_elem<FMT>(cq, j));
                        ss = fmaf(v.x, v.x, ss); ss = fmaf(v.y, v.y, ss);
                        ss = fmaf(v.z, v.z, ss); ss = fmaf(v.w, v.w, ss);
                    }
                }
            }
            ss += xor_lane<32>(ss, bp32);
            ss += xor_lane<16>(ss, bp32);
            ss += xor_lane<8>(ss, bp32);
            ss += xor_lane<4>(ss, bp32);
            ss += xor_lane<2>(ss, bp32);
            ss += xor_lane<1>(ss, bp32);
            const float inv = 1.0f / sqrtf(ss / (float)K + eps);
#pragma unroll
            for (int j = 0; j < XF4; ++j)
                xc.xv[r][0][j] = f4scale(xc.xv[r][0][j], inv, gv[j]);
        }
    }
#pragma unroll
    for (int r = 0; r < NB; ++r)
        x_chunk_transform<FMT>(xc.xv[r][0], xc.sv[r][0]);
}

// x of CPL chunk slots (lane + 64 i) of NB gathered rows (xrow[r] == nullptr: a zero row),
// straight into registers; no norm.
template <int FMT, int NB, int CPL>
__device__ __forceinline__ void load_x_rows(XCache<FMT, NB, CPL> &xc,
                                            const float *const *xrow, int C, int lane)
{
    constexpr int XF4 = Fc<FMT>::XF4;
#pragma unroll
    for (int r = 0; r < NB; ++r)
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            const int cx = c < C ? c : C - 1;
#pragma unroll
            for (int j = 0; j < XF4; ++j)
                xc.xv[r][i][j] = xrow[r] ? *reinterpret_cast<const float4 *>(
                                               xrow[r] + chunk_elem<FMT>(cx, j))
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
            x_chunk_transform<FMT>(xc.xv[r][i], xc.sv[r][i]);
        }
}

// ------------------------------------------------------------------------------------ GEMV family

// Grid-stride over row groups with prefetch distance 2: group g is decoded while the team's
// next two groups are in flight, using two register buffers.  A row of C chunks is split over
// KS = ceil(C / 64) waves (KS in {1, 2, 4}); each wave takes one 16-byte chunk per lane of its
// K slice, and the KS waves of a team combine their row sums in LDS (slices added in order)
// before one of them runs the epilogue.
template <int FMT, int NB, int KS, int EPI, bool NRM>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(SP<FMT, NB, 1, EPI == E_GUS ? 2 : 1>::WPE)))
void k_stream(GemvArgs a)
{
    constexpr int MATS = EPI == E_GUS ? 2 : 1;
    using P = SP<FMT, NB, 1, MATS>;
    constexpr int R = P::R, IP = P::IP;
    constexpr int LG = IP == 1 ? 0 : IP == 2 ? 1 : IP == 4 ? 2 : IP == 8 ? 3 : IP == 16 ? 4 : 5;
    constexpr int TEAMS = 4 / KS;

    __shared__ unsigned long long s_key[NB * 4];
    __shared__ float s_comb[KS > 1 ? 2 : 1][4][IP][MATS];
    __shared__ float s_out[4][QG_OUT_GROUPS][IP];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ks = wave % KS, team = wave / KS;
    const int C = (int)(a.qs_row / 16);

    const uint32_t qbytes = (uint32_t)(a.N * a.qs_row), sbytes = (uint32_t)(a.N * a.sc_row);
    BufMat mat[MATS];
    mat[0] = buf_mat(a.qs0, a.sc0, qbytes, sbytes);
    if constexpr (MATS == 2)
        mat[MATS - 1] = buf_mat(a.qs1, a.sc1, qbytes, sbytes);
    const LaneOff<1> lo = lane_offsets<FMT, 1>(ks * 64 + lane, C);
    const uint32_t qrow = (uint32_t)a.qs_row, srow = (uint32_t)a.sc_row;

    const int64_t T = (a.N + R - 1) / R;
    const int64_t W = (int64_t)gridDim.x * TEAMS;
    const int64_t g0 = (int64_t)blockIdx.x * TEAMS + team;
    // every wave of the workgroup runs the same number of steps (the combine has barriers)
    const int64_t steps = KS > 1 ? (T - (int64_t)blockIdx.x * TEAMS + W - 1) / W : 0;

    // the first two groups of this wave are in flight while x is staged
    // residual operand of the (row, batch row) this lane writes, fetched with its group
    const int lg_items = IP == 1 ? 0 : IP == 2 ? 1 : IP == 4 ? 2 : IP == 8 ? 3 : IP == 16 ? 4 : 5;
    const int item0 = lane >> (6 - lg_items);
    const int64_t res_col = (int64_t)(item0 % NB) * a.N;
    const int res_u = item0 / NB;
    auto load_res = [&](int64_t gg) -> float {
        if constexpr (EPI == E_RES) {
            const int64_t nr = gg * R + res_u;
            return a.res[res_col + (nr < a.N ? nr : a.N - 1)];
        } else {
            return 0.f;
        }
    };

    const int cme = ks * 64 + lane;   // this lane's chunk of the row
    const int bp32 = (lane ^ 32) << 2;
    // x first (its loads retire first), then the first two row groups
    XCache<FMT, NB, 1> xc;
    load_x_direct<FMT, NB, KS, NRM>(xc, a.x, a.gamma, a.eps, a.K, C, cme, lane, bp32);

    GroupBuf<FMT, 1, MATS, R> bufA, bufB;
    load_group(bufA, mat, qrow, srow, a.N, lo, g0);
    float resA = load_res(g0);
    load_group(bufB, mat, qrow, srow, a.N, lo, g0 + W);
    float resB = load_res(g0 + W);

    // the item this lane reports after the reduction, and whether it writes it
    const int my_item = lane >> (6 - LG);
    const bool writer = (lane & ((64 >> LG) - 1)) == 0 && my_item < P::ITEMS;
    const int my_u = my_item / NB, my_r = my_item % NB;
    unsigned long long best = 0ull;

    // Outputs wait in a small per-wave LDS buffer and leave in batches: a vector store among
    // the in-flight weight loads would make the compiler wait for every load (one counter
    // tracks both on this target).
    int nout = 0;
    int64_t gout = g0;
    auto flush = [&]() {
        for (int L = lane; L < nout * P::ITEMS; L += 64) {
            const int k = L / P::ITEMS, item = L % P::ITEMS;
            const int64_t n = (gout + (int64_t)k * W) * R + item / NB;
            if (n < a.N)
                a.y[(int64_t)(item % NB) * a.N + n] = s_out[wave][k][item];
        }
    };
    // the value this lane's item contributes to y (residual, gated product), argmax bookkeeping
    auto epilogue = [&](const float (&v)[MATS], int64_t gg, float res) {
        const int64_t n = gg * R + my_u;
        float out;
        if constexpr (EPI == E_RES) {
            out = v[0] + res;
        } else if constexpr (EPI == E_GUS) {
            const float gt = v[0], up = v[MATS - 1];
            out = gt / (1.0f + expf(-gt)) * up;
        } else {
            out = v[0];
        }
        if constexpr (EPI == E_ARGMAX) {
            if (writer && n < a.N) {
                const unsigned long long k = argmax_key(out, n);
                best = k > best ? k : best;
            }
        }
        if (writer)
            s_out[wave][nout][my_item] = out;
    };
    // reduce one computed group; with KS > 1 combine the slices through LDS (buffer `par`)
    auto finish = [&](float (&acc)[IP][MATS], int64_t gg, int par, float res) {
        xpose_reduce<IP, MATS>(acc, lane, bp32);
        if constexpr (KS == 1) {
            epilogue(acc[0], gg, res);
        } else {
            if (writer)
#pragma unroll
                for (int m = 0; m < MATS; ++m)
                    s_comb[par][wave][my_item][m] = acc[0][m];
            __syncthreads();
            if (ks == 0) {
                float v[MATS];
#pragma unroll
                for (int m = 0; m < MATS; ++m) {
                    v[m] = 0.f;
                    if (writer)
                        for (int q = 0; q < KS; ++q)
                            v[m] += s_comb[par][wave + q][my_item][m];
                }
                epilogue(v, gg, res);
            }
        }
        if (++nout == QG_OUT_GROUPS) {
            if (KS == 1 || ks == 0)
                flush();
            // retire the stores here (vmcnt 0, other counters untouched), so that only loads
            // are outstanding where the loop continues and the compiler's waits stay exact
            __builtin_amdgcn_s_waitcnt(0x0F70);
            nout = 0;
            gout = gg + W;
        }
    };

    int64_t g = g0;
    for (int64_t it = 0; KS > 1 ? it < steps : g < T; ++it) {
        {
            float acc[IP][MATS];
            compute_group<FMT, NB, 1, MATS, R, IP>(bufA, xc, C, cme, acc);
            const float res = resA;
            load_group(bufA, mat, qrow, srow, a.N, lo, g + 2 * W);
            resA = load_res(g + 2 * W);
            finish(acc, g, 0, res);
        }
        g += W;
        ++it;
        if (KS > 1 ? it >= steps : g >= T)
            break;
        {
            float acc[IP][MATS];
            compute_group<FMT, NB, 1, MATS, R, IP>(bufB, xc, C, cme, acc);
            const float res = resB;
            load_group(bufB, mat, qrow, srow, a.N, lo, g + 2 * W);
            resB = load_res(g + 2 * W);
            finish(acc, g, 1, res);
        }
        g += W;
    }
    if (KS == 1 || ks == 0)
        flush();

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
                s_key[r * 4 + wave] = k;
        }
        __syncthreads();
        if (threadIdx.x < NB) {
            const int r = threadIdx.x;
            unsigned long long k = s_key[r * 4];
            for (int w = 1; w < 4; ++w)
                k = s_key[r * 4 + w] > k ? s_key[r * 4 + w] : k;
            a.keys[(int64_t)blockIdx.x * NB + r] = k;
        }
    }
}

// idx[r] from the per-workgroup partial keys [n_part][nb] of an argmax launch (one workgroup).
__global__ __launch_bounds__(256) void k_argmax_fold(const unsigned long long *part, int n_part,
                                                     int nb, int32_t *idx)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int r = wave; r < nb; r += 4) {
        unsigned long long k = 0ull;
        for (int b = lane; b < n_part; b += 64) {
            const unsigned long long o = part[(int64_t)b * nb + r];
            k = o > k ? o : k;
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

// Workgroup (expert e, row tile): the (row, slot) pairs routed to e are found by a parallel scan
// (kept in (row, slot) order), their x rows staged, and the tile's rows of W_e streamed by the
// four waves, writing part[r][t][n] = (W_e x_r)[n].  k_moe_combine then forms
// y[r][n] = sum_t wts[r][t] part[r][t][n] in ascending t.
template <int FMT, int NB, int CPL>
__device__ void moe_stream(const MoeArgs &a, const uint8_t *eq, const uint8_t *es, const int *pr,
                           const int *pt, int np,
                           int64_t row0, int64_t rows)
{
    using P = SP<FMT, NB, CPL, 1>;
    constexpr int R = P::R, IP = P::IP;
    constexpr int LG = IP == 1 ? 0 : IP == 2 ? 1 : IP == 4 ? 2 : IP == 8 ? 3 : IP == 16 ? 4 : 5;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int C = (int)(a.qs_row / 16);
    const float *xrow[NB];
#pragma unroll
    for (int r = 0; r < NB; ++r)
        xrow[r] = r < np ? a.x + (int64_t)pr[r] * a.K : nullptr;

    // rows of this tile, relative to row0, in groups of R; four waves, prefetch distance 2
    const int64_t T = (rows + R - 1) / R;
    const int64_t W = 4;
    int64_t g = wave;
    const BufMat tm[1] = {buf_mat(eq + row0 * a.qs_row, es + row0 * a.sc_row,
                                  (uint32_t)(rows * a.qs_row), (uint32_t)(rows * a.sc_row))};
    const LaneOff<CPL> lo = lane_offsets<FMT, CPL>(lane, C);
    const uint32_t qrow = (uint32_t)a.qs_row, srow = (uint32_t)a.sc_row;
    XCache<FMT, NB, CPL> xc;
    load_x_rows<FMT, NB, CPL>(xc, xrow, C, lane);
    GroupBuf<FMT, CPL, 1, R> bufA, bufB;
    load_group(bufA, tm, qrow, srow, rows, lo, g);
    load_group(bufB, tm, qrow, srow, rows, lo, g + W);

    const int my_item = lane >> (6 - LG);
    const bool writer = (lane & ((64 >> LG) - 1)) == 0 && my_item < P::ITEMS;
    const int my_u = my_item / NB, my_r = my_item % NB;
    auto finish = [&](float (&acc)[IP][1], int64_t gg) {
        xpose_reduce<IP, 1>(acc, lane, (lane ^ 32) << 2);
        const int64_t n = gg * R + my_u;
        if (writer && n < rows && my_r < np)
            a.part[((int64_t)pr[my_r] * a.topk + pt[my_r]) * a.N + row0 + n] = acc[0][0];
    };
    while (g < T) {
        {
            float acc[IP][1];
            compute_group<FMT, NB, CPL, 1, R, IP>(bufA, xc, C, lane, acc);
            load_group(bufA, tm, qrow, srow, rows, lo, g + 2 * W);
            finish(acc, g);
        }
        g += W;
        if (g >= T)
            break;
        {
            float acc[IP][1];
            compute_group<FMT, NB, CPL, 1, R, IP>(bufB, xc, C, lane, acc);
            load_group(bufB, tm, qrow, srow, rows, lo, g + 2 * W);
            finish(acc, g);
        }
        g += W;
    }
}

template <int FMT, int CPL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void k_moe_stream(MoeArgs a)
{
    __shared__ int s_pr[QG_PAIRS_MAX];
    __shared__ int s_pt[QG_PAIRS_MAX];
    __shared__ int s_cnt[QG_PAIRS_MAX / 64];

    const int64_t e = blockIdx.x % a.n_exp;
    const int64_t tile = blockIdx.x / a.n_exp;
    const int64_t tile_rows = a.tile_rows;
    const int64_t row0 = tile * tile_rows;
    const int64_t rows = (a.N - row0) < tile_rows ? (a.N - row0) : tile_rows;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

    // parallel scan of the routing table: pair p = (p / topk, p % topk) is ours if ids[p] == e
    const int npairs = a.nb * a.topk;
    int32_t id = -1;
    if ((int)threadIdx.x < npairs)
        id = a.ids[threadIdx.x];
    const bool mine = id == (int32_t)e;
    const bool bad = (int)threadIdx.x < npairs && (id < 0 || id >= a.n_exp);
    const unsigned long long ball = __ballot(mine);
    if (lane == 0 && wave < QG_PAIRS_MAX / 64)
        s_cnt[wave] = __popcll(ball);
    if (bad && e == 0 && tile == 0)
        atomicOr(a.err, 1u);
    __syncthreads();
    if (mine) {
        int pos = __popcll(ball & ((1ull << lane) - 1ull));
        for (int w = 0; w < wave; ++w)
            pos += s_cnt[w];
        s_pr[pos] = (int)threadIdx.x / a.topk;
        s_pt[pos] = (int)threadIdx.x % a.topk;
    }
    __syncthreads();
    int np = 0;
    for (int w = 0; w < QG_PAIRS_MAX / 64; ++w)
        np += s_cnt[w];

    const uint8_t *eq = a.qs + e * a.N * a.qs_row, *es = a.sc + e * a.N * a.sc_row;
    for (int g0 = 0; g0 < np; g0 += a.group_max) {
        const int ng = np - g0 < a.group_max ? np - g0 : a.group_max;
        // group_max = 4 / CPL keeps rows x chunks <= 4 (x held in registers)
        if (ng == 1) {
            moe_stream<FMT, 1, CPL>(a, eq, es, s_pr + g0, s_pt + g0, ng, row0, rows);
        } else if constexpr (CPL <= 2) {
            if (ng == 2) {
                moe_stream<FMT, 2, CPL>(a, eq, es, s_pr + g0, s_pt + g0, ng, row0, rows);
            } else if constexpr (CPL == 1) {
                moe_stream<FMT, 4, CPL>(a, eq, es, s_pr + g0, s_pt + g0, ng, row0, rows);
            }
        }
    }
}

// y[r][n] = sum_t wts[r][t] part[r][t][n], t ascending, skipping out-of-range expert ids.
__global__ __launch_bounds__(256) void k_moe_combine(const float *part, const int32_t *ids,
                                                     const float *wts, int nb, int topk,
                                                     int64_t n_exp, int64_t N, float *y)
{
    const int64_t total = (int64_t)nb * N;
    for (int64_t f = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; f < total;
         f += (int64_t)gridDim.x * blockDim.x) {
        const int r = (int)(f / N);
        const int64_t n = f % N;
        float acc = 0.f;
        for (int t = 0; t < topk; ++t) {
            const int32_t id = ids[r * topk + t];
            if (id < 0 || id >= n_exp)
                continue;
            acc = fmaf(wts[r * topk + t], part[((int64_t)r * topk + t) * N + n], acc);
        }
        y[f] = acc;
    }
}

// ------------------------------------------------------------------------------------ launchers

template <int FMT, int EPI, bool NRM, int CPL>
static int launch_stream_nb(const GemvArgs &a, int grid, size_t lds, hipStream_t s)
{
    switch (a.nb) {
    case 1: hipLaunchKernelGGL((k_stream<FMT, 1, CPL, EPI, NRM>), dim3(grid), dim3(256), lds, s, a); break;
    case 2: hipLaunchKernelGGL((k_stream<FMT, 2, CPL, EPI, NRM>), dim3(grid), dim3(256), lds, s, a); break;
    case 3: hipLaunchKernelGGL((k_stream<FMT, 3, CPL, EPI, NRM>), dim3(grid), dim3(256), lds, s, a); break;
    case 4: hipLaunchKernelGGL((k_stream<FMT, 4, CPL, EPI, NRM>), dim3(grid), dim3(256), lds, s, a); break;
    default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

template <int FMT, int EPI, bool NRM>
static int launch_stream_cpl(int cpl, const GemvArgs &a, int grid, size_t lds, hipStream_t s)
{
    switch (cpl) {
    case 1: return launch_stream_nb<FMT, EPI, NRM, 1>(a, grid, lds, s);
    case 2: return launch_stream_nb<FMT, EPI, NRM, 2>(a, grid, lds, s);
    case 4: return launch_stream_nb<FMT, EPI, NRM, 4>(a, grid, lds, s);
    default: return (int)hipErrorInvalidValue;
    }
}

template <int FMT>
static int launch_stream_fmt(int epi, bool nrm, int cpl, const GemvArgs &a, int grid, size_t lds,
                             hipStream_t s)
{
    switch (epi) {
    case E_STORE:
        return nrm ? launch_stream_cpl<FMT, E_STORE, true>(cpl, a, grid, lds, s)
                   : launch_stream_cpl<FMT, E_STORE, false>(cpl, a, grid, lds, s);
    case E_RES:
        return launch_stream_cpl<FMT, E_RES, false>(cpl, a, grid, lds, s);
    case E_GUS:
        return launch_stream_cpl<FMT, E_GUS, true>(cpl, a, grid, lds, s);
    case E_ARGMAX:
        return launch_stream_cpl<FMT, E_ARGMAX, false>(cpl, a, grid, lds, s);
    default:
        return (int)hipErrorInvalidValue;
    }
}

int launch_stream(int fmt, int epi, bool nrm, int cpl, const GemvArgs &a, int grid,
                  size_t lds_bytes, void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (fmt == FQ4_0)
        return launch_stream_fmt<FQ4_0>(epi, nrm, cpl, a, grid, lds_bytes, s);
    if (fmt == FQ8_0)
        return launch_stream_fmt<FQ8_0>(epi, nrm, cpl, a, grid, lds_bytes, s);
    if (fmt == FQ4_K)
        return launch_stream_fmt<FQ4_K>(epi, nrm, cpl, a, grid, lds_bytes, s);
    return (int)hipErrorInvalidValue;
}

template <int FMT>
static int launch_moe_fmt(int cpl, const MoeArgs &a, int grid, size_t lds, hipStream_t s)
{
    switch (cpl) {
    case 1: hipLaunchKernelGGL((k_moe_stream<FMT, 1>), dim3(grid), dim3(256), lds, s, a); break;
    case 2: hipLaunchKernelGGL((k_moe_stream<FMT, 2>), dim3(grid), dim3(256), lds, s, a); break;
    case 4: hipLaunchKernelGGL((k_moe_stream<FMT, 4>), dim3(grid), dim3(256), lds, s, a); break;
    default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

int launch_moe(int fmt, int cpl, const MoeArgs &a, int grid, size_t lds_bytes, void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    int err = (int)hipErrorInvalidValue;
    if (fmt == FQ4_0)
        err = launch_moe_fmt<FQ4_0>(cpl, a, grid, lds_bytes, s);
    else if (fmt == FQ8_0)
        err = launch_moe_fmt<FQ8_0>(cpl, a, grid, lds_bytes, s);
    else if (fmt == FQ4_K)
        err = launch_moe_fmt<FQ4_K>(cpl, a, grid, lds_bytes, s);
    if (err)
        return err;
    const int64_t total = (int64_t)a.nb * a.N;
    const int cgrid = (int)((total + 255) / 256 < 1024 ? (total + 255) / 256 : 1024);
    hipLaunchKernelGGL(k_moe_combine, dim3(cgrid), dim3(256), 0, s, a.part, a.ids, a.wts, a.nb,
                       a.topk, a.n_exp, a.N, a.y);
    return (int)hipGetLastError();
}

int launch_argmax_fold(const unsigned long long *part, int n_part, int nb, int32_t *idx,
                       void *stream)
{
    hipLaunchKernelGGL(k_argmax_fold, dim3(1), dim3(256), 0, static_cast<hipStream_t>(stream),
                       part, n_part, nb, idx);
    return (int)hipGetLastError();
}

// ------------------------------------------------------------------------------------ occupancy

template <int FMT, int EPI, bool NRM, int CPL>
static const void *stream_fn_nb(int nb)
{
    switch (nb) {
    case 1: return reinterpret_cast<const void *>(&k_stream<FMT, 1, CPL, EPI, NRM>);
    case 2: return reinterpret_cast<const void *>(&k_stream<FMT, 2, CPL, EPI, NRM>);
    case 3: return reinterpret_cast<const void *>(&k_stream<FMT, 3, CPL, EPI, NRM>);
    case 4: return reinterpret_cast<const void *>(&k_stream<FMT, 4, CPL, EPI, NRM>);
    default: return nullptr;
    }
}

template <int FMT, int EPI, bool NRM>
static const void *stream_fn_cpl(int cpl, int nb)
{
    return cpl == 1 ? stream_fn_nb<FMT, EPI, NRM, 1>(nb)
         : cpl == 2 ? stream_fn_nb<FMT, EPI, NRM, 2>(nb)
         : cpl == 4 ? stream_fn_nb<FMT, EPI, NRM, 4>(nb) : nullptr;
}

template <int FMT>
static const void *stream_fn_fmt(int epi, bool nrm, int cpl, int nb)
{
    switch (epi) {
    case E_STORE:
        return nrm ? stream_fn_cpl<FMT, E_STORE, true>(cpl, nb)
                   : stream_fn_cpl<FMT, E_STORE, false>(cpl, nb);
    case E_RES: return stream_fn_cpl<FMT, E_RES, false>(cpl, nb);
    case E_GUS: return stream_fn_cpl<FMT, E_GUS, true>(cpl, nb);
    case E_ARGMAX: return stream_fn_cpl<FMT, E_ARGMAX, false>(cpl, nb);
    default: return nullptr;
    }
}

int stream_resident_wgs(int fmt, int epi, bool nrm, int cpl, int nb, size_t lds_bytes)
{
    const void *fn = fmt == FQ4_0 ? stream_fn_fmt<FQ4_0>(epi, nrm, cpl, nb)
                   : fmt == FQ8_0 ? stream_fn_fmt<FQ8_0>(epi, nrm, cpl, nb)
                   : fmt == FQ4_K ? stream_fn_fmt<FQ4_K>(epi, nrm, cpl, nb) : nullptr;
    if (!fn)
        return 0;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, lds_bytes) != hipSuccess)
        return 0;
    return cus * per_cu;
}

}  // namespace qg

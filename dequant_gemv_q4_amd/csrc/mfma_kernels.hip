// mfma_kernels.hip -- row-batch (5 <= nb <= 16) dequant GEMV on the gfx950 matrix cores.
//
// With a batch of up to 16 activation rows the product is a small dense contraction, so it runs
// on v_mfma_f32_16x16x32_f16: D[b][n] = sum_k X[b][k] W[n][k] over one quant block of 32 k at a
// time, b the batch row (padded to 16) and n one of 16 weight rows.  The weights sit in the B
// operand, so each lane's four results belong to a single weight row and take a single block
// scale: acc += d * D (f32, VALU).  Same arithmetic as the vector path:
//  - weights: nibbles (or Q8_0 bytes + 128) are placed in the mantissa of 1024.0 (f16 0x6400) by
//    one and-or per pair, then the offset (1032, or 1152 for a high nibble held x16 and for Q8_0)
//    is subtracted with one packed f16 add: exact q - 8 (16 (q - 8)) or exact q;
//  - x: each batch row scaled by a power of two that puts its largest |x| in [2^14, 2^15),
//    rounded to f16 (relative error <= 2^-11); x at a high-nibble position carries 1/16.  The row
//    scale is undone, exactly, on the results.
// Operand layouts (CDNA4 16x16x32 f16): lane l holds A[l % 16][8 (l / 16) + 0..7] and
// B[8 (l / 16) + 0..7][l % 16], and D[4 (l / 16) + 0..3][l % 16].  A k position may be any
// element as long as A and B agree, so the eight halves a lane holds for one block are the eight
// elements of one dword of quant bytes (Q4_0: bytes 4j..4j+3, their low and high nibbles; Q8_0:
// bytes 4j..4j+3 of both 16-byte halves of the block).
//
// Loads: lane (row i = l % 16, c = l / 16) reads the 16-byte chunk 4 s + c of weight row i for
// step s; a 4 x 4 transpose of dwords across the four 16-lane rows (v_permlane32_swap, then
// v_permlane16_swap) leaves in lane (i, j) dword j of each of the four chunks: the B operands of
// the step's four blocks (Q4_0) or two blocks (Q8_0).
//
// Q4_K ("Crate inferencelayer" docs, gemv_q4_k_lcpp_src; w = d sc q - dmin m per 32-weight
// sub-block): a step is half a super-block, four 16-byte chunks; chunks 2p and 2p + 1 hold one
// sub-block in their low nibbles and the next in their high nibbles, so each sub-block is one
// 32-k product over the low (or high) nibbles of dword j of the two chunks.  Its weights are
// centred as on the vector path (k_center: B = q - c, exact) and the term (a c - b) sum x comes
// from a second product of the same x with all-ones weights; the x sums are those of the f16 x
// the products use.
#include <hip/hip_runtime.h>

#include "mfma_common.h"

#include <mutex>
#include <vector>

namespace qg {

template <int OFF>
__device__ __forceinline__ float mf_xor(float v)
{
    return __shfl_xor(v, OFF);
}

// Persistent workgroups of 16 waves; x (the 16 padded batch rows, all of K) is staged once per
// workgroup.  Work comes in groups of TPW consecutive 16-row tiles (group g = blockIdx.x,
// blockIdx.x + gridDim.x, ...: the grid reads one dense window).  In a group, wave w takes tile
// w / KS and K slice w % KS (KS = 16 / TPW waves per tile), i.e. steps slice, slice + KS, ...,
// streamed through two register buffers.  With KS > 1 the slices' partial tiles are added in LDS
// in slice order.  K class KC: K <= 2048 KC (x: 8 KC float4s per lane).  SV: a step's block
// scales of a row are contiguous and aligned (K a multiple of 128 for Q4_0, 64 for Q8_0), so one
// 8- or 4-byte load per lane fetches them (else one 2-byte load per block).
template <int FMT, int EPI, bool NRM, int KC, int TPW, bool SV>
__global__ __launch_bounds__(MF_THREADS) void k_mfma(GemvArgs a)
{
    constexpr int MATS = EPI == E_GUS ? 2 : 1;
    // blocks (K-quants: 32-weight sub-blocks; Q6_K: 16-weight ones) per step
    constexpr int BPS = FMT == FQ8_0 ? 2 : FMT == FQ6_K ? 8 : 4;
    // Q1_0: the step's four sign words come with its round (16 bytes of a row per step)
    constexpr int QW = FMT == FQ1_0 ? 4 : 0;
    // scale dwords of a step: the f16 d of its blocks (two a dword), the K-quants' 16-byte
    // header, IQ4_XS's 8-byte header, the affine format's (s, c) per block, Q6_K's eight signed
    // scales and its f16 d, Q1_0's one f16 d
    constexpr int SW = fmt_min(FMT) || FMT == FAQ4 ? 4 : FMT == FQ6_K ? 3
                     : FMT == FQ8_0 || FMT == FQ1_0 ? 1 : 2;
    // high-bit dwords of a step (Q5_0, Q5_K: one per chunk; Q6_K: two per chunk)
    constexpr int HW = FMT == FQ5_0 || FMT == FQ5_K ? 4 : FMT == FQ6_K ? 8 : 0;
    constexpr int AW = QW + SW + HW;             // dwords a step takes from its round's loads
    constexpr int MF_XR = 8 * KC;                // float4s of x a lane stages
    constexpr int KS = MF_WAVES / TPW;           // waves per tile
    constexpr int PD = TPW >= 8 && MATS == 1 ? 4 : 2;   // steps in flight per wave (8: slower)
    // steps whose scales one load brings (SV); the gated product holds two matrices' loads and
    // keeps one step per load (registers)
    constexpr int SG = MATS == 2 ? 1 : PD < 4 ? PD : 4;
    extern __shared__ float4 mf_lds[];
    __shared__ float s_rs[16];
    __shared__ unsigned long long s_best[16];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // C: 16-byte pieces of a row; S: steps of 128 weights (Q8_0: 64)
    const int C = (int)(a.qs_row / 16), S = FMT == FQ1_0 ? C : (C + 3) / 4, KB = (int)(a.K / 32);
    const int K4 = (int)(a.K / 4);
    uint8_t *XA = reinterpret_cast<uint8_t *>(mf_lds);                   // [KB][4][16] x 16 B
    float *PART = reinterpret_cast<float *>(XA + (size_t)KB * 1024);    // [16][MATS][4][64]

    // ---- x loads (this lane's float4s of batch row `wave`) and gamma
    const int bx = wave;   // the batch row this wave stages
    const bool xrow = bx < a.nb;
    float4 xv[MF_XR];
#pragma unroll
    for (int i = 0; i < MF_XR; ++i) {
        const int f = lane + 64 * i;
        const int fc = f < K4 ? f : K4 - 1;
        xv[i] = reinterpret_cast<const float4 *>(a.x)[(int64_t)(xrow ? bx : 0) * K4 + fc];
    }
    // the weight pointers' kernel-argument line is fetched now, beside x's, not after x arrives
    asm volatile("" ::"s"(a.qs0), "s"(a.sc0));
    if constexpr (MATS == 2)
        asm volatile("" ::"s"(a.qs1), "s"(a.sc1));
    // gamma (norm): K4 <= 512 float4s, one per thread, staged in the (not yet used) result area
    float4 gone = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (NRM)
        gone = reinterpret_cast<const float4 *>(a.gamma)[tid < K4 ? tid : K4 - 1];
    float4 *G4 = reinterpret_cast<float4 *>(PART);
    if (tid < 16)
        s_best[tid] = 0ull;

    const int ir = lane & 15, lc = lane >> 4;
    const uint32_t qbytes = (uint32_t)(a.N * a.qs_row), sbytes = (uint32_t)(a.N * a.sc_row);
    const uint32_t hbytes = (uint32_t)(a.N * a.hb_row);
    const uint32_t dbytes = (uint32_t)(a.N * a.d_row);
    __amdgpu_buffer_rsrc_t rq[MATS], rsc[MATS], rhb[MATS], rdd[MATS];
    rq[0] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.qs0), (short)0, (int)qbytes, 0x00020000);
    rsc[0] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.sc0), (short)0, (int)sbytes, 0x00020000);
    rhb[0] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(HW ? a.hb0 : a.qs0), (short)0, (int)(HW ? hbytes : 0u), 0x00020000);
    rdd[0] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(FMT == FQ6_K ? a.dd0 : a.qs0), (short)0, (int)(FMT == FQ6_K ? dbytes : 0u), 0x00020000);
    if constexpr (MATS == 2) {
        rq[1] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.qs1), (short)0, (int)qbytes, 0x00020000);
        rsc[1] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.sc1), (short)0, (int)sbytes, 0x00020000);
        rhb[1] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(HW ? a.hb1 : a.qs1), (short)0, (int)(HW ? hbytes : 0u), 0x00020000);
        rdd[1] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(FMT == FQ6_K ? a.dd1 : a.qs1), (short)0, (int)(FMT == FQ6_K ? dbytes : 0u), 0x00020000);
    }
    // IQ4 formats: each matrix's codebook, every entry + 128 as an unsigned byte
    uint4 cbt[MATS];
#pragma unroll
    for (int m = 0; m < MATS; ++m) {
        cbt[m] = make_uint4(0u, 0u, 0u, 0u);
        if constexpr (fmt_codebook(FMT)) {
            const uint4 t = *reinterpret_cast<const uint4 *>(m == 0 ? a.cb0 : a.cb1);
            cbt[m] = make_uint4(t.x ^ 0x80808080u, t.y ^ 0x80808080u, t.z ^ 0x80808080u,
                                t.w ^ 0x80808080u);
        }
    }
    const int64_t NT = (a.N + 15) / 16, G = (NT + TPW - 1) / TPW;
    const int my_t = wave / KS, slice = wave % KS;
    const int nst = S > slice ? (S - 1 - slice) / KS + 1 : 0;   // this wave's steps per tile

    // one step's loads: the lane's 16-byte chunk of its row and the step's block scales.  SV: the
    // first step of a round of PD steps also loads the round's scales, lane (i, c) those of step
    // k + c % PD of row i (one load instruction per round instead of one per step, each touching
    // 16 scale lines); a step takes its scales from lane i + 16 (k % PD)
    struct StepBuf {
        uint32_t q[MATS][4];
        uint16_t s[MATS][BPS];        // per-block scale loads
        uint32_t sw[MATS][AW];        // SV: scales (then high bits) of step k + c % SG as loaded
    };
    auto load_step = [&](StepBuf &sb, int64_t n, int k, bool round_first) {
        const int kk = k < nst ? k : nst - 1;              // past the wave's steps: its last
        const int st = slice + KS * (kk > 0 ? kk : 0);      // (a wave with none: a clamped chunk)
        const int ch = 4 * st + lc < C ? 4 * st + lc : C - 1;
        const int ks = k + lc % SG < nst ? k + lc % SG : nst - 1;
        const int sst = slice + KS * (ks > 0 ? ks : 0);     // the step whose scales this lane loads
#pragma unroll
        for (int m = 0; m < MATS; ++m) {
            if constexpr (QW == 0) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(
                    rq[m], (int)((uint32_t)n * (uint32_t)a.qs_row + 16u * (uint32_t)ch), 0, QG_WCPOL);
                sb.q[m][0] = v[0]; sb.q[m][1] = v[1]; sb.q[m][2] = v[2]; sb.q[m][3] = v[3];
            } else {
                sb.q[m][0] = sb.q[m][1] = sb.q[m][2] = sb.q[m][3] = 0u;
            }
            if constexpr (SV) {
                // raw dwords: halves are split where they are used, so that no instruction
                // touches the load's result before its step is computed
                if (!round_first)   // known at compile time where the loop is unrolled
                    continue;
                if constexpr (FMT == FQ1_0) {
                    // the step's 16 bytes of sign words and its f16 d
                    const auto w = __builtin_amdgcn_raw_buffer_load_b128(
                        rq[m], (int)((uint32_t)n * (uint32_t)a.qs_row + 16u * (uint32_t)sst), 0, QG_WCPOL);
                    sb.sw[m][0] = w[0]; sb.sw[m][1] = w[1]; sb.sw[m][2] = w[2]; sb.sw[m][3] = w[3];
                    sb.sw[m][4] = __builtin_amdgcn_raw_buffer_load_b16(
                        rsc[m], (int)((uint32_t)n * (uint32_t)a.sc_row + 2u * (uint32_t)sst), 0, QG_WCPOL);
                    continue;
                }
                if constexpr (FMT == FQ6_K) {
                    // the eight signed scales of half sst % 2 of super-block sst / 2, its d, and
                    // the step's four chunks' high-bit word pairs
                    const auto w = __builtin_amdgcn_raw_buffer_load_b64(
                        rsc[m], (int)((uint32_t)n * (uint32_t)a.sc_row + 8u * (uint32_t)sst), 0, QG_WCPOL);
                    sb.sw[m][0] = w[0];
                    sb.sw[m][1] = w[1];
                    sb.sw[m][2] = __builtin_amdgcn_raw_buffer_load_b16(
                        rdd[m], (int)((uint32_t)n * (uint32_t)a.d_row + 2u * (uint32_t)(sst >> 1)), 0, QG_WCPOL);
                    const int ho = (int)((uint32_t)n * (uint32_t)a.hb_row + 32u * (uint32_t)sst);
                    const auto h0 = __builtin_amdgcn_raw_buffer_load_b128(rhb[m], ho, 0, QG_WCPOL);
                    const auto h1 = __builtin_amdgcn_raw_buffer_load_b128(rhb[m], ho + 16, 0, QG_WCPOL);
                    sb.sw[m][3] = h0[0]; sb.sw[m][4] = h0[1]; sb.sw[m][5] = h0[2]; sb.sw[m][6] = h0[3];
                    sb.sw[m][7] = h1[0]; sb.sw[m][8] = h1[1]; sb.sw[m][9] = h1[2]; sb.sw[m][10] = h1[3];
                    continue;
                }
                if constexpr (HW == 4) {
                    // the high-bit words of the step's four chunks
                    const int ho = (int)((uint32_t)n * (uint32_t)a.hb_row + 16u * (uint32_t)sst);
                    const auto w = __builtin_amdgcn_raw_buffer_load_b128(rhb[m], ho, 0, QG_WCPOL);
                    sb.sw[m][SW + 0] = w[0];
                    sb.sw[m][SW + 1] = w[1];
                    sb.sw[m][SW + 2] = w[2];
                    sb.sw[m][SW + 3] = w[3];
                }
                if constexpr (SW == 4) {
                    // K-quants: the header of super-block sst / 2 (two steps each); the affine
                    // format: (s, c) of the step's four blocks
                    const uint32_t off = fmt_min(FMT) ? 16u * (uint32_t)(sst >> 1) : 16u * (uint32_t)sst;
                    const int so = (int)((uint32_t)n * (uint32_t)a.sc_row + off);
                    const auto w = __builtin_amdgcn_raw_buffer_load_b128(rsc[m], so, 0, QG_WCPOL);
                    sb.sw[m][0] = w[0];
                    sb.sw[m][1] = w[1];
                    sb.sw[m][2] = w[2];
                    sb.sw[m][3] = w[3];
                    continue;
                }
                // f16 d per block (IQ4_XS: the 8-byte header of super-block sst / 2)
                const uint32_t off = FMT == FIQ4_XS ? 8u * (uint32_t)(sst >> 1) : 2u * BPS * (uint32_t)sst;
                const int so = (int)((uint32_t)n * (uint32_t)a.sc_row + off);
                if constexpr (BPS == 4) {
                    const auto w = __builtin_amdgcn_raw_buffer_load_b64(rsc[m], so, 0, QG_WCPOL);
                    sb.sw[m][0] = w[0];
                    sb.sw[m][1] = w[1];
                } else {
                    sb.sw[m][0] = __builtin_amdgcn_raw_buffer_load_b32(rsc[m], so, 0, QG_WCPOL);
                }
            } else {
#pragma unroll
                for (int b = 0; b < BPS; ++b) {
                    const int blk = BPS * st + b < KB ? BPS * st + b : KB - 1;
                    sb.s[m][b] = __builtin_amdgcn_raw_buffer_load_b16(
                        rsc[m], (int)((uint32_t)n * (uint32_t)a.sc_row + 2u * (uint32_t)blk), 0,
                        QG_WCPOL);
                }
            }
        }
    };
    auto tile_row = [&](int64_t grp) -> int64_t {
        const int64_t t = grp * TPW + my_t;
        const int64_t r = t * 16 + ir;
        return r < a.N ? r : a.N - 1;
    };
    // the first group's first PD steps go out once this wave's x has arrived
    StepBuf sbuf[PD];
    const int64_t grp0 = blockIdx.x;
    auto issue_first = [&]() {
#pragma unroll
        for (int p = 0; p < PD; ++p) {
            load_step(sbuf[p], tile_row(grp0), p, p % SG == 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if constexpr (NRM) {
        if (tid < K4)
            G4[tid] = gone;
        __syncthreads();
    }

    // ---- batch row `wave`: norm, scale, f16 pairs into the A layout
    {
        float ss = 0.f, mx = 0.f;
#pragma unroll
        for (int i = 0; i < MF_XR; ++i) {
            const int f = lane + 64 * i;
            float4 v = xv[i];
            if (f >= K4 || !xrow)
                v = make_float4(0.f, 0.f, 0.f, 0.f);
            if constexpr (NRM) {
                float q = v.x * v.x;
                q = fmaf(v.y, v.y, q);
                q = fmaf(v.z, v.z, q);
                q = fmaf(v.w, v.w, q);
                ss += q;
                const float4 g = G4[f < K4 ? f : K4 - 1];
                v = make_float4(v.x * g.x, v.y * g.y, v.z * g.z, v.w * g.w);
            }
            xv[i] = v;
            mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
        float inv = 1.0f;
        if constexpr (NRM) {
            ss += mf_xor<32>(ss);
            ss += mf_xor<16>(ss);
            ss += mf_xor<8>(ss);
            ss += mf_xor<4>(ss);
            ss += mf_xor<2>(ss);
            ss += mf_xor<1>(ss);
            inv = 1.0f / sqrtf(ss / (float)a.K + a.eps);
        }
        mx = fmaxf(mx, mf_xor<32>(mx));
        mx = fmaxf(mx, mf_xor<16>(mx));
        mx = fmaxf(mx, mf_xor<8>(mx));
        mx = fmaxf(mx, mf_xor<4>(mx));
        mx = fmaxf(mx, mf_xor<2>(mx));
        mx = fmaxf(mx, mf_xor<1>(mx));
        int e2 = 0;
        frexpf(mx * inv, &e2);
        const int sk = 15 - e2 < 127 ? 15 - e2 : 127;       // 2^sk stays a finite f32
        const float sc = inv * ldexpf(1.0f, sk), sh = sc * 0.0625f;
        if (lane == 0)
            s_rs[wave] = ldexpf(1.0f, -sk);
        // the first weight loads go out once this wave's x has arrived (x requests first in the
        // memory queues), before its conversion
        __builtin_amdgcn_sched_barrier(0);
        issue_first();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < MF_XR; ++i) {
            const int f = lane + 64 * i;
            if (f < K4) {
                const float e[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int el = 4 * f + t;
                    if constexpr (FMT == FQ6_K) {
                        // 16-k products: [16-element block][lane column c][row][4 halves],
                        // halves (b0, b2, b1, b3) of dword c
                        const int b16 = el >> 4, c = (el >> 2) & 3, tt = el & 3;
                        const int h = tt == 0 ? 0 : tt == 2 ? 1 : tt == 1 ? 2 : 3;
                        *reinterpret_cast<_Float16 *>(XA + (((size_t)(b16 * 4 + c) * 16 + bx) * 4 + h) * 2) =
                            (_Float16)(e[t] * sc);
                    } else {
                        const int blk = el >> 5;
                        int j, h;
                        bool hi;
                        mf_slot<FMT>(el & 31, j, h, hi);
                        const _Float16 hv = (_Float16)(e[t] * (hi ? sh : sc));
                        *reinterpret_cast<_Float16 *>(XA + (((size_t)(blk * 4 + j) * 16 + bx) * 8 + h) * 2) = hv;
                    }
                }
            }
        }
    }
    __syncthreads();

    const MfConst kc = mf_const<FMT>();
    // one step: transpose, B operands, one MFMA per block, scaled accumulation
    auto compute = [&](const StepBuf &sb, const uint32_t (&scl)[MATS][AW], int k,
                       float (&acc)[MATS][4]) {
        const int st = slice + KS * k;
        const mf4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < MATS; ++m) {
            if constexpr (FMT == FQ1_0) {
                // four 32-weight blocks of one scale: the products chain in the accumulator.
                // Lane (i, c) takes elements 4c + t and 4c + t + 16 (t < 4) of each block as the
                // pair t: the inverted sign bits shifted to the f16 sign bits over 1.0, 1.0
                mf4 D = zero;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t w = ~scl[m][b];
                    struct W4 {
                        uint32_t v[4];
                    } p;
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        p.v[t] = mf_and_or(w << (15 - 4 * lc - t), 0x80008000u, kc.c1);
                    const mh8 aop = *reinterpret_cast<const mh8 *>(
                        XA + ((size_t)((4 * st + b) * 4 + lc) * 16 + ir) * 16);
                    D = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, __builtin_bit_cast(mh8, p), D, 0, 0, 0);
                }
                const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(scl[m][4] & 0xffffu));
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[m][r] = fmaf(d, D[r], acc[m][r]);
                continue;
            }
            uint32_t q[4] = {sb.q[m][0], sb.q[m][1], sb.q[m][2], sb.q[m][3]};
            mf_xpose(q);
            if constexpr (FMT == FQ6_K) {
                // the step is half n of super-block st / 2: chunk u (< 4) holds the 16-weight
                // sub-block u of the half in its low nibbles (scale u) and u + 4 in its high ones;
                // lane (i, j) has dword j of each chunk: k = 4j..4j+3 of a 16-k product.  Six-bit
                // values: nibble | two high bits << 4, then q - 32 exact
                const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(scl[m][2] & 0xffffu));
                const int rot = (2 * lc + 28) & 31;   // bits 8m + 2j, +1 -> 8m + 4, 8m + 5
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t h0 = scl[m][3 + 2 * u], h1 = scl[m][4 + 2 * u];
                    const uint32_t lo = mf_and_or(q[u], 0x0F0F0F0Fu,
                                                  __builtin_amdgcn_alignbit(h0, h0, rot) & 0x30303030u);
                    const uint32_t hi = mf_and_or(q[u] >> 4, 0x0F0F0F0Fu,
                                                  __builtin_amdgcn_alignbit(h1, h1, rot) & 0x30303030u);
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const uint32_t by = half ? hi : lo;
                        struct W2 {
                            uint32_t v[2];
                        } p = {{mf_hadd(mf_and_or(by, kc.m_b, kc.c), 0xE420E420u),
                                mf_hadd(mf_and_or(by >> 8, kc.m_b, kc.c), 0xE420E420u)}};
                        const int b16 = 16 * (st >> 1) + 8 * (st & 1) + 4 * half + u;
                        const mh4 aop = *reinterpret_cast<const mh4 *>(
                            XA + ((size_t)(b16 * 4 + lc) * 16 + ir) * 8);
                        const mf4 D = __builtin_amdgcn_mfma_f32_16x16x16f16(
                            aop, __builtin_bit_cast(mh4, p), zero, 0, 0, 0);
                        const float sv = (float)(int8_t)((scl[m][half] >> (8 * u)) & 0xffu);
                        const float a_ = d * sv;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[m][r] = fmaf(a_, D[r], acc[m][r]);
                    }
                }
                continue;
            }
            if constexpr (FMT == FQ5_0 || fmt_codebook(FMT) || FMT == FAQ4) {
                // one 32-weight block per chunk: lane (i, j) holds dword j of block b's chunk
#pragma unroll
                for (int b = 0; b < BPS; ++b) {
                    const int blk = BPS * st + b;
                    const mh8 aop = *reinterpret_cast<const mh8 *>(
                        XA + ((size_t)(blk * 4 + lc) * 16 + ir) * 16);
                    if constexpr (FMT == FAQ4) {
                        // centred (aq_center): pairs q - c (high nibbles 16 (q - c)), and
                        // (s c + bias) times the block's x sum (a product with weights 1 / 16)
                        const uint32_t sc2 = scl[m][b];
                        const float s_ = (float)__builtin_bit_cast(_Float16, (uint16_t)(sc2 & 0xffffu));
                        const float nb_ = -(float)__builtin_bit_cast(_Float16, (uint16_t)(sc2 >> 16));
                        const float c = aq_center(s_, nb_);
                        const mh8 bop = mf_bop_aq(q[b], mf_splat_off(c), mf_splat_off(16.0f * c), kc);
                        const mf4 D = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, zero, 0, 0, 0);
                        const mf4 Sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, mf_ones_q4(), zero, 0, 0, 0);
                        const float res = fmaf(s_, c, -nb_);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[m][r] = fmaf(res, Sx[r], fmaf(s_, D[r], acc[m][r]));
                        continue;
                    }
                    mh8 bop;
                    if constexpr (FMT == FQ5_0) {
                        const uint32_t h = scl[m][SW + b];
                        bop = mf_bop_bytes(mf_join5_lo(q[b], h, lc), mf_join5_hi(q[b], h, lc),
                                           0xE410E410u, kc);   // -1040: 1024 + q -> q - 16
                    } else {
                        bop = mf_bop_cb(q[b], cbt[m], kc);
                    }
                    float d;
                    if constexpr (FMT == FIQ4_XS) {
                        // header: f16 d, the high scale bits (sub-block s at bits 2s, 2s + 1 of
                        // the next 16), then the low 4-bit scales (s at bits 4s..4s+3)
                        const int sbk = 4 * (st & 1) + b;
                        const uint32_t ls = ((scl[m][1] >> (4 * sbk)) & 15u) |
                                            (((scl[m][0] >> (16 + 2 * sbk)) & 3u) << 4);
                        d = (float)__builtin_bit_cast(_Float16, (uint16_t)(scl[m][0] & 0xffffu)) *
                            (float)((int)ls - 32);
                    } else {
                        d = (float)__builtin_bit_cast(_Float16,
                                                       (uint16_t)(scl[m][b >> 1] >> (16 * (b & 1))));
                    }
                    const mf4 D = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, zero, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[m][r] = fmaf(d, D[r], acc[m][r]);
                }
                continue;
            }
            if constexpr (fmt_min(FMT)) {
                // the step is half h of super-block st / 2: its chunks 4h + b (b < 4).  Chunk pair
                // (4h + 2p, 4h + 2p + 1) holds sub-block 4h + 2p in its low nibbles (the pair's
                // 32 weights, lane (i, j) dword j of each) and 4h + 2p + 1 in its high nibbles.
                // Centred weights (k_center): B = q - c exact; the offset term (a c - b) sum x
                // comes from a second product with all-ones weights (sum of the same f16 x)
                const uint4 hdr = make_uint4(scl[m][0], scl[m][1], scl[m][2], scl[m][3]);
                const int half = st & 1;
#pragma unroll
                for (int p2 = 0; p2 < 2; ++p2) {
                    const ChunkScale cs = chunk_scale<FQ4_K>(hdr, 4 * half + 2 * p2);
                    const uint32_t q0 = q[2 * p2], q1 = q[2 * p2 + 1];
#pragma unroll
                    for (int hi = 0; hi < 2; ++hi) {
                        const float a_ = hi ? cs.a2 : cs.a, b_ = hi ? cs.b2 : cs.b;
                        const float c = k_center(a_, b_);
                        mh8 bop;
                        if constexpr (FMT == FQ5_K) {
                            // nibbles joined with their fifth bits into bytes (0..31)
                            const uint32_t h0 = scl[m][SW + 2 * p2], h1 = scl[m][SW + 2 * p2 + 1];
                            bop = hi ? mf_bop_bytes(mf_join5_hi(q0, h0, lc), mf_join5_hi(q1, h1, lc),
                                                    mf_splat_off(c), kc)
                                     : mf_bop_bytes(mf_join5_lo(q0, h0, lc), mf_join5_lo(q1, h1, lc),
                                                    mf_splat_off(c), kc);
                        } else {
                            bop = mf_bop_k(hi ? q0 >> 4 : q0, hi ? q1 >> 4 : q1, mf_splat_off(c), kc);
                        }
                        const int blk = 8 * (st >> 1) + 4 * half + 2 * p2 + hi;
                        const mh8 aop = *reinterpret_cast<const mh8 *>(
                            XA + ((size_t)(blk * 4 + lc) * 16 + ir) * 16);
                        const mf4 D = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, zero, 0, 0, 0);
                        const mf4 Sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, kc_ones(), zero, 0, 0, 0);
                        const float res = fmaf(a_, c, -b_);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[m][r] = fmaf(res, Sx[r], fmaf(a_, D[r], acc[m][r]));
                    }
                }
                continue;
            }
#pragma unroll
            for (int b = 0; b < BPS; ++b) {
                const int blk = BPS * st + b;
                // SV: K is a whole number of steps, so every block of a step exists
                const float d =
                    SV ? (float)__builtin_bit_cast(
                             _Float16, (uint16_t)(scl[m][b >> 1] >> (16 * (b & 1))))
                       : blk < KB ? (float)__builtin_bit_cast(_Float16, sb.s[m][b]) : 0.f;
                const mh8 bop = FMT == FQ8_0 ? mf_bop<FMT>(q[2 * b], q[2 * b + 1], kc)
                                             : mf_bop<FMT>(q[b], 0u, kc);
                const int blc = SV || blk < KB ? blk : KB - 1;
                const mh8 aop = *reinterpret_cast<const mh8 *>(
                    XA + ((size_t)(blc * 4 + lc) * 16 + ir) * 16);
                const mf4 zero = {0.f, 0.f, 0.f, 0.f};
                const mf4 D = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, zero, 0, 0, 0);
                acc[m][0] = fmaf(d, D[0], acc[m][0]);
                acc[m][1] = fmaf(d, D[1], acc[m][1]);
                acc[m][2] = fmaf(d, D[2], acc[m][2]);
                acc[m][3] = fmaf(d, D[3], acc[m][3]);
            }
        }
    };
    // result of (batch row b, tile row nn) from the summed, row-scaled values v
    auto epilogue = [&](const float (&v)[MATS], int b, int64_t nn) {
        const bool ok = b < a.nb && nn < a.N;
        float out;
        if constexpr (EPI == E_GUS) {
            out = gated(v[0], v[MATS - 1], a.act);
        } else if constexpr (EPI == E_RES) {
            out = v[0] + (ok ? a.res[(int64_t)b * a.res_rstride + nn] : 0.f);
        } else {
            out = v[0];
        }
        if (ok) {
            a.y[(int64_t)b * a.N + nn] = out;
            if constexpr (EPI == E_ARGMAX)
                atomicMax(&s_best[b], argmax_key(out, nn));
        }
    };

    for (int64_t grp = grp0; grp < G; grp += gridDim.x) {
        const int64_t n = tile_row(grp);
        float acc[MATS][4];
#pragma unroll
        for (int m = 0; m < MATS; ++m)
            acc[m][0] = acc[m][1] = acc[m][2] = acc[m][3] = 0.f;
        if (grp != grp0) {
#pragma unroll
            for (int p = 0; p < PD; ++p)
                load_step(sbuf[p], n, p, p % SG == 0);
        }
        // rounds of PD steps (the loop has one exit, at the end of a round); a step past the
        // wave's own is skipped, its buffer re-loaded with the wave's last step
        for (int k = 0; k < nst; k += PD) {
            uint32_t scl[PD][MATS][AW];
#pragma unroll
            for (int p = 0; p < PD; ++p) {
                // at the first step of a scale group, its steps' scales: step p + j's from lane
                // ir + 16 j of the group's first buffer (before that buffer is loaded again)
                if (p % SG == 0)
#pragma unroll
                    for (int j = 0; j < SG; ++j)
#pragma unroll
                        for (int m = 0; m < MATS; ++m)
#pragma unroll
                            for (int d = 0; d < AW; ++d)
                                scl[p + j][m][d] =
                                    !SV ? 0u
                                    : SG == 1 ? sbuf[p].sw[m][d]
                                              : (uint32_t)__builtin_amdgcn_ds_bpermute(
                                                    (ir + 16 * j) << 2, (int)sbuf[p].sw[m][d]);
                if (k + p < nst)
                    compute(sbuf[p], scl[p], k + p, acc);
                load_step(sbuf[p], n, k + p + PD, p % SG == 0);
            }
        }
        const int64_t tile = grp * TPW + my_t;
        if constexpr (KS == 1) {
            // the wave owns its tile: lane l holds batch rows 4 (l / 16) + r of row l % 16
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int b = 4 * lc + r;
                float v[MATS];
#pragma unroll
                for (int m = 0; m < MATS; ++m)
                    v[m] = acc[m][r] * s_rs[b];
                epilogue(v, b, tile * 16 + ir);
            }
        } else {
#pragma unroll
            for (int m = 0; m < MATS; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    PART[((wave * MATS + m) * 4 + r) * 64 + lane] = acc[m][r];
            __syncthreads();
            for (int e = tid; e < TPW * 256; e += MF_THREADS) {
                const int tt = e >> 8, b = (e >> 4) & 15, ri = e & 15;
                const int src = (b >> 2) * 16 + ri, r = b & 3;
                float v[MATS];
#pragma unroll
                for (int m = 0; m < MATS; ++m) {
                    float sum = 0.f;
                    for (int q = 0; q < KS; ++q)
                        sum += PART[(((tt * KS + q) * MATS + m) * 4 + r) * 64 + src];
                    v[m] = sum * s_rs[b];
                }
                epilogue(v, b, (grp * TPW + tt) * 16 + ri);
            }
            __syncthreads();
        }
    }

    if constexpr (EPI == E_ARGMAX) {
        __syncthreads();
        if (tid < a.nb)
            a.keys[(int64_t)blockIdx.x * a.nb + tid] = s_best[tid];
    }
}

// ------------------------------------------------------------------------------------ host side

// The norm variants take K <= 2048 only: with the longer class x, its statistics and the weight
// loads do not fit in the 128 registers a lane has at 1024 threads.
template <int FMT, int EPI, bool NRM, int KC, bool SV>
static const void *mfma_fn_tpw(int tpw)
{
    switch (tpw) {
    case 1: return reinterpret_cast<const void *>(&k_mfma<FMT, EPI, NRM, KC, 1, SV>);
    case 2: return reinterpret_cast<const void *>(&k_mfma<FMT, EPI, NRM, KC, 2, SV>);
    case 4: return reinterpret_cast<const void *>(&k_mfma<FMT, EPI, NRM, KC, 4, SV>);
    case 8: return reinterpret_cast<const void *>(&k_mfma<FMT, EPI, NRM, KC, 8, SV>);
    case 16: return reinterpret_cast<const void *>(&k_mfma<FMT, EPI, NRM, KC, 16, SV>);
    default: return nullptr;
    }
}

template <int FMT, int EPI, bool NRM, int KC>
static const void *mfma_fn_sv(bool sv, int tpw)
{
    if constexpr (FMT != FQ4_0 && FMT != FQ8_0)   // these take whole steps only (sv)
        return sv ? mfma_fn_tpw<FMT, EPI, NRM, KC, true>(tpw) : nullptr;
    else
        return sv ? mfma_fn_tpw<FMT, EPI, NRM, KC, true>(tpw)
                  : mfma_fn_tpw<FMT, EPI, NRM, KC, false>(tpw);
}

template <int FMT, int EPI, bool NRM>
static const void *mfma_fn_ns(int kc, bool sv, int tpw)
{
    if (kc == 1)
        return mfma_fn_sv<FMT, EPI, NRM, 1>(sv, tpw);
    if constexpr (!NRM) {
        if (kc == 2)
            return mfma_fn_sv<FMT, EPI, NRM, 2>(sv, tpw);
    }
    return nullptr;
}

template <int FMT>
static const void *mfma_fn_fmt(int epi, bool nrm, int kc, bool sv, int tpw)
{
    switch (epi) {
    case E_STORE:
        return nrm ? mfma_fn_ns<FMT, E_STORE, true>(kc, sv, tpw)
                   : mfma_fn_ns<FMT, E_STORE, false>(kc, sv, tpw);
    case E_RES:
        return nrm ? mfma_fn_ns<FMT, E_RES, true>(kc, sv, tpw)
                   : mfma_fn_ns<FMT, E_RES, false>(kc, sv, tpw);
    case E_GUS: return mfma_fn_ns<FMT, E_GUS, true>(kc, sv, tpw);
    case E_ARGMAX: return mfma_fn_ns<FMT, E_ARGMAX, false>(kc, sv, tpw);
    default: return nullptr;
    }
}

static const void *mfma_fn(int fmt, int epi, bool nrm, int kc, bool sv, int tpw)
{
    switch (fmt) {
    case FQ4_0: return mfma_fn_fmt<FQ4_0>(epi, nrm, kc, sv, tpw);
    case FQ8_0: return mfma_fn_fmt<FQ8_0>(epi, nrm, kc, sv, tpw);
    case FQ4_K: return mfma_fn_fmt<FQ4_K>(epi, nrm, kc, sv, tpw);
    case FQ5_K: return mfma_fn_fmt<FQ5_K>(epi, nrm, kc, sv, tpw);
    case FQ5_0: return mfma_fn_fmt<FQ5_0>(epi, nrm, kc, sv, tpw);
    case FIQ4_NL: return mfma_fn_fmt<FIQ4_NL>(epi, nrm, kc, sv, tpw);
    case FIQ4_XS: return mfma_fn_fmt<FIQ4_XS>(epi, nrm, kc, sv, tpw);
    case FAQ4: return mfma_fn_fmt<FAQ4>(epi, nrm, kc, sv, tpw);
    case FQ6_K: return mfma_fn_fmt<FQ6_K>(epi, nrm, kc, sv, tpw);
    case FQ1_0: return mfma_fn_fmt<FQ1_0>(epi, nrm, kc, sv, tpw);
    default: return nullptr;
    }
}

// Plan of the row-batch kernel: K class (1: K <= 2048, 2: K <= 4096), tiles per group (16 / waves
// per tile), grid and LDS bytes; false if the kernel does not take these sizes (format, K too long
// for the staged x, LDS).
bool plan_mfma(int fmt, int epi, bool nrm, int64_t N, int64_t K, int nb, MfmaPlan *p)
{
    if (!fmt_valid(fmt))
        return false;
    if (nb < 1 || nb > 16 || K > MF_KMAX || N < 1)
        return false;
    p->kc = K <= 2048 ? 1 : 2;
    // whole steps: 128 weights (Q8_0: 64) per step
    p->sv = fmt == FQ8_0 ? K % 64 == 0 : K % 128 == 0;
    if (fmt != FQ4_0 && fmt != FQ8_0 && !p->sv)
        return false;   // the other formats take whole steps only
    const int mats = epi == E_GUS ? 2 : 1;
    p->lds = (size_t)(K / 32) * 1024 + (size_t)MF_WAVES * mats * 4 * 64 * 4;
    // one workgroup per CU; enough tiles per group that the groups fill the CUs once, at most
    // one wave per tile
    int dev = 0, cus = 0, max_lds = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess)
        return false;
    const int64_t NT = (N + 15) / 16;
    int tpw = 1;
    while (tpw < 16 && NT >= (int64_t)cus * tpw * 2)
        tpw *= 2;
    p->tpw = tpw;
    const int64_t groups = (NT + tpw - 1) / tpw;
    p->grid = (int)(groups < cus ? groups : cus);
    const void *fn = mfma_fn(fmt, epi, nrm, p->kc, p->sv, p->tpw);
    hipFuncAttributes attr;
    if (!fn || hipFuncGetAttributes(&attr, fn) != hipSuccess)
        return false;
    return attr.sharedSizeBytes + p->lds <= (size_t)max_lds;
}

int launch_mfma(int fmt, int epi, bool nrm, const MfmaPlan &p, const GemvArgs &a, void *stream)
{
    const void *fn = mfma_fn(fmt, epi, nrm, p.kc, p.sv, p.tpw);
    if (!fn)
        return (int)hipErrorInvalidValue;
    void *args[] = {const_cast<GemvArgs *>(&a)};
    return (int)hipLaunchKernel(fn, dim3(p.grid), dim3(MF_THREADS), args, p.lds,
                                static_cast<hipStream_t>(stream));
}

}  // namespace qg

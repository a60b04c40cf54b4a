// gemm_kernels.hip -- wide row-batch dequant GEMM (prefill chunks of many rows) on the gfx950
// matrix cores: Y[M][N] = X[M][K] W[N][K]^T with W block-quantized (Q4_0, Q8_0).
//
// "Module gpu" (cherenkov qwen4_exp docs), module prefill: a prompt chunk of up to a few thousand
// tokens goes through a layer at once so that each weight is streamed once for the whole chunk;
// "Crate inferencelayer" docs, gemm_q1_src / gemm_q4_src: a classic blocked GEMM whose tiles share
// one weight stream, one Q4 block (32 k) per inner step, the activation tile staged in shared
// memory.  Here:
//  - x is first turned into f16 once per call (k_xprep): each row scaled by the power of two that
//    puts its largest |x| in [2^14, 2^15), laid out per 32-k block in the order the A operand of
//    v_mfma_f32_16x16x32_f16 takes it (mf_elem), the high-nibble positions of Q4_0 times 1/16;
//  - a workgroup (4 waves, 2 x 2) owns a 128 x 128 tile of Y; a wave owns 64 x 64 (4 x 4 MFMA
//    tiles).  Per step of 128 k (Q4_0: 4 blocks; Q8_0: 64 k, 2 blocks) the wave loads its 64
//    weight rows' 16-byte chunks (one load per lane per 16 rows), transposes them across the
//    lane rows (mf_xpose) and decodes exact f16 weights (mf_bop).  Q4_0: the block scale splits
//    exactly into d_hi (8 significant bits) + d_lo, so d_hi (q - 8) and d_lo (q - 8) are exact
//    f16 operands and two MFMAs per block accumulate the scaled product straight into the MFMA
//    accumulators; Q8_0 (8-bit q): one MFMA per block gives D = A B and acc += d D on the VALU.
//    Either way the weights stay exact; only x is rounded, by at most 2^-11 of itself;
//  - x tiles come from LDS, double-buffered: the next step's x and weights are loaded while the
//    current step computes;
//  - the grid walks the tiles XCD by XCD (workgroup i runs on XCD i % 8): each XCD owns a range of
//    weight tiles and walks them row-tile-major, so the workgroups resident on an XCD share a few x
//    row tiles and the XCD's weight tiles in its L2.
#include <hip/hip_runtime.h>

#include "mfma_common.h"

namespace qg {

constexpr int GM_THREADS = 256;
constexpr int GM_WT = 2;                          // 16-row weight tiles per wave
constexpr int GM_BM = 128, GM_BN = 32 * GM_WT;    // rows of x, rows of W per workgroup
static_assert(GM_BM == QG_GEMM_BM && GM_BN == QG_GEMM_BN, "the host plans with these tiles");

// x [M][K] f32 -> xh [Mp][K] f16 in the A-operand order of each 32-k block, and rs[r] = the factor
// undoing row r's scale; rows M..Mp-1 are zero (rs 0).  One workgroup per row.
template <int FMT>
__global__ __launch_bounds__(256) void k_xprep(const float *x, int64_t M, int64_t K,
                                               _Float16 *xh, float *rs)
{
    __shared__ float s_mx[4];
    const int64_t r = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const float *xr = x + (r < M ? r : 0) * K;
    float mx = 0.f;
    if (r < M)
        for (int64_t e = t; e < K; e += 256)
            mx = fmaxf(mx, fabsf(xr[e]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        mx = fmaxf(mx, __shfl_xor(mx, off));
    if (lane == 0)
        s_mx[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(s_mx[0], s_mx[1]), fmaxf(s_mx[2], s_mx[3]));
    int e2 = 0;
    frexpf(mx, &e2);                                   // max |x| = f 2^e2, f in [0.5, 1)
    const int sk = 15 - e2 < 127 ? 15 - e2 : 127;      // 2^sk stays a finite f32
    const float sc = r < M ? ldexpf(1.0f, sk) : 0.f;
    if (t == 0)
        rs[r] = r < M ? ldexpf(1.0f, -sk) : 0.f;
    _Float16 *dst = xh + r * K;
    for (int64_t i = t; i < K; i += 256) {
        const int64_t blk = i >> 5;
        const int pos = (int)(i & 31), j = pos >> 3, h = pos & 7;
        bool hi = false;
        const int e = mf_elem<FMT>(j, h, hi);
        const float v = r < M ? xr[blk * 32 + e] * sc * (hi ? 0.0625f : 1.0f) : 0.f;
        dst[i] = (_Float16)v;
    }
}

template <int FMT>
__global__ __launch_bounds__(GM_THREADS, 2) void k_gemm(GemmArgs a)
{
    constexpr int BPS = FMT == FQ8_0 ? 2 : 4;          // blocks per step (4 chunks of 16 B)
    constexpr int KSTEP = 32 * BPS;                     // k per step
    constexpr int LROW = KSTEP + 8;                     // LDS row stride in halves (+16 B pad)
    constexpr int XSEG = GM_BM * KSTEP / 8;             // 16-byte x segments per step
    constexpr int XPT = XSEG / GM_THREADS;              // per thread
    __shared__ __attribute__((aligned(16))) _Float16 xs[2][GM_BM * LROW];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int ir = lane & 15, lc = lane >> 4;

    // tile of this workgroup (workgroup id i runs on XCD i % 8): XCD x owns weight tiles
    // [x NTX, (x + 1) NTX) and walks them row-tile-major, so the workgroups resident on an XCD at
    // a time share a few x row tiles and all of the XCD's weight tiles, both held in its L2
    // (x tile-major would sweep all of x through the L2 for every few weight tiles)
    const int NTX = (a.n_tiles + 7) / 8;
    const int id = blockIdx.x, xcd = id & 7, k8 = id >> 3;
    const int n_base = xcd * NTX;
    const int ntx = a.n_tiles - n_base < NTX ? a.n_tiles - n_base : NTX;
    if (ntx <= 0 || k8 >= ntx * a.m_tiles)
        return;
    const int m_tile = k8 / ntx, n_tile = n_base + k8 % ntx;
    const int64_t m0 = (int64_t)m_tile * GM_BM, n0 = (int64_t)n_tile * GM_BN;

    const int C = (int)(a.qs_row / 16), S = (C + 3) / 4, KB = (int)(a.K / 32);
    const uint32_t qbytes = (uint32_t)(a.N * a.qs_row), sbytes = (uint32_t)(a.N * a.sc_row);
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.qs), (short)0, (int)qbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.sc), (short)0, (int)sbytes, 0x00020000);

    // the four weight rows (one per 16-row tile) this lane loads; rows past N read row N - 1
    uint32_t wrow[GM_WT];
#pragma unroll
    for (int wt = 0; wt < GM_WT; ++wt) {
        const int64_t n = n0 + 16 * GM_WT * wn + 16 * wt + ir;
        wrow[wt] = (uint32_t)(n < a.N ? n : a.N - 1);
    }

    struct Step {
        uint32_t q[GM_WT][4];        // [weight tile][dword]
        uint16_t d[GM_WT][BPS];      // [weight tile][block] scale bits
    };
    auto load_w = [&](Step &st, int s) {
        const int sc = s < S ? s : S - 1;
        const int ch = 4 * sc + lc < C ? 4 * sc + lc : C - 1;
#pragma unroll
        for (int wt = 0; wt < GM_WT; ++wt) {
            const auto q = __builtin_amdgcn_raw_buffer_load_b128(
                rq, (int)(wrow[wt] * (uint32_t)a.qs_row + 16u * (uint32_t)ch), 0, 0);
            st.q[wt][0] = q[0]; st.q[wt][1] = q[1]; st.q[wt][2] = q[2]; st.q[wt][3] = q[3];
#pragma unroll
            for (int b = 0; b < BPS; ++b) {
                const int blk = BPS * sc + b < KB ? BPS * sc + b : KB - 1;
                st.d[wt][b] = __builtin_amdgcn_raw_buffer_load_b16(
                    rsc, (int)(wrow[wt] * (uint32_t)a.sc_row + 2u * (uint32_t)blk), 0, 0);
            }
        }
    };
    // x of step s: segment g = tid + 256 u is row g / (KSTEP / 8), 16-byte column g % (KSTEP / 8);
    // columns past K (the last step of a K that is not a multiple of the step) are zero.  Loads
    // are unconditional (a clamped address, then a select) so the loop has no branches.
    auto load_x = [&](uint4 (&xr)[XPT], int s) {
#pragma unroll
        for (int u = 0; u < XPT; ++u) {
            const int g = tid + GM_THREADS * u;
            const int row = g / (KSTEP / 8), col = g % (KSTEP / 8);
            const int64_t k0 = (int64_t)s * KSTEP + 8 * col;
            const bool in = k0 < a.K;
            const uint4 val =
                *reinterpret_cast<const uint4 *>(a.xh + (m0 + row) * a.K + (in ? k0 : 0));
            xr[u] = in ? val : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_x = [&](const uint4 (&xr)[XPT], int buf) {
#pragma unroll
        for (int u = 0; u < XPT; ++u) {
            const int g = tid + GM_THREADS * u;
            const int row = g / (KSTEP / 8), col = g % (KSTEP / 8);
            *reinterpret_cast<uint4 *>(&xs[buf][row * LROW + 8 * col]) = xr[u];
        }
    };

    float acc[4][GM_WT][4];     // Q8_0: per-block scaled sums (VALU)
    mf4 macc[4][GM_WT];         // Q4_0: sums kept in the MFMA accumulators
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < GM_WT; ++j) {
            acc[i][j][0] = acc[i][j][1] = acc[i][j][2] = acc[i][j][3] = 0.f;
            macc[i][j] = mf4{0.f, 0.f, 0.f, 0.f};
        }

    const MfConst kc = mf_const<FMT>();
    // one step from LDS buffer `buf` and the weights in st
    auto compute = [&](Step &st, int s, int buf) {
#pragma unroll
        for (int wt = 0; wt < GM_WT; ++wt)
            mf_xpose(st.q[wt]);
#pragma unroll
        for (int b = 0; b < BPS; ++b) {
            const int blk = BPS * s + b;
            mh8 A[4];
#pragma unroll
            for (int bt = 0; bt < 4; ++bt)
                A[bt] = *reinterpret_cast<const mh8 *>(
                    &xs[buf][(64 * wm + 16 * bt + ir) * LROW + 32 * b + 8 * lc]);
            if constexpr (FMT == FQ4_0) {
                // exact scaled weights: d = d_hi + d_lo with d_hi the top 8 significant bits of
                // the f16 scale, d_lo the rest (3 bits); |q - 8| <= 8 needs at most 3 more bits,
                // so d_hi (q - 8) and d_lo (q - 8) are exact f16 values (the high-nibble halves,
                // held x16, too).  Two MFMAs per block accumulate them straight into the
                // accumulators (no per-block scaling on the VALU): first the d_hi products of
                // all 16 tiles, then the d_lo ones, so an accumulator's two updates are 16
                // independent MFMAs apart.
                mh8 Bh[GM_WT], Bl[GM_WT];
#pragma unroll
                for (int wt = 0; wt < GM_WT; ++wt) {
                    const mh8 B = mf_bop<FMT>(st.q[wt][b], 0u, kc);
                    const uint16_t db = blk < KB ? st.d[wt][b] : (uint16_t)0;
                    const _Float16 dh = __builtin_bit_cast(_Float16, (uint16_t)(db & 0xFFF8u));
                    const _Float16 dl = __builtin_bit_cast(_Float16, db) - dh;
                    Bh[wt] = B * dh;
                    Bl[wt] = B * dl;
                }
#pragma unroll
                for (int wt = 0; wt < GM_WT; ++wt)
#pragma unroll
                    for (int bt = 0; bt < 4; ++bt)
                        macc[bt][wt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[bt], Bh[wt], macc[bt][wt], 0, 0, 0);
#pragma unroll
                for (int wt = 0; wt < GM_WT; ++wt)
#pragma unroll
                    for (int bt = 0; bt < 4; ++bt)
                        macc[bt][wt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[bt], Bl[wt], macc[bt][wt], 0, 0, 0);
                continue;
            }
#pragma unroll
            for (int wt = 0; wt < GM_WT; ++wt) {
                const mh8 B = FMT == FQ8_0 ? mf_bop<FMT>(st.q[wt][2 * b], st.q[wt][2 * b + 1], kc)
                                           : mf_bop<FMT>(st.q[wt][b], 0u, kc);
                const float d = blk < KB ? (float)__builtin_bit_cast(_Float16, st.d[wt][b]) : 0.f;
                const mf4 zero = {0.f, 0.f, 0.f, 0.f};
                mf4 D[4];
#pragma unroll
                for (int bt = 0; bt < 4; ++bt)
                    D[bt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[bt], B, zero, 0, 0, 0);
#pragma unroll
                for (int bt = 0; bt < 4; ++bt) {
                    acc[bt][wt][0] = fmaf(d, D[bt][0], acc[bt][wt][0]);
                    acc[bt][wt][1] = fmaf(d, D[bt][1], acc[bt][wt][1]);
                    acc[bt][wt][2] = fmaf(d, D[bt][2], acc[bt][wt][2]);
                    acc[bt][wt][3] = fmaf(d, D[bt][3], acc[bt][wt][3]);
                }
                // one (block, weight tile) group at a time: its results are consumed before the
                // next group's MFMAs issue, so few result registers are live
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // steps in pairs, the two register sets taking turns (no copies between them); every step
    // loads the next one's weights and x (a clamped step past the end reloads the last) and
    // stores that x into the other LDS buffer after computing, then one barrier
    Step s0, s1;
    uint4 xr[XPT];
    load_w(s0, 0);
    load_x(xr, 0);
    store_x(xr, 0);
    __syncthreads();
    for (int s = 0; s < S; s += 2) {
        load_w(s1, s + 1);
        load_x(xr, s + 1 < S ? s + 1 : s);
        compute(s0, s, 0);
        store_x(xr, 1);
        __syncthreads();
        if (s + 1 >= S)
            break;
        load_w(s0, s + 2);
        load_x(xr, s + 2 < S ? s + 2 : s + 1);
        compute(s1, s + 1, 1);
        store_x(xr, 0);
        __syncthreads();
    }

    // lane (ir, lc) holds D[4 lc + v][ir]: x row 16 bt + 4 lc + v, weight row 16 wt + ir
#pragma unroll
    for (int bt = 0; bt < 4; ++bt)
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) {
            const int64_t r = m0 + 64 * wm + 16 * bt + 4 * lc + vv;
            if (r >= a.M)
                continue;
            const float f = a.rs[r];
#pragma unroll
            for (int wt = 0; wt < GM_WT; ++wt) {
                const int64_t n = n0 + 16 * GM_WT * wn + 16 * wt + ir;
                const float v = FMT == FQ4_0 ? macc[bt][wt][vv] : acc[bt][wt][vv];
                if (n < a.N)
                    a.y[r * a.N + n] = v * f;
            }
        }
}

int launch_gemm(int fmt, const GemmArgs &a0, const float *x, void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    const GemmArgs &a = a0;
    const int64_t Mp = (int64_t)a.m_tiles * GM_BM;
    if (fmt == FQ4_0)
        hipLaunchKernelGGL(k_xprep<FQ4_0>, dim3((unsigned)Mp), dim3(256), 0, s, x, a.M, a.K,
                           a.xh, a.rs);
    else
        hipLaunchKernelGGL(k_xprep<FQ8_0>, dim3((unsigned)Mp), dim3(256), 0, s, x, a.M, a.K,
                           a.xh, a.rs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return (int)e;
    const int grid = 8 * ((a.n_tiles + 7) / 8) * a.m_tiles;
    if (fmt == FQ4_0)
        hipLaunchKernelGGL(k_gemm<FQ4_0>, dim3(grid), dim3(GM_THREADS), 0, s, a);
    else
        hipLaunchKernelGGL(k_gemm<FQ8_0>, dim3(grid), dim3(GM_THREADS), 0, s, a);
    return (int)hipGetLastError();
}

}  // namespace qg

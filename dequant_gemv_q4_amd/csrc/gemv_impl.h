// gemv_impl.h -- the K-tiled dequant-GEMV kernel template of libqgemv (any batch size, any K; the
// fallback for shapes the streaming and matrix-core kernels do not take), included by
// gemv_kernels.hip and gemv_kernels_x.hip, which instantiate it per format.
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"

namespace qg {

// ------------------------------------------------------------------------------------ GEMV kernel

template <int FMT, int NB, int EPI, bool NRM>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a)
{
    constexpr int MATS = EPI == E_GUS ? 2 : 1;
    constexpr int U = rows_in_flight(NB, MATS);
    constexpr int XF4 = Fc<FMT>::XF4, CE = Fc<FMT>::CE;
    extern __shared__ float4 lds4[];
    __shared__ float s_inv[NB];
    __shared__ float s_red[NB * 4];
    __shared__ unsigned long long s_key[NB * 4];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lpr = 1 << a.lpr_log2, G = 64 >> a.lpr_log2;
    const int slot = lane >> a.lpr_log2, lir = lane & (lpr - 1);
    const int ct = a.kt / CE;
    float4 *X4 = lds4;
    float *S = reinterpret_cast<float *>(lds4 + (size_t)NB * XF4 * ct);

    const float *xrow[NB];
#pragma unroll
    for (int r = 0; r < NB; ++r)
        xrow[r] = a.x + (int64_t)r * a.K;
    if constexpr (NRM)
        row_inv_rms<NB>(xrow, a.K, a.eps, s_inv, s_red);

    MatPtr mat[MATS];
    mat[0] = MatPtr{a.qs0, a.sc0, a.hb0, a.dd0, make_uint4(0u, 0u, 0u, 0u)};
    if constexpr (MATS == 2)
        mat[MATS - 1] = MatPtr{a.qs1, a.sc1, a.hb1, a.dd1, make_uint4(0u, 0u, 0u, 0u)};
    if constexpr (fmt_codebook(FMT)) {
        mat[0].cbt = *reinterpret_cast<const uint4 *>(a.cb0);
        if constexpr (MATS == 2)
            mat[MATS - 1].cbt = *reinterpret_cast<const uint4 *>(a.cb1);
    }
    const RowBytes rb{a.qs_row, a.sc_row, a.hb_row, a.d_row};

    unsigned long long best[NB];
#pragma unroll
    for (int r = 0; r < NB; ++r)
        best[r] = 0ull;

    for (int64_t st = blockIdx.x; st < a.n_steps; st += gridDim.x) {
        const int64_t row0 = st * a.rows_per_step + (int64_t)wave * U * G;
        float acc[MATS][U][NB];
#pragma unroll
        for (int m = 0; m < MATS; ++m)
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int r = 0; r < NB; ++r)
                    acc[m][u][r] = 0.f;
        for (int t = 0; t < a.n_kt; ++t) {
            if (a.n_kt > 1 || st == (int64_t)blockIdx.x) {
                __syncthreads();
                stage_tile<FMT, NB, NRM>(xrow, a.gamma, s_inv, t, a.kt, X4, S);
            }
            tile_compute<FMT, NB, U, MATS>(mat, rb, row0, a.N, G, slot, lir, lpr,
                                           t, ct, X4, S, acc);
        }
#pragma unroll
        for (int m = 0; m < MATS; ++m)
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int r = 0; r < NB; ++r)
                    acc[m][u][r] = group_sum(acc[m][u][r], lpr);
        if (lir == 0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t n = row0 + (int64_t)u * G + slot;
                if (n >= a.N)
                    continue;
#pragma unroll
                for (int r = 0; r < NB; ++r) {
                    const int64_t o = (int64_t)r * a.N + n;
                    if constexpr (EPI == E_STORE) {
                        a.y[o] = acc[0][u][r];
                    } else if constexpr (EPI == E_RES) {
                        a.y[o] = acc[0][u][r] + a.res[(int64_t)r * a.res_rstride + n];
                    } else if constexpr (EPI == E_GUS) {
                        a.y[o] = gated(acc[0][u][r], acc[MATS - 1][u][r], a.act);
                    } else {
                        const float v = acc[0][u][r];
                        a.y[o] = v;
                        const unsigned long long k = argmax_key(v, n);
                        best[r] = k > best[r] ? k : best[r];
                    }
                }
            }
        }
    }

    if constexpr (EPI == E_ARGMAX) {
        // workgroup max per row as this workgroup's partial key
#pragma unroll
        for (int r = 0; r < NB; ++r) {
            unsigned long long k = best[r];
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
            a.keys[(int64_t)blockIdx.x * NB + r] = k;   // folded by k_argmax_fold
        }
    }
}

template <int FMT, int EPI, bool NRM>
inline int launch_gemv_nb(const GemvArgs &a, int grid, size_t lds, hipStream_t s)
{
#define QG_NB_CASE(NBV)                                                                     \
    case NBV:                                                                               \
        hipLaunchKernelGGL((k_gemv<FMT, NBV, EPI, NRM>), dim3(grid), dim3(256), lds, s, a); \
        break;
    switch (a.nb) {
        QG_NB_CASE(1) QG_NB_CASE(2) QG_NB_CASE(3) QG_NB_CASE(4)
        QG_NB_CASE(5) QG_NB_CASE(6) QG_NB_CASE(7) QG_NB_CASE(8)
        QG_NB_CASE(9) QG_NB_CASE(10) QG_NB_CASE(11) QG_NB_CASE(12)
        QG_NB_CASE(13) QG_NB_CASE(14) QG_NB_CASE(15) QG_NB_CASE(16)
    default:
        return (int)hipErrorInvalidValue;
    }
#undef QG_NB_CASE
    return (int)hipGetLastError();
}

template <int FMT>
inline int launch_gemv_fmt(int epi, bool nrm, const GemvArgs &a, int grid, size_t lds,
                           hipStream_t s)
{
    switch (epi) {
    case E_STORE:
        return nrm ? launch_gemv_nb<FMT, E_STORE, true>(a, grid, lds, s)
                   : launch_gemv_nb<FMT, E_STORE, false>(a, grid, lds, s);
    case E_RES:
        return nrm ? launch_gemv_nb<FMT, E_RES, true>(a, grid, lds, s)
                   : launch_gemv_nb<FMT, E_RES, false>(a, grid, lds, s);
    case E_GUS:
        return launch_gemv_nb<FMT, E_GUS, true>(a, grid, lds, s);
    case E_ARGMAX:
        return launch_gemv_nb<FMT, E_ARGMAX, false>(a, grid, lds, s);
    default:
        return (int)hipErrorInvalidValue;
    }
}

}  // namespace qg

// gemv_kernels.hip -- gfx950 kernels of libqgemv: pack, vector dequant-GEMV family, routed experts.
//
// Vector path (one wave64 owns U rows per step; LPR lanes split one row's 16-byte chunks):
//   * x (or rmsnorm(x)) is staged once per workgroup in LDS as float4s laid out
//     [row][float4-in-chunk][chunk], so lane i of a wave reads float4 i: conflict-free ds_read_b128.
//   * each lane issues one aligned 16-byte global load per chunk and row (32 Q4 weights or 16 Q8
//     weights), decodes in registers to the exact signed weights (q - 8, the signed byte, or the
//     Q4_K nibble) and FMAs in f32.
//   * Q4_K's -dmin*m term multiplies a per-chunk sum S of x, summed in the order the dot uses.
//   * a lane-group butterfly reduces the LPR partials; every lane holds the bitwise same total.
//
// Formats and formulas ("Crate inferencelayer" docs): Q4_0 w = (q - 8) d (q4_0_to_q8_0n);
// Q8_0 w = d q (gemv_q8_0n_k_lcpp_src); Q4_K w = d sc q - dmin m (gemv_q5k_k_lcpp_src, minus the
// fifth bit).  Fused steps ("honeycrisp mod.rs"): RMSNorm prologue (Op::RmsNorm { eps }),
// silu(gate) * up (fused_norm_swiglu_down), matmul + residual (forward_decode_fused_layers).
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
    mat[0] = MatPtr{a.qs0, a.sc0};
    if constexpr (MATS == 2)
        mat[MATS - 1] = MatPtr{a.qs1, a.sc1};

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
            tile_compute<FMT, NB, U, MATS>(mat, a.qs_row, a.sc_row, row0, a.N, G, slot, lir, lpr,
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

// ------------------------------------------------------------------------------------ pack

// GGUF-native blocks (row-major, K/bw blocks per row) -> planes.  Block number blk (= row * nblk +
// block) moves its quant bytes to qs + blk * QB and its scale bytes to sc + blk * SB: for Q4_0
// (QB, SB) = (16, 2), Q8_0 (32, 2), Q4_K (128, 16) -- the Q4_K scale bytes are d, dmin and the 12
// packed (scale, min) bytes, unchanged.
template <int FMT>
__global__ __launch_bounds__(256) void k_pack(const uint8_t *src, int64_t nblocks, uint8_t *qs,
                                              uint8_t *sc)
{
    constexpr int BB = FMT == FQ4_0 ? 18 : FMT == FQ8_0 ? 34 : 144;
    constexpr int SB = FMT == FQ4_K ? 16 : 2;
    constexpr int QB = BB - SB;
    for (int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; blk < nblocks;
         blk += (int64_t)gridDim.x * blockDim.x) {
        const uint8_t *b = src + blk * BB;
        uint8_t *dq = qs + blk * QB;
        uint8_t *ds = sc + blk * SB;
        for (int k = 0; k < SB; ++k)
            ds[k] = b[k];
        for (int k = 0; k < QB; ++k)
            dq[k] = b[SB + k];
    }
}

// ------------------------------------------------------------------------------------ QK norm + RoPE

// Attention-side epilogue of a fused QKV GEMV ("honeycrisp mod.rs", pipe_qk_norm_rope: one group
// per head, the Q heads then the K heads, with q_norm / k_norm weights, rope_half and eps; the
// cos / sin tables hold one row of rope_half values per position).  In place on y[r] =
// [Q heads | K heads | V heads] of head_dim values each: every Q and K head is RMS-normalized
// over its head_dim values and scaled by its gamma (skipped when that gamma is NULL), then the
// first 2 rope_half values are rotated in pairs (j, j + rope_half) by the angle whose cosine and
// sine are cos[r][j], sin[r][j]; V heads are left as they are.  One wave per (row, head); a
// lane holds elements lane + 64 i; the pair partner comes through the wave's own LDS row.
__global__ __launch_bounds__(256) void k_qk_norm_rope(float *y, int64_t row_stride, int nb,
                                                      int nq, int nkv, int hd, int rh,
                                                      const float *qg, const float *kg, float eps,
                                                      const float *cs, const float *sn)
{
    __shared__ float buf[4][QG_HEAD_DIM_MAX];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int heads = nq + nkv;
    const int64_t item = (int64_t)blockIdx.x * 4 + wave;
    if (item >= (int64_t)nb * heads)
        return;                                    // no workgroup barrier below: waves may leave
    const int r = (int)(item / heads), h = (int)(item % heads);
    float *yh = y + (int64_t)r * row_stride + (int64_t)h * hd;
    const float *gam = h < nq ? qg : kg;
    constexpr int NI = QG_HEAD_DIM_MAX / 64;
    float v[NI];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < hd ? yh[e] : 0.f;
        ss = fmaf(v[i], v[i], ss);
    }
    if (gam) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            ss += __shfl_xor(ss, off);
        const float inv = 1.0f / sqrtf(ss / (float)hd + eps);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int e = lane + 64 * i;
            if (e < hd)
                v[i] = v[i] * inv * gam[e];
        }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int e = lane + 64 * i;
        if (e < hd)
            buf[wave][e] = v[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const float *cr = cs + (int64_t)r * rh, *sr = sn + (int64_t)r * rh;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int e = lane + 64 * i;
        if (e < hd) {
            float out = v[i];
            if (e < rh) {
                out = v[i] * cr[e] - buf[wave][e + rh] * sr[e];
            } else if (e < 2 * rh) {
                const int j = e - rh;
                out = v[i] * cr[j] + buf[wave][j] * sr[j];
            }
            yh[e] = out;
        }
    }
}

// ------------------------------------------------------------------------------------ launchers

int launch_qk_norm_rope(float *y, int64_t row_stride, int nb, int nq, int nkv, int hd, int rh,
                        const float *qg, const float *kg, float eps, const float *cs,
                        const float *sn, void *stream)
{
    const int64_t items = (int64_t)nb * (nq + nkv);
    hipLaunchKernelGGL(k_qk_norm_rope, dim3((unsigned)((items + 3) / 4)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), y, row_stride, nb, nq, nkv, hd, rh, qg,
                       kg, eps, cs, sn);
    return (int)hipGetLastError();
}

int launch_pack(int fmt, const void *src, int64_t N, int64_t K, void *dst, void *stream)
{
    Layout L;
    if (!layout(fmt, N, K, &L))
        return (int)hipErrorInvalidValue;
    const int64_t nblocks = N * (K / L.block_w);
    uint8_t *qs = static_cast<uint8_t *>(dst);
    uint8_t *sc = qs + L.sc_off;
    const int64_t want = (nblocks + 255) / 256;
    const int grid = (int)(want < 65536 ? want : 65536);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint8_t *in = static_cast<const uint8_t *>(src);
    if (fmt == FQ4_0)
        hipLaunchKernelGGL(k_pack<FQ4_0>, dim3(grid), dim3(256), 0, s, in, nblocks, qs, sc);
    else if (fmt == FQ8_0)
        hipLaunchKernelGGL(k_pack<FQ8_0>, dim3(grid), dim3(256), 0, s, in, nblocks, qs, sc);
    else
        hipLaunchKernelGGL(k_pack<FQ4_K>, dim3(grid), dim3(256), 0, s, in, nblocks, qs, sc);
    return (int)hipGetLastError();
}

template <int FMT, int EPI, bool NRM>
static int launch_gemv_nb(const GemvArgs &a, int grid, size_t lds, hipStream_t s)
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
static int launch_gemv_fmt(int epi, bool nrm, const GemvArgs &a, int grid, size_t lds,
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

int launch_gemv(int fmt, int epi, bool nrm, const GemvArgs &a, int grid, size_t lds_bytes,
                void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (fmt == FQ4_0)
        return launch_gemv_fmt<FQ4_0>(epi, nrm, a, grid, lds_bytes, s);
    if (fmt == FQ8_0)
        return launch_gemv_fmt<FQ8_0>(epi, nrm, a, grid, lds_bytes, s);
    if (fmt == FQ4_K)
        return launch_gemv_fmt<FQ4_K>(epi, nrm, a, grid, lds_bytes, s);
    return (int)hipErrorInvalidValue;
}

}  // namespace qg

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

#include "gemv_impl.h"

namespace qg {

// ------------------------------------------------------------------------------------ pack

// GGUF-native blocks (row-major, K/bw blocks per row) -> planes.  Block number blk (= row * nblk +
// block) moves its quant bytes to qs + blk * QB and its scale bytes to sc + blk * SB: Q4_0,
// Q5_0, IQ4_NL and Q1_0 (16, 2), Q8_0 (32, 2), the affine Q4 (16, 4: scale and bias), IQ4_XS
// (128, 8: d and the packed sub-scales), Q4_K and Q5_K (128, 16: d, dmin and the 12 packed
// (scale, min) bytes, unchanged), Q6_K (128, 16: the 16 signed scales; its d goes to
// dd + blk * 2).  The IQ4 formats' 16-byte codebook (cb) is written once, after every plane.  The high
// bits of Q5_0 / Q5_K / Q6_K go to hb + blk * HB, re-laid per 32 weights (q5_bits, q6_bits) so
// that the kernels insert them into the nibble bytes with one shift and one and-or per dword.
//
// Fifth bits of one 16-byte nibble chunk, 4 bytes: the bit of the low nibble of chunk byte
// 4k + m at bit 8m + k, the bit of its high nibble at bit 8m + 4 + k (k, m < 4).
__device__ __forceinline__ uint32_t q5_bits(const uint8_t (&lo)[16], const uint8_t (&hi)[16])
{
    uint32_t w = 0;
    for (int k = 0; k < 4; ++k)
        for (int m = 0; m < 4; ++m) {
            w |= (uint32_t)(lo[4 * k + m] & 1) << (8 * m + k);
            w |= (uint32_t)(hi[4 * k + m] & 1) << (8 * m + 4 + k);
        }
    return w;
}

// Q6_K: the two high bits of the low (high) nibble of chunk byte 4k + m at bits 8m + 2k, +1 of
// the first (second) word.
__device__ __forceinline__ uint32_t q6_bits(const uint8_t (&two)[16])
{
    uint32_t w = 0;
    for (int k = 0; k < 4; ++k)
        for (int m = 0; m < 4; ++m)
            w |= (uint32_t)(two[4 * k + m] & 3) << (8 * m + 2 * k);
    return w;
}

template <int FMT>
__global__ __launch_bounds__(256) void k_pack(const uint8_t *src, int64_t nblocks, uint8_t *qs,
                                              uint8_t *sc, uint8_t *hb, uint8_t *dd, uint4 cbv,
                                              uint8_t *cb)
{
    constexpr int BB = FMT == FQ4_0 ? 18 : FMT == FQ5_0 ? 22 : FMT == FQ8_0 ? 34
                     : FMT == FQ4_K ? 144 : FMT == FQ5_K ? 176 : FMT == FQ6_K ? 210
                     : FMT == FIQ4_NL ? 18 : FMT == FIQ4_XS ? 136 : FMT == FQ1_0 ? 18 : 20;
    if (fmt_codebook(FMT) && blockIdx.x == 0 && threadIdx.x == 0)
        *reinterpret_cast<uint4 *>(cb) = cbv;
    for (int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; blk < nblocks;
         blk += (int64_t)gridDim.x * blockDim.x) {
        const uint8_t *b = src + blk * BB;
        if constexpr (FMT == FQ4_0 || FMT == FQ8_0 || FMT == FQ4_K || fmt_generic(FMT)) {
            constexpr int SB = FMT == FQ4_K ? 16 : FMT == FIQ4_XS ? 8 : FMT == FAQ4 ? 4 : 2;
            constexpr int QB = BB - SB;
            for (int k = 0; k < SB; ++k)
                sc[blk * SB + k] = b[k];
            for (int k = 0; k < QB; ++k)
                qs[blk * QB + k] = b[SB + k];
        } else if constexpr (FMT == FQ5_0) {
            // d (2), qh (4, little-endian: bit j for element j), nibbles (16)
            sc[blk * 2] = b[0];
            sc[blk * 2 + 1] = b[1];
            const uint32_t qh = (uint32_t)b[2] | ((uint32_t)b[3] << 8) | ((uint32_t)b[4] << 16) |
                                ((uint32_t)b[5] << 24);
            uint8_t lo[16], hi[16];
            for (int i = 0; i < 16; ++i) {
                qs[blk * 16 + i] = b[6 + i];
                lo[i] = (uint8_t)((qh >> i) & 1u);          // element i: low nibble of byte i
                hi[i] = (uint8_t)((qh >> (16 + i)) & 1u);   // element 16 + i: its high nibble
            }
            const uint32_t w = q5_bits(lo, hi);
            for (int k = 0; k < 4; ++k)
                hb[blk * 4 + k] = (uint8_t)(w >> (8 * k));
        } else if constexpr (FMT == FQ5_K) {
            // d, dmin, 12 scale bytes (16), qh (32), nibbles (128); chunk q = bytes 16q..16q+15 of
            // the nibbles: byte 32c + 16h + i (c = q / 2, h = q % 2) takes bits 2c (low nibble)
            // and 2c + 1 (high nibble) of qh[16h + i]
            for (int k = 0; k < 16; ++k)
                sc[blk * 16 + k] = b[k];
            for (int k = 0; k < 128; ++k)
                qs[blk * 128 + k] = b[48 + k];
            for (int q = 0; q < 8; ++q) {
                const int c = q >> 1, h = q & 1;
                uint8_t lo[16], hi[16];
                for (int i = 0; i < 16; ++i) {
                    lo[i] = (uint8_t)((b[16 + 16 * h + i] >> (2 * c)) & 1);
                    hi[i] = (uint8_t)((b[16 + 16 * h + i] >> (2 * c + 1)) & 1);
                }
                const uint32_t w = q5_bits(lo, hi);
                for (int k = 0; k < 4; ++k)
                    hb[blk * 32 + 4 * q + k] = (uint8_t)(w >> (8 * k));
            }
        } else {
            // Q6_K: ql (128), qh (64), 16 signed scales, d.  Chunk t = ql bytes 16t..16t+15
            // (n = t / 4, u = t % 4); its byte i pairs with qh[32n + 16 (u % 2) + i], whose bits
            // 0-1 / 4-5 (u < 2) or 2-3 / 6-7 (u >= 2) are the low / high nibble's high bits
            for (int k = 0; k < 128; ++k)
                qs[blk * 128 + k] = b[k];
            for (int k = 0; k < 16; ++k)
                sc[blk * 16 + k] = b[192 + k];
            dd[blk * 2] = b[208];
            dd[blk * 2 + 1] = b[209];
            for (int t = 0; t < 8; ++t) {
                const int n = t >> 2, u = t & 3, sh = u >= 2 ? 2 : 0;
                uint8_t lo[16], hi[16];
                for (int i = 0; i < 16; ++i) {
                    const uint8_t h = b[128 + 32 * n + 16 * (u & 1) + i];
                    lo[i] = (uint8_t)((h >> sh) & 3);
                    hi[i] = (uint8_t)((h >> (sh + 4)) & 3);
                }
                const uint32_t wa = q6_bits(lo), wb = q6_bits(hi);
                for (int k = 0; k < 4; ++k) {
                    hb[blk * 64 + 8 * t + k] = (uint8_t)(wa >> (8 * k));
                    hb[blk * 64 + 8 * t + 4 + k] = (uint8_t)(wb >> (8 * k));
                }
            }
        }
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

int launch_pack(int fmt, const void *src, int64_t N, int64_t K, const int8_t *codebook, void *dst,
                void *stream)
{
    Layout L;
    if (!layout(fmt, N, K, &L))
        return (int)hipErrorInvalidValue;
    const int64_t nblocks = N * (K / L.block_w);
    uint8_t *qs = static_cast<uint8_t *>(dst);
    uint8_t *sc = qs + L.sc_off, *hb = qs + L.hb_off, *dd = qs + L.d_off, *cb = qs + L.cb_off;
    // the codebook travels by value (a kernel argument): the host table is read before return
    uint32_t cw[4] = {0u, 0u, 0u, 0u};
    if (fmt_codebook(fmt))
        for (int e = 0; e < 16; ++e)
            cw[e / 4] |= (uint32_t)(uint8_t)codebook[e] << (8 * (e % 4));
    const uint4 cbv = make_uint4(cw[0], cw[1], cw[2], cw[3]);
    const int64_t want = (nblocks + 255) / 256;
    const int grid = (int)(want < 65536 ? want : 65536);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint8_t *in = static_cast<const uint8_t *>(src);
#define QG_PACK(F)                                                                                \
    hipLaunchKernelGGL(k_pack<F>, dim3(grid), dim3(256), 0, s, in, nblocks, qs, sc, hb, dd, cbv, cb)
    switch (fmt) {
    case FQ4_0: QG_PACK(FQ4_0); break;
    case FQ5_0: QG_PACK(FQ5_0); break;
    case FQ8_0: QG_PACK(FQ8_0); break;
    case FQ4_K: QG_PACK(FQ4_K); break;
    case FQ5_K: QG_PACK(FQ5_K); break;
    case FQ6_K: QG_PACK(FQ6_K); break;
    case FIQ4_NL: QG_PACK(FIQ4_NL); break;
    case FIQ4_XS: QG_PACK(FIQ4_XS); break;
    case FQ1_0: QG_PACK(FQ1_0); break;
    default: QG_PACK(FAQ4); break;
    }
#undef QG_PACK
    return (int)hipGetLastError();
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

// qgemv_internal.h -- library-internal declarations shared by the ABI layer and the kernels.
// Not installed; the public interface is include/qgemv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qg {

enum Fmt { FQ4_0 = 2, FQ5_0 = 6, FQ8_0 = 8, FQ4_K = 12, FQ5_K = 13, FQ6_K = 14, FIQ4_NL = 20,
           FIQ4_XS = 23, FQ1_0 = 40, FAQ4 = 41 };

// Formats the K-tiled kernel serves with a per-element decode (codebook, sign and affine
// formats): fewer bytes per weight, where the byte ratio is the speed ratio.
__host__ __device__ constexpr bool fmt_generic(int f)
{
    return f == FIQ4_NL || f == FIQ4_XS || f == FQ1_0 || f == FAQ4;
}
// Formats whose weights come from a 16-entry codebook stored with the packed matrix.
__host__ __device__ constexpr bool fmt_codebook(int f) { return f == FIQ4_NL || f == FIQ4_XS; }
// Quant bytes of the chunk (32 weights; Q8_0 16) one lane takes: Q1_0's 32 sign bits are 4 bytes.
__host__ __device__ constexpr int fmt_chunk_bytes(int f) { return f == FQ1_0 ? 4 : 16; }

// Format classes.  Super-block formats hold 256 weights per block; high-bit formats carry a plane
// of fifth (Q5) or fifth-and-sixth (Q6_K) bits beside the nibbles; min formats have the
// d sc q - dmin m form; the Q4 formats hold their high-nibble weights x16 in the f16 pairs.
__host__ __device__ constexpr bool fmt_super(int f) { return f == FQ4_K || f == FQ5_K || f == FQ6_K; }
__host__ __device__ constexpr bool fmt_hbits(int f) { return f == FQ5_0 || f == FQ5_K || f == FQ6_K; }
__host__ __device__ constexpr bool fmt_min(int f) { return f == FQ4_K || f == FQ5_K; }
__host__ __device__ constexpr bool fmt_q4(int f) { return f == FQ4_0 || f == FQ4_K || f == FAQ4; }
// 32-bit words of high bits per 16-byte chunk of nibbles (32 weights).
__host__ __device__ constexpr int fmt_hwords(int f) { return f == FQ6_K ? 2 : fmt_hbits(f) ? 1 : 0; }
// Formats whose chunk carries two sub-block scales (a low-nibble and a high-nibble sub-block).
__host__ __device__ constexpr bool fmt_two_sub(int f) { return fmt_super(f); }

// Epilogue kinds of the GEMV kernels: store; add a residual row or a bias (E_RES); gated product
// act(g) u of two matrices (E_GUS); store and argmax keys (E_ARGMAX).
enum Epi { E_STORE = 0, E_RES = 1, E_GUS = 2, E_ARGMAX = 3 };
// Activations of the gated product.
enum Act { A_SILU = 0, A_GELU_TANH = 1 };

// Argmax: partial keys are kept per workgroup (and batch row), so its launches have at most this
// many workgroups.
#define QG_ARGMAX_MAX_GRID 4096

// Routed experts: at most this many (row, slot) pairs per call (16 rows x top-8).
#define QG_PAIRS_MAX 128
// Routed experts: threads per workgroup of the common variants, and of the variants that hold
// more in registers.  The Q4_K variant with one chunk slot per lane needs about 160 VGPRs (four x
// rows held as f16 pairs), so three waves fit on a SIMD: 12 waves per workgroup, one workgroup
// per CU.  Q4_K with four chunk slots per lane (rows of 8192) and the variants with four groups
// in flight need more than 168 VGPRs and keep two waves per SIMD (8 waves per workgroup).
#ifndef QG_MOE_THREADS
#define QG_MOE_THREADS 768
#endif
#define QG_MOE_THREADS_WIDE 512
__host__ __device__ constexpr int moe_threads(int fmt, int cpl, int pd)
{
    return (fmt == FQ4_K && cpl >= 4) || pd >= 4 ? QG_MOE_THREADS_WIDE : QG_MOE_THREADS;
}
#ifndef QG_MOE_PD
#define QG_MOE_PD 2       // row groups a routed-expert wave keeps in flight (2 or 4)
#endif
// Routed experts: most experts a call may have (a 128-bit pair mask and a count per expert are
// kept in LDS; at most 4 experts per thread in the scan).
#define QG_MOE_EXPERTS_MAX 1024
// Routed experts: most LDS bytes for the results a workgroup collects.
#ifndef QG_MOE_POOL_LDS
#define QG_MOE_POOL_LDS 32768
#endif

// Packed device layout of one N x K matrix: a plane of quant bytes (row n at n * qs_row) and a
// plane of scale bytes (row n at n * sc_row), each starting 256-B aligned.  Same bytes per weight
// as the GGUF blocks.
struct Layout {
    int64_t qs_row;     // quant bytes per row: Q8_0 K, Q1_0 K/8 (sign bits), others K/2 (nibbles)
    int64_t sc_row;     // scale bytes per row: K/16, IQ4_XS K/32, Q1_0 K/64, affine Q4 K/8
    int64_t sc_off;     // byte offset of the scale plane (qs plane rounded up to 256 B)
    int64_t hb_row;     // high-bit bytes per row: Q5_0 / Q5_K K/8, Q6_K K/4, others 0
    int64_t hb_off;     // byte offset of the high-bit plane (after the scale plane)
    int64_t d_row;      // Q6_K: bytes of the super-block d values per row (K/128), others 0
    int64_t d_off;      // byte offset of that plane
    int64_t cb_off;     // IQ4 formats: byte offset of the 16-byte codebook (after every plane)
    int64_t total;      // packed bytes
    int64_t gguf_row;   // GGUF bytes per row
    int block_w;        // weights per GGUF block
    int block_b;        // bytes per GGUF block
};

// Facts of the quant chunk one lane processes (16 bytes; Q1_0 4): x float4s it multiplies (xf4),
// x elements (ce), block sums it needs (ns), and the K granularity a tile must keep (tile_align).
struct FmtFacts {
    int xf4, ce, ns, tile_align;
};

__host__ __device__ constexpr FmtFacts fmt_facts(int fmt)
{
    return fmt == FQ8_0 ? FmtFacts{4, 16, 1, 32}
         : fmt == FQ1_0 ? FmtFacts{8, 32, 1, 128}
         : fmt == FIQ4_XS ? FmtFacts{8, 32, 1, 256}
         : fmt_super(fmt) ? FmtFacts{8, 32, 2, 256}
                          : FmtFacts{8, 32, 1, 32};
}

// Rows a wave keeps in flight per step of the vector kernel, by row-batch size and matrix count.
__host__ __device__ constexpr int rows_in_flight(int nb, int mats)
{
    return nb == 1 ? (mats == 1 ? 4 : 2) : (nb <= 4 ? (mats == 1 ? 2 : 1) : 1);
}

// Rows one wave of the streaming kernels finishes per group (R), by batch rows, 16-byte chunks
// per lane and row (CPL), and matrices (2 for the gated product).
#ifndef QG_R_NB1
#define QG_R_NB1 2        // rows per group of the single-row-batch streaming kernel
#endif
#ifndef QG_WPE_NB1
#define QG_WPE_NB1 4      // waves per SIMD the single-row-batch streaming kernel is sized for
#endif
#ifndef QG_WCPOL
#define QG_WCPOL 0        // cache policy bits of the matrix-core kernel's weight loads
#endif
#ifndef QG_WCPOL_STREAM
#define QG_WCPOL_STREAM 2 // the vector kernels' weight loads: non-temporal (x and gamma stay cached)
#endif
#ifndef QG_TILE_GROUPS
#define QG_TILE_GROUPS 8  // most consecutive row groups a streaming workgroup takes at a time
#endif
#ifndef QG_PD_MAX
#define QG_PD_MAX 2       // most row groups a single-row-batch streaming wave keeps in flight
#endif
__host__ __device__ constexpr int stream_rows(int nb, int cpl, int mats)
{
    return nb == 1 ? ((mats == 1 ? QG_R_NB1 : (QG_R_NB1 + 1) / 2) / cpl > 0
                          ? (mats == 1 ? QG_R_NB1 : (QG_R_NB1 + 1) / 2) / cpl : 1)
                   : (cpl == 1 ? 2 : 1);
}
// Rows per group of the GEMV streaming kernel for a format: Q1_0's lane chunks are 4 bytes, so its
// groups take four times the rows (the same bytes per group as the 16-byte formats; the per-group
// reduction and epilogue are spread over four times the weights).
__host__ __device__ constexpr int stream_rows_fmt(int fmt, int nb, int cpl, int mats)
{
    return stream_rows(nb, cpl, mats) * (fmt == FQ1_0 ? 4 : 1);
}

// LDS bytes of one staged x tile of nb rows and kt elements (float4 region, then block sums).
__host__ __device__ constexpr size_t lds_tile_bytes(int fmt, int nb, int kt)
{
    return (size_t)nb * kt * 4 + (size_t)nb * (kt / fmt_facts(fmt).ce) * fmt_facts(fmt).ns * 4;
}

bool fmt_valid(int fmt);
bool layout(int fmt, int64_t N, int64_t K, Layout *out);

// Arguments of the vector GEMV kernel family, passed by value.
struct GemvArgs {
    const uint8_t *qs0, *sc0;   // matrix 0 (the only matrix, or the gate)
    const uint8_t *qs1, *sc1;   // matrix 1 (the up matrix of the gated product)
    const uint8_t *hb0, *hb1;   // high-bit planes of the two matrices (high-bit formats)
    const uint8_t *dd0, *dd1;   // Q6_K: planes of the super-block d values
    const int8_t *cb0, *cb1;    // IQ4 formats: the 16-entry codebooks of the two matrices
    const float *x;             // [nb][K]
    const float *gamma;         // [K] (norm prologue)
    const float *res;           // residual [nb][N] (res_rstride N) or bias [N] (res_rstride 0)
    float *y;                   // [nb][N]
    int32_t *idx;               // [nb] (argmax)
    unsigned long long *keys;   // argmax: partial key per workgroup and batch row (workspace)
    int64_t N, K;
    int64_t qs_row, sc_row, hb_row, d_row;
    float eps;
    int64_t res_rstride;        // elements between the batch rows of res (0: one row for all)
    int act;                    // gated product: 0 silu(g) u, 1 gelu_tanh(g) u
    int nb;
    int lpr_log2;               // log2 of lanes cooperating on one row
    int kt;                     // K elements per LDS tile
    int n_kt;                   // tiles per row
    int rows_per_step;          // rows one workgroup finishes per step
    int64_t n_steps;            // workgroup steps covering N rows
    int tg_log2;                // streaming kernels: log2 of the row groups per tile
};

// Arguments of the routed-expert kernels.
struct MoeArgs {
    const uint8_t *qs, *sc;     // packed expert stack: n_exp * N rows
    const float *x;             // [nb][K]
    const int32_t *ids;         // [nb][topk]
    const float *wts;           // [nb][topk]
    float *y;                   // [nb][N]
    float *part;                // workspace: [nb][topk][N] partial outputs
    unsigned int *err;          // workspace: sticky flag (bit 0: an expert id out of range)
    int64_t n_exp, N, K;
    int64_t qs_row, sc_row;
    int nb, topk;
    int pool_max;               // most row groups one workgroup's range may hold
};

// Tile of the wide row-batch GEMM: rows of x per workgroup, k per step; rows of W per workgroup
// are 128 or (Q4_0, when the tiles fill the device) 256.
#define QG_GEMM_BM 128   // rows of x per tile: 128, or 64 when M <= 64
#define QG_GEMM_KSTEP 128
// Arguments of the wide row-batch GEMM (gemm_kernels.hip).
struct GemmArgs {
    const uint8_t *qs, *sc;     // packed W (Q4_0 / Q8_0 / Q1_0)
    _Float16 *xh;               // workspace: x as f16 in operand chunks, [m_tiles * bm / 16][KBp][512]
    float *rs;                  // workspace: factor undoing each x row's scale, [m_tiles * bm]
    float *part;                // workspace: partial tiles of the K splits, [splits][M][N] (splits > 1)
    float *y;                   // [M][N]
    int64_t N, K, M;
    int64_t qs_row, sc_row;
    int n_tiles, m_tiles;       // tiles of W (bn rows) and of x (bm rows)
    int bn;                     // rows of W per tile: 128, 256 or 512 (Q4_0)
    int bm;                     // rows of x per tile: 128 or 64
    int KBp;                    // 32-k blocks of a padded x row: steps * QG_GEMM_KSTEP / 32
    int steps, sps, splits;     // K steps, steps per split, splits (ceil(steps / sps))
};
// x preparation then the GEMM, both on `stream`.
int launch_gemm(int fmt, const GemmArgs &a, const float *x, void *stream);

// Launch helpers (gemv_kernels.hip).  Return a hipError_t value (0 = success).
int launch_pack(int fmt, const void *src, int64_t N, int64_t K, const int8_t *codebook, void *dst,
                void *stream);
int launch_gemv(int fmt, int epi, bool nrm, const GemvArgs &a, int grid, size_t lds_bytes,
                void *stream);
// The same for the high-bit formats (gemv_kernels_x.hip).
int launch_gemv_x(int fmt, int epi, bool nrm, const GemvArgs &a, int grid, size_t lds_bytes,
                  void *stream);
int launch_stream(int fmt, int epi, bool nrm, int cpl, int pd, const GemvArgs &a, int grid,
                  size_t lds_bytes, void *stream);
// The streaming kernel variant (function and threads per workgroup) of a high-bit format
// (stream_kernels_x.hip); *fn = nullptr if there is none.
void stream_fn_x(int fmt, int epi, bool nrm, int ks, int nb, int pd, const void **fn,
                 int *threads);
// The same for the codebook, sign and affine formats (stream_kernels_g.hip).
void stream_fn_g(int fmt, int epi, bool nrm, int ks, int nb, int pd, const void **fn,
                 int *threads);
// Routed experts: the expert kernel (x rows per set 4 / cpl, pd groups in flight per wave), then
// the combine.
int launch_moe(int fmt, int cpl, int pd, const MoeArgs &a, int grid, size_t lds_bytes,
               void *stream);
// Row-batch kernel on the matrix cores (mfma_kernels.hip): persistent workgroups over groups of
// 16-row tiles.
struct MfmaPlan {
    int kc;       // K class: 1 (K <= 2048) or 2 (K <= 4096)
    bool sv;      // one load per lane fetches a step's block scales (aligned scale rows)
    int tpw;      // tiles per group (16 / waves per tile)
    int grid;
    size_t lds;
};
bool plan_mfma(int fmt, int epi, bool nrm, int64_t N, int64_t K, int nb, MfmaPlan *p);
int launch_mfma(int fmt, int epi, bool nrm, const MfmaPlan &p, const GemvArgs &a, void *stream);
int launch_argmax_fold(const unsigned long long *part, int n_part, int nb, int32_t *idx,
                       void *stream);
// Per-head QK RMSNorm + RoPE in place on a QKV output (gemv_kernels.hip).
#define QG_HEAD_DIM_MAX 256
int launch_qk_norm_rope(float *y, int64_t row_stride, int nb, int nq, int nkv, int hd, int rh,
                        const float *qg, const float *kg, float eps, const float *cs,
                        const float *sn, void *stream);
// Device address of this device's copy of the library's fixed scratch array (the argmax partial
// keys of the no-allocation entry point) and its size; looked up once per device.  0 = ok.
int noalloc_scratch(void **ptr, size_t *bytes);
// Workgroups of a streaming launch that are resident at once on the current device (0 if the
// query fails).
int stream_resident_wgs(int fmt, int epi, bool nrm, int cpl, int nb, int pd, size_t lds_bytes,
                        int *waves);
int moe_resident_wgs(int fmt, int cpl, int pd, size_t lds_bytes);

}  // namespace qg

/*
 * qgemv.h -- C ABI of libqgemv: block-quantized weight GEMV for LLM decode on MI355X (gfx950).
 *
 * The operations are the dequant-in-GEMV family of one decode step, for one token or a row
 * batch of nb <= 16 positions (activations row-major [nb][...], the row-batched steps of
 * "Module gpu", cherenkov qwen4_exp docs, module summary), fused with the neighbouring steps
 * "honeycrisp mod.rs" encodes around its quantized matmuls: RMSNorm prologue, gate+up with the
 * SiLU-gated product, residual add, and greedy argmax of the lm_head.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Formats (GGUF type ids where GGUF has one): QG_Q4_0 = 2, QG_Q5_0 = 6, QG_Q8_0 = 8,
 *    QG_Q4_K = 12, QG_Q5_K = 13, QG_Q6_K = 14, QG_IQ4_NL = 20, QG_IQ4_XS = 23, and two ids of
 *    this library's own, QG_Q1_0 = 40 and QG_AQ4 = 41 ("Crate inferencelayer" docs, the
 *    gemv_*_lcpp_src family; the affine Q4 of "Module gpu").
 *      Q4_0: 32 weights in 18 B (f16 d, 16 B nibbles), w = (q - 8) * d.
 *      Q5_0: 32 weights in 22 B (f16 d, 4 B of fifth bits, 16 B nibbles), w = d * (q - 16),
 *            q = nib | bit << 4 (element j: bit j).
 *      Q8_0: 32 weights in 34 B (f16 d, 32 x i8),     w = d * q.
 *      Q4_K: 256 weights in 144 B (f16 d, f16 dmin, 12 B of eight packed 6-bit (scale, min)
 *            pairs, 128 B nibbles), w = d * sc_j * q - dmin * m_j.
 *      Q5_K: 256 weights in 176 B (Q4_K's d, dmin, 12 B pack, then 32 B of fifth bits, 128 B
 *            nibbles; sub-block s takes bit s of qh[l]), w = d * sc_j * q - dmin * m_j.
 *      Q6_K: 256 weights in 210 B (128 B low nibbles, 64 B high bit pairs, 16 signed scales,
 *            f16 d), w = d * sc * (q - 32) with one scale per 16 weights.
 *      IQ4_NL: 32 weights in 18 B (f16 d, 16 B of 4-bit indices in Q4_0's nibble order),
 *            w = d * cb[q] with cb a 16-entry table of signed bytes (gemv_iq4_nl_k_lcpp_src).
 *      IQ4_XS: 256 weights in 136 B (f16 d, a 16-bit word of high scale bits (sub-block s at
 *            bits 2s, 2s+1), 4 B of low 4-bit scales (sub-block s at bits 4s..4s+3), 128 B of
 *            indices, 16 B per 32-weight sub-block), w = d * (ls - 32) * cb[q]
 *            (gemv_iq4_xs_k_lcpp_src).
 *      Q1_0: 128 weights in 18 B (f16 d, 16 B of sign bits: bit i % 8 of byte i / 8 for
 *            element i), w = +d for a set bit, -d for a clear one (gemv_q1_k_lcpp_src).
 *      AQ4:  32 weights in 20 B (f16 scale s, f16 bias c, 16 B nibbles: element 2i the low
 *            nibble of byte i, 2i + 1 its high nibble), w = s * q + c ("Module gpu", struct Q).
 *    The field orders and bit orders of IQ4_NL, IQ4_XS, Q1_0 and AQ4 are this library's reading
 *    of pages that name the formats without printing their layout.  The IQ4 formats' codebook
 *    is an input (qgemv_pack_codebook), stored inside the packed matrix.
 *    Routed experts (qgemv_moe) take Q4_0, Q8_0 and Q4_K; the row-batch GEMM (qgemm) Q4_0, Q8_0
 *    and Q1_0.
 *  - W arguments of the compute entry points are in the PACKED device layout written by
 *    qgemv_pack (same bytes per weight as GGUF, split into planes so every hot load is an
 *    aligned 16-byte load).  Rows are in output order; K is the reduction length.  A W buffer
 *    must span the whole qgemv_packed_bytes(fmt, N, K): the kernels may read into the padding
 *    after each plane (whole dwords of the scale plane), never past it.
 *  - Every pointer of a compute call is a DEVICE pointer (HIP device memory).  The caller owns
 *    all memory; the library never allocates or frees and carries no data from one call to the
 *    next (on the host it caches per-device occupancy queries and launch plans, which only shape
 *    launches).
 *  - x is f32 [nb][K], outputs f32 [nb][N], all row-major and contiguous.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every call only
 *    enqueues work on that stream and returns; nothing synchronizes the host.
 *  - `ws` is a device workspace of at least qgemv_workspace_bytes(...) bytes (may be NULL when
 *    that is 0).  It is scratch that every call writes before it reads (argmax: one partial key
 *    per workgroup; experts: partial outputs), except the sticky bad-id flag of qgemv_moe, so a
 *    qgemv_moe workspace must be zero-filled once after allocation.  Calls that share one
 *    workspace must be ordered on one stream.  The argmax and expert operations follow their
 *    main kernel with a small fold / combine kernel on `stream`.  A call of 5..16 rows that the
 *    matrix-core kernel does not take (K > 4096, or K > 2048 with the norm prologue) runs as
 *    batches of at most 4 rows, each its own launch (pair), one after the other on `stream`.
 *  - Errors: every argument is validated on the host before anything is launched; a failed
 *    check returns its status and launches nothing.  QG_ERR_LAUNCH reports a HIP error from the
 *    launch itself.  qgemv_status_str gives a static description.
 *  - No CPU fallback: a call the kernels cannot serve is an error, never a host computation.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { QG_Q4_0 = 2, QG_Q5_0 = 6, QG_Q8_0 = 8, QG_Q4_K = 12, QG_Q5_K = 13, QG_Q6_K = 14,
       QG_IQ4_NL = 20, QG_IQ4_XS = 23, QG_Q1_0 = 40, QG_AQ4 = 41 };

enum {
    QG_OK = 0,
    QG_ERR_NULL = 1,       /* a required pointer is NULL */
    QG_ERR_FORMAT = 2,     /* unknown format id, or a format the entry point does not take */
    QG_ERR_SHAPE = 3,      /* N < 1, nb outside [1, 16], K not a positive multiple of the block,
                              topk outside [1, 8], n_exp < 1, or a size beyond the limits */
    QG_ERR_ALIGN = 4,      /* W or a workspace not 256-B aligned, x or gamma not 16-B aligned, or
                              an output, residual, id or weight array not 4-B aligned */
    QG_ERR_WORKSPACE = 5,  /* ws smaller than qgemv_workspace_bytes() */
    QG_ERR_LAUNCH = 6,     /* the HIP launch reported an error */
    QG_ERR_ALIAS = 7       /* an output overlaps an input in a way the call does not allow */
};

/* Operation ids for qgemv_workspace_bytes. */
enum { QG_OP_GEMV = 0, QG_OP_NRM = 1, QG_OP_GUS_NRM = 2, QG_OP_RES = 3, QG_OP_ARGMAX = 4,
       QG_OP_MOE = 5, QG_OP_NRM_BIAS = 6 };

/* Activations of the gated product (qgemv_gus_act_nrm). */
enum { QG_ACT_SILU = 0, QG_ACT_GELU_TANH = 1 };

/* Limits checked by every entry point. */
#define QG_MAX_NB 16
#define QG_MAX_TOPK 8
#define QG_MAX_K 65536

/* Bytes of the packed device layout of an N x K matrix, or -1 if (fmt, N, K) is invalid.
 * Equal to the GGUF byte count rounded up to 256 B per plane (two planes: quants and scales; the
 * Q5 formats add a plane of fifth bits, Q6_K one of high bit pairs and one of its d values, the
 * IQ4 formats 256 B that hold the 16-byte codebook).
 * Host-only, no HIP call. */
int64_t qgemv_packed_bytes(int fmt, int64_t N, int64_t K);

/* Re-lay GGUF-native blocks (w_gguf: N rows of K/bs consecutive blocks, the native row order of
 * "honeycrisp mod.rs", transpose_q8_blocks) into the packed layout (w_packed, at least
 * qgemv_packed_bytes bytes, 256-B aligned).  A pure byte move, done once per matrix; the
 * analogue of the pad/re-layout passes of "Crate inferencelayer" (q8_0_pad_blocks,
 * q6k_pad_blocks).  Both pointers are device pointers and must not overlap.  For Q4_K expert
 * stacks pass N = n_exp * rows.  The IQ4 formats need their codebook: qgemv_pack returns
 * QG_ERR_NULL for them; use qgemv_pack_codebook. */
int qgemv_pack(int fmt, const void *w_gguf, int64_t N, int64_t K, void *w_packed, void *stream);

/* qgemv_pack with the 16-entry codebook of the IQ4 formats ("Crate inferencelayer",
 * gemv_iq4_nl_k_lcpp_src: a nonlinear table of signed values applied as the weights are read).
 * codebook is a HOST pointer to 16 signed bytes (entry q = codebook[q]), copied before the call
 * returns and stored inside w_packed, so every later call on that matrix uses it.  Required
 * (QG_ERR_NULL if NULL) for QG_IQ4_NL and QG_IQ4_XS; ignored, and may be NULL, for the other
 * formats. */
int qgemv_pack_codebook(int fmt, const void *w_gguf, int64_t N, int64_t K, const int8_t *codebook,
                        void *w_packed, void *stream);

/* Workspace bytes an operation needs for these sizes (0 if none), or -1 on invalid sizes.
 * n_exp and topk are read only for QG_OP_MOE.  Host-only. */
int64_t qgemv_workspace_bytes(int op, int fmt, int64_t N, int64_t K, int nb, int64_t n_exp,
                              int topk);

/* y[r][n] = sum_k W[n][k] x[r][k].  ("Crate inferencelayer", gemv_q4_k_lcpp_src and its
 * Q8_0 / Q4_K siblings; "honeycrisp mod.rs", quant_matmul.)  y must not overlap x or W. */
int qgemv(int fmt, const void *W, int64_t N, int64_t K, const float *x, int nb, float *y,
          void *ws, size_t ws_bytes, void *stream);

/* y = W rmsnorm(x): n[r][k] = x[r][k] * gamma[k] / sqrt(mean_k x[r][k]^2 + eps), then the GEMV.
 * ("honeycrisp mod.rs", fused_norm_quant_matmul_multi and the Op::RmsNorm { eps } arm.)
 * gamma is f32 [K].  A concatenated Q|K|V matrix is passed as one W of N = nq + nk + nv rows. */
int qgemv_nrm(int fmt, const void *W, int64_t N, int64_t K, const float *x, const float *gamma,
              float eps, int nb, float *y, void *ws, size_t ws_bytes, void *stream);

/* h[r][n] = silu(g) * u with g = Wg n_r, u = Wu n_r and n = rmsnorm(x) as in qgemv_nrm;
 * silu(g) = g / (1 + e^-g).  ("honeycrisp mod.rs", fused_norm_swiglu_down: mid = silu(gate) * up;
 * "Crate inferencelayer", mlp_gate_q8_0n_lcpp_src: act(gate) * up.)  Wg and Wu are two packed
 * matrices of the same format and shape N x K; h is f32 [nb][N]. */
int qgemv_gus_nrm(int fmt, const void *Wg, const void *Wu, int64_t N, int64_t K, const float *x,
                  const float *gamma, float eps, int nb, float *h, void *ws, size_t ws_bytes,
                  void *stream);

/* y = W rmsnorm(x) + bias: qgemv_nrm with bias[n] added to every batch row at the output
 * ("honeycrisp mod.rs", pipe_q8_nrm_mb64_bias: "add bias[row] at output"; the Qwen2-style
 * attention bias of the fused QKV).  bias is f32 [N], 4-B aligned, not overlapping y. */
int qgemv_nrm_bias(int fmt, const void *W, int64_t N, int64_t K, const float *x,
                   const float *gamma, float eps, const float *bias, int nb, float *y, void *ws,
                   size_t ws_bytes, void *stream);

/* qgemv_gus_nrm with a choice of activation: h = act(g) * u, act = QG_ACT_SILU (g / (1 + e^-g))
 * or QG_ACT_GELU_TANH (0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))), the GeluTanh variant of
 * "honeycrisp mod.rs", pipe_q8_large4_gus_nrm_gelu).  Any other act is QG_ERR_SHAPE. */
int qgemv_gus_act_nrm(int fmt, const void *Wg, const void *Wu, int64_t N, int64_t K,
                      const float *x, const float *gamma, float eps, int act, int nb, float *h,
                      void *ws, size_t ws_bytes, void *stream);

/* Per-head QK RMSNorm + RoPE, in place on the output of a fused QKV GEMV ("honeycrisp mod.rs",
 * pipe_qk_norm_rope and its launch: one group per head, Q heads then K heads).  qkv is f32
 * [nb][(n_q_heads + 2 n_kv_heads) head_dim]: the Q heads, then the K heads, then the V heads.
 * Each Q (K) head h: v = v * q_gamma / sqrt(mean(v^2) + eps) over its head_dim values
 * (k_gamma for K heads; a NULL gamma skips that normalization), then for j < rope_half the pair
 * (v[j], v[j + rope_half]) becomes (v[j] c - v[j + rope_half] s, v[j + rope_half] c + v[j] s)
 * with c = rope_cos[r][j], s = rope_sin[r][j] (the caller's tables, one row of rope_half values
 * per batch row: the position's row of the [max_seq][rope_half] tables); values from
 * 2 rope_half on are not rotated.  V heads are not touched.  Limits: head_dim even, <= 256;
 * 0 <= rope_half <= head_dim / 2; nb in [1, 16]. */
int qgemv_qk_norm_rope(float *qkv, int nb, int n_q_heads, int n_kv_heads, int head_dim,
                       int rope_half, const float *q_gamma, const float *k_gamma, float eps,
                       const float *rope_cos, const float *rope_sin, void *stream);

/* y[r][n] = sum_k W[n][k] x[r][k] + res[r][n].  ("honeycrisp mod.rs", fused matmul + residual in
 * forward_decode_fused_layers.)  res is f32 [nb][N]; y may equal res (in place), no other
 * overlap is allowed. */
int qgemv_res(int fmt, const void *W, int64_t N, int64_t K, const float *x, const float *res,
              int nb, float *y, void *ws, size_t ws_bytes, void *stream);

/* logits[r][n] = sum_k W[n][k] x[r][k] and idx[r] = the lowest n holding the maximum of row r
 * (greedy argmax on the GPU, no logits read-back: "Module gpu", sampling; "Crate
 * inferencelayer", crate summary).  idx is int32 [nb].  Needs a workspace. */
int qgemv_argmax(int fmt, const void *W, int64_t N, int64_t K, const float *x, int nb,
                 float *logits, int32_t *idx, void *ws, size_t ws_bytes, void *stream);

/* qgemv_argmax without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * same kernels, with the partial keys in a fixed scratch array the library holds on each device
 * it runs on (512 KiB, from the first call until the process ends).  The call itself allocates
 * nothing.  The array is shared by every call on that device and keeps the last call's partial
 * keys (each launch writes every key it reads, so nothing needs clearing): calls that may overlap
 * on one device (different streams, or concurrent graph replays) race and must be ordered by the
 * caller.  Sizes and errors as qgemv_argmax; the scratch covers every accepted size. */
int qgemv_argmax_noalloc(int fmt, const void *W, int64_t N, int64_t K, const float *x, int nb,
                         float *logits, int32_t *idx, void *stream);

/* Routed experts: y[r][n] = sum_{t=0..topk-1} wts[r][t] * (W_{ids[r][t]} x_r)[n], the terms added
 * in ascending t.  ("Module gpu", type alias RouteStep: expert ids and routing weights of one
 * step; module experts.)  W_experts holds n_exp packed N x K matrices back to back (pack them
 * as one matrix of n_exp * N rows).  ids int32 [nb][topk]; wts f32 [nb][topk].  An id outside
 * [0, n_exp) adds nothing to its row and sets a sticky flag in the workspace that
 * qgemv_moe_error reports.  Limits: n_exp <= 1024 (QG_ERR_SHAPE beyond), and each expert's
 * quant plane (N * K/2 bytes, Q8_0 N * K) under 2 GiB.  Needs a workspace. */
int qgemv_moe(int fmt, const void *W_experts, int64_t n_exp, int64_t N, int64_t K, const float *x,
              int nb, const int32_t *ids, const float *wts, int topk, float *y, void *ws,
              size_t ws_bytes, void *stream);

/* Wide row batch (prefill chunks): y[m][n] = sum_k W[n][k] x[m][k] for M rows of x at once, so
 * every weight streams once for the whole chunk ("Module gpu", module prefill; "Crate
 * inferencelayer", gemm_q4_src / gemm_q8_0n_src / gemm_q1_src: tiles sharing one weight stream,
 * one 32-weight block per inner step; gemm_q4_splitk_src / gemm_q4_splitk_reduce_src: K split
 * over workgroups when the tiles do not fill the device).  Formats Q4_0, Q8_0 and Q1_0 (others:
 * QG_ERR_FORMAT).  x f32 [M][K], y f32 [M][N], 4-B aligned; 1 <= M <= QG_GEMM_MAX_M.  ws: at
 * least qgemm_workspace_bytes(fmt, N, K, M) bytes, 256-B aligned, written before it is read (x
 * converted to f16 once per call, split-K partial tiles); two launches on `stream` (three when
 * K is split: the partial tiles are then added in a fixed order).  Up to QG_MAX_NB rows with x
 * 16-B aligned, where qgemv runs on its matrix-core or streaming kernel, the call runs that
 * row-batch GEMV instead (one launch, faster there; the workspace is then not touched).  Either way: exact weights, x rounded to f16 after a
 * power-of-two scaling (of each row; of each 32-weight chunk on the GEMV's vector path, nb <= 4),
 * f32 accumulation. */
#define QG_GEMM_MAX_M (1 << 20)
int64_t qgemm_workspace_bytes(int fmt, int64_t N, int64_t K, int64_t M);
int qgemm(int fmt, const void *W, int64_t N, int64_t K, const float *x, int64_t M, float *y,
          void *ws, size_t ws_bytes, void *stream);

/* Reads and clears the bad-expert-id flag qgemv_moe leaves in its workspace (*flag = 1 if any id
 * of an earlier call on this workspace was out of range; any other nonzero value means a launch
 * broke the kernel's own sizing contract, a library bug).  Unlike every other entry point this
 * one SYNCHRONIZES `stream` (it copies the flag to the host).  The sizes must be those the
 * workspace was sized for. */
int qgemv_moe_error(const void *ws, int64_t n_exp, int64_t N, int64_t K, int fmt, int *flag,
                    void *stream);

/* Static, human-readable text of a status code. */
const char *qgemv_status_str(int status);

/* Version of the packed layout; changes whenever qgemv_pack's output changes. */
int qgemv_layout_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */

/*
 * oracle.c -- plain, slow, f64 CPU oracle for block-quantized GEMV in LLM decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * helper with the HIP library; it reads the GGUF-native block bytes that the
 * seeded generators write, never the packed device layout.
 *
 * Every value is carried in double precision.  Each function names the page
 * and item its arithmetic follows:
 *   [ILayer]  "Crate inferencelayer" (docs.rs, inferencelayer 0.2.4), items
 *             under "Functions".
 *   [Gpu]     "Module gpu" (cherenkov qwen4_exp::gpu docs), items under
 *             "Structs", "Modules" and "Type Aliases".
 *   [Honey]   "honeycrisp mod.rs" (Apple-Silicon Metal backend source), items
 *             named by the Rust function or match arm they sit in.
 *
 * The pages never print a worked numeric example, so the tests pin this file
 * with hand-built blocks, closed forms and invariants instead.  Two things
 * stay "parity unpinned": agreement with a real GGUF artifact, and the exact
 * GGUF bit order of Q4_0 nibbles and Q4_K (scale, min) pairs, which the pages
 * leave open (readings listed in the design notes).
 *
 * Parallelism: output rows are independent, so an OpenMP loop runs over them.
 * The order of the K-sum inside one output is the plain ascending k order.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

int orc_threads(void);

#define ORC_Q4_0 2
#define ORC_Q5_0 6
#define ORC_Q8_0 8
#define ORC_Q4_K 12
#define ORC_Q5_K 13
#define ORC_Q6_K 14
#define ORC_IQ4_NL 20
#define ORC_IQ4_XS 23
#define ORC_Q1_0 40
#define ORC_AQ4 41

/* The 16-entry codebook of the IQ4 formats.  The pages say the codebook is a
 * 16-entry nonlinear table of signed values applied in the shader ([ILayer]
 * gemv_iq4_nl_k_lcpp_src) but print none of its values, so it is an input:
 * orc_set_codebook installs the table the next decodes use. */
static int8_t orc_cb[16];

void orc_set_codebook(const int8_t *cb)
{
    memcpy(orc_cb, cb, 16);
}

/* ---------------------------------------------------------------------------
 * IEEE 754 binary16 -> double, exact for every bit pattern (little-endian
 * storage is a reading: the pages say the blocks are read "as-is" from GGUF,
 * [ILayer] gemv_q8_0n_k_lcpp_src, and GGUF is little-endian).
 * ------------------------------------------------------------------------- */
double orc_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 31;
    int mant = h & 1023;
    double v;
    if (expo == 0)
        v = ldexp((double)mant, -24);                 /* zero / subnormal */
    else if (expo == 31)
        v = mant ? NAN : INFINITY;
    else
        v = ldexp((double)(mant + 1024), expo - 25);  /* 1.m * 2^(e-15) */
    return sign ? -v : v;
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Bytes of one block and weights per block, per format. */
int64_t orc_block_bytes(int fmt)
{
    switch (fmt) {
    case ORC_Q4_0: return 18;   /* [ILayer] gemv_q1_k_lcpp_src: Q4_0 is 18 B per 32 weights */
    case ORC_Q5_0: return 22;   /* [ILayer] gemv_q5_0n_k_lcpp_src: f16 d, 4 B qh, 16 B nibbles */
    case ORC_Q8_0: return 34;   /* [ILayer] gemv_q8_0n_k_lcpp_src: f16 d + 32 x i8 */
    case ORC_Q4_K: return 144;  /* f16 d, f16 dmin, 12 B packed 6-bit pairs, 128 B nibbles */
    case ORC_Q5_K: return 176;  /* [ILayer] gemv_q5k_k_lcpp_src: Q4_K's fields + 32 B qh */
    case ORC_Q6_K: return 210;  /* [ILayer] gemv_q6k_k_lcpp_src: 128 ql, 64 qh, 16 i8 scales, d */
    case ORC_IQ4_NL: return 18; /* [ILayer] iq4_nl_pad_blocks: IQ4_NL blocks are 18 bytes */
    case ORC_IQ4_XS: return 136;/* [ILayer] gemv_iq4_xs_k_lcpp_src: 136-byte superblocks */
    case ORC_Q1_0: return 18;   /* [ILayer] gemv_q1_k_lcpp_src: 4.5 B per 32 weights, 128 per scale */
    case ORC_AQ4: return 20;    /* [Gpu] struct Q: affine Q4, f16 scale and bias per 32 (a reading) */
    default: return -1;
    }
}

int64_t orc_block_weights(int fmt)
{
    switch (fmt) {
    case ORC_Q4_0: return 32;
    case ORC_Q5_0: return 32;
    case ORC_Q8_0: return 32;
    case ORC_Q4_K: return 256;  /* [Honey] quant_matmul: Q4_K when k % 256 == 0 */
    case ORC_Q5_K: return 256;
    case ORC_Q6_K: return 256;
    case ORC_IQ4_NL: return 32;
    case ORC_IQ4_XS: return 256;
    case ORC_Q1_0: return 128;
    case ORC_AQ4: return 32;
    default: return -1;
    }
}

/* Q4_0: w = (q - 8) * d.  [ILayer] q4_0_to_q8_0n states the exact upcast
 * d8 = d4, q8 = nib - 8, i.e. each weight is d times the nibble less 8.
 * Nibble order (a reading): the low nibble of byte j is element j, the high
 * nibble is element j + 16. */
static void dq_q4_0(const uint8_t *b, double *w)
{
    double d = orc_f16(rd16(b));
    const uint8_t *qs = b + 2;
    for (int j = 0; j < 16; ++j) {
        int lo = qs[j] & 15;
        int hi = qs[j] >> 4;
        w[j] = (double)(lo - 8) * d;
        w[j + 16] = (double)(hi - 8) * d;
    }
}

/* Q8_0: w = d * q with q a signed byte.  [ILayer] gemv_q8_0n_k_lcpp_src. */
static void dq_q8_0(const uint8_t *b, double *w)
{
    double d = orc_f16(rd16(b));
    const int8_t *qs = (const int8_t *)(b + 2);
    for (int j = 0; j < 32; ++j)
        w[j] = d * (double)qs[j];
}

/* The 6-bit (scale, min) pair of sub-block j from the 12 packed bytes.
 * [ILayer] gemv_q5k_k_lcpp_src says Q5_K uses "the same 6-bit pack as Q4_K";
 * the bit positions below are the GGUF K-quant reading of that pack:
 * pairs 0..3 sit in the low 6 bits of bytes j and j+4; pairs 4..7 take their
 * low 4 bits from byte j+4 (scale: low half, min: high half) and their top
 * 2 bits from the spare top bits of bytes j-4 (scale) and j (min). */
void orc_q4k_scale_min(const uint8_t *s, int j, int *sc, int *m)
{
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* Q4_K super-block of 256 weights: w = d * sc_j * q - dmin * m_j
 * (form given for the 5-bit sibling in [ILayer] gemv_q5k_k_lcpp_src, minus
 * the fifth bit).  Element order (a reading): chunk c = 0..3 covers 64
 * elements; byte qs[32c + l] holds element 64c + l in its low nibble
 * (sub-block 2c) and element 64c + 32 + l in its high nibble (sub-block
 * 2c + 1). */
static void dq_q4_k(const uint8_t *b, double *w)
{
    double d = orc_f16(rd16(b));
    double dmin = orc_f16(rd16(b + 2));
    const uint8_t *s = b + 4;
    const uint8_t *qs = b + 16;
    for (int c = 0; c < 4; ++c) {
        int sc0, m0, sc1, m1;
        orc_q4k_scale_min(s, 2 * c, &sc0, &m0);
        orc_q4k_scale_min(s, 2 * c + 1, &sc1, &m1);
        for (int l = 0; l < 32; ++l) {
            int lo = qs[32 * c + l] & 15;
            int hi = qs[32 * c + l] >> 4;
            w[64 * c + l] = d * (double)sc0 * (double)lo - dmin * (double)m0;
            w[64 * c + 32 + l] = d * (double)sc1 * (double)hi - dmin * (double)m1;
        }
    }
}

/* Q5_0: w = d ((nib | bit << 4) - 16).  [ILayer] gemv_q5_0n_k_lcpp_src (and
 * q5_0_to_q8_0n: q8 = (nib | bit << 4) - 16).  Field order d, qh, qs as the
 * page's padded layout lists them.  Bit order (a reading): element j takes its
 * nibble as Q4_0 does (low nibble of byte j for j < 16, high nibble of byte
 * j - 16 otherwise) and its fifth bit from bit j of the little-endian qh word. */
static void dq_q5_0(const uint8_t *b, double *w)
{
    double d = orc_f16(rd16(b));
    uint32_t qh = (uint32_t)b[2] | ((uint32_t)b[3] << 8) | ((uint32_t)b[4] << 16) |
                  ((uint32_t)b[5] << 24);
    const uint8_t *qs = b + 6;
    for (int j = 0; j < 16; ++j) {
        int lo = (qs[j] & 15) | (int)(((qh >> j) & 1u) << 4);
        int hi = (qs[j] >> 4) | (int)(((qh >> (j + 16)) & 1u) << 4);
        w[j] = d * (double)(lo - 16);
        w[j + 16] = d * (double)(hi - 16);
    }
}

/* Q5_K super-block of 256: w = d sc_j q - dmin m_j with q = nib | bit << 4.
 * [ILayer] gemv_q5k_k_lcpp_src: Q4_K's d, dmin and 12-byte 6-bit pack, then
 * 32 qh bytes, then 128 nibble bytes; sub-block s takes bit s of qh[l].  The
 * nibble order and l (the element's place within its sub-block of 32) follow
 * the Q4_K reading. */
static void dq_q5_k(const uint8_t *b, double *w)
{
    double d = orc_f16(rd16(b));
    double dmin = orc_f16(rd16(b + 2));
    const uint8_t *s = b + 4;
    const uint8_t *qh = b + 16;
    const uint8_t *qs = b + 48;
    for (int c = 0; c < 4; ++c) {
        int sc0, m0, sc1, m1;
        orc_q4k_scale_min(s, 2 * c, &sc0, &m0);
        orc_q4k_scale_min(s, 2 * c + 1, &sc1, &m1);
        for (int l = 0; l < 32; ++l) {
            int lo = (qs[32 * c + l] & 15) | (((qh[l] >> (2 * c)) & 1) << 4);
            int hi = (qs[32 * c + l] >> 4) | (((qh[l] >> (2 * c + 1)) & 1) << 4);
            w[64 * c + l] = d * (double)sc0 * (double)lo - dmin * (double)m0;
            w[64 * c + 32 + l] = d * (double)sc1 * (double)hi - dmin * (double)m1;
        }
    }
}

/* Q6_K super-block of 256: 128 ql bytes (low 4 bits), 64 qh bytes (high 2
 * bits), 16 signed 8-bit scales (one per 16 weights), f16 d ([ILayer]
 * gemv_q6k_k_lcpp_src gives these fields in this order).  w = d sc (q - 32)
 * with q = low | high << 4 in 0..63.  Which bits of which bytes form element
 * e (a reading; the page gives field sizes only): in each half n of 128
 * elements, for l < 32, byte ql[64n + l] holds element 128n + l (low nibble)
 * and 128n + 64 + l (high nibble), byte ql[64n + 32 + l] holds 128n + 32 + l
 * and 128n + 96 + l, and qh[32n + l] holds their high bits in bit pairs 0-1,
 * 2-3, 4-5, 6-7 for elements 128n + l, + 32, + 64, + 96; element 128n + i
 * takes scale 8n + i / 16. */
static void dq_q6_k(const uint8_t *b, double *w)
{
    const uint8_t *ql = b, *qh = b + 128;
    const int8_t *sc = (const int8_t *)(b + 192);
    double d = orc_f16(rd16(b + 208));
    for (int n = 0; n < 2; ++n) {
        for (int l = 0; l < 32; ++l) {
            int q1 = (ql[64 * n + l] & 15) | (((qh[32 * n + l] >> 0) & 3) << 4);
            int q2 = (ql[64 * n + 32 + l] & 15) | (((qh[32 * n + l] >> 2) & 3) << 4);
            int q3 = (ql[64 * n + l] >> 4) | (((qh[32 * n + l] >> 4) & 3) << 4);
            int q4 = (ql[64 * n + 32 + l] >> 4) | (((qh[32 * n + l] >> 6) & 3) << 4);
            int e = 128 * n + l;
            w[e] = d * (double)sc[8 * n + e % 128 / 16] * (double)(q1 - 32);
            w[e + 32] = d * (double)sc[8 * n + (e + 32) % 128 / 16] * (double)(q2 - 32);
            w[e + 64] = d * (double)sc[8 * n + (e + 64) % 128 / 16] * (double)(q3 - 32);
            w[e + 96] = d * (double)sc[8 * n + (e + 96) % 128 / 16] * (double)(q4 - 32);
        }
    }
}

/* IQ4_NL: 32 weights, f16 d + 16 bytes of codebook indices; w = d cb[idx].
 * [ILayer] gemv_iq4_nl_k_lcpp_src (the 16-entry nonlinear codebook applied in
 * the shader), iq4_nl_pad_blocks (18-byte blocks: f16 d then the 16 index
 * bytes).  Index order (a reading): as Q4_0, element j in the low nibble of
 * byte j, element j + 16 in its high nibble. */
static void dq_iq4_nl(const uint8_t *b, double *w)
{
    double d = orc_f16(rd16(b));
    for (int j = 0; j < 16; ++j) {
        w[j] = d * (double)orc_cb[b[2 + j] & 15];
        w[j + 16] = d * (double)orc_cb[b[2 + j] >> 4];
    }
}

/* IQ4_XS: 256 weights, f16 d, packed 6-bit sub-scales biased by -32, then 8
 * sub-blocks of 32 codebook indices ([ILayer] gemv_iq4_xs_k_lcpp_src).  The
 * 6-bit packing (a reading): a 16-bit word of high 2-bit pairs (sub-block s at
 * bits 2s, 2s+1), then 4 bytes of low nibbles (sub-block s at bits 4s..4s+3 of
 * the little-endian word); sub-block s's weights are d (ls - 32) cb[idx] with
 * its 16 index bytes holding elements 32s + j (low nibble) and 32s + 16 + j
 * (high nibble). */
static void dq_iq4_xs(const uint8_t *b, double *w)
{
    double d = orc_f16(rd16(b));
    uint32_t sh = rd16(b + 2);
    uint32_t sl = (uint32_t)b[4] | ((uint32_t)b[5] << 8) | ((uint32_t)b[6] << 16) |
                  ((uint32_t)b[7] << 24);
    const uint8_t *qs = b + 8;
    for (int s = 0; s < 8; ++s) {
        int ls = (int)((sl >> (4 * s)) & 15u) | (int)(((sh >> (2 * s)) & 3u) << 4);
        double dl = d * (double)(ls - 32);
        for (int j = 0; j < 16; ++j) {
            w[32 * s + j] = dl * (double)orc_cb[qs[16 * s + j] & 15];
            w[32 * s + 16 + j] = dl * (double)orc_cb[qs[16 * s + j] >> 4];
        }
    }
}

/* Q1_0: 128 weights, f16 d then 16 bytes of sign bits; bit i of the
 * little-endian bit stream (bit i % 8 of byte i / 8) is element i's sign,
 * 1 -> +d, 0 -> -d.  [ILayer] gemv_q1_k_lcpp_src ("bit i is x-element i's
 * sign, 1 -> +1, 0 -> -1", one f16 scale per 128 weights, 4.5 bytes per 32);
 * the field order (d first) is a reading, as for the other block types. */
static void dq_q1_0(const uint8_t *b, double *w)
{
    double d = orc_f16(rd16(b));
    for (int i = 0; i < 128; ++i)
        w[i] = ((b[2 + i / 8] >> (i % 8)) & 1) ? d : -d;
}

/* Affine Q4 (AQ4): 32 weights, f16 scale s, f16 bias c, 16 nibble bytes;
 * w = s q + c.  [Gpu] struct Q ("affine-Q4 projection") and struct HalfSet
 * (x as even / odd halves plus per-32 group sums: the sums multiply the bias).
 * Nibble order (a reading matching the even / odd split): element 2i is the
 * low nibble of byte i, element 2i + 1 its high nibble. */
static void dq_aq4(const uint8_t *b, double *w)
{
    double sc = orc_f16(rd16(b)), c = orc_f16(rd16(b + 2));
    for (int i = 0; i < 16; ++i) {
        w[2 * i] = sc * (double)(b[4 + i] & 15) + c;
        w[2 * i + 1] = sc * (double)(b[4 + i] >> 4) + c;
    }
}

/* Dequantize one row of K weights (K a multiple of the block size) from its
 * GGUF-native bytes.  A row is K/bs consecutive blocks ([Honey]
 * transpose_q8_blocks: [n_rows, n_blocks, block] is the native order). */
int orc_dequant_row(int fmt, const uint8_t *row, int64_t K, double *w)
{
    int64_t bb = orc_block_bytes(fmt), bw = orc_block_weights(fmt);
    if (bb < 0 || K % bw != 0)
        return -1;
    for (int64_t b = 0; b < K / bw; ++b) {
        const uint8_t *blk = row + b * bb;
        double *out = w + b * bw;
        switch (fmt) {
        case ORC_Q4_0: dq_q4_0(blk, out); break;
        case ORC_Q5_0: dq_q5_0(blk, out); break;
        case ORC_Q8_0: dq_q8_0(blk, out); break;
        case ORC_Q4_K: dq_q4_k(blk, out); break;
        case ORC_Q5_K: dq_q5_k(blk, out); break;
        case ORC_Q6_K: dq_q6_k(blk, out); break;
        case ORC_IQ4_NL: dq_iq4_nl(blk, out); break;
        case ORC_IQ4_XS: dq_iq4_xs(blk, out); break;
        case ORC_Q1_0: dq_q1_0(blk, out); break;
        default: dq_aq4(blk, out); break;
        }
    }
    return 0;
}

int64_t orc_row_bytes(int fmt, int64_t K)
{
    int64_t bb = orc_block_bytes(fmt), bw = orc_block_weights(fmt);
    if (bb < 0 || K % bw != 0)
        return -1;
    return K / bw * bb;
}

/* ---------------------------------------------------------------------------
 * GEMV: y[r][i] = sum_k w[n_i][k] * v[r][k], and A[r][i] = sum_k |w v|,
 * the scale of the tolerance.  v is [nb][K] row-major (the row batch of
 * [Gpu] module docs: nb consecutive positions, activations [nb][...]).
 * rows == NULL means all N rows (nrows == N); otherwise only the listed rows
 * are computed, and y, A are [nb][nrows].
 * ------------------------------------------------------------------------- */
int orc_gemv(int fmt, const uint8_t *W, int64_t N, int64_t K, const double *v, int64_t nb,
             const int64_t *rows, int64_t nrows, double *y, double *A)
{
    int64_t rb = orc_row_bytes(fmt, K);
    if (rb < 0)
        return -1;
    if (!rows)
        nrows = N;
    int err = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t i = 0; i < nrows; ++i) {
            int64_t n = rows ? rows[i] : i;
            if (n < 0 || n >= N || !w) {
                err = -1;
                continue;
            }
            orc_dequant_row(fmt, W + n * rb, K, w);
            for (int64_t r = 0; r < nb; ++r) {
                const double *vr = v + r * K;
                double s = 0.0, a = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    double p = w[k] * vr[k];
                    s += p;
                    a += fabs(p);
                }
                y[r * nrows + i] = s;
                if (A)
                    A[r * nrows + i] = a;
            }
        }
        free(w);
    }
    return err;
}

/* RMSNorm of each row: n_k = x_k * gamma_k / sqrt(mean_k x_k^2 + eps).
 * [Honey] execute, arm Op::RmsNorm { eps }: gamma has shape [d] and the op
 * runs over the flattened batch; eps inside the root and the plain gamma
 * multiply are readings (the weights module of [ILayer] folds any (1 + w)
 * convention into gamma at load, so kernels take gamma as is). */
void orc_rmsnorm(const double *x, const double *gamma, int64_t nb, int64_t K, double eps,
                 double *out)
{
    for (int64_t r = 0; r < nb; ++r) {
        const double *xr = x + r * K;
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k)
            ss += xr[k] * xr[k];
        double inv = 1.0 / sqrt(ss / (double)K + eps);
        for (int64_t k = 0; k < K; ++k)
            out[r * K + k] = xr[k] * inv * gamma[k];
    }
}

/* SiLU-gated product h = silu(g) * u, silu(g) = g / (1 + e^-g).
 * [Honey] fused_norm_swiglu_down, step "mid = silu(gate) * up". */
void orc_swiglu(const double *g, const double *u, int64_t n, double *h)
{
    for (int64_t i = 0; i < n; ++i)
        h[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
}

/* GELU-gated product h = gelu(g) * u with the tanh form of GELU,
 * gelu(g) = g/2 (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))).  [Honey] pipeline
 * field pipe_q8_large4_gus_nrm_gelu, the "GeluTanh variant" of the fused
 * gate/up + norm step; the tanh form is the one the variant's name gives. */
void orc_gelu_tanh_gate(const double *g, const double *u, int64_t n, double *h)
{
    const double k0 = sqrt(2.0 / M_PI);
    for (int64_t i = 0; i < n; ++i) {
        double x = g[i];
        h[i] = 0.5 * x * (1.0 + tanh(k0 * (x + 0.044715 * x * x * x))) * u[i];
    }
}

/* Per-head QK RMSNorm + RoPE in place on y[nb][(nq + 2 nkv) hd] ([Honey] the
 * QK-norm + RoPE step of the fused QKV chain: one group per head over the Q
 * heads then the K heads, with q_norm / k_norm weights, rope_half, eps, and
 * cos / sin tables of rope_half values per position).  Q head h is normalized
 * by 1/sqrt(mean of its squares + eps) and scaled by qg (K heads by kg; a NULL
 * gamma skips the normalization), then each pair (j, j + rh), j < rh, is
 * rotated by the angle whose cosine / sine are cs[r][j] / sn[r][j].  The pair
 * layout (j with j + rh) is a reading: the page gives only the half size.
 * V heads are not touched. */
void orc_qk_norm_rope(double *y, int64_t nb, int64_t nq, int64_t nkv, int64_t hd, int64_t rh,
                      const double *qg, const double *kg, double eps, const double *cs,
                      const double *sn)
{
    int64_t row = (nq + 2 * nkv) * hd;
    for (int64_t r = 0; r < nb; ++r) {
        for (int64_t h = 0; h < nq + nkv; ++h) {
            double *v = y + r * row + h * hd;
            const double *gam = h < nq ? qg : kg;
            if (gam) {
                double ss = 0.0;
                for (int64_t k = 0; k < hd; ++k)
                    ss += v[k] * v[k];
                double inv = 1.0 / sqrt(ss / (double)hd + eps);
                for (int64_t k = 0; k < hd; ++k)
                    v[k] = v[k] * inv * gam[k];
            }
            for (int64_t j = 0; j < rh; ++j) {
                double c = cs[r * rh + j], s = sn[r * rh + j];
                double a = v[j], b = v[j + rh];
                v[j] = a * c - b * s;
                v[j + rh] = b * c + a * s;
            }
        }
    }
}

/* y = W v + r.  [Honey] forward_decode_fused_layers, the fused matmul +
 * residual: y[row] = matmul(x, w)[row] + residual[row]. */
int orc_gemv_res(int fmt, const uint8_t *W, int64_t N, int64_t K, const double *v,
                 const double *r, int64_t nb, const int64_t *rows, int64_t nrows, double *y,
                 double *A)
{
    if (!rows)
        nrows = N;
    if (orc_gemv(fmt, W, N, K, v, nb, rows, nrows, y, A))
        return -1;
    for (int64_t b = 0; b < nb; ++b)
        for (int64_t i = 0; i < nrows; ++i) {
            int64_t n = rows ? rows[i] : i;
            y[b * nrows + i] += r[b * N + n];
        }
    return 0;
}

/* Greedy argmax of each row of y[nb][N]: the lowest index of the maximum.
 * [Gpu] module sampling: logits projection then greedy argmax. */
void orc_argmax(const double *y, int64_t nb, int64_t N, int64_t *idx)
{
    for (int64_t r = 0; r < nb; ++r) {
        const double *yr = y + r * N;
        int64_t best = 0;
        for (int64_t n = 1; n < N; ++n)
            if (yr[n] > yr[best])
                best = n;
        idx[r] = best;
    }
}

/* Routed experts: y[r] = sum_{t = 0..topk-1} p[r][t] * (W_{id[r][t]} x_r), the
 * terms added in ascending t.  [Gpu] type alias RouteStep carries the
 * tokens, expert ids and routing weights of one step; the weights are
 * applied to each selected expert's output and summed per row.
 * W holds n_exp matrices of N x K back to back.  Also writes A = sum_t p *
 * (sum_k |w x|), the tolerance scale. */
int orc_moe(int fmt, const uint8_t *W, int64_t n_exp, int64_t N, int64_t K, const double *x,
            int64_t nb, const int32_t *ids, const double *p, int64_t topk, const int64_t *rows,
            int64_t nrows, double *y, double *A)
{
    int64_t rb = orc_row_bytes(fmt, K);
    if (rb < 0)
        return -1;
    if (!rows)
        nrows = N;
    double *ye = (double *)malloc((size_t)nrows * sizeof(double));
    double *ae = (double *)malloc((size_t)nrows * sizeof(double));
    if (!ye || !ae) {
        free(ye);
        free(ae);
        return -1;
    }
    int err = 0;
    for (int64_t r = 0; r < nb && !err; ++r) {
        for (int64_t i = 0; i < nrows; ++i) {
            y[r * nrows + i] = 0.0;
            if (A)
                A[r * nrows + i] = 0.0;
        }
        for (int64_t t = 0; t < topk; ++t) {
            int32_t e = ids[r * topk + t];
            if (e < 0 || e >= n_exp) {
                err = -1;
                break;
            }
            const uint8_t *We = W + (int64_t)e * N * rb;
            if (orc_gemv(fmt, We, N, K, x + r * K, 1, rows, nrows, ye, ae)) {
                err = -1;
                break;
            }
            double pt = p[r * topk + t];
            for (int64_t i = 0; i < nrows; ++i) {
                y[r * nrows + i] += pt * ye[i];
                if (A)
                    A[r * nrows + i] += fabs(pt) * ae[i];
            }
        }
    }
    free(ye);
    free(ae);
    return err;
}

/* Sets the number of OpenMP threads later parallel loops use (the bench times the oracle with
 * one thread and with all of them); returns the number now in effect. */
int orc_set_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
    return orc_threads();
}

/* Number of OpenMP threads the oracle's parallel loops use. */
int orc_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}

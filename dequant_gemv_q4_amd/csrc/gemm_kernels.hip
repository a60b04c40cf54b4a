// gemm_kernels.hip -- wide row-batch dequant GEMM (prefill chunks of many rows) on the gfx950
// matrix cores: Y[M][N] = X[M][K] W[N][K]^T with W block-quantized (Q4_0, Q8_0, Q1_0).
//
// "Module gpu" (cherenkov qwen4_exp docs), module prefill: a prompt chunk of up to a few thousand
// tokens goes through a layer at once so that each weight is streamed once for the whole chunk;
// "Crate inferencelayer" docs, gemm_q1_src / gemm_q4_src: a classic blocked GEMM whose tiles share
// one weight stream, one Q4 block (32 k) per inner step, the activation tile staged in shared
// memory; gemm_q4_splitk_src / gemm_q4_splitk_reduce_src: K split over workgroups when the tiles
// alone do not fill the device, the partial sums folded by a second pass.  Here:
//  - x is first turned into f16 once per call (k_xprep): each row scaled by the power of two that
//    puts its largest |x| in [2^14, 2^15), the high-nibble positions of Q4_0 times 1/16, and laid
//    out in 1 KB chunks (16 rows x one 32-k block) whose 64 16-byte pieces are the A operands of
//    v_mfma_f32_16x16x32_f16 in lane order (mf_elem), zero past K and past M;
//  - a workgroup (8 waves) owns a BM x 128 WPW tile of Y: BM = 128 x rows (64 when M <= 64, a
//    128-row tile being then half zero rows) against the widest weight tile that still fills the
//    device (Q4_0: 512, 256 or 128 weight rows; Q1_0 and Q8_0: 256 or 128); wave w owns all BM x
//    rows against its WPW groups of 16 weight rows (BM / 16 x WPW MFMA tiles), so each weight is
//    decoded once per workgroup and feeds BM / 16 MFMAs per block (the decode is VALU work; eight
//    x tiles per decoded weight tile keep it under the matrix-core time), and each x operand read
//    from LDS feeds WPW weight tiles.  A step covers 128 k (4 blocks);
//  - x chunks, weight chunks (16 rows x 64 bytes for Q4_0, 128 for Q8_0, 16 for Q1_0) and the
//    block scales go from global memory straight into LDS (global_load_lds: no registers, no LDS
//    store instructions), three stages deep (two where three do not fit in LDS: Q4_0's 512-row
//    tiles, Q8_0's 256-row ones): the loads of step s + 2 (s + 1) are issued while step s
//    computes.  One barrier per step;
//  - the kernel is persistent (one workgroup per compute unit, each walking a list of tiles): the
//    load stream runs across tile boundaries, so the next tile's first loads overlap the current
//    tile's last steps and its stores, and there is no per-wave launch ramp between tiles;
//  - a wave reads the weight chunks it loaded itself from LDS, transposes them across the lane
//    rows (mf_xpose) and decodes exact f16 weights (mf_bop).  Q4_0 (q - 8) and Q8_0 (q): one
//    MFMA per block gives D = A B and acc += d D on the VALU (those FMAs run beside the other
//    wave's products; splitting d into two exact f16 halves for two scaled products per block
//    keeps the sums in the accumulators but doubles the matrix work, 130 vs 108 us at
//    2048 x 8192 x 2048); Q1_0 (sign bits, one f16 d per 128 weights, "Crate inferencelayer"
//    docs, gemm_q1_src): the weights are +-d, exact f16, one MFMA per block accumulating in
//    place.  Either way the weights stay exact; only x is rounded, by at most 2^-11 of itself;
//  - the grid walks the tiles XCD by XCD (workgroup i runs on XCD i % 8): each XCD owns a range of
//    weight tiles and walks them row-tile-major, so the workgroups resident on an XCD share a few x
//    row tiles and the XCD's weight tiles in its L2;
//  - when the tiles are too few for the device the K steps are split over several workgroups; each
//    writes its partial tile to the workspace and k_gemm_fold adds the splits in a fixed order.
#include <hip/hip_runtime.h>

#include "mfma_common.h"

namespace qg {

constexpr int GM_THREADS = 512;                   // 8 waves
constexpr int GM_BM = 128;                        // rows of x per tile (the larger of 128, 64)
constexpr int GM_BPS = 4;                         // 32-k blocks per step
constexpr int GM_STAGES = 3;
static_assert(GM_BM == QG_GEMM_BM && GM_BPS * 32 == QG_GEMM_KSTEP, "the host plans with these tiles");

// LDS stage of one step: x chunks [row group 0..BM/16-1][block 0..3] (1 KB each), then weight chunks
// [row group][half] (1 KB each: 16 rows x 4 chunks of 16 B), then the scales [row][block], one
// dword each (a 2-byte copy to LDS fills its lane's dword, zero-extended).  A wave owns WPW
// 16-row weight groups: the most (Q4_0 up to four, Q1_0 and Q8_0 two) whose tiles alone still
// fill the device, since each x operand read from LDS then feeds WPW products, else one (more,
// smaller tiles).
// Q1_0: a step is one 128-weight block, 16 bytes of sign bits per row ([row][4 dwords], one
// dword wave-load per 16 rows) and one scale per row (lane r of the wave's 256-byte area).
template <int FMT, int WPW_, int BM_ = GM_BM>
struct GemmStage {
    static constexpr int BM = BM_;                             // x rows per tile (64 or 128)
    static constexpr int NBT = BM / 16;                        // MFMA tiles along M
    static constexpr int WH = FMT == FQ8_0 ? 2 : 1;            // weight wave-loads per row group
    static constexpr int WPW = WPW_;                           // weight row groups per wave
    static constexpr int BN = 8 * 16 * WPW;                    // weight rows per workgroup
    static constexpr int XB = NBT * GM_BPS * 1024;
    static constexpr int WB = FMT == FQ1_0 ? BN * 16 : BN / 16 * WH * 1024;
    static constexpr int SB = FMT == FQ1_0 ? BN / 16 * 256 : BN * GM_BPS * 4;
    static constexpr int BYTES = XB + WB + SB;
    static constexpr int XPW = NBT * GM_BPS / 8;               // x wave-loads per wave
    // ring depth: three stages where they fit in the 160 KB of LDS (beside the row factors), else two
    static constexpr int STG = 3 * BYTES + 3 * BM * 4 <= 160 * 1024 ? GM_STAGES : 2;
};

// s_waitcnt with vmcnt(N), lgkmcnt(0), expcnt left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void gm_wait()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Global -> LDS copies (global_load_lds): lane l's 16 bytes land at LDS address M0 + 16 l, M0
// being the wave's destination; a 4-byte copy lands at M0 + 4 l and a 2-byte copy writes lane
// l's value zero-extended to the dword at M0 + 4 l.  Written as asm so that the compiler does not
// track them for its waits: it would otherwise wait for every copy in flight before any LDS read;
// the kernel waits for each stage with vmcnt itself.  The memory clobber tells the compiler that
// LDS changes here.  One wait state between the M0 write and the copy.
__device__ __forceinline__ void gm_dma16(const void *src, const void *lds_dst)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_dst);
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void gm_dma4(const void *src, const void *lds_dst)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_dst);
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void gm_dma2(const void *src, const void *lds_dst)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_dst);
    asm volatile("s_nop 0\n\tglobal_load_lds_ushort %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}

// workgroup barrier that the compiler may not move memory accesses across (the LDS reads of a
// stage must stay after the wait for its loads and before the loads that overwrite it)
__device__ __forceinline__ void gm_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// x [M][K] f32 -> xh chunks [Mp / 16][KBp][64 lanes][8 halves] in the A-operand order of each
// 32-k block, and rs[r] = the factor undoing row r's scale; rows past M and columns past K are
// zero (rs 0 past M).  One wave per row: piece q of the row (block q / 4, j = q % 4; chunk lane
// 16 j + r % 16) holds elements 4j..4j+3 and 16+4j..16+4j+3 of its block in both formats
// (mf_elem(j, h) = mf_elem(0, h) + 4 j).  With PPL > 0 each lane keeps its PPL pieces
// q = lane + 64 i in registers, so the row is read once: the wave's largest |x| (the power-of-two
// scale) comes from the held values; PPL = 0 (rows of more than 512 pieces) finds the largest
// |x| in a first pass and re-reads the row, from the cache, in the second.
template <int FMT, int PPL>
__global__ __launch_bounds__(256) void k_xprep(const float *x, int64_t M, int64_t K, int KBp,
                                               _Float16 *xh, float *rs)
{
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const bool live = r < M;
    const bool vec = ((uintptr_t)x & 15) == 0;          // K % 32 == 0: every row is aligned too
    const float *xr = x + (live ? r : 0) * K;
    const int KB = (int)(K / 32);
    auto load_piece = [&](int q, float (&lo)[4], float (&hi4)[4]) {
        const int blk = q >> 2, j = q & 3;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            lo[i] = hi4[i] = 0.f;
        if (live && blk < KB) {
            const float *xb = xr + (int64_t)blk * 32 + 4 * j;
            if (vec) {
                const float4 a = *reinterpret_cast<const float4 *>(xb);
                const float4 b = *reinterpret_cast<const float4 *>(xb + 16);
                lo[0] = a.x; lo[1] = a.y; lo[2] = a.z; lo[3] = a.w;
                hi4[0] = b.x; hi4[1] = b.y; hi4[2] = b.z; hi4[3] = b.w;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    lo[i] = xb[i];
                    hi4[i] = xb[16 + i];
                }
            }
        }
    };
    _Float16 *dst = xh + (r / 16) * (int64_t)KBp * 512 + (int64_t)(r % 16) * 8;
    auto store_piece = [&](int q, const float (&lo)[4], const float (&hi4)[4], float sc) {
        mh8 v;
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            bool hi = false;
            const int e = mf_elem<FMT>(0, h, hi);
            const float xv = e >= 16 ? hi4[e - 16] : lo[e];
            v[h] = (_Float16)(xv * sc * (hi ? 0.0625f : 1.0f));
        }
        *reinterpret_cast<mh8 *>(dst + ((int64_t)(q >> 2) * 64 + 16 * (q & 3)) * 8) = v;
    };
    auto scale_of = [&](float mx) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            mx = fmaxf(mx, __shfl_xor(mx, off));
        int e2 = 0;
        frexpf(mx, &e2);                                   // max |x| = f 2^e2, f in [0.5, 1)
        const int sk = 15 - e2 < 127 ? 15 - e2 : 127;      // 2^sk stays a finite f32
        if (lane == 0)
            rs[r] = live ? ldexpf(1.0f, -sk) : 0.f;
        return live ? ldexpf(1.0f, sk) : 0.f;
    };
    const int NP = 4 * KBp;                                // pieces of the padded row
    if constexpr (PPL > 0) {
        float lo[PPL][4], hi4[PPL][4];
        float mx = 0.f;
#pragma unroll
        for (int i = 0; i < PPL; ++i) {
            load_piece(lane + 64 * i, lo[i], hi4[i]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                mx = fmaxf(mx, fmaxf(fabsf(lo[i][e]), fabsf(hi4[i][e])));
        }
        const float sc = scale_of(mx);
#pragma unroll
        for (int i = 0; i < PPL; ++i)
            if (lane + 64 * i < NP)
                store_piece(lane + 64 * i, lo[i], hi4[i], sc);
    } else {
        float mx = 0.f;
        if (live) {
            if (vec) {
#pragma unroll 8
                for (int64_t e = 4 * lane; e < K; e += 256) {
                    const float4 v = *reinterpret_cast<const float4 *>(xr + e);
                    mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
                }
            } else {
#pragma unroll 8
                for (int64_t e = lane; e < K; e += 64)
                    mx = fmaxf(mx, fabsf(xr[e]));
            }
        }
        const float sc = scale_of(mx);
#pragma unroll 4
        for (int q = lane; q < NP; q += 64) {
            float lo[4], hi4[4];
            load_piece(q, lo, hi4);
            store_piece(q, lo, hi4, sc);
        }
    }
}

template <int FMT, int WPW, int BM>
__global__ __launch_bounds__(GM_THREADS, 1) void k_gemm(GemmArgs a)
{
    using G = GemmStage<FMT, WPW, BM>;
    constexpr int NBT = G::NBT;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[G::STG * G::BYTES];
    __shared__ __attribute__((aligned(16))) float s_rs[3][BM];   // row factors of 3 tiles

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ir = lane & 15, lc = lane >> 4;
    // the pointers' kernel-argument line is fetched with the tile counts', not after them
    asm volatile("" ::"s"(a.qs), "s"(a.xh));

    // tiles of this workgroup (workgroup id i runs on XCD i % 8): XCD x owns weight tiles
    // [x NTX, (x + 1) NTX) and numbers its tiles k8 row-tile-major, then split by split; its
    // workgroups take k8 = slot, slot + nslots, ..., so the ones resident at a time work on a
    // window of consecutive k8 (a few x row tiles, all of the XCD's weight tiles) held in its L2
    const int NTX = (a.n_tiles + 7) / 8;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, nslots = gridDim.x >> 3;
    const int n_base = xcd * NTX;
    const int ntx = a.n_tiles - n_base < NTX ? a.n_tiles - n_base : NTX;
    const int ntiles = ntx > 0 ? ntx * a.m_tiles * a.splits : 0;
    if (slot >= ntiles)
        return;
    struct Tile {
        int64_t m0, n0;
        int s0, S, split;
    };
    auto tile_of = [&](int k8) {
        Tile t;
        const int rest = k8 / ntx;
        t.n0 = (int64_t)(n_base + k8 % ntx) * G::BN;
        t.m0 = (int64_t)(rest % a.m_tiles) * BM;
        t.split = rest / a.m_tiles;
        t.s0 = t.split * a.sps;
        t.S = a.steps - t.s0 < a.sps ? a.steps - t.s0 : a.sps;   // >= 1 (host plan)
        return t;
    };

    const int C = (int)(a.qs_row / 16), KB = (int)(a.K / 32);

    // This lane's weight and scale row pointers of a tile (rows past N read row N - 1), formed
    // once per tile by the issue cursor.  Weights: row group g = WPW wave + wt, lane (ir, lc) ->
    // row 16 g + ir (Q1_0: row 16 g + l / 4, dword l % 4 of a block); scales: lane l -> row
    // 16 g + l / 4 (Q1_0: row 16 g + l % 16, lanes 16.. repeating those rows).
    struct RowPtrs {
        const uint8_t *w[G::WPW];
        const uint8_t *sc[G::WPW];
    };
    auto row_ptrs = [&](const Tile &t) {
        RowPtrs rp;
#pragma unroll
        for (int wt = 0; wt < G::WPW; ++wt) {
            const int64_t r0 = t.n0 + 16 * (G::WPW * wave + wt);
            const int64_t wi = r0 + (FMT == FQ1_0 ? lane >> 2 : ir);
            const int64_t si = r0 + (FMT == FQ1_0 ? lane & 15 : lane >> 2);
            rp.w[wt] = a.qs + (wi < a.N ? wi : a.N - 1) * a.qs_row + (FMT == FQ1_0 ? 4 * (lane & 3) : 0);
            rp.sc[wt] = a.sc + (si < a.N ? si : a.N - 1) * a.sc_row;
        }
        return rp;
    };

    // loads of step s of tile t into ring slot `ring`.  x: chunk c = XPW wave + u of the stage is
    // row group c / 4, block c % 4.  Weights: lane (ir, lc) of row group g loads chunk 4 h + lc of
    // the step (chunks past the row its last chunk); Q1_0: the block's sign dword.  Scales: block
    // l % 4 of the step (dword 4 row + block of the scale area); Q1_0: the block's scale.  With a
    // tile's first step, the first BM / 64 waves also load its BM row factors.
    auto issue = [&](const Tile &t, const RowPtrs &rp, int s_rel, int ring, int rs_slot) {
        const int s = t.s0 + s_rel;
        uint8_t *st = lds + ring * G::BYTES;
        const _Float16 *xsrc = a.xh + (t.m0 / 16) * (int64_t)a.KBp * 512 + (int64_t)lane * 8;
#pragma unroll
        for (int u = 0; u < G::XPW; ++u) {
            const int c = G::XPW * wave + u;
            const _Float16 *src =
                xsrc + ((int64_t)(c / GM_BPS) * a.KBp + (int64_t)s * GM_BPS + c % GM_BPS) * 512;
            gm_dma16(src, st + c * 1024);
        }
        if constexpr (FMT == FQ1_0) {
#pragma unroll
            for (int wt = 0; wt < G::WPW; ++wt) {
                const int g = G::WPW * wave + wt;
                gm_dma4(rp.w[wt] + 16 * (uint32_t)s, st + G::XB + g * 256);
                gm_dma2(rp.sc[wt] + 2 * (uint32_t)s, st + G::XB + G::WB + g * 256);
            }
        } else {
            const int b0 = s * GM_BPS + (lane & 3);
            const int blk = b0 < KB ? b0 : KB - 1;
#pragma unroll
            for (int wt = 0; wt < G::WPW; ++wt) {
                const int g = G::WPW * wave + wt;                  // weight row group
#pragma unroll
                for (int h = 0; h < G::WH; ++h) {
                    const int ch0 = (s * G::WH + h) * 4 + lc;
                    const int ch = ch0 < C ? ch0 : C - 1;
                    gm_dma16(rp.w[wt] + 16 * (uint32_t)ch, st + G::XB + (g * G::WH + h) * 1024);
                }
                gm_dma2(rp.sc[wt] + 2 * (uint32_t)blk, st + G::XB + G::WB + g * 256);
            }
        }
        if (s_rel == 0 && wave < BM / 64)
            gm_dma4(a.rs + t.m0 + 64 * wave + lane, &s_rs[rs_slot][64 * wave]);
    };

    float acc[NBT][G::WPW][4];  // Q4_0, Q8_0: per-block scaled sums (VALU)
    mf4 macc[NBT][G::WPW];      // Q1_0: sums kept in the MFMA accumulators
    auto zero_acc = [&]() {
#pragma unroll
        for (int i = 0; i < NBT; ++i)
#pragma unroll
            for (int wt = 0; wt < G::WPW; ++wt) {
                acc[i][wt][0] = acc[i][wt][1] = acc[i][wt][2] = acc[i][wt][3] = 0.f;
                macc[i][wt] = mf4{0.f, 0.f, 0.f, 0.f};
            }
    };
    zero_acc();

    const MfConst kc = mf_const<FMT>();
    auto compute = [&](const Tile &t, int s_rel, int ring) {
        const int s = t.s0 + s_rel;
        const uint8_t *st = lds + ring * G::BYTES;
        if constexpr (FMT == FQ1_0) {
            // row ir of each of the wave's row groups: its four sign words and its scale; lane
            // column lc of block b takes the pairs (element 4 lc + p, element 4 lc + p + 16),
            // p = 0..3, as +-d: the sign bits moved to bits 15 and 31 (a set bit is +d), then
            // xor-ed into the f16 pair (d, d)
            uint4 qv[G::WPW];
            uint32_t dp[G::WPW];
#pragma unroll
            for (int wt = 0; wt < G::WPW; ++wt) {
                const int g = G::WPW * wave + wt;
                qv[wt] = *reinterpret_cast<const uint4 *>(st + G::XB + (16 * g + ir) * 16);
                const uint32_t db = *reinterpret_cast<const uint32_t *>(st + G::XB + G::WB +
                                                                       g * 256 + 4 * ir) & 0xFFFFu;
                dp[wt] = db | (db << 16);
            }
#pragma unroll
            for (int b = 0; b < GM_BPS; ++b) {
                mh8 A[NBT];
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt)
                    A[bt] = *reinterpret_cast<const mh8 *>(st + (bt * GM_BPS + b) * 1024 + 16 * lane);
#pragma unroll
                for (int wt = 0; wt < G::WPW; ++wt) {
                    const uint4 q4 = qv[wt];
                    const uint32_t w = ~(b == 0 ? q4.x : b == 1 ? q4.y : b == 2 ? q4.z : q4.w);
                    uint4 bw;
                    bw.x = (((w >> (4 * lc + 0)) << 15) & 0x80008000u) ^ dp[wt];
                    bw.y = (((w >> (4 * lc + 1)) << 15) & 0x80008000u) ^ dp[wt];
                    bw.z = (((w >> (4 * lc + 2)) << 15) & 0x80008000u) ^ dp[wt];
                    bw.w = (((w >> (4 * lc + 3)) << 15) & 0x80008000u) ^ dp[wt];
                    const mh8 B = __builtin_bit_cast(mh8, bw);
#pragma unroll
                    for (int bt = 0; bt < NBT; ++bt)
                        macc[bt][wt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[bt], B, macc[bt][wt], 0, 0, 0);
                }
            }
            (void)s;
            return;
        }
        // this wave's weights (row groups WPW wave + wt, loaded by this wave); after the transpose
        // q[wt][h][b'] is dword lc of chunk 4 h + b' of row ir
        uint32_t q[G::WPW][G::WH][4];
        uint4 dsc[G::WPW];
#pragma unroll
        for (int wt = 0; wt < G::WPW; ++wt) {
            const int g = G::WPW * wave + wt;
#pragma unroll
            for (int h = 0; h < G::WH; ++h) {
                const uint4 v = *reinterpret_cast<const uint4 *>(st + G::XB + (g * G::WH + h) * 1024 +
                                                                 16 * lane);
                q[wt][h][0] = v.x; q[wt][h][1] = v.y; q[wt][h][2] = v.z; q[wt][h][3] = v.w;
            }
            dsc[wt] = *reinterpret_cast<const uint4 *>(st + G::XB + G::WB + (16 * g + ir) * 16);
        }
#pragma unroll
        for (int wt = 0; wt < G::WPW; ++wt)
#pragma unroll
            for (int h = 0; h < G::WH; ++h)
                mf_xpose(q[wt][h]);
#pragma unroll
        for (int b = 0; b < GM_BPS; ++b) {
            const int blk = GM_BPS * s + b;
            mh8 A[NBT];
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt)
                A[bt] = *reinterpret_cast<const mh8 *>(st + (bt * GM_BPS + b) * 1024 + 16 * lane);
#pragma unroll
            for (int wt = 0; wt < G::WPW; ++wt) {
                const uint32_t dw = b == 0 ? dsc[wt].x : b == 1 ? dsc[wt].y : b == 2 ? dsc[wt].z : dsc[wt].w;
                // exact weights (Q4_0: q - 8, the high-nibble halves x16; Q8_0: q, block b being
                // chunks 2 b, 2 b + 1 of the step) in one product per block, D = A B with the
                // f32 sums of exact products, then acc += d D on the VALU, where it overlaps the
                // other wave's products
                const int h = FMT == FQ4_0 ? 0 : b >> 1, p = 2 * (b & 1);
                const mh8 B = FMT == FQ4_0 ? mf_bop<FMT>(q[wt][0][b], 0u, kc)
                                           : mf_bop<FMT>(q[wt][h][p], q[wt][h][p + 1], kc);
                const uint16_t db = (uint16_t)(dw & 0xFFFFu);
                const float d = blk < KB ? (float)__builtin_bit_cast(_Float16, db) : 0.f;
                const mf4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int bt = 0; bt < NBT; bt += 4) {
                    mf4 D[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        D[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[bt + i], B, zero, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[bt + i][wt][0] = fmaf(d, D[i][0], acc[bt + i][wt][0]);
                        acc[bt + i][wt][1] = fmaf(d, D[i][1], acc[bt + i][wt][1]);
                        acc[bt + i][wt][2] = fmaf(d, D[i][2], acc[bt + i][wt][2]);
                        acc[bt + i][wt][3] = fmaf(d, D[i][3], acc[bt + i][wt][3]);
                    }
                }
            }
        }
    };

    // lane (ir, lc) holds D[4 lc + v][ir] of tile (bt, wt): x row 16 bt + 4 lc + v, weight row
    // 16 (WPW wave + wt) + ir
    auto epilogue = [&](const Tile &t, int rs_slot) {
        const bool fold = a.splits > 1;
        float *out = fold ? a.part + (int64_t)t.split * a.M * a.N : a.y;
#pragma unroll
        for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
            for (int vv = 0; vv < 4; ++vv) {
                const int rl = 16 * bt + 4 * lc + vv;
                const int64_t r = t.m0 + rl;
                if (r >= a.M)
                    continue;
                const float f = fold ? 1.0f : s_rs[rs_slot][rl];
#pragma unroll
                for (int wt = 0; wt < G::WPW; ++wt) {
                    const int64_t n = t.n0 + 16 * (G::WPW * wave + wt) + ir;
                    const float v = FMT == FQ1_0 ? macc[bt][wt][vv] : acc[bt][wt][vv];
                    if (n < a.N)
                        out[r * a.N + n] = v * f;
                }
            }
    };

    // One stream of (tile, step) pairs per workgroup; the loads run STG - 1 steps ahead of the
    // compute, across tile boundaries (the next tile's first loads overlap this tile's last steps
    // and its stores).  Ring slot of stream position p: p % STG.
    constexpr int LPS = G::XPW + G::WPW * (G::WH + 1);   // loads per thread per step (+1 at a tile's start)
    int ik8 = slot, is = 0, itn = 0, pi = 0;  // issue cursor: tile, step, tile ordinal, position
    Tile ti = tile_of(ik8);
    RowPtrs rpi = row_ptrs(ti);
    auto issue_next = [&]() {
        if (ik8 >= ntiles)
            return;
        issue(ti, rpi, is, pi % G::STG, itn % 3);
        ++pi;
        if (++is == ti.S) {
            is = 0;
            ++itn;
            ik8 += nslots;
            if (ik8 < ntiles) {
                ti = tile_of(ik8);
                rpi = row_ptrs(ti);
            }
        }
    };
#pragma unroll
    for (int p = 0; p < G::STG - 1; ++p)
        issue_next();
    int ck8 = slot, cs = 0, ctn = 0, pc = 0;  // compute cursor
    Tile tc = tile_of(ck8);
    while (true) {
        // this thread's loads of position pc have landed (those of pc + 1 .. pc + STG - 2 may
        // still be in flight; the stores of a finished tile are waited for too), and after the
        // barrier everyone's have; every wave is also done reading position pc - 1, whose ring
        // slot the loads of pc + STG - 1 overwrite
        if (pi - pc >= G::STG - 1)
            gm_wait<LPS * (G::STG - 2)>();
        else
            gm_wait<0>();
        gm_barrier();
        issue_next();
        compute(tc, cs, pc % G::STG);
        ++pc;
        if (++cs == tc.S) {
            epilogue(tc, ctn % 3);
            zero_acc();
            cs = 0;
            ++ctn;
            ck8 += nslots;
            if (ck8 >= ntiles)
                break;
            tc = tile_of(ck8);
        }
    }
}

// y[r][n] = rs[r] (sum over the splits, in split order, of part[split][r][n])
__global__ __launch_bounds__(256) void k_gemm_fold(const float *part, const float *rs, int splits,
                                                   int64_t M, int64_t N, float *y)
{
    const int64_t total = M * N, stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
        float v = 0.f;
        for (int sp = 0; sp < splits; ++sp)
            v += part[sp * total + i];
        y[i] = v * rs[i / N];
    }
}

int launch_gemm(int fmt, const GemmArgs &a, const float *x, void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    // x preparation: one wave per row of the padded x, its pieces held in registers when there
    // are at most 512
    const unsigned groups = (unsigned)((int64_t)a.m_tiles * a.bm / 4);
    const int np = 4 * a.KBp;
    const int ppl = np <= 64 ? 1 : np <= 128 ? 2 : np <= 256 ? 4 : np <= 512 ? 8 : 0;
    using XP = void (*)(const float *, int64_t, int64_t, int, _Float16 *, float *);
    XP xp = nullptr;
    switch (ppl) {
    case 1: xp = fmt == FQ4_0 ? k_xprep<FQ4_0, 1> : fmt == FQ1_0 ? k_xprep<FQ1_0, 1> : k_xprep<FQ8_0, 1>; break;
    case 2: xp = fmt == FQ4_0 ? k_xprep<FQ4_0, 2> : fmt == FQ1_0 ? k_xprep<FQ1_0, 2> : k_xprep<FQ8_0, 2>; break;
    case 4: xp = fmt == FQ4_0 ? k_xprep<FQ4_0, 4> : fmt == FQ1_0 ? k_xprep<FQ1_0, 4> : k_xprep<FQ8_0, 4>; break;
    case 8: xp = fmt == FQ4_0 ? k_xprep<FQ4_0, 8> : fmt == FQ1_0 ? k_xprep<FQ1_0, 8> : k_xprep<FQ8_0, 8>; break;
    default: xp = fmt == FQ4_0 ? k_xprep<FQ4_0, 0> : fmt == FQ1_0 ? k_xprep<FQ1_0, 0> : k_xprep<FQ8_0, 0>; break;
    }
    hipLaunchKernelGGL(xp, dim3(groups), dim3(256), 0, s, x, a.M, a.K, a.KBp, a.xh, a.rs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return (int)e;
    // persistent: at most one workgroup per compute unit (the LDS ring takes most of a CU), 32 per
    // XCD, each walking its XCD's tiles
    const int per_xcd = ((a.n_tiles + 7) / 8) * a.m_tiles * a.splits;
    const int grid = 8 * (per_xcd < 32 ? per_xcd : 32);
    void (*kern)(GemmArgs) = nullptr;
    if (a.bm == 64) {
        if (fmt == FQ4_0)
            kern = a.bn == 256 ? k_gemm<FQ4_0, 2, 64> : k_gemm<FQ4_0, 1, 64>;
        else if (fmt == FQ1_0)
            kern = a.bn == 256 ? k_gemm<FQ1_0, 2, 64> : k_gemm<FQ1_0, 1, 64>;
        else
            kern = a.bn == 256 ? k_gemm<FQ8_0, 2, 64> : k_gemm<FQ8_0, 1, 64>;
    } else {
        if (fmt == FQ4_0)
            kern = a.bn == 512 ? k_gemm<FQ4_0, 4, 128>
                 : a.bn == 256 ? k_gemm<FQ4_0, 2, 128> : k_gemm<FQ4_0, 1, 128>;
        else if (fmt == FQ1_0)
            kern = a.bn == 256 ? k_gemm<FQ1_0, 2, 128> : k_gemm<FQ1_0, 1, 128>;
        else
            kern = a.bn == 256 ? k_gemm<FQ8_0, 2, 128> : k_gemm<FQ8_0, 1, 128>;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(GM_THREADS), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1)
        return (int)e;
    const int64_t total = a.M * a.N;
    const int64_t fg = (total + 255) / 256 < 2048 ? (total + 255) / 256 : 2048;
    hipLaunchKernelGGL(k_gemm_fold, dim3((unsigned)fg), dim3(256), 0, s, a.part, a.rs, a.splits,
                       a.M, a.N, a.y);
    return (int)hipGetLastError();
}

}  // namespace qg

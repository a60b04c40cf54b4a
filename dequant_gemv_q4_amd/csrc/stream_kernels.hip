// stream_kernels.hip -- instantiations and launchers of the streaming dequant-GEMV kernels for the
// Q4_0, Q8_0 and Q4_K formats, the argmax fold, the routed-expert kernels, the fixed scratch of the
// no-allocation entry point and the occupancy queries.
#include "stream_impl.h"

#include <mutex>
#include <vector>

namespace qg {

// idx[r] from the per-workgroup partial keys [n_part][nb] of an argmax launch (one workgroup of
// 16 waves, one batch row per wave).  A lane's keys are loaded eight at a time, all issued before
// the first compare, so a row of up to 512 partial keys costs one memory latency.
__global__ __launch_bounds__(1024) void k_argmax_fold(const unsigned long long *part, int n_part,
                                                      int nb, int32_t *idx)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int r = wave; r < nb; r += 16) {
        unsigned long long k = 0ull;
        for (int b0 = lane; b0 < n_part; b0 += 64 * 8) {
            unsigned long long o[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int b = b0 + 64 * u;
                o[u] = b < n_part ? part[(int64_t)b * nb + r] : 0ull;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                k = o[u] > k ? o[u] : k;
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

// Routed experts.  The (row, slot) pairs of the routing table are grouped by expert (ascending
// id; pairs in (row, slot) order) into sets of at most NBX pairs; set s multiplies the N x K
// matrix of its expert e_s by the x rows of its pairs.  The row groups of all sets, laid end to
// end (set s owns virtual groups [s GS, (s + 1) GS)), are cut into equal contiguous ranges, one
// per workgroup, so that every workgroup streams the same number of weight bytes whatever the
// routing.  The host launches at least as many workgroups as there are pairs, so a range
// touches at most two sets; their x rows are staged in LDS by loader waves while the other
// waves issue their first weight loads.  Waves then claim the range's groups from an LDS
// counter (as in the GEMV kernels) and keep the x pairs of the set they are in, reloading them
// when a claim crosses into the second set.  Results collect in LDS and leave in one pass to
// part[pair][n]; k_moe_combine then forms y[r][n] = sum_t wts[r][t] part[r][t][n], t ascending.
template <int FMT, int CPL, int PD>
__global__ __launch_bounds__(moe_threads(FMT, CPL, PD))
__attribute__((amdgpu_waves_per_eu(moe_threads(FMT, CPL, PD) / 256)))
void k_moe(MoeArgs a)
{
    constexpr int NBX = 4 / CPL;                  // x rows a wave holds in registers
    constexpr int R = stream_rows(NBX, CPL, 1);
    constexpr int ITX = R * NBX, IPX = pow2_ceil(ITX);
    constexpr int LG = IPX == 1 ? 0 : IPX == 2 ? 1 : IPX == 4 ? 2 : IPX == 8 ? 3 : 4;
    constexpr int NT = moe_threads(FMT, CPL, PD), WV = NT / 64;
    constexpr int XPL = 8;   // float4s in flight per loader lane while a row is copied
    extern __shared__ float4 lds4[];
    __shared__ int s_pair[QG_PAIRS_MAX][NBX];
    __shared__ int s_e[QG_PAIRS_MAX], s_nb[QG_PAIRS_MAX];
    __shared__ int s_wsum[WV];
    __shared__ float s_rs[2 * NBX];   // factor undoing each staged row's scale
    __shared__ int s_next, s_xcnt;

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int P = a.nb * a.topk;
    const int C = (int)(a.qs_row / 16), K4 = (int)(a.K / 4);
    const int N = (int)a.N, E = (int)a.n_exp;
    // [E][4] per-expert masks of the pairs (bit t of the 128), then [E] set bases and counts
    uint32_t *pmask = reinterpret_cast<uint32_t *>(lds4);
    int *hist = reinterpret_cast<int *>(pmask + 4 * E);

    // 1. the sets.  Every workgroup builds the same sets: each expert's pairs are marked in a
    // bit mask (the order of the atomic ors does not matter), a pair's rank among its expert's
    // pairs is the number of lower pair indices in the mask, an exclusive scan over the experts
    // of ceil(count / NBX) places each expert's sets, and every pair goes into its set in rank
    // order.
    for (int e = t; e < 4 * E; e += NT)
        pmask[e] = 0u;
    if (t == 0) {
        s_next = PD * WV;
        s_xcnt = 0;
    }
    __syncthreads();
    int id = -1;
    if (t < P) {
        id = a.ids[t];
        if (id < 0 || id >= E) {
            if (blockIdx.x == 0)
                atomicOr(a.err, 1u);
            id = -1;
        } else {
            atomicOr(&pmask[4 * id + (t >> 5)], 1u << (t & 31));
        }
    }
    __syncthreads();
    int cnt[4], csum = 0;   // thread t scans experts [4t, 4t + 4)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int e = 4 * t + k;
        cnt[k] = 0;
        if (e < E) {
            const uint4 m = reinterpret_cast<const uint4 *>(pmask)[e];
            cnt[k] = __popc(m.x) + __popc(m.y) + __popc(m.z) + __popc(m.w);
        }
        csum += (cnt[k] + NBX - 1) / NBX;
    }
    int inc = csum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(inc, off);
        inc += lane >= off ? v : 0;
    }
    if (lane == 63)
        s_wsum[wave] = inc;
    __syncthreads();
    int run = inc - csum, n_sets = 0;
    for (int w = 0; w < WV; ++w) {
        run += w < wave ? s_wsum[w] : 0;
        n_sets += s_wsum[w];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int e = 4 * t + k;
        if (e < E)
            hist[e] = (run << 8) | cnt[k];   // first set of expert e, its pair count (<= 128)
        run += (cnt[k] + NBX - 1) / NBX;
    }
    __syncthreads();
    if (id >= 0) {
        int rank = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t m = pmask[4 * id + w];
            const int lo = t - 32 * w;   // pairs below t in this word
            rank += lo >= 32 ? __popc(m) : lo > 0 ? __popc(m & ((1u << lo) - 1u)) : 0;
        }
        const int h = hist[id];
        const int set = (h >> 8) + rank / NBX, pos = rank % NBX;
        s_pair[set][pos] = t;
        if (pos == 0) {
            s_e[set] = id;
            s_nb[set] = (h & 255) - rank < NBX ? (h & 255) - rank : NBX;
        }
    }
    __syncthreads();

    // Every value below is the same in all lanes; divisions and LDS reads produce it in vector
    // registers, and readfirstlane makes it scalar again, so that the branches on it stay scalar
    // and the buffer resources built from it need no per-lane loop.  V < 2^31 (checked by the host).
    auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
    const int GS = (N + R - 1) / R;
    const int64_t V = (int64_t)uni(n_sets) * GS;
    const int v0 = uni((int)(V * blockIdx.x / gridDim.x));
    const int v1 = uni((int)(V * (blockIdx.x + 1) / gridDim.x));
    int L = v1 - v0;
    const int s0 = L > 0 ? uni(v0 / GS) : 0;
    const int s1 = L > 0 ? uni((v1 - 1) / GS) : 0;
    if (L > a.pool_max || s1 > s0 + 1) {   // outside the launch's contract: flag, do nothing
        if (t == 0)
            atomicOr(a.err, 2u);
        L = 0;
    }
    L = uni(L);
    const int nb0 = L > 0 ? uni(s_nb[s0]) : 0;
    const int nb1 = L > 0 && s1 > s0 ? uni(s_nb[s1]) : 0;
    const int j0 = v0 - s0 * GS;                    // group of set s0 at local index 0
    const int b1 = GS - j0;                         // local index where set s0 + 1 starts
    // local group gl: set (0 or 1, -1 past the range) and group within the set
    auto locate = [&](int gl, int &ls, int &j) {
        ls = gl >= L ? -1 : gl < b1 ? 0 : 1;
        j = ls < 0 ? -1 : ls == 0 ? gl + j0 : gl - b1;
    };

    // Staged x: staged row q = ls * NBX + r is row r of set s0 + ls.  Loader wave q copies its
    // row to LDS (raw, in X4[q]), takes the row's largest |value| on the way, and converts the
    // chunk slots of each lane to f16 pairs and offset sums once, in XP[q][slot][k][lane]
    // (uint4 k < NP / 4: pairs; k = NP / 4: the sums); the waves entering a set then only read
    // them.  The results pool reuses the raw rows' space (no result is written before every
    // loader has finished).
    constexpr int NP = XH<FMT, NBX, CPL>::NP, NZ = XH<FMT, NBX, CPL>::NZ, NQ4 = NP / 4 + 1;
    static_assert(2 * NBX <= WV, "one loader wave per staged row");
    uint4 *XP = reinterpret_cast<uint4 *>(lds4 + E + (E + 3) / 4);
    float4 *X4 = reinterpret_cast<float4 *>(XP + (size_t)2 * NBX * CPL * NQ4 * 64);
    float *s_out = reinterpret_cast<float *>(X4);   // [pool][ITX] results, item r * R + u
    const int xw = nb0 + nb1;
    const bool xloader = wave < xw;

    // the two experts' matrices (one buffer resource each: every plane is under 2 GiB)
    const int64_t eqb = a.N * a.qs_row, esb = a.N * a.sc_row;
    const int64_t e0 = L > 0 ? uni(s_e[s0]) : 0;
    const int64_t e1 = L > 0 && s1 > s0 ? uni(s_e[s1]) : e0;
    const LaneOff<CPL> lo = lane_offsets<FMT, CPL>(lane, C);
    const RowB rw{(uint32_t)a.qs_row, (uint32_t)a.sc_row, 0u, 0u};
    const int bp32 = (lane ^ 32) << 2;

    GroupBuf<FMT, CPL, 1, R> buf[PD];
    int gcur[PD];
    auto load = [&](int p, int gl) {
        int ls, j;
        locate(gl, ls, j);
        const int64_t e = uni((int)(ls == 1 ? e1 : e0));
        const BufMat m[1] = {buf_mat(a.qs + e * eqb, a.sc + e * esb, (uint32_t)eqb, (uint32_t)esb)};
        load_group(buf[p], m, rw, a.N, lo, j);
    };
    auto issue_first = [&]() {
#pragma unroll
        for (int p = 0; p < PD; ++p) {
            gcur[p] = p * WV + wave;
            load(p, gcur[p]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (!xloader)
        issue_first();
    if (xloader) {
        const int ls = wave < nb0 ? 0 : 1, r = ls ? wave - nb0 : wave, q = ls * NBX + r;
        const float4 *xs = reinterpret_cast<const float4 *>(a.x) +
                           (int64_t)(s_pair[s0 + ls][r] / a.topk) * K4;
        float4 *xq = X4 + (size_t)q * K4;
        float mx = 0.f;
        for (int e0 = 0; e0 < K4; e0 += 64 * XPL) {
            float4 v[XPL];
#pragma unroll
            for (int i = 0; i < XPL; ++i) {
                const int e = e0 + 64 * i + lane;
                v[i] = xs[e < K4 ? e : K4 - 1];
            }
#pragma unroll
            for (int i = 0; i < XPL; ++i) {
                const int e = e0 + 64 * i + lane;
                if (e < K4)
                    xq[e] = v[i];
                mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)),
                                     fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
            }
        }
        mx = fmaxf(mx, xor_lane<32>(mx, bp32));
        mx = fmaxf(mx, xor_lane<16>(mx, bp32));
        mx = fmaxf(mx, xor_lane<8>(mx, bp32));
        mx = fmaxf(mx, xor_lane<4>(mx, bp32));
        mx = fmaxf(mx, xor_lane<2>(mx, bp32));
        mx = fmaxf(mx, xor_lane<1>(mx, bp32));
        int e2 = 0;
        frexpf(mx, &e2);                                // max |x| = f 2^e2, f in [0.5, 1)
        const int sk = 15 - e2 < 127 ? 15 - e2 : 127;   // 2^sk stays a finite f32
        const float sc = ldexpf(1.0f, sk);
        if (lane == 0)
            s_rs[q] = ldexpf(1.0f, -sk);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            const int cx = c < C ? c : C - 1;
            float4 xv[Fc<FMT>::XF4];
#pragma unroll
            for (int j = 0; j < Fc<FMT>::XF4; ++j)
                xv[j] = xq[chunk_elem<FMT>(cx, j) / 4];
            uint32_t pp[NP];
            float zz[NZ];
            x_pairs<FMT>(xv, sc, pp, zz);
            uint4 *dst = XP + (size_t)(q * CPL + i) * NQ4 * 64 + lane;
#pragma unroll
            for (int k = 0; k < NP / 4; ++k)
                dst[k * 64] = make_uint4(pp[4 * k], pp[4 * k + 1], pp[4 * k + 2], pp[4 * k + 3]);
            uint4 zq = make_uint4(0u, 0u, 0u, 0u);
            zq.x = __float_as_uint(zz[0]);
            if constexpr (NZ == 2)
                zq.y = __float_as_uint(zz[1]);
            dst[(NP / 4) * 64] = zq;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        if (lane == 0)
            __hip_atomic_fetch_add(&s_xcnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        issue_first();
    }
    while (__hip_atomic_load(&s_xcnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < xw)
        __builtin_amdgcn_s_sleep(1);
    asm volatile("" ::: "memory");

    XH<FMT, NBX, CPL> xh;
    const WConst wk = w_const<FMT>();
    int cur = -1, nbc = 0;
    float my_rs = 1.f;
    const int my_item = lane >> (6 - LG);
    const int my_u = my_item / NBX, my_r = my_item % NBX;
    const bool writer = (lane & ((64 >> LG) - 1)) == 0 && my_item < ITX;

    if (gcur[0] < L) {
        for (;;) {
#pragma unroll
            for (int p = 0; p < PD; ++p) {
                const int gl = gcur[p];
                float acc[IPX][1];
                if (gl < L) {
                    int ls, j;
                    locate(gl, ls, j);
                    if (ls != cur) {   // entering a set: its x pairs and row scales
                        cur = uni(ls);
                        nbc = uni(ls == 0 ? nb0 : nb1);
#pragma unroll
                        for (int r = 0; r < NBX; ++r)
                            if (r < nbc)
#pragma unroll
                                for (int i = 0; i < CPL; ++i) {
                                    const uint4 *src =
                                        XP + (size_t)((ls * NBX + r) * CPL + i) * NQ4 * 64 + lane;
#pragma unroll
                                    for (int k = 0; k < NP / 4; ++k) {
                                        const uint4 v = src[k * 64];
                                        xh.p[r][i][4 * k] = v.x;
                                        xh.p[r][i][4 * k + 1] = v.y;
                                        xh.p[r][i][4 * k + 2] = v.z;
                                        xh.p[r][i][4 * k + 3] = v.w;
                                    }
                                    const uint4 zq = src[(NP / 4) * 64];
                                    xh.z[r][i][0] = __uint_as_float(zq.x);
                                    if constexpr (NZ == 2)
                                        xh.z[r][i][1] = __uint_as_float(zq.y);
                                }
                        my_rs = s_rs[ls * NBX + (my_r < nbc ? my_r : 0)];
                    }
                    if (nbc == 1) {
                        compute_group_h<FMT, 1, CPL, 1, R, IPX, NBX>(buf[p], xh, wk, C, lane, acc);
                    } else if constexpr (NBX >= 2) {
                        if (nbc == 2)
                            compute_group_h<FMT, 2, CPL, 1, R, IPX, NBX>(buf[p], xh, wk, C, lane, acc);
                        else if constexpr (NBX >= 4) {
                            if (nbc == 3)
                                compute_group_h<FMT, 3, CPL, 1, R, IPX, NBX>(buf[p], xh, wk, C, lane, acc);
                            else
                                compute_group_h<FMT, 4, CPL, 1, R, IPX, NBX>(buf[p], xh, wk, C, lane, acc);
                        }
                    }
                }
                int nx = 0;
                if (lane == 0)
                    nx = atomicAdd(&s_next, 1);
                nx = __builtin_amdgcn_readfirstlane(nx);
                load(p, nx);
                if (gl < L) {
                    xpose_reduce<IPX, 1>(acc, lane, bp32);
                    if (writer && my_r < nbc)
                        s_out[gl * ITX + my_r * R + my_u] = acc[0][0] * my_rs;
                }
                gcur[p] = nx;
            }
            if (gcur[0] >= L)
                break;
        }
    }

    // 3. results to part[pair][n], contiguous in n for each (set, row) run
    __syncthreads();
    const int LR = L * R;
    for (int i = t; i < NBX * LR; i += NT) {
        const int r = i / LR, rem = i - r * LR;
        const int gl = rem / R, u = rem - gl * R;
        int ls, j;
        locate(gl, ls, j);
        const int n = j * R + u;
        if (r < (ls == 0 ? nb0 : nb1) && n < N) {
            const int pair = s_pair[s0 + ls][r];
            a.part[(int64_t)pair * N + n] = s_out[gl * ITX + r * R + u];
        }
    }
}

// y[r][n] = sum_t wts[r][t] part[r][t][n], t ascending, skipping out-of-range expert ids.  A
// thread forms four consecutive n of one row; every part load is issued before the first add
// (a load under the id test would wait for the one before it).
__global__ __launch_bounds__(256) void k_moe_combine(const float *part, const int32_t *ids,
                                                     const float *wts, int nb, int topk,
                                                     int64_t n_exp, int64_t N, float *y)
{
    const int64_t N4 = (N + 3) / 4;
    const int64_t f = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (f >= (int64_t)nb * N4)
        return;
    const int r = (int)(f / N4);
    const int64_t n0 = (f - r * N4) * 4;
    float4 v[QG_MAX_TOPK];
    bool ok[QG_MAX_TOPK];
    float w[QG_MAX_TOPK];
#pragma unroll
    for (int t = 0; t < QG_MAX_TOPK; ++t) {
        const int tt = t < topk ? t : 0;
        const int32_t id = ids[r * topk + tt];
        ok[t] = t < topk && id >= 0 && id < n_exp;
        w[t] = wts[r * topk + tt];
        const float *pr = part + ((int64_t)r * topk + tt) * N;
        if (n0 + 3 < N && (N & 3) == 0) {
            v[t] = *reinterpret_cast<const float4 *>(pr + n0);
        } else {
            v[t].x = pr[n0];
            v[t].y = pr[n0 + 1 < N ? n0 + 1 : n0];
            v[t].z = pr[n0 + 2 < N ? n0 + 2 : n0];
            v[t].w = pr[n0 + 3 < N ? n0 + 3 : n0];
        }
    }
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int t = 0; t < QG_MAX_TOPK; ++t) {
        if (ok[t]) {
            acc.x = fmaf(w[t], v[t].x, acc.x);
            acc.y = fmaf(w[t], v[t].y, acc.y);
            acc.z = fmaf(w[t], v[t].z, acc.z);
            acc.w = fmaf(w[t], v[t].w, acc.w);
        }
    }
    float *yr = y + (int64_t)r * N;
    if (n0 + 3 < N && (N & 3) == 0) {
        *reinterpret_cast<float4 *>(yr + n0) = acc;
    } else {
        yr[n0] = acc.x;
        if (n0 + 1 < N) yr[n0 + 1] = acc.y;
        if (n0 + 2 < N) yr[n0 + 2] = acc.z;
        if (n0 + 3 < N) yr[n0 + 3] = acc.w;
    }
}

static StreamFn stream_fn(int fmt, int epi, bool nrm, int ks, int nb, int pd)
{
    if (fmt_hbits(fmt) || fmt_generic(fmt)) {
        const void *fn = nullptr;
        int threads = 0;
        if (fmt_hbits(fmt))
            stream_fn_x(fmt, epi, nrm, ks, nb, pd, &fn, &threads);
        else
            stream_fn_g(fmt, epi, nrm, ks, nb, pd, &fn, &threads);
        return {fn, threads};
    }
    return fmt == FQ4_0 ? stream_fn_fmt<FQ4_0>(epi, nrm, ks, nb, pd)
         : fmt == FQ8_0 ? stream_fn_fmt<FQ8_0>(epi, nrm, ks, nb, pd)
         : fmt == FQ4_K ? stream_fn_fmt<FQ4_K>(epi, nrm, ks, nb, pd) : StreamFn{nullptr, 0};
}

int launch_stream(int fmt, int epi, bool nrm, int cpl, int pd, const GemvArgs &a, int grid,
                  size_t lds_bytes, void *stream)
{
    const StreamFn f = stream_fn(fmt, epi, nrm, cpl, a.nb, pd);
    if (!f.fn)
        return (int)hipErrorInvalidValue;
    void *args[] = {const_cast<GemvArgs *>(&a)};
    return (int)hipLaunchKernel(f.fn, dim3(grid), dim3(f.threads), args, lds_bytes,
                                static_cast<hipStream_t>(stream));
}

template <int FMT>
static const void *moe_fn_fmt(int cpl, int pd)
{
    switch (cpl * 8 + pd) {
    case 1 * 8 + 2: return reinterpret_cast<const void *>(&k_moe<FMT, 1, 2>);
    case 1 * 8 + 4: return reinterpret_cast<const void *>(&k_moe<FMT, 1, 4>);
    case 2 * 8 + 2: return reinterpret_cast<const void *>(&k_moe<FMT, 2, 2>);
    case 2 * 8 + 4: return reinterpret_cast<const void *>(&k_moe<FMT, 2, 4>);
    case 4 * 8 + 2: return reinterpret_cast<const void *>(&k_moe<FMT, 4, 2>);
    case 4 * 8 + 4:   // Q4_K would spill
        if constexpr (FMT != FQ4_K)
            return reinterpret_cast<const void *>(&k_moe<FMT, 4, 4>);
        return nullptr;
    default: return nullptr;
    }
}

static const void *moe_fn(int fmt, int cpl, int pd)
{
    return fmt == FQ4_0 ? moe_fn_fmt<FQ4_0>(cpl, pd)
         : fmt == FQ8_0 ? moe_fn_fmt<FQ8_0>(cpl, pd)
         : fmt == FQ4_K ? moe_fn_fmt<FQ4_K>(cpl, pd) : nullptr;
}

int launch_moe(int fmt, int cpl, int pd, const MoeArgs &a, int grid, size_t lds_bytes,
               void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    const void *fn = moe_fn(fmt, cpl, pd);
    if (!fn)
        return (int)hipErrorInvalidValue;
    void *args[] = {const_cast<MoeArgs *>(&a)};
    const hipError_t err = hipLaunchKernel(fn, dim3(grid), dim3(moe_threads(fmt, cpl, pd)), args,
                                           lds_bytes, s);
    if (err != hipSuccess)
        return (int)err;
    const int64_t quads = (int64_t)a.nb * ((a.N + 3) / 4);
    hipLaunchKernelGGL(k_moe_combine, dim3((int)((quads + 255) / 256)), dim3(256), 0, s, a.part,
                       a.ids, a.wts, a.nb, a.topk, a.n_exp, a.N, a.y);
    return (int)hipGetLastError();
}

// The fixed scratch of the no-allocation argmax entry point: one partial key per workgroup and
// batch row at the largest grid and batch an argmax launch may have (512 KiB per device, held
// until the process ends).  Host code never passes the array's name to a kernel: on the host it
// is a stand-in, not a device address; noalloc_scratch looks the device address up once per
// device and every launch takes that pointer.
static __device__ __align__(256) unsigned long long scratch[QG_ARGMAX_MAX_GRID * QG_MAX_NB];

int noalloc_scratch(void **ptr, size_t *bytes)
{
    constexpr int kMaxDev = 64;
    static std::mutex mu;
    static void *dev_ptr[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev)
        return -1;
    std::lock_guard<std::mutex> lk(mu);
    if (!dev_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return -1;
        dev_ptr[dev] = p;
    }
    *ptr = dev_ptr[dev];
    *bytes = sizeof(scratch);
    return 0;
}

int launch_argmax_fold(const unsigned long long *part, int n_part, int nb, int32_t *idx,
                       void *stream)
{
    hipLaunchKernelGGL(k_argmax_fold, dim3(1), dim3(1024), 0, static_cast<hipStream_t>(stream),
                       part, n_part, nb, idx);
    return (int)hipGetLastError();
}

// ------------------------------------------------------------------------------------ occupancy

// Workgroups of this streaming variant that fit on the device at once with lds_bytes of dynamic
// LDS (0 if it does not fit at all or the query fails), and its waves per workgroup.  Cached per
// device and variant.
// Workgroups of kernel fn (threads per workgroup, dynamic LDS bytes) resident at once on the
// current device, cached per (kernel, device, LDS size); 0 if the query fails or LDS is too big.
static int resident_wgs(const void *fn, int threads, size_t lds_bytes)
{
    int dev = 0;
    if (!fn || hipGetDevice(&dev) != hipSuccess)
        return 0;
    struct Entry {
        const void *fn;
        int dev;
        size_t lds;
        int resident;
    };
    static std::mutex mu;
    static std::vector<Entry> cache;
    {
        std::lock_guard<std::mutex> lk(mu);
        for (const Entry &e : cache)
            if (e.fn == fn && e.dev == dev && e.lds == lds_bytes)
                return e.resident;
    }
    int cus = 0, per_cu = 0, max_lds = 0;
    hipFuncAttributes attr;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess ||
        hipFuncGetAttributes(&attr, fn) != hipSuccess)
        return 0;
    int resident = 0;
    if (attr.sharedSizeBytes + lds_bytes <= (size_t)max_lds &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds_bytes) ==
            hipSuccess)
        resident = cus * per_cu;
    std::lock_guard<std::mutex> lk(mu);
    cache.push_back({fn, dev, lds_bytes, resident});
    return resident;
}

int stream_resident_wgs(int fmt, int epi, bool nrm, int cpl, int nb, int pd, size_t lds_bytes,
                        int *waves)
{
    const StreamFn f = stream_fn(fmt, epi, nrm, cpl, nb, pd);
    if (!f.fn)
        return 0;
    *waves = f.threads / 64;
    return resident_wgs(f.fn, f.threads, lds_bytes);
}

int moe_resident_wgs(int fmt, int cpl, int pd, size_t lds_bytes)
{
    return resident_wgs(moe_fn(fmt, cpl, pd), moe_threads(fmt, cpl, pd), lds_bytes);
}

}  // namespace qg

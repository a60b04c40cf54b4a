// abi.cpp -- the C ABI of libqgemv: argument validation, launch planning, workspace sizing.
//
// Every entry point validates all of its arguments on the host before it launches anything, so a
// failed check returns a status and leaves the stream untouched.  The planner is a pure function
// of (format, N, K, nb, op): tile length in K, lanes per row, rows per workgroup step and grid.
#include <hip/hip_runtime.h>

#include <string.h>

#include <mutex>
#include <unordered_map>

#include "../../include/qgemv.h"
#include "qgemv_internal.h"

#ifndef QG_BUF_MAX
#define QG_BUF_MAX (1LL << 31)     // largest plane the buffer-addressed kernels take
#endif
#ifndef QG_MFMA_MIN_NB
#define QG_MFMA_MIN_NB 5          // batch rows from which the matrix-core kernel takes a call
#endif
#ifndef QG_POOL_LDS
#define QG_POOL_LDS 32768         // most LDS bytes of results one streaming workgroup holds
#endif
#ifndef QG_MAX_GRID
#define QG_MAX_GRID 1024          // workgroups of the grid-stride GEMV kernels
#endif
#ifndef QG_LDS_BUDGET
#define QG_LDS_BUDGET (64 * 1024)  // staged x bytes per workgroup (two workgroups per CU fit)
#endif

namespace qg {

static int64_t round256(int64_t v) { return (v + 255) / 256 * 256; }

bool fmt_valid(int fmt)
{
    return fmt == FQ4_0 || fmt == FQ5_0 || fmt == FQ8_0 || fmt == FQ4_K || fmt == FQ5_K ||
           fmt == FQ6_K || fmt_generic(fmt);
}

// Packed layout: the quant plane (nibbles, or Q8_0 bytes), the scale plane (f16 d per 32, or the
// 16-byte Q4_K / Q5_K header, or the 16 signed Q6_K scales per 256), then for the high-bit
// formats a plane of the fifth (sixth) bits re-laid per 32 weights, and for Q6_K a plane of its
// f16 d per 256.  Each plane starts 256-B aligned; the bytes per weight equal GGUF's.
bool layout(int fmt, int64_t N, int64_t K, Layout *L)
{
    if (!fmt_valid(fmt) || N < 1 || K < 1)
        return false;
    const int bw = (fmt_super(fmt) || fmt == FIQ4_XS) ? 256 : fmt == FQ1_0 ? 128 : 32;
    const int bb = fmt == FQ4_0 ? 18 : fmt == FQ5_0 ? 22 : fmt == FQ8_0 ? 34 : fmt == FQ4_K ? 144
                 : fmt == FQ5_K ? 176 : fmt == FQ6_K ? 210 : fmt == FIQ4_NL ? 18
                 : fmt == FIQ4_XS ? 136 : fmt == FQ1_0 ? 18 : 20;
    if (K % bw != 0 || K > QG_MAX_K)
        return false;
    L->block_w = bw;
    L->block_b = bb;
    L->qs_row = fmt == FQ8_0 ? K : fmt == FQ1_0 ? K / 8 : K / 2;
    // scale bytes per row: f16 d per 32 (K/16), IQ4_XS's 8-byte header per 256 (K/32), Q1_0's
    // f16 d per 128 (K/64), the affine format's f16 scale and bias per 32 (K/8)
    L->sc_row = fmt == FIQ4_XS ? K / 32 : fmt == FQ1_0 ? K / 64 : fmt == FAQ4 ? K / 8 : K / 16;
    L->hb_row = fmt == FQ6_K ? K / 4 : fmt_hbits(fmt) ? K / 8 : 0;
    L->d_row = fmt == FQ6_K ? K / 128 : 0;
    L->sc_off = round256(N * L->qs_row);
    L->hb_off = L->sc_off + round256(N * L->sc_row);
    L->d_off = L->hb_off + round256(N * L->hb_row);
    L->cb_off = L->d_off + round256(N * L->d_row);
    L->total = L->cb_off + (fmt_codebook(fmt) ? 256 : 0);
    L->gguf_row = K / bw * bb;
    return true;
}

struct Plan {
    int lpr_log2, kt, n_kt, rows_per_step;
    int64_t n_steps;
    int grid;
    size_t lds;
};

// Tile length: the whole row if its staged x fits the LDS budget, else the smallest number of
// equal tiles (each a multiple of the format's tile granularity) that fits.
static bool plan_tiles(int fmt, int64_t K, int nb, Plan *p)
{
    const FmtFacts F = fmt_facts(fmt);
    for (int64_t n_kt = 1; n_kt <= K / F.tile_align; ++n_kt) {
        if (K % n_kt || (K / n_kt) % F.tile_align)
            continue;
        const int kt = (int)(K / n_kt);
        if (lds_tile_bytes(fmt, nb, kt) <= (size_t)QG_LDS_BUDGET) {
            p->kt = kt;
            p->n_kt = (int)n_kt;
            p->lds = lds_tile_bytes(fmt, nb, kt);
            const int ct = kt / F.ce;
            int lpr = 1;
            while (lpr < 64 && ct % (2 * lpr) == 0)
                lpr *= 2;   // largest power of two dividing ct, at most 64
            int lg = 0;
            while ((1 << lg) < lpr)
                ++lg;
            p->lpr_log2 = lg;
            return true;
        }
    }
    return false;
}

static bool plan_gemv(int fmt, int64_t N, int64_t K, int nb, int mats, Plan *p)
{
    if (!plan_tiles(fmt, K, nb, p))
        return false;
    const int G = 64 >> p->lpr_log2;
    p->rows_per_step = 4 * rows_in_flight(nb, mats) * G;
    p->n_steps = (N + p->rows_per_step - 1) / p->rows_per_step;
    p->grid = (int)(p->n_steps < QG_MAX_GRID ? p->n_steps : QG_MAX_GRID);
    return true;
}

// Streaming path (whole wave per row, x in registers): nb <= 4 and at most 4 chunks of 16 bytes
// per lane and row (longer rows are split over up to four waves).  Returns the chunks-per-row
// class (1, 2, 4 = waves per row), or 0.
static int stream_cpl(int fmt, int64_t K, int nb)
{
    if (nb > 4)
        return 0;
    const int64_t C = fmt == FQ8_0 ? K / 16 : K / 32;   // lane chunks per row
    return C <= 64 ? 1 : C <= 128 ? 2 : C <= 256 ? 4 : 0;
}

struct StreamPlan {
    int cpl;     // waves a row's K is split over
    int pd;      // row groups in flight per wave
    int tg_log2; // log2 of the row groups per tile
    int grid;
    size_t lds;
};

static bool plan_stream(int fmt, int epi, bool nrm, int64_t N, int64_t K, int nb, StreamPlan *sp)
{
    const int cpl = stream_cpl(fmt, K, nb);
    if (!cpl)
        return false;
    const int mats = epi == E_GUS ? 2 : 1;
    const int R = stream_rows_fmt(fmt, nb, 1, mats);
    const int64_t groups = (N + R - 1) / R;
    const int64_t items = (int64_t)R * nb;            // results per row group
    // tiles of up to QG_TILE_GROUPS groups, smaller when that leaves CUs without a tile
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return false;
    int tgl = 0;
    while ((1 << (tgl + 1)) <= QG_TILE_GROUPS && (groups >> (tgl + 1)) >= cus)
        ++tgl;
    sp->tg_log2 = tgl;
    const int64_t TGr = (int64_t)1 << tgl;
    const int64_t n_tiles = (groups + TGr - 1) / TGr;
    // LDS: x of the nb rows (norm: x * gamma; and one f32 square sum per 4), then the results
    // of the workgroup's pool of row groups
    const size_t x_lds = (size_t)nb * K * 4 + (nrm ? (size_t)nb * K : 0);
    sp->cpl = cpl;
    // The deepest prefetch whose own grid (one pass of resident workgroups) still gives every
    // team that many groups.  Each variant has its own register use, hence its own residency.
    const int pd_max = nb == 1 ? QG_PD_MAX : 2;
    for (int pd = pd_max; pd >= 1; pd /= 2) {
        int waves = 0;
        // residency with the largest pool this grid could need (results of pool_max groups)
        int resident = stream_resident_wgs(fmt, epi, nrm, cpl, nb, pd, x_lds, &waves);
        if (resident <= 0)
            continue;
        const int teams = waves / cpl;                // a row's K is split over cpl waves
        int64_t want = (groups + teams - 1) / teams;
        if (want > n_tiles)
            want = n_tiles;
        int grid = (int)(want < resident ? want : resident);
        if (epi == E_ARGMAX && grid > QG_ARGMAX_MAX_GRID)
            grid = QG_ARGMAX_MAX_GRID;
        // keep a pool's results within QG_POOL_LDS (more, smaller pools for very tall matrices)
        const int64_t min_grid = (groups * items * 4 + QG_POOL_LDS - 1) / QG_POOL_LDS;
        if (grid < min_grid) {
            if (epi == E_ARGMAX && min_grid > QG_ARGMAX_MAX_GRID)
                return false;
            grid = (int)min_grid;
        }
        const int64_t pool_max = (n_tiles + grid - 1) / grid * TGr;
        const size_t lds = x_lds + (size_t)pool_max * items * 4;
        const int64_t per_team = (n_tiles / grid) * TGr / teams;
        if (pd > 1 && per_team < pd)
            continue;
        const int fit = stream_resident_wgs(fmt, epi, nrm, cpl, nb, pd, lds, &waves);
        if (fit <= 0)
            continue;
        if (fit < grid && grid <= resident && fit >= min_grid)
            grid = fit;                               // the pool's LDS lowered the residency
        sp->pd = pd;
        sp->grid = grid;
        sp->lds = x_lds + (size_t)((n_tiles + grid - 1) / grid * TGr) * items * 4;
        if (stream_resident_wgs(fmt, epi, nrm, cpl, nb, pd, sp->lds, &waves) <= 0)
            continue;
        return true;
    }
    return false;   // too much LDS for every variant: the tiled kernel takes the call
}

// Routed experts: 16-byte chunks per lane (1, 2 or 4 per row; the kernel holds 4 / cpl x rows
// per set in registers), groups in flight per wave, workgroups, result slots and LDS.  The grid
// has at least nb * topk workgroups, so that a workgroup's range (at most nb * topk sets of GS
// row groups, split evenly) spans at most two sets; at least the resident count; and enough that
// a range's results fit the result LDS.  query = false skips the device query (validation only).
struct MoePlan {
    int cpl, pd, grid, pool_max;
    size_t lds;
};

static bool plan_moe(int fmt, int64_t n_exp, int64_t N, int64_t K, int nb, int topk, bool query,
                     MoePlan *p)
{
    if (n_exp < 1 || n_exp > QG_MOE_EXPERTS_MAX)   // the per-expert counts live in LDS
        return false;
    if (fmt_hbits(fmt) || fmt_generic(fmt))         // the expert kernel takes Q4_0, Q8_0, Q4_K
        return false;
    const int64_t C = (fmt == FQ8_0 ? K : K / 2) / 16;
    p->cpl = C <= 64 ? 1 : C <= 128 ? 2 : C <= 256 ? 4 : 0;
    if (!p->cpl)
        return false;
    const int nbx = 4 / p->cpl;
    const int R = stream_rows(nbx, p->cpl, 1);
    const int64_t GS = (N + R - 1) / R;
    const int64_t P = (int64_t)nb * topk;
    if (P * GS > 0x7fffffffLL)
        return false;
    p->pd = QG_MOE_PD;
    // expert pair masks and set bases; two sets' x rows as f16 pairs and offset sums (uint4s per
    // row, chunk slot and lane: NP / 4 + 1 with NP = 16 pairs per chunk, 8 for Q8_0); then the
    // rows' raw copies, whose space the results reuse
    const int nq4 = (fmt == FQ8_0 ? 8 : 16) / 4 + 1;
    const size_t fixed_lds = (size_t)n_exp * 16 + (size_t)(n_exp + 3) / 4 * 16 +
                             (size_t)2 * nbx * p->cpl * nq4 * 64 * 16;
    const size_t raw_lds = (size_t)2 * nbx * (K / 4) * 16;
    const int64_t itx = (int64_t)R * nbx;
    const int64_t budget = QG_MOE_POOL_LDS / (itx * 4);   // result groups the LDS may hold
    const int resident = query ? moe_resident_wgs(fmt, p->cpl, p->pd,
                                                  fixed_lds + (raw_lds > QG_MOE_POOL_LDS
                                                                   ? raw_lds : QG_MOE_POOL_LDS))
                               : 0;
    int64_t grid = resident > P ? resident : P;
    const int64_t need = (P * GS + budget - 1) / budget;
    grid = grid > need ? grid : need;
    if (grid > 0x7fffffffLL)
        return false;
    p->grid = (int)grid;
    p->pool_max = (int)((P * GS + grid - 1) / grid);
    const size_t pool_lds = (size_t)p->pool_max * itx * 4;
    p->lds = fixed_lds + (raw_lds > pool_lds ? raw_lds : pool_lds);
    return true;
}

}  // namespace qg

using namespace qg;

// ------------------------------------------------------------------------------------ validation

static bool al(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

static bool overlap(const void *a, int64_t na, const void *b, int64_t nb)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

static int check_common(int fmt, const void *W, int64_t N, int64_t K, const float *x, int nb,
                        const void *y, Layout *L)
{
    if (!fmt_valid(fmt))
        return QG_ERR_FORMAT;
    if (!W || !x || !y)
        return QG_ERR_NULL;
    if (nb < 1 || nb > QG_MAX_NB || N < 1 || N > 0x7fffffffLL || !layout(fmt, N, K, L))
        return QG_ERR_SHAPE;
    if (!al(W, 256) || !al(x, 16) || !al(y, 4))
        return QG_ERR_ALIGN;
    const int64_t ybytes = (int64_t)nb * N * 4;
    if (overlap(y, ybytes, x, (int64_t)nb * K * 4) || overlap(y, ybytes, W, L->total))
        return QG_ERR_ALIAS;
    return QG_OK;
}

static int launch_status(int herr) { return herr == 0 ? QG_OK : QG_ERR_LAUNCH; }

static GemvArgs gemv_args(const Layout &L, const void *W, int64_t N, int64_t K, const float *x,
                          int nb, float *y)
{
    GemvArgs a;
    memset(&a, 0, sizeof(a));
    a.qs0 = static_cast<const uint8_t *>(W);
    a.sc0 = a.qs0 + L.sc_off;
    a.hb0 = a.qs0 + L.hb_off;
    a.dd0 = a.qs0 + L.d_off;
    a.hb_row = L.hb_row;
    a.d_row = L.d_row;
    a.cb0 = reinterpret_cast<const int8_t *>(a.qs0 + L.cb_off);
    a.x = x;
    a.y = y;
    a.N = N;
    a.K = K;
    a.nb = nb;
    a.qs_row = L.qs_row;
    a.sc_row = L.sc_row;
    return a;
}

// The launch plan of one GEMV-family call: which kernel takes it and that kernel's plan.
struct GemvPlan {
    int kind;   // 0: matrix cores, 1: streaming, 2: K-tiled
    MfmaPlan mp;
    StreamPlan sp;
    Plan p;
};

// Batch rows from which the matrix-core kernel takes a call.  Fewer than QG_MFMA_MIN_NB already
// do on matrices of at least 2^24 weights outside the gated product, for the formats whose
// vector path spends the most per decoded weight on its one dot chain per batch row (same-box
// timings, 65536 x 2048, vector -> matrix cores): three rows for Q4_0 (nb 4: 26.4 -> 21.3 us,
// argmax 30.5 -> 23.6; nb 3: 22.7 -> 20.9), Q4_K (nb 4: 30.7 -> 26.8; 3: 28.1 -> 27.3), Q5_0 (4:
// 29.2 -> 26.6; 3: 27.1 -> 25.9), IQ4_NL (4: 30.8 -> 23.3; 3: 27.5 -> 23.2), IQ4_XS (4: 29.6 ->
// 24.0; 3: 27.1 -> 23.2) and Q1_0 (4: 23.4 -> 18.3; 3: 19.7 -> 18.3); four rows for Q5_K (4: 34.4
// -> 31.7; 3: 31.6 -> 32.2).  Q8_0 (twice the bytes per weight, 4: 31.9 -> 33.8), Q6_K (4: 30.5 ->
// 30.8), the affine format (4: 28.3 -> 29.5), the gated product (the Q4_0 MLP, 4: even; 3: 19.6 ->
// 20.8), smaller matrices (the 2048 x 1536 Q8_0 QKV, 4: 6.7 -> 7.2) and two rows (19.9 -> 21.3)
// keep the vector path.
static int mfma_min_nb(int fmt, int epi, int64_t N, int64_t K)
{
    int m = QG_MFMA_MIN_NB;
    if (epi != E_GUS && N * K >= ((int64_t)1 << 24)) {
        if (fmt == FQ4_0 || fmt == FQ4_K || fmt == FQ5_0 || fmt == FIQ4_NL || fmt == FIQ4_XS ||
            fmt == FQ1_0)
            m = 3;
        else if (fmt == FQ5_K)
            m = 4;
    }
    return m < QG_MFMA_MIN_NB ? m : QG_MFMA_MIN_NB;
}

// Choose the kernel: the matrix-core kernel from mfma_min_nb batch rows when it takes the shape,
// else the streaming kernel when the shape allows it (a whole wave per row), else the tiled
// kernel (any nb, any K).  false: no kernel takes the shape.
static bool plan_call(int fmt, int epi, bool nrm, int64_t N, int64_t K, int nb, GemvPlan *g)
{
    Layout L;
    if (!layout(fmt, N, K, &L))
        return false;
    // the streaming and matrix kernels address each plane with 32-bit buffer offsets
    const bool small = N * L.qs_row < QG_BUF_MAX && N * L.sc_row < QG_BUF_MAX &&
                       N * L.hb_row < QG_BUF_MAX && N * L.d_row < QG_BUF_MAX;
    if (small && nb >= mfma_min_nb(fmt, epi, N, K) && plan_mfma(fmt, epi, nrm, N, K, nb, &g->mp) &&
        g->mp.grid <= QG_ARGMAX_MAX_GRID) {
        g->kind = 0;
        return true;
    }
    if (small && plan_stream(fmt, epi, nrm, N, K, nb, &g->sp)) {
        g->kind = 1;
        return true;
    }
    g->kind = 2;
    return plan_gemv(fmt, N, K, nb, epi == E_GUS ? 2 : 1, &g->p);
}

// Plans are a function of (device, format, op, N, K, nb) alone, so they are kept: after the first
// call of a shape, an eager call queries nothing from the device.
struct PlanKey {
    int dev, fmt, epi, nrm, nb;
    int64_t N, K;
    bool operator==(const PlanKey &o) const
    {
        return dev == o.dev && fmt == o.fmt && epi == o.epi && nrm == o.nrm && nb == o.nb &&
               N == o.N && K == o.K;
    }
};
struct PlanKeyHash {
    size_t operator()(const PlanKey &k) const
    {
        uint64_t h = 1469598103934665603ull;
        const int64_t v[7] = {k.dev, k.fmt, k.epi, k.nrm, k.nb, k.N, k.K};
        for (int64_t x : v)
            h = (h ^ (uint64_t)x) * 1099511628211ull;
        return (size_t)h;
    }
};

static bool cached_plan(int fmt, int epi, bool nrm, int64_t N, int64_t K, int nb, GemvPlan *g)
{
    static std::mutex mu;
    static std::unordered_map<PlanKey, GemvPlan, PlanKeyHash> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return false;
    const PlanKey key{dev, fmt, epi, nrm ? 1 : 0, nb, N, K};
    {
        std::lock_guard<std::mutex> lk(mu);
        auto it = cache.find(key);
        if (it != cache.end()) {
            *g = it->second;
            return true;
        }
    }
    if (!plan_call(fmt, epi, nrm, N, K, nb, g))
        return false;
    std::lock_guard<std::mutex> lk(mu);
    if (cache.size() < 4096)   // a bound on the memory a stream of odd shapes can take
        cache.emplace(key, *g);
    return true;
}

// Launch one member of the GEMV family on the kernel its plan names.  An argmax launch is
// followed by the one-workgroup fold of its per-workgroup partial keys.
static int run_gemv(int fmt, int epi, bool nrm, GemvArgs a, void *stream)
{
    int grid = 0, herr = 0;
    GemvPlan g;
    if (!cached_plan(fmt, epi, nrm, a.N, a.K, a.nb, &g))
        return QG_ERR_SHAPE;
    // 5..16 rows that only the K-tiled kernel takes (K > 4096, or the norm prologue with
    // K > 2048, or K not whole 128-weight steps) run as batches of at most 4 rows on the vector
    // path where it takes the shape: every output row depends on its own x row alone (2048 x
    // 8192 Q4_0 + residual: 8 rows 44.7 -> ~20 us, 16 rows 106 -> ~40 us).  The argmax batches
    // reuse the workspace one after the other on the stream.
    if (g.kind == 2 && a.nb > 4) {
        GemvPlan g4;
        if (cached_plan(fmt, epi, nrm, a.N, a.K, 4, &g4) && g4.kind == 1) {
            for (int r0 = 0; r0 < a.nb; r0 += 4) {
                GemvArgs c = a;
                c.nb = a.nb - r0 < 4 ? a.nb - r0 : 4;
                c.x = a.x + (int64_t)r0 * a.K;
                c.y = a.y + (int64_t)r0 * a.N;
                if (a.res)
                    c.res = a.res + (int64_t)r0 * a.res_rstride;
                if (a.idx)
                    c.idx = a.idx + r0;
                const int st = run_gemv(fmt, epi, nrm, c, stream);
                if (st != QG_OK)
                    return st;
            }
            return QG_OK;
        }
    }
    if (g.kind == 0) {
        const MfmaPlan &mp = g.mp;
        grid = mp.grid;
        herr = launch_mfma(fmt, epi, nrm, mp, a, stream);
    } else if (g.kind == 1) {
        const StreamPlan &sp = g.sp;
        grid = sp.grid;
        a.tg_log2 = sp.tg_log2;
        herr = launch_stream(fmt, epi, nrm, sp.cpl, sp.pd, a, sp.grid, sp.lds, stream);
    } else {
        const Plan &p = g.p;
        a.lpr_log2 = p.lpr_log2;
        a.kt = p.kt;
        a.n_kt = p.n_kt;
        a.rows_per_step = p.rows_per_step;
        a.n_steps = p.n_steps;
        grid = p.grid;
        herr = (fmt_hbits(fmt) || fmt_generic(fmt))
                   ? launch_gemv_x(fmt, epi, nrm, a, p.grid, p.lds, stream)
                   : launch_gemv(fmt, epi, nrm, a, p.grid, p.lds, stream);
    }
    if (herr == 0 && epi == E_ARGMAX)
        herr = launch_argmax_fold(a.keys, grid, a.nb, a.idx, stream);
    return launch_status(herr);
}

// Workspace of argmax: one 64-bit partial key per workgroup and batch row.
static int64_t ws_argmax_bytes(int nb) { return (int64_t)QG_ARGMAX_MAX_GRID * nb * 8; }

// Workspace of the routed experts: the sticky bad-id flag, then the partial outputs
// [nb][topk][N].
static int64_t ws_moe_bytes(int64_t N, int nb, int topk)
{
    return 256 + round256((int64_t)nb * topk * N * 4);
}

extern "C" {

int qgemv_layout_version(void) { return 1; }

const char *qgemv_status_str(int status)
{
    switch (status) {
    case QG_OK: return "ok";
    case QG_ERR_NULL: return "a required pointer is NULL";
    case QG_ERR_FORMAT: return "unknown or unsupported format (Q4_0=2, Q5_0=6, Q8_0=8, Q4_K=12, Q5_K=13, Q6_K=14, IQ4_NL=20, IQ4_XS=23, Q1_0=40, affine Q4=41; experts: Q4_0, Q8_0, Q4_K; qgemm: Q4_0, Q8_0, Q1_0)";
    case QG_ERR_SHAPE: return "bad shape (N, K, nb, M, topk or n_exp out of range, or K not a multiple of the block)";
    case QG_ERR_ALIGN: return "misaligned pointer (W and workspaces need 256 B, x and gamma 16 B (qgemm x: 4 B), other arrays 4 B)";
    case QG_ERR_WORKSPACE: return "workspace missing or smaller than qgemv_workspace_bytes() / qgemm_workspace_bytes()";
    case QG_ERR_LAUNCH: return "HIP launch failed";
    case QG_ERR_ALIAS: return "an output overlaps an input";
    default: return "unknown status";
    }
}

int64_t qgemv_packed_bytes(int fmt, int64_t N, int64_t K)
{
    Layout L;
    if (!layout(fmt, N, K, &L))
        return -1;
    return L.total;
}

int qgemv_pack(int fmt, const void *w_gguf, int64_t N, int64_t K, void *w_packed, void *stream)
{
    return qgemv_pack_codebook(fmt, w_gguf, N, K, nullptr, w_packed, stream);
}

int qgemv_pack_codebook(int fmt, const void *w_gguf, int64_t N, int64_t K, const int8_t *codebook,
                        void *w_packed, void *stream)
{
    if (!fmt_valid(fmt))
        return QG_ERR_FORMAT;
    if (!w_gguf || !w_packed || (fmt_codebook(fmt) && !codebook))
        return QG_ERR_NULL;
    Layout L;
    if (!layout(fmt, N, K, &L))
        return QG_ERR_SHAPE;
    if (!al(w_packed, 256))
        return QG_ERR_ALIGN;
    if (overlap(w_gguf, N * L.gguf_row, w_packed, L.total))
        return QG_ERR_ALIAS;
    return launch_status(launch_pack(fmt, w_gguf, N, K, codebook, w_packed, stream));
}

int64_t qgemv_workspace_bytes(int op, int fmt, int64_t N, int64_t K, int nb, int64_t n_exp,
                              int topk)
{
    Layout L;
    if (!layout(fmt, N, K, &L) || nb < 1 || nb > QG_MAX_NB)
        return -1;
    switch (op) {
    case QG_OP_GEMV:
    case QG_OP_NRM:
    case QG_OP_GUS_NRM:
    case QG_OP_RES:
    case QG_OP_NRM_BIAS:
        return 0;
    case QG_OP_ARGMAX:
        return ws_argmax_bytes(nb);
    case QG_OP_MOE: {
        MoePlan mp;
        if (n_exp < 1 || topk < 1 || topk > QG_MAX_TOPK ||
            !plan_moe(fmt, n_exp, N, K, nb, topk, false, &mp))
            return -1;
        return ws_moe_bytes(N, nb, topk);
    }
    default:
        return -1;
    }
}

int qgemv(int fmt, const void *W, int64_t N, int64_t K, const float *x, int nb, float *y,
          void *ws, size_t ws_bytes, void *stream)
{
    (void)ws;
    (void)ws_bytes;
    Layout L;
    int st = check_common(fmt, W, N, K, x, nb, y, &L);
    if (st != QG_OK)
        return st;
    return run_gemv(fmt, E_STORE, false, gemv_args(L, W, N, K, x, nb, y), stream);
}

int qgemv_nrm(int fmt, const void *W, int64_t N, int64_t K, const float *x, const float *gamma,
              float eps, int nb, float *y, void *ws, size_t ws_bytes, void *stream)
{
    (void)ws;
    (void)ws_bytes;
    Layout L;
    int st = check_common(fmt, W, N, K, x, nb, y, &L);
    if (st != QG_OK)
        return st;
    if (!gamma)
        return QG_ERR_NULL;
    if (!al(gamma, 16))
        return QG_ERR_ALIGN;
    if (overlap(y, (int64_t)nb * N * 4, gamma, K * 4))
        return QG_ERR_ALIAS;
    if (!(eps >= 0.0f))
        return QG_ERR_SHAPE;
    GemvArgs a = gemv_args(L, W, N, K, x, nb, y);
    a.gamma = gamma;
    a.eps = eps;
    return run_gemv(fmt, E_STORE, true, a, stream);
}

int qgemv_nrm_bias(int fmt, const void *W, int64_t N, int64_t K, const float *x,
                   const float *gamma, float eps, const float *bias, int nb, float *y, void *ws,
                   size_t ws_bytes, void *stream)
{
    (void)ws;
    (void)ws_bytes;
    Layout L;
    int st = check_common(fmt, W, N, K, x, nb, y, &L);
    if (st != QG_OK)
        return st;
    if (!gamma || !bias)
        return QG_ERR_NULL;
    if (!al(gamma, 16) || !al(bias, 4))
        return QG_ERR_ALIGN;
    const int64_t yb = (int64_t)nb * N * 4;
    if (overlap(y, yb, gamma, K * 4) || overlap(y, yb, bias, N * 4))
        return QG_ERR_ALIAS;
    if (!(eps >= 0.0f))
        return QG_ERR_SHAPE;
    GemvArgs a = gemv_args(L, W, N, K, x, nb, y);
    a.gamma = gamma;
    a.eps = eps;
    a.res = bias;
    a.res_rstride = 0;
    return run_gemv(fmt, E_RES, true, a, stream);
}

int qgemv_gus_nrm(int fmt, const void *Wg, const void *Wu, int64_t N, int64_t K, const float *x,
                  const float *gamma, float eps, int nb, float *h, void *ws, size_t ws_bytes,
                  void *stream)
{
    return qgemv_gus_act_nrm(fmt, Wg, Wu, N, K, x, gamma, eps, QG_ACT_SILU, nb, h, ws, ws_bytes,
                             stream);
}

int qgemv_gus_act_nrm(int fmt, const void *Wg, const void *Wu, int64_t N, int64_t K,
                      const float *x, const float *gamma, float eps, int act, int nb, float *h,
                      void *ws, size_t ws_bytes, void *stream)
{
    (void)ws;
    (void)ws_bytes;
    if (act != QG_ACT_SILU && act != QG_ACT_GELU_TANH)
        return QG_ERR_SHAPE;
    Layout L;
    int st = check_common(fmt, Wg, N, K, x, nb, h, &L);
    if (st != QG_OK)
        return st;
    if (!Wu || !gamma)
        return QG_ERR_NULL;
    if (!al(Wu, 256) || !al(gamma, 16))
        return QG_ERR_ALIGN;
    const int64_t hb = (int64_t)nb * N * 4;
    if (overlap(h, hb, Wu, L.total) || overlap(h, hb, gamma, K * 4))
        return QG_ERR_ALIAS;
    if (!(eps >= 0.0f))
        return QG_ERR_SHAPE;
    GemvArgs a = gemv_args(L, Wg, N, K, x, nb, h);
    a.qs1 = static_cast<const uint8_t *>(Wu);
    a.sc1 = a.qs1 + L.sc_off;
    a.hb1 = a.qs1 + L.hb_off;
    a.dd1 = a.qs1 + L.d_off;
    a.cb1 = reinterpret_cast<const int8_t *>(a.qs1 + L.cb_off);
    a.gamma = gamma;
    a.eps = eps;
    a.act = act;
    return run_gemv(fmt, E_GUS, true, a, stream);
}

int qgemv_res(int fmt, const void *W, int64_t N, int64_t K, const float *x, const float *res,
              int nb, float *y, void *ws, size_t ws_bytes, void *stream)
{
    (void)ws;
    (void)ws_bytes;
    Layout L;
    int st = check_common(fmt, W, N, K, x, nb, y, &L);
    if (st != QG_OK)
        return st;
    if (!res)
        return QG_ERR_NULL;
    if (!al(res, 4))
        return QG_ERR_ALIGN;
    const int64_t yb = (int64_t)nb * N * 4;
    if (res != y && overlap(y, yb, res, yb))
        return QG_ERR_ALIAS;
    GemvArgs a = gemv_args(L, W, N, K, x, nb, y);
    a.res = res;
    a.res_rstride = N;
    return run_gemv(fmt, E_RES, false, a, stream);
}

int qgemv_argmax(int fmt, const void *W, int64_t N, int64_t K, const float *x, int nb,
                 float *logits, int32_t *idx, void *ws, size_t ws_bytes, void *stream)
{
    Layout L;
    int st = check_common(fmt, W, N, K, x, nb, logits, &L);
    if (st != QG_OK)
        return st;
    if (!idx || !ws)
        return idx ? QG_ERR_WORKSPACE : QG_ERR_NULL;
    if (!al(idx, 4) || !al(ws, 256))
        return QG_ERR_ALIGN;
    if ((int64_t)ws_bytes < ws_argmax_bytes(nb))
        return QG_ERR_WORKSPACE;
    const int64_t lb = (int64_t)nb * N * 4, xb = (int64_t)nb * K * 4, wsb = (int64_t)ws_bytes;
    if (overlap(idx, nb * 4, logits, lb) || overlap(ws, wsb, logits, lb) ||
        overlap(ws, wsb, idx, nb * 4) || overlap(idx, nb * 4, x, xb) ||
        overlap(idx, nb * 4, W, L.total) || overlap(ws, wsb, x, xb) || overlap(ws, wsb, W, L.total))
        return QG_ERR_ALIAS;
    GemvArgs a = gemv_args(L, W, N, K, x, nb, logits);
    a.idx = idx;
    a.keys = static_cast<unsigned long long *>(ws);
    return run_gemv(fmt, E_ARGMAX, false, a, stream);
}

int qgemv_argmax_noalloc(int fmt, const void *W, int64_t N, int64_t K, const float *x, int nb,
                         float *logits, int32_t *idx, void *stream)
{
    Layout L;
    int st = check_common(fmt, W, N, K, x, nb, logits, &L);
    if (st != QG_OK)
        return st;
    if (!idx)
        return QG_ERR_NULL;
    if (!al(idx, 4))
        return QG_ERR_ALIGN;
    const int64_t lb = (int64_t)nb * N * 4;
    if (overlap(idx, nb * 4, logits, lb) || overlap(idx, nb * 4, x, (int64_t)nb * K * 4) ||
        overlap(idx, nb * 4, W, L.total))
        return QG_ERR_ALIAS;
    // every argmax launch has at most QG_ARGMAX_MAX_GRID workgroups, so its partial keys fit
    if (ws_argmax_bytes(nb) > (int64_t)((size_t)QG_ARGMAX_MAX_GRID * QG_MAX_NB * 8))
        return QG_ERR_SHAPE;
    void *sp = nullptr;
    size_t sbytes = 0;
    if (noalloc_scratch(&sp, &sbytes) != 0)
        return QG_ERR_LAUNCH;
    if ((int64_t)sbytes < ws_argmax_bytes(nb))
        return QG_ERR_WORKSPACE;
    GemvArgs a = gemv_args(L, W, N, K, x, nb, logits);
    a.idx = idx;
    a.keys = static_cast<unsigned long long *>(sp);
    return run_gemv(fmt, E_ARGMAX, false, a, stream);
}

int qgemv_moe(int fmt, const void *W_experts, int64_t n_exp, int64_t N, int64_t K, const float *x,
              int nb, const int32_t *ids, const float *wts, int topk, float *y, void *ws,
              size_t ws_bytes, void *stream)
{
    Layout L;
    int st = check_common(fmt, W_experts, N, K, x, nb, y, &L);
    if (st != QG_OK)
        return st;
    if (fmt_hbits(fmt) || fmt_generic(fmt))
        return QG_ERR_FORMAT;
    if (!ids || !wts)
        return QG_ERR_NULL;
    if (!ws)
        return QG_ERR_WORKSPACE;
    if (n_exp < 1 || topk < 1 || topk > QG_MAX_TOPK || n_exp * N > 0x7fffffffLL)
        return QG_ERR_SHAPE;
    Layout LE;   // the expert stack is packed as one matrix of n_exp * N rows
    if (!layout(fmt, n_exp * N, K, &LE))
        return QG_ERR_SHAPE;
    if (!al(ids, 4) || !al(wts, 4) || !al(ws, 256))
        return QG_ERR_ALIGN;
    MoePlan mp;
    // every expert's planes are addressed through 32-bit buffer offsets
    if (N * L.qs_row >= QG_BUF_MAX || N * L.sc_row >= QG_BUF_MAX ||
        !plan_moe(fmt, n_exp, N, K, nb, topk, true, &mp))
        return QG_ERR_SHAPE;
    if ((int64_t)ws_bytes < ws_moe_bytes(N, nb, topk))
        return QG_ERR_WORKSPACE;
    const int64_t yb = (int64_t)nb * N * 4, wsb = (int64_t)ws_bytes, rb = (int64_t)nb * topk * 4;
    if (overlap(y, yb, W_experts, LE.total) || overlap(y, yb, ws, wsb) || overlap(y, yb, ids, rb) ||
        overlap(y, yb, wts, rb) || overlap(ws, wsb, W_experts, LE.total) ||
        overlap(ws, wsb, x, (int64_t)nb * K * 4) || overlap(ws, wsb, ids, rb) ||
        overlap(ws, wsb, wts, rb))
        return QG_ERR_ALIAS;
    MoeArgs a;
    memset(&a, 0, sizeof(a));
    a.qs = static_cast<const uint8_t *>(W_experts);
    a.sc = a.qs + LE.sc_off;
    a.x = x;
    a.ids = ids;
    a.wts = wts;
    a.y = y;
    uint8_t *w8 = static_cast<uint8_t *>(ws);
    a.err = reinterpret_cast<unsigned int *>(w8);
    a.part = reinterpret_cast<float *>(w8 + 256);
    a.n_exp = n_exp;
    a.N = N;
    a.K = K;
    a.qs_row = L.qs_row;
    a.sc_row = L.sc_row;
    a.nb = nb;
    a.topk = topk;
    a.pool_max = mp.pool_max;
    return launch_status(launch_moe(fmt, mp.cpl, mp.pd, a, mp.grid, mp.lds, stream));
}

int qgemv_qk_norm_rope(float *qkv, int nb, int n_q_heads, int n_kv_heads, int head_dim,
                       int rope_half, const float *q_gamma, const float *k_gamma, float eps,
                       const float *rope_cos, const float *rope_sin, void *stream)
{
    if (!qkv || (rope_half > 0 && (!rope_cos || !rope_sin)))
        return QG_ERR_NULL;
    if (nb < 1 || nb > QG_MAX_NB || n_q_heads < 1 || n_kv_heads < 0 || head_dim < 2 ||
        head_dim > QG_HEAD_DIM_MAX || head_dim % 2 || rope_half < 0 || 2 * rope_half > head_dim ||
        !(eps >= 0.0f) || (int64_t)(n_q_heads + 2 * (int64_t)n_kv_heads) * head_dim > 0x7fffffffLL)
        return QG_ERR_SHAPE;
    if (!al(qkv, 4) || (q_gamma && !al(q_gamma, 4)) || (k_gamma && !al(k_gamma, 4)) ||
        (rope_cos && !al(rope_cos, 4)) || (rope_sin && !al(rope_sin, 4)))
        return QG_ERR_ALIGN;
    const int64_t row = (int64_t)(n_q_heads + 2 * n_kv_heads) * head_dim;
    const int64_t yb = (int64_t)nb * row * 4, tb = (int64_t)nb * rope_half * 4;
    if ((q_gamma && overlap(qkv, yb, q_gamma, (int64_t)head_dim * 4)) ||
        (k_gamma && overlap(qkv, yb, k_gamma, (int64_t)head_dim * 4)) ||
        (rope_half > 0 && (overlap(qkv, yb, rope_cos, tb) || overlap(qkv, yb, rope_sin, tb))))
        return QG_ERR_ALIAS;
    return launch_status(launch_qk_norm_rope(qkv, row, nb, n_q_heads, n_kv_heads, head_dim,
                                             rope_half, q_gamma, k_gamma, eps, rope_cos,
                                             rope_sin, stream));
}

// Tiles, K steps and K splits of a qgemm call, from the shape alone (so the workspace size is
// too).  Weight tiles: the widest that alone give the 256 compute units a tile each (Q4_0 up to
// 512 rows, the others, and any format against 64-row x tiles, 256), else 128 rows.  x tiles of
// 128 rows, or of 64 for M <= 64 (half the operand copies and products of a 128-row tile that
// would be half zero rows); when the output tiles are still fewer than the compute units the K
// steps are dealt out to several workgroups per tile, at least two steps each.
struct GemmPlan {
    int64_t m_tiles, n_tiles, bm, bn, steps, sps, splits;
    int64_t xh_bytes, rs_bytes, part_bytes;
};

static int64_t gemm_bn(int fmt, int64_t m_tiles, int64_t N)
{
    if (fmt == QG_Q4_0 && m_tiles * ((N + 511) / 512) >= 256)
        return 512;
    return m_tiles * ((N + 255) / 256) >= 256 ? 256 : 128;
}

static GemmPlan gemm_plan(int fmt, int64_t N, int64_t K, int64_t M)
{
    GemmPlan p;
    p.bm = M <= 64 ? 64 : QG_GEMM_BM;
    p.m_tiles = (M + p.bm - 1) / p.bm;
    p.bn = gemm_bn(fmt, p.m_tiles, N);
    if (p.bm == 64 && p.bn > 256)
        p.bn = 256;
    p.n_tiles = (N + p.bn - 1) / p.bn;
    p.steps = (K + QG_GEMM_KSTEP - 1) / QG_GEMM_KSTEP;
    const int64_t tiles = p.m_tiles * p.n_tiles;
    p.sps = p.steps;
    if (tiles < 192 && p.steps >= 4) {
        const int64_t want = (256 + tiles - 1) / tiles;
        const int64_t sps = (p.steps + want - 1) / want;
        p.sps = sps < 2 ? 2 : sps;
    }
    p.splits = (p.steps + p.sps - 1) / p.sps;
    const int64_t Mp = p.m_tiles * p.bm;
    p.xh_bytes = round256(Mp * p.steps * QG_GEMM_KSTEP * 2);
    p.rs_bytes = round256(Mp * 4);
    p.part_bytes = p.splits > 1 ? round256(p.splits * M * N * 4) : 0;
    return p;
}

int64_t qgemm_workspace_bytes(int fmt, int64_t N, int64_t K, int64_t M)
{
    Layout L;
    if ((fmt != QG_Q4_0 && fmt != QG_Q8_0 && fmt != QG_Q1_0) || M < 1 || M > QG_GEMM_MAX_M ||
        !layout(fmt, N, K, &L))
        return -1;
    const GemmPlan p = gemm_plan(fmt, N, K, M);
    return p.xh_bytes + p.rs_bytes + p.part_bytes;
}

int qgemm(int fmt, const void *W, int64_t N, int64_t K, const float *x, int64_t M, float *y,
          void *ws, size_t ws_bytes, void *stream)
{
    if (!fmt_valid(fmt))
        return QG_ERR_FORMAT;
    if (fmt != QG_Q4_0 && fmt != QG_Q8_0 && fmt != QG_Q1_0)
        return QG_ERR_FORMAT;
    if (!W || !x || !y)
        return QG_ERR_NULL;
    Layout L;
    if (M < 1 || M > QG_GEMM_MAX_M || N < 1 || N > 0x7fffffffLL || !layout(fmt, N, K, &L) ||
        N * L.qs_row >= QG_BUF_MAX || N * L.sc_row >= QG_BUF_MAX ||
        (N / 128 + 8) * ((M + 63) / 64) > 0x7fffffffLL)   // the tile count
        return QG_ERR_SHAPE;
    const GemmPlan p = gemm_plan(fmt, N, K, M);
    if ((p.n_tiles + 7) * p.m_tiles * p.splits > 0x7fffffffLL ||
        p.m_tiles * p.bm / 16 * p.steps * QG_GEMM_KSTEP / 32 > 0x7fffffffLL)
        return QG_ERR_SHAPE;
    if (!ws)
        return QG_ERR_WORKSPACE;
    if (!al(W, 256) || !al(x, 4) || !al(y, 4) || !al(ws, 256))
        return QG_ERR_ALIGN;
    const int64_t need = qgemm_workspace_bytes(fmt, N, K, M);
    if ((int64_t)ws_bytes < need)
        return QG_ERR_WORKSPACE;
    const int64_t yb = M * N * 4, xb = M * K * 4, wsb = (int64_t)ws_bytes;
    if (overlap(y, yb, x, xb) || overlap(y, yb, W, L.total) || overlap(y, yb, ws, wsb) ||
        overlap(ws, wsb, x, xb) || overlap(ws, wsb, W, L.total))
        return QG_ERR_ALIAS;
    // Up to QG_MAX_NB rows the row-batch GEMV kernels do the same product faster (one launch,
    // no x preparation or fold pass; 8192 x 2048 Q4_0, GEMM -> GEMV: 16 rows 15.4 -> 8.4 us, 4
    // rows 14.8 -> 8.3, 1 row 14.5 -> 5.5), where their own requirements hold (x 16-byte
    // aligned) and the GEMV takes the shape on the matrix cores or the streaming kernel (not the
    // K-tiled fallback); the workspace is then not touched.
    if (M <= QG_MAX_NB) {
        Layout Lg;
        GemvPlan g;
        if (check_common(fmt, W, N, K, x, (int)M, y, &Lg) == QG_OK &&
            cached_plan(fmt, E_STORE, false, N, K, (int)M, &g) && g.kind != 2)
            return run_gemv(fmt, E_STORE, false, gemv_args(Lg, W, N, K, x, (int)M, y), stream);
    }
    GemmArgs a;
    memset(&a, 0, sizeof(a));
    a.qs = static_cast<const uint8_t *>(W);
    a.sc = a.qs + L.sc_off;
    uint8_t *w8 = static_cast<uint8_t *>(ws);
    a.xh = reinterpret_cast<_Float16 *>(w8);
    a.rs = reinterpret_cast<float *>(w8 + p.xh_bytes);
    a.part = p.splits > 1 ? reinterpret_cast<float *>(w8 + p.xh_bytes + p.rs_bytes) : nullptr;
    a.y = y;
    a.N = N;
    a.K = K;
    a.M = M;
    a.qs_row = L.qs_row;
    a.sc_row = L.sc_row;
    a.n_tiles = (int)p.n_tiles;
    a.m_tiles = (int)p.m_tiles;
    a.bn = (int)p.bn;
    a.bm = (int)p.bm;
    a.KBp = (int)(p.steps * QG_GEMM_KSTEP / 32);
    a.steps = (int)p.steps;
    a.sps = (int)p.sps;
    a.splits = (int)p.splits;
    return launch_status(launch_gemm(fmt, a, x, stream));
}

int qgemv_moe_error(const void *ws, int64_t n_exp, int64_t N, int64_t K, int fmt, int *flag,
                    void *stream)
{
    if (!ws || !flag)
        return QG_ERR_NULL;
    if (!fmt_valid(fmt))
        return QG_ERR_FORMAT;
    MoePlan mp;
    if (!plan_moe(fmt, n_exp, N, K, 1, 1, false, &mp))
        return QG_ERR_SHAPE;
    const uint8_t *errp = static_cast<const uint8_t *>(ws);
    unsigned int v = 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(&v, errp, 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return QG_ERR_LAUNCH;
    *flag = (int)v;
    if (v) {
        const unsigned int zero = 0;
        if (hipMemcpyAsync(const_cast<uint8_t *>(errp), &zero, 4, hipMemcpyHostToDevice, s) !=
                hipSuccess ||
            hipStreamSynchronize(s) != hipSuccess)
            return QG_ERR_LAUNCH;
    }
    return QG_OK;
}

}  // extern "C"

// stream_kernels_g.hip -- the streaming dequant-GEMV kernels instantiated for the codebook formats
// (IQ4_NL, IQ4_XS: "Crate inferencelayer" docs, gemv_iq4_nl_k_lcpp_src, gemv_iq4_xs_k_lcpp_src),
// the sign format (Q1_0: gemv_q1_k_lcpp_src) and the affine Q4 ("Module gpu", struct Q, with x
// as even / odd halves and per-32 sums, struct HalfSet).  A translation unit of its own so that
// the formats compile in parallel.
#include "stream_impl.h"

namespace qg {

void stream_fn_g(int fmt, int epi, bool nrm, int ks, int nb, int pd, const void **fn,
                 int *threads)
{
    const StreamFn f = fmt == FIQ4_NL ? stream_fn_fmt<FIQ4_NL>(epi, nrm, ks, nb, pd)
                     : fmt == FIQ4_XS ? stream_fn_fmt<FIQ4_XS>(epi, nrm, ks, nb, pd)
                     : fmt == FQ1_0 ? stream_fn_fmt<FQ1_0>(epi, nrm, ks, nb, pd)
                     : fmt == FAQ4 ? stream_fn_fmt<FAQ4>(epi, nrm, ks, nb, pd)
                                   : StreamFn{nullptr, 0};
    *fn = f.fn;
    *threads = f.threads;
}

}  // namespace qg

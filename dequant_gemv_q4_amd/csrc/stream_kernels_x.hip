// stream_kernels_x.hip -- the streaming dequant-GEMV kernels instantiated for the high-bit formats
// (Q5_0, Q5_K, Q6_K: "Crate inferencelayer" docs, gemv_q5_0n_k_lcpp_src, gemv_q5k_k_lcpp_src,
// gemv_q6k_k_lcpp_src).  A translation unit of its own so that the formats compile in parallel.
#include "stream_impl.h"

namespace qg {

void stream_fn_x(int fmt, int epi, bool nrm, int ks, int nb, int pd, const void **fn,
                 int *threads)
{
    const StreamFn f = fmt == FQ5_0 ? stream_fn_fmt<FQ5_0>(epi, nrm, ks, nb, pd)
                     : fmt == FQ5_K ? stream_fn_fmt<FQ5_K>(epi, nrm, ks, nb, pd)
                     : fmt == FQ6_K ? stream_fn_fmt<FQ6_K>(epi, nrm, ks, nb, pd)
                                    : StreamFn{nullptr, 0};
    *fn = f.fn;
    *threads = f.threads;
}

}  // namespace qg

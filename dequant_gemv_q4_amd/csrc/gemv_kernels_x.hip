// gemv_kernels_x.hip -- the K-tiled dequant-GEMV kernel instantiated for the high-bit formats
// (Q5_0, Q5_K, Q6_K: "Crate inferencelayer" docs, gemv_q5_0n_k_lcpp_src, gemv_q5k_k_lcpp_src,
// gemv_q6k_k_lcpp_src), the codebook formats (IQ4_NL, IQ4_XS: gemv_iq4_nl_k_lcpp_src,
// gemv_iq4_xs_k_lcpp_src), the sign format (Q1_0: gemv_q1_k_lcpp_src) and the affine Q4 ("Module
// gpu", struct Q).  A translation unit of its own so that the formats compile in parallel.
#include "gemv_impl.h"

namespace qg {

int launch_gemv_x(int fmt, int epi, bool nrm, const GemvArgs &a, int grid, size_t lds_bytes,
                  void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (fmt == FQ5_0)
        return launch_gemv_fmt<FQ5_0>(epi, nrm, a, grid, lds_bytes, s);
    if (fmt == FQ5_K)
        return launch_gemv_fmt<FQ5_K>(epi, nrm, a, grid, lds_bytes, s);
    if (fmt == FQ6_K)
        return launch_gemv_fmt<FQ6_K>(epi, nrm, a, grid, lds_bytes, s);
    if (fmt == FIQ4_NL)
        return launch_gemv_fmt<FIQ4_NL>(epi, nrm, a, grid, lds_bytes, s);
    if (fmt == FIQ4_XS)
        return launch_gemv_fmt<FIQ4_XS>(epi, nrm, a, grid, lds_bytes, s);
    if (fmt == FQ1_0)
        return launch_gemv_fmt<FQ1_0>(epi, nrm, a, grid, lds_bytes, s);
    if (fmt == FAQ4)
        return launch_gemv_fmt<FAQ4>(epi, nrm, a, grid, lds_bytes, s);
    return (int)hipErrorInvalidValue;
}

}  // namespace qg

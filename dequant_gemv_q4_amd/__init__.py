"""dequant_gemv_q4_amd -- block-quantized dequant-GEMV for LLM decode on MI355X (gfx950):
hand-written HIP kernels behind the C ABI of include/qgemv.h (Q4_0, Q5_0, Q8_0, Q4_K, Q5_K,
Q6_K, IQ4_NL, IQ4_XS, Q1_0 and an affine Q4).

The functions exported here are the C entry points under the same names (see ``_binding``);
``device`` holds torch-side plumbing (device buffers for packed weights and workspaces).
"""
from ._binding import (  # noqa: F401
    ACT_GELU_TANH, ACT_SILU, AQ4, IQ4_NL, IQ4_XS, LIB_PATH, OP_ARGMAX, OP_GEMV, OP_GUS_NRM, OP_MOE,
    OP_NRM, OP_NRM_BIAS, OP_RES, Q1_0, Q4_0, Q4_K, Q5_0, Q5_K, Q6_K, Q8_0, QgemvError,
    header_functions, lib, qgemm, qgemm_workspace_bytes, qgemv, qgemv_argmax,
    qgemv_argmax_noalloc, qgemv_gus_act_nrm, qgemv_gus_nrm, qgemv_layout_version, qgemv_moe,
    qgemv_moe_error, qgemv_nrm, qgemv_nrm_bias, qgemv_pack, qgemv_pack_codebook,
    qgemv_packed_bytes, qgemv_qk_norm_rope, qgemv_res, qgemv_status_str, qgemv_workspace_bytes,
)

"""ctypes binding of libqgemv (include/qgemv.h): argument marshalling only.

Every function has the name and argument order of its C entry point.  Array arguments may be
torch tensors (their data pointer is passed; device tensors for the compute calls) or plain
integer addresses.  ``stream`` defaults to torch's current HIP stream.  A non-zero status
raises :class:`QgemvError`; nothing is ever computed on the host.
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqgemv.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "qgemv.h")

Q4_0, Q5_0, Q8_0, Q4_K, Q5_K, Q6_K = 2, 6, 8, 12, 13, 14
IQ4_NL, IQ4_XS, Q1_0, AQ4 = 20, 23, 40, 41
OP_GEMV, OP_NRM, OP_GUS_NRM, OP_RES, OP_ARGMAX, OP_MOE, OP_NRM_BIAS = range(7)
ACT_SILU, ACT_GELU_TANH = 0, 1
STATUS = {0: "QG_OK", 1: "QG_ERR_NULL", 2: "QG_ERR_FORMAT", 3: "QG_ERR_SHAPE", 4: "QG_ERR_ALIGN",
          5: "QG_ERR_WORKSPACE", 6: "QG_ERR_LAUNCH", 7: "QG_ERR_ALIAS"}


class QgemvError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({text})")
        self.status = status


_lib = None
_vp, _i64, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

_SIGS = {
    "qgemv_packed_bytes": (_i64, [_i32, _i64, _i64]),
    "qgemv_pack": (_i32, [_i32, _vp, _i64, _i64, _vp, _vp]),
    "qgemv_pack_codebook": (_i32, [_i32, _vp, _i64, _i64, _vp, _vp, _vp]),
    "qgemv_workspace_bytes": (_i64, [_i32, _i32, _i64, _i64, _i32, _i64, _i32]),
    "qgemv": (_i32, [_i32, _vp, _i64, _i64, _vp, _i32, _vp, _vp, _sz, _vp]),
    "qgemv_nrm": (_i32, [_i32, _vp, _i64, _i64, _vp, _vp, _f32, _i32, _vp, _vp, _sz, _vp]),
    "qgemv_gus_nrm": (_i32, [_i32, _vp, _vp, _i64, _i64, _vp, _vp, _f32, _i32, _vp, _vp, _sz, _vp]),
    "qgemv_nrm_bias": (_i32, [_i32, _vp, _i64, _i64, _vp, _vp, _f32, _vp, _i32, _vp, _vp, _sz, _vp]),
    "qgemv_gus_act_nrm": (_i32, [_i32, _vp, _vp, _i64, _i64, _vp, _vp, _f32, _i32, _i32, _vp, _vp,
                                 _sz, _vp]),
    "qgemv_qk_norm_rope": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _f32, _vp, _vp,
                                  _vp]),
    "qgemv_res": (_i32, [_i32, _vp, _i64, _i64, _vp, _vp, _i32, _vp, _vp, _sz, _vp]),
    "qgemv_argmax": (_i32, [_i32, _vp, _i64, _i64, _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
    "qgemv_argmax_noalloc": (_i32, [_i32, _vp, _i64, _i64, _vp, _i32, _vp, _vp, _vp]),
    "qgemv_moe": (_i32, [_i32, _vp, _i64, _i64, _i64, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _sz, _vp]),
    "qgemm_workspace_bytes": (_i64, [_i32, _i64, _i64, _i64]),
    "qgemm": (_i32, [_i32, _vp, _i64, _i64, _vp, _i64, _vp, _vp, _sz, _vp]),
    "qgemv_moe_error": (_i32, [_vp, _i64, _i64, _i64, _i32, ctypes.POINTER(ctypes.c_int), _vp]),
    "qgemv_status_str": (ctypes.c_char_p, [_i32]),
    "qgemv_layout_version": (_i32, []),
}


def lib():
    """Load libqgemv.so (fails loudly if it was not built: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libqgemv.so not built ({LIB_PATH}); run "
                               "`python -m dequant_gemv_q4_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/qgemv.h declares."""
    txt = open(HEADER_PATH).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(qgem[mv][A-Za-z0-9_]*)\s*\(", txt, re.M)


def _p(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _nbytes(ws):
    if ws is None:
        return 0
    if isinstance(ws, int):
        raise TypeError("pass ws_bytes together with an integer workspace address")
    return ws.numel() * ws.element_size()


def _check(fn, st):
    if st != 0:
        raise QgemvError(fn, st, lib().qgemv_status_str(st).decode())


def qgemv_status_str(status: int) -> str:
    return lib().qgemv_status_str(status).decode()


def qgemv_layout_version() -> int:
    return lib().qgemv_layout_version()


def qgemv_packed_bytes(fmt: int, N: int, K: int) -> int:
    return lib().qgemv_packed_bytes(fmt, N, K)


def qgemv_workspace_bytes(op: int, fmt: int, N: int, K: int, nb: int, n_exp: int = 0,
                          topk: int = 0) -> int:
    return lib().qgemv_workspace_bytes(op, fmt, N, K, nb, n_exp, topk)


def qgemv_pack(fmt, w_gguf, N, K, w_packed, stream=None):
    _check("qgemv_pack", lib().qgemv_pack(fmt, _p(w_gguf), N, K, _p(w_packed), _stream(stream)))


def qgemv_pack_codebook(fmt, w_gguf, N, K, codebook, w_packed, stream=None):
    """codebook: 16 signed bytes on the host (any sequence of ints in [-128, 127]), or None."""
    cb = None
    if codebook is not None:
        vals = [int(v) for v in codebook]
        if len(vals) != 16:
            raise ValueError("the codebook has 16 entries")
        cb = (ctypes.c_int8 * 16)(*vals)
    _check("qgemv_pack_codebook",
           lib().qgemv_pack_codebook(fmt, _p(w_gguf), N, K,
                                     None if cb is None else ctypes.addressof(cb), _p(w_packed),
                                     _stream(stream)))


def qgemv(fmt, W, N, K, x, nb, y, ws=None, ws_bytes=None, stream=None):
    _check("qgemv", lib().qgemv(fmt, _p(W), N, K, _p(x), nb, _p(y), _p(ws),
                                _nbytes(ws) if ws_bytes is None else ws_bytes, _stream(stream)))


def qgemv_nrm(fmt, W, N, K, x, gamma, eps, nb, y, ws=None, ws_bytes=None, stream=None):
    _check("qgemv_nrm", lib().qgemv_nrm(fmt, _p(W), N, K, _p(x), _p(gamma), eps, nb, _p(y), _p(ws),
                                        _nbytes(ws) if ws_bytes is None else ws_bytes,
                                        _stream(stream)))


def qgemv_gus_nrm(fmt, Wg, Wu, N, K, x, gamma, eps, nb, h, ws=None, ws_bytes=None, stream=None):
    _check("qgemv_gus_nrm", lib().qgemv_gus_nrm(fmt, _p(Wg), _p(Wu), N, K, _p(x), _p(gamma), eps,
                                                nb, _p(h), _p(ws),
                                                _nbytes(ws) if ws_bytes is None else ws_bytes,
                                                _stream(stream)))


def qgemv_nrm_bias(fmt, W, N, K, x, gamma, eps, bias, nb, y, ws=None, ws_bytes=None, stream=None):
    _check("qgemv_nrm_bias", lib().qgemv_nrm_bias(fmt, _p(W), N, K, _p(x), _p(gamma), eps, _p(bias),
                                                  nb, _p(y), _p(ws),
                                                  _nbytes(ws) if ws_bytes is None else ws_bytes,
                                                  _stream(stream)))


def qgemv_gus_act_nrm(fmt, Wg, Wu, N, K, x, gamma, eps, act, nb, h, ws=None, ws_bytes=None,
                      stream=None):
    _check("qgemv_gus_act_nrm", lib().qgemv_gus_act_nrm(fmt, _p(Wg), _p(Wu), N, K, _p(x),
                                                        _p(gamma), eps, act, nb, _p(h), _p(ws),
                                                        _nbytes(ws) if ws_bytes is None
                                                        else ws_bytes, _stream(stream)))


def qgemv_qk_norm_rope(qkv, nb, n_q_heads, n_kv_heads, head_dim, rope_half, q_gamma, k_gamma, eps,
                       rope_cos, rope_sin, stream=None):
    _check("qgemv_qk_norm_rope", lib().qgemv_qk_norm_rope(_p(qkv), nb, n_q_heads, n_kv_heads,
                                                          head_dim, rope_half, _p(q_gamma),
                                                          _p(k_gamma), eps, _p(rope_cos),
                                                          _p(rope_sin), _stream(stream)))


def qgemv_res(fmt, W, N, K, x, res, nb, y, ws=None, ws_bytes=None, stream=None):
    _check("qgemv_res", lib().qgemv_res(fmt, _p(W), N, K, _p(x), _p(res), nb, _p(y), _p(ws),
                                        _nbytes(ws) if ws_bytes is None else ws_bytes,
                                        _stream(stream)))


def qgemv_argmax(fmt, W, N, K, x, nb, logits, idx, ws, ws_bytes=None, stream=None):
    _check("qgemv_argmax", lib().qgemv_argmax(fmt, _p(W), N, K, _p(x), nb, _p(logits), _p(idx),
                                              _p(ws), _nbytes(ws) if ws_bytes is None else ws_bytes,
                                              _stream(stream)))


def qgemv_argmax_noalloc(fmt, W, N, K, x, nb, logits, idx, stream=None):
    _check("qgemv_argmax_noalloc", lib().qgemv_argmax_noalloc(fmt, _p(W), N, K, _p(x), nb,
                                                              _p(logits), _p(idx), _stream(stream)))


def qgemv_moe(fmt, W_experts, n_exp, N, K, x, nb, ids, wts, topk, y, ws, ws_bytes=None,
              stream=None):
    _check("qgemv_moe", lib().qgemv_moe(fmt, _p(W_experts), n_exp, N, K, _p(x), nb, _p(ids),
                                        _p(wts), topk, _p(y), _p(ws),
                                        _nbytes(ws) if ws_bytes is None else ws_bytes,
                                        _stream(stream)))


def qgemm_workspace_bytes(fmt: int, N: int, K: int, M: int) -> int:
    return lib().qgemm_workspace_bytes(fmt, N, K, M)


def qgemm(fmt, W, N, K, x, M, y, ws, ws_bytes=None, stream=None):
    _check("qgemm", lib().qgemm(fmt, _p(W), N, K, _p(x), M, _p(y), _p(ws),
                                _nbytes(ws) if ws_bytes is None else ws_bytes, _stream(stream)))


def qgemv_moe_error(ws, n_exp, N, K, fmt, stream=None) -> int:
    flag = ctypes.c_int(0)
    _check("qgemv_moe_error", lib().qgemv_moe_error(_p(ws), n_exp, N, K, fmt, ctypes.byref(flag),
                                                    _stream(stream)))
    return flag.value

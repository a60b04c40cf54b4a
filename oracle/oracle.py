"""ctypes front of the f64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU
baseline leg are the only callers.  Nothing here is shared with the HIP
library; inputs are the GGUF-native block bytes the seeded generators write.

Every composite below is the plain composition the pages describe:
  * ``qgemv``        y = W x                                    (f64 dot)
  * ``qgemv_nrm``    y = W rmsnorm(x)     ("honeycrisp mod.rs", fused_norm_quant_matmul_multi)
  * ``qgemv_gus_nrm`` h = silu(Wg n) * (Wu n), n = rmsnorm(x)   ("honeycrisp mod.rs", fused_norm_swiglu_down)
  * ``qgemv_res``    y = W x + r          ("honeycrisp mod.rs", fused matmul + residual)
  * ``qgemv_argmax`` logits = W x, idx = lowest index of the row max ("Module gpu", sampling)
  * ``qgemv_moe``    y[r] = sum_t p[r,t] W_{id[r,t]} x_r        ("Module gpu", RouteStep)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

Q4_0, Q5_0, Q8_0, Q4_K, Q5_K, Q6_K = 2, 6, 8, 12, 13, 14
IQ4_NL, IQ4_XS, Q1_0, AQ4 = 20, 23, 40, 41

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared",
               "-fPIC", "-std=c99", "-Wall", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.orc_f16.restype = ctypes.c_double
        lib.orc_f16.argtypes = [ctypes.c_uint16]
        lib.orc_block_bytes.restype = ctypes.c_int64
        lib.orc_block_weights.restype = ctypes.c_int64
        lib.orc_row_bytes.restype = ctypes.c_int64
        lib.orc_row_bytes.argtypes = [ctypes.c_int, ctypes.c_int64]
        lib.orc_dequant_row.argtypes = [ctypes.c_int, _u8p, ctypes.c_int64, _dp]
        lib.orc_q4k_scale_min.argtypes = [_u8p, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                          ctypes.POINTER(ctypes.c_int)]
        lib.orc_gemv.argtypes = [ctypes.c_int, _u8p, ctypes.c_int64, ctypes.c_int64, _dp,
                                 ctypes.c_int64, _i64p, ctypes.c_int64, _dp, _dp]
        lib.orc_gemv_res.argtypes = [ctypes.c_int, _u8p, ctypes.c_int64, ctypes.c_int64, _dp, _dp,
                                     ctypes.c_int64, _i64p, ctypes.c_int64, _dp, _dp]
        lib.orc_rmsnorm.argtypes = [_dp, _dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_double, _dp]
        lib.orc_swiglu.argtypes = [_dp, _dp, ctypes.c_int64, _dp]
        lib.orc_argmax.argtypes = [_dp, ctypes.c_int64, ctypes.c_int64, _i64p]
        lib.orc_gelu_tanh_gate.argtypes = [_dp, _dp, ctypes.c_int64, _dp]
        lib.orc_set_codebook.argtypes = [ctypes.POINTER(ctypes.c_int8)]
        lib.orc_qk_norm_rope.argtypes = [_dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_int64, _dp, _dp,
                                         ctypes.c_double, _dp, _dp]
        lib.orc_moe.argtypes = [ctypes.c_int, _u8p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                _dp, ctypes.c_int64, _i32p, _dp, ctypes.c_int64, _i64p,
                                ctypes.c_int64, _dp, _dp]
        _lib = lib
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a, ctype):
    return a.ctypes.data_as(ctype)


def set_codebook(cb) -> None:
    """Install the 16-entry signed codebook the IQ4 decodes use (an input: the pages print none)."""
    c = _c(np.asarray(cb).reshape(16), np.int8)
    _load().orc_set_codebook(c.ctypes.data_as(ctypes.POINTER(ctypes.c_int8)))


def threads() -> int:
    """Threads the oracle's OpenMP loops use (``OMP_NUM_THREADS`` or all cores)."""
    return int(_load().orc_threads())


def set_threads(n: int) -> int:
    """Use n OpenMP threads from now on; returns the count in effect."""
    return int(_load().orc_set_threads(int(n)))


def f16(bits: int) -> float:
    return float(_load().orc_f16(int(bits) & 0xFFFF))


def block_bytes(fmt: int) -> int:
    return int(_load().orc_block_bytes(fmt))


def block_weights(fmt: int) -> int:
    return int(_load().orc_block_weights(fmt))


def row_bytes(fmt: int, K: int) -> int:
    rb = int(_load().orc_row_bytes(fmt, K))
    if rb < 0:
        raise ValueError(f"format {fmt} cannot hold K={K}")
    return rb


def q4k_scale_min(scales12: bytes | np.ndarray, j: int) -> tuple[int, int]:
    s = _c(np.frombuffer(bytes(scales12), dtype=np.uint8), np.uint8)
    sc, m = ctypes.c_int(), ctypes.c_int()
    _load().orc_q4k_scale_min(_ptr(s, _u8p), j, ctypes.byref(sc), ctypes.byref(m))
    return sc.value, m.value


def dequant(fmt: int, W: np.ndarray, K: int) -> np.ndarray:
    """Dequantize every row of W (uint8 [N, row_bytes]) to f64 [N, K]."""
    W = _c(W, np.uint8).reshape(-1, row_bytes(fmt, K))
    out = np.empty((W.shape[0], K), dtype=np.float64)
    lib = _load()
    for n in range(W.shape[0]):
        row = W[n]
        if lib.orc_dequant_row(fmt, _ptr(row, _u8p), K, _ptr(out[n], _dp)) != 0:
            raise ValueError("dequant failed")
    return out


def _rows_arg(rows, N):
    if rows is None:
        return None, N
    r = _c(rows, np.int64)
    return r, r.shape[0]


def gemv(fmt: int, W: np.ndarray, N: int, K: int, v: np.ndarray, rows=None):
    """y[nb, nrows] = W[rows] v^T in f64 and A = sum_k |w v| (tolerance scale)."""
    v = _c(v, np.float64).reshape(-1, K)
    W = _c(W, np.uint8).reshape(N, row_bytes(fmt, K))
    r, nr = _rows_arg(rows, N)
    y = np.empty((v.shape[0], nr), dtype=np.float64)
    A = np.empty_like(y)
    rc = _load().orc_gemv(fmt, _ptr(W, _u8p), N, K, _ptr(v, _dp), v.shape[0],
                          None if r is None else _ptr(r, _i64p), nr, _ptr(y, _dp), _ptr(A, _dp))
    if rc:
        raise ValueError("oracle gemv failed")
    return y, A


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    gamma = _c(gamma, np.float64)
    K = gamma.shape[0]
    x = _c(x, np.float64).reshape(-1, K)
    out = np.empty_like(x)
    _load().orc_rmsnorm(_ptr(x, _dp), _ptr(gamma, _dp), x.shape[0], K, float(eps), _ptr(out, _dp))
    return out


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = _c(g, np.float64)
    u = _c(u, np.float64)
    assert g.shape == u.shape
    h = np.empty_like(g)
    _load().orc_swiglu(_ptr(g, _dp), _ptr(u, _dp), g.size, _ptr(h, _dp))
    return h


def gelu_tanh_gate(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = _c(g, np.float64)
    u = _c(u, np.float64)
    assert g.shape == u.shape
    h = np.empty_like(g)
    _load().orc_gelu_tanh_gate(_ptr(g, _dp), _ptr(u, _dp), g.size, _ptr(h, _dp))
    return h


def qk_norm_rope(qkv: np.ndarray, n_q_heads: int, n_kv_heads: int, head_dim: int, rope_half: int,
                 q_gamma, k_gamma, eps: float, rope_cos: np.ndarray, rope_sin: np.ndarray):
    """Per-head QK RMSNorm + RoPE of a QKV output [nb][(nq + 2 nkv) hd]; returns a new array."""
    row = (n_q_heads + 2 * n_kv_heads) * head_dim
    y = _c(qkv, np.float64).reshape(-1, row).copy()
    nb = y.shape[0]
    cs = _c(rope_cos, np.float64).reshape(nb, rope_half)
    sn = _c(rope_sin, np.float64).reshape(nb, rope_half)
    qg = None if q_gamma is None else _c(q_gamma, np.float64)
    kg = None if k_gamma is None else _c(k_gamma, np.float64)
    _load().orc_qk_norm_rope(_ptr(y, _dp), nb, n_q_heads, n_kv_heads, head_dim, rope_half,
                             None if qg is None else _ptr(qg, _dp),
                             None if kg is None else _ptr(kg, _dp), float(eps),
                             _ptr(cs, _dp), _ptr(sn, _dp))
    return y


def argmax(y: np.ndarray) -> np.ndarray:
    y = _c(y, np.float64)
    y2 = y.reshape(-1, y.shape[-1])
    idx = np.empty(y2.shape[0], dtype=np.int64)
    _load().orc_argmax(_ptr(y2, _dp), y2.shape[0], y2.shape[1], _ptr(idx, _i64p))
    return idx


# --------------------------------------------------------------------------- composites

def qgemv(fmt, W, N, K, x, rows=None):
    return gemv(fmt, W, N, K, x, rows)


def qgemv_nrm(fmt, W, N, K, x, gamma, eps, rows=None):
    return gemv(fmt, W, N, K, rmsnorm(x, gamma, eps), rows)


def qgemv_res(fmt, W, N, K, x, r, rows=None):
    v = _c(x, np.float64).reshape(-1, K)
    r = _c(r, np.float64).reshape(v.shape[0], N)
    W = _c(W, np.uint8).reshape(N, row_bytes(fmt, K))
    ri, nr = _rows_arg(rows, N)
    y = np.empty((v.shape[0], nr), dtype=np.float64)
    A = np.empty_like(y)
    rc = _load().orc_gemv_res(fmt, _ptr(W, _u8p), N, K, _ptr(v, _dp), _ptr(r, _dp), v.shape[0],
                              None if ri is None else _ptr(ri, _i64p), nr, _ptr(y, _dp),
                              _ptr(A, _dp))
    if rc:
        raise ValueError("oracle gemv_res failed")
    return y, A


def qgemv_gus_nrm(fmt, Wg, Wu, N, K, x, gamma, eps, rows=None):
    """Returns (h, g, u, Ag, Au) with h = silu(g) * u."""
    n = rmsnorm(x, gamma, eps)
    g, Ag = gemv(fmt, Wg, N, K, n, rows)
    u, Au = gemv(fmt, Wu, N, K, n, rows)
    return swiglu(g, u), g, u, Ag, Au


def qgemv_nrm_bias(fmt, W, N, K, x, gamma, eps, bias, rows=None):
    """y = W rmsnorm(x) + bias ("honeycrisp mod.rs", pipe_q8_nrm_mb64_bias: bias[row] added at
    the output); A as for the GEMV."""
    y, A = gemv(fmt, W, N, K, rmsnorm(x, gamma, eps), rows)
    b = _c(bias, np.float64)
    return y + (b if rows is None else b[np.asarray(rows)])[None, :], A


def qgemv_gus_act_nrm(fmt, Wg, Wu, N, K, x, gamma, eps, act, rows=None):
    """Returns (h, g, u, Ag, Au) with h = act(g) * u; act 0 = silu, 1 = GELU (tanh form)."""
    n = rmsnorm(x, gamma, eps)
    g, Ag = gemv(fmt, Wg, N, K, n, rows)
    u, Au = gemv(fmt, Wu, N, K, n, rows)
    h = swiglu(g, u) if act == 0 else gelu_tanh_gate(g, u)
    return h, g, u, Ag, Au


def qgemv_argmax(fmt, W, N, K, x):
    y, A = gemv(fmt, W, N, K, x)
    return y, A, argmax(y)


def qgemv_moe(fmt, W, n_exp, N, K, x, ids, p, rows=None):
    x = _c(x, np.float64).reshape(-1, K)
    nb = x.shape[0]
    ids = _c(ids, np.int32).reshape(nb, -1)
    topk = ids.shape[1]
    p = _c(p, np.float64).reshape(nb, topk)
    W = _c(W, np.uint8).reshape(-1)
    ri, nr = _rows_arg(rows, N)
    y = np.empty((nb, nr), dtype=np.float64)
    A = np.empty_like(y)
    rc = _load().orc_moe(fmt, _ptr(W, _u8p), n_exp, N, K, _ptr(x, _dp), nb, _ptr(ids, _i32p),
                         _ptr(p, _dp), topk, None if ri is None else _ptr(ri, _i64p), nr,
                         _ptr(y, _dp), _ptr(A, _dp))
    if rc:
        raise ValueError("oracle moe failed (expert id out of range?)")
    return y, A

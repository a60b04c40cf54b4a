"""GPU parity on inputs built to break inexact arithmetic, and on the accepted shapes the common
workloads do not reach.

* Sparse weights: blocks whose weights are mostly zero (Q4_0 nibble 8, Q8_0 byte 0) with one to
  three non-zero weights, against same-sign x.  A kernel that removes a weight offset by
  subtracting a second, offset-only sum loses the small products in the rounding of the large
  ones; the per-output bound 1e-3 sum |w x| has to hold here too.
* The integer brute force (Q4_0, Q8_0, Q4_K; K = 32, 64, 256): d = 2^-k and small-integer x make
  every product and partial sum exact, so the GPU must equal the f64 oracle bit for bit, at every
  batch size (vector and matrix-core paths).
* Q4_0 against its exact Q8_0 upcast ("Crate inferencelayer" docs, q4_0_to_q8_0n: d8 = d4,
  q8 = nib - 8): on integer inputs both formats give the same bits.
* Shapes the matrix-core kernel does not take at nb >= 5 (K > 4096, the norm prologue with
  K > 2048): batches of at most 4 rows on the vector path where its rows fit (<= 256 chunks), else
  the K-tiled kernel, which also serves rows longer than 256 chunks at nb <= 4; and Q8_0 bytes of
  -128.
"""
import numpy as np
import pytest

from gpu_common import (assert_within, dev, gpu_matrix, gus_tol, host, require_gpu, say,
                        tol_gemv, torch)

import dequant_gemv_q4_amd as q
from dequant_gemv_q4_amd import device as D
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    oracle.build(force=False)


def _gemv(fmt, W, N, K, x):
    nb = x.shape[0]
    y = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv(fmt, gpu_matrix(fmt, W, N, K), N, K, dev(x), nb, y)
    return host(y)


def _sparse_matrix(fmt, g, N, K, nz_max=3):
    """Blocks of mostly-zero weights: 1..nz_max non-zero weights per 32 (Q4_0 / Q8_0), or the
    Q4_K super-block with d = dmin, every sc = 1 and m = 8 (w = d (q - 8)) and mostly q = 8."""
    W = wl.matrix(fmt, g, N, K).reshape(N, -1, wl.BLOCK_BYTES[fmt]).copy()
    if fmt == q.Q4_0:
        nib = np.full((N, W.shape[1], 32), 8, dtype=np.int64)
    elif fmt == q.Q8_0:
        nib = np.zeros((N, W.shape[1], 32), dtype=np.int64)
    else:
        nib = np.full((N, W.shape[1], 256), 8, dtype=np.int64)
    per = nib.shape[2]
    for n in range(N):
        for b in range(nib.shape[1]):
            k = int(g.integers(1, nz_max + 1))
            pos = g.choice(per, size=k, replace=False)
            if fmt == q.Q8_0:
                nib[n, b, pos] = g.integers(1, 128, size=k) * g.choice([-1, 1], size=k)
            else:
                nib[n, b, pos] = g.choice([v for v in range(16) if v != 8], size=k)
    if fmt == q.Q4_0:
        W[..., 2:] = (nib[..., :16] | (nib[..., 16:] << 4)).astype(np.uint8)
    elif fmt == q.Q8_0:
        W[..., 2:] = nib.astype(np.int8).view(np.uint8)
    else:
        W[..., 2:4] = W[..., 0:2]                                   # dmin = d
        W[..., 4:16] = np.array([1, 1, 1, 1, 8, 8, 8, 8, 0x81, 0x81, 0x81, 0x81], np.uint8)
        for c in range(4):
            lo = nib[..., 64 * c:64 * c + 32]
            hi = nib[..., 64 * c + 32:64 * c + 64]
            W[..., 16 + 32 * c:16 + 32 * c + 32] = (lo | (hi << 4)).astype(np.uint8)
    return W.reshape(N, -1)


SPARSE_CASES = [(q.Q4_0, 64, 32, 1), (q.Q4_0, 64, 64, 2), (q.Q4_0, 50, 2048, 1),
                (q.Q4_0, 40, 64, 4), (q.Q4_0, 48, 64, 8), (q.Q4_0, 33, 2048, 16),
                (q.Q8_0, 64, 32, 1), (q.Q8_0, 50, 64, 3), (q.Q8_0, 40, 1536, 16),
                (q.Q4_K, 64, 256, 1), (q.Q4_K, 40, 2048, 2), (q.Q4_K, 33, 512, 9)]


@pytest.mark.parametrize("fmt,N,K,nb", SPARSE_CASES)
def test_sparse_weights_same_sign_x(fmt, N, K, nb):
    say(f"sparse fmt={fmt} N={N} K={K} nb={nb}")
    g = wl.rng(900 + fmt, N * 3 + K + nb)
    W = _sparse_matrix(fmt, g, N, K)
    x = g.uniform(0.9, 1.0, size=(nb, K)).astype(np.float32)
    y = _gemv(fmt, W, N, K, x)
    yr, A = oracle.gemv(fmt, W, N, K, x)
    assert_within(y, yr, tol_gemv(A, yr), f"sparse fmt={fmt} N={N} K={K} nb={nb}")


@pytest.mark.parametrize("fmt,K", [(q.Q4_0, 64), (q.Q8_0, 64), (q.Q4_K, 256)])
def test_sparse_weights_routed_experts(fmt, K):
    say(f"sparse moe fmt={fmt} K={K}")
    n_exp, N, nb, topk = 6, 64, 5, 3
    g = wl.rng(950 + fmt, K)
    W = _sparse_matrix(fmt, g, n_exp * N, K)
    x = g.uniform(0.9, 1.0, size=(nb, K)).astype(np.float32)
    ids, p = wl.route_top_k(g.standard_normal((nb, n_exp)), topk)
    ws = D.workspace(q.OP_MOE, fmt, N, K, nb, n_exp, topk)
    y = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv_moe(fmt, gpu_matrix(fmt, W, n_exp * N, K), n_exp, N, K, dev(x), nb, dev(ids), dev(p),
                topk, y, ws)
    yr, A = oracle.qgemv_moe(fmt, W, n_exp, N, K, x, ids, p)
    assert_within(host(y), yr, tol_gemv(A, yr), f"sparse moe fmt={fmt}")


def _integer_matrix(fmt, g, N, K):
    """Random quants with every scale a power of two (d = 2^-k, Q4_K: dmin = 2^-j too)."""
    W = wl.matrix(fmt, g, N, K).reshape(N, -1, wl.BLOCK_BYTES[fmt]).copy()
    ns = 2 if fmt == q.Q4_K else 1
    for s in range(ns):
        e = g.integers(2, 7, size=W.shape[:2])
        W[..., 2 * s:2 * s + 2] = (2.0 ** -e).astype("<f2")[..., None].view(np.uint8)
    if fmt == q.Q8_0:
        W[0, 0, 2:] = 0x80                                          # a block of -128 bytes
    return W.reshape(N, -1)


@pytest.mark.parametrize("fmt,K", [(q.Q4_0, 32), (q.Q4_0, 64), (q.Q8_0, 32), (q.Q8_0, 64),
                                   (q.Q4_K, 256)])
@pytest.mark.parametrize("nb", [1, 2, 4, 5, 8, 16])
def test_integer_brute_force_is_bitwise(fmt, K, nb):
    say(f"integer fmt={fmt} K={K} nb={nb}")
    N = 16
    g = wl.rng(980 + fmt, K * 17 + nb)
    W = _integer_matrix(fmt, g, N, K)
    x = g.integers(-7, 8, size=(nb, K)).astype(np.float32)
    y = _gemv(fmt, W, N, K, x)
    yr, _ = oracle.gemv(fmt, W, N, K, x)
    assert np.array_equal(y.astype(np.float64), yr), (fmt, K, nb)


@pytest.mark.parametrize("nb", [1, 3, 9])
def test_q4_0_equals_its_q8_0_upcast(nb):
    say(f"upcast nb={nb}")
    N, K = 48, 2048
    g = wl.rng(990, nb)
    W4 = _integer_matrix(q.Q4_0, g, N, K).reshape(N, -1, 18)
    nib = np.concatenate([W4[..., 2:] & 15, W4[..., 2:] >> 4], axis=-1).astype(np.int16)
    W8 = np.empty(W4.shape[:2] + (34,), np.uint8)
    W8[..., :2] = W4[..., :2]
    W8[..., 2:] = (nib - 8).astype(np.int8).view(np.uint8)
    x = g.integers(-7, 8, size=(nb, K)).astype(np.float32)
    y4 = _gemv(q.Q4_0, W4.reshape(N, -1), N, K, x)
    y8 = _gemv(q.Q8_0, W8.reshape(N, -1), N, K, x)
    assert np.array_equal(y4, y8)


TILED_CASES = [(q.Q4_0, 70, 16384, 1), (q.Q4_0, 33, 65536, 2), (q.Q8_0, 50, 8192, 2),
               (q.Q8_0, 40, 8192, 3), (q.Q4_0, 40, 8192, 8), (q.Q8_0, 31, 6144, 12),
               (q.Q4_0, 40, 16384, 8), (q.Q4_0, 37, 8192, 13)]


@pytest.mark.parametrize("fmt,N,K,nb", TILED_CASES)
def test_k_tiled_shapes(fmt, N, K, nb):
    say(f"tiled fmt={fmt} N={N} K={K} nb={nb}")
    g = wl.rng(1000 + fmt, N + K + nb)
    W = wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (nb, K))
    y = _gemv(fmt, W, N, K, x)
    yr, A = oracle.gemv(fmt, W, N, K, x)
    assert_within(y, yr, tol_gemv(A, yr), f"tiled fmt={fmt} N={N} K={K} nb={nb}")


@pytest.mark.parametrize("fmt,N,K,nb", [(q.Q4_0, 60, 4096, 6), (q.Q8_0, 45, 4096, 8),
                                       (q.Q4_0, 50, 16384, 6)])
def test_k_tiled_norm_and_gated(fmt, N, K, nb):
    say(f"tiled nrm/gus fmt={fmt} N={N} K={K} nb={nb}")
    g = wl.rng(1100 + fmt, N + nb)
    W = wl.matrix(fmt, g, N, K)
    Wu = wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (nb, K))
    gamma = wl.gamma_f32(g, K)
    y = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv_nrm(fmt, gpu_matrix(fmt, W, N, K), N, K, dev(x), dev(gamma), 1e-5, nb, y)
    yr, A = oracle.qgemv_nrm(fmt, W, N, K, x, gamma, 1e-5)
    assert_within(host(y), yr, tol_gemv(A, yr), f"tiled nrm fmt={fmt}")
    h = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv_gus_nrm(fmt, gpu_matrix(fmt, W, N, K), gpu_matrix(fmt, Wu, N, K), N, K, dev(x),
                    dev(gamma), 1e-5, nb, h)
    hr, gr, ur, Ag, Au = oracle.qgemv_gus_nrm(fmt, W, Wu, N, K, x, gamma, 1e-5)
    assert_within(host(h), hr, gus_tol(gr, ur, Ag, Au), f"tiled gus fmt={fmt}")


@pytest.mark.parametrize("N,K,nb", [(300, 1536, 1), (77, 2048, 4), (65, 1024, 16)])
def test_q8_0_minus_128_bytes(N, K, nb):
    say(f"q8 -128 N={N} K={K} nb={nb}")
    g = wl.rng(1200, N + nb)
    W = wl.q8_0_matrix(g, N, K).reshape(N, -1, 34).copy()
    mask = g.random(W[..., 2:].shape) < 0.25
    W[..., 2:][mask] = 0x80
    W = W.reshape(N, -1)
    x = wl.normal_f32(g, (nb, K))
    y = _gemv(q.Q8_0, W, N, K, x)
    yr, A = oracle.gemv(q.Q8_0, W, N, K, x)
    assert_within(y, yr, tol_gemv(A, yr), f"q8 -128 N={N} K={K} nb={nb}")


@pytest.mark.parametrize("nb", [5, 7, 16])
def test_batched_vector_path_epilogues(nb):
    """5..16 rows of K = 8192 run as batches of at most 4 rows on the vector path: the residual
    (in place), norm + bias and argmax epilogues of each batch take their own rows (and the argmax
    its own index slots)."""
    fmt, N, K = q.Q4_0, 300, 8192
    say(f"batched vector path nb={nb}")
    g = wl.rng(1200, nb)
    W = wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (nb, K))
    Wd = gpu_matrix(fmt, W, N, K)

    res = wl.normal_f32(g, (nb, N))
    yres = dev(res.copy())
    q.qgemv_res(fmt, Wd, N, K, dev(x), yres, nb, yres)            # in place
    yr, A = oracle.qgemv_res(fmt, W, N, K, x, res)
    assert_within(host(yres), yr, tol_gemv(A, yr), "res")

    gamma = wl.gamma_f32(g, K)
    bias = wl.normal_f32(g, (N,))
    yb = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv_nrm_bias(fmt, Wd, N, K, dev(x), dev(gamma), 1e-5, dev(bias), nb, yb)
    yr, A = oracle.qgemv_nrm_bias(fmt, W, N, K, x, gamma, 1e-5, bias)
    assert_within(host(yb), yr, tol_gemv(A, yr), "nrm bias")

    logits = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    idx = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
    ws = D.workspace(q.OP_ARGMAX, fmt, N, K, nb)
    q.qgemv_argmax(fmt, Wd, N, K, dev(x), nb, logits, idx, ws)
    lg, ig = host(logits), host(idx)
    for r in range(nb):
        i = int(ig[r])
        assert 0 <= i < N and lg[r, i] == lg[r].max() and int(np.argmax(lg[r])) == i, r
    yr, A = oracle.gemv(fmt, W, N, K, x)
    assert_within(lg, yr, tol_gemv(A, yr), "argmax logits")

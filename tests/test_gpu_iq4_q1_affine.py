"""The codebook, sign and affine formats on the GPU against the f64 oracle: IQ4_NL and IQ4_XS
("Crate inferencelayer" docs, gemv_iq4_nl_k_lcpp_src, gemv_iq4_xs_k_lcpp_src: a 16-entry signed
codebook, here an input stored with the packed matrix), Q1_0 (gemv_q1_k_lcpp_src: one sign bit
per weight and one f16 scale per 128) and the affine Q4 ("Module gpu", struct Q, w = s q + c),
through every GEMV entry point, on the streaming kernel (nb <= 4, rows split over 1, 2 or 4
waves) and the K-tiled kernel (nb >= 5); integer inputs bit for bit; IQ4_NL under the codebook
i - 8 bit for bit equal to Q4_0 on the same bytes."""
import numpy as np
import pytest

from gpu_common import assert_within, dev, gus_tol, host, require_gpu, say, tol_gemv, torch

import dequant_gemv_q4_amd as q
from dequant_gemv_q4_amd import device as D
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

NEW = [q.IQ4_NL, q.IQ4_XS, q.Q1_0, q.AQ4]
CB = wl.iq4_codebook()
LINEAR_CB = np.arange(16) - 8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    oracle.build(force=False)


def _cb(fmt, cb=CB):
    return cb if fmt in (q.IQ4_NL, q.IQ4_XS) else None


def _packed(fmt, W, N, K, cb=CB):
    return D.pack(fmt, W, N, K, codebook=_cb(fmt, cb))


def _oracle_gemv(fmt, W, N, K, x, cb=CB):
    oracle.set_codebook(cb)
    return oracle.gemv(fmt, W, N, K, x)


def _gemv(fmt, Wp, N, K, x):
    nb = x.shape[0]
    y = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv(fmt, Wp, N, K, dev(x), nb, y)
    return host(y)


@pytest.mark.parametrize("fmt", NEW)
def test_pack_planes(fmt):
    """Quant bytes and scale bytes land in their planes unchanged; the IQ4 codebook follows."""
    N, K = 13, 512
    g = np.random.default_rng(5)
    W = wl.matrix(fmt, g, N, K)
    Wp = host(_packed(fmt, W, N, K))
    blk = W.reshape(-1, wl.BLOCK_BYTES[fmt])
    sb = {q.IQ4_NL: 2, q.IQ4_XS: 8, q.Q1_0: 2, q.AQ4: 4}[fmt]
    qs, sc = blk[:, sb:].reshape(-1), blk[:, :sb].reshape(-1)
    r256 = lambda v: (v + 255) // 256 * 256
    sc_off = r256(qs.size)
    assert np.array_equal(Wp[:qs.size], qs)
    assert np.array_equal(Wp[sc_off:sc_off + sc.size], sc)
    cb_off = sc_off + r256(sc.size)
    if fmt in (q.IQ4_NL, q.IQ4_XS):
        assert np.array_equal(Wp[cb_off:cb_off + 16].view(np.int8), CB)
        assert Wp.size == cb_off + 256
    else:
        assert Wp.size == cb_off
    assert Wp.size == q.qgemv_packed_bytes(fmt, N, K)


CASES = [(f, N, K, nb) for f in NEW for (N, K, nb) in
         [(1, 256, 1), (37, 256, 3), (517, 2048, 1), (300, 4096, 2), (129, 8192, 1),
          (201, 2048, 4), (77, 1792, 5), (150, 2048, 8), (65, 2048, 16), (33, 4096, 12),
          (40, 8192, 6)]]


@pytest.mark.parametrize("fmt,N,K,nb", CASES)
def test_qgemv_new_formats(fmt, N, K, nb):
    say(f"qgemv fmt={fmt} N={N} K={K} nb={nb}")
    g = wl.rng(3000 + fmt, N * 7 + K + nb)
    W = wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (nb, K))
    y = _gemv(fmt, _packed(fmt, W, N, K), N, K, x)
    yr, A = _oracle_gemv(fmt, W, N, K, x)
    assert_within(y, yr, tol_gemv(A, yr), f"qgemv fmt={fmt} N={N} K={K} nb={nb}")


def _exact_matrix(fmt, g, N, K):
    """Power-of-two scales (and affine biases that are integer multiples of them; IQ4_XS
    sub-scales ls - 32 in [-4, 4]), so that every partial sum of an integer x is exact in f32."""
    bb = wl.BLOCK_BYTES[fmt]
    W = wl.matrix(fmt, g, N, K).reshape(N, -1, bb).copy()
    nbk = W.shape[1]
    s = 2.0 ** -g.integers(2, 7, size=(N, nbk))
    W[..., 0:2] = s.astype("<f2")[..., None].view(np.uint8)
    if fmt == q.AQ4:
        W[..., 2:4] = (-s * g.integers(0, 16, size=(N, nbk))).astype("<f2")[..., None].view(np.uint8)
    if fmt == q.IQ4_XS:
        ls = g.integers(28, 37, size=(N, nbk, 8))
        sh = np.zeros((N, nbk), np.uint32)
        sl = np.zeros((N, nbk), np.uint32)
        for j in range(8):
            sh |= ((ls[..., j] >> 4) & 3).astype(np.uint32) << (2 * j)
            sl |= (ls[..., j] & 15).astype(np.uint32) << (4 * j)
        W[..., 2:4] = sh.astype("<u2")[..., None].view(np.uint8)
        W[..., 4:8] = sl.astype("<u4")[..., None].view(np.uint8)
    return W.reshape(N, -1)


@pytest.mark.parametrize("fmt", NEW)
@pytest.mark.parametrize("nb", [1, 3, 4, 7, 16])
def test_integer_inputs_bitwise(fmt, nb):
    say(f"integer fmt={fmt} nb={nb}")
    N, K = 24, 256
    g = wl.rng(3100 + fmt, nb)
    W = _exact_matrix(fmt, g, N, K)
    x = g.integers(-3, 4, size=(nb, K)).astype(np.float32)
    y = _gemv(fmt, _packed(fmt, W, N, K), N, K, x)
    yr, _ = _oracle_gemv(fmt, W, N, K, x)
    assert np.array_equal(y.astype(np.float64), yr)


@pytest.mark.parametrize("nb", [1, 2, 4, 6, 16])
def test_iq4_nl_with_linear_codebook_equals_q4_0(nb):
    """Codebook entry i = i - 8 makes IQ4_NL's bytes a Q4_0 matrix: the two must agree bit for bit.
    Up to 4 batch rows both run the streaming kernel (the same products in the same order, any
    scales); from 5 rows Q4_0 runs on the matrix cores and IQ4_NL on the K-tiled kernel, whose
    sums are ordered differently, so the scales there are powers of two (every sum exact)."""
    say(f"iq4_nl linear codebook nb={nb}")
    N, K = 300, 2048
    g = wl.rng(3200, nb)
    W = wl.q4_0_matrix(g, N, K)
    if nb > 4:
        W = W.reshape(N, -1, 18).copy()
        W[..., 0:2] = (2.0 ** -g.integers(2, 7, size=W.shape[:2])).astype("<f2")[..., None].view(np.uint8)
        W = W.reshape(N, -1)
    x = g.integers(-7, 8, size=(nb, K)).astype(np.float32)
    y_nl = _gemv(q.IQ4_NL, _packed(q.IQ4_NL, W, N, K, LINEAR_CB), N, K, x)
    y_q4 = _gemv(q.Q4_0, D.pack(q.Q4_0, W, N, K), N, K, x)
    assert np.array_equal(y_nl, y_q4)


@pytest.mark.parametrize("nb", [1, 5])
def test_affine_centred_cancellation(nb):
    """Affine blocks whose weights mostly sit at zero (c = -s q0 with most nibbles q0) and
    same-sign x: the centred arithmetic keeps the error relative to sum |w x|."""
    say(f"aq4 cancellation nb={nb}")
    N, K = 48, 1024
    g = wl.rng(3300, nb)
    W = wl.aq4_matrix(g, N, K).reshape(N, -1, 20).copy()
    s = g.uniform(0.01, 0.02, size=W.shape[:2])
    q0 = g.integers(0, 16, size=W.shape[:2])
    W[..., 0:2] = s.astype("<f2")[..., None].view(np.uint8)
    sf = W[..., 0:2].copy().view("<f2")[..., 0].astype(np.float64)
    W[..., 2:4] = (-sf * q0).astype("<f2")[..., None].view(np.uint8)
    W[..., 4:20] = (q0 * 17).astype(np.uint8)[..., None]
    for n in range(N):
        for b in range(W.shape[1]):
            pos = g.choice(16, size=2, replace=False)
            W[n, b, 4 + pos] = g.integers(0, 256, size=2, dtype=np.uint8)
    W = W.reshape(N, -1)
    x = g.uniform(0.9, 1.0, size=(nb, K)).astype(np.float32)
    y = _gemv(q.AQ4, _packed(q.AQ4, W, N, K), N, K, x)
    yr, A = _oracle_gemv(q.AQ4, W, N, K, x)
    assert_within(y, yr, tol_gemv(A, yr), "aq4 cancellation")


@pytest.mark.parametrize("fmt,N,K,nb", [(q.IQ4_NL, 300, 2048, 1), (q.IQ4_XS, 200, 2048, 3),
                                        (q.Q1_0, 130, 4096, 2), (q.AQ4, 170, 2048, 1),
                                        (q.IQ4_XS, 70, 2048, 9), (q.Q1_0, 50, 2048, 6),
                                        (q.AQ4, 60, 4096, 7), (q.IQ4_NL, 90, 1024, 16)])
def test_fused_ops_new_formats(fmt, N, K, nb):
    say(f"fused fmt={fmt} N={N} K={K} nb={nb}")
    g = wl.rng(3400 + fmt, N + nb)
    W, Wu = wl.matrix(fmt, g, N, K), wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (nb, K))
    gamma = wl.gamma_f32(g, K)
    r = wl.normal_f32(g, (nb, N))
    bias = wl.normal_f32(g, (N,))
    Wp, Wup = _packed(fmt, W, N, K), _packed(fmt, Wu, N, K)
    oracle.set_codebook(CB)
    y = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv_nrm(fmt, Wp, N, K, dev(x), dev(gamma), 1e-5, nb, y)
    yr, A = oracle.qgemv_nrm(fmt, W, N, K, x, gamma, 1e-5)
    assert_within(host(y), yr, tol_gemv(A, yr), f"nrm fmt={fmt}")
    q.qgemv_nrm_bias(fmt, Wp, N, K, dev(x), dev(gamma), 1e-5, dev(bias), nb, y)
    yr, A = oracle.qgemv_nrm_bias(fmt, W, N, K, x, gamma, 1e-5, bias)
    assert_within(host(y), yr, tol_gemv(A, yr), f"nrm bias fmt={fmt}")
    q.qgemv_res(fmt, Wp, N, K, dev(x), dev(r), nb, y)
    yr, A = oracle.qgemv_res(fmt, W, N, K, x, r)
    assert_within(host(y), yr, tol_gemv(A, yr), f"res fmt={fmt}")
    q.qgemv_gus_nrm(fmt, Wp, Wup, N, K, dev(x), dev(gamma), 1e-5, nb, y)
    hr, gr, ur, Ag, Au = oracle.qgemv_gus_nrm(fmt, W, Wu, N, K, x, gamma, 1e-5)
    assert_within(host(y), hr, gus_tol(gr, ur, Ag, Au), f"gus fmt={fmt}")
    logits = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    idx = torch.empty((nb,), dtype=torch.int32, device="cuda")
    q.qgemv_argmax(fmt, Wp, N, K, dev(x), nb, logits, idx, D.workspace(q.OP_ARGMAX, fmt, N, K, nb))
    yr, A = oracle.gemv(fmt, W, N, K, x)
    lg, ig = host(logits), host(idx)
    tol = tol_gemv(A, yr)
    assert_within(lg, yr, tol, f"argmax logits fmt={fmt}")
    for b in range(nb):
        i, m = int(ig[b]), int(np.argmax(yr[b]))
        assert int(np.argmax(lg[b])) == i
        assert i == m or yr[b, m] - yr[b, i] <= tol[b, m] + tol[b, i]


@pytest.mark.parametrize("nb", [2, 6])
def test_gate_and_up_keep_their_own_codebooks(nb):
    """The gated product reads each matrix's codebook from its own packed buffer."""
    say(f"gus two codebooks nb={nb}")
    fmt, N, K = q.IQ4_NL, 96, 2048
    g = wl.rng(3500, 1)
    W, Wu = wl.matrix(fmt, g, N, K), wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (nb, K))
    gamma = wl.gamma_f32(g, K)
    cb2 = (LINEAR_CB * 9).astype(np.int8)
    Wp, Wup = _packed(fmt, W, N, K, CB), _packed(fmt, Wu, N, K, cb2)
    y = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv_gus_nrm(fmt, Wp, Wup, N, K, dev(x), dev(gamma), 1e-5, nb, y)
    oracle.set_codebook(CB)
    gr, Ag = oracle.qgemv_nrm(fmt, W, N, K, x, gamma, 1e-5)
    oracle.set_codebook(cb2)
    ur, Au = oracle.qgemv_nrm(fmt, Wu, N, K, x, gamma, 1e-5)
    hr = gr / (1.0 + np.exp(-gr)) * ur
    assert_within(host(y), hr, gus_tol(gr, ur, Ag, Au), "gus two codebooks")

"""The high-bit formats on the GPU against the f64 oracle: Q5_0, Q5_K and Q6_K ("Crate
inferencelayer" docs: gemv_q5_0n_k_lcpp_src, gemv_q5k_k_lcpp_src, gemv_q6k_k_lcpp_src) through
every GEMV entry point, on the streaming kernel (nb <= 4, rows split over 1, 2 or 4 waves) and the
K-tiled kernel (nb >= 5, long rows); integer inputs bit for bit; Q5_0 against its exact Q8_0
upcast (q5_0_to_q8_0n: d8 = d5, q8 = q5 - 16)."""
import math

import numpy as np
import pytest

from gpu_common import (REL, assert_within, dev, gpu_matrix, gus_tol, host, require_gpu, say,
                        tol_gemv, torch)

import dequant_gemv_q4_amd as q
from dequant_gemv_q4_amd import device as D
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

NEW = [q.Q5_0, q.Q5_K, q.Q6_K]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    oracle.build(force=False)


def _gemv(fmt, W, N, K, x):
    nb = x.shape[0]
    y = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv(fmt, gpu_matrix(fmt, W, N, K), N, K, dev(x), nb, y)
    return host(y)


@pytest.mark.parametrize("fmt", NEW)
def test_pack_planes(fmt):
    """Quant bytes, scale bytes (and Q6_K's d values) land in their planes unchanged."""
    N, K = 13, 512
    g = np.random.default_rng(3)
    W = wl.matrix(fmt, g, N, K)
    Wp = host(gpu_matrix(fmt, W, N, K))
    blk = W.reshape(-1, wl.BLOCK_BYTES[fmt])
    r256 = lambda v: (v + 255) // 256 * 256
    if fmt == q.Q5_0:
        qs, sc = blk[:, 6:22].reshape(-1), blk[:, 0:2].reshape(-1)
    elif fmt == q.Q5_K:
        qs, sc = blk[:, 48:176].reshape(-1), blk[:, 0:16].reshape(-1)
    else:
        qs, sc = blk[:, 0:128].reshape(-1), blk[:, 192:208].reshape(-1)
    sc_off = r256(qs.size)
    assert np.array_equal(Wp[:qs.size], qs)
    assert np.array_equal(Wp[sc_off:sc_off + sc.size], sc)
    if fmt == q.Q6_K:
        hb_off = sc_off + r256(sc.size)
        d_off = hb_off + r256(N * K // 4)
        assert np.array_equal(Wp[d_off:d_off + 2 * blk.shape[0]], blk[:, 208:210].reshape(-1))
    assert Wp.size == q.qgemv_packed_bytes(fmt, N, K)


CASES = [(f, N, K, nb) for f in NEW for (N, K, nb) in
         [(1, 256, 1), (37, 256, 3), (517, 2048, 1), (300, 4096, 2), (129, 8192, 1),
          (201, 2048, 4), (77, 1536 if f == q.Q5_0 else 1792, 5), (150, 2048, 8),
          (65, 2048, 16), (33, 4096, 12), (40, 8192, 6)]]


@pytest.mark.parametrize("fmt,N,K,nb", CASES)
def test_qgemv_high_bit_formats(fmt, N, K, nb):
    say(f"qgemv fmt={fmt} N={N} K={K} nb={nb}")
    g = wl.rng(2000 + fmt, N * 7 + K + nb)
    W = wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (nb, K))
    y = _gemv(fmt, W, N, K, x)
    yr, A = oracle.gemv(fmt, W, N, K, x)
    assert_within(y, yr, tol_gemv(A, yr), f"qgemv fmt={fmt} N={N} K={K} nb={nb}")


def _pow2_scales(fmt, g, W):
    W = W.copy()
    if fmt == q.Q5_0:
        W[..., 0:2] = (2.0 ** -g.integers(2, 7, size=W.shape[:2])).astype("<f2")[..., None].view(np.uint8)
    elif fmt == q.Q5_K:
        for o in (0, 2):
            W[..., o:o + 2] = (2.0 ** -g.integers(2, 7, size=W.shape[:2])).astype("<f2")[..., None].view(np.uint8)
    else:
        W[..., 208:210] = (2.0 ** -g.integers(2, 7, size=W.shape[:2])).astype("<f2")[..., None].view(np.uint8)
    return W


@pytest.mark.parametrize("fmt", NEW)
@pytest.mark.parametrize("nb", [1, 3, 4, 7, 16])
def test_integer_inputs_bitwise(fmt, nb):
    say(f"integer fmt={fmt} nb={nb}")
    N, K = 24, 256 if fmt != q.Q5_0 else 64
    g = wl.rng(2100 + fmt, nb)
    W = _pow2_scales(fmt, g, wl.matrix(fmt, g, N, K).reshape(N, -1, wl.BLOCK_BYTES[fmt]))
    W = W.reshape(N, -1)
    x = g.integers(-7, 8, size=(nb, K)).astype(np.float32)
    y = _gemv(fmt, W, N, K, x)
    yr, _ = oracle.gemv(fmt, W, N, K, x)
    assert np.array_equal(y.astype(np.float64), yr)


@pytest.mark.parametrize("nb", [1, 4, 9])
def test_q5_0_equals_its_q8_0_upcast(nb):
    say(f"q5 upcast nb={nb}")
    N, K = 40, 2048
    g = wl.rng(2200, nb)
    W5 = _pow2_scales(q.Q5_0, g, wl.q5_0_matrix(g, N, K).reshape(N, -1, 22))
    qh = W5[..., 2:6].copy().view("<u4")[..., 0]
    W8 = np.empty(W5.shape[:2] + (34,), np.uint8)
    W8[..., :2] = W5[..., :2]
    for j in range(16):
        lo = (W5[..., 6 + j] & 15).astype(np.int16) | (((qh >> j) & 1) << 4).astype(np.int16)
        hi = (W5[..., 6 + j] >> 4).astype(np.int16) | (((qh >> (j + 16)) & 1) << 4).astype(np.int16)
        W8[..., 2 + j] = (lo - 16).astype(np.int8).view(np.uint8)
        W8[..., 18 + j] = (hi - 16).astype(np.int8).view(np.uint8)
    x = g.integers(-7, 8, size=(nb, K)).astype(np.float32)
    y5 = _gemv(q.Q5_0, W5.reshape(N, -1), N, K, x)
    y8 = _gemv(q.Q8_0, W8.reshape(N, -1), N, K, x)
    assert np.array_equal(y5, y8)


@pytest.mark.parametrize("fmt,N,K,nb", [(q.Q5_0, 300, 2048, 1), (q.Q5_K, 200, 2048, 3),
                                        (q.Q6_K, 130, 4096, 2), (q.Q5_K, 70, 2048, 9),
                                        (q.Q6_K, 50, 2048, 6)])
def test_fused_ops_high_bit_formats(fmt, N, K, nb):
    say(f"fused fmt={fmt} N={N} K={K} nb={nb}")
    g = wl.rng(2300 + fmt, N + nb)
    W, Wu = wl.matrix(fmt, g, N, K), wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (nb, K))
    gamma = wl.gamma_f32(g, K)
    r = wl.normal_f32(g, (nb, N))
    bias = wl.normal_f32(g, (N,))
    Wp, Wup = gpu_matrix(fmt, W, N, K), gpu_matrix(fmt, Wu, N, K)
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


@pytest.mark.parametrize("nb", [2, 9])
def test_q5_k_centred_cancellation(nb):
    """Q5_K sub-blocks whose weights mostly sit at one value (d sc q = dmin m for the common q,
    same-sign x): the centred arithmetic keeps the error relative to sum |w x| (streaming and
    matrix-core kernels)."""
    say(f"q5_k cancellation nb={nb}")
    N, K = 48, 512
    g = wl.rng(2400, 1)
    W = wl.q5_k_matrix(g, N, K).reshape(N, -1, 176).copy()
    W[..., 2:4] = W[..., 0:2]                                    # dmin = d
    W[..., 4:16] = np.array([1, 1, 1, 1, 0x54, 0x54, 0x54, 0x54, 0x41, 0x41, 0x41, 0x41], np.uint8)
    # every (sc, m) = (1, 20): w = d (q - 20); most q = 20 = nibble 4 with fifth bit 1
    W[..., 16:48] = 0xFF
    W[..., 48:176] = 0x44
    for n in range(N):
        for b in range(W.shape[1]):
            pos = g.choice(128, size=3, replace=False)
            W[n, b, 48 + pos] = g.integers(0, 256, size=3, dtype=np.uint8)
    W = W.reshape(N, -1)
    for j in range(8):
        assert oracle.q4k_scale_min(W[0, 4:16].tobytes(), j) == (1, 20)
    x = g.uniform(0.9, 1.0, size=(nb, K)).astype(np.float32)
    y = _gemv(q.Q5_K, W, N, K, x)
    yr, A = oracle.gemv(q.Q5_K, W, N, K, x)
    assert_within(y, yr, tol_gemv(A, yr), "q5_k cancellation")


def test_experts_reject_high_bit_formats():
    W = torch.zeros(q.qgemv_packed_bytes(q.Q5_K, 2 * 64, 256), dtype=torch.uint8, device="cuda")
    x = torch.zeros((1, 256), dtype=torch.float32, device="cuda")
    ids = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    p = torch.ones((1, 1), dtype=torch.float32, device="cuda")
    y = torch.empty((1, 64), dtype=torch.float32, device="cuda")
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(q.QgemvError) as e:
        q.qgemv_moe(q.Q5_K, W, 2, 64, 256, x, 1, ids, p, 1, y, ws)
    assert e.value.status == 2

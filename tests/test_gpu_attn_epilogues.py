"""Attention-side epilogues of the fused QKV and the gated MLP on the GPU against the oracle:
bias at the output of the norm + GEMV ("honeycrisp mod.rs", pipe_q8_nrm_mb64_bias), the GeluTanh
gated product (pipe_q8_large4_gus_nrm_gelu), and the per-head QK RMSNorm + RoPE
(pipe_qk_norm_rope) on the QKV output.

The QK-norm + RoPE step is held to f32 arithmetic on its own input (the GPU's QKV output, itself
checked at the GEMV bound): each output is a rotation of two normalized values n_e, n_p, so
|err| <= 2^-18 (|n_e| + |n_p|) covers the f32 sum of squares over at most 256 values, the square
root, the division and the two products (a few ulp each)."""
import math

import numpy as np
import pytest

from gpu_common import (REL, assert_within, dev, gpu_matrix, host, require_gpu, say, tol_gemv,
                        torch)

import dequant_gemv_q4_amd as q
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    oracle.build(force=False)


@pytest.mark.parametrize("fmt,N,K,nb", [(q.Q8_0, 2048, 1536, 1), (q.Q8_0, 2048, 1536, 4),
                                        (q.Q8_0, 2048, 1536, 16), (q.Q4_0, 515, 2048, 2),
                                        (q.Q4_K, 300, 2048, 3), (q.Q4_0, 77, 2048, 9)])
def test_nrm_bias(fmt, N, K, nb):
    say(f"nrm bias fmt={fmt} N={N} K={K} nb={nb}")
    g = wl.rng(1400 + fmt, N + nb)
    W = wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (nb, K))
    gamma = wl.gamma_f32(g, K)
    bias = wl.normal_f32(g, (N,))
    y = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv_nrm_bias(fmt, gpu_matrix(fmt, W, N, K), N, K, dev(x), dev(gamma), 1e-5, dev(bias), nb, y)
    yr, A = oracle.qgemv_nrm_bias(fmt, W, N, K, x, gamma, 1e-5, bias)
    assert_within(host(y), yr, tol_gemv(A, yr), f"nrm bias fmt={fmt} nb={nb}")


def gelu_tol(g, u, Ag, Au):
    """h = gelu(g) u from |dg| <= 1e-3 Ag, |du| <= 1e-3 Au; sup |gelu'| < 1.2 (tanh form)."""
    ge = g * 0.5 * (1 + np.tanh(math.sqrt(2 / math.pi) * (g + 0.044715 * g ** 3)))
    return REL * (1.2 * Ag * np.abs(u) + np.abs(ge) * Au) + REL * REL * 1.2 * Ag * Au


@pytest.mark.parametrize("fmt,N,K,nb", [(q.Q4_0, 1000, 2048, 1), (q.Q8_0, 300, 1536, 2),
                                        (q.Q4_K, 130, 2048, 1), (q.Q4_0, 77, 2048, 9),
                                        (q.Q4_0, 60, 4096, 6)])
def test_gus_gelu_tanh(fmt, N, K, nb):
    say(f"gus gelu fmt={fmt} N={N} K={K} nb={nb}")
    g = wl.rng(1500 + fmt, N + nb)
    Wg, Wu = wl.matrix(fmt, g, N, K), wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (nb, K))
    gamma = wl.gamma_f32(g, K)
    h = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv_gus_act_nrm(fmt, gpu_matrix(fmt, Wg, N, K), gpu_matrix(fmt, Wu, N, K), N, K, dev(x),
                        dev(gamma), 1e-5, q.ACT_GELU_TANH, nb, h)
    hr, gr, ur, Ag, Au = oracle.qgemv_gus_act_nrm(fmt, Wg, Wu, N, K, x, gamma, 1e-5, 1)
    assert_within(host(h), hr, gelu_tol(gr, ur, Ag, Au), f"gus gelu fmt={fmt}")


def _rope_tables(g, nb, rh, theta=1e6, hd=128):
    pos = g.integers(0, 4096, size=nb)
    j = np.arange(rh)
    ang = pos[:, None] / theta ** (2.0 * j[None, :] / hd)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


@pytest.mark.parametrize("nb,nq,nkv,hd,rh,norm", [(1, 12, 2, 128, 64, True), (4, 12, 2, 128, 64, True),
                                                  (16, 12, 2, 128, 64, True), (3, 8, 4, 64, 16, True),
                                                  (2, 5, 1, 256, 128, True), (2, 6, 2, 128, 32, False),
                                                  (1, 4, 0, 96, 48, True)])
def test_qk_norm_rope(nb, nq, nkv, hd, rh, norm):
    say(f"qk norm rope nb={nb} nq={nq} nkv={nkv} hd={hd} rh={rh} norm={norm}")
    g = wl.rng(1600, nb * 100 + hd + rh)
    row = (nq + 2 * nkv) * hd
    y = wl.normal_f32(g, (nb, row)) * np.float32(3.0)
    qg = wl.gamma_f32(g, hd) if norm else None
    kg = wl.gamma_f32(g, hd) if norm else None
    cs, sn = _rope_tables(g, nb, rh, hd=hd)
    yd = dev(y)
    q.qgemv_qk_norm_rope(yd, nb, nq, nkv, hd, rh, None if qg is None else dev(qg),
                         None if kg is None else dev(kg), 1e-6, dev(cs), dev(sn))
    got = host(yd)
    ref = oracle.qk_norm_rope(y, nq, nkv, hd, rh, qg, kg, 1e-6, cs, sn)
    # partner magnitudes: the normalized values before the rotation
    nrm = oracle.qk_norm_rope(y, nq, nkv, hd, rh, qg, kg, 1e-6, np.ones_like(cs), np.zeros_like(sn))
    part = nrm.copy()
    for h in range(nq + nkv):
        a = slice(h * hd, h * hd + rh)
        b = slice(h * hd + rh, h * hd + 2 * rh)
        part[:, a], part[:, b] = nrm[:, b], nrm[:, a]
    tol = 2.0 ** -18 * (np.abs(nrm) + np.abs(part))
    assert np.array_equal(got[:, (nq + nkv) * hd:], y[:, (nq + nkv) * hd:])   # V untouched
    assert_within(got, ref, tol, f"qk norm rope nb={nb} hd={hd}")


def test_qkv_chain_bias_norm_rope():
    """The Qwen2.5-style QKV workload (Q8_0 2048 x 1536, 12 Q heads and 2 KV heads of 128) with
    the bias, then the QK norm + RoPE on the GPU's own QKV output."""
    w = wl.qkv_q8(nb=4)
    a = w.arrays
    g = wl.rng(1700, 4)
    nb, nq, nkv, hd, rh = 4, 12, 2, 128, 64
    bias = wl.normal_f32(g, (w.N,))
    y = torch.empty((nb, w.N), dtype=torch.float32, device="cuda")
    q.qgemv_nrm_bias(q.Q8_0, gpu_matrix(q.Q8_0, a["W"], w.N, w.K), w.N, w.K, dev(a["x"]),
                     dev(a["gamma"]), w.params["eps"], dev(bias), nb, y)
    yg = host(y)
    yr, A = oracle.qgemv_nrm_bias(q.Q8_0, a["W"], w.N, w.K, a["x"], a["gamma"], w.params["eps"], bias)
    assert_within(yg, yr, tol_gemv(A, yr), "qkv bias")
    qg, kg = wl.gamma_f32(g, hd), wl.gamma_f32(g, hd)
    cs, sn = _rope_tables(g, nb, rh)
    q.qgemv_qk_norm_rope(y, nb, nq, nkv, hd, rh, dev(qg), dev(kg), 1e-6, dev(cs), dev(sn))
    ref = oracle.qk_norm_rope(yg, nq, nkv, hd, rh, qg, kg, 1e-6, cs, sn)
    nrm = oracle.qk_norm_rope(yg, nq, nkv, hd, rh, qg, kg, 1e-6, np.ones_like(cs), np.zeros_like(sn))
    assert_within(host(y), ref, 2.0 ** -17 * (np.abs(nrm).max(axis=1, keepdims=True)), "qkv norm rope")

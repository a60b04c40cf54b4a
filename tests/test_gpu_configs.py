"""Parity of the five workloads at their full sizes, through the same entry points and launch
configuration the bench times, against the f64 oracle (every output is compared: the oracle
finishes the largest of them in well under a second)."""
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


def test_single_gemv_1024():
    w = wl.single_gemv()
    say(f"workload {w.name}")
    W, x = w.arrays["W"], w.arrays["x"]
    y = torch.empty((1, w.N), dtype=torch.float32, device="cuda")
    q.qgemv(q.Q4_0, gpu_matrix(q.Q4_0, W, w.N, w.K), w.N, w.K, dev(x), 1, y)
    yr, A = oracle.qgemv(q.Q4_0, W, w.N, w.K, x)
    assert_within(host(y), yr, tol_gemv(A, yr), w.name)


def test_decode_mlp_chain():
    """gate+up+SwiGLU (with the RMSNorm prologue) then down + residual, the down step checked on
    the GPU's own h so each launch is held to its own bound."""
    w = wl.decode_mlp()
    say(f"workload {w.name}")
    a = w.arrays
    H, I, eps = 2048, 8192, w.params["eps"]
    xd = dev(a["x"])
    h = torch.empty((1, I), dtype=torch.float32, device="cuda")
    y = torch.empty((1, H), dtype=torch.float32, device="cuda")
    Wg, Wu, Wd = (gpu_matrix(q.Q4_0, a[k], *s) for k, s in (("Wg", (I, H)), ("Wu", (I, H)),
                                                            ("Wd", (H, I))))
    q.qgemv_gus_nrm(q.Q4_0, Wg, Wu, I, H, xd, dev(a["gamma"]), eps, 1, h)
    q.qgemv_res(q.Q4_0, Wd, H, I, h, xd, 1, y)
    hg = host(h)
    hr, gr, ur, Ag, Au = oracle.qgemv_gus_nrm(q.Q4_0, a["Wg"], a["Wu"], I, H, a["x"], a["gamma"], eps)
    assert_within(hg, hr, gus_tol(gr, ur, Ag, Au), "mlp gate/up")
    yr, A = oracle.qgemv_res(q.Q4_0, a["Wd"], H, I, hg, a["x"])
    assert_within(host(y), yr, tol_gemv(A, yr), "mlp down+res")


@pytest.mark.parametrize("nb", [1, 4, 16])
def test_qkv_q8_nrm(nb):
    w = wl.qkv_q8(nb=nb)
    say(f"workload {w.name}")
    a = w.arrays
    y = torch.empty((nb, w.N), dtype=torch.float32, device="cuda")
    q.qgemv_nrm(q.Q8_0, gpu_matrix(q.Q8_0, a["W"], w.N, w.K), w.N, w.K, dev(a["x"]),
                dev(a["gamma"]), w.params["eps"], nb, y)
    yr, A = oracle.qgemv_nrm(q.Q8_0, a["W"], w.N, w.K, a["x"], a["gamma"], w.params["eps"])
    assert_within(host(y), yr, tol_gemv(A, yr), w.name)


@pytest.mark.parametrize("nb", [1, 4])
def test_lm_head_argmax(nb):
    w = wl.lm_head(nb=nb)
    say(f"workload {w.name}")
    a = w.arrays
    logits = torch.empty((nb, w.N), dtype=torch.float32, device="cuda")
    idx = torch.empty((nb,), dtype=torch.int32, device="cuda")
    ws = D.workspace(q.OP_ARGMAX, q.Q4_0, w.N, w.K, nb)
    q.qgemv_argmax(q.Q4_0, gpu_matrix(q.Q4_0, a["W"], w.N, w.K), w.N, w.K, dev(a["x"]), nb,
                   logits, idx, ws)
    yr, A = oracle.gemv(q.Q4_0, a["W"], w.N, w.K, a["x"])
    lg, ig = host(logits), host(idx)
    tol = tol_gemv(A, yr)
    assert_within(lg, yr, tol, w.name)
    ir = oracle.argmax(yr)
    for r in range(nb):
        i, m = int(ig[r]), int(ir[r])
        assert lg[r, i] == lg[r].max() and int(np.argmax(lg[r])) == i
        assert i == m or yr[r, m] - yr[r, i] <= tol[r, m] + tol[r, i], (r, i, m)


def test_moe_q4k_top8():
    w = wl.moe_q4k()
    say(f"workload {w.name}")
    a = w.arrays
    n_exp, topk, nb = w.params["n_exp"], w.params["topk"], w.nb
    ws = D.workspace(q.OP_MOE, q.Q4_K, w.N, w.K, nb, n_exp, topk)
    y = torch.empty((nb, w.N), dtype=torch.float32, device="cuda")
    q.qgemv_moe(q.Q4_K, gpu_matrix(q.Q4_K, a["W"], n_exp * w.N, w.K), n_exp, w.N, w.K, dev(a["x"]),
                nb, dev(a["ids"]), dev(a["p"]), topk, y, ws)
    yr, A = oracle.qgemv_moe(q.Q4_K, a["W"], n_exp, w.N, w.K, a["x"], a["ids"], a["p"])
    assert_within(host(y), yr, tol_gemv(A, yr), w.name)
    assert q.qgemv_moe_error(ws, n_exp, w.N, w.K, q.Q4_K) == 0

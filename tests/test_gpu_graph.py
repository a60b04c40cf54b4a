"""Launches captured in a HIP graph (what bench.py times) give exactly the eager results: every
entry point is captured once, the graph is replayed three times with eager work on other inputs
and host synchronizations in between, and every replay is compared bit for bit with the eager
call on the same inputs."""
import numpy as np
import pytest

from gpu_common import dev, gpu_matrix, host, require_gpu, say, torch

import dequant_gemv_q4_amd as q
from dequant_gemv_q4_amd import device as D
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _check(name, run, outs, other):
    """run() issues the call writing the tensors in `outs`; other() is unrelated eager work."""
    say(f"graph {name}")
    run()
    torch.cuda.synchronize()
    ref = [host(o).copy() for o in outs]
    for o in outs:
        o.zero_()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.zero_()
        other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert np.array_equal(host(o), r), (name, rep)


def _mat(fmt, seed, N, K):
    g = np.random.default_rng(seed)
    W = wl.matrix(fmt, g, N, K)
    return W, gpu_matrix(fmt, W, N, K), g


def test_graph_replays_match_eager():
    N, K = 3000, 2048
    W, Wp, g = _mat(q.Q4_0, 1, N, K)
    W2, Wp2, _ = _mat(q.Q4_0, 2, N, K)
    x1 = dev(wl.normal_f32(g, (1, K)))
    x16 = dev(wl.normal_f32(g, (16, K)))
    gamma = dev(wl.gamma_f32(g, K))
    y1 = torch.empty((1, N), dtype=torch.float32, device="cuda")
    y16 = torch.empty((16, N), dtype=torch.float32, device="cuda")
    other_y = torch.empty((1, N), dtype=torch.float32, device="cuda")
    xo = dev(wl.normal_f32(g, (1, K)))

    def other():
        q.qgemv(q.Q4_0, Wp2, N, K, xo, 1, other_y)

    _check("qgemv nb=1", lambda: q.qgemv(q.Q4_0, Wp, N, K, x1, 1, y1), [y1], other)
    _check("qgemv nb=16", lambda: q.qgemv(q.Q4_0, Wp, N, K, x16, 16, y16), [y16], other)
    _check("qgemv_nrm nb=1", lambda: q.qgemv_nrm(q.Q4_0, Wp, N, K, x1, gamma, 1e-5, 1, y1),
           [y1], other)
    h = torch.empty((1, N), dtype=torch.float32, device="cuda")
    _check("qgemv_gus_nrm", lambda: q.qgemv_gus_nrm(q.Q4_0, Wp, Wp2, N, K, x1, gamma, 1e-5, 1, h),
           [h], other)
    r = dev(wl.normal_f32(g, (1, N)))
    _check("qgemv_res", lambda: q.qgemv_res(q.Q4_0, Wp, N, K, x1, r, 1, y1), [y1], other)
    ws = D.workspace(q.OP_ARGMAX, q.Q4_0, N, K, 4)
    x4 = dev(wl.normal_f32(g, (4, K)))
    lg = torch.empty((4, N), dtype=torch.float32, device="cuda")
    idx = torch.empty((4,), dtype=torch.int32, device="cuda")
    _check("qgemv_argmax nb=4", lambda: q.qgemv_argmax(q.Q4_0, Wp, N, K, x4, 4, lg, idx, ws),
           [lg, idx], other)


def test_graph_replays_match_eager_experts():
    n_exp, N, K, nb, topk = 16, 256, 512, 6, 3
    g = np.random.default_rng(5)
    W = wl.matrix(q.Q4_K, g, n_exp * N, K)
    Wp = gpu_matrix(q.Q4_K, W, n_exp * N, K)
    ids, p = wl.route_top_k(g.standard_normal((nb, n_exp)), topk)
    x = dev(wl.normal_f32(g, (nb, K)))
    y = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    ws = D.workspace(q.OP_MOE, q.Q4_K, N, K, nb, n_exp, topk)
    idsd, pd = dev(ids), dev(p)
    _, Wp2, _ = _mat(q.Q4_0, 3, 1000, 1024)
    xo = dev(wl.normal_f32(g, (1, 1024)))
    yo = torch.empty((1, 1000), dtype=torch.float32, device="cuda")

    def other():
        q.qgemv(q.Q4_0, Wp2, 1000, 1024, xo, 1, yo)

    _check("qgemv_moe", lambda: q.qgemv_moe(q.Q4_K, Wp, n_exp, N, K, x, nb, idsd, pd, topk, y, ws),
           [y], other)

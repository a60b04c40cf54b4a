"""The no-allocation argmax entry point, called through the C ABI, against qgemv_argmax (same
kernels, workspace from the caller): logits and indices must be bit for bit the same, on two calls
in a row, the second with a smaller input (the fixed scratch keeps the first call's partial keys,
which the second must overwrite before it reads them)."""
import ctypes

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


def _case(fmt, N, K, nb, seed):
    g = wl.rng(1300 + fmt, seed)
    W = wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (nb, K))
    return gpu_matrix(fmt, W, N, K), dev(x)


def _noalloc_raw(fmt, Wp, N, K, xd, nb, logits, idx):
    """Straight through the C symbol (ctypes), torch's current stream."""
    fn = q.lib().qgemv_argmax_noalloc
    st = fn(fmt, ctypes.c_void_p(Wp.data_ptr()), N, K, ctypes.c_void_p(xd.data_ptr()), nb,
            ctypes.c_void_p(logits.data_ptr()), ctypes.c_void_p(idx.data_ptr()),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, q.qgemv_status_str(st)


@pytest.mark.parametrize("fmt,big,small", [
    (q.Q4_0, (65536, 2048, 4), (5000, 1024, 1)),     # many partial keys, then few
    (q.Q8_0, (20000, 1536, 16), (777, 512, 3)),     # row-batch kernel, then vector kernel
    (q.Q4_K, (9000, 2048, 2), (300, 256, 1)),
    (q.Q4_0, (3000, 8192, 7), (500, 8192, 6)),      # long rows: batches of at most 4 rows
])
def test_noalloc_matches_workspace_argmax(fmt, big, small):
    for i, (N, K, nb) in enumerate((big, small)):
        say(f"noalloc argmax fmt={fmt} N={N} K={K} nb={nb}")
        Wp, xd = _case(fmt, N, K, nb, i)
        ws = D.workspace(q.OP_ARGMAX, fmt, N, K, nb)
        l_ref = torch.empty((nb, N), dtype=torch.float32, device="cuda")
        i_ref = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
        q.qgemv_argmax(fmt, Wp, N, K, xd, nb, l_ref, i_ref, ws)
        l_na = torch.empty((nb, N), dtype=torch.float32, device="cuda")
        i_na = torch.full((nb,), -2, dtype=torch.int32, device="cuda")
        _noalloc_raw(fmt, Wp, N, K, xd, nb, l_na, i_na)
        lr, ln = host(l_ref), host(l_na)
        assert np.array_equal(lr, ln)
        assert np.array_equal(host(i_ref), host(i_na))
        for r in range(nb):
            assert int(host(i_na)[r]) == int(np.argmax(ln[r]))


def test_noalloc_rejects_bad_arguments():
    Wp, xd = _case(q.Q4_0, 64, 256, 1, 9)
    y = torch.empty((1, 64), dtype=torch.float32, device="cuda")
    idx = torch.empty((1,), dtype=torch.int32, device="cuda")
    with pytest.raises(q.QgemvError):
        q.qgemv_argmax_noalloc(q.Q4_0, Wp, 64, 256, xd, 17, y, idx)       # nb > 16
    with pytest.raises(q.QgemvError):
        q.qgemv_argmax_noalloc(q.Q4_0, Wp, 64, 256, xd, 1, y, None)      # no idx

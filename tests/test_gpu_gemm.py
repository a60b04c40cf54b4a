"""The wide row-batch GEMM (prefill chunks, M > 16 rows of x; "Module gpu", module prefill) on the
GPU against the f64 oracle: Q4_0, Q8_0 and Q1_0, M from 1 to 2048 and ragged sizes (partial x and
W tiles, 64-row x tiles for M <= 64 and 128-row ones above, every weight-tile width, K not a
multiple of the 128-k step, K split over workgroups with a shorter last split), every output
compared up to M = 512 and sampled rows and columns beyond; integer inputs bit for bit; x only
4-byte aligned."""
import numpy as np
import pytest

from gpu_common import assert_within, dev, gpu_matrix, host, require_gpu, say, tol_gemv, torch

import dequant_gemv_q4_amd as q
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    oracle.build(force=False)


def _gemm(fmt, Wp, N, K, x):
    M = x.shape[0]
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(q.qgemm_workspace_bytes(fmt, N, K, M), dtype=torch.uint8, device="cuda")
    q.qgemm(fmt, Wp, N, K, dev(x), M, y, ws)
    return host(y)


@pytest.mark.parametrize("fmt,M,N,K", [(q.Q4_0, 17, 300, 2048), (q.Q4_0, 64, 1000, 1024),
                                       (q.Q4_0, 512, 517, 2048), (q.Q8_0, 17, 129, 1536),
                                       (q.Q8_0, 64, 2048, 1536), (q.Q8_0, 512, 260, 2048),
                                       (q.Q4_0, 200, 130, 96), (q.Q8_0, 131, 77, 32),
                                       (q.Q4_0, 1, 64, 4096), (q.Q4_0, 129, 257, 8192),
                                       (q.Q4_0, 40, 200, 608), (q.Q8_0, 33, 150, 608),
                                       (q.Q4_0, 100, 3000, 1024), (q.Q1_0, 17, 300, 2048),
                                       (q.Q1_0, 512, 517, 1024), (q.Q1_0, 200, 130, 128),
                                       (q.Q1_0, 131, 1000, 640), (q.Q4_0, 65, 300, 256),
                                       (q.Q1_0, 64, 1000, 128), (q.Q8_0, 1, 16, 32),
                                       (q.Q4_0, 12, 500, 8192)])
def test_qgemm_parity(fmt, M, N, K):
    say(f"qgemm fmt={fmt} M={M} N={N} K={K}")
    g = wl.rng(3000 + fmt, M + N + K)
    W = wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (M, K))
    y = _gemm(fmt, gpu_matrix(fmt, W, N, K), N, K, x)
    yr, A = oracle.gemv(fmt, W, N, K, x)
    assert_within(y, yr, tol_gemv(A, yr), f"qgemm fmt={fmt} M={M} N={N} K={K}")


@pytest.mark.parametrize("fmt,M,N,K", [(q.Q4_0, 2048, 4096, 2048), (q.Q8_0, 2048, 2048, 1536),
                                       (q.Q4_0, 1950, 4000, 1056), (q.Q1_0, 2048, 4096, 2048),
                                       (q.Q1_0, 1950, 4000, 1152), (q.Q4_0, 2048, 8192, 2048),
                                       (q.Q4_0, 1990, 7900, 1056), (q.Q8_0, 2048, 4096, 1536),
                                       (q.Q8_0, 1990, 4000, 1056), (q.Q4_0, 512, 8192, 2048),
                                       (q.Q8_0, 500, 8000, 1056), (q.Q1_0, 450, 8100, 640)])
def test_qgemm_large_sampled(fmt, M, N, K):
    """Full-size launch; the oracle checks 64 sampled x rows against 256 sampled W rows.  The
    Q4_0, Q1_0 and Q8_0 cases at N ~ 4000 take the 256-row weight tiles (Q8_0 with the two-stage
    ring), the Q4_0 ones at N ~ 8000 the 512-row tiles with the two-stage ring (the second of each
    pair ragged in M, N and K)."""
    say(f"qgemm large fmt={fmt} M={M} N={N} K={K}")
    g = wl.rng(3100 + fmt, M)
    W = wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (M, K))
    y = _gemm(fmt, gpu_matrix(fmt, W, N, K), N, K, x)
    rows = np.sort(g.choice(M, 64, replace=False))
    cols = np.sort(g.choice(N, 256, replace=False))
    yr, A = oracle.gemv(fmt, W, N, K, x[rows], rows=cols)
    assert_within(y[np.ix_(rows, cols)], yr, tol_gemv(A, yr), f"qgemm large fmt={fmt}")


@pytest.mark.parametrize("fmt", [q.Q4_0, q.Q8_0, q.Q1_0])
def test_qgemm_integer_inputs_bitwise(fmt):
    say(f"qgemm integer fmt={fmt}")
    M, N, K = 150, 140, 512
    g = wl.rng(3200 + fmt, 1)
    W = wl.matrix(fmt, g, N, K).reshape(N, -1, wl.BLOCK_BYTES[fmt]).copy()
    W[..., 0:2] = (2.0 ** -g.integers(2, 7, size=W.shape[:2])).astype("<f2")[..., None].view(np.uint8)
    W = W.reshape(N, -1)
    x = g.integers(-7, 8, size=(M, K)).astype(np.float32)
    y = _gemm(fmt, gpu_matrix(fmt, W, N, K), N, K, x)
    yr, _ = oracle.gemv(fmt, W, N, K, x)
    assert np.array_equal(y.astype(np.float64), yr)


@pytest.mark.parametrize("fmt,M,N,K", [(q.Q4_0, 40, 66000, 256), (q.Q8_0, 33, 66000, 256),
                                       (q.Q1_0, 64, 65600, 384)])
def test_qgemm_few_rows_tall_matrix(fmt, M, N, K):
    """M <= 64 takes 64-row x tiles; against more than 65280 weight rows the 256-row weight tiles
    alone fill the device (every other small-M case takes 128-row ones with split K).  The oracle
    checks every x row against 256 sampled W rows."""
    say(f"qgemm tall fmt={fmt} M={M} N={N} K={K}")
    g = wl.rng(3500 + fmt, M)
    W = wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (M, K))
    y = _gemm(fmt, gpu_matrix(fmt, W, N, K), N, K, x)
    cols = np.sort(g.choice(N, 256, replace=False))
    yr, A = oracle.gemv(fmt, W, N, K, x, rows=cols)
    assert_within(y[:, cols], yr, tol_gemv(A, yr), f"qgemm tall fmt={fmt}")


@pytest.mark.parametrize("M,K", [(70, 1024), (70, 8192), (5, 1024)])
def test_qgemm_x_only_4_byte_aligned(M, K):
    """x starting 4 bytes past a 16-byte boundary (the boundary accepts 4-byte alignment): the x
    preparation takes scalar loads, with the row held in registers (K = 1024) and re-read
    (K = 8192); with M <= 16 such an x keeps the call on the GEMM kernels (an aligned one goes to
    the row-batch GEMV)."""
    say(f"qgemm x+4 bytes M={M} K={K}")
    N = 300
    g = wl.rng(3400 + M, K)
    W = wl.q4_0_matrix(g, N, K)
    x = wl.normal_f32(g, (M, K))
    big = torch.empty(M * K + 4, dtype=torch.float32, device="cuda")
    big[1:1 + M * K].copy_(dev(x).reshape(-1))
    xv = big[1:1 + M * K].view(M, K)
    assert xv.data_ptr() % 16 == 4
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(q.qgemm_workspace_bytes(q.Q4_0, N, K, M), dtype=torch.uint8, device="cuda")
    q.qgemm(q.Q4_0, gpu_matrix(q.Q4_0, W, N, K), N, K, xv, M, y, ws)
    yr, A = oracle.gemv(q.Q4_0, W, N, K, x)
    assert_within(host(y), yr, tol_gemv(A, yr), f"qgemm x+4 M={M} K={K}")


def test_qgemm_rows_match_row_batch_gemv():
    """The first 16 rows of a wide call against qgemv on the same 16 rows (both bounded by the
    oracle; here the two GPU paths are held to each other's bound)."""
    say("qgemm vs qgemv")
    M, N, K = 300, 400, 2048
    g = wl.rng(3300, 2)
    W = wl.q4_0_matrix(g, N, K)
    x = wl.normal_f32(g, (M, K))
    Wp = gpu_matrix(q.Q4_0, W, N, K)
    y = _gemm(q.Q4_0, Wp, N, K, x)
    y16 = torch.empty((16, N), dtype=torch.float32, device="cuda")
    q.qgemv(q.Q4_0, Wp, N, K, dev(x[:16]), 16, y16)
    _, A = oracle.gemv(q.Q4_0, W, N, K, x[:16])
    assert np.all(np.abs(y[:16] - host(y16)) <= 2e-3 * A)


def test_qgemm_rejects_other_formats_and_small_workspace():
    W = torch.zeros(q.qgemv_packed_bytes(q.Q4_K, 64, 256), dtype=torch.uint8, device="cuda")
    x = torch.zeros((20, 256), dtype=torch.float32, device="cuda")
    y = torch.empty((20, 64), dtype=torch.float32, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(q.QgemvError) as e:
        q.qgemm(q.Q4_K, W, 64, 256, x, 20, y, ws)
    assert e.value.status == 2
    W0 = torch.zeros(q.qgemv_packed_bytes(q.Q4_0, 64, 256), dtype=torch.uint8, device="cuda")
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(q.QgemvError) as e:
        q.qgemm(q.Q4_0, W0, 64, 256, x, 20, y, small)
    assert e.value.status == 5

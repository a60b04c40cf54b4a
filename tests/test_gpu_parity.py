"""GPU parity of every entry point against the f64 oracle, element by element, on seeded inputs:
small shapes that span several tiles and a ragged tail, the exactness pins that hold bitwise on
the GPU (zero weights, scale doubling, linearity, integer brute force, determinism), and the
edge cases (single block, single row, nb up to 16, multi-tile K)."""
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


def _run_gemv(fmt, Wp, N, K, x):
    nb = x.shape[0]
    y = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv(fmt, Wp, N, K, dev(x), nb, y)
    return host(y)


# ------------------------------------------------------------------------------------ pack

@pytest.mark.parametrize("fmt,N,K", [(q.Q4_0, 37, 96), (q.Q8_0, 19, 64), (q.Q4_K, 11, 512)])
def test_pack_layout(fmt, N, K):
    say(f"pack fmt={fmt} N={N} K={K}")
    g = np.random.default_rng(1)
    W = wl.matrix(fmt, g, N, K)
    Wp = host(gpu_matrix(fmt, W, N, K))
    bb = wl.BLOCK_BYTES[fmt]
    sb = 16 if fmt == q.Q4_K else 2
    blk = W.reshape(-1, bb)
    qs = blk[:, sb:].reshape(-1)
    sc = blk[:, :sb].reshape(-1)
    sc_off = (qs.size + 255) // 256 * 256
    assert np.array_equal(Wp[:qs.size], qs)
    assert np.array_equal(Wp[sc_off:sc_off + sc.size], sc)


# ------------------------------------------------------------------------------------ qgemv

GEMV_CASES = [
    # (fmt, N, K, nb): ragged N, one-block K, multi-chunk rows, multi-tile K (nb large), nb 1..16
    (q.Q4_0, 1, 32, 1), (q.Q4_0, 37, 32, 3), (q.Q4_0, 1037, 1024, 1), (q.Q4_0, 517, 2048, 1),
    (q.Q4_0, 300, 8192, 1), (q.Q4_0, 129, 96, 2), (q.Q4_0, 201, 2048, 4), (q.Q4_0, 77, 1536, 5),
    (q.Q4_0, 150, 2048, 7), (q.Q4_0, 100, 2048, 8), (q.Q4_0, 65, 2048, 16), (q.Q4_0, 33, 4096, 12),
    # row batches whose scale rows are not 8 (Q4_0) / 4 (Q8_0) byte aligned: per-block scale loads
    (q.Q4_0, 40, 96, 8), (q.Q4_0, 29, 1120, 16), (q.Q8_0, 45, 96, 6),
    (q.Q8_0, 1, 32, 1), (q.Q8_0, 301, 1536, 1), (q.Q8_0, 2048 + 5, 1536, 4), (q.Q8_0, 99, 1536, 16),
    (q.Q8_0, 45, 4096, 3), (q.Q8_0, 70, 2048, 9),
    (q.Q4_K, 1, 256, 1), (q.Q4_K, 61, 2048, 1), (q.Q4_K, 130, 768, 2), (q.Q4_K, 90, 2048, 16),
    (q.Q4_K, 33, 4096, 6),
]


@pytest.mark.parametrize("fmt,N,K,nb", GEMV_CASES)
def test_qgemv_parity(fmt, N, K, nb):
    say(f"qgemv fmt={fmt} N={N} K={K} nb={nb}")
    g = wl.rng(100 + fmt, N * 7 + K + nb)
    W = wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (nb, K))
    y = _run_gemv(fmt, gpu_matrix(fmt, W, N, K), N, K, x)
    yr, A = oracle.gemv(fmt, W, N, K, x)
    assert_within(y, yr, tol_gemv(A, yr), f"qgemv fmt={fmt} N={N} K={K} nb={nb}")


@pytest.mark.parametrize("fmt", [q.Q4_0, q.Q8_0, q.Q4_K])
def test_zero_weights_give_exact_zero(fmt):
    """All Q4_0 nibbles 8 / all Q8_0 bytes 0 / Q4_K scales and mins 0: y is exactly 0."""
    say(f"zero weights fmt={fmt}")
    N, K, nb = 300, 2048, 3
    g = np.random.default_rng(4)
    W = wl.matrix(fmt, g, N, K).reshape(N, -1, wl.BLOCK_BYTES[fmt])
    if fmt == q.Q4_0:
        W[..., 2:] = 0x88
    elif fmt == q.Q8_0:
        W[..., 2:] = 0
    else:
        W[..., 4:16] = 0
    W = W.reshape(N, -1)
    x = wl.normal_f32(g, (nb, K))
    y = _run_gemv(fmt, gpu_matrix(fmt, W, N, K), N, K, x)
    assert np.all(y == 0.0)


@pytest.mark.parametrize("fmt", [q.Q4_0, q.Q8_0, q.Q4_K])
def test_scale_doubling_and_linearity_are_bitwise(fmt):
    say(f"scale doubling fmt={fmt}")
    N, K, nb = 257, 1024 if fmt != q.Q4_K else 2048, 2
    g = np.random.default_rng(6)
    W = wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (nb, K))
    y1 = _run_gemv(fmt, gpu_matrix(fmt, W, N, K), N, K, x)
    W2 = W.copy().reshape(N, -1, wl.BLOCK_BYTES[fmt])
    for s in range(2 if fmt == q.Q4_K else 1):
        h = W2[..., 2 * s:2 * s + 2].copy().view("<u2")
        h += 1 << 10
        W2[..., 2 * s:2 * s + 2] = h.view(np.uint8)
    y2 = _run_gemv(fmt, gpu_matrix(fmt, W2.reshape(N, -1), N, K), N, K, x)
    assert np.array_equal(y2, 2 * y1)
    y3 = _run_gemv(fmt, gpu_matrix(fmt, W, N, K), N, K, 2 * x)
    assert np.array_equal(y3, 2 * y1)


def test_integer_inputs_are_exact():
    """d = 2^-4 and small integer x: every product and partial sum is exactly representable, so
    the GPU equals the oracle bit for bit."""
    say("integer brute force")
    N, K, nb = 64, 64, 2
    g = np.random.default_rng(8)
    W = wl.q4_0_matrix(g, N, K).reshape(N, -1, 18)
    W[..., 0:2] = np.array([0.0625], dtype="<f2").view(np.uint8)
    W = W.reshape(N, -1)
    x = g.integers(-3, 4, size=(nb, K)).astype(np.float32)
    y = _run_gemv(q.Q4_0, gpu_matrix(q.Q4_0, W, N, K), N, K, x)
    yr, _ = oracle.gemv(q.Q4_0, W, N, K, x)
    assert np.array_equal(y.astype(np.float64), yr)


def test_rows_of_a_batch_match_single_row_calls():
    say("row independence")
    N, K, nb = 333, 2048, 4
    g = np.random.default_rng(10)
    W = wl.q4_0_matrix(g, N, K)
    Wp = gpu_matrix(q.Q4_0, W, N, K)
    x = wl.normal_f32(g, (nb, K))
    yb = _run_gemv(q.Q4_0, Wp, N, K, x)
    for r in range(nb):
        y1 = _run_gemv(q.Q4_0, Wp, N, K, x[r:r + 1])
        assert np.array_equal(yb[r:r + 1], y1), r


def test_repeated_launches_are_bitwise_identical():
    say("determinism")
    N, K, nb = 4099, 2048, 1
    g = np.random.default_rng(12)
    W = wl.q4_0_matrix(g, N, K)
    Wp = gpu_matrix(q.Q4_0, W, N, K)
    xd = dev(wl.normal_f32(g, (nb, K)))
    outs = []
    for _ in range(10):
        y = torch.empty((nb, N), dtype=torch.float32, device="cuda")
        q.qgemv(q.Q4_0, Wp, N, K, xd, nb, y)
        outs.append(host(y))
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("fmt,N,K,nb", [(q.Q4_0, 8209, 512, 16), (q.Q4_0, 16411, 256, 8),
                                        (q.Q8_0, 33000, 256, 13), (q.Q4_0, 65573, 256, 16),
                                        (q.Q8_0, 8200, 3072, 7), (q.Q4_0, 1000, 4096, 16)])
def test_row_batch_tile_groups(fmt, N, K, nb):
    """Row batches of 5..16 on tall matrices: several 16-row tiles per work group and fewer waves
    per tile (K split 8, 4, 2 ways, or one wave per tile), ragged last group, and the long-K
    class (K > 2048)."""
    say(f"row batch fmt={fmt} N={N} K={K} nb={nb}")
    g = wl.rng(700 + fmt, N + nb)
    W = wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (nb, K))
    y = _run_gemv(fmt, gpu_matrix(fmt, W, N, K), N, K, x)
    yr, A = oracle.gemv(fmt, W, N, K, x)
    assert_within(y, yr, tol_gemv(A, yr), f"row batch fmt={fmt} N={N}")


def test_x_scale_extremes():
    """x rows spanning many binades (and one row of zeros, one tiny, one huge): the per-row
    power-of-two scaling keeps every path inside its bound."""
    say("x scale extremes")
    N, K = 300, 2048
    g = np.random.default_rng(31)
    W = wl.q4_0_matrix(g, N, K)
    Wp = gpu_matrix(q.Q4_0, W, N, K)
    base = wl.normal_f32(g, (16, K))
    mags = np.float32(2.0) ** g.integers(-12, 13, size=(16, K)).astype(np.float32)
    x = (base * mags).astype(np.float32)
    x[1] = 0.0
    x[2] *= np.float32(1e-36)
    x[3] *= np.float32(1e25)
    for nb in (1, 3, 16):
        xs = np.ascontiguousarray(x[:nb])
        y = _run_gemv(q.Q4_0, Wp, N, K, xs)
        yr, A = oracle.gemv(q.Q4_0, W, N, K, xs)
        assert np.all(np.isfinite(y))
        assert_within(y, yr, tol_gemv(A, yr), f"x extremes nb={nb}")


# ------------------------------------------------------------------------------------ fused ops

@pytest.mark.parametrize("fmt,N,K,nb", [(q.Q4_0, 515, 2048, 1), (q.Q8_0, 2048, 1536, 4),
                                        (q.Q8_0, 300, 1536, 16), (q.Q4_K, 200, 2048, 3),
                                        (q.Q4_0, 100, 8192, 2)])
def test_qgemv_nrm_parity(fmt, N, K, nb):
    say(f"nrm fmt={fmt} N={N} K={K} nb={nb}")
    g = wl.rng(200 + fmt, N + nb)
    W = wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (nb, K))
    gamma = wl.gamma_f32(g, K)
    y = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv_nrm(fmt, gpu_matrix(fmt, W, N, K), N, K, dev(x), dev(gamma), 1e-5, nb, y)
    yr, A = oracle.qgemv_nrm(fmt, W, N, K, x, gamma, 1e-5)
    assert_within(host(y), yr, tol_gemv(A, yr), f"nrm fmt={fmt}")


@pytest.mark.parametrize("fmt,N,K,nb", [(q.Q4_0, 1000, 2048, 1), (q.Q4_0, 257, 1024, 3),
                                        (q.Q8_0, 300, 1536, 2), (q.Q4_K, 130, 2048, 1),
                                        (q.Q4_0, 77, 2048, 9)])
def test_qgemv_gus_nrm_parity(fmt, N, K, nb):
    say(f"gus_nrm fmt={fmt} N={N} K={K} nb={nb}")
    g = wl.rng(300 + fmt, N + nb)
    Wg = wl.matrix(fmt, g, N, K)
    Wu = wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (nb, K))
    gamma = wl.gamma_f32(g, K)
    h = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv_gus_nrm(fmt, gpu_matrix(fmt, Wg, N, K), gpu_matrix(fmt, Wu, N, K), N, K, dev(x),
                    dev(gamma), 1e-5, nb, h)
    hr, gr, ur, Ag, Au = oracle.qgemv_gus_nrm(fmt, Wg, Wu, N, K, x, gamma, 1e-5)
    assert_within(host(h), hr, gus_tol(gr, ur, Ag, Au), f"gus fmt={fmt}")


def test_gus_zero_gate_gives_zero():
    say("gus zero gate")
    N, K = 300, 2048
    g = np.random.default_rng(14)
    Wg = wl.q4_0_matrix(g, N, K).reshape(N, -1, 18)
    Wg[..., 2:] = 0x88
    Wu = wl.q4_0_matrix(g, N, K)
    x = wl.normal_f32(g, (1, K))
    gamma = wl.gamma_f32(g, K)
    h = torch.empty((1, N), dtype=torch.float32, device="cuda")
    q.qgemv_gus_nrm(q.Q4_0, gpu_matrix(q.Q4_0, Wg.reshape(N, -1), N, K),
                    gpu_matrix(q.Q4_0, Wu, N, K), N, K, dev(x), dev(gamma), 1e-5, 1, h)
    assert np.all(host(h) == 0.0)


@pytest.mark.parametrize("fmt,N,K,nb,inplace", [(q.Q4_0, 2048, 8192, 1, False),
                                                (q.Q4_0, 500, 2048, 2, True),
                                                (q.Q8_0, 300, 1536, 4, True),
                                                (q.Q4_K, 129, 2048, 1, False),
                                                (q.Q4_0, 333, 2048, 11, True),
                                                (q.Q8_0, 9001, 1024, 16, False)])
def test_qgemv_res_parity(fmt, N, K, nb, inplace):
    say(f"res fmt={fmt} N={N} K={K} nb={nb} inplace={inplace}")
    g = wl.rng(400 + fmt, N + nb)
    W = wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (nb, K))
    r = wl.normal_f32(g, (nb, N))
    rd = dev(r)
    y = rd if inplace else torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv_res(fmt, gpu_matrix(fmt, W, N, K), N, K, dev(x), rd, nb, y)
    yr, A = oracle.qgemv_res(fmt, W, N, K, x, r)
    assert_within(host(y), yr, tol_gemv(A, yr), f"res fmt={fmt}")


def test_res_zero_weights_is_identity():
    say("res identity")
    N, K = 700, 2048
    W = np.frombuffer((np.array([0.5], "<f2").tobytes() + bytes([0x88] * 16)) * (N * K // 32),
                      dtype=np.uint8).reshape(N, -1)
    g = np.random.default_rng(16)
    x = wl.normal_f32(g, (1, K))
    r = wl.normal_f32(g, (1, N))
    y = torch.empty((1, N), dtype=torch.float32, device="cuda")
    q.qgemv_res(q.Q4_0, gpu_matrix(q.Q4_0, W, N, K), N, K, dev(x), dev(r), 1, y)
    assert np.array_equal(host(y), r)


def _argmax_check(logits, idx, yr, A, what):
    tol = tol_gemv(A, yr)
    assert_within(logits, yr, tol, what)
    for r in range(yr.shape[0]):
        i = int(idx[r])
        # the GPU's index is the lowest maximum of its own logits ...
        assert logits[r, i] == logits[r].max() and np.argmax(logits[r]) == i, (what, r)
        # ... and the oracle's maximum, unless the two are within both tolerances
        m = int(oracle.argmax(yr[r:r + 1])[0])
        assert i == m or yr[r, m] - yr[r, i] <= tol[r, m] + tol[r, i], (what, r, i, m)


@pytest.mark.parametrize("fmt,N,K,nb", [(q.Q4_0, 5000, 2048, 1), (q.Q4_0, 4097, 1024, 4),
                                        (q.Q8_0, 999, 1536, 2), (q.Q4_K, 777, 2048, 16),
                                        (q.Q4_0, 20011, 512, 16), (q.Q8_0, 1500, 1024, 6)])
def test_qgemv_argmax_parity(fmt, N, K, nb):
    say(f"argmax fmt={fmt} N={N} K={K} nb={nb}")
    g = wl.rng(500 + fmt, N + nb)
    W = wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (nb, K))
    Wp = gpu_matrix(fmt, W, N, K)
    ws = D.workspace(q.OP_ARGMAX, fmt, N, K, nb)
    yr, A = oracle.gemv(fmt, W, N, K, x)
    for rep in range(3):   # the workspace must come back clean after every call
        logits = torch.empty((nb, N), dtype=torch.float32, device="cuda")
        idx = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
        q.qgemv_argmax(fmt, Wp, N, K, dev(x), nb, logits, idx, ws)
        _argmax_check(host(logits), host(idx), yr, A, f"argmax fmt={fmt} rep={rep}")


def test_argmax_ties_go_to_lowest_index():
    say("argmax ties")
    N, K = 3000, 1024
    g = np.random.default_rng(18)
    W = wl.q4_0_matrix(g, N, K).reshape(N, -1, 18)
    big = W[5].copy()
    big[:, 0:2] = np.array([0.05], "<f2").view(np.uint8)
    big[:, 2:] = 0xff                                   # every weight 7 * 0.05
    for n in (5, 700, 2999):
        W[n] = big
    W = W.reshape(N, -1)
    x = np.abs(wl.normal_f32(g, (2, K)))
    logits = torch.empty((2, N), dtype=torch.float32, device="cuda")
    idx = torch.empty((2,), dtype=torch.int32, device="cuda")
    ws = D.workspace(q.OP_ARGMAX, q.Q4_0, N, K, 2)
    q.qgemv_argmax(q.Q4_0, gpu_matrix(q.Q4_0, W, N, K), N, K, dev(x), 2, logits, idx, ws)
    assert list(host(idx)) == [5, 5]


# ------------------------------------------------------------------------------------ experts

@pytest.mark.parametrize("fmt,n_exp,N,K,nb,topk", [(q.Q4_K, 8, 200, 512, 5, 3),
                                                   (q.Q4_0, 10, 129, 1024, 16, 8),
                                                   (q.Q8_0, 4, 300, 1536, 2, 1),
                                                   (q.Q8_0, 3, 130, 2048, 16, 2),
                                                   (q.Q4_0, 5, 70, 8192, 7, 3),
                                                   (q.Q4_K, 64, 1024, 2048, 16, 8),
                                                   # Q4_K rows of two and four chunks per lane
                                                   (q.Q4_K, 6, 100, 4096, 4, 2),
                                                   (q.Q4_K, 5, 64, 8192, 3, 2)])
def test_qgemv_moe_parity(fmt, n_exp, N, K, nb, topk):
    say(f"moe fmt={fmt} n_exp={n_exp} N={N} K={K} nb={nb} topk={topk}")
    g = wl.rng(600 + fmt, n_exp + N + nb)
    W = wl.matrix(fmt, g, n_exp * N, K)
    x = wl.normal_f32(g, (nb, K))
    ids, p = wl.route_top_k(g.standard_normal((nb, n_exp)), topk)
    Wp = gpu_matrix(fmt, W, n_exp * N, K)
    ws = D.workspace(q.OP_MOE, fmt, N, K, nb, n_exp, topk)
    yr, A = oracle.qgemv_moe(fmt, W, n_exp, N, K, x, ids, p)
    for rep in range(2):
        y = torch.empty((nb, N), dtype=torch.float32, device="cuda")
        q.qgemv_moe(fmt, Wp, n_exp, N, K, dev(x), nb, dev(ids), dev(p), topk, y, ws)
        assert_within(host(y), yr, tol_gemv(A, yr), f"moe fmt={fmt} rep={rep}")
    assert q.qgemv_moe_error(ws, n_exp, N, K, fmt) == 0


def test_moe_top1_equals_plain_gemv_bitwise():
    say("moe top1")
    n_exp, N, K, nb = 5, 300, 2048, 4
    g = np.random.default_rng(20)
    W = wl.q4_k_matrix(g, n_exp * N, K)
    x = wl.normal_f32(g, (nb, K))
    ids = np.array([[3], [0], [3], [4]], dtype=np.int32)
    p = np.ones((nb, 1), dtype=np.float32)
    Wp = gpu_matrix(q.Q4_K, W, n_exp * N, K)
    ws = D.workspace(q.OP_MOE, q.Q4_K, N, K, nb, n_exp, 1)
    y = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv_moe(q.Q4_K, Wp, n_exp, N, K, dev(x), nb, dev(ids), dev(p), 1, y, ws)
    y = host(y)
    for r in range(nb):
        e = int(ids[r, 0])
        ye = _run_gemv(q.Q4_K, gpu_matrix(q.Q4_K, W[e * N:(e + 1) * N], N, K), N, K, x[r:r + 1])
        assert np.array_equal(y[r:r + 1], ye), r


def test_moe_bad_id_sets_the_flag_and_adds_nothing():
    say("moe bad id")
    n_exp, N, K, nb, topk = 4, 64, 256, 2, 2
    g = np.random.default_rng(22)
    W = wl.q4_k_matrix(g, n_exp * N, K)
    x = wl.normal_f32(g, (nb, K))
    ids = np.array([[1, 7], [2, 0]], dtype=np.int32)       # 7 is out of range
    p = np.array([[0.5, 0.5], [0.25, 0.75]], dtype=np.float32)
    ws = D.workspace(q.OP_MOE, q.Q4_K, N, K, nb, n_exp, topk)
    y = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv_moe(q.Q4_K, gpu_matrix(q.Q4_K, W, n_exp * N, K), n_exp, N, K, dev(x), nb, dev(ids),
                dev(p), topk, y, ws)
    assert q.qgemv_moe_error(ws, n_exp, N, K, q.Q4_K) == 1
    assert q.qgemv_moe_error(ws, n_exp, N, K, q.Q4_K) == 0   # read-and-clear
    ids_ok = ids.copy()
    ids_ok[0, 1] = 1
    p_ok = p.copy()
    p_ok[0, 1] = 0.0
    yr, A = oracle.qgemv_moe(q.Q4_K, W, n_exp, N, K, x, ids_ok, p_ok)
    assert_within(host(y), yr, tol_gemv(A, yr), "moe bad id")

"""Pins of the f64 oracle against facts fixed by the pages and by mathematics.

None of these checks re-calls the oracle against itself: each compares it with a hand-worked
fixture (tests/golden/), an independent library (numpy's float16), a closed form or an
invariant chosen so that a plausible slip (a dropped term, a wrong sign or index, swapped
nibbles, a transposed operand) fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle
from conftest import golden_bytes, read_golden

Q4_0, Q8_0, Q4_K = oracle.Q4_0, oracle.Q8_0, oracle.Q4_K


@pytest.fixture(scope="module", autouse=True)
def _build():
    oracle.build(force=False)


def f16_bytes(val: float) -> bytes:
    return np.array([val], dtype="<f2").tobytes()


# ----------------------------------------------------------------------------- f16

def test_f16_golden_table():
    for bits, val in read_golden("f16_bits.txt"):
        got = oracle.f16(int(bits, 16))
        want = float(val)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (bits, got, want)


def test_f16_every_pattern_matches_numpy():
    bits = np.arange(1 << 16, dtype=np.uint32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    got = np.array([oracle.f16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ----------------------------------------------------------------------------- block decode

def _golden_weights(name):
    rows = read_golden(name)
    blk = golden_bytes(rows, "bytes")
    want = [float(r[-1]) for r in rows if r[0].isdigit()]
    return np.frombuffer(blk, dtype=np.uint8), np.array(want)


def test_q4_0_hand_block():
    blk, want = _golden_weights("q4_0_hand_block.txt")
    assert blk.size == 18 and want.size == 32
    got = oracle.dequant(Q4_0, blk, 32)[0]
    assert np.array_equal(got, want)


def test_q8_0_hand_block():
    blk, want = _golden_weights("q8_0_hand_block.txt")
    assert blk.size == 34 and want.size == 32
    got = oracle.dequant(Q8_0, blk, 32)[0]
    assert np.array_equal(got, want)


def _q4k_golden():
    rows = read_golden("q4_k_hand_block.txt")
    scales = golden_bytes(rows, "scales")
    pairs = {int(r[1]): (int(r[2]), int(r[3])) for r in rows if r[0] == "pair"}
    elems = {int(r[1]): (int(r[2]), float(r[3])) for r in rows if r[0] == "elem"}
    return scales, pairs, elems


def _q4k_hand_block(scales: bytes) -> np.ndarray:
    qs = bytes(((i & 15) | ((15 - (i & 15)) << 4)) for i in range(128))
    blk = f16_bytes(1.0) + f16_bytes(0.5) + scales + qs
    return np.frombuffer(blk, dtype=np.uint8)


def test_q4_k_hand_scale_pairs():
    scales, pairs, _ = _q4k_golden()
    assert len(scales) == 12 and len(pairs) == 8
    for j, (sc, m) in pairs.items():
        assert oracle.q4k_scale_min(scales, j) == (sc, m), j


def test_q4_k_hand_elements():
    scales, _, elems = _q4k_golden()
    w = oracle.dequant(Q4_K, _q4k_hand_block(scales), 256)[0]
    for e, (_nib, val) in elems.items():
        assert w[e] == val, (e, w[e], val)


def _q4_0_from_q4k_nibbles(qs128: bytes, d: float) -> np.ndarray:
    """8 Q4_0 blocks holding the same 256 nibbles in Q4_K element order (block 2c takes the low
    nibbles of qs[32c..32c+31], block 2c+1 the high ones)."""
    out = bytearray()
    for c in range(4):
        chunk = qs128[32 * c:32 * c + 32]
        for part in (0, 1):
            nib = [(b >> (4 * part)) & 15 for b in chunk]       # 32 elements of this sub-block
            out += f16_bytes(d)
            out += bytes(nib[j] | (nib[j + 16] << 4) for j in range(16))
    return np.frombuffer(bytes(out), dtype=np.uint8)


def test_q4_k_reduces_to_q4_0():
    """d = dmin = delta, all sc = 1, all m = 8  =>  w = delta * (q - 8), i.e. eight Q4_0 blocks."""
    g = np.random.default_rng(11)
    delta = 0.0078125
    # every pair (1, 8): pairs 0..3 low 6 bits 1 / 8, pairs 4..7: low nibbles 1 / 8, top bits 0
    scales = bytes([1, 1, 1, 1, 8, 8, 8, 8, 0x81, 0x81, 0x81, 0x81])
    for j in range(8):
        assert oracle.q4k_scale_min(scales, j) == (1, 8)
    for _ in range(20):
        qs = g.integers(0, 256, 128, dtype=np.uint8).tobytes()
        blk = np.frombuffer(f16_bytes(delta) + f16_bytes(delta) + scales + qs, dtype=np.uint8)
        wk = oracle.dequant(Q4_K, blk, 256)[0]
        w0 = oracle.dequant(Q4_0, _q4_0_from_q4k_nibbles(qs, delta), 256)[0]
        assert np.array_equal(wk, w0)


def _pack_one_pair(j: int, sc: int, m: int) -> bytes:
    """12 scale bytes holding (sc, m) at pair j and zeros elsewhere, from the bit positions of the
    6-bit pack (pairs 0..3 in low 6 bits of s[j], s[j+4]; pairs 4..7 split into a nibble of s[j+4]
    and the top 2 bits of s[j-4] / s[j])."""
    s = [0] * 12
    if j < 4:
        s[j] |= sc
        s[j + 4] |= m
    else:
        s[j + 4] |= (sc & 15) | ((m & 15) << 4)
        s[j - 4] |= (sc >> 4) << 6
        s[j] |= (m >> 4) << 6
    return bytes(s)


def test_q4_k_six_bit_sweep():
    """Each pair and each 6-bit value: nibbles all 1, x = indicator of sub-block j  =>
    y = 32 d sc_j  (with dmin = 0), and y = -32 dmin m_j (with d = 0)."""
    qs = bytes([0x11] * 128)
    for j in range(8):
        ind = np.zeros((1, 256))
        c, part = divmod(j, 2)
        ind[0, 64 * c + 32 * part: 64 * c + 32 * part + 32] = 1.0
        for v in range(64):
            s_sc = _pack_one_pair(j, v, 0)
            s_m = _pack_one_pair(j, 0, v)
            b1 = np.frombuffer(f16_bytes(0.5) + f16_bytes(0.0) + s_sc + qs, dtype=np.uint8)
            b2 = np.frombuffer(f16_bytes(0.0) + f16_bytes(0.25) + s_m + qs, dtype=np.uint8)
            y1, _ = oracle.gemv(Q4_K, b1, 1, 256, ind)
            y2, _ = oracle.gemv(Q4_K, b2, 1, 256, ind)
            assert y1[0, 0] == 32 * 0.5 * v, (j, v, y1)
            assert y2[0, 0] == -32 * 0.25 * v, (j, v, y2)
            # and nothing leaks into the other sub-blocks
            wk = oracle.dequant(Q4_K, b1, 256)[0]
            assert np.count_nonzero(wk) == (32 if v else 0)


def test_q4_0_upcast_to_q8_0_is_exact():
    """'Crate inferencelayer' docs, q4_0_to_q8_0n: d8 = d4, q8 = nib - 8 is lossless."""
    g = np.random.default_rng(5)
    N, K = 7, 96
    d = g.uniform(0.001, 0.02, size=(N, K // 32)).astype("<f2")
    nib = g.integers(0, 16, size=(N, K // 32, 32))
    q4 = bytearray()
    q8 = bytearray()
    for n in range(N):
        for b in range(K // 32):
            db = d[n, b].tobytes()
            q4 += db + bytes(int(nib[n, b, j] | (nib[n, b, j + 16] << 4)) for j in range(16))
            q8 += db + (nib[n, b] - 8).astype(np.int8).tobytes()
    W4 = np.frombuffer(bytes(q4), dtype=np.uint8)
    W8 = np.frombuffer(bytes(q8), dtype=np.uint8)
    assert np.array_equal(oracle.dequant(Q4_0, W4, K), oracle.dequant(Q8_0, W8, K))
    x = g.standard_normal((3, K))
    y4, _ = oracle.gemv(Q4_0, W4, N, K, x)
    y8, _ = oracle.gemv(Q8_0, W8, N, K, x)
    assert np.array_equal(y4, y8)


# ----------------------------------------------------------------------------- GEMV

def _distinct_scale_matrix(fmt, N, K):
    """Every block of the matrix gets its own scale d(n, b) = (n * nblk + b + 1) / 16 and weights
    all equal to d (Q4_0 nibble 9, Q8_0 q = 1)."""
    nblk = K // 32
    out = bytearray()
    for n in range(N):
        for b in range(nblk):
            d = (n * nblk + b + 1) / 16.0
            if fmt == Q4_0:
                out += f16_bytes(d) + bytes([0x99] * 16)
            else:
                out += f16_bytes(d) + bytes([1] * 32)
    return np.frombuffer(bytes(out), dtype=np.uint8)


@pytest.mark.parametrize("fmt", [Q4_0, Q8_0])
def test_gemv_one_hot_picks_row_and_block(fmt):
    """x = e_k selects column k: y[n] = w[n][k] = d(n, k // 32).  N != K catches a transposed
    operand, distinct scales catch a wrong row or block stride."""
    N, K = 5, 96
    W = _distinct_scale_matrix(fmt, N, K)
    nblk = K // 32
    for k in range(K):
        x = np.zeros((1, K))
        x[0, k] = 1.0
        y, A = oracle.gemv(fmt, W, N, K, x)
        want = np.array([(n * nblk + k // 32 + 1) / 16.0 for n in range(N)])
        assert np.array_equal(y[0], want), k
        assert np.array_equal(A[0], np.abs(want))


def test_gemv_hand_block_dot():
    """The Q4_0 hand block dotted with x = (1, 2, ..., 32), worked by hand:
    low half  sum_{j<16} (j+1) * 0.5 (j - 8):  0.5 * (-120 + 392)  =  136
    high half sum_{j<16} (j+17) * 0.5 (7 - j): 0.5 * (532 - 1068)  = -268
    y = -132;  A = sum |w x| = 0.5 * (120 + 392) + 0.5 * (532 + 1068) = 256 + 800 = 1056."""
    rows = read_golden("q4_0_hand_block.txt")
    blk = np.frombuffer(golden_bytes(rows, "bytes"), dtype=np.uint8)
    x = np.arange(1, 33, dtype=np.float64)[None, :]
    y, A = oracle.gemv(Q4_0, blk, 1, 32, x)
    assert y[0, 0] == -132.0
    assert A[0, 0] == 1056.0


@pytest.mark.parametrize("fmt", [Q4_0, Q8_0, Q4_K])
def test_gemv_zero_weights_give_exact_zero(fmt):
    g = np.random.default_rng(3)
    N, K = 6, 512
    if fmt == Q4_0:
        blk = f16_bytes(0.0173) + bytes([0x88] * 16)           # every nibble 8 -> w = 0
        W = np.frombuffer(blk * (N * K // 32), dtype=np.uint8)
    elif fmt == Q8_0:
        W = np.frombuffer((f16_bytes(0.0173) + bytes(32)) * (N * K // 32), dtype=np.uint8)
    else:
        blk = f16_bytes(0.0173) + f16_bytes(0.002) + bytes(12) + g.integers(0, 256, 128, dtype=np.uint8).tobytes()
        W = np.frombuffer(blk * (N * K // 256), dtype=np.uint8)
    x = g.standard_normal((3, K))
    y, A = oracle.gemv(fmt, W, N, K, x)
    assert np.all(y == 0.0) and np.all(A == 0.0)


@pytest.mark.parametrize("fmt", [Q4_0, Q8_0, Q4_K])
def test_gemv_scale_doubling_is_exact(fmt):
    """Adding 1 to every f16 exponent doubles each scale exactly, so y doubles exactly."""
    import workloads as wl
    g = np.random.default_rng(9)
    N, K = 9, 512
    W = wl.matrix(fmt, g, N, K)
    x = g.standard_normal((2, K))
    y1, _ = oracle.gemv(fmt, W, N, K, x)
    W2 = W.copy().reshape(N, -1, wl.BLOCK_BYTES[fmt])
    nscale = 2 if fmt == Q4_K else 1
    for s in range(nscale):
        h = W2[..., 2 * s:2 * s + 2].copy().view("<u2")
        h += 1 << 10
        W2[..., 2 * s:2 * s + 2] = h.view(np.uint8)
    y2, _ = oracle.gemv(fmt, W2.reshape(N, -1), N, K, x)
    assert np.array_equal(y2, 2 * y1)


def test_gemv_linear_in_x():
    import workloads as wl
    g = np.random.default_rng(13)
    N, K = 11, 256
    W = wl.q4_0_matrix(g, N, K)
    x1 = g.standard_normal((1, K))
    x2 = g.standard_normal((1, K))
    y1, A1 = oracle.gemv(Q4_0, W, N, K, x1)
    y2, A2 = oracle.gemv(Q4_0, W, N, K, x2)
    yd, _ = oracle.gemv(Q4_0, W, N, K, 2 * x1)
    ys, _ = oracle.gemv(Q4_0, W, N, K, x1 + x2)
    assert np.array_equal(yd, 2 * y1)
    assert np.all(np.abs(ys - (y1 + y2)) <= 1e-12 * (A1 + A2))


def test_gemv_row_subset_matches_full():
    import workloads as wl
    g = np.random.default_rng(17)
    N, K = 40, 256
    W = wl.q4_0_matrix(g, N, K)
    x = g.standard_normal((3, K))
    y, A = oracle.gemv(Q4_0, W, N, K, x)
    rows = np.array([39, 0, 17, 17, 5])
    ys, As = oracle.gemv(Q4_0, W, N, K, x, rows=rows)
    assert np.array_equal(ys, y[:, rows]) and np.array_equal(As, A[:, rows])


# ----------------------------------------------------------------------------- RMSNorm

def test_rmsnorm_constant_row():
    """x = c everywhere, gamma = 1: n = c / sqrt(c^2 + eps).  With c = 1e-3, eps = 1e-5 the value
    (0.3015...) tells eps inside the root from eps outside it or a missing eps."""
    K = 64
    c, eps = 1e-3, 1e-5
    n = oracle.rmsnorm(np.full((1, K), c), np.ones(K), eps)
    want = c / math.sqrt(c * c + eps)
    assert np.all(np.abs(n - want) <= 1e-15 * want)
    assert abs(want - 0.30151134457776363) < 1e-15


def test_rmsnorm_mean_not_sum_and_gamma():
    """sum x^2 = K and eps = 0  =>  rms = 1 and n = x * gamma exactly up to rounding; a sum in
    place of the mean would give n = x gamma / sqrt(K)."""
    g = np.random.default_rng(2)
    K = 128
    x = g.standard_normal(K)
    x *= math.sqrt(K / np.sum(x * x))
    gamma = g.uniform(0.5, 1.5, K)
    n = oracle.rmsnorm(x[None], gamma, 0.0)[0]
    assert np.all(np.abs(n - x * gamma) <= 1e-14 * np.abs(x * gamma) + 1e-300)


def test_rmsnorm_rows_independent_and_scale_invariant():
    g = np.random.default_rng(4)
    K = 96
    base = g.standard_normal(K)
    x = np.stack([base, 3.0 * base, 0.125 * base])
    gamma = g.uniform(0.5, 1.5, K)
    n = oracle.rmsnorm(x, gamma, 0.0)
    assert np.allclose(n[1], n[0], rtol=1e-14, atol=0) and np.allclose(n[2], n[0], rtol=1e-14, atol=0)


# ----------------------------------------------------------------------------- SwiGLU

SIGMA_1 = 0.7310585786300049   # logistic(1) = e / (1 + e)
SIGMA_2 = 0.8807970779778823   # logistic(2) = e^2 / (1 + e^2)


def test_swiglu_closed_forms():
    g = np.array([0.0, 1.0, 2.0, 40.0, -40.0, 0.0])
    u = np.array([5.0, 2.0, 1.0, 1.0, 1.0, -3.0])
    h = oracle.swiglu(g, u)
    assert h[0] == 0.0 and h[5] == 0.0
    assert abs(h[1] - 2 * SIGMA_1) < 1e-15          # silu on the gate: silu(1) * 2
    assert abs(h[2] - 2 * SIGMA_2) < 1e-15          # swapping roles would give silu(1)*2 here
    assert abs(h[3] - 40.0) < 1e-12                 # silu(g) -> g for large g
    assert abs(h[4]) < 1e-15                        # silu(g) -> 0 for very negative g


def test_swiglu_odd_part_identity():
    """silu(g) - silu(-g) = g for every g (u = 1)."""
    g = np.linspace(-6, 6, 101)
    hp = oracle.swiglu(g, np.ones_like(g))
    hm = oracle.swiglu(-g, np.ones_like(g))
    assert np.all(np.abs((hp - hm) - g) <= 1e-14 * (1 + np.abs(g)))


def test_gus_nrm_zero_gate_or_up_gives_zero():
    import workloads as wl
    g = np.random.default_rng(8)
    N, K = 12, 256
    Wz = np.frombuffer((f16_bytes(0.01) + bytes([0x88] * 16)) * (N * K // 32), dtype=np.uint8)
    Wr = wl.q4_0_matrix(g, N, K)
    x = g.standard_normal((2, K))
    gamma = g.uniform(0.5, 1.5, K)
    h1, *_ = oracle.qgemv_gus_nrm(Q4_0, Wz, Wr, N, K, x, gamma, 1e-5)
    h2, *_ = oracle.qgemv_gus_nrm(Q4_0, Wr, Wz, N, K, x, gamma, 1e-5)
    assert np.all(h1 == 0.0) and np.all(h2 == 0.0)


# ----------------------------------------------------------------------------- residual, argmax

def test_residual_with_zero_weights_is_identity():
    g = np.random.default_rng(21)
    N, K = 10, 64
    W = np.frombuffer((f16_bytes(0.5) + bytes([0x88] * 16)) * (N * K // 32), dtype=np.uint8)
    x = g.standard_normal((2, K))
    r = g.standard_normal((2, N))
    y, _ = oracle.qgemv_res(Q4_0, W, N, K, x, r)
    assert np.array_equal(y, r)


def test_residual_adds_the_product():
    N, K = 5, 96
    W = _distinct_scale_matrix(Q4_0, N, K)
    x = np.zeros((1, K))
    x[0, 40] = 1.0
    r = np.arange(N, dtype=np.float64)[None] * 100.0
    y, _ = oracle.qgemv_res(Q4_0, W, N, K, x, r)
    want = np.array([(n * 3 + 1 + 1) / 16.0 + 100.0 * n for n in range(N)])
    assert np.array_equal(y[0], want)


def test_argmax_ties_go_to_lowest_index():
    y = np.array([[1.0, 3.0, 2.0, 3.0], [-5.0, -5.0, -6.0, -7.0], [0.0, 0.0, 0.0, 0.0],
                  [-1.0, 2.0, 9.0, -9.0]])
    assert list(oracle.argmax(y)) == [1, 0, 0, 2]


# ----------------------------------------------------------------------------- routed experts

def test_moe_same_expert_everywhere_is_plain_gemv():
    import workloads as wl
    g = np.random.default_rng(31)
    n_exp, N, K, nb, topk = 4, 16, 256, 3, 8
    W = wl.q4_k_matrix(g, n_exp * N, K)
    x = g.standard_normal((nb, K))
    ids = np.full((nb, topk), 2, dtype=np.int32)
    p = np.full((nb, topk), 0.125)
    y, A = oracle.qgemv_moe(Q4_K, W, n_exp, N, K, x, ids, p)
    y0, A0 = oracle.gemv(Q4_K, W.reshape(n_exp, -1)[2], N, K, x)
    assert np.all(np.abs(y - y0) <= 1e-13 * A0)
    # top-1 with weight 1 is bit-for-bit the plain GEMV
    y1, _ = oracle.qgemv_moe(Q4_K, W, n_exp, N, K, x, ids[:, :1], np.ones((nb, 1)))
    assert np.array_equal(y1, y0)


def test_moe_weighted_sum_exact():
    """Experts with one-hot-readable outputs: expert 0 row n gives d0(n, b), expert 1 gives
    d1(n, b); with p = (0.25, 0.75) and x = e_k the result is exact."""
    N, K = 4, 64
    Wa = _distinct_scale_matrix(Q4_0, N, K)
    Wb = _distinct_scale_matrix(Q4_0, N, K).copy().reshape(N, -1, 18)
    h = Wb[..., 0:2].copy().view("<u2")
    h += 1 << 10                                    # expert 1 = 2 x expert 0
    Wb[..., 0:2] = h.view(np.uint8)
    W = np.concatenate([Wa, Wb.reshape(-1)])
    x = np.zeros((2, K))
    x[0, 3] = 1.0
    x[1, 50] = 1.0
    ids = np.array([[0, 1], [1, 0]], dtype=np.int32)
    p = np.array([[0.25, 0.75], [0.5, 0.5]])
    y, _ = oracle.qgemv_moe(Q4_0, W, 2, N, K, x, ids, p)
    want0 = [(0.25 * 1 + 0.75 * 2) * (n * 2 + 0 + 1) / 16.0 for n in range(N)]
    want1 = [(0.5 * 2 + 0.5 * 1) * (n * 2 + 1 + 1) / 16.0 for n in range(N)]
    assert np.array_equal(y[0], want0) and np.array_equal(y[1], want1)


def test_moe_rejects_bad_expert_id():
    import workloads as wl
    g = np.random.default_rng(1)
    W = wl.q4_0_matrix(g, 2 * 4, 32)
    with pytest.raises(ValueError):
        oracle.qgemv_moe(Q4_0, W, 2, 4, 32, np.ones((1, 32)), np.array([[2]], np.int32), np.ones((1, 1)))


# ----------------------------------------------------------------------------- gate / up roles

def test_gus_nrm_gate_and_up_take_their_own_roles():
    """x = e_0 with K = 64, gamma = 1, eps = 0 normalizes to exactly 8 e_0, so row n of each
    matrix contributes 8 w[n][0].  Weights are built so that (g, u) per row is a hand-chosen
    pair of small integers; h must be silu(g) u ("honeycrisp mod.rs", fused_norm_swiglu_down:
    silu on the gate), and every pair is chosen so that the swapped composite silu(u) g differs.
    The values use logistic(1) and logistic(2) only."""
    K = 64
    pairs = [(1, 2), (2, 1), (-1, 2), (2, -1), (0, 3)]
    want = [2 * SIGMA_1, 2 * SIGMA_2, -2 * (1 - SIGMA_1), -2 * SIGMA_2, 0.0]
    # silu(u) g, the composite with the roles swapped, for the first four pairs
    swapped = [2 * SIGMA_2, 2 * SIGMA_1, -2 * SIGMA_2, -2 * (1 - SIGMA_1)]
    N = len(pairs)

    def mat(vals):
        # d = 1/8 (f16 0x3000); element 0 of row n has nibble 8 + v (so w = v / 8), others 8
        out = bytearray()
        for v in vals:
            for b in range(K // 32):
                nib = [8] * 32
                if b == 0:
                    nib[0] = 8 + v
                out += f16_bytes(0.125) + bytes(nib[j] | (nib[j + 16] << 4) for j in range(16))
        return np.frombuffer(bytes(out), dtype=np.uint8)

    Wg = mat([p[0] for p in pairs])
    Wu = mat([p[1] for p in pairs])
    x = np.zeros((1, K))
    x[0, 0] = 1.0
    h, g, u, Ag, Au = oracle.qgemv_gus_nrm(Q4_0, Wg, Wu, N, K, x, np.ones(K), 0.0)
    assert np.array_equal(g[0], [p[0] for p in pairs])
    assert np.array_equal(u[0], [p[1] for p in pairs])
    assert np.array_equal(Ag[0], np.abs(g[0])) and np.array_equal(Au[0], np.abs(u[0]))
    for n in range(N):
        assert abs(h[0, n] - want[n]) <= 1e-15, (n, h[0, n], want[n])
        if n < 4:
            assert abs(h[0, n] - swapped[n]) > 0.1, n


# ----------------------------------------------------------------------------- brute force

def _blocks_from_nibbles(d_bits, nib):
    """Q4_0 bytes of one row: per block the f16 bits of d, then byte j = nib[j] | nib[j+16] << 4."""
    out = bytearray()
    for b in range(len(d_bits)):
        out += int(d_bits[b]).to_bytes(2, "little")
        q = nib[32 * b:32 * b + 32]
        out += bytes(int(q[j]) | (int(q[j + 16]) << 4) for j in range(16))
    return bytes(out)


@pytest.mark.parametrize("K", [32, 64])
def test_q4_0_brute_force_second_form(K):
    """Every row of up to 16 with random nibbles, small-integer x and d = 2^-k: the oracle equals,
    exactly, the block form d (sum_j q_j x_j - 8 sum_j x_j) worked in integers here, and
    A = sum |w x| equals d sum |q - 8| |x| (every value is a dyadic rational that f64 holds)."""
    g = np.random.default_rng(40 + K)
    for trial in range(20):
        N = int(g.integers(1, 17))
        nb = int(g.integers(1, 4))
        nblk = K // 32
        kexp = g.integers(1, 9, size=(N, nblk))                 # d = 2^-k
        nib = g.integers(0, 16, size=(N, K))
        x = g.integers(-9, 10, size=(nb, K))
        W = bytearray()
        for n in range(N):
            dbits = [int(np.array([2.0 ** -int(k)], "<f2").view("<u2")[0]) for k in kexp[n]]
            W += _blocks_from_nibbles(dbits, nib[n])
        y, A = oracle.gemv(Q4_0, np.frombuffer(bytes(W), np.uint8), N, K, x.astype(np.float64))
        for r in range(nb):
            for n in range(N):
                s = 0.0
                a = 0.0
                for b in range(nblk):
                    qx = sum(int(nib[n, 32 * b + j]) * int(x[r, 32 * b + j]) for j in range(32))
                    sx = sum(int(x[r, 32 * b + j]) for j in range(32))
                    ab = sum(abs(int(nib[n, 32 * b + j]) - 8) * abs(int(x[r, 32 * b + j]))
                             for j in range(32))
                    d = 2.0 ** -int(kexp[n, b])
                    s += d * (qx - 8 * sx)
                    a += d * ab
                assert y[r, n] == s, (trial, r, n, y[r, n], s)
                assert A[r, n] == a, (trial, r, n)


def test_q8_0_brute_force_integer_form():
    """Q8_0 with every signed byte (including -128) and small-integer x: y = d sum q x exactly."""
    g = np.random.default_rng(77)
    for K in (32, 64):
        N, nb = 16, 2
        q8 = g.integers(-128, 128, size=(N, K))
        q8[0, :32] = -128
        kexp = g.integers(1, 9, size=(N, K // 32))
        x = g.integers(-9, 10, size=(nb, K))
        W = bytearray()
        for n in range(N):
            for b in range(K // 32):
                W += np.array([2.0 ** -int(kexp[n, b])], "<f2").tobytes()
                W += q8[n, 32 * b:32 * b + 32].astype(np.int8).tobytes()
        y, _ = oracle.gemv(Q8_0, np.frombuffer(bytes(W), np.uint8), N, K, x.astype(np.float64))
        for r in range(nb):
            for n in range(N):
                s = sum(2.0 ** -int(kexp[n, j // 32]) * int(q8[n, j]) * int(x[r, j]) for j in range(K))
                assert y[r, n] == s, (K, r, n)


# ----------------------------------------------------------------------------- GELU (tanh form)

def test_gelu_tanh_closed_forms_and_erf_form():
    """gelu(0) = 0; gelu(g) - gelu(-g) = g (the tanh term is odd); gelu(g) -> g for large g and
    -> 0 for very negative g; and the tanh form stays within 1e-3 of the exact g Phi(g) (Phi
    from math.erf, independent of the oracle) over [-6, 6]; a missing 1/2, a wrong sign or a
    wrong cubic coefficient fails one of these."""
    g = np.linspace(-6, 6, 241)
    h = oracle.gelu_tanh_gate(g, np.ones_like(g))
    hm = oracle.gelu_tanh_gate(-g, np.ones_like(g))
    assert oracle.gelu_tanh_gate(np.zeros(1), np.ones(1))[0] == 0.0
    assert np.all(np.abs((h - hm) - g) <= 1e-13 * (1 + np.abs(g)))
    big = oracle.gelu_tanh_gate(np.array([30.0, -30.0]), np.array([1.0, 1.0]))
    assert abs(big[0] - 30.0) < 1e-12 and abs(big[1]) < 1e-12
    exact = np.array([x * 0.5 * (1 + math.erf(x / math.sqrt(2))) for x in g])
    assert np.max(np.abs(h - exact)) < 1e-3
    # u multiplies linearly
    u = np.linspace(-2, 2, 241)
    assert np.allclose(oracle.gelu_tanh_gate(g, u), h * u, rtol=1e-15, atol=0)


def test_gus_act_gelu_uses_the_gate():
    """The same hand-built (g, u) rows as the SiLU roles pin, through the GELU composite: the
    gate's GELU multiplies the up value (GELU values at 1 and 2 from the erf form agree with the
    tanh form within 1e-3, and the swapped composite differs by far more)."""
    K = 64
    pairs = [(1, 2), (2, 1), (2, -1)]

    def mat(vals):
        out = bytearray()
        for v in vals:
            for b in range(K // 32):
                nib = [8] * 32
                if b == 0:
                    nib[0] = 8 + v
                out += f16_bytes(0.125) + bytes(nib[j] | (nib[j + 16] << 4) for j in range(16))
        return np.frombuffer(bytes(out), dtype=np.uint8)

    x = np.zeros((1, K))
    x[0, 0] = 1.0
    h, g, u, _, _ = oracle.qgemv_gus_act_nrm(Q4_0, mat([p[0] for p in pairs]),
                                              mat([p[1] for p in pairs]), len(pairs), K, x,
                                              np.ones(K), 0.0, 1)
    phi = lambda t: 0.5 * (1 + math.erf(t / math.sqrt(2)))
    for n, (gv, uv) in enumerate(pairs):
        assert abs(h[0, n] - gv * phi(gv) * uv) < 1e-3 * abs(uv)
        assert abs(h[0, n] - uv * phi(uv) * gv) > 0.1


# ----------------------------------------------------------------------------- QK norm + RoPE

def test_qk_norm_rope_hand_example():
    """One Q head of 4 values [3, 4, 0, 0], gamma 1, eps 0: rms = 2.5, normalized [1.2, 1.6, 0, 0].
    Rope half 2 with (c, s) = (0.6, 0.8) for pair (0, 2) and (0, 1) for pair (1, 3):
    (1.2, 0) -> (0.72, 0.96) and (1.6, 0) -> (0, 1.6).  The K head [0, 0, 0, 2] normalizes to
    [0, 0, 0, 2] (rms 1), then (0, 0) -> (0, 0) and (0, 2) -> (-2, 0).  V head untouched."""
    y = np.array([[3.0, 4.0, 0.0, 0.0, 0.0, 0.0, 0.0, 2.0, 7.0, -1.0, 0.5, 9.0]])
    out = oracle.qk_norm_rope(y, 1, 1, 4, 2, np.ones(4), np.ones(4), 0.0,
                              np.array([[0.6, 0.0]]), np.array([[0.8, 1.0]]))
    want = [0.72, 0.0, 0.96, 1.6, 0.0, -2.0, 0.0, 0.0, 7.0, -1.0, 0.5, 9.0]
    assert np.allclose(out[0], want, rtol=0, atol=1e-15), out


def test_qk_norm_rope_invariants():
    g = np.random.default_rng(61)
    nb, nq, nkv, hd, rh = 3, 4, 2, 64, 16
    row = (nq + 2 * nkv) * hd
    y = g.standard_normal((nb, row))
    th = g.uniform(-3, 3, (nb, rh))
    c, s = np.cos(th), np.sin(th)
    qg, kg = g.uniform(0.5, 1.5, hd), g.uniform(0.5, 1.5, hd)
    out = oracle.qk_norm_rope(y, nq, nkv, hd, rh, qg, kg, 1e-6, c, s)
    # V heads untouched, bit for bit
    assert np.array_equal(out[:, (nq + nkv) * hd:], y[:, (nq + nkv) * hd:])
    # the rotation back (c, -s) gives the normalized heads: mean of (v / gamma)^2 ~ 1
    back = oracle.qk_norm_rope(out, nq, nkv, hd, rh, None, None, 0.0, c, -s)
    for h in range(nq + nkv):
        v = back[:, h * hd:(h + 1) * hd] / (qg if h < nq else kg)
        ms = np.mean(v * v, axis=1)
        raw = y[:, h * hd:(h + 1) * hd]
        want = np.mean(raw * raw, axis=1) / (np.mean(raw * raw, axis=1) + 1e-6)
        assert np.allclose(ms, want, rtol=1e-12, atol=0)
    # each rotated pair keeps its length; values past 2 rh are only normalized
    q0 = oracle.qk_norm_rope(y, nq, nkv, hd, rh, qg, kg, 1e-6, np.ones((nb, rh)), np.zeros((nb, rh)))
    for h in range(nq + nkv):
        a0, b0 = q0[:, h * hd:h * hd + rh], q0[:, h * hd + rh:h * hd + 2 * rh]
        a1, b1 = out[:, h * hd:h * hd + rh], out[:, h * hd + rh:h * hd + 2 * rh]
        assert np.allclose(a0 * a0 + b0 * b0, a1 * a1 + b1 * b1, rtol=1e-12, atol=1e-15)
        assert np.array_equal(q0[:, h * hd + 2 * rh:(h + 1) * hd], out[:, h * hd + 2 * rh:(h + 1) * hd])
    # a quarter turn (c, s) = (0, 1) maps (a, b) -> (-b, a) exactly
    qt = oracle.qk_norm_rope(y, nq, nkv, hd, rh, qg, kg, 1e-6, np.zeros((nb, rh)), np.ones((nb, rh)))
    for h in range(nq + nkv):
        assert np.array_equal(qt[:, h * hd:h * hd + rh], -q0[:, h * hd + rh:h * hd + 2 * rh])
        assert np.array_equal(qt[:, h * hd + rh:h * hd + 2 * rh], q0[:, h * hd:h * hd + rh])


def test_nrm_bias_with_zero_weights_is_the_bias():
    g = np.random.default_rng(63)
    N, K = 9, 64
    W = np.frombuffer((f16_bytes(0.5) + bytes([0x88] * 16)) * (N * K // 32), dtype=np.uint8)
    bias = g.standard_normal(N)
    y, A = oracle.qgemv_nrm_bias(Q4_0, W, N, K, g.standard_normal((2, K)), np.ones(K), 1e-5, bias)
    assert np.array_equal(y, np.stack([bias, bias])) and np.all(A == 0)


# ----------------------------------------------------------------------------- Q5_0, Q5_K, Q6_K

Q5_0, Q5_K, Q6_K = oracle.Q5_0, oracle.Q5_K, oracle.Q6_K


def test_q5_0_hand_block():
    """d = 0.25; element j (j < 16) has nibble j % 16 and fifth bit 1 for odd j; element j + 16
    has nibble 15 - j and fifth bit 1 for j < 8 (qh = 0x00FFAAAA little-endian):
    w = 0.25 (q - 16) with q listed by hand below."""
    qs = bytes((j & 15) | ((15 - j) << 4) for j in range(16))
    qh = (0x00FFAAAA).to_bytes(4, "little")
    blk = np.frombuffer(f16_bytes(0.25) + qh + qs, dtype=np.uint8)
    q = [j | (16 if j % 2 else 0) for j in range(16)] + [(15 - j) | (16 if j < 8 else 0) for j in range(16)]
    # spelled out: elements 0..15 -> 0,17,2,19,4,21,6,23,8,25,10,27,12,29,14,31
    assert q[:16] == [0, 17, 2, 19, 4, 21, 6, 23, 8, 25, 10, 27, 12, 29, 14, 31]
    assert q[16:] == [31, 30, 29, 28, 27, 26, 25, 24, 7, 6, 5, 4, 3, 2, 1, 0]
    w = oracle.dequant(Q5_0, blk, 32)[0]
    assert np.array_equal(w, 0.25 * (np.array(q, dtype=np.float64) - 16))


def test_q5_0_upcast_to_q8_0_is_exact():
    """'Crate inferencelayer' docs, q5_0_to_q8_0n: d8 = d5, q8 = (nib | bit << 4) - 16 is a
    lossless re-encoding."""
    g = np.random.default_rng(71)
    N, K = 6, 128
    import workloads as wl
    W5 = wl.q5_0_matrix(g, N, K).reshape(N, -1, 22)
    W8 = np.empty(W5.shape[:2] + (34,), np.uint8)
    W8[..., :2] = W5[..., :2]
    qh = W5[..., 2:6].copy().view("<u4")[..., 0]
    for j in range(16):
        lo = (W5[..., 6 + j] & 15) | (((qh >> j) & 1) << 4).astype(np.uint8)
        hi = (W5[..., 6 + j] >> 4) | (((qh >> (j + 16)) & 1) << 4).astype(np.uint8)
        W8[..., 2 + j] = (lo.astype(np.int16) - 16).astype(np.int8).view(np.uint8)
        W8[..., 18 + j] = (hi.astype(np.int16) - 16).astype(np.int8).view(np.uint8)
    W5, W8 = W5.reshape(N, -1), W8.reshape(N, -1)
    assert np.array_equal(oracle.dequant(Q5_0, W5, K), oracle.dequant(Q8_0, W8, K))
    x = g.standard_normal((2, K))
    assert np.array_equal(oracle.gemv(Q5_0, W5, N, K, x)[0], oracle.gemv(Q8_0, W8, N, K, x)[0])


def _q5k_from_q4k(b4: np.ndarray, qh: bytes) -> np.ndarray:
    b4 = b4.reshape(-1)
    return np.frombuffer(b4[:16].tobytes() + qh + b4[16:].tobytes(), dtype=np.uint8)


def test_q5_k_without_fifth_bits_is_q4_k_and_each_bit_adds_16_d_sc():
    """'Crate inferencelayer' docs, gemv_q5k_k_lcpp_src: Q4_K plus the fifth-bit plane, sub-block
    s taking bit s of qh[l].  With qh = 0 the weights equal Q4_K's on the same fields; setting
    only bit s of qh[l] raises exactly element (sub-block s, place l) by 16 d sc_s."""
    import workloads as wl
    g = np.random.default_rng(73)
    b4 = wl.q4_k_matrix(g, 1, 256)
    w4 = oracle.dequant(Q4_K, b4, 256)[0]
    assert np.array_equal(oracle.dequant(Q5_K, _q5k_from_q4k(b4, bytes(32)), 256)[0], w4)
    d = float(b4.reshape(-1)[0:2].view("<f2")[0])
    scales = b4.reshape(-1)[4:16].tobytes()
    for s_ in range(8):
        sc, _ = oracle.q4k_scale_min(scales, s_)
        for l in (0, 5, 31):
            qh = bytearray(32)
            qh[l] = 1 << s_
            w5 = oracle.dequant(Q5_K, _q5k_from_q4k(b4, bytes(qh)), 256)[0]
            e = 64 * (s_ // 2) + 32 * (s_ % 2) + l
            diff = w5 - w4
            assert diff[e] == 16 * d * sc and np.count_nonzero(diff) == (1 if sc else 0), (s_, l)


def _q6k_block(ql, qh, sc, d):
    return np.frombuffer(bytes(ql) + bytes(qh) + np.asarray(sc, np.int8).tobytes() + f16_bytes(d),
                         dtype=np.uint8)


def test_q6_k_zero_point_and_one_hot_sweep():
    """q = 32 everywhere (every low nibble 0, every high pair 2 = 0b10) gives w = 0.  Then each
    element on its own: its low nibble set to v and its high pair to 3 gives q = 48 + v, so only
    that element moves, to d sc (16 + v), with the scale of its sixteen."""
    ql0 = [0] * 128
    qh0 = [0xAA] * 64                       # every 2-bit field = 2
    sc = [((i * 37) % 255) - 127 for i in range(16)]
    d = 0.0078125
    assert np.all(oracle.dequant(Q6_K, _q6k_block(ql0, qh0, sc, d), 256)[0] == 0.0)
    for e in range(256):
        n, i = divmod(e, 128)
        quarter, l = divmod(i, 32)              # element 128 n + 32 quarter + l
        byte = 64 * n + l + (32 if quarter in (1, 3) else 0)
        shift = 4 if quarter >= 2 else 0
        v = (e * 7) % 16
        ql = list(ql0)
        ql[byte] |= v << shift
        qh = list(qh0)
        qh[32 * n + l] |= 3 << (2 * quarter)
        w = oracle.dequant(Q6_K, _q6k_block(ql, qh, sc, d), 256)[0]
        want = d * sc[8 * n + i // 16] * (16 + v)
        assert w[e] == want and np.count_nonzero(w) == (1 if want else 0), e


def test_k_quant_brute_force_second_forms():
    """K = 256 and 512, small-integer x, power-of-two d and dmin: the oracle equals, exactly, the
    sub-block forms worked in integers here: Q5_K sum_j (d sc_j sum q x - dmin m_j sum x) and
    Q6_K sum_j d sc_j sum (q - 32) x."""
    import workloads as wl
    g = np.random.default_rng(79)
    for K in (256, 512):
        for fmt in (Q5_K, Q6_K):
            N = 8
            W = wl.matrix(fmt, g, N, K).reshape(N, -1, wl.BLOCK_BYTES[fmt]).copy()
            e = g.integers(2, 8, size=W.shape[:2])
            doff = 0 if fmt == Q5_K else 208
            W[..., doff:doff + 2] = (2.0 ** -e).astype("<f2")[..., None].view(np.uint8)
            if fmt == Q5_K:
                W[..., 2:4] = (2.0 ** -(e + 1)).astype("<f2")[..., None].view(np.uint8)
            W = W.reshape(N, -1)
            x = g.integers(-5, 6, size=(2, K))
            y, _ = oracle.gemv(fmt, W, N, K, x.astype(np.float64))
            blk = W.reshape(N, -1, wl.BLOCK_BYTES[fmt])
            for r in range(2):
                for n in range(N):
                    tot = 0.0
                    for b in range(K // 256):
                        B = blk[n, b]
                        xs = x[r, 256 * b:256 * b + 256]
                        if fmt == Q5_K:
                            d = float(B[0:2].view("<f2")[0]); dm = float(B[2:4].view("<f2")[0])
                            for c in range(4):
                                for part in (0, 1):
                                    s_ = 2 * c + part
                                    sc, m = oracle.q4k_scale_min(B[4:16].tobytes(), s_)
                                    qx = sx = 0
                                    for l in range(32):
                                        nib = (int(B[48 + 32 * c + l]) >> (4 * part)) & 15
                                        q5 = nib | (((int(B[16 + l]) >> s_) & 1) << 4)
                                        qx += q5 * int(xs[64 * c + 32 * part + l])
                                        sx += int(xs[64 * c + 32 * part + l])
                                    tot += d * sc * qx - dm * m * sx
                        else:
                            d = float(B[208:210].view("<f2")[0])
                            scs = B[192:208].view(np.int8)
                            for hh in range(2):
                                for l in range(32):
                                    for qq in range(4):
                                        src = 64 * hh + l + (32 if qq in (1, 3) else 0)
                                        nib = (int(B[src]) >> (4 if qq >= 2 else 0)) & 15
                                        hi = (int(B[128 + 32 * hh + l]) >> (2 * qq)) & 3
                                        el = 128 * hh + 32 * qq + l
                                        tot += d * int(scs[8 * hh + (32 * qq + l) // 16]) * ((nib | hi << 4) - 32) * int(xs[el])
                    assert y[r, n] == tot, (fmt, K, r, n)


# ----------------------------------------------------------------------------- IQ4, Q1, affine Q4

IQ4_NL, IQ4_XS, Q1_0, AQ4 = oracle.IQ4_NL, oracle.IQ4_XS, oracle.Q1_0, oracle.AQ4
LINEAR_CB = np.arange(16) - 8          # codebook of Q4_0's own values


def test_iq4_nl_with_the_linear_codebook_is_q4_0():
    """Codebook i - 8 turns IQ4_NL into Q4_0 on the same 18 bytes (d, then index bytes in Q4_0's
    order): the dequantized rows must agree exactly; a second codebook is applied per index."""
    import workloads as wl
    g = np.random.default_rng(81)
    W = wl.q4_0_matrix(g, 5, 128)
    oracle.set_codebook(LINEAR_CB)
    assert np.array_equal(oracle.dequant(IQ4_NL, W, 128), oracle.dequant(Q4_0, W, 128))
    cb = wl.iq4_codebook()
    oracle.set_codebook(cb)
    blk = np.frombuffer(f16_bytes(0.5) + bytes((j & 15) | ((15 - j) << 4) for j in range(16)),
                        np.uint8)
    w = oracle.dequant(IQ4_NL, blk, 32)[0]
    want = [0.5 * int(cb[j]) for j in range(16)] + [0.5 * int(cb[15 - j]) for j in range(16)]
    assert np.array_equal(w, want)


def test_iq4_xs_sub_scales():
    """With every sub-scale 33 (ls - 32 = 1) and the linear codebook, an IQ4_XS super-block is
    eight Q4_0 blocks with the same d.  Then each sub-block s and each ls in 0..63 on its own:
    only sub-block s changes, by the factor ls - 32."""
    import workloads as wl
    g = np.random.default_rng(83)
    oracle.set_codebook(LINEAR_CB)
    d = 0.0625
    qs = g.integers(0, 256, 128, dtype=np.uint8)

    def blk(ls):
        sh = sum(((v >> 4) & 3) << (2 * s) for s, v in enumerate(ls))
        sl = sum((v & 15) << (4 * s) for s, v in enumerate(ls))
        return np.frombuffer(f16_bytes(d) + int(sh).to_bytes(2, "little") + int(sl).to_bytes(4, "little")
                             + qs.tobytes(), np.uint8)

    base = oracle.dequant(IQ4_XS, blk([33] * 8), 256)[0]
    q4 = np.concatenate([np.frombuffer(f16_bytes(d) + qs[16 * s:16 * s + 16].tobytes(), np.uint8)
                         for s in range(8)])
    assert np.array_equal(base, oracle.dequant(Q4_0, q4, 256)[0])
    for s in range(8):
        for v in (0, 1, 31, 32, 47, 63):
            ls = [33] * 8
            ls[s] = v
            w = oracle.dequant(IQ4_XS, blk(ls), 256)[0]
            want = base.copy()
            want[32 * s:32 * s + 32] *= (v - 32)
            assert np.array_equal(w, want), (s, v)


def test_q1_0_signs_and_brute_force():
    """Bit i of the sign bytes is element i: 1 -> +d, 0 -> -d; and with small-integer x the
    oracle equals d (2 sum_{bit=1} x - sum x) exactly."""
    d = 0.25
    bits = bytes([0b10110001] + [0] * 14 + [0xFF])
    w = oracle.dequant(Q1_0, np.frombuffer(f16_bytes(d) + bits, np.uint8), 128)[0]
    want = np.full(128, -d)
    for i in (0, 4, 5, 7):
        want[i] = d
    want[120:128] = d
    assert np.array_equal(w, want)
    g = np.random.default_rng(87)
    N, K = 9, 256
    W = np.concatenate([np.frombuffer(f16_bytes(2.0 ** -int(g.integers(1, 6))) +
                                      g.integers(0, 256, 16, dtype=np.uint8).tobytes(), np.uint8)
                        for _ in range(N * K // 128)]).reshape(N, -1)
    x = g.integers(-9, 10, size=(2, K))
    y, _ = oracle.gemv(Q1_0, W, N, K, x.astype(np.float64))
    for r in range(2):
        for n in range(N):
            tot = 0.0
            for b in range(K // 128):
                B = W[n, 18 * b:18 * b + 18]
                dd = float(B[0:2].view("<f2")[0])
                on = sum(int(x[r, 128 * b + i]) for i in range(128) if (B[2 + i // 8] >> (i % 8)) & 1)
                tot += dd * (2 * on - int(x[r, 128 * b:128 * b + 128].sum()))
            assert y[r, n] == tot


def test_aq4_even_odd_order_and_q4_0_equivalence():
    """Element 2i is the low nibble of byte i, 2i + 1 its high nibble; w = s q + c.  With c = -8 s
    an AQ4 block equals the Q4_0 block holding the same 32 nibbles in Q4_0's order."""
    g = np.random.default_rng(89)
    for _ in range(10):
        nib = g.integers(0, 16, 32)
        s = 2.0 ** -int(g.integers(2, 8))
        aq = np.frombuffer(f16_bytes(s) + f16_bytes(-8 * s) +
                           bytes(int(nib[2 * i]) | (int(nib[2 * i + 1]) << 4) for i in range(16)),
                           np.uint8)
        q4 = np.frombuffer(f16_bytes(s) + bytes(int(nib[j]) | (int(nib[j + 16]) << 4) for j in range(16)),
                           np.uint8)
        assert np.array_equal(oracle.dequant(AQ4, aq, 32)[0], oracle.dequant(Q4_0, q4, 32)[0])
    # a hand block: s = 0.5, c = 0.25, bytes 0x21 0x43 ...: elements 1, 2, 3, 4, ...
    blk = np.frombuffer(f16_bytes(0.5) + f16_bytes(0.25) +
                        bytes(((2 * i + 1) & 15) | (((2 * i + 2) & 15) << 4) for i in range(16)), np.uint8)
    w = oracle.dequant(AQ4, blk, 32)[0]
    assert np.array_equal(w, [0.5 * ((e + 1) & 15) + 0.25 for e in range(32)])

"""Seeded synthetic inputs for block-quantized GEMV, in GGUF-native block bytes.

Shared by the oracle's tests, the GPU parity tests and the bench.  This module
holds none of the GEMV method's arithmetic: it only draws random numbers and
lays them out as the block formats store them.

Block formats written here (little-endian, GGUF order of fields):
  * Q4_0: 18 B per 32 weights = f16 d, then 16 bytes of nibbles.
  * Q8_0: 34 B per 32 weights = f16 d, then 32 signed bytes.
  * Q4_K: 144 B per 256 weights = f16 d, f16 dmin, 12 bytes holding 8 packed
    6-bit (scale, min) pairs, then 128 bytes of nibbles.

Drawing every nibble byte uniformly makes each nibble U{0..15}.  The 12 Q4_K
scale bytes are a bijective packing of 8 x (6 + 6) bits, so uniform bytes give
independent U{0..63} scales and mins without knowing the packing.

Seeds: ``numpy.random.default_rng([cfg, tensor_id])`` with tensor ids
x=0, gamma=1, W/gate=2, up=3, down=4, router=5, experts=6.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

Q4_0, Q5_0, Q8_0, Q4_K, Q5_K, Q6_K = 2, 6, 8, 12, 13, 14
IQ4_NL, IQ4_XS, Q1_0, AQ4 = 20, 23, 40, 41
FMT_NAME = {Q4_0: "q4_0", Q5_0: "q5_0", Q8_0: "q8_0", Q4_K: "q4_k", Q5_K: "q5_k", Q6_K: "q6_k",
            IQ4_NL: "iq4_nl", IQ4_XS: "iq4_xs", Q1_0: "q1_0", AQ4: "aq4"}
BLOCK_BYTES = {Q4_0: 18, Q5_0: 22, Q8_0: 34, Q4_K: 144, Q5_K: 176, Q6_K: 210,
               IQ4_NL: 18, IQ4_XS: 136, Q1_0: 18, AQ4: 20}
BLOCK_WEIGHTS = {Q4_0: 32, Q5_0: 32, Q8_0: 32, Q4_K: 256, Q5_K: 256, Q6_K: 256,
                 IQ4_NL: 32, IQ4_XS: 256, Q1_0: 128, AQ4: 32}

T_X, T_GAMMA, T_W, T_UP, T_DOWN, T_ROUTER, T_EXPERTS = 0, 1, 2, 3, 4, 5, 6

# value ranges of the drawn scales, per format
Q4_0_D = (0.001, 0.02)
Q8_0_D = (0.0005, 0.01)
Q4_K_D = (1e-4, 5e-4)


def rng(cfg: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([cfg, tensor_id])


def row_bytes(fmt: int, K: int) -> int:
    assert K % BLOCK_WEIGHTS[fmt] == 0, (fmt, K)
    return K // BLOCK_WEIGHTS[fmt] * BLOCK_BYTES[fmt]


def _f16_bytes(vals: np.ndarray) -> np.ndarray:
    """f64 draws rounded to f16 (round-to-nearest-even), as little-endian bytes."""
    h = np.ascontiguousarray(vals.astype("<f2"))
    return h.view(np.uint8).reshape(*vals.shape, 2)


def q4_0_matrix(g: np.random.Generator, N: int, K: int, d_range=Q4_0_D) -> np.ndarray:
    """uint8 [N, K/32*18]: d ~ U[d_range] as f16, nibble bytes uniform."""
    nbk = K // 32
    blk = np.empty((N, nbk, 18), dtype=np.uint8)
    blk[..., 0:2] = _f16_bytes(g.uniform(*d_range, size=(N, nbk)))
    blk[..., 2:18] = g.integers(0, 256, size=(N, nbk, 16), dtype=np.uint8)
    return blk.reshape(N, nbk * 18)


def q8_0_matrix(g: np.random.Generator, N: int, K: int, d_range=Q8_0_D) -> np.ndarray:
    """uint8 [N, K/32*34]: d ~ U[d_range] as f16, q ~ U{-127..127} as signed bytes."""
    nbk = K // 32
    blk = np.empty((N, nbk, 34), dtype=np.uint8)
    blk[..., 0:2] = _f16_bytes(g.uniform(*d_range, size=(N, nbk)))
    q = g.integers(-127, 128, size=(N, nbk, 32), dtype=np.int16).astype(np.int8)
    blk[..., 2:34] = q.view(np.uint8)
    return blk.reshape(N, nbk * 34)


def q4_k_matrix(g: np.random.Generator, N: int, K: int, d_range=Q4_K_D) -> np.ndarray:
    """uint8 [N, K/256*144]: d, dmin ~ U[d_range] as f16; scale bytes and nibble bytes uniform."""
    nbk = K // 256
    blk = np.empty((N, nbk, 144), dtype=np.uint8)
    blk[..., 0:2] = _f16_bytes(g.uniform(*d_range, size=(N, nbk)))
    blk[..., 2:4] = _f16_bytes(g.uniform(*d_range, size=(N, nbk)))
    blk[..., 4:16] = g.integers(0, 256, size=(N, nbk, 12), dtype=np.uint8)
    blk[..., 16:144] = g.integers(0, 256, size=(N, nbk, 128), dtype=np.uint8)
    return blk.reshape(N, nbk * 144)


def q5_0_matrix(g: np.random.Generator, N: int, K: int, d_range=Q4_0_D) -> np.ndarray:
    """uint8 [N, K/32*22]: d ~ U[d_range] as f16, then 4 bytes of fifth bits and 16 nibble bytes,
    all uniform (so q = nib | bit << 4 ~ U{0..31})."""
    nbk = K // 32
    blk = np.empty((N, nbk, 22), dtype=np.uint8)
    blk[..., 0:2] = _f16_bytes(g.uniform(*d_range, size=(N, nbk)))
    blk[..., 2:22] = g.integers(0, 256, size=(N, nbk, 20), dtype=np.uint8)
    return blk.reshape(N, nbk * 22)


def q5_k_matrix(g: np.random.Generator, N: int, K: int, d_range=Q4_K_D) -> np.ndarray:
    """uint8 [N, K/256*176]: d, dmin ~ U[d_range] as f16; scale, fifth-bit and nibble bytes
    uniform."""
    nbk = K // 256
    blk = np.empty((N, nbk, 176), dtype=np.uint8)
    blk[..., 0:2] = _f16_bytes(g.uniform(*d_range, size=(N, nbk)))
    blk[..., 2:4] = _f16_bytes(g.uniform(*d_range, size=(N, nbk)))
    blk[..., 4:176] = g.integers(0, 256, size=(N, nbk, 172), dtype=np.uint8)
    return blk.reshape(N, nbk * 176)


def q6_k_matrix(g: np.random.Generator, N: int, K: int, d_range=Q4_K_D) -> np.ndarray:
    """uint8 [N, K/256*210]: ql and qh bytes uniform (q ~ U{0..63}), 16 scales ~ U{-127..127}
    as signed bytes, d ~ U[d_range] as f16 (last)."""
    nbk = K // 256
    blk = np.empty((N, nbk, 210), dtype=np.uint8)
    blk[..., 0:192] = g.integers(0, 256, size=(N, nbk, 192), dtype=np.uint8)
    sc = g.integers(-127, 128, size=(N, nbk, 16), dtype=np.int16).astype(np.int8)
    blk[..., 192:208] = sc.view(np.uint8)
    blk[..., 208:210] = _f16_bytes(g.uniform(*d_range, size=(N, nbk)))
    return blk.reshape(N, nbk * 210)


def iq4_codebook() -> np.ndarray:
    """A 16-entry signed, monotone, nonlinear codebook for the IQ4 formats (int8).  The pages
    give no values for the codebook, so the synthetic workloads use this one: 127 t |t|^0.6 at
    16 evenly spaced t in [-1, 1], rounded."""
    t = (np.arange(16) - 7.5) / 7.5
    return np.round(127 * t * np.abs(t) ** 0.6).astype(np.int8)


def iq4_nl_matrix(g: np.random.Generator, N: int, K: int, d_range=(0.0005, 0.002)) -> np.ndarray:
    """uint8 [N, K/32*18]: d ~ U[d_range] as f16, index bytes uniform."""
    nbk = K // 32
    blk = np.empty((N, nbk, 18), dtype=np.uint8)
    blk[..., 0:2] = _f16_bytes(g.uniform(*d_range, size=(N, nbk)))
    blk[..., 2:18] = g.integers(0, 256, size=(N, nbk, 16), dtype=np.uint8)
    return blk.reshape(N, nbk * 18)


def iq4_xs_matrix(g: np.random.Generator, N: int, K: int, d_range=(2e-5, 1e-4)) -> np.ndarray:
    """uint8 [N, K/256*136]: d ~ U[d_range] as f16; sub-scale and index bytes uniform."""
    nbk = K // 256
    blk = np.empty((N, nbk, 136), dtype=np.uint8)
    blk[..., 0:2] = _f16_bytes(g.uniform(*d_range, size=(N, nbk)))
    blk[..., 2:136] = g.integers(0, 256, size=(N, nbk, 134), dtype=np.uint8)
    return blk.reshape(N, nbk * 136)


def q1_0_matrix(g: np.random.Generator, N: int, K: int, d_range=(0.01, 0.05)) -> np.ndarray:
    """uint8 [N, K/128*18]: d ~ U[d_range] as f16, sign bytes uniform."""
    nbk = K // 128
    blk = np.empty((N, nbk, 18), dtype=np.uint8)
    blk[..., 0:2] = _f16_bytes(g.uniform(*d_range, size=(N, nbk)))
    blk[..., 2:18] = g.integers(0, 256, size=(N, nbk, 16), dtype=np.uint8)
    return blk.reshape(N, nbk * 18)


def aq4_matrix(g: np.random.Generator, N: int, K: int, d_range=Q4_0_D) -> np.ndarray:
    """uint8 [N, K/32*20]: scale s ~ U[d_range], bias c = -s U[6, 9] (weights spread about 0 as
    Q4_0's do), both f16; nibble bytes uniform."""
    nbk = K // 32
    blk = np.empty((N, nbk, 20), dtype=np.uint8)
    sc = g.uniform(*d_range, size=(N, nbk))
    blk[..., 0:2] = _f16_bytes(sc)
    blk[..., 2:4] = _f16_bytes(-sc * g.uniform(6.0, 9.0, size=(N, nbk)))
    blk[..., 4:20] = g.integers(0, 256, size=(N, nbk, 16), dtype=np.uint8)
    return blk.reshape(N, nbk * 20)


def matrix(fmt: int, g: np.random.Generator, N: int, K: int) -> np.ndarray:
    return {Q4_0: q4_0_matrix, Q5_0: q5_0_matrix, Q8_0: q8_0_matrix, Q4_K: q4_k_matrix,
            Q5_K: q5_k_matrix, Q6_K: q6_k_matrix, IQ4_NL: iq4_nl_matrix, IQ4_XS: iq4_xs_matrix,
            Q1_0: q1_0_matrix, AQ4: aq4_matrix}[fmt](g, N, K)


def normal_f32(g: np.random.Generator, shape) -> np.ndarray:
    return g.standard_normal(size=shape).astype(np.float32)


def gamma_f32(g: np.random.Generator, K: int) -> np.ndarray:
    return g.uniform(0.5, 1.5, size=K).astype(np.float32)


def route_top_k(z: np.ndarray, topk: int) -> tuple[np.ndarray, np.ndarray]:
    """Routing drawn from router logits z [nb, n_exp]: the topk largest (ties to the lower
    expert index), weights softmax over the selected logits (f64, stored f32).

    This is input preparation upstream of the routed GEMV, which takes (ids, weights) as
    given."""
    if not 1 <= topk <= z.shape[1]:
        raise ValueError(f"topk={topk} needs 1 <= topk <= n_exp={z.shape[1]}")
    order = np.argsort(-z, axis=1, kind="stable")[:, :topk]
    zs = np.take_along_axis(z, order, axis=1).astype(np.float64)
    e = np.exp(zs - zs.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    return order.astype(np.int32), p.astype(np.float32)


@dataclass
class Workload:
    """One synthetic workload: named arrays on the host (numpy)."""
    name: str
    fmt: int
    N: int
    K: int
    nb: int
    arrays: dict = field(default_factory=dict)
    params: dict = field(default_factory=dict)

    def weight_bytes(self) -> int:
        return int(sum(v.nbytes for k, v in self.arrays.items() if k.startswith("W")))


# --------------------------------------------------------------------------- the five workloads

def single_gemv(nb: int = 1, seed: int = 0, N: int = 1024, K: int = 1024) -> Workload:
    """Single Q4_0 GEMV, nb=1: W[1024 x 1024], x ~ N(0,1); seed 0."""
    w = Workload("q4_0_gemv_1024x1024", Q4_0, N, K, nb)
    w.arrays["W"] = q4_0_matrix(rng(seed, T_W), N, K)
    w.arrays["x"] = normal_f32(rng(seed, T_X), (nb, K))
    return w


def decode_mlp(seed: int = 1, hidden: int = 2048, inter: int = 8192) -> Workload:
    """LFM2-1.2B-like decode MLP, nb=1: RMSNorm(eps 1e-5, gamma ~ U[0.5,1.5]) on x[2048],
    Q4_0 gate+up [8192 x 2048] + SwiGLU, Q4_0 down [2048 x 8192] + residual."""
    w = Workload("lfm2_mlp_q4_0_2048x8192", Q4_0, inter, hidden, 1)
    w.arrays["x"] = normal_f32(rng(seed, T_X), (1, hidden))
    w.arrays["gamma"] = gamma_f32(rng(seed, T_GAMMA), hidden)
    w.arrays["Wg"] = q4_0_matrix(rng(seed, T_W), inter, hidden)
    w.arrays["Wu"] = q4_0_matrix(rng(seed, T_UP), inter, hidden)
    w.arrays["Wd"] = q4_0_matrix(rng(seed, T_DOWN), hidden, inter)
    w.params["eps"] = 1e-5
    return w


def qkv_q8(nb: int = 1, seed: int = 2, hidden: int = 1536, n_out: int = 1536 + 256 + 256) -> Workload:
    """Qwen2.5-coder-style attention input: RMSNorm + Q8_0 QKV W[2048 x 1536]."""
    w = Workload(f"qkv_q8_0_{n_out}x{hidden}_nb{nb}", Q8_0, n_out, hidden, nb)
    w.arrays["W"] = q8_0_matrix(rng(seed, T_W), n_out, hidden)
    w.arrays["x"] = normal_f32(rng(seed, T_X), (nb, hidden))
    w.arrays["gamma"] = gamma_f32(rng(seed, T_GAMMA), hidden)
    w.params["eps"] = 1e-5
    return w


def lm_head(nb: int = 1, seed: int = 3, vocab: int = 65536, hidden: int = 2048) -> Workload:
    """lm_head + argmax: Q4_0 W[65536 x 2048], x ~ N(0,1), nb in {1, 4}."""
    w = Workload(f"lm_head_q4_0_{vocab}x{hidden}_nb{nb}", Q4_0, vocab, hidden, nb)
    w.arrays["W"] = q4_0_matrix(rng(seed, T_W), vocab, hidden)
    w.arrays["x"] = normal_f32(rng(seed, T_X), (nb, hidden))
    return w


def moe_q4k(nb: int = 16, seed: int = 4, n_exp: int = 64, N: int = 1024, K: int = 2048,
            topk: int = 8) -> Workload:
    """Q4_K routed experts: 64 experts [1024 x 2048], top-8 per row by seeded router logits
    with softmax weights; nb=16 rows."""
    w = Workload(f"moe_q4_k_{n_exp}x{N}x{K}_top{topk}_nb{nb}", Q4_K, N, K, nb)
    w.arrays["W"] = q4_k_matrix(rng(seed, T_EXPERTS), n_exp * N, K)
    w.arrays["x"] = normal_f32(rng(seed, T_X), (nb, K))
    z = rng(seed, T_ROUTER).standard_normal(size=(nb, n_exp))
    ids, p = route_top_k(z, topk)
    w.arrays["ids"] = ids
    w.arrays["p"] = p
    w.params.update(n_exp=n_exp, topk=topk)
    return w

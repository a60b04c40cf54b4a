"""Seeded generators: determinism, value ranges and routing validity (no GPU)."""
import hashlib

import numpy as np

import workloads as wl


def _h(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_generation_is_deterministic_and_tensor_ids_differ():
    a = wl.q4_0_matrix(wl.rng(3, wl.T_W), 64, 256)
    b = wl.q4_0_matrix(wl.rng(3, wl.T_W), 64, 256)
    c = wl.q4_0_matrix(wl.rng(3, wl.T_UP), 64, 256)
    assert _h(a) == _h(b) and _h(a) != _h(c)


def _scales(blk, off):
    return blk[..., off:off + 2].copy().view("<f2").astype(np.float64)[..., 0]


def test_q4_0_ranges():
    W = wl.q4_0_matrix(wl.rng(0, wl.T_W), 256, 1024)
    assert W.shape == (256, 32 * 18)
    blk = W.reshape(256, 32, 18)
    d = _scales(blk, 0)
    lo, hi = wl.Q4_0_D
    assert d.min() >= np.float16(lo) - 1e-6 and d.max() <= np.float16(hi) + 1e-6
    nib = np.concatenate([(blk[..., 2:] & 15).ravel(), (blk[..., 2:] >> 4).ravel()])
    counts = np.bincount(nib, minlength=16)
    assert counts.size == 16 and counts.min() > 0.9 * counts.mean()


def test_q8_0_ranges():
    W = wl.q8_0_matrix(wl.rng(2, wl.T_W), 128, 1536)
    blk = W.reshape(128, 48, 34)
    q = blk[..., 2:].view(np.int8)
    assert q.min() == -127 and q.max() == 127
    d = _scales(blk, 0)
    assert d.min() >= np.float16(wl.Q8_0_D[0]) - 1e-7 and d.max() <= np.float16(wl.Q8_0_D[1]) + 1e-7


def test_q4_k_ranges():
    W = wl.q4_k_matrix(wl.rng(4, wl.T_EXPERTS), 64, 2048)
    blk = W.reshape(64, 8, 144)
    for off in (0, 2):
        v = _scales(blk, off)
        assert v.min() >= np.float16(wl.Q4_K_D[0]) - 1e-7 and v.max() <= np.float16(wl.Q4_K_D[1]) + 1e-7


def test_routing_valid():
    w = wl.moe_q4k()
    ids, p = w.arrays["ids"], w.arrays["p"]
    assert ids.shape == (16, 8) and p.shape == (16, 8)
    z = wl.rng(4, wl.T_ROUTER).standard_normal(size=(16, 64))
    for r in range(16):
        assert len(set(ids[r].tolist())) == 8
        assert np.all(np.diff(z[r, ids[r]]) <= 0)            # descending logits
        assert set(ids[r].tolist()) == set(np.argsort(-z[r])[:8].tolist())
        assert abs(float(p[r].astype(np.float64).sum()) - 1.0) < 1e-6
        assert np.all(np.diff(p[r]) <= 0) and np.all(p[r] > 0)


def test_workload_shapes():
    m = wl.decode_mlp()
    assert m.arrays["Wg"].shape == (8192, 2048 // 32 * 18)
    assert m.arrays["Wd"].shape == (2048, 8192 // 32 * 18)
    q = wl.qkv_q8(nb=4)
    assert q.arrays["W"].shape == (2048, 1536 // 32 * 34) and q.arrays["x"].shape == (4, 1536)
    assert wl.single_gemv().weight_bytes() == 589824

"""Host-side checks of the C ABI (no GPU): the library loads, exports every function the header
declares, sizes packed layouts and workspaces, and rejects bad arguments before any HIP call."""
import ctypes

import pytest

import dequant_gemv_q4_amd as q
from dequant_gemv_q4_amd import _binding as B

# Fake, suitably aligned addresses: every call below fails validation before touching them.
A256 = 0x7f0000000000
X16 = 0x7f0001000000
Y16 = 0x7f0002000000


@pytest.fixture(scope="module")
def lib():
    return q.lib()


def test_every_header_function_is_exported(lib):
    names = q.header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
        assert isinstance(getattr(lib, n), ctypes._CFuncPtr)
    assert set(names) == set(B._SIGS), "binding and header disagree"


def test_packed_bytes_equal_gguf_bytes():
    for fmt, bw, bb in ((q.Q4_0, 32, 18), (q.Q8_0, 32, 34), (q.Q4_K, 256, 144), (q.Q5_0, 32, 22),
                        (q.Q5_K, 256, 176), (q.Q6_K, 256, 210), (q.IQ4_NL, 32, 18),
                        (q.IQ4_XS, 256, 136), (q.Q1_0, 128, 18), (q.AQ4, 32, 20)):
        for N, K in ((1024, 1024), (65536, 2048), (2048, 8192), (16, 256)):
            gguf = N * K // bw * bb
            got = q.qgemv_packed_bytes(fmt, N, K)
            assert gguf <= got <= gguf + 1024, (fmt, N, K, got, gguf)
    assert q.qgemv_packed_bytes(q.Q4_0, 65536, 2048) == 75497472


def test_packed_bytes_rejects_bad_shapes():
    assert q.qgemv_packed_bytes(q.Q4_0, 16, 48) == -1        # K not a multiple of 32
    assert q.qgemv_packed_bytes(q.Q4_K, 16, 512 + 32) == -1  # K not a multiple of 256
    assert q.qgemv_packed_bytes(q.Q4_0, 0, 64) == -1
    assert q.qgemv_packed_bytes(7, 16, 64) == -1
    assert q.qgemv_packed_bytes(q.IQ4_XS, 16, 512 + 32) == -1
    assert q.qgemv_packed_bytes(q.Q1_0, 16, 64) == -1        # K not a multiple of 128
    assert q.qgemv_packed_bytes(q.AQ4, 16, 48) == -1


def test_workspace_sizes():
    assert q.qgemv_workspace_bytes(q.OP_GEMV, q.Q4_0, 1024, 1024, 1) == 0
    assert q.qgemv_workspace_bytes(q.OP_GUS_NRM, q.Q4_0, 8192, 2048, 1) == 0
    assert q.qgemv_workspace_bytes(q.OP_ARGMAX, q.Q4_0, 65536, 2048, 4) >= 256 + 4 * 8
    moe = q.qgemv_workspace_bytes(q.OP_MOE, q.Q4_K, 1024, 2048, 16, 64, 8)
    assert moe >= 16 * 8 * 1024 * 4
    assert q.qgemv_workspace_bytes(q.OP_MOE, q.Q4_K, 1024, 2048, 16, 64, 9) == -1
    assert q.qgemv_workspace_bytes(q.OP_ARGMAX, q.Q4_0, 1024, 1024, 17) == -1
    assert q.qgemv_workspace_bytes(99, q.Q4_0, 1024, 1024, 1) == -1


def _st(fn, *args):
    return getattr(q.lib(), fn)(*args)


def test_qgemv_validation_codes(lib):
    ok = (q.Q4_0, A256, 1024, 1024, X16, 1, Y16, None, 0, None)
    def call(**kw):
        a = list(ok)
        names = ["fmt", "W", "N", "K", "x", "nb", "y", "ws", "wsb", "s"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return lib.qgemv(*a)
    assert call(fmt=5) == 2
    assert call(W=None) == 1
    assert call(x=None) == 1
    assert call(y=None) == 1
    assert call(nb=0) == 3 and call(nb=17) == 3
    assert call(N=0) == 3
    assert call(K=48) == 3 and call(K=0) == 3 and call(K=131072) == 3
    assert call(W=A256 + 16) == 4
    assert call(x=X16 + 4) == 4
    assert call(y=Y16 + 2) == 4
    assert call(y=A256 + 64) == 7           # output inside the weights
    assert call(y=X16) == 7                 # output on the input


def test_other_entry_points_validate(lib):
    # qgemv_nrm: gamma NULL / misaligned, negative eps
    assert lib.qgemv_nrm(q.Q4_0, A256, 64, 64, X16, None, 1e-5, 1, Y16, None, 0, None) == 1
    assert lib.qgemv_nrm(q.Q4_0, A256, 64, 64, X16, X16 + 1024 + 4, 1e-5, 1, Y16, None, 0, None) == 4
    assert lib.qgemv_nrm(q.Q4_0, A256, 64, 64, X16, X16 + 1024, -1.0, 1, Y16, None, 0, None) == 3
    # qgemv_gus_nrm: Wu NULL and misaligned
    assert lib.qgemv_gus_nrm(q.Q4_0, A256, None, 64, 64, X16, X16 + 1024, 1e-5, 1, Y16, None, 0, None) == 1
    assert lib.qgemv_gus_nrm(q.Q4_0, A256, A256 + 8, 64, 64, X16, X16 + 1024, 1e-5, 1, Y16, None, 0, None) == 4
    # qgemv_res: residual partially overlapping the output is refused, identical is fine
    assert lib.qgemv_res(q.Q4_0, A256, 64, 64, X16, None, 1, Y16, None, 0, None) == 1
    assert lib.qgemv_res(q.Q4_0, A256, 64, 64, X16, Y16 + 4, 1, Y16, None, 0, None) == 7
    # qgemv_argmax: workspace missing / too small
    assert lib.qgemv_argmax(q.Q4_0, A256, 64, 64, X16, 1, Y16, Y16 + 4096, None, 0, None) == 5
    assert lib.qgemv_argmax(q.Q4_0, A256, 64, 64, X16, 1, Y16, Y16 + 4096, A256 + (1 << 24), 16, None) == 5
    assert lib.qgemv_argmax(q.Q4_0, A256, 64, 64, X16, 1, Y16, None, A256 + (1 << 24), 4096, None) == 1
    # qgemv_moe: topk out of range, workspace too small
    ws = A256 + (1 << 26)
    assert lib.qgemv_moe(q.Q4_K, A256, 4, 64, 256, X16, 2, Y16 + 8192, Y16 + 16384, 9, Y16, ws, 1 << 20, None) == 3
    assert lib.qgemv_moe(q.Q4_K, A256, 0, 64, 256, X16, 2, Y16 + 8192, Y16 + 16384, 2, Y16, ws, 1 << 20, None) == 3
    assert lib.qgemv_moe(q.Q4_K, A256, 4, 64, 256, X16, 2, Y16 + 8192, Y16 + 16384, 2, Y16, ws, 64, None) == 5
    assert lib.qgemv_moe(q.Q4_K, A256, 4, 64, 256, X16, 2, None, Y16 + 16384, 2, Y16, ws, 1 << 20, None) == 1
    # qgemv_pack: format, alignment, overlap
    assert lib.qgemv_pack(3, A256, 64, 64, A256 + (1 << 20), None) == 2
    assert lib.qgemv_pack(q.Q4_0, A256, 64, 64, A256 + (1 << 20) + 128, None) == 4
    assert lib.qgemv_pack(q.Q4_0, A256, 64, 64, A256, None) == 7
    # the codebook formats need their codebook; the others ignore it
    for fmt in (q.IQ4_NL, q.IQ4_XS):
        assert lib.qgemv_pack(fmt, A256, 64, 256, A256 + (1 << 20), None) == 1
        assert lib.qgemv_pack_codebook(fmt, A256, 64, 256, None, A256 + (1 << 20), None) == 1
    cb = (ctypes.c_int8 * 16)(*range(-8, 8))
    assert lib.qgemv_pack_codebook(q.IQ4_NL, A256, 64, 256, ctypes.addressof(cb),
                                   A256 + (1 << 20) + 128, None) == 4
    # routed experts take Q4_0, Q8_0 and Q4_K only
    ws = A256 + (1 << 26)
    for fmt in (q.IQ4_NL, q.IQ4_XS, q.Q1_0, q.AQ4, q.Q5_0, q.Q6_K):
        assert lib.qgemv_moe(fmt, A256, 4, 64, 256, X16, 2, Y16 + 8192, Y16 + 16384, 2, Y16, ws,
                             1 << 20, None) == 2


def test_status_strings():
    for s in range(8):
        assert q.qgemv_status_str(s)
    assert "unknown" in q.qgemv_status_str(99)

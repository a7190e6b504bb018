"""C-ABI checks that need no GPU: the library loads, exports every function
include/qmv.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import bit_affine_quantized_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmv.h")

FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation runs first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:int|const char\s*\*)\s*(\w+)\s*\(", text, re.M)


def test_header_declares_the_boundary():
    names = set(declared_functions())
    assert {"qmv_pack", "qmv", "qmv_gate_up", "qmv_silu_gate_resid",
            "gather_qmv", "qmv_dequantize", "qmv_unpack_codes",
            "qmv_last_error"} <= names


def test_library_exports_every_declared_symbol():
    L = q.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(declared_functions()) - {"qmv_last_error"} == set(q.SIGNATURES)


def _qmv(**kw):
    a = dict(x=FAKE, w=FAKE, s=FAKE, b=FAKE, y=FAKE, M=1, N=16, K=64, g=64,
             bits=4, transpose=1, out=0)
    a.update(kw)
    return q.lib().qmv(a["x"], a["w"], a["s"], a["b"], a["y"], a["M"], a["N"],
                       a["K"], a["g"], a["bits"], a["transpose"], a["out"],
                       None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(bits=7), q.QMV_EINVAL, "bits=7"),
    (dict(bits=1), q.QMV_EINVAL, "bits=1"),
    (dict(g=48, K=96), q.QMV_EINVAL, "group_size=48"),
    (dict(g=16, K=64), q.QMV_EINVAL, "group_size=16"),
    (dict(K=96), q.QMV_EINVAL, "not a multiple"),
    (dict(N=0), q.QMV_EINVAL, "positive"),
    (dict(K=0), q.QMV_EINVAL, "positive"),
    (dict(M=0), q.QMV_EINVAL, "M=0"),
    (dict(x=None), q.QMV_EINVAL, "null"),
    (dict(w=None), q.QMV_EINVAL, "null"),
    (dict(y=None), q.QMV_EINVAL, "null"),
    (dict(out=2), q.QMV_EINVAL, "out_dtype"),
    (dict(transpose=2), q.QMV_EINVAL, "transpose=2"),
    # transpose=0 packs along N: N must be a multiple of the group size
    (dict(transpose=0, N=48, K=64), q.QMV_EINVAL, "N=48 is not a multiple"),
    (dict(transpose=0, N=64, K=0), q.QMV_EINVAL, "positive"),
    (dict(transpose=0, N=128, w=ctypes.c_void_p(0x1008)), q.QMV_EINVAL, "aligned"),
    (dict(x=ctypes.c_void_p(0x1002)), q.QMV_EINVAL, "aligned"),
    (dict(w=ctypes.c_void_p(0x1008)), q.QMV_EINVAL, "aligned"),
])
def test_qmv_rejects_bad_arguments(kw, code, msg):
    assert _qmv(**kw) == code
    assert msg in q.lib().qmv_last_error().decode()


def test_pack_rejects_bad_arguments():
    L = q.lib()
    assert L.qmv_pack(FAKE, 4, 64, 64, 7, FAKE, FAKE, FAKE, None) == q.QMV_EINVAL
    assert L.qmv_pack(None, 4, 64, 64, 4, FAKE, FAKE, FAKE, None) == q.QMV_EINVAL
    assert L.qmv_pack(FAKE, 4, 100, 64, 4, FAKE, FAKE, FAKE, None) == q.QMV_EINVAL


def test_fused_reject_bad_arguments():
    L = q.lib()
    assert L.qmv_gate_up(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                         16, 64, 64, 4, None) == q.QMV_EINVAL
    assert L.qmv_silu_gate_resid(FAKE, None, None, FAKE, FAKE, FAKE, FAKE, 16,
                                 64, 64, 8, 0, None) == q.QMV_EINVAL
    assert L.qmv_silu_gate_resid(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 16,
                                 64, 64, 8, 5, None) == q.QMV_EINVAL


def test_gather_rejects_bad_arguments():
    L = q.lib()
    base = [FAKE, 1, FAKE, FAKE, FAKE, 4]
    tail = [FAKE, 1, 16, 64, 64, 4]
    # exactly one index array
    assert L.gather_qmv(*base, FAKE, None, 8, *tail, 1, 0, 0, None) == q.QMV_EINVAL
    assert "both" in L.qmv_last_error().decode()
    # P must be positive when indices are given
    assert L.gather_qmv(*base, FAKE, FAKE, 0, *tail, 1, 0, 0, None) == q.QMV_EINVAL
    # E must be positive
    assert L.gather_qmv(FAKE, 1, FAKE, FAKE, FAKE, 0, FAKE, FAKE, 8, *tail, 1,
                        0, 0, None) == q.QMV_EINVAL
    # transpose=0 not implemented
    assert L.gather_qmv(*base, FAKE, FAKE, 8, *tail, 0, 0, 0, None) == \
        q.QMV_EUNSUPPORTED
    # one expert's packed weight at 2 GiB: past the 32-bit offsets
    assert L.gather_qmv(*base, FAKE, FAKE, 8, FAKE, 1, 1 << 20, 4096, 64, 4, 1,
                        0, 0, None) == q.QMV_EUNSUPPORTED
    assert "2 GiB" in L.qmv_last_error().decode()


def test_unpack_rejects_bad_arguments():
    L = q.lib()
    assert L.qmv_unpack_codes(FAKE, 4, 48, 4, FAKE, None) == q.QMV_EINVAL
    assert L.qmv_unpack_codes(FAKE, 4, 64, 7, FAKE, None) == q.QMV_EINVAL
    assert L.qmv_unpack_codes(None, 4, 64, 4, FAKE, None) == q.QMV_EINVAL


def test_dequantize_rejects_bad_arguments():
    L = q.lib()

    def call(**kw):
        a = dict(w=FAKE, s=FAKE, b=FAKE, out=FAKE, N=4, K=64, g=64, bits=4, dt=0)
        a.update(kw)
        rc = L.qmv_dequantize(a["w"], a["s"], a["b"], a["out"], a["N"], a["K"],
                              a["g"], a["bits"], a["dt"], None)
        return rc, L.qmv_last_error().decode()
    for kw, msg in [(dict(bits=7), "bits=7"), (dict(g=48, K=96), "group_size=48"),
                    (dict(K=96), "not a multiple"), (dict(N=0), "positive"),
                    (dict(w=None), "null"), (dict(out=None), "null"),
                    (dict(dt=2), "out_dtype"),
                    (dict(out=ctypes.c_void_p(0x1004)), "aligned"),
                    (dict(w=ctypes.c_void_p(0x1008)), "aligned")]:
        rc, m = call(**kw)
        assert rc == q.QMV_EINVAL and msg in m, (kw, rc, m)


def test_error_message_clears_on_success_path_is_thread_local():
    import threading
    L = q.lib()
    _qmv(bits=7)
    seen = {}

    def other():
        seen["msg"] = L.qmv_last_error().decode()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "bits=7" in L.qmv_last_error().decode()


def _ws_bytes(M, N, K, g=64, bits=4, transpose=1):
    out = ctypes.c_size_t(12345)
    rc = q.lib().qmv_workspace_bytes(M, N, K, g, bits, transpose,
                                      ctypes.byref(out))
    return rc, int(out.value)


@pytest.mark.parametrize("M", (1, 2, 3, 4))
def test_workspace_none_for_matvec_slabs(M):
    assert _ws_bytes(M, 14336, 4096) == (q.QMV_OK, 0)


@pytest.mark.parametrize("M", (5, 8, 16))
@pytest.mark.parametrize("K", (2048, 4096))
def test_workspace_none_for_one_pass_matrix_cores(M, K):
    """4-bit, K = 2048 or 4096, 5-16 rows of x: one pass, no slices."""
    assert _ws_bytes(M, 4096, K) == (q.QMV_OK, 0)


@pytest.mark.parametrize("M,N,K,transpose", [(1, 4096, 4096, 0), (4, 4096, 4096, 0),
                                             (8, 4096, 8192, 1), (17, 4096, 4096, 1),
                                             (64, 4096, 4096, 1), (300, 1024, 2048, 1)])
def test_workspace_split_k_sizes(M, N, K, transpose):
    rc, nbytes = _ws_bytes(M, N, K, transpose=transpose)
    assert rc == q.QMV_OK
    # S slices x (rows of x in the largest slab) x N fp32 partial sums
    assert nbytes > 0 and nbytes % (4 * N) == 0
    rows = min(M, 4) if transpose == 0 else 16 * ((min(M, 64) + 15) // 16)
    assert (nbytes // (4 * N)) % rows == 0


def test_workspace_bytes_validates_sizes():
    rc, _ = _ws_bytes(1, 16, 96)           # K not a multiple of 64
    assert rc == q.QMV_EINVAL
    rc, _ = _ws_bytes(0, 16, 64)
    assert rc == q.QMV_EINVAL
    assert q.lib().qmv_workspace_bytes(1, 16, 64, 64, 4, 1, None) == q.QMV_EINVAL


def test_with_workspace_too_small_is_rejected_before_any_launch():
    rc, need = _ws_bytes(1, 4096, 4096, transpose=0)
    assert rc == q.QMV_OK and need > 0
    L = q.lib()
    rc = L.qmv_with_workspace(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4096, 4096, 64, 4,
                              0, 0, FAKE, need - 16, None)
    assert rc == q.QMV_EINVAL
    assert b"workspace" in L.qmv_last_error()
    rc = L.qmv_with_workspace(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4096, 4096, 64, 4,
                              0, 0, ctypes.c_void_p(0x1008), need, None)
    assert rc == q.QMV_EINVAL and b"aligned" in L.qmv_last_error()


def test_noalloc_rejects_calls_beyond_its_scratch():
    """qmv_noalloc's static scratch holds 16 MiB; a larger split-K call is
    refused before any HIP call."""
    rc, need = _ws_bytes(3, 65536, 65536, transpose=0)
    assert rc == q.QMV_OK and need > 16 << 20
    L = q.lib()
    rc = L.qmv_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 65536, 65536, 64, 4, 0, 0, None)
    assert rc == q.QMV_EINVAL
    assert b"scratch" in L.qmv_last_error()

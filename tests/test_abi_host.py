"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before launching anything (no GPU
needed: every call here fails validation or only computes sizes)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
LIB = os.path.join(ROOT, "gated_delta_rule_48_amd", "libkda.so")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(kda_\w+)\s*\(", src, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libkda.so not built")
    return ctypes.CDLL(LIB)


def test_header_declares_expected_entry_points():
    names = _declared()
    for n in ("kda_chunk_fwd", "kda_recurrent_step", "kda_chunk_fwd_workspace_size",
              "kda_chunk_fwd_check", "kda_status_string", "kda_version", "kda_chunk_bwd",
              "kda_chunk_bwd_workspace_size", "kda_prepare_inputs", "kda_recurrent_step_raw",
              "kda_chunk_fwd_c128", "kda_chunk_fwd_c128_workspace_size"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), f"missing export {name}"


def _sizes(lib):
    f = lib.kda_chunk_fwd_workspace_size
    f.restype = ctypes.c_size_t
    f.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_int, ctypes.c_int]
    return f


def test_workspace_size_rules(lib):
    f = _sizes(lib)
    assert f(32768, 1, 32, 128, 128, 0, 0) > 0
    assert f(32768, 1, 32, 96, 128, 0, 0) == 0         # d_k unsupported
    assert f(32768, 0, 32, 128, 128, 0, 0) == 0        # no sequences
    assert f(-1, 1, 32, 128, 128, 0, 0) == 0
    assert f(32768, 1, 32, 128, 128, 7, 0) == 0        # bad dtype
    # monotone in T, and fp32 intermediates need more than bf16
    assert f(65536, 1, 32, 128, 128, 0, 0) > f(32768, 1, 32, 128, 128, 0, 0)
    assert f(32768, 1, 32, 128, 128, 1, 0) > f(32768, 1, 32, 128, 128, 0, 0)


def _chunk(lib):
    f = lib.kda_chunk_fwd
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    f.restype = ctypes.c_int
    f.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, ctypes.c_int, ctypes.c_int, vp, vp, vp,
                  ctypes.c_size_t, vp]
    return f


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def test_chunk_fwd_rejects_bad_arguments(lib):
    f = _chunk(lib)
    P = FAKE
    args = dict(q=P, k=P, v=P, g=P, beta=P, S0=None, cu=None, N=1, T=128, H=2, dk=64, dv=64, dt=0, gk=0,
                o=P, S_T=None, ws=P, wsb=1 << 40, stream=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["cu"], a["N"], a["T"], a["H"], a["dk"],
                 a["dv"], a["dt"], a["gk"], a["o"], a["S_T"], a["ws"], a["wsb"], a["stream"])

    assert call(dk=96) == UNSUPPORTED
    assert call(dv=32) == UNSUPPORTED
    assert call(dt=3) == UNSUPPORTED
    assert call(gk=9) == UNSUPPORTED
    assert call(H=0) == INVALID
    assert call(N=0) == INVALID
    assert call(T=-5) == INVALID
    assert call(N=3) == INVALID                   # 128 % 3 != 0 without cu_seqlens
    assert call(q=None) == INVALID
    assert call(q=P + 2) == INVALID               # q read in element pairs
    assert call(o=P + 1) == INVALID               # not element aligned
    assert call(ws=None) == WORKSPACE
    assert call(ws=P + 16) == WORKSPACE           # workspace must be 256-byte aligned
    assert call(wsb=16) == WORKSPACE
    # one intra-chunk workgroup per (chunk, head) in a single grid dimension:
    # ceil(T / 64) + N chunks times H must stay below 2^23
    assert call(T=64 * (2**23 - 2), H=1, ws=None) == WORKSPACE   # 2^23 - 1 pairs: accepted
    assert call(T=64 * (2**23 - 1), H=1, ws=None) == UNSUPPORTED  # 2^23 pairs
    assert call(T=2**31 - 64, H=64) == UNSUPPORTED


def _c128(lib):
    f = lib.kda_chunk_fwd_c128
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    f.restype = ctypes.c_int
    f.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, ctypes.c_int, ctypes.c_int, vp, vp, vp,
                  ctypes.c_size_t, vp, vp]
    s = lib.kda_chunk_fwd_c128_workspace_size
    s.restype = ctypes.c_size_t
    s.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_int, ctypes.c_int]
    return f, s


def test_chunk128_workspace_and_support(lib):
    f, size = _c128(lib)
    s64 = _sizes(lib)
    for dk in (64, 128):
        for dv in (64, 128):
            assert size(32768, 1, 32, dk, dv, 0, 0) > 0          # bf16: every head size
            assert size(32768, 1, 32, dk, dv, 0, 1) > 0
    assert size(256, 1, 2, 64, 64, 1, 0) > 0                     # fp32: d = 64 only
    assert size(256, 1, 2, 128, 128, 1, 0) == 0
    assert size(256, 1, 2, 64, 128, 1, 0) == 0
    assert size(256, 1, 2, 96, 64, 0, 0) == 0
    assert size(256, 0, 2, 64, 64, 0, 0) == 0
    # a 128-token chunk keeps a 128 x 128 block of P per chunk: more
    # workspace than 64-token chunks at the same size
    assert size(32768, 1, 32, 128, 128, 0, 0) > s64(32768, 1, 32, 128, 128, 0, 0)
    P = FAKE
    args = dict(q=P, k=P, v=P, g=P, beta=P, S0=None, cu=None, N=1, T=256, H=2, dk=64, dv=64, dt=1, gk=0,
                o=P, S_T=None, ws=P, wsb=1 << 40, stream=None, ev=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["cu"], a["N"], a["T"], a["H"], a["dk"],
                 a["dv"], a["dt"], a["gk"], a["o"], a["S_T"], a["ws"], a["wsb"], a["stream"], a["ev"])

    assert call(dk=128, dv=128) == UNSUPPORTED    # fp32 at d = 128
    assert call(dk=96, dt=0) == UNSUPPORTED
    assert call(N=0) == INVALID
    assert call(N=3) == INVALID                   # 256 % 3 != 0 without cu_seqlens
    assert call(q=None) == INVALID
    assert call(ws=None) == WORKSPACE
    assert call(wsb=16) == WORKSPACE
    # 1024 threads per (chunk, head) workgroup: ceil(T / 128) + N chunks
    # times H must stay below 2^22
    assert call(T=128 * (2**22 - 2), H=1, ws=None, dt=0) == WORKSPACE
    assert call(T=128 * (2**22 - 1), H=1, ws=None, dt=0) == UNSUPPORTED


def test_recurrent_step_rejects_bad_arguments(lib):
    f = lib.kda_recurrent_step
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    f.restype = ctypes.c_int
    f.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, vp, vp]
    P = FAKE
    assert f(P, P, P, P, P, P, 4, 2, 64, 48, 0, 0, P, None) == UNSUPPORTED
    assert f(P, P, P, P, P, None, 4, 2, 64, 64, 0, 0, P, None) == INVALID
    assert f(P, P, P, P, P, P, -1, 2, 64, 64, 0, 0, P, None) == INVALID
    assert f(P, P, P, P, P, P + 4, 4, 2, 64, 64, 0, 0, P, None) == INVALID   # S needs 16 bytes
    assert f(P, P, P, P, P + 1, P, 4, 2, 64, 64, 0, 0, P, None) == INVALID
    assert f(None, None, None, None, None, None, 0, 2, 64, 64, 0, 0, None, None) == OK   # nothing to do


def test_chunk_bwd_rejects_bad_arguments(lib):
    f = lib.kda_chunk_bwd
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    f.restype = ctypes.c_int
    f.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, ctypes.c_int, ctypes.c_int, vp, vp,
                  vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    sz = lib.kda_chunk_bwd_workspace_size
    sz.restype = ctypes.c_size_t
    sz.argtypes = [i64, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int]
    P = FAKE
    names = ["q", "k", "v", "g", "beta", "S0", "cu", "N", "T", "H", "dk", "dv", "dt", "gk", "dO", "dST",
             "dq", "dkk", "dvv", "dg", "db", "dS0", "ws", "wsb", "stream"]
    args = dict(q=P, k=P, v=P, g=P, beta=P, S0=None, cu=None, N=1, T=128, H=2, dk=64, dv=64, dt=0, gk=0,
                dO=P, dST=None, dq=P, dkk=P, dvv=P, dg=P, db=P, dS0=None, ws=P, wsb=1 << 40, stream=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(*[a[n] for n in names])

    assert call(dk=96) == UNSUPPORTED
    assert call(dt=5) == UNSUPPORTED
    assert call(H=0) == INVALID
    assert call(N=3) == INVALID
    assert call(dO=None) == INVALID
    assert call(dg=None) == INVALID
    assert call(db=P + 1) == INVALID
    assert call(dS0=P + 2) == INVALID
    assert call(ws=P + 16) == WORKSPACE
    assert call(wsb=1024) == WORKSPACE
    assert sz(128, 1, 2, 64, 64, 0, 0) > 0
    assert sz(128, 1, 2, 64, 80, 0, 0) == 0
    assert sz(256, 1, 2, 64, 64, 0, 0) > sz(128, 1, 2, 64, 64, 0, 0)
    # bf16 inputs keep the operands of the sequential passes in bf16:
    # less workspace than fp32 inputs, and a bf16-sized workspace is too small
    # for an fp32 call of one head
    bf, f32 = sz(4096, 1, 1, 128, 128, 0, 0), sz(4096, 1, 1, 128, 128, 1, 0)
    assert 0 < bf < f32
    assert call(T=4096, H=1, dk=128, dv=128, dt=1, wsb=bf) == WORKSPACE


def test_prepare_inputs_rejects_bad_arguments(lib):
    f = lib.kda_prepare_inputs
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    f.restype = ctypes.c_int
    f.argtypes = [vp, vp, vp, vp, i64, i32, i32, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp]
    P = FAKE
    assert f(P, P, P, P, 16, 2, 96, 0, 0, P, P, P, P, None) == UNSUPPORTED
    assert f(P, P, P, P, 16, 2, 64, 4, 0, P, P, P, P, None) == UNSUPPORTED
    assert f(P, P, P, P, 16, 0, 64, 0, 0, P, P, P, P, None) == INVALID
    assert f(P, P, P, P, -1, 2, 64, 0, 0, P, P, P, P, None) == INVALID
    assert f(None, P, P, P, 16, 2, 64, 0, 0, P, P, P, P, None) == INVALID
    assert f(P, P, P, P, 16, 2, 64, 1, 0, P, P, P + 2, P, None) == INVALID   # fp32 needs 4-byte alignment
    assert f(None, None, None, None, 0, 2, 64, 0, 0, None, None, None, None, None) == OK   # nothing to do


def test_recurrent_step_raw_rejects_bad_arguments(lib):
    f = lib.kda_recurrent_step_raw
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    f.restype = ctypes.c_int
    f.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, vp, vp]
    P = FAKE
    assert f(P, P, P, P, P, P, 4, 2, 64, 48, 0, 0, P, None) == UNSUPPORTED
    assert f(P, P, P, P, P, P + 4, 4, 2, 64, 64, 0, 0, P, None) == INVALID


def test_chunk_fwd_noalloc_rejects_before_any_device_call(lib):
    """Unsupported sizes, bad counts and problems beyond the static scratch
    are refused on the host, before the scratch is looked up or anything is
    launched (so this runs without a GPU)."""
    f = lib.kda_chunk_fwd_noalloc
    f.restype = ctypes.c_int
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    f.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, ctypes.c_int, ctypes.c_int, vp, vp, vp]
    P = 1 << 20
    assert f(P, P, P, P, P, None, None, 1, 128, 2, 48, 64, 0, 0, P, None, None) == UNSUPPORTED
    assert f(P, P, P, P, P, None, None, 1, 128, 0, 64, 64, 0, 0, P, None, None) == INVALID
    assert f(P, P, P, P, P, None, None, 0, 128, 2, 64, 64, 0, 0, P, None, None) == INVALID
    assert f(P, P, P, P, P, None, None, 1, -1, 2, 64, 64, 0, 0, P, None, None) == INVALID
    # 8192 tokens x 32 heads at d = 128 need ~580 MB of workspace: beyond the 128 MiB scratch
    assert f(P, P, P, P, P, None, None, 1, 8192, 32, 128, 128, 0, 0, P, None, None) == 7


def test_status_strings(lib):
    f = lib.kda_status_string
    f.restype = ctypes.c_char_p
    f.argtypes = [ctypes.c_int]
    for code in range(8):
        assert f(code).startswith(b"KDA_")
    assert f(99) == b"KDA_ERR_UNKNOWN"

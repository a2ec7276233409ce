"""MI355X-native Kimi Delta Attention (KDA) hot path.

Thin Python binding over the C ABI of ``libkda.so`` (declared in
``include/kda.h``).  It only marshals arguments: every step of the path runs
in the library's HIP kernels.  PyTorch provides device memory and streams.

    chunk_fwd(q, k, v, g, beta, S0=..., cu_seqlens=...) -> (o, S_T)
    chunk_fwd_noalloc(q, k, v, g, beta, out=o, S_T=..., ...) -> (o, S_T)
        (the same, with the library's static scratch instead of a workspace)
    recurrent_step(q, k, v, g, beta, S) -> o            (S updated in place)
    chunk_bwd(q, k, v, g, beta, dO, S0=..., dS_T=..., cu_seqlens=...)
        -> (dq, dk, dv, dg, dbeta, dS0)                  (gradients of the forward)
    prepare_inputs(q_raw, k_raw, g_raw, beta_raw) -> (q, k, g, beta)
    recurrent_step_raw(q_raw, k_raw, v, g_raw, beta_raw, S) -> o

The library must have been built (``__graft_entry__.build()`` or
``python gated_delta_rule_48_amd/build.py``); importing the functions'
backing library fails loudly otherwise.  There is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["chunk_fwd", "chunk_fwd_workspace_size", "chunk_fwd_check", "chunk_fwd_noalloc", "recurrent_step",
           "chunk_bwd", "chunk_bwd_workspace_size", "prepare_inputs", "recurrent_step_raw",
           "KDAError", "LIB_PATH", "load_library", "STATUS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARG", 2: "KDA_ERR_UNSUPPORTED", 3: "KDA_ERR_WORKSPACE",
          4: "KDA_ERR_HIP", 5: "KDA_ERR_BAD_SEQLENS", 6: "KDA_ERR_TIMEOUT", 7: "KDA_ERR_TOO_LARGE"}
_BF16, _F32 = 0, 1
_PER_CHANNEL, _PER_HEAD = 0, 1

_lib = None


class KDAError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


def load_library():
    """Load libkda.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lib.kda_status_string.restype = ctypes.c_char_p
        lib.kda_status_string.argtypes = [ctypes.c_int]
        lib.kda_version.restype = i32
        lib.kda_chunk_fwd_workspace_size.restype = sz
        lib.kda_chunk_fwd_workspace_size.argtypes = [i64, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int]
        lib.kda_chunk_fwd.restype = ctypes.c_int
        lib.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, ctypes.c_int,
                                      ctypes.c_int, vp, vp, vp, sz, vp]
        lib.kda_chunk_fwd_instrumented.restype = ctypes.c_int
        lib.kda_chunk_fwd_instrumented.argtypes = lib.kda_chunk_fwd.argtypes + [vp]
        lib.kda_chunk_fwd_raw.restype = ctypes.c_int
        lib.kda_chunk_fwd_raw.argtypes = lib.kda_chunk_fwd.argtypes
        lib.kda_chunk_fwd_c128_workspace_size.restype = sz
        lib.kda_chunk_fwd_c128_workspace_size.argtypes = lib.kda_chunk_fwd_workspace_size.argtypes
        lib.kda_chunk_fwd_c128.restype = ctypes.c_int
        lib.kda_chunk_fwd_c128.argtypes = lib.kda_chunk_fwd.argtypes + [vp]
        lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
        lib.kda_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, ctypes.c_int,
                                              ctypes.c_int, vp, vp, vp]
        lib.kda_chunk_fwd_check.restype = ctypes.c_int
        lib.kda_chunk_fwd_check.argtypes = [vp, vp]
        lib.kda_chunk_bwd_workspace_size.restype = sz
        lib.kda_chunk_bwd_workspace_size.argtypes = lib.kda_chunk_fwd_workspace_size.argtypes
        lib.kda_chunk_bwd.restype = ctypes.c_int
        lib.kda_chunk_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, ctypes.c_int,
                                      ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.kda_prepare_inputs.restype = ctypes.c_int
        lib.kda_prepare_inputs.argtypes = [vp, vp, vp, vp, i64, i32, i32, ctypes.c_int, ctypes.c_int,
                                           vp, vp, vp, vp, vp]
        lib.kda_recurrent_step_raw.restype = ctypes.c_int
        lib.kda_recurrent_step_raw.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_int,
                                               ctypes.c_int, vp, vp]
        lib.kda_recurrent_step.restype = ctypes.c_int
        lib.kda_recurrent_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_int,
                                           ctypes.c_int, vp, vp]
        _lib = lib
    return _lib


def _check(code):
    if code != 0:
        raise KDAError(code, load_library().kda_status_string(code).decode())


def _dt(t):
    if t.dtype == torch.bfloat16:
        return _BF16
    if t.dtype == torch.float32:
        return _F32
    raise TypeError(f"unsupported dtype {t.dtype}: bfloat16 or float32")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev_contig(name, t, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _shapes(**named):
    for name, (t, shape) in named.items():
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def chunk_fwd_workspace_size(T_total, N, H, d_k, d_v, dtype=torch.bfloat16, per_head_gate=False, chunk=64):
    """Bytes of workspace ``chunk_fwd`` needs (0 for unsupported sizes)."""
    dt = _BF16 if dtype == torch.bfloat16 else _F32
    lib = load_library()
    fn = lib.kda_chunk_fwd_c128_workspace_size if _chunk_size(chunk) == 128 else lib.kda_chunk_fwd_workspace_size
    return int(fn(int(T_total), int(N), int(H), int(d_k), int(d_v), dt, _PER_HEAD if per_head_gate else _PER_CHANNEL))


def _chunk_size(chunk):
    if chunk not in (64, 128):
        raise ValueError(f"chunk must be 64 or 128, got {chunk}")
    return chunk


def chunk_fwd(q, k, v, g, beta, *, S0=None, cu_seqlens=None, N=None, per_head_gate=False,
              out=None, S_T=None, workspace=None, stream=None, output_final_state=True, events=None,
              raw=False, check=True, chunk=64):
    """Chunked KDA forward (prefill).

    q, k: [T, H, dk] packed (with ``cu_seqlens`` int32 [N+1] on the device, or
    ``N`` equal sequences), or [B, T, H, dk] (B equal sequences).  v: [.., dv];
    g: [.., dk] per-channel log-gate, or [T, H] / [B, T, H] with
    ``per_head_gate``; beta: [T, H] / [B, T, H].  q, k, v, g, beta share one
    dtype (bfloat16 or float32).  S0: fp32 [N, H, dk, dv] or None.
    Returns (o with q's dtype and v's leading shape, S_T fp32 [N, H, dk, dv]
    or None).  ``events``: optional sequence of four raw hipEvent_t handles
    (ints) recorded before the chunk-map, intra-chunk and walk kernels and
    after the walk kernel (kda_chunk_fwd_instrumented).  ``raw``: q, k, g,
    beta are raw projections and the pre-path transforms run inside the
    intra-chunk kernel (kda_chunk_fwd_raw; no ``events``).  ``check``: wait
    for the stream and raise KDAError if the device rejected the sequence
    offsets or a bounded wait gave up (kda_chunk_fwd_check); pass False to
    keep the call asynchronous and check the workspace later.  ``chunk``:
    tokens per chunk, 64 (kda_chunk_fwd) or 128 (kda_chunk_fwd_c128; not
    with ``raw``).
    """
    if raw and events is not None:
        raise ValueError("events are not recorded for raw inputs")
    if _chunk_size(chunk) == 128 and raw:
        raise ValueError("raw inputs are taken with 64-token chunks only")
    batched = q.dim() == 4
    if batched:
        B, T = q.shape[0], q.shape[1]
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens requires packed [T, H, d] inputs")
        N = B
        q, k, v = q.reshape(B * T, *q.shape[2:]), k.reshape(B * T, *k.shape[2:]), v.reshape(B * T, *v.shape[2:])
        g = g.reshape(B * T, *g.shape[2:])
        beta = beta.reshape(B * T, *beta.shape[2:])
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [T, H, d] (or [B, T, H, d])")
    T_total, H, dk = q.shape
    dv = v.shape[2]
    _shapes(k=(k, (T_total, H, dk)), v=(v, (T_total, H, dv)), beta=(beta, (T_total, H)),
            g=(g, (T_total, H) if per_head_gate else (T_total, H, dk)))
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        _dev_contig(name, t, q.dtype)
    if cu_seqlens is not None:
        _dev_contig("cu_seqlens", cu_seqlens, torch.int32)
        N = cu_seqlens.numel() - 1
    elif N is None:
        N = 1
    dt = _dt(q)
    gk = _PER_HEAD if per_head_gate else _PER_CHANNEL
    if S0 is not None:
        _dev_contig("S0", S0, torch.float32)
        if tuple(S0.shape) != (N, H, dk, dv):
            raise ValueError(f"S0 must be [{N}, {H}, {dk}, {dv}]")
    o = out if out is not None else torch.empty((T_total, H, dv), dtype=q.dtype, device=q.device)
    _dev_contig("out", o, q.dtype)
    _shapes(out=(o, (T_total, H, dv)))
    if output_final_state and S_T is None:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    if S_T is not None:
        _dev_contig("S_T", S_T, torch.float32)
        _shapes(S_T=(S_T, (N, H, dk, dv)))
    lib = load_library()
    size_fn = lib.kda_chunk_fwd_c128_workspace_size if chunk == 128 else lib.kda_chunk_fwd_workspace_size
    need = int(size_fn(T_total, N, H, dk, dv, dt, gk))
    if need == 0:
        raise KDAError(2, f"unsupported sizes T={T_total} N={N} H={H} dk={dk} dv={dv}")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _dev_contig("workspace", workspace)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(cu_seqlens),
            N, T_total, H, dk, dv, dt, gk, _ptr(o), _ptr(S_T), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    if chunk == 128:
        arr = None
        if events is not None:
            if len(events) != 4:
                raise ValueError("events must hold four hipEvent_t handles")
            arr = (ctypes.c_void_p * 4)(*[int(e) for e in events])
        _check(lib.kda_chunk_fwd_c128(*args, arr))
    elif events is None:
        _check((lib.kda_chunk_fwd_raw if raw else lib.kda_chunk_fwd)(*args))
    else:
        if len(events) != 4:
            raise ValueError("events must hold four hipEvent_t handles")
        arr = (ctypes.c_void_p * 4)(*[int(e) for e in events])
        _check(lib.kda_chunk_fwd_instrumented(*args, arr))
    if check:
        chunk_fwd_check(workspace, stream=stream)
    if batched:
        o = o.reshape(N, T_total // N, H, dv)
    return o, S_T


def chunk_fwd_raw(q_raw, k_raw, v, g_raw, beta_raw, **kw):
    """``chunk_fwd`` from raw projections (kda_chunk_fwd_raw): q_raw, k_raw
    are scaled to unit L2 norm over dk, g_raw goes through -softplus and
    beta_raw through the logistic function inside the intra-chunk kernel,
    each result rounded once to the input dtype.  Keyword arguments as for
    ``chunk_fwd``."""
    return chunk_fwd(q_raw, k_raw, v, g_raw, beta_raw, raw=True, **kw)


def chunk_fwd_noalloc(q, k, v, g, beta, *, out, S_T=None, S0=None, cu_seqlens=None, N=None,
                      per_head_gate=False, stream=None):
    """``chunk_fwd`` through kda_chunk_fwd_noalloc: no workspace, the library's
    static scratch instead (at most KDA_NOALLOC_SCRATCH_BYTES of workspace,
    else KDAError KDA_ERR_TOO_LARGE).  Packed [T, H, d] inputs only; the
    caller passes the outputs (``out`` [T, H, dv]; ``S_T`` fp32 [N, H, dk, dv]
    or None), and nothing is allocated here either.  Calls that overlap on one
    GPU race on the shared scratch.  Returns (out, S_T)."""
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be packed [T, H, d]")
    T_total, H, dk = q.shape
    dv = v.shape[2]
    _shapes(k=(k, (T_total, H, dk)), v=(v, (T_total, H, dv)), beta=(beta, (T_total, H)),
            g=(g, (T_total, H) if per_head_gate else (T_total, H, dk)), out=(out, (T_total, H, dv)))
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("out", out)):
        _dev_contig(name, t, q.dtype)
    if cu_seqlens is not None:
        _dev_contig("cu_seqlens", cu_seqlens, torch.int32)
        N = cu_seqlens.numel() - 1
    elif N is None:
        N = 1
    for name, t in (("S0", S0), ("S_T", S_T)):
        if t is not None:
            _dev_contig(name, t, torch.float32)
            _shapes(**{name: (t, (N, H, dk, dv))})
    _check(load_library().kda_chunk_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(cu_seqlens), N, T_total, H, dk, dv,
        _dt(q), _PER_HEAD if per_head_gate else _PER_CHANNEL, _ptr(out), _ptr(S_T), _stream(stream)))
    return out, S_T


def chunk_fwd_check(workspace, stream=None):
    """Synchronise and raise KDAError if the last call on this workspace had its
    device cu_seqlens rejected or a bounded wait gave up."""
    _check(load_library().kda_chunk_fwd_check(_ptr(workspace), _stream(stream)))


def prepare_inputs(q_raw, k_raw, g_raw, beta_raw, *, per_head_gate=False, out=None, stream=None):
    """Pre-path transforms in one pass (kda_prepare_inputs): q, k L2-normalised
    per token and head, g = -softplus(g_raw), beta = sigmoid(beta_raw).

    q_raw, k_raw: [T, H, dk]; g_raw: [T, H, dk] (or [T, H] with
    ``per_head_gate``); beta_raw: [T, H]; one dtype (bfloat16 or float32).
    ``out``: optional (q, k, g, beta) to write into (may be the inputs
    themselves).  Returns (q, k, g, beta).
    """
    if q_raw.dim() != 3:
        raise ValueError("q_raw, k_raw must be [T, H, d]")
    T, H, dk = q_raw.shape
    _shapes(k_raw=(k_raw, (T, H, dk)), beta_raw=(beta_raw, (T, H)),
            g_raw=(g_raw, (T, H) if per_head_gate else (T, H, dk)))
    for name, t in (("q_raw", q_raw), ("k_raw", k_raw), ("g_raw", g_raw), ("beta_raw", beta_raw)):
        _dev_contig(name, t, q_raw.dtype)
    outs = out if out is not None else tuple(torch.empty_like(x) for x in (q_raw, k_raw, g_raw, beta_raw))
    for name, t, ref in zip(("q", "k", "g", "beta"), outs, (q_raw, k_raw, g_raw, beta_raw)):
        _dev_contig(name, t, q_raw.dtype)
        _shapes(**{name: (t, tuple(ref.shape))})
    _check(load_library().kda_prepare_inputs(
        _ptr(q_raw), _ptr(k_raw), _ptr(g_raw), _ptr(beta_raw), T, H, dk, _dt(q_raw),
        _PER_HEAD if per_head_gate else _PER_CHANNEL, *[_ptr(t) for t in outs], _stream(stream)))
    return tuple(outs)


def recurrent_step_raw(q_raw, k_raw, v, g_raw, beta_raw, S, *, per_head_gate=False, out=None, stream=None):
    """One decode step from raw projections (kda_recurrent_step_raw): the
    pre-path transforms of ``prepare_inputs`` are applied inside the step.
    Shapes as for ``recurrent_step``; S updated in place; returns o."""
    return recurrent_step(q_raw, k_raw, v, g_raw, beta_raw, S, per_head_gate=per_head_gate, out=out,
                          stream=stream, _raw=True)


def recurrent_step(q, k, v, g, beta, S, *, per_head_gate=False, out=None, stream=None, _raw=False):
    """One decode step, in place on S (fp32 [N, H, dk, dv]).

    q, k: [N, H, dk]; v: [N, H, dv]; g: [N, H, dk] (or [N, H] with
    ``per_head_gate``); beta: [N, H].  Returns o [N, H, dv] (q's dtype).
    """
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [N, H, d]")
    N, H, dk = q.shape
    dv = v.shape[2]
    _shapes(k=(k, (N, H, dk)), v=(v, (N, H, dv)), beta=(beta, (N, H)),
            g=(g, (N, H) if per_head_gate else (N, H, dk)))
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        _dev_contig(name, t, q.dtype)
    _dev_contig("S", S, torch.float32)
    if tuple(S.shape) != (N, H, dk, dv):
        raise ValueError(f"S must be [{N}, {H}, {dk}, {dv}]")
    o = out if out is not None else torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    _dev_contig("out", o, q.dtype)
    _shapes(out=(o, (N, H, dv)))
    lib = load_library()
    fn = lib.kda_recurrent_step_raw if _raw else lib.kda_recurrent_step
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S), N, H, dk, dv, _dt(q),
              _PER_HEAD if per_head_gate else _PER_CHANNEL, _ptr(o), _stream(stream)))
    return o


def chunk_bwd_workspace_size(T_total, N, H, d_k, d_v, dtype=torch.bfloat16, per_head_gate=False):
    """Bytes of workspace ``chunk_bwd`` needs (0 for unsupported sizes)."""
    dt = _BF16 if dtype == torch.bfloat16 else _F32
    return int(load_library().kda_chunk_bwd_workspace_size(
        int(T_total), int(N), int(H), int(d_k), int(d_v), dt, _PER_HEAD if per_head_gate else _PER_CHANNEL))


def chunk_bwd(q, k, v, g, beta, dO, *, S0=None, dS_T=None, cu_seqlens=None, N=None, per_head_gate=False,
              need_dS0=True, workspace=None, stream=None):
    """Gradients of ``chunk_fwd`` (kda_chunk_bwd).

    Takes the forward's inputs (packed [T, H, d] layout, as for ``chunk_fwd``)
    and the cotangents dO ([T, H, dv], q's dtype) and dS_T (fp32
    [N, H, dk, dv] or None = zeros).  Returns (dq, dk, dv, dg, dbeta, dS0):
    the first five with the shapes and dtype of q, k, v, g, beta; dS0 fp32
    [N, H, dk, dv] (None when ``need_dS0`` is False).  ``workspace`` may be
    smaller than ``chunk_bwd_workspace_size`` for all heads (at least the size
    for one head): the heads are then processed in groups that fit.
    """
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [T, H, d]")
    T_total, H, dk = q.shape
    dv = v.shape[2]
    _shapes(k=(k, (T_total, H, dk)), v=(v, (T_total, H, dv)), beta=(beta, (T_total, H)),
            g=(g, (T_total, H) if per_head_gate else (T_total, H, dk)), dO=(dO, (T_total, H, dv)))
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("dO", dO)):
        _dev_contig(name, t, q.dtype)
    if cu_seqlens is not None:
        _dev_contig("cu_seqlens", cu_seqlens, torch.int32)
        N = cu_seqlens.numel() - 1
    elif N is None:
        N = 1
    for name, t in (("S0", S0), ("dS_T", dS_T)):
        if t is not None:
            _dev_contig(name, t, torch.float32)
            _shapes(**{name: (t, (N, H, dk, dv))})
    dt = _dt(q)
    gk = _PER_HEAD if per_head_gate else _PER_CHANNEL
    dq, dk_, dv_, dg, db = (torch.empty_like(x) for x in (q, k, v, g, beta))
    dS0 = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device) if need_dS0 else None
    lib = load_library()
    need = int(lib.kda_chunk_bwd_workspace_size(T_total, N, H, dk, dv, dt, gk))
    if need == 0:
        raise KDAError(2, f"unsupported sizes T={T_total} N={N} H={H} dk={dk} dv={dv}")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _dev_contig("workspace", workspace)
    _check(lib.kda_chunk_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(cu_seqlens), N, T_total, H, dk, dv,
        dt, gk, _ptr(dO), _ptr(dS_T), _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dg), _ptr(db), _ptr(dS0),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return dq, dk_, dv_, dg, db, dS0

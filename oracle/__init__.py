"""fp64 CPU oracle for the Kimi Delta Attention (KDA) recurrence.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` import this package.  It shares no code
with the HIP library and never imports it.

Three independent formulations of the same map (q, k, v, g, beta, S0) -> (o, S_T):

``recurrence``   the sequential token-by-token update, in C (``kda_oracle.c``),
                 fp64, OpenMP over (sequence, head).  This is the oracle the
                 GPU path is compared against.
``chunked``      the chunkwise-parallel algebra in numpy fp64: chunks of C
                 tokens, all deltas of a chunk obtained at once by solving the
                 unit-lower-triangular system (I + A) U = ..., then one state
                 hand-off per chunk ("From GPT-2 to Kimi K3", section on the
                 parallelisation trick: masked attention inside a chunk,
                 state and one matmul between chunks, Householder-style
                 reparametrisation of the deltas).
``dense_dplr``   the explicit transition matrix M_t = Diag(a) - beta k (a*k)^T,
                 a diagonal-plus-rank-one matrix whose low-rank factors are
                 both the key ("Kimi Linear architecture", section on KDA;
                 "Kimi Delta Attention ... 1M context", paragraph on the
                 specialised DPLR transition), then S <- M S + beta k v^T.

Every function is pinned in ``tests/test_oracle_pins.py`` against closed forms,
invariants, exact rational arithmetic and hand-worked fixtures.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

BF16, F32, F64 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O3, no fast-math: IEEE fp64 throughout) into oracle/."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.kda_oracle_recurrence.restype = ctypes.c_int
        vp = ctypes.c_void_p
        lib.kda_oracle_recurrence.argtypes = [
            vp, vp, vp, vp, vp, ctypes.c_int, vp, vp,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int, vp, vp, vp, ctypes.c_int]
        _lib = lib
    return _lib


def _dtype_code(*arrays):
    kinds = {a.dtype for a in arrays}
    if len(kinds) != 1:
        raise TypeError(f"q, k, v, g, beta must share one dtype, got {kinds}")
    dt = kinds.pop()
    if dt == np.uint16:
        return BF16
    if dt == np.float32:
        return F32
    if dt == np.float64:
        return F64
    raise TypeError(f"unsupported input dtype {dt} (uint16 bf16 bits, float32, float64)")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def recurrence(q, k, v, g, beta, *, S0=None, cu_seqlens=None,
               per_head_gate=False, o_positions=None, threads=0):
    """Sequential fp64 KDA recurrence (C, OpenMP).

    q, k: [T, H, dk]; v: [T, H, dv]; g: [T, H, dk] (or [T, H] with
    ``per_head_gate``); beta: [T, H].  All five share one dtype: uint16 (bf16
    bit patterns), float32 or float64; values are widened exactly to fp64.
    S0: [N, H, dk, dv] (any float dtype, converted to fp64) or None (zeros).
    cu_seqlens: N+1 offsets into T (default: one sequence).
    o_positions: optional sorted token indices; o then holds only those rows.

    Returns (o fp64 [T or len(o_positions), H, dv], S_T fp64 [N, H, dk, dv]).
    """
    lib = _load()
    arrs = [np.ascontiguousarray(x) for x in (q, k, v, g, beta)]
    q, k, v, g, beta = arrs
    code = _dtype_code(*arrs)
    T, H, dk = q.shape
    dv = v.shape[2]
    if k.shape != (T, H, dk) or v.shape[:2] != (T, H) or beta.shape != (T, H):
        raise ValueError("shape mismatch")
    if per_head_gate:
        if g.shape != (T, H):
            raise ValueError("per-head gate must be [T, H]")
    elif g.shape != (T, H, dk):
        raise ValueError("per-channel gate must be [T, H, dk]")
    cu = np.array([0, T] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("bad cu_seqlens")
    s0 = None if S0 is None else np.ascontiguousarray(S0, dtype=np.float64)
    if s0 is not None and s0.shape != (N, H, dk, dv):
        raise ValueError("S0 shape")
    slot = None
    if o_positions is None:
        o = np.zeros((T, H, dv), dtype=np.float64)
    else:
        pos = np.asarray(o_positions, dtype=np.int64)
        slot = np.full(T, -1, dtype=np.int64)
        slot[pos] = np.arange(len(pos), dtype=np.int64)
        o = np.zeros((len(pos), H, dv), dtype=np.float64)
    S_T = np.zeros((N, H, dk, dv), dtype=np.float64)
    rc = lib.kda_oracle_recurrence(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), code, _ptr(s0),
        _ptr(cu), N, H, dk, dv, int(bool(per_head_gate)), _ptr(o), _ptr(slot),
        _ptr(S_T), int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    return o, S_T


def widen(x):
    """bf16 bit patterns (uint16) / float32 / float64 -> float64, exactly."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def _split(T, cu_seqlens):
    cu = [0, T] if cu_seqlens is None else [int(c) for c in cu_seqlens]
    return cu


def _gate_full(g, H, dk, per_head_gate):
    g = widen(g)
    if per_head_gate:
        return np.repeat(g[:, :, None], dk, axis=2)
    return g


def chunked(q, k, v, g, beta, *, chunk=64, S0=None, cu_seqlens=None,
            per_head_gate=False):
    """Chunkwise-parallel form of the same recurrence, numpy fp64, naive.

    For a chunk with start state S and local tokens t = 1..n:
      b_t   = sum of g over the chunk up to and including t (per channel)
      A_ti  = beta_t * sum_c k_tc k_ic exp(b_tc - b_ic)          (i < t)
      (I + A) U' = diag(beta) V,   (I + A) W = diag(beta) (K * exp(b))
      U     = U' - W S                       (the true deltas u_t)
      O     = (Q * exp(b)) S + M U,  M_ti = sum_c q_tc k_ic exp(b_tc - b_ic) (i <= t)
      S    <- Diag(exp(b_n)) S + (K * exp(b_n - b))^T U
    The triangular system is handed to numpy.linalg.solve; nothing is fused.
    """
    q, k, v, beta = widen(q), widen(k), widen(v), widen(beta)
    T, H, dk = q.shape
    dv = v.shape[2]
    gf = _gate_full(g, H, dk, per_head_gate)
    cu = _split(T, cu_seqlens)
    N = len(cu) - 1
    o = np.zeros((T, H, dv))
    S_T = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[n, h], dtype=np.float64)
            for s in range(cu[n], cu[n + 1], chunk):
                e = min(s + chunk, cu[n + 1])
                Q, K, V = q[s:e, h], k[s:e, h], v[s:e, h]
                B = beta[s:e, h]
                b = np.cumsum(gf[s:e, h], axis=0)             # [n, dk]
                D = np.exp(b[:, None, :] - b[None, :, :])       # [t, i, c] = exp(b_tc - b_ic)
                KK = np.einsum("tc,ic,tic->ti", K, K, D)
                QK = np.einsum("tc,ic,tic->ti", Q, K, D)
                nt = e - s
                A = np.tril(B[:, None] * KK, -1)
                M = np.tril(QK, 0)
                IA = np.eye(nt) + A
                Up = np.linalg.solve(IA, B[:, None] * V)
                W = np.linalg.solve(IA, B[:, None] * (K * np.exp(b)))
                U = Up - W @ S
                o[s:e, h] = (Q * np.exp(b)) @ S + M @ U
                S = np.exp(b[-1])[:, None] * S + (K * np.exp(b[-1][None, :] - b)).T @ U
            S_T[n, h] = S
    return o, S_T


def dense_dplr(q, k, v, g, beta, *, S0=None, cu_seqlens=None, per_head_gate=False):
    """Explicit diagonal-plus-low-rank transition, numpy fp64.

    M_t = Diag(a_t) - beta_t k_t (a_t * k_t)^T  (d_k x d_k), a_t = exp(g_t);
    S_t = M_t S_{t-1} + beta_t k_t v_t^T;  o_t = S_t^T q_t.
    """
    q, k, v, beta = widen(q), widen(k), widen(v), widen(beta)
    T, H, dk = q.shape
    dv = v.shape[2]
    gf = _gate_full(g, H, dk, per_head_gate)
    cu = _split(T, cu_seqlens)
    N = len(cu) - 1
    o = np.zeros((T, H, dv))
    S_T = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[n, h], dtype=np.float64)
            for t in range(cu[n], cu[n + 1]):
                a = np.exp(gf[t, h])
                kt = k[t, h]
                Mt = np.diag(a) - beta[t, h] * np.outer(kt, a * kt)
                S = Mt @ S + beta[t, h] * np.outer(kt, v[t, h])
                o[t, h] = S.T @ q[t, h]
            S_T[n, h] = S
    return o, S_T


def rel_err(got, ref):
    """max |got - ref| / max |ref| over the whole tensor (the parity metric).

    The largest absolute deviation anywhere in the tensor, divided by the
    largest magnitude of the reference (not of ``got``, and not a mean), so a
    single wrong element is enough to fail a bound.  ``got`` and ``ref`` must
    have the same shape (no broadcasting).  Any NaN or infinity in ``got`` or
    ``ref`` gives +inf.  Two empty tensors give 0; an all-zero reference gives
    the plain max |got - ref|.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise ValueError(f"rel_err: shapes differ, got {got.shape} vs ref {ref.shape}")
    if got.size == 0:
        return 0.0
    if not (np.all(np.isfinite(got)) and np.all(np.isfinite(ref))):
        return float("inf")
    num = float(np.max(np.abs(got - ref)))
    den = float(np.max(np.abs(ref)))
    if den == 0.0:
        return num
    return num / den

"""fp64 CPU oracle for the gradients of the KDA recurrence.

TEST INFRASTRUCTURE ONLY.  Only ``tests/`` and ``bench.py``'s ``cpu_baseline``
leg import this module.  It shares no code with the HIP library.

``recurrence_grad`` differentiates the plain sequential recurrence (the same
six steps as ``kda_oracle.c``: exp of the gate, decay, read, scaled delta,
write, read-out) with PyTorch's reverse-mode autograd, in float64 on the CPU.
The scalar being differentiated is

    L = sum_t <dO_t, o_t> + sum_{n,h} <dS_T[n,h], S_T[n,h]>,

so the returned tensors are the vector-Jacobian products of the map
(q, k, v, g, beta, S0) -> (o, S_T) with the cotangents (dO, dS_T).  This is
what a chunked backward pass must produce ("From GPT-2 to Kimi K3", section
on the parallelisation trick: the chunked form is what makes training
parallel; "Kimi Linear architecture", section on linear attention: the
chunkwise form serves training and prefill).

``adjoint`` is the same vector-Jacobian product written out by hand in C
(``kda_oracle_adjoint`` in ``kda_oracle.c``): reverse-mode through the six
steps token by token, the state recomputed from checkpoints, fp64, OpenMP over
(sequence, head).  It needs no tape, so it runs at the full benchmark lengths
(32K and 1M tokens), where autograd does not fit.

The autograd tape and the hand-written adjoint are independent routes to the
derivative; the tests pin both against a hand-derived one-token closed form
and against central finite differences of the C forward oracle, the adjoint
also against exact identities of the loss (L is linear in q and jointly
linear in (v, S0)) at long lengths, and the two against each other.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _dtype_code, _load, _ptr, widen


def _torch():
    import torch
    return torch


def recurrence_grad(q, k, v, g, beta, dO, *, S0=None, dS_T=None, cu_seqlens=None,
                    per_head_gate=False):
    """Gradients of L (module docstring) w.r.t. q, k, v, g, beta and S0.

    Shapes as for ``oracle.recurrence``: q, k, g [T, H, dk] (g [T, H] with
    ``per_head_gate``), v and dO [T, H, dv], beta [T, H], S0 and dS_T
    [N, H, dk, dv] or None (zeros).  Inputs may be bf16 bit patterns
    (uint16), float32 or float64 and are widened exactly.

    Returns float64 numpy arrays (dq, dk, dv, dg, dbeta, dS0) with the shapes
    of (q, k, v, g, beta, S0 as [N, H, dk, dv]).
    """
    torch = _torch()
    f64 = torch.float64
    qd, kd, vd, gd, bd = (torch.from_numpy(widen(x)) for x in (q, k, v, g, beta))
    T, H, dk = qd.shape
    dv = vd.shape[2]
    cu = [0, T] if cu_seqlens is None else [int(c) for c in cu_seqlens]
    N = len(cu) - 1
    s0 = torch.zeros((N, H, dk, dv), dtype=f64) if S0 is None else torch.from_numpy(
        np.array(S0, dtype=np.float64))
    dOt = torch.from_numpy(widen(dO))
    dST = torch.zeros((N, H, dk, dv), dtype=f64) if dS_T is None else torch.from_numpy(
        np.array(dS_T, dtype=np.float64))
    leaves = [x.clone().requires_grad_(True) for x in (qd, kd, vd, gd, bd, s0)]
    ql, kl, vl, gl, bl, s0l = leaves
    loss = torch.zeros((), dtype=f64)
    for n in range(N):
        S = s0l[n]                                    # [H, dk, dv]
        for t in range(cu[n], cu[n + 1]):
            gt = gl[t][:, None].expand(H, dk) if per_head_gate else gl[t]
            a = torch.exp(gt)                         # [H, dk]
            S = a[:, :, None] * S                     # forget first, per channel
            r = torch.einsum("hcv,hc->hv", S, kl[t])  # read what the key retrieves
            u = bl[t][:, None] * (vl[t] - r)          # scaled delta
            S = S + kl[t][:, :, None] * u[:, None, :]  # write the delta
            o = torch.einsum("hcv,hc->hv", S, ql[t])  # read out after the write
            loss = loss + (o * dOt[t]).sum()
        loss = loss + (S * dST[n]).sum()
    loss.backward()
    return tuple(x.grad.detach().numpy().copy() for x in leaves)


def adjoint(q, k, v, g, beta, dO, *, S0=None, dS_T=None, cu_seqlens=None,
            per_head_gate=False, positions=None, threads=0):
    """The gradients of ``recurrence_grad`` from the hand-written fp64 C
    adjoint (module docstring).

    q, k, v, g, beta share one dtype (uint16 bf16 bits, float32 or float64)
    as for ``oracle.recurrence``; dO [T, H, dv] and dS_T [N, H, dk, dv] may be
    bf16 bits or any float dtype (widened exactly).  ``positions``: optional
    sorted token indices; the per-token gradients then hold only those rows
    (dS0 is always complete).

    Returns float64 (dq, dk, dv, dg, dbeta, dS0).
    """
    lib = _load()
    fn = lib.kda_oracle_adjoint
    if fn.argtypes is None:
        vp = ctypes.c_void_p
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp,
                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                       ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int]
    q, k, v, g, beta = (np.ascontiguousarray(x) for x in (q, k, v, g, beta))
    code = _dtype_code(q, k, v, g, beta)
    T, H, dk = q.shape
    dv = v.shape[2]
    if per_head_gate:
        if g.shape != (T, H):
            raise ValueError("per-head gate must be [T, H]")
    elif g.shape != (T, H, dk):
        raise ValueError("per-channel gate must be [T, H, dk]")
    cu = np.array([0, T] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("bad cu_seqlens")
    dOc = np.ascontiguousarray(dO)
    if dOc.shape != (T, H, dv):
        raise ValueError("dO shape")
    dO_code = _dtype_code(dOc)
    s0 = None if S0 is None else np.ascontiguousarray(S0, dtype=np.float64)
    dst = None if dS_T is None else np.ascontiguousarray(widen(dS_T))
    for x in (s0, dst):
        if x is not None and x.shape != (N, H, dk, dv):
            raise ValueError("state shape")
    slot = None
    rows = T
    if positions is not None:
        pos = np.asarray(positions, dtype=np.int64)
        slot = np.full(T, -1, dtype=np.int64)
        slot[pos] = np.arange(len(pos), dtype=np.int64)
        rows = len(pos)
    dq = np.zeros((rows, H, dk))
    dkk = np.zeros((rows, H, dk))
    dvv = np.zeros((rows, H, dv))
    dg = np.zeros((rows, H) if per_head_gate else (rows, H, dk))
    db = np.zeros((rows, H))
    dS0 = np.zeros((N, H, dk, dv))
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), code, _ptr(s0), _ptr(dOc), dO_code, _ptr(dst),
            _ptr(cu), N, H, dk, dv, int(bool(per_head_gate)), _ptr(slot), _ptr(dq), _ptr(dkk),
            _ptr(dvv), _ptr(dg), _ptr(db), _ptr(dS0), int(threads))
    if rc != 0:
        raise RuntimeError(f"adjoint oracle failed with code {rc}")
    return dq, dkk, dvv, dg, db, dS0

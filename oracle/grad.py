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

The autograd tape is an independent route to the derivative; the tests pin it
against a hand-derived one-token closed form and against central finite
differences of the C forward oracle.
"""
from __future__ import annotations

import numpy as np

from . import widen


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

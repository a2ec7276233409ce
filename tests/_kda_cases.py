"""Shared helpers for the GPU parity tests: numpy <-> torch marshalling of
the seeded inputs and the tolerance rule.  Holds none of the method's
arithmetic."""
import numpy as np
import torch

import synth

# max|gpu - oracle| / max|oracle| bounds, per input dtype
TOL = {"f32": 1e-4, "bf16": 1e-2}


def to_dev(a, dtype, device="cuda"):
    """numpy input (uint16 bf16 bits or float32) -> device tensor of `dtype`."""
    if a is None:
        return None
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def to_np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def chunk_case(H, dk, dv, dtype, gate, lengths, s0_sigma=0.1, seed=0, gate_mu=0.0):
    cfg = synth.small_chunk_config(H=H, dk=dk, dv=dv, dtype=dtype, gate=gate, gate_mu=gate_mu,
                                   s0_sigma=s0_sigma, seed=seed)
    return synth.chunk_inputs(cfg, lengths=lengths)


def dev_inputs(d, dtype):
    out = {n: to_dev(d[n], dtype) for n in ("q", "k", "v", "g", "beta")}
    out["S0"] = None if d["S0"] is None else torch.from_numpy(d["S0"]).cuda()
    out["cu_seqlens"] = torch.from_numpy(d["cu_seqlens"].astype(np.int32)).cuda()
    return out

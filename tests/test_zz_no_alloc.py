"""The allocation-free chunked forward (kda_chunk_fwd_noalloc) against the
workspace entry point (kda_chunk_fwd), through the C ABI: two calls in a
row, the second on a smaller input, each bit-identical to kda_chunk_fwd with
a fresh workspace and within the parity bound of the fp64 oracle; a problem
beyond the static scratch is rejected before anything is launched."""
import sys

import numpy as np
import pytest
import torch

import oracle
from _kda_cases import TOL, chunk_case, dev_inputs, to_np64

pytestmark = pytest.mark.gpu

kda = pytest.importorskip("gated_delta_rule_48_amd")


def _say(msg):
    sys.stdout.write(f"\n[case] {msg}\n")
    sys.stdout.flush()


@pytest.mark.parametrize("dtype,gate", [("bf16", "channel"), ("f32", "head")])
def test_noalloc_matches_workspace_entry_point(dtype, gate):
    # the second call is smaller: the scratch keeps the first call's contents
    for i, (H, lengths) in enumerate(((4, [300, 0, 129, 64, 700]), (2, [70]))):
        _say(f"noalloc call {i}: {dtype} {gate} H={H} lengths={lengths}")
        d = chunk_case(H, 128, 128, dtype, gate, lengths, seed=40 + i)
        x = dev_inputs(d, dtype)
        T, N = int(d["cu_seqlens"][-1]), len(lengths)
        ph = gate == "head"
        o_ref, S_ref = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], S0=x["S0"],
                                     cu_seqlens=x["cu_seqlens"], per_head_gate=ph)
        o = torch.full_like(o_ref, 7.0)
        S = torch.full_like(S_ref, 7.0)
        kda.chunk_fwd_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"], out=o, S_T=S, S0=x["S0"],
                              cu_seqlens=x["cu_seqlens"], per_head_gate=ph)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
        o64, S64 = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"],
                                     cu_seqlens=d["cu_seqlens"], per_head_gate=ph)
        assert oracle.rel_err(to_np64(o), o64) <= TOL[dtype]
        assert oracle.rel_err(to_np64(S), S64) <= TOL[dtype]


def test_noalloc_rejects_beyond_scratch():
    _say("noalloc too large")
    H, dk, dv = 32, 128, 128
    T = 8192  # 8192 x 32 head-tokens: ~580 MB of workspace, above the 128 MiB scratch
    assert kda.chunk_fwd_workspace_size(T, 1, H, dk, dv) > (128 << 20)
    z = torch.zeros((T, H, dk), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    o = torch.full((T, H, dv), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kda.KDAError) as ei:
        kda.chunk_fwd_noalloc(z, z, z, z, b, out=o)
    assert ei.value.code == 7
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)

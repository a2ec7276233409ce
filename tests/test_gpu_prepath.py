"""GPU parity of the pre-path transforms: kda_prepare_inputs (a pass of its
own) and kda_recurrent_step_raw (fused into the decode step), against the
fp64 pre-path oracle followed by the fp64 recurrence.

Bounds: the transformed tensors are rounded once to the output type, so
each element is within the unit roundoff of the fp64 value (2^-8 = 3.9e-3
for bf16, 2^-24 for fp32), plus the fp32 arithmetic (~1e-6): 4e-3 relative
per element for bf16, 1e-5 for fp32.  The
recurrence outputs use the bounds stated for the method: max|d|/max|ref| <=
1e-2 (bf16) and 1e-4 (fp32).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import prepath, rel_err

from _kda_cases import TOL, to_dev, to_np64

pytestmark = pytest.mark.gpu

kda = pytest.importorskip("gated_delta_rule_48_amd")

ELEM_TOL = {"bf16": 4e-3, "f32": 1e-5}


def _elem_rel(got, ref):
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gate", ["channel", "head"])
@pytest.mark.parametrize("dk", [64, 128])
def test_prepare_inputs_matches_oracle(dtype, gate, dk):
    rng = np.random.default_rng(40 + dk)
    T, H = 333, 3
    raw = synth.draw_raw_tokens(rng, T, H, dk, 16, dtype, gate, 0.0)
    if dtype == "bf16":
        raw["q"][5, 1] = 0          # an all-zero row stays zero
        raw["g"].reshape(-1)[:4] = synth.bf16_bits(np.array([30.0, -30.0, 0.0, 9.0], dtype=np.float32))
    else:
        raw["q"][5, 1] = 0.0
        raw["g"].reshape(-1)[:4] = [30.0, -30.0, 0.0, 9.0]
    x = {n: to_dev(raw[n], dtype) for n in ("q", "k", "g", "beta")}
    q, k, g, b = kda.prepare_inputs(x["q"], x["k"], x["g"], x["beta"], per_head_gate=(gate == "head"))
    torch.cuda.synchronize()
    ref = prepath.prepare(raw["q"], raw["k"], raw["g"], raw["beta"])
    for name, got, r in zip("qkgb", (q, k, g, b), ref):
        e = _elem_rel(to_np64(got), r)
        print(f"prepare {dtype} {gate} dk={dk} {name}: {e:.2e}", flush=True)
        assert e <= ELEM_TOL[dtype], (name, e)
    assert not np.any(to_np64(q)[5, 1])


def test_prepare_inputs_in_place():
    rng = np.random.default_rng(47)
    raw = synth.draw_raw_tokens(rng, 100, 2, 128, 16, "bf16", "channel", 0.0)
    x = {n: to_dev(raw[n], "bf16") for n in ("q", "k", "g", "beta")}
    want = kda.prepare_inputs(x["q"], x["k"], x["g"], x["beta"])
    got = kda.prepare_inputs(x["q"], x["k"], x["g"], x["beta"], out=(x["q"], x["k"], x["g"], x["beta"]))
    torch.cuda.synchronize()
    for a, b in zip(want, got):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prepare_then_chunk_fwd(dtype):
    """Raw projections -> kda_prepare_inputs -> kda_chunk_fwd against the
    fp64 pre-path oracle -> fp64 recurrence (packed, two sequences)."""
    rng = np.random.default_rng(48)
    lengths = [200, 77]
    T, H, dk, dv = sum(lengths), 2, 128, 128
    raw = synth.draw_raw_tokens(rng, T, H, dk, dv, dtype, "channel", -1.0)
    x = {n: to_dev(raw[n], dtype) for n in ("q", "k", "v", "g", "beta")}
    q, k, g, b = kda.prepare_inputs(x["q"], x["k"], x["g"], x["beta"])
    cu = np.array([0, lengths[0], T], dtype=np.int32)
    o, S_T = kda.chunk_fwd(q, k, x["v"], g, b, cu_seqlens=torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    pq, pk, pg, pb = prepath.prepare(raw["q"], raw["k"], raw["g"], raw["beta"])
    o_ref, S_ref = oracle.recurrence(pq, pk, oracle.widen(raw["v"]), pg, pb, cu_seqlens=cu)
    eo, es = rel_err(to_np64(o), o_ref), rel_err(to_np64(S_T), S_ref)
    print(f"prepare+chunk_fwd {dtype}: o {eo:.2e} S_T {es:.2e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def _raw_case(rng, lengths, H, dk, dv, dtype, gate, gate_mu):
    raw = synth.draw_raw_tokens(rng, sum(lengths), H, dk, dv, dtype, gate, gate_mu)
    return raw, np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def _run_raw(raw, cu, dtype, gate, S0=None):
    x = {n: to_dev(raw[n], dtype) for n in ("q", "k", "v", "g", "beta")}
    o, S_T = kda.chunk_fwd_raw(x["q"], x["k"], x["v"], x["g"], x["beta"], S0=S0,
                               cu_seqlens=torch.from_numpy(cu).cuda(), per_head_gate=(gate == "head"))
    torch.cuda.synchronize()
    return to_np64(o), to_np64(S_T)


def _oracle_raw(raw, cu, gate, S0=None):
    pq, pk, pg, pb = prepath.prepare(raw["q"], raw["k"], raw["g"], raw["beta"])
    return oracle.recurrence(pq, pk, oracle.widen(raw["v"]), pg, pb, S0=S0, cu_seqlens=cu,
                             per_head_gate=(gate == "head"))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gate", ["channel", "head"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_chunk_fwd_raw_matches_oracle(dtype, gate, dk, dv):
    """The prefill from raw projections (pre-path fused into the intra-chunk
    kernel) against the fp64 pre-path oracle followed by the fp64 recurrence:
    ragged packed sequences (one empty), a non-zero S0, an all-zero q row and
    an all-zero k row, and raw gates far out in both tails."""
    rng = np.random.default_rng(60 + dk + dv)
    lengths = [150, 0, 64, 71]
    H = 2
    raw, cu = _raw_case(rng, lengths, H, dk, dv, dtype, gate, 0.0)
    zero = 0 if dtype == "bf16" else 0.0
    raw["q"][3, 1] = zero
    raw["k"][70, 0] = zero
    tails = np.array([30.0, -30.0, 12.0, -12.0], dtype=np.float32)
    raw["g"].reshape(-1)[7:11] = synth.bf16_bits(tails) if dtype == "bf16" else tails
    S0 = (rng.standard_normal((len(lengths), H, dk, dv)) * 0.1).astype(np.float32)
    o, S = _run_raw(raw, cu, dtype, gate, S0=torch.from_numpy(S0).cuda())
    o_ref, S_ref = _oracle_raw(raw, cu, gate, S0=S0)
    eo, es = rel_err(o, o_ref), rel_err(S, S_ref)
    print(f"chunk_fwd_raw {dtype} {gate} dk={dk} dv={dv}: o {eo:.2e} S_T {es:.2e}", flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    assert eo <= TOL[dtype] and es <= TOL[dtype]
    assert not np.any(o[3, 1])  # q = 0 reads nothing


def test_chunk_fwd_raw_32k():
    """The 32K x 32 benchmark shape (bf16, d = 128, per-channel gate)
    from raw projections drawn with the benchmark recipe (gate pre-activation
    from N(-1, 1))."""
    rng = np.random.default_rng(64)
    raw, cu = _raw_case(rng, [32768], 32, 128, 128, "bf16", "channel", -1.0)
    o, S = _run_raw(raw, cu, "bf16", "channel")
    o_ref, S_ref = _oracle_raw(raw, cu, "channel")
    eo, es = rel_err(o, o_ref), rel_err(S, S_ref)
    print(f"chunk_fwd_raw 32k: o {eo:.2e} S_T {es:.2e}", flush=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_chunk_fwd_raw_equals_prepared_in_fp32():
    """fp32: the fused pre-path and kda_prepare_inputs followed by
    kda_chunk_fwd differ only in the summation order of the norms (a few
    fp32 ulps in the prepared q and k), so their outputs agree far inside
    the fp32 bound."""
    rng = np.random.default_rng(65)
    raw, cu = _raw_case(rng, [300, 45], 3, 128, 128, "f32", "channel", 0.0)
    o_raw, S_raw = _run_raw(raw, cu, "f32", "channel")
    x = {n: to_dev(raw[n], "f32") for n in ("q", "k", "v", "g", "beta")}
    q, k, g, b = kda.prepare_inputs(x["q"], x["k"], x["g"], x["beta"])
    o, S_T = kda.chunk_fwd(q, k, x["v"], g, b, cu_seqlens=torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    assert rel_err(o_raw, to_np64(o)) <= 1e-5 and rel_err(S_raw, to_np64(S_T)) <= 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gate", ["channel", "head"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_recurrent_step_raw(dtype, gate, dk, dv):
    """Three fused decode steps from raw projections against the oracle."""
    rng = np.random.default_rng(49)
    N, H = 5, 3
    S0 = (rng.standard_normal((N, H, dk, dv)) * 0.1).astype(np.float32)
    S = torch.from_numpy(S0).cuda()
    S_ref = S0.astype(np.float64)
    for step in range(3):
        raw = synth.draw_raw_tokens(rng, N, H, dk, dv, dtype, gate, 0.0)
        x = {n: to_dev(raw[n], dtype) for n in ("q", "k", "v", "g", "beta")}
        o = kda.recurrent_step_raw(x["q"], x["k"], x["v"], x["g"], x["beta"], S, per_head_gate=(gate == "head"))
        torch.cuda.synchronize()
        pq, pk, pg, pb = prepath.prepare(raw["q"], raw["k"], raw["g"], raw["beta"])
        o_ref, S_ref = oracle.recurrence(pq, pk, oracle.widen(raw["v"]), pg, pb, S0=S_ref,
                                         cu_seqlens=list(range(N + 1)), per_head_gate=(gate == "head"))
        eo = rel_err(to_np64(o), o_ref)
        assert eo <= TOL[dtype], (step, eo)
    es = rel_err(S.cpu().numpy(), S_ref)
    print(f"decode raw {dtype} {gate} dk={dk} dv={dv}: o {eo:.2e} S {es:.2e}", flush=True)
    assert es <= TOL[dtype]

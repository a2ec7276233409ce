"""Parity of the 128-token chunk path (kda_chunk_fwd_c128, through the C ABI)
with the fp64 oracle.

Same bar as the 64-token path: max|gpu - oracle| / max|oracle| <= 1e-4 for
fp32 inputs and <= 1e-2 for bf16 inputs with fp32 state, for o and S_T.
The oracle is the sequential recurrence, which does not depend on the chunk
size; its chunked form at C = 128 is pinned to it in test_oracle_pins.py.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from _kda_cases import TOL, chunk_case, dev_inputs, to_np64

pytestmark = pytest.mark.gpu

kda = pytest.importorskip("gated_delta_rule_48_amd")


def _announce(msg):
    sys.stdout.write(f"\n[case] {msg}\n")
    sys.stdout.flush()


def _run(d, dtype, gate, chunk=128, **kw):
    x = dev_inputs(d, dtype)
    o, S_T = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], S0=x["S0"], cu_seqlens=x["cu_seqlens"],
                           per_head_gate=(gate == "head"), chunk=chunk, **kw)
    torch.cuda.synchronize()
    return to_np64(o), to_np64(S_T)


def _oracle(d, gate):
    return oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"], cu_seqlens=d["cu_seqlens"],
                             per_head_gate=(gate == "head"))


def _close(name, got, ref, tol):
    err = oracle.rel_err(got, ref)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert err <= tol, f"{name}: rel err {err:.3e} > {tol:.0e}"
    return err


def _parity(d, dtype, gate):
    o, S = _run(d, dtype, gate)
    o_ref, S_ref = _oracle(d, gate)
    return _close("o", o, o_ref, TOL[dtype]), _close("S_T", S, S_ref, TOL[dtype])


# every compiled variant: bf16 at every head size, fp32 at d = 64
VARIANTS = [("bf16", 64, 64), ("bf16", 64, 128), ("bf16", 128, 64), ("bf16", 128, 128), ("f32", 64, 64)]


@pytest.mark.parametrize("gate", ["channel", "head"])
@pytest.mark.parametrize("dtype,dk,dv", VARIANTS)
def test_c128_every_instantiation(dtype, dk, dv, gate):
    """Several 128-token chunks with a ragged tail, an empty sequence, a
    single token and chunk-boundary lengths, nonzero S0."""
    _announce(f"c128 instantiation {dtype} {gate} {dk}x{dv}")
    d = chunk_case(2, dk, dv, dtype, gate, [70, 0, 129, 1, 256, 383], s0_sigma=0.1, seed=dk * 5 + dv + 1)
    print("errs", _parity(d, dtype, gate), flush=True)


@pytest.mark.parametrize("lengths", [[1], [127, 128, 129], [255, 256, 257]], ids=["one", "around128", "around256"])
def test_c128_lengths_f32(lengths):
    _announce(f"c128 lengths {lengths}")
    d = chunk_case(2, 64, 64, "f32", "channel", lengths, s0_sigma=0.1, seed=sum(lengths))
    _parity(d, "f32", "channel")


def test_c128_strong_decay():
    """Gates from N(+3, 1): the chunk-local log-decay reaches about -400 over
    128 tokens, far below the fp32 range; only the in-tile factors (eight
    tokens) are formed from it directly."""
    _announce("c128 strong decay")
    d = chunk_case(2, 128, 128, "bf16", "channel", [300], s0_sigma=0.1, seed=5, gate_mu=3.0)
    _parity(d, "bf16", "channel")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_c128_gate_at_contract_edge(dtype):
    """g = -10 everywhere: e^-80 over eight tokens, the edge of the documented
    gate range (in-tile factors up to e^80)."""
    _announce(f"c128 gate edge {dtype}")
    dk = 64 if dtype == "f32" else 128
    d = chunk_case(2, dk, 64, dtype, "channel", [260, 128], s0_sigma=0.1, seed=12)
    g = np.full(d["g"].shape, -10.0, dtype=np.float32)
    d["g"] = synth.bf16_bits(g) if dtype == "bf16" else g
    _parity(d, dtype, "channel")


def test_c128_no_decay_and_beta_zero():
    """g = 0 (DeltaNet): the state carries over every chunk; beta = 0: the
    initial state only decays (A = 0, T = I, W = U' = 0)."""
    _announce("c128 no decay / beta zero")
    d = chunk_case(2, 64, 64, "f32", "channel", [400], s0_sigma=0.1, seed=6)
    d["g"] = np.zeros_like(d["g"])
    _parity(d, "f32", "channel")
    d = chunk_case(2, 64, 64, "f32", "channel", [300, 128], s0_sigma=0.1, seed=11)
    d["beta"] = np.zeros_like(d["beta"])
    _parity(d, "f32", "channel")


def test_c128_many_ragged_sequences():
    """300 packed sequences of 0..300 tokens, H = 3."""
    _announce("c128 many ragged sequences")
    rng = np.random.default_rng(13)
    lengths = rng.integers(0, 301, size=300)
    lengths[:12] = [0, 1, 127, 128, 129, 255, 256, 257, 0, 0, 1, 300]
    d = chunk_case(3, 64, 64, "bf16", "channel", list(lengths), s0_sigma=0.1, seed=13)
    _parity(d, "bf16", "channel")


@pytest.mark.parametrize("lengths", [[16384], [8192, 100], [3000, 0, 1, 4097]],
                         ids=["long", "long_short", "with_empty"])
def test_c128_segmented(lengths):
    """bf16, d = 128, H = 2: few (sequence, head) pairs, so the 128-token
    walk cuts each pair's chunks into segments joined through their affine
    maps; short and empty sequences leave whole segments empty."""
    _announce(f"c128 segmented {lengths}")
    d = chunk_case(2, 128, 128, "bf16", "channel", lengths, s0_sigma=0.1, seed=31 + len(lengths))
    o, S = _run(d, "bf16", "channel")
    o_ref, S_ref = _oracle(d, "channel")
    print(f"segmented: o {oracle.rel_err(o, o_ref):.2e} S_T {oracle.rel_err(S, S_ref):.2e}", flush=True)
    _close("o", o, o_ref, TOL["bf16"])
    _close("S_T", S, S_ref, TOL["bf16"])
    for n, L in enumerate(lengths):
        if L == 0:
            assert np.array_equal(S[n], np.asarray(d["S0"][n], dtype=np.float64))


def test_c128_deterministic():
    _announce("c128 determinism")
    d = chunk_case(2, 128, 128, "bf16", "channel", [8192, 100], s0_sigma=0.1, seed=34)
    a = _run(d, "bf16", "channel")
    b = _run(d, "bf16", "channel")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_c128_agrees_with_c64():
    """Both chunk sizes compute the same recurrence: o and S_T agree to the
    bf16 bound (not bitwise: the sums are grouped differently)."""
    _announce("c128 vs c64")
    d = chunk_case(2, 128, 128, "bf16", "head", [1000, 37], s0_sigma=0.1, seed=40)
    o1, S1 = _run(d, "bf16", "head", chunk=64)
    o2, S2 = _run(d, "bf16", "head", chunk=128)
    assert oracle.rel_err(o2, o1) <= 1e-2 and oracle.rel_err(S2, S1) <= 1e-2


def test_c128_bad_seqlens_and_unsupported():
    _announce("c128 bad cu_seqlens / unsupported")
    d = chunk_case(2, 64, 64, "bf16", "channel", [128, 128], seed=13)
    x = dev_inputs(d, "bf16")
    bad = torch.tensor([0, 200, 128], dtype=torch.int32, device="cuda")  # decreasing
    o = torch.full((256, 2, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kda.KDAError) as ei:
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], cu_seqlens=bad, out=o, chunk=128)
    assert ei.value.code == 5
    assert torch.all(o == 7.0)
    f = torch.zeros(8, 1, 128, device="cuda")
    with pytest.raises(kda.KDAError) as ei:  # fp32 at d = 128
        kda.chunk_fwd(f, f, f, f, torch.zeros(8, 1, device="cuda"), chunk=128)
    assert ei.value.code == 2


# ------------------------------------------------------- benchmark configs
def test_c128_config_tiny_f32():
    """B=1, T=256, H=2, d=64, fp32, per-channel gate, S0 = 0, C = 128."""
    _announce("c128 config kda_tiny_f32")
    d = synth.chunk_inputs(synth.CONFIGS["kda_tiny_f32"])
    print("tiny errs", _parity(d, "f32", "channel"), flush=True)


def test_c128_config_gdn_varlen_bf16():
    """8 packed sequences (U{256..8192}), H=16, d=128, per-head gate, C = 128."""
    _announce("c128 config gdn_varlen_bf16")
    d = synth.chunk_inputs(synth.CONFIGS["gdn_varlen_bf16"])
    print("varlen errs", _parity(d, "bf16", "head"), flush=True)


def test_c128_config_32k_bf16():
    """B=1, T=32768, H=32, d=128, per-channel gate from N(-1,1), C = 128."""
    _announce("c128 config kda_32k_bf16")
    d = synth.chunk_inputs(synth.CONFIGS["kda_32k_bf16"])
    print("32k errs", _parity(d, "bf16", "channel"), flush=True)

"""GPU parity of the chunked backward pass (kda_chunk_bwd) against the fp64
gradient oracle (autograd of the sequential recurrence).

Every gradient (dq, dk, dv, dg, dbeta, dS0) is compared element by element:
max|gpu - oracle| / max|oracle| <= 1e-4 for fp32 inputs and <= 1e-2 for bf16
inputs (fp32 state and fp32 arithmetic inside), the bounds stated for the
forward path.  Small cases use the autograd oracle; the benchmark workloads
(T = 32768 x 32 heads, the packed 8-sequence Gated DeltaNet batch, and
T = 1,048,576 x 16 heads) use the hand-written fp64 C adjoint with dense
cotangents dO and dS_T, so that the reverse state walk carries a nonzero
cotangent through every chunk.  A causality property is checked as well: with
dO zero after the first P tokens and dS_T = 0, the gradients of those P tokens
are those of the P-token problem and every later gradient is exactly zero.
"""
import os
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import rel_err
from oracle.grad import adjoint, recurrence_grad

from _kda_cases import TOL, chunk_case, to_dev, to_np64

pytestmark = pytest.mark.gpu

kda = pytest.importorskip("gated_delta_rule_48_amd")

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


def _run(d, dtype, gate, dO, dST, with_s0=True, with_dst=True):
    x = {n: to_dev(d[n], dtype) for n in ("q", "k", "v", "g", "beta")}
    S0 = torch.from_numpy(d["S0"]).cuda() if (with_s0 and d["S0"] is not None) else None
    cu = torch.from_numpy(d["cu_seqlens"].astype(np.int32)).cuda()
    got = kda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], to_dev(dO, dtype), S0=S0,
                        dS_T=torch.from_numpy(dST).cuda() if with_dst else None, cu_seqlens=cu,
                        per_head_gate=(gate == "head"))
    torch.cuda.synchronize()
    return [to_np64(t) for t in got]


def _ref(d, gate, dO, dST, with_s0=True, with_dst=True):
    return recurrence_grad(d["q"], d["k"], d["v"], d["g"], d["beta"], dO,
                           S0=d["S0"] if with_s0 else None, dS_T=dST if with_dst else None,
                           cu_seqlens=d["cu_seqlens"], per_head_gate=(gate == "head"))


def _compare(got, ref, tol, tag):
    errs = {n: rel_err(gv, rv) for n, gv, rv in zip(NAMES, got, ref)}
    print(tag, " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= tol, (tag, n, e)
    return errs


def _case(H, dk, dv, dtype, gate, lengths, seed, **kw):
    d = chunk_case(H, dk, dv, dtype, gate, lengths, seed=seed, **kw)
    T, N = int(d["cu_seqlens"][-1]), len(lengths)
    dO, dST = synth.draw_cotangents(np.random.default_rng(seed + 1000), T, N, H, dk, dv, dtype)
    return d, dO, dST


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gate", ["channel", "head"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_bwd_every_instantiation(dtype, gate, dk, dv):
    d, dO, dST = _case(2, dk, dv, dtype, gate, [150, 70], seed=7)
    _compare(_run(d, dtype, gate, dO, dST), _ref(d, gate, dO, dST), TOL[dtype],
             f"bwd {dtype} {gate} dk={dk} dv={dv}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_empty_one_token_and_exact_chunk(dtype):
    d, dO, dST = _case(3, 128, 128, dtype, "channel", [0, 1, 64, 129, 0], seed=8)
    got = _run(d, dtype, "channel", dO, dST)
    _compare(got, _ref(d, "channel", dO, dST), TOL[dtype], f"bwd edges {dtype}")
    # an empty sequence passes the state cotangent straight through
    assert np.array_equal(got[5][0], dST[0].astype(np.float64))
    assert np.array_equal(got[5][4], dST[4].astype(np.float64))


def test_bwd_without_s0_and_state_cotangent():
    d, dO, dST = _case(2, 128, 128, "f32", "channel", [200], seed=9)
    got = _run(d, "f32", "channel", dO, dST, with_s0=False, with_dst=False)
    _compare(got, _ref(d, "channel", dO, dST, with_s0=False, with_dst=False), TOL["f32"], "bwd no S0/dS_T")


def _set_gate(d, dtype, g32):
    """Replace the log-gate by the float32 values g32 (rounded to the case's dtype)."""
    g32 = np.asarray(g32, dtype=np.float32)
    d["g"] = synth.bf16_bits(g32) if dtype == "bf16" else g32


def test_bwd_moderate_gate():
    """g = -2.5 on every channel: 32 tokens of decay reach e^-80 (the limit
    of a single reference row per chunk)."""
    d, dO, dST = _case(2, 64, 64, "f32", "channel", [128, 100], seed=10)
    _set_gate(d, "f32", np.full(d["g"].shape, -2.5))
    _compare(_run(d, "f32", "channel", dO, dST), _ref(d, "channel", dO, dST), TOL["f32"], "bwd g=-2.5")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_gate_minus_ten(dtype):
    """g = -10 on every channel: eight tokens of decay reach e^-80, the edge
    of the supported range; a whole chunk decays by e^-640."""
    d, dO, dST = _case(2, 128, 128, dtype, "channel", [150, 64, 37], seed=20)
    _set_gate(d, dtype, np.full(d["g"].shape, -10.0))
    _compare(_run(d, dtype, "channel", dO, dST), _ref(d, "channel", dO, dST), TOL[dtype], f"bwd g=-10 {dtype}")


def _mixed_gate(shape, seed, fast):
    """Per-channel gates: a third of the (head, channel) pairs forget fast
    (g = `fast` at every token), a third slowly (g = -0.1), the rest draw g
    uniformly from [-10, 0] at every token."""
    T, H, dk = shape
    rng = np.random.default_rng(seed)
    kind = rng.integers(0, 3, size=(1, H, dk))
    g = np.where(kind == 0, fast, np.where(kind == 1, -0.1, rng.uniform(-10.0, 0.0, size=(T, H, dk))))
    return np.ascontiguousarray(np.broadcast_to(g, (T, H, dk)), dtype=np.float32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_mixed_fast_and_slow_channels(dtype):
    """Fast channels at the edge of the range (g = -10), slow ones (g = -0.1)
    and channels uniform in [-10, 0], side by side."""
    d, dO, dST = _case(2, 128, 128, dtype, "channel", [200, 90], seed=21)
    _set_gate(d, dtype, _mixed_gate(d["g"].shape, 2121, -10.0))
    _compare(_run(d, dtype, "channel", dO, dST), _ref(d, "channel", dO, dST), TOL[dtype], f"bwd mixed {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_beyond_range_stays_finite(dtype):
    """Channels at g = -30 (beyond the exact range: eight tokens decay by
    e^-240) next to slow ones: every gradient stays finite."""
    d, dO, dST = _case(2, 128, 128, dtype, "channel", [200, 90], seed=24)
    _set_gate(d, dtype, _mixed_gate(d["g"].shape, 2424, -30.0))
    got = _run(d, dtype, "channel", dO, dST)
    errs = {n: rel_err(np.nan_to_num(gv, nan=0.0, posinf=0.0, neginf=0.0), rv)
            for n, gv, rv in zip(NAMES, got, _ref(d, "channel", dO, dST))}
    print(f"bwd beyond range {dtype}", " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    for n, gv in zip(NAMES, got):
        assert np.all(np.isfinite(gv)), n


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_strong_decay_tail(dtype):
    """The forward's strong-decay input distribution (g = -softplus of
    N(3, 1), about -98 nats over 32 tokens) through the backward."""
    d, dO, dST = _case(2, 128, 128, dtype, "channel", [200, 70], seed=26, gate_mu=3.0)
    _compare(_run(d, dtype, "channel", dO, dST), _ref(d, "channel", dO, dST), TOL[dtype], f"bwd mu=3 {dtype}")


def test_bwd_strong_per_head_gate():
    """The Gated DeltaNet special case at g = -8 per (token, head)."""
    d, dO, dST = _case(2, 128, 128, "f32", "head", [129, 64], seed=22)
    _set_gate(d, "f32", np.full(d["g"].shape, -8.0))
    _compare(_run(d, "f32", "head", dO, dST), _ref(d, "head", dO, dST), TOL["f32"], "bwd head g=-8")


def test_bwd_longer_bench_distribution():
    """Bench-like inputs (gate mean -1, bf16) over 16 chunks and 4 heads."""
    d, dO, dST = _case(4, 128, 128, "bf16", "channel", [1024], seed=11, gate_mu=-1.0)
    _compare(_run(d, "bf16", "channel", dO, dST), _ref(d, "channel", dO, dST), TOL["bf16"], "bwd 1024x4 bf16")


def test_bwd_deterministic():
    d, dO, dST = _case(2, 128, 128, "bf16", "channel", [300], seed=12)
    a = _run(d, "bf16", "channel", dO, dST)
    b = _run(d, "bf16", "channel", dO, dST)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_full_size_prefix_support():
    """T = 32768, H = 32, d = 128, bf16 (the prefill benchmark workload)."""
    cfg = synth.CONFIGS["kda_32k_bf16"]
    d = synth.chunk_inputs(cfg)
    T, H, dk, dv = cfg.T, cfg.H, cfg.dk, cfg.dv
    P = 256
    rng = np.random.default_rng(3031)
    dO = np.zeros((T, H, dv), dtype=np.uint16)
    dO[:P] = synth.bf16_bits(rng.standard_normal((P, H, dv), dtype=np.float32))
    x = {n: to_dev(d[n], "bf16") for n in ("q", "k", "v", "g", "beta")}
    got = kda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], to_dev(dO, "bf16"),
                        cu_seqlens=torch.tensor([0, T], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    got = [t.float().cpu().numpy() for t in got]
    for gv in got[:5]:
        assert not np.any(gv[P:]), "gradient beyond the support of dO"
    sub = {n: d[n][:P] for n in ("q", "k", "v", "g", "beta")}
    ref = recurrence_grad(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], dO[:P])
    for n, gv, rv in zip(NAMES, [g[:P] for g in got[:5]] + [got[5]], ref):
        e = rel_err(gv, rv)
        print(f"bwd 32k prefix {n}={e:.2e}", flush=True)
        assert e <= TOL["bf16"], (n, e)


def test_bwd_varlen_gated_deltanet_full_size_prefix_support():
    """The packed 8-sequence Gated DeltaNet workload (per-head gate, S0 given,
    H = 16, d = 128, bf16): dO is zero except on the first 128 tokens of every
    sequence and dS_T = 0, so each sequence's prefix gradients and dS0 are
    those of the 128-token problems, and every other gradient is zero."""
    cfg = synth.CONFIGS["gdn_varlen_bf16"]
    d = synth.chunk_inputs(cfg)
    cu = d["cu_seqlens"].astype(np.int64)
    T, H, dk, dv, N = int(cu[-1]), cfg.H, cfg.dk, cfg.dv, len(cu) - 1
    P = 128
    rng = np.random.default_rng(2021)
    dO = np.zeros((T, H, dv), dtype=np.uint16)
    rows = np.concatenate([np.arange(cu[n], cu[n] + P) for n in range(N)])
    dO[rows] = synth.bf16_bits(rng.standard_normal((len(rows), H, dv), dtype=np.float32))
    x = {n: to_dev(d[n], "bf16") for n in ("q", "k", "v", "g", "beta")}
    got = kda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], to_dev(dO, "bf16"),
                        S0=torch.from_numpy(d["S0"]).cuda(),
                        cu_seqlens=torch.from_numpy(d["cu_seqlens"].astype(np.int32)).cuda(), per_head_gate=True)
    torch.cuda.synchronize()
    got = [t.float().cpu().numpy() for t in got]
    mask = np.zeros(T, dtype=bool)
    mask[rows] = True
    for gv in got[:5]:
        assert not np.any(gv[~mask]), "gradient beyond the support of dO"
    sub = {n: d[n][rows] for n in ("q", "k", "v", "g", "beta")}
    ref = recurrence_grad(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], dO[rows], S0=d["S0"],
                          cu_seqlens=np.arange(N + 1) * P, per_head_gate=True)
    for n_, gv, rv in zip(NAMES, [g[rows] for g in got[:5]] + [got[5]], ref):
        e = rel_err(gv, rv)
        print(f"bwd gdn varlen prefix {n_}={e:.2e}", flush=True)
        assert e <= TOL["bf16"], (n_, e)


def test_bwd_no_tokens_passes_state_cotangent():
    """T = 0 (every sequence empty): dS0 = dS_T exactly, nothing else to do."""
    H, dk, dv, N = 2, 64, 128, 3
    rng = np.random.default_rng(77)
    dST = rng.standard_normal((N, H, dk, dv)).astype(np.float32)
    e = torch.empty((0, H, dk), dtype=torch.bfloat16, device="cuda")
    ev = torch.empty((0, H, dv), dtype=torch.bfloat16, device="cuda")
    eb = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    got = kda.chunk_bwd(e, e, ev, e, eb, ev, dS_T=torch.from_numpy(dST).cuda(),
                        cu_seqlens=torch.zeros(N + 1, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(got[5].cpu().numpy(), dST)


@pytest.mark.parametrize("dtype,gate", [("bf16", "channel"), ("f32", "head")])
def test_bwd_head_groups_bit_identical(dtype, gate):
    """A workspace for two heads processes five heads in groups of 2, 2, 1;
    the results equal those of one pass over all heads bit for bit."""
    d, dO, dST = _case(5, 128, 128, dtype, gate, [150, 70], seed=13)
    full = _run(d, dtype, gate, dO, dST)
    T = int(d["cu_seqlens"][-1])
    small = kda.chunk_bwd_workspace_size(T, 2, 2, 128, 128, torch.bfloat16 if dtype == "bf16" else torch.float32)
    assert small < kda.chunk_bwd_workspace_size(T, 2, 5, 128, 128)
    x = {n: to_dev(d[n], dtype) for n in ("q", "k", "v", "g", "beta")}
    got = kda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], to_dev(dO, dtype),
                        S0=torch.from_numpy(d["S0"]).cuda(), dS_T=torch.from_numpy(dST).cuda(),
                        cu_seqlens=torch.from_numpy(d["cu_seqlens"].astype(np.int32)).cuda(),
                        per_head_gate=(gate == "head"),
                        workspace=torch.empty(small, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    for a, b in zip(full, got):
        assert np.array_equal(a, to_np64(b))


def test_bwd_1m_tokens_in_head_groups_prefix_support():
    """The 1M-token workload (T = 1,048,576, H = 16, d = 128, bf16) through a
    workspace for four heads (four groups of four).  dO is zero after the
    first 256 tokens and dS_T = 0: those tokens' gradients and dS0 are the
    256-token problem's, and every later gradient is exactly zero."""
    cfg = synth.CONFIGS["kda_1m_bf16"]
    T, H, dk, dv = cfg.T, cfg.H, cfg.dk, cfg.dv
    shapes = {"q": (T, H, dk), "k": (T, H, dk), "v": (T, H, dv), "g": (T, H, dk), "beta": (T, H)}
    dev = {n: torch.empty(s, dtype=torch.bfloat16, device="cuda") for n, s in shapes.items()}
    first = None
    for b, start, blk in synth.iter_token_blocks(cfg, workers=8):
        rows = blk["q"].shape[0]
        for n in shapes:
            dev[n][start:start + rows].copy_(torch.from_numpy(blk[n].view(np.int16)).view(torch.bfloat16))
        if start == 0:
            first = blk
    P = 256
    dO = torch.zeros((T, H, dv), dtype=torch.bfloat16, device="cuda")
    dO_head = synth.bf16_bits(np.random.default_rng(4040).standard_normal((P, H, dv), dtype=np.float32))
    dO[:P].copy_(torch.from_numpy(dO_head.view(np.int16)).view(torch.bfloat16))
    ws = torch.empty(kda.chunk_bwd_workspace_size(T, 1, 4, dk, dv), dtype=torch.uint8, device="cuda")
    got = kda.chunk_bwd(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dO, workspace=ws)
    torch.cuda.synchronize()
    for gv in got[:5]:
        assert int(torch.count_nonzero(gv[P:])) == 0, "gradient beyond the support of dO"
    ref = recurrence_grad(first["q"][:P], first["k"][:P], first["v"][:P], first["g"][:P], first["beta"][:P],
                          dO_head)
    for n_, gv, rv in zip(NAMES, [to_np64(g[:P]) for g in got[:5]] + [to_np64(got[5])], ref):
        e = rel_err(gv, rv)
        print(f"bwd 1m prefix {n_}={e:.2e}", flush=True)
        assert e <= TOL["bf16"], (n_, e)


def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def _say(msg):
    sys.stdout.write(f"\n[case] {msg}\n")
    sys.stdout.flush()


def _dense_cotangents(seed, T, N, H, dk, dv, block=1 << 16):
    """dO ~ N(0, 1) as bf16 bits, drawn in blocks of rows; dS_T ~ N(0, 1) fp32."""
    rng = np.random.default_rng(seed)
    dO = np.empty((T, H, dv), dtype=np.uint16)
    for s0 in range(0, T, block):
        e = min(T, s0 + block)
        dO[s0:e] = synth.bf16_bits(rng.standard_normal((e - s0, H, dv), dtype=np.float32))
    dST = rng.standard_normal((N, H, dk, dv), dtype=np.float32)
    return dO, dST


def test_bwd_full_size_dense():
    """T = 32768, H = 32, d = 128, bf16 (the prefill benchmark workload) with
    dense dO and dS_T: every gradient, every element, against the C adjoint."""
    _say("bwd 32k x 32 dense")
    cfg = synth.CONFIGS["kda_32k_bf16"]
    d = synth.chunk_inputs(cfg)
    T, H, dk, dv = cfg.T, cfg.H, cfg.dk, cfg.dv
    dO, dST = _dense_cotangents(3032, T, 1, H, dk, dv)
    x = {n: to_dev(d[n], "bf16") for n in ("q", "k", "v", "g", "beta")}
    got = kda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], to_dev(dO, "bf16"),
                        dS_T=torch.from_numpy(dST).cuda())
    torch.cuda.synchronize()
    got = [to_np64(t) for t in got]
    _say("bwd 32k x 32 dense: oracle")
    ref = adjoint(d["q"], d["k"], d["v"], d["g"], d["beta"], dO, dS_T=dST, threads=_threads())
    _compare(got, ref, TOL["bf16"], "bwd 32k dense")


def test_bwd_varlen_gated_deltanet_dense():
    """The packed 8-sequence Gated DeltaNet workload (per-head gate, S0 given,
    H = 16, d = 128, bf16) with dense dO and dS_T, against the C adjoint."""
    _say("bwd gdn varlen dense")
    cfg = synth.CONFIGS["gdn_varlen_bf16"]
    d = synth.chunk_inputs(cfg)
    cu = d["cu_seqlens"].astype(np.int64)
    T, H, dk, dv, N = int(cu[-1]), cfg.H, cfg.dk, cfg.dv, len(cu) - 1
    dO, dST = _dense_cotangents(2022, T, N, H, dk, dv)
    x = {n: to_dev(d[n], "bf16") for n in ("q", "k", "v", "g", "beta")}
    got = kda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], to_dev(dO, "bf16"),
                        S0=torch.from_numpy(d["S0"]).cuda(), dS_T=torch.from_numpy(dST).cuda(),
                        cu_seqlens=torch.from_numpy(cu.astype(np.int32)).cuda(), per_head_gate=True)
    torch.cuda.synchronize()
    got = [to_np64(t) for t in got]
    ref = adjoint(d["q"], d["k"], d["v"], d["g"], d["beta"], dO, S0=d["S0"], dS_T=dST, cu_seqlens=cu,
                  per_head_gate=True, threads=_threads())
    _compare(got, ref, TOL["bf16"], "bwd gdn varlen dense")


def test_bwd_1m_dense_sampled_in_head_groups():
    """The 1M-token workload (T = 1,048,576, H = 16, d = 128, bf16) with dense
    dO and dS_T, through a workspace for four heads: the gradients at 4096
    seeded positions and the full dS0, against the C adjoint (which walks all
    16,384 chunks of every head in fp64)."""
    _say("bwd 1m x 16 dense: inputs")
    cfg = synth.CONFIGS["kda_1m_bf16"]
    T, H, dk, dv = cfg.T, cfg.H, cfg.dk, cfg.dv
    shapes = {"q": (T, H, dk), "k": (T, H, dk), "v": (T, H, dv), "g": (T, H, dk), "beta": (T, H)}
    host = {n: np.empty(s, dtype=np.uint16) for n, s in shapes.items()}
    dev = {n: torch.empty(s, dtype=torch.bfloat16, device="cuda") for n, s in shapes.items()}
    for b, start, blk in synth.iter_token_blocks(cfg, workers=8):
        rows = blk["q"].shape[0]
        for n in shapes:
            host[n][start:start + rows] = blk[n]
            dev[n][start:start + rows].copy_(torch.from_numpy(blk[n].view(np.int16)).view(torch.bfloat16))
    dO, dST = _dense_cotangents(4041, T, 1, H, dk, dv)
    pos = synth.sample_positions(T, 4096, seed=4042)
    _say("bwd 1m x 16 dense: gpu")
    ws = torch.empty(kda.chunk_bwd_workspace_size(T, 1, 4, dk, dv), dtype=torch.uint8, device="cuda")
    got = kda.chunk_bwd(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], to_dev(dO, "bf16"),
                        dS_T=torch.from_numpy(dST).cuda(), workspace=ws)
    idx = torch.from_numpy(pos).cuda()
    got = [to_np64(t[idx]) for t in got[:5]] + [to_np64(got[5])]
    torch.cuda.synchronize()
    del dev, ws
    _say("bwd 1m x 16 dense: oracle")
    ref = adjoint(host["q"], host["k"], host["v"], host["g"], host["beta"], dO, dS_T=dST, positions=pos,
                  threads=_threads())
    _compare(got, ref, TOL["bf16"], "bwd 1m dense")

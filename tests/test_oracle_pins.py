"""Pins for the fp64 oracle, against facts the pages and the mathematics fix.

Each test states which mistake in the oracle it would catch.  None of them
retypes the oracle's own update: they use hand-worked fixtures, closed forms
obtained by solving the recurrence for special inputs, invariants, exact
rational arithmetic of the product form, and agreement between three
independently written formulations.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")
TOL = 1e-12


def _rand(rng, T, H, dk, dv, per_head=False, unit_keys=True, s0=True, N=1):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = -np.logaddexp(0.0, rng.standard_normal((T, H) if per_head else (T, H, dk)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    S0 = rng.standard_normal((N, H, dk, dv)) * 0.3 if s0 else None
    return q, k, v, g, beta, S0


def _all_forms(q, k, v, g, beta, **kw):
    chunk = kw.pop("chunk", 16)
    a = oracle.recurrence(q, k, v, g, beta, **kw)
    b = oracle.chunked(q, k, v, g, beta, chunk=chunk, **kw)
    c = oracle.dense_dplr(q, k, v, g, beta, **kw)
    return a, b, c


# ----------------------------------------------------------------- fixtures
def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("ex", _golden(), ids=lambda e: e["name"])
def test_hand_worked_examples(ex):
    """Hand-derived steps; catches a wrong read (undecayed S), a transposed
    state, reading o before the write, a gate on the wrong axis of S."""
    q, k, v = (np.array(ex[n], dtype=np.float64) for n in ("q", "k", "v"))
    beta = np.array(ex["beta"], dtype=np.float64)
    g = np.log(np.array(ex["alpha"], dtype=np.float64))
    S0 = np.array(ex["S0"], dtype=np.float64)
    kw = dict(S0=S0, per_head_gate=ex["per_head_gate"])
    for chunk in (1, 2, 64):
        for o, S in _all_forms(q, k, v, g, beta, chunk=chunk, **kw):
            np.testing.assert_allclose(o, ex["o"], rtol=0, atol=1e-12)
            np.testing.assert_allclose(S, ex["S_T"], rtol=0, atol=1e-12)


# ------------------------------------------------- closed-form special cases
def test_zero_change_when_value_already_stored():
    """Delta rule: if v_t equals what the (decayed) state already returns for
    k_t, the state only decays.  Catches reading the undecayed state or
    writing v instead of the difference."""
    rng = np.random.default_rng(1)
    H, dk, dv = 2, 6, 5
    S = rng.standard_normal((1, H, dk, dv))
    for step in range(5):
        q, k, _, g, beta, _ = _rand(rng, 1, H, dk, dv, s0=False)
        a = np.exp(g[0])                                  # [H, dk]
        decayed = a[None, :, :, None] * S                 # Diag(a) S
        v = np.einsum("nhcj,hc->hj", decayed, k[0])[None]  # what k reads now
        o, S_T = oracle.recurrence(q, k, v, g, beta, S0=S)
        np.testing.assert_allclose(S_T, decayed, rtol=0, atol=1e-13)
        np.testing.assert_allclose(o[0], np.einsum("nhcj,hc->hj", decayed, q[0]), atol=1e-13)
        S = S_T


def test_orthonormal_overwrite_and_rewrite():
    """beta=1, no decay, keys = rows of an orthogonal matrix: after writing
    every key once the state retrieves exactly v_i for k_i whatever S0 was
    (S_T = K^T V); rewriting one key changes only that key's value."""
    rng = np.random.default_rng(2)
    d, dv, H = 8, 5, 1
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    K = Qm.T                                               # rows orthonormal
    V = rng.standard_normal((d, dv))
    S0 = rng.standard_normal((1, H, d, dv))
    k = K[:, None, :]
    q = k.copy()                                           # read back the key just written
    v = V[:, None, :]
    g = np.zeros((d, H, d))
    beta = np.ones((d, H))
    o, S_T = oracle.recurrence(q, k, v, g, beta, S0=S0)
    np.testing.assert_allclose(S_T[0, 0], K.T @ V, atol=1e-12)
    np.testing.assert_allclose(o[:, 0], V, atol=1e-12)    # o_t = v_t right after the write
    # rewrite key 3 with a new value
    vnew = rng.standard_normal((1, H, dv))
    o2, S2 = oracle.recurrence(K[3][None, None], K[3][None, None], vnew, np.zeros((1, H, d)),
                               np.ones((1, H)), S0=S_T)
    R = K @ S2[0, 0]
    np.testing.assert_allclose(R[3], vnew[0, 0], atol=1e-12)
    np.testing.assert_allclose(np.delete(R, 3, 0), np.delete(V, 3, 0), atol=1e-12)


@pytest.mark.parametrize("with_s0", [False, True])
def test_reduces_to_linear_attention_with_orthogonal_keys(with_s0):
    """alpha = 1 and mutually orthonormal keys: the erase term only ever sees
    S0, so O = Q S0 + tril(Q K^T) U with U = diag(beta)(V - K S0), and with
    S0 = 0 this is additive linear attention (identity feature map).  Catches
    a wrong causal mask (strict vs inclusive), a lost beta, a wrong sign."""
    rng = np.random.default_rng(3)
    T, d, dv = 7, 9, 4
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    K = Qm[:T]                                             # T orthonormal rows
    Q = rng.standard_normal((T, d))
    V = rng.standard_normal((T, dv))
    beta = rng.uniform(0.1, 1.0, T)
    S0 = rng.standard_normal((d, dv)) if with_s0 else np.zeros((d, dv))
    U = beta[:, None] * (V - K @ S0)
    O = Q @ S0 + np.tril(Q @ K.T) @ U
    ST = S0 + K.T @ U
    o, S_T = oracle.recurrence(Q[:, None], K[:, None], V[:, None], np.zeros((T, 1, d)),
                               beta[:, None], S0=S0[None, None])
    np.testing.assert_allclose(o[:, 0], O, atol=1e-12)
    np.testing.assert_allclose(S_T[0, 0], ST, atol=1e-12)


@pytest.mark.parametrize("per_head", [False, True])
def test_full_erase(per_head):
    """alpha = 0 (g = -inf) wipes the memory before each write:
    S_t = beta_t k_t v_t^T and o_t = beta_t (q_t . k_t) v_t."""
    rng = np.random.default_rng(4)
    T, H, dk, dv = 5, 2, 4, 3
    q, k, v, _, beta, S0 = _rand(rng, T, H, dk, dv)
    g = np.full((T, H) if per_head else (T, H, dk), -np.inf)
    o, S_T = oracle.recurrence(q, k, v, g, beta, S0=S0, per_head_gate=per_head)
    exp_o = beta[:, :, None] * np.sum(q * k, axis=-1)[:, :, None] * v
    np.testing.assert_allclose(o, exp_o, atol=1e-13)
    exp_S = beta[-1][:, None, None] * k[-1][:, :, None] * v[-1][:, None, :]
    np.testing.assert_allclose(S_T[0], exp_S, atol=1e-13)


@pytest.mark.parametrize("per_head", [False, True])
def test_decay_horizon(per_head):
    """beta = 0 leaves only the forgetting: S_t = Diag(prod_{tau<=t} a_tau) S0,
    so o_t = S0^T (q_t * prod a).  Catches an off-by-one in the decay
    product, decay along d_v instead of d_k, or a decay applied after o."""
    rng = np.random.default_rng(5)
    T, H, dk, dv = 9, 2, 5, 3
    q, k, v, g, _, S0 = _rand(rng, T, H, dk, dv, per_head=per_head)
    beta = np.zeros((T, H))
    o, S_T = oracle.recurrence(q, k, v, g, beta, S0=S0, per_head_gate=per_head)
    a = np.exp(g if not per_head else np.repeat(g[:, :, None], dk, axis=2))
    P = np.cumprod(a, axis=0)                              # [T, H, dk]
    exp_o = np.einsum("hcj,thc->thj", S0[0], q * P)
    np.testing.assert_allclose(o, exp_o, atol=1e-13)
    np.testing.assert_allclose(S_T[0], P[-1][:, :, None] * S0[0], atol=1e-13)


def test_alpha_one_is_deltanet_fixed_point():
    """alpha = 1, beta = 1, repeating the same unit key and value: after the
    first write the state stops changing (delta = 0), and retrieval returns
    v.  Catches a decay leaking in when g = 0."""
    rng = np.random.default_rng(6)
    d, dv = 6, 4
    k1 = rng.standard_normal(d)
    k1 /= np.linalg.norm(k1)
    v1 = rng.standard_normal(dv)
    T = 4
    k = np.tile(k1, (T, 1, 1))
    v = np.tile(v1, (T, 1, 1))
    S0 = rng.standard_normal((1, 1, d, dv))
    o, S_T = oracle.recurrence(k, k, v, np.zeros((T, 1, d)), np.ones((T, 1)), S0=S0)
    np.testing.assert_allclose(o[:, 0], np.tile(v1, (T, 1)), atol=1e-12)
    o1, S1 = oracle.recurrence(k[:1], k[:1], v[:1], np.zeros((1, 1, d)), np.ones((1, 1)), S0=S0)
    np.testing.assert_allclose(S_T, S1, atol=1e-12)


# --------------------------------------------------- exact rational brute force
def _frac_product_form(q, k, v, alpha, beta, S0):
    """S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T, exact rationals."""
    dk, dv = len(S0), len(S0[0])
    S = [row[:] for row in S0]
    outs = []
    for t in range(len(q)):
        a, kt, vt, qt, b = alpha[t], k[t], v[t], q[t], beta[t]
        D = [[a[c] * S[c][j] for j in range(dv)] for c in range(dk)]
        M = [[(1 if c == e else 0) - b * kt[c] * kt[e] for e in range(dk)] for c in range(dk)]
        S = [[sum(M[c][e] * D[e][j] for e in range(dk)) + b * kt[c] * vt[j] for j in range(dv)]
             for c in range(dk)]
        outs.append([sum(S[c][j] * qt[c] for c in range(dk)) for j in range(dv)])
    return outs, S


@pytest.mark.parametrize("seed", range(6))
def test_exact_rational_product_form(seed):
    """Tiny cases (T <= 3, d <= 3) computed exactly in rationals from the
    product form of the transition; alpha is a power of two so exp(ln alpha)
    is exact to an ulp."""
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(1, 4))
    dk, dv = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    fr = lambda x: Fraction(int(x), 4)
    qi = rng.integers(-4, 5, (T, dk))
    ki = rng.integers(-4, 5, (T, dk))
    vi = rng.integers(-4, 5, (T, dv))
    si = rng.integers(-4, 5, (dk, dv))
    bi = rng.integers(0, 5, T)
    ai = rng.integers(0, 4, (T, dk))                          # alpha = 2^-ai
    q = [[fr(x) for x in r] for r in qi]
    k = [[fr(x) for x in r] for r in ki]
    v = [[fr(x) for x in r] for r in vi]
    S0 = [[fr(x) for x in r] for r in si]
    beta = [fr(x) for x in bi]
    alpha = [[Fraction(1, 2 ** int(x)) for x in r] for r in ai]
    outs, S = _frac_product_form(q, k, v, alpha, beta, S0)
    f = lambda a: np.array(a, dtype=np.float64)
    o, S_T = oracle.recurrence(f(qi / 4)[:, None], f(ki / 4)[:, None], f(vi / 4)[:, None],
                               (-ai * math.log(2.0))[:, None, :].astype(np.float64),
                               f(bi / 4)[:, None], S0=f(si / 4)[None, None])
    np.testing.assert_allclose(o[:, 0], f([[float(x) for x in r] for r in outs]), atol=1e-12)
    np.testing.assert_allclose(S_T[0, 0], f([[float(x) for x in r] for r in S]), atol=1e-12)


# ----------------------------------------------- three formulations agree
@settings(max_examples=40, deadline=None)
@given(T=st.integers(1, 150), dk=st.integers(1, 12), dv=st.integers(1, 12),
       chunk=st.sampled_from([1, 3, 16, 64]), per_head=st.booleans(),
       seed=st.integers(0, 2 ** 31))
def test_sequential_chunked_dplr_agree(T, dk, dv, chunk, per_head, seed):
    """The sequential recurrence, the chunk algebra (any C, ragged last
    chunk) and the explicit DPLR product agree to fp64 rounding."""
    rng = np.random.default_rng(seed)
    q, k, v, g, beta, S0 = _rand(rng, T, 2, dk, dv, per_head=per_head)
    (o1, s1), (o2, s2), (o3, s3) = _all_forms(q, k, v, g, beta, S0=S0, chunk=chunk,
                                              per_head_gate=per_head)
    for o, s in ((o2, s2), (o3, s3)):
        assert oracle.rel_err(o, o1) < 1e-11
        assert oracle.rel_err(s, s1) < 1e-11


@pytest.mark.parametrize("per_head", [False, True])
def test_chunked_c128_agrees(per_head):
    """The chunk algebra at C = 128, the other chunk size the pages name
    (three chunks, the last ragged), agrees with the sequential recurrence."""
    rng = np.random.default_rng(128 + per_head)
    q, k, v, g, beta, S0 = _rand(rng, 300, 2, 8, 6, per_head=per_head)
    (o1, s1), (o2, s2), (o3, s3) = _all_forms(q, k, v, g, beta, S0=S0, chunk=128, per_head_gate=per_head)
    for o, s in ((o2, s2), (o3, s3)):
        assert oracle.rel_err(o, o1) < 1e-11
        assert oracle.rel_err(s, s1) < 1e-11


def test_varlen_equals_separate_sequences_and_empty():
    """Packed sequences never mix; an empty sequence returns S0 unchanged."""
    rng = np.random.default_rng(7)
    lens = [5, 0, 17, 1, 64, 70]
    T = sum(lens)
    H, dk, dv = 2, 5, 4
    q, k, v, g, beta, _ = _rand(rng, T, H, dk, dv, s0=False)
    S0 = rng.standard_normal((len(lens), H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, S_T = oracle.recurrence(q, k, v, g, beta, S0=S0, cu_seqlens=cu)
    oc, Sc = oracle.chunked(q, k, v, g, beta, S0=S0, cu_seqlens=cu, chunk=16)
    assert oracle.rel_err(oc, o) < 1e-12 and oracle.rel_err(Sc, S_T) < 1e-12
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        if e == s:
            np.testing.assert_array_equal(S_T[n], S0[n])
            continue
        on, Sn = oracle.recurrence(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e], S0=S0[n:n + 1])
        np.testing.assert_array_equal(o[s:e], on)
        np.testing.assert_array_equal(S_T[n], Sn[0])


def test_split_invariance_and_sampled_rows():
    """Two calls chained through S_T equal one call (the state is the whole
    memory); recording a sample of rows returns the same rows."""
    rng = np.random.default_rng(8)
    T, H, dk, dv = 40, 2, 6, 5
    q, k, v, g, beta, S0 = _rand(rng, T, H, dk, dv)
    o, S = oracle.recurrence(q, k, v, g, beta, S0=S0)
    o1, S1 = oracle.recurrence(q[:13], k[:13], v[:13], g[:13], beta[:13], S0=S0)
    o2, S2 = oracle.recurrence(q[13:], k[13:], v[13:], g[13:], beta[13:], S0=S1)
    np.testing.assert_array_equal(np.concatenate([o1, o2]), o)
    np.testing.assert_array_equal(S2, S)
    pos = [0, 3, 13, 39]
    os_, Ss = oracle.recurrence(q, k, v, g, beta, S0=S0, o_positions=pos)
    np.testing.assert_array_equal(os_, o[pos])
    np.testing.assert_array_equal(Ss, S)


def test_linearity_in_values_and_state():
    """For fixed q, k, g, beta the map (V, S0) -> (o, S_T) is linear."""
    rng = np.random.default_rng(9)
    T, H, dk, dv = 30, 2, 5, 4
    q, k, v1, g, beta, s1 = _rand(rng, T, H, dk, dv)
    v2 = rng.standard_normal(v1.shape)
    s2 = rng.standard_normal(s1.shape)
    c = -1.7
    oa, Sa = oracle.recurrence(q, k, v1, g, beta, S0=s1)
    ob, Sb = oracle.recurrence(q, k, v2, g, beta, S0=s2)
    oc, Sc = oracle.recurrence(q, k, v1 + c * v2, g, beta, S0=s1 + c * s2)
    np.testing.assert_allclose(oc, oa + c * ob, atol=1e-12)
    np.testing.assert_allclose(Sc, Sa + c * Sb, atol=1e-12)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_input_widening_is_exact(dtype):
    """The C oracle's bf16 / fp32 decoding gives bit-identical results to
    feeding the same values already widened to fp64 by numpy."""
    cfg = synth.small_chunk_config(H=2, dk=8, dv=6, dtype=dtype, seed=11)
    d = synth.chunk_inputs(cfg, lengths=[37, 20])
    o1, S1 = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"],
                               cu_seqlens=d["cu_seqlens"])
    w = [oracle.widen(d[n]) for n in ("q", "k", "v", "g", "beta")]
    if dtype == "bf16":
        ref = [synth.bf16_to_f32(d[n]).astype(np.float64) for n in ("q", "k", "v", "g", "beta")]
        for a, b in zip(w, ref):
            np.testing.assert_array_equal(a, b)
    o2, S2 = oracle.recurrence(*w, S0=d["S0"], cu_seqlens=d["cu_seqlens"])
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


def test_bf16_rounding_is_round_to_nearest_even():
    """Generator rounding: ties go to the even mantissa, others to nearest."""
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, -2.5],
                 dtype=np.float32)
    got = synth.bf16_to_f32(synth.bf16_bits(x))
    np.testing.assert_array_equal(got, np.array([1.0, 1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -2.5],
                                                dtype=np.float32))


# ------------------------------------------------------------ parity metric
# rel_err is the metric every GPU parity bound is stated in: the largest
# absolute deviation over the whole tensor divided by the largest magnitude of
# the reference.  Hand values, chosen so that a mean instead of a max, a
# denominator taken from `got`, an absolute error, a silently broadcast shape
# or a swallowed NaN each give a different number.
def test_rel_err_hand_values():
    # one element off by 2 against max|ref| = 4: 0.5 (a mean of |diff| would
    # give 1.0 / 4 = 0.25 or 1.0; dividing by max|got| = 2 would give 1.0)
    assert oracle.rel_err([1.0, 2.0], [1.0, 4.0]) == 0.5
    # the deviation is absolute: a sign flip of the largest element counts 2x
    assert oracle.rel_err([-3.0, 1.0], [3.0, 1.0]) == 2.0
    # max over every element, not the first or the last
    assert oracle.rel_err([[0.0, 0.0, 0.5], [2.0, 0.0, 0.0]],
                          [[0.0, 0.0, 0.0], [2.0, 0.0, 0.0]]) == 0.25
    # an all-zero reference falls back to the absolute max deviation
    assert oracle.rel_err([0.0, -0.125], [0.0, 0.0]) == 0.125
    # identical tensors and two empty tensors give exactly 0
    assert oracle.rel_err([1.5, -2.5], [1.5, -2.5]) == 0.0
    assert oracle.rel_err(np.zeros((0, 3)), np.zeros((0, 3))) == 0.0
    # the denominator is the reference's: scaling both by 10 changes nothing,
    # scaling only `got` does
    assert oracle.rel_err([10.0, 20.0], [10.0, 40.0]) == 0.5
    assert oracle.rel_err([2.0, 8.0], [1.0, 4.0]) == 1.0


def test_rel_err_rejects_shape_mismatch_and_non_finite():
    with pytest.raises(ValueError):
        oracle.rel_err(np.zeros(3), np.zeros((1, 3)))
    with pytest.raises(ValueError):
        oracle.rel_err(np.zeros(0), np.ones(2))
    assert oracle.rel_err([np.nan, 1.0], [1.0, 1.0]) == math.inf
    assert oracle.rel_err([np.inf, 1.0], [1.0, 1.0]) == math.inf
    assert oracle.rel_err([1.0, 1.0], [1.0, np.nan]) == math.inf

"""Pins for the gradient oracles (``oracle.grad.recurrence_grad``, autograd of
the sequential recurrence, and ``oracle.grad.adjoint``, the hand-written fp64
C adjoint).

These tests tie both to things that do not come from either:

* a one-token closed form, derived by hand from the transition
  S_1 = (I - beta k k^T) Diag(a) S_0 + beta k v^T, o = S_1^T q, with
  L = <dO, o> + <dS_T, S_1> = <G, S_1> and G = q dO^T + dS_T;
* central finite differences of the C forward oracle (a separate program) in
  every input element, for per-channel and per-head gates and two packed
  sequences;
* linearity of a vector-Jacobian product in its cotangents;
* for the adjoint at lengths autograd cannot reach (thousands of tokens,
  several checkpoint stretches), exact identities of the loss: L is linear in
  q (o_t = S_t^T q_t and the state does not depend on q) and jointly linear in
  (v, S0) (the state is), so L(x + d) - L(x) = <dL/dx, d> up to rounding, with
  L evaluated by the C forward oracle;
* the two implementations against each other on varied packed batches.

A dropped term, a wrong sign, a transposed operand or a gate applied after
the read in the oracle's update fails the finite-difference test; a mistake
in how the cotangents enter fails the closed form.
"""
import numpy as np
import pytest

import oracle
from oracle.grad import adjoint, recurrence_grad

GRADS = {"autograd": recurrence_grad, "adjoint": adjoint}


def _inputs(rng, T, H, dk, dv, N=1, per_head=False):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = -np.logaddexp(0.0, rng.standard_normal((T, H) if per_head else (T, H, dk)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    S0 = rng.standard_normal((N, H, dk, dv)) * 0.5
    return q, k, v, g, beta, S0


@pytest.mark.parametrize("impl", sorted(GRADS))
def test_one_token_closed_form(impl):
    """T = 1 per sequence: every gradient written out by hand."""
    rng = np.random.default_rng(11)
    H, dk, dv = 3, 5, 4
    lengths = [1, 1]
    T = sum(lengths)
    q, k, v, g, beta, S0 = _inputs(rng, T, H, dk, dv, N=len(lengths))
    dO = rng.standard_normal((T, H, dv))
    dST = rng.standard_normal((len(lengths), H, dk, dv))
    got = GRADS[impl](q, k, v, g, beta, dO, S0=S0, dS_T=dST, cu_seqlens=[0, 1, 2])
    for n in range(len(lengths)):
        for h in range(H):
            t = n
            a = np.exp(g[t, h])
            Sp = a[:, None] * S0[n, h]                 # decayed start state
            r = Sp.T @ k[t, h]
            u = beta[t, h] * (v[t, h] - r)
            S1 = Sp + np.outer(k[t, h], u)
            G = np.outer(q[t, h], dO[t, h]) + dST[n, h]
            Gk = G.T @ k[t, h]
            dSp = G - beta[t, h] * np.outer(k[t, h], Gk)
            want = {
                0: S1 @ dO[t, h],                                           # dq
                1: beta[t, h] * (G @ (v[t, h] - r) - Sp @ Gk),             # dk
                2: beta[t, h] * Gk,                                         # dv
                3: (dSp * Sp).sum(axis=1),                                  # dg
                4: Gk @ (v[t, h] - r),                                      # dbeta
            }
            for i, w in want.items():
                assert np.allclose(got[i][t, h], w, rtol=1e-12, atol=1e-12), i
            assert np.allclose(got[5][n, h], a[:, None] * dSp, rtol=1e-12, atol=1e-12)


def _loss(x, dO, dST, cu, per_head):
    q, k, v, g, beta, S0 = x
    o, S_T = oracle.recurrence(q, k, v, g, beta, S0=S0, cu_seqlens=cu, per_head_gate=per_head)
    return float((o * dO).sum() + (S_T * dST).sum())


@pytest.mark.parametrize("impl", sorted(GRADS))
@pytest.mark.parametrize("per_head", [False, True])
def test_finite_differences_of_forward_oracle(per_head, impl):
    """Every element of every input: central differences of the C oracle."""
    rng = np.random.default_rng(12 + per_head)
    cu = [0, 4, 9]
    T, H, dk, dv = 9, 2, 3, 2
    x = list(_inputs(rng, T, H, dk, dv, N=2, per_head=per_head))
    dO = rng.standard_normal((T, H, dv))
    dST = rng.standard_normal((2, H, dk, dv))
    grads = GRADS[impl](*x[:5], dO, S0=x[5], dS_T=dST, cu_seqlens=cu, per_head_gate=per_head)
    eps = 1e-6
    for i, (xi, gi) in enumerate(zip(x, grads)):
        assert gi.shape == xi.shape
        fd = np.zeros_like(xi)
        for idx in np.ndindex(xi.shape):
            keep = xi[idx]
            xi[idx] = keep + eps
            lp = _loss(x, dO, dST, cu, per_head)
            xi[idx] = keep - eps
            lm = _loss(x, dO, dST, cu, per_head)
            xi[idx] = keep
            fd[idx] = (lp - lm) / (2 * eps)
        scale = max(1.0, np.abs(gi).max())
        assert np.abs(fd - gi).max() <= 1e-7 * scale, (i, np.abs(fd - gi).max())


def test_linear_in_cotangents():
    rng = np.random.default_rng(13)
    T, H, dk, dv = 12, 2, 4, 3
    q, k, v, g, beta, S0 = _inputs(rng, T, H, dk, dv)
    dO1, dO2 = rng.standard_normal((2, T, H, dv))
    dS1, dS2 = rng.standard_normal((2, 1, H, dk, dv))
    g1 = recurrence_grad(q, k, v, g, beta, dO1, S0=S0, dS_T=dS1)
    g2 = recurrence_grad(q, k, v, g, beta, dO2, S0=S0, dS_T=dS2)
    g3 = recurrence_grad(q, k, v, g, beta, 2.0 * dO1 - 3.0 * dO2, S0=S0, dS_T=2.0 * dS1 - 3.0 * dS2)
    for a, b, c in zip(g1, g2, g3):
        assert np.allclose(c, 2.0 * a - 3.0 * b, rtol=1e-12, atol=1e-12)


def test_zero_length_sequence_passes_state_gradient_through():
    """An empty sequence has S_T = S0, so dS0 = dS_T exactly."""
    rng = np.random.default_rng(14)
    T, H, dk, dv = 5, 1, 3, 2
    q, k, v, g, beta, _ = _inputs(rng, T, H, dk, dv)
    S0 = rng.standard_normal((2, H, dk, dv))
    dO = rng.standard_normal((T, H, dv))
    dST = rng.standard_normal((2, H, dk, dv))
    got = recurrence_grad(q, k, v, g, beta, dO, S0=S0, dS_T=dST, cu_seqlens=[0, 0, 5])
    assert np.array_equal(got[5][0], dST[0])


@pytest.mark.parametrize("per_head", [False, True])
def test_adjoint_matches_autograd(per_head):
    """Packed sequences of assorted lengths (empty, one token, several
    checkpoint stretches, a ragged tail), with and without S0 and dS_T."""
    rng = np.random.default_rng(15 + per_head)
    lengths = [0, 1, 37, 300, 17]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T, H, dk, dv = int(cu[-1]), 2, 6, 5
    q, k, v, g, beta, S0 = _inputs(rng, T, H, dk, dv, N=len(lengths), per_head=per_head)
    dO = rng.standard_normal((T, H, dv))
    dST = rng.standard_normal((len(lengths), H, dk, dv))
    for s0, dst in ((S0, dST), (None, None)):
        a = adjoint(q, k, v, g, beta, dO, S0=s0, dS_T=dst, cu_seqlens=cu, per_head_gate=per_head)
        b = recurrence_grad(q, k, v, g, beta, dO, S0=s0, dS_T=dst, cu_seqlens=cu, per_head_gate=per_head)
        for x, y in zip(a, b):
            assert x.shape == y.shape
            assert oracle.rel_err(x, y) < 1e-12


def test_adjoint_exact_identities_at_length():
    """T = 3000 (about 55 checkpoint stretches): L is linear in q and jointly
    linear in (v, S0), so a finite step of any size changes L by exactly the
    inner product of the gradient with the step (up to fp64 rounding)."""
    rng = np.random.default_rng(16)
    T, H, dk, dv = 3000, 2, 8, 6
    q, k, v, g, beta, S0 = _inputs(rng, T, H, dk, dv)
    dO = rng.standard_normal((T, H, dv))
    dST = rng.standard_normal((1, H, dk, dv))
    dq, _, dv_, _, _, dS0 = adjoint(q, k, v, g, beta, dO, S0=S0, dS_T=dST)
    L0 = _loss([q, k, v, g, beta, S0], dO, dST, [0, T], False)
    Dq = rng.standard_normal(q.shape)
    Lq = _loss([q + Dq, k, v, g, beta, S0], dO, dST, [0, T], False)
    assert abs((Lq - L0) - (dq * Dq).sum()) <= 1e-9 * max(1.0, abs(Lq - L0))
    Dv, DS = rng.standard_normal(v.shape), rng.standard_normal(S0.shape)
    Lv = _loss([q, k, v + Dv, g, beta, S0 + DS], dO, dST, [0, T], False)
    want = (dv_ * Dv).sum() + (dS0 * DS).sum()
    assert abs((Lv - L0) - want) <= 1e-9 * max(1.0, abs(Lv - L0))


def test_adjoint_selected_rows_and_bf16_bits():
    """Gradients of selected tokens only, and bf16-bit inputs and cotangents,
    give the same values as the full computation on the widened inputs."""
    import synth
    rng = np.random.default_rng(17)
    T, H, dk, dv = 400, 2, 8, 8
    q, k, v, g, beta, S0 = _inputs(rng, T, H, dk, dv)
    bits = [synth.bf16_bits(x.astype(np.float32)) for x in (q, k, v, g, beta)]
    dO = synth.bf16_bits(rng.standard_normal((T, H, dv)).astype(np.float32))
    full = adjoint(*bits, dO, S0=S0)
    wide = adjoint(*(oracle.widen(b) for b in bits), oracle.widen(dO), S0=S0)
    for x, y in zip(full, wide):
        assert np.array_equal(x, y)
    pos = np.array([0, 5, 63, 64, 399])
    part = adjoint(*bits, dO, S0=S0, positions=pos)
    for x, y in zip(part[:5], full[:5]):
        assert np.array_equal(x, y[pos])
    assert np.array_equal(part[5], full[5])

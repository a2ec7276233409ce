"""Pins for the gradient oracle (``oracle.grad.recurrence_grad``).

The gradient oracle differentiates the sequential recurrence with autograd.
These tests tie it to things that do not come from that tape:

* a one-token closed form, derived by hand from the transition
  S_1 = (I - beta k k^T) Diag(a) S_0 + beta k v^T, o = S_1^T q, with
  L = <dO, o> + <dS_T, S_1> = <G, S_1> and G = q dO^T + dS_T;
* central finite differences of the C forward oracle (a separate program) in
  every input element, for per-channel and per-head gates and two packed
  sequences;
* linearity of a vector-Jacobian product in its cotangents.

A dropped term, a wrong sign, a transposed operand or a gate applied after
the read in the oracle's update fails the finite-difference test; a mistake
in how the cotangents enter fails the closed form.
"""
import numpy as np
import pytest

import oracle
from oracle.grad import recurrence_grad


def _inputs(rng, T, H, dk, dv, N=1, per_head=False):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = -np.logaddexp(0.0, rng.standard_normal((T, H) if per_head else (T, H, dk)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    S0 = rng.standard_normal((N, H, dk, dv)) * 0.5
    return q, k, v, g, beta, S0


def test_one_token_closed_form():
    """T = 1 per sequence: every gradient written out by hand."""
    rng = np.random.default_rng(11)
    H, dk, dv = 3, 5, 4
    lengths = [1, 1]
    T = sum(lengths)
    q, k, v, g, beta, S0 = _inputs(rng, T, H, dk, dv, N=len(lengths))
    dO = rng.standard_normal((T, H, dv))
    dST = rng.standard_normal((len(lengths), H, dk, dv))
    got = recurrence_grad(q, k, v, g, beta, dO, S0=S0, dS_T=dST, cu_seqlens=[0, 1, 2])
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


@pytest.mark.parametrize("per_head", [False, True])
def test_finite_differences_of_forward_oracle(per_head):
    """Every element of every input: central differences of the C oracle."""
    rng = np.random.default_rng(12 + per_head)
    cu = [0, 4, 9]
    T, H, dk, dv = 9, 2, 3, 2
    x = list(_inputs(rng, T, H, dk, dv, N=2, per_head=per_head))
    dO = rng.standard_normal((T, H, dv))
    dST = rng.standard_normal((2, H, dk, dv))
    grads = recurrence_grad(*x[:5], dO, S0=x[5], dS_T=dST, cu_seqlens=cu, per_head_gate=per_head)
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

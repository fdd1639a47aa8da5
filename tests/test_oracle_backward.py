"""Pins of the fp64 oracle's backward: hand-worked values, finite differences,
a library autograd and conservation invariants."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention_backward, attention_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked_attention.json")


def _ev(expr):
    return float(eval(expr, {"__builtins__": {}}, {"log": math.log}))


def _mat(rows):
    return np.array([[_ev(x) for x in r] for r in rows])


@pytest.mark.parametrize("causal", [False, True])
def test_handworked_backward(causal):
    g = json.load(open(GOLDEN))
    q, k, v, do = (_mat(g[x]) for x in ("q", "k", "v", "dout"))
    dq, dk, dv = attention_backward(q, k, v, do, causal=causal, scale=g["scale"])
    np.testing.assert_allclose(dq, _mat(g["backward"]["dq"]), atol=1e-13)
    np.testing.assert_allclose(dk, _mat(g["backward"]["dk"]), atol=1e-13)
    np.testing.assert_allclose(dv, _mat(g["backward"]["dv"]), atol=1e-13)


def _loss(q, k, v, do, causal, scale):
    o, _ = attention_forward(q, k, v, causal=causal, scale=scale)
    return float((o * do).sum())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 5, 16])
def test_finite_differences(rng, causal, n):
    d, scale, h = 4, 0.8, 1e-6
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    grads = attention_backward(q, k, v, do, causal=causal, scale=scale)
    for which, g in zip(range(3), grads):
        num = np.zeros_like(g)
        for idx in np.ndindex(g.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            num[idx] = (_loss(*args_p, do, causal, scale) - _loss(*args_m, do, causal, scale)) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd_fp64(rng, causal):
    B, H, n, d = 1, 2, 29, 8
    scale = 1 / math.sqrt(d)
    q, k, v, do = (rng.standard_normal((B, H, n, d)) for _ in range(4))
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    o.backward(torch.from_numpy(do))
    dq, dk, dv = attention_backward(q, k, v, do, causal=causal, scale=scale)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_conservation(rng, causal):
    n, d = 40, 8
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    dq, dk, dv = attention_backward(q, k, v, do, causal=causal, scale=0.4, row_block=7)
    # Each probability row sums to one, so the value gradients sum to dO's sum
    # and the score gradients of a row sum to zero, hence sum_j dK_j = 0.
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    if causal:
        np.testing.assert_allclose(dq[0], 0.0, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_saved_output_path(rng, causal):
    """The `out` form of the backward (D_i = sum_d dO_id out_id): with the exact
    forward output it equals the default form (D_i = sum_j P_ij dP_ij, the same
    number since O_i = sum_j P_ij V_j); with one entry of one output row moved by
    eps, the gradients move by the closed form of dS changing by -P_ij·dO_ic·eps
    in row i alone: dQ_i by -scale·dO_ic·eps·sum_j P_ij K_j, dK_j by
    -scale·dO_ic·eps·P_ij·Q_i, dV not at all."""
    n, d, scale, eps = 11, 6, 0.7, 1e-3
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    o, _ = attention_forward(q, k, v, causal=causal, scale=scale)
    base = attention_backward(q, k, v, do, causal=causal, scale=scale)
    same = attention_backward(q, k, v, do, causal=causal, scale=scale, out=o)
    for a, b in zip(base, same):
        np.testing.assert_allclose(b, a, rtol=0, atol=1e-12)
    i, c = 7, 2
    o2 = o.copy()
    o2[i, c] += eps
    dq2, dk2, dv2 = attention_backward(q, k, v, do, causal=causal, scale=scale, out=o2)
    s = scale * (q @ k.T)
    if causal:
        s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dD = do[i, c] * eps
    want_dq = base[0].copy()
    want_dq[i] -= scale * dD * (p[i] @ k)
    want_dk = base[1] - scale * dD * p[i][:, None] * q[i][None, :]
    np.testing.assert_allclose(dq2, want_dq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk2, want_dk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv2, base[2], rtol=0, atol=1e-14)

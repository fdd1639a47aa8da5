"""Pins of the fp64 oracle's forward against facts the definition fixes.

None of these re-types the oracle's formula: each checks a hand-worked
example, a closed form, an invariant, a special case or a library routine.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import attention_forward, attention_forward_rows, online_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked_attention.json")


def _ev(expr: str) -> float:
    """Evaluate the tiny closed-form expressions of the golden file."""
    return float(eval(expr, {"__builtins__": {}}, {"log": math.log, "Fraction": Fraction}))


def _mat(rows):
    return np.array([[_ev(x) for x in r] for r in rows], dtype=np.float64)


def _vec(xs):
    return np.array([_ev(x) for x in xs], dtype=np.float64)


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("causal", [False, True])
def test_handworked_forward(golden, causal):
    q, k, v = _mat(golden["q"]), _mat(golden["k"]), _mat(golden["v"])
    o, lse = attention_forward(q, k, v, causal=causal, scale=golden["scale"])
    ref = golden["causal" if causal else "noncausal"]
    np.testing.assert_allclose(o, _mat(ref["o"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, _vec(ref["lse"]), rtol=0, atol=1e-13)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_identity_v_exposes_probabilities(rng, causal):
    # With V = I (one-hot value columns) O is the probability matrix itself.
    n = 24
    q, k = _rand(rng, n, 8), _rand(rng, n, 8)
    p, _ = attention_forward(q, k, np.eye(n), causal=causal, scale=0.7)
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
    if causal:
        assert np.all(np.triu(p, 1) == 0.0)
        assert np.all(np.diag(p) > 0)
    # Ratios of probabilities in one row are exp of score differences.
    s = 0.7 * q @ k.T
    i = n - 1
    np.testing.assert_allclose(p[i, 1:] / p[i, 0], np.exp(s[i, 1:] - s[i, 0]), rtol=1e-11)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_gives_constant_output(rng, causal):
    n, d = 33, 16
    c = _rand(rng, d)
    o, _ = attention_forward(_rand(rng, 2, n, d), _rand(rng, 2, n, d), np.broadcast_to(c, (2, n, d)),
                             causal=causal)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), atol=1e-12)


def test_single_key_returns_its_value(rng):
    q, k, v = _rand(rng, 5, 1, 8), _rand(rng, 5, 1, 8), _rand(rng, 5, 1, 8)
    for causal in (False, True):
        o, lse = attention_forward(q, k, v, causal=causal, scale=0.3)
        np.testing.assert_allclose(o, v, atol=1e-14)
        np.testing.assert_allclose(lse[..., 0], 0.3 * np.einsum("hd,hd->h", q[:, 0], k[:, 0]), atol=1e-13)


def test_causal_row0_and_last_row(rng):
    n, d = 40, 16
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    o, lse = attention_forward(q, k, v, causal=True, scale=0.25)
    np.testing.assert_allclose(o[0], v[0], atol=1e-14)
    np.testing.assert_allclose(lse[0], 0.25 * q[0] @ k[0], atol=1e-13)
    # The last causal row sees every key, so it equals the non-causal last row.
    o2, lse2 = attention_forward(q, k, v, causal=False, scale=0.25)
    np.testing.assert_allclose(o[-1], o2[-1], atol=1e-13)
    np.testing.assert_allclose(lse[-1], lse2[-1], atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_is_uniform_average(rng, causal):
    n, d = 17, 8
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    o, lse = attention_forward(q, k, v, causal=causal, scale=0.0)
    counts = np.arange(1, n + 1) if causal else np.full(n, n)
    ref = (np.cumsum(v, axis=0) / counts[:, None]) if causal else np.broadcast_to(v.mean(0), (n, d))
    np.testing.assert_allclose(o, ref, atol=1e-13)
    np.testing.assert_allclose(lse, np.log(counts), atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_moves_lse_only(rng, causal):
    n, d = 20, 8
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    c = _rand(rng, d)
    o1, l1 = attention_forward(q, k, v, causal=causal, scale=0.5)
    o2, l2 = attention_forward(q, k + c, v, causal=causal, scale=0.5)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, 0.5 * q @ c, atol=1e-12)


def test_permutations_noncausal(rng):
    n, d = 19, 8
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    o, lse = attention_forward(q, k, v)
    pk = rng.permutation(n)
    o2, lse2 = attention_forward(q, k[pk], v[pk])
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, atol=1e-13)
    pq = rng.permutation(n)
    o3, lse3 = attention_forward(q[pq], k, v)
    np.testing.assert_allclose(o3, o[pq], atol=1e-13)
    np.testing.assert_allclose(lse3, lse[pq], atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tile", [1, 3, 16, 64])
def test_online_equals_two_pass(rng, causal, tile):
    n, d = 45, 12
    q, k, v = _rand(rng, 2, n, d), _rand(rng, 2, n, d), _rand(rng, 2, n, d)
    o1, l1 = attention_forward(q, k, v, causal=causal, scale=0.9)
    o2, l2 = online_forward(q, k, v, causal=causal, scale=0.9, tile=tile)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2, l1, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_fp64(rng, causal):
    B, H, n, d = 2, 3, 37, 16
    q, k, v = (_rand(rng, B, H, n, d) for _ in range(3))
    scale = 1.0 / math.sqrt(d)
    o, lse = attention_forward(q, k, v, causal=causal, scale=scale)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)
    s = scale * (tq @ tk.transpose(-1, -2))
    if causal:
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12)


def test_rows_subset_matches_full(rng):
    n, d = 50, 8
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    rows = np.array([0, 7, 31, 49])
    o, lse = attention_forward(q, k, v, causal=True)
    o2, lse2 = attention_forward_rows(q, k, v, rows, causal=True)
    np.testing.assert_allclose(o2, o[rows], atol=1e-14)
    np.testing.assert_allclose(lse2, lse[rows], atol=1e-14)


def test_row_blocks_do_not_change_result(rng):
    n, d = 70, 8
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    a = attention_forward(q, k, v, causal=True, row_block=1024)
    b = attention_forward(q, k, v, causal=True, row_block=9)
    np.testing.assert_allclose(a[0], b[0], atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], atol=1e-14)


def test_empty_sequence():
    z = np.zeros((1, 2, 0, 8))
    o, lse = attention_forward(z, z, z, causal=True)
    assert o.shape == (1, 2, 0, 8) and lse.shape == (1, 2, 0)


def test_large_scores_stay_finite(rng):
    # exp of the raw scores would overflow fp64; the max subtraction must not.
    n, d = 16, 4
    q, k, v = 40 * _rand(rng, n, d), 40 * _rand(rng, n, d), _rand(rng, n, d)
    o, lse = attention_forward(q, k, v, scale=10.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    s = 10.0 * q @ k.T
    np.testing.assert_allclose(o, v[np.argmax(s, axis=1)], atol=1e-6)

"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them: the pins are strong enough to trust the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle.attention as A


def _sdpa_pin(causal):
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((1, 2, 9, 4)) for _ in range(3))
    o, lse = A.attention_forward(q, k, v, causal=causal, scale=0.5)
    t = [torch.from_numpy(x) for x in (q, k, v)]
    ref = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=causal, scale=0.5).numpy()
    s = 0.5 * (t[0] @ t[1].transpose(-1, -2))
    if causal:
        s = s.masked_fill(torch.ones(9, 9, dtype=torch.bool).triu(1), float("-inf"))
    return np.allclose(o, ref, atol=1e-10) and np.allclose(lse, torch.logsumexp(s, -1).numpy(), atol=1e-10)


def _bwd_pin(causal):
    rng = np.random.default_rng(6)
    q, k, v, do = (rng.standard_normal((1, 1, 7, 4)) for _ in range(4))
    t = [torch.from_numpy(x).requires_grad_() for x in (q, k, v)]
    torch.nn.functional.scaled_dot_product_attention(*t, is_causal=causal, scale=0.5).backward(torch.from_numpy(do))
    g = A.attention_backward(q, k, v, do, causal=causal, scale=0.5)
    return all(np.allclose(a, b.grad.numpy(), atol=1e-10) for a, b in zip(g, t))


def _all_pins():
    return all(f(c) for f in (_sdpa_pin, _bwd_pin) for c in (False, True))


MUTATIONS = {
    "scale dropped": ("_scores", lambda q, k, scale: q @ k.T),
    "keys transposed into queries": ("_scores", lambda q, k, scale: scale * (q @ q[: k.shape[0]].T)
                                     if q.shape[0] >= k.shape[0] else scale * (k[: q.shape[0]] @ k.T)),
    "mask hides the diagonal": ("_mask", lambda s, rows, causal: np.where(
        np.arange(s.shape[1])[None] >= rows[:, None], -np.inf, s) if causal else s),
    "mask reversed": ("_mask", lambda s, rows, causal: np.where(
        np.arange(s.shape[1])[None] < rows[:, None], -np.inf, s) if causal else s),
    "mask ignored": ("_mask", lambda s, rows, causal: s),
    "softmax not normalised": ("_softmax_rows", lambda s: (np.exp(s - s.max(1, keepdims=True)),
                                                           s.max(1) + np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)))),
    "lse without max": ("_softmax_rows", lambda s: (np.exp(s - s.max(1, keepdims=True)) / np.exp(s - s.max(1, keepdims=True)).sum(1, keepdims=True),
                                                    np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)))),
    "dS sign flipped": ("_dscores", lambda p, dp, D=None: -p * (dp - ((p * dp).sum(1) if D is None else D)[:, None])),
    "dS drops D": ("_dscores", lambda p, dp, D=None: p * dp),
}


def test_unmutated_oracle_passes_pins():
    assert _all_pins()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(monkeypatch, name):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(A, attr, fn)
    with np.errstate(all="ignore"):
        assert not _all_pins(), f"mutation '{name}' slipped past the pins"

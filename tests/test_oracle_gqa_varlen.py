"""Pins of the oracle's grouped-head and packed variable-length forms: torch
SDPA's own GQA path (a library routine), independent per-head and
per-sequence loops over the pinned dense functions, and finite differences."""
import math

import numpy as np
import pytest
import torch

from oracle import (attention_backward, attention_backward_gqa, attention_backward_varlen, attention_forward,
                    attention_forward_gqa, attention_forward_varlen)


def _r(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv", [(4, 1), (4, 2), (6, 3), (4, 4)])
def test_gqa_forward_matches_torch(rng, causal, H, Hkv):
    B, N, d = 2, 23, 8
    q, k, v = _r(rng, B, H, N, d), _r(rng, B, Hkv, N, d), _r(rng, B, Hkv, N, d)
    o, lse = attention_forward_gqa(q, k, v, causal=causal, scale=0.4)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v)), is_causal=causal, scale=0.4, enable_gqa=True)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)
    for h in range(H):  # per-head loop over the pinned dense forward
        oh, lh = attention_forward(q[:, h], k[:, h // (H // Hkv)], v[:, h // (H // Hkv)], causal=causal, scale=0.4)
        np.testing.assert_allclose(o[:, h], oh, atol=1e-13)
        np.testing.assert_allclose(lse[:, h], lh, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_backward_matches_torch_autograd(rng, causal):
    B, H, Hkv, N, d = 1, 6, 2, 17, 8
    q, k, v, do = _r(rng, B, H, N, d), _r(rng, B, Hkv, N, d), _r(rng, B, Hkv, N, d), _r(rng, B, H, N, d)
    t = [torch.from_numpy(x).requires_grad_() for x in (q, k, v)]
    torch.nn.functional.scaled_dot_product_attention(*t, is_causal=causal, scale=0.3, enable_gqa=True).backward(
        torch.from_numpy(do))
    g = attention_backward_gqa(q, k, v, do, causal=causal, scale=0.3)
    for a, b in zip(g, t):
        np.testing.assert_allclose(a, b.grad.numpy(), atol=1e-12)


def test_gqa_backward_finite_differences(rng):
    B, H, Hkv, N, d, h_ = 1, 4, 2, 5, 3, 1e-6
    q, k, v, do = _r(rng, B, H, N, d), _r(rng, B, Hkv, N, d), _r(rng, B, Hkv, N, d), _r(rng, B, H, N, d)
    gk = attention_backward_gqa(q, k, v, do, causal=True, scale=0.7)[1]
    num = np.zeros_like(k)
    for idx in np.ndindex(k.shape):
        kp, km = k.copy(), k.copy()
        kp[idx] += h_
        km[idx] -= h_
        lp = (attention_forward_gqa(q, kp, v, causal=True, scale=0.7)[0] * do).sum()
        lm = (attention_forward_gqa(q, km, v, causal=True, scale=0.7)[0] * do).sum()
        num[idx] = (lp - lm) / (2 * h_)
    np.testing.assert_allclose(gk, num, rtol=1e-6, atol=1e-7)


def _packed(rng, lens, H, Hkv, d):
    total = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return cu, _r(rng, total, H, d), _r(rng, total, Hkv, d), _r(rng, total, Hkv, d), _r(rng, total, H, d)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_forward_is_per_sequence_dense(rng, causal):
    lens = [5, 1, 0, 19, 8]
    cu, q, k, v, _ = _packed(rng, lens, 4, 2, 8)
    o, lse = attention_forward_varlen(q, k, v, cu, causal=causal, scale=0.5)
    for b, L in enumerate(lens):
        t0 = cu[b]
        for h in range(4):
            tq = torch.from_numpy(q[t0:t0 + L, h])[None]
            tk = torch.from_numpy(k[t0:t0 + L, h // 2])[None]
            tv = torch.from_numpy(v[t0:t0 + L, h // 2])[None]
            if L == 0:
                continue
            ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.5)
            np.testing.assert_allclose(o[t0:t0 + L, h], ref[0].numpy(), atol=1e-12)
            s = 0.5 * (tq[0] @ tk[0].T)
            if causal:
                s = s.masked_fill(torch.ones(L, L, dtype=torch.bool).triu(1), float("-inf"))
            np.testing.assert_allclose(lse[h, t0:t0 + L], torch.logsumexp(s, -1).numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_backward_is_per_sequence_dense(rng, causal):
    lens = [7, 3, 12]
    cu, q, k, v, do = _packed(rng, lens, 2, 1, 4)
    dq, dk, dv = attention_backward_varlen(q, k, v, do, cu, causal=causal, scale=0.6)
    for b, L in enumerate(lens):
        t0 = cu[b]
        for h in range(2):
            gq, gk, gv = attention_backward(q[t0:t0 + L, h], k[t0:t0 + L, 0], v[t0:t0 + L, 0], do[t0:t0 + L, h],
                                            causal=causal, scale=0.6)
            np.testing.assert_allclose(dq[t0:t0 + L, h], gq, atol=1e-13)
        # the single key/value head gathers both query heads' gradients
        gk = sum(attention_backward(q[t0:t0 + L, h], k[t0:t0 + L, 0], v[t0:t0 + L, 0], do[t0:t0 + L, h],
                                    causal=causal, scale=0.6)[1] for h in range(2))
        np.testing.assert_allclose(dk[t0:t0 + L, 0], gk, atol=1e-12)

"""Pins of the fp64 oracle's paged chunked prefill: reduction to the dense
causal forward (no prefix), to paged decode row by row (each query of a
chunk is a decode step over the keys it may see), to torch SDPA with an
explicit mask, and the empty-row convention."""
import numpy as np
import pytest
import torch

from oracle import attention_forward, decode_paged, prefill_paged
from workloads import prefill_inputs


def _rows(p, b):
    return int(p.cu_seqlens_q[b]), int(p.cu_seqlens_q[b + 1])


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_matches_decode_row_by_row(causal):
    """Query i of a chunk sees keys 0 .. i + L - n (causal) or all L keys: that
    is exactly a decode step over a cache cut to that many tokens."""
    p = prefill_inputs([5, 1, 9], [21, 7, 9], H=4, Hkv=2, d=8, seed=3, page_size=4)
    o, lse = prefill_paged(p.q, p.kv_pool, p.block_table, p.seq_lens_k, p.cu_seqlens_q, causal=causal,
                           scale=0.3, page_size=4)
    for b in range(3):
        t0, t1 = _rows(p, b)
        L, n = int(p.seq_lens_k[b]), t1 - t0
        for i in range(n):
            seen = i + L - n + 1 if causal else L
            od, ld = decode_paged(p.q[t0 + i][None], p.kv_pool, p.block_table[b][None], [seen], scale=0.3,
                                  page_size=4)
            np.testing.assert_allclose(o[t0 + i], od[0], atol=1e-13)
            np.testing.assert_allclose(lse[:, t0 + i], ld[0], atol=1e-13)


def test_no_prefix_is_the_dense_causal_forward():
    p = prefill_inputs([13, 6], [13, 6], H=2, Hkv=2, d=8, seed=5, page_size=4)
    o, lse = prefill_paged(p.q, p.kv_pool, p.block_table, p.seq_lens_k, p.cu_seqlens_q, causal=True,
                           page_size=4)
    pool = p.kv_pool.double().numpy()
    for b in range(2):
        t0, t1 = _rows(p, b)
        n = t1 - t0
        K = np.stack([pool[int(p.block_table[b, t // 4]), 0, t % 4] for t in range(n)])  # [n, H, d]
        V = np.stack([pool[int(p.block_table[b, t // 4]), 1, t % 4] for t in range(n)])
        for h in range(2):
            of, lf = attention_forward(p.q[t0:t1, h], K[:, h], V[:, h], causal=True)
            np.testing.assert_allclose(o[t0:t1, h], of, atol=1e-13)
            np.testing.assert_allclose(lse[h, t0:t1], lf, atol=1e-13)


def test_matches_torch_sdpa_with_explicit_mask():
    p = prefill_inputs([6, 3], [17, 3], H=6, Hkv=3, d=8, seed=9, page_size=8)
    o, _ = prefill_paged(p.q, p.kv_pool, p.block_table, p.seq_lens_k, p.cu_seqlens_q, causal=True,
                         scale=0.25, page_size=8)
    pool = p.kv_pool.double()
    for b in range(2):
        t0, t1 = _rows(p, b)
        n, L = t1 - t0, int(p.seq_lens_k[b])
        K = torch.stack([pool[int(p.block_table[b, t // 8]), 0, t % 8] for t in range(L)])  # [L, Hkv, d]
        V = torch.stack([pool[int(p.block_table[b, t // 8]), 1, t % 8] for t in range(L)])
        allowed = torch.arange(L)[None, :] <= (torch.arange(n) + (L - n))[:, None]     # [n, L]
        ref = torch.nn.functional.scaled_dot_product_attention(
            p.q[t0:t1].double().transpose(0, 1)[None], K.transpose(0, 1)[None], V.transpose(0, 1)[None],
            attn_mask=allowed, scale=0.25, enable_gqa=True)
        np.testing.assert_allclose(o[t0:t1], ref[0].transpose(0, 1).numpy(), atol=1e-12)


def test_query_that_sees_no_key_is_empty():
    # three queries against two cached keys: the first query precedes every key
    p = prefill_inputs([3], [2], H=2, Hkv=1, d=4, seed=1, page_size=4)
    o, lse = prefill_paged(p.q, p.kv_pool, p.block_table, p.seq_lens_k, p.cu_seqlens_q, causal=True,
                           page_size=4)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[:, 0]))
    assert np.all(np.isfinite(lse[:, 1:]))
    # query 1 sees only key 0, so its output is that key's value row
    pool = p.kv_pool.double().numpy()
    np.testing.assert_allclose(o[1], np.repeat(pool[int(p.block_table[0, 0]), 1, 0], 2, axis=0), atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_sequence_without_keys_is_empty(causal):
    """A sequence with no cached key: every one of its queries has an empty
    softmax (O = 0, LSE = -inf), and the neighbouring sequence still equals
    its own prefill computed alone."""
    p = prefill_inputs([4, 3], [0, 6], H=2, Hkv=1, d=8, seed=8, page_size=4)
    o, lse = prefill_paged(p.q, p.kv_pool, p.block_table, p.seq_lens_k, p.cu_seqlens_q, causal=causal,
                           scale=0.5, page_size=4)
    assert (o[:4] == 0).all() and np.isneginf(lse[:, :4]).all()
    t0, t1 = _rows(p, 1)
    o1, l1 = prefill_paged(p.q[t0:t1], p.kv_pool, p.block_table[1:], p.seq_lens_k[1:],
                           torch.tensor([0, t1 - t0], dtype=torch.int32), causal=causal, scale=0.5, page_size=4)
    np.testing.assert_allclose(o[t0:t1], o1, atol=1e-15)
    np.testing.assert_allclose(lse[:, t0:t1], l1, atol=1e-15)

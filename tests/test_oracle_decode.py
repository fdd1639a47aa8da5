"""Pins of the fp64 oracle's paged decode: reduction to the contiguous forward,
page-order independence and poison independence."""
import numpy as np
import pytest
import torch

from oracle import attention_forward, decode_paged
from workloads import paged_inputs


def _scatter_into_pool(rng, K, V, page, spare=3):
    """Place contiguous per-sequence K/V [L, H, d] into a shuffled page pool."""
    S = len(K)
    pages = [(k.shape[0] + page - 1) // page for k in K]
    total = sum(pages) + spare
    H, d = K[0].shape[1:]
    pool = rng.standard_normal((total, 2, page, H, d))
    perm = rng.permutation(total)
    table = -np.ones((S, max(pages)), dtype=np.int64)
    off = 0
    for s in range(S):
        table[s, :pages[s]] = perm[off:off + pages[s]]
        off += pages[s]
        for t in range(K[s].shape[0]):
            pool[table[s, t // page], 0, t % page] = K[s][t]
            pool[table[s, t // page], 1, t % page] = V[s][t]
    return pool, table


def test_paged_equals_contiguous_forward(rng):
    page, H, d = 8, 3, 4
    lens = [1, 8, 9, 21]
    K = [rng.standard_normal((L, H, d)) for L in lens]
    V = [rng.standard_normal((L, H, d)) for L in lens]
    q = rng.standard_normal((len(lens), H, d))
    pool, table = _scatter_into_pool(rng, K, V, page)
    o, lse = decode_paged(q, pool, table, lens, scale=0.5, page_size=page)
    for s, L in enumerate(lens):
        for h in range(H):
            o2, l2 = attention_forward(q[s, h][None], K[s][:, h], V[s][:, h], scale=0.5)
            np.testing.assert_allclose(o[s, h], o2[0], atol=1e-13)
            np.testing.assert_allclose(lse[s, h], l2[0], atol=1e-13)
    # A single cached token returns its value.
    np.testing.assert_allclose(o[0], V[0][0], atol=1e-14)


def test_independent_of_page_placement(rng):
    page, H, d = 4, 2, 4
    lens = [7, 13]
    K = [rng.standard_normal((L, H, d)) for L in lens]
    V = [rng.standard_normal((L, H, d)) for L in lens]
    q = rng.standard_normal((2, H, d))
    a = decode_paged(q, *_scatter_into_pool(rng, K, V, page), lens, page_size=page)
    b = decode_paged(q, *_scatter_into_pool(rng, K, V, page, spare=9), lens, page_size=page)
    np.testing.assert_allclose(a[0], b[0], atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], atol=1e-14)


def test_poisoned_tails_and_spare_pages_are_never_read():
    kw = dict(num_seqs=3, H=2, d=8, len_lo=5, len_hi=60, max_blocks=4, seed=7, page_size=16)
    clean = paged_inputs(**kw)
    dirty = paged_inputs(poison=True, spare_pages=0, **kw)
    a = decode_paged(clean.q, clean.kv_pool, clean.block_table, clean.seq_lens, page_size=16)
    b = decode_paged(dirty.q, dirty.kv_pool, dirty.block_table, dirty.seq_lens, page_size=16)
    assert np.all(np.isfinite(b[0]))
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_workload_generator_layout():
    p = paged_inputs(num_seqs=4, H=2, d=8, len_lo=3, len_hi=40, max_blocks=3, seed=3,
                     page_size=16, poison=True, spare_pages=5)
    used = p.block_table[p.block_table >= 0]
    assert used.unique().numel() == used.numel()          # pages are not shared
    for s, L in enumerate(p.seq_lens.tolist()):
        n = (L + 15) // 16
        assert (p.block_table[s, :n] >= 0).all() and (p.block_table[s, n:] == -1).all()
    spare = sorted(set(range(p.kv_pool.shape[0])) - set(used.tolist()))
    assert len(spare) == 5 and torch.isnan(p.kv_pool[spare].float()).all()


@pytest.mark.parametrize("H,Hkv", [(4, 2), (6, 1), (8, 4)])
def test_grouped_decode_matches_torch_sdpa(rng, H, Hkv):
    """Grouped key/value heads: O matches torch's own grouped-query SDPA (fp64)
    on the gathered contiguous K/V, and the whole result equals plain decode
    on a pool whose key/value heads are repeated for every query head."""
    page, d = 8, 4
    lens = [1, 8, 9, 21]
    K = [rng.standard_normal((L, Hkv, d)) for L in lens]
    V = [rng.standard_normal((L, Hkv, d)) for L in lens]
    q = rng.standard_normal((len(lens), H, d))
    pool, table = _scatter_into_pool(rng, K, V, page)
    o, lse = decode_paged(q, pool, table, lens, scale=0.5, page_size=page)
    for s, L in enumerate(lens):
        qt = torch.from_numpy(q[s])[None, :, None, :]              # [1, H, 1, d]
        kt = torch.from_numpy(K[s]).permute(1, 0, 2)[None]         # [1, Hkv, L, d]
        vt = torch.from_numpy(V[s]).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.5, enable_gqa=True)
        np.testing.assert_allclose(o[s], ref[0, :, 0].numpy(), atol=1e-12)
    g = H // Hkv
    o2, lse2 = decode_paged(q, np.repeat(pool, g, axis=3), table, lens, scale=0.5, page_size=page)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, atol=1e-14)


def test_mqa_decode_heads_share_one_cache(rng):
    page, H, d = 4, 5, 3
    lens = [6, 11]
    K = [rng.standard_normal((L, 1, d)) for L in lens]
    V = [rng.standard_normal((L, 1, d)) for L in lens]
    q = rng.standard_normal((2, H, d))
    o, lse = decode_paged(q, *_scatter_into_pool(rng, K, V, page), lens, page_size=page)
    for s in range(2):
        for h in range(H):
            o1, l1 = attention_forward(q[s, h][None], K[s][:, 0], V[s][:, 0], scale=1 / np.sqrt(d))
            np.testing.assert_allclose(o[s, h], o1[0], atol=1e-13)
            np.testing.assert_allclose(lse[s, h], l1[0], atol=1e-13)


def test_empty_sequence_is_an_empty_softmax(rng):
    page, H, d = 4, 2, 3
    K = [rng.standard_normal((5, H, d)), np.zeros((0, H, d))]
    V = [rng.standard_normal((5, H, d)), np.zeros((0, H, d))]
    q = rng.standard_normal((2, H, d))
    pool, table = _scatter_into_pool(rng, K, V, page)
    table = np.concatenate([table, -np.ones((2, 1), dtype=np.int64)], axis=1)
    o, lse = decode_paged(q, pool, table, [5, 0], page_size=page)
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))
    assert np.all(np.isfinite(o[0])) and np.all(np.isfinite(lse[0]))

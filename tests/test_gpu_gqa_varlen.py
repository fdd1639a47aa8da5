"""GPU parity of grouped key/value heads (GQA/MQA) and packed variable-length
batches against the fp64 oracle, element by element over every output.

Lengths mix empty, single-token, sub-tile, tile-multiple and multi-tile
sequences so that every ragged tail and the sequence boundaries inside the
packed rows are exercised; the group sizes cover MHA (1), GQA (2, 4) and MQA.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import BF16_MAX, BF16_MEAN, F32_MAX, LSE_MAX, check, grouped, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X")
    import exact_attention_fwd_amd  # noqa: F401  (fails loudly if libfa.so is missing)
    yield


def fa():
    import exact_attention_fwd_amd
    return exact_attention_fwd_amd


def cuda(*ts):
    return [t.to(DEV) for t in ts]


# ---------------------------------------------------------------- GQA / MQA
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv,N", [(8, 1, 300), (8, 2, 257), (6, 3, 64), (4, 4, 130)])
def test_gqa_forward_backward(H, Hkv, N, causal, d):
    q, k, v, do = workloads.gqa_inputs(2, H, Hkv, N, d, "bf16", seed=7 * H + Hkv + N + d, with_dout=True)
    scale = 1 / math.sqrt(d)
    print(f"[gqa] B=2 H={H} Hkv={Hkv} N={N} d={d} causal={causal}", flush=True)
    qd, kd, vd, dod = cuda(q, k, v, do)
    o, lse = fa().forward(qd, kd, vd, causal=causal)
    dq, dk, dv = fa().backward(qd, kd, vd, o, dod, lse, causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward_gqa(q, k, v, causal=causal, scale=scale)
    check("gqa O", to64(o), ro, BF16_MAX, BF16_MEAN)
    check("gqa LSE", to64(lse), rl, LSE_MAX)
    assert dk.shape == k.shape and dv.shape == v.shape
    rq, rk, rv = oracle.attention_backward_gqa(q, k, v, do, causal=causal, scale=scale)
    check("gqa dq", to64(dq), rq, BF16_MAX, BF16_MEAN)
    g = H // Hkv
    check("gqa dk", to64(dk), rk, grouped(BF16_MAX, g), grouped(BF16_MEAN, g))
    check("gqa dv", to64(dv), rv, grouped(BF16_MAX, g), grouped(BF16_MEAN, g))


def test_gqa_forward_fp32():
    q, k, v = workloads.gqa_inputs(1, 4, 2, 77, 64, "f32", seed=5)
    o, lse = fa().forward(*cuda(q, k, v), causal=True)
    ro, rl = oracle.attention_forward_gqa(q, k, v, causal=True)
    check("gqa fp32 O", to64(o), ro, F32_MAX)
    check("gqa fp32 LSE", to64(lse), rl, LSE_MAX)


def test_gqa_rejects_indivisible_heads():
    q, k, v = cuda(*workloads.gqa_inputs(1, 6, 4, 16, 64, "bf16", seed=1))
    with pytest.raises(ValueError):
        fa().forward(q, k, v)
    # the C ABI itself rejects it too (FA_ERR_BAD_SHAPE)
    rc = fa().lib().fa_forward_gqa(1, 1, 6, 4, 16, 64, q.data_ptr(), k.data_ptr(), v.data_ptr(), q.data_ptr(), None,
                                   0, 0.125, None)
    assert rc == 2


# ------------------------------------------------------- packed variable length
LENS = {
    "mixed": [300, 0, 1, 64, 129, 7, 513],
    "one": [1000],
    "tiny": [1, 1, 2, 0, 3],
    "tiles": [256, 64, 320],
}


def _varlen_compare(lens, H, Hkv, d, causal, dtype="bf16", with_bwd=True, seed=0):
    cu, q, k, v, do = workloads.varlen_inputs(lens, H, Hkv, d, dtype, seed=seed, with_dout=True)
    scale = 1 / math.sqrt(d)
    mx = max(lens)
    print(f"[varlen] lens={lens} H={H} Hkv={Hkv} d={d} causal={causal} {dtype}", flush=True)
    cud, qd, kd, vd, dod = cuda(cu, q, k, v, do)
    o, lse = fa().forward_varlen(qd, kd, vd, cud, mx, causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward_varlen(q, k, v, cu, causal=causal, scale=scale)
    if dtype == "f32":
        check("varlen fp32 O", to64(o), ro, F32_MAX)
    else:
        check("varlen O", to64(o), ro, BF16_MAX, BF16_MEAN)
    check("varlen LSE", to64(lse), rl, LSE_MAX)
    if not with_bwd:
        return
    dq, dk, dv = fa().backward_varlen(qd, kd, vd, o, dod, lse, cud, mx, causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward_varlen(q, k, v, do, cu, causal=causal, scale=scale)
    check("varlen dq", to64(dq), rq, BF16_MAX, BF16_MEAN)
    g = H // Hkv
    check("varlen dk", to64(dk), rk, grouped(BF16_MAX, g), grouped(BF16_MEAN, g))
    check("varlen dv", to64(dv), rv, grouped(BF16_MAX, g), grouped(BF16_MEAN, g))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lens", ["mixed", "one", "tiny", "tiles"])
def test_varlen_forward_backward(lens, causal, d):
    _varlen_compare(LENS[lens], 4, 2, d, causal, seed=len(LENS[lens]) + d)


def test_varlen_blocks_ordered_per_kv_head():
    """B=2, H=16, Hkv=8: each XCD's share of the head-major units is whole
    key/value heads of both sequences, so the workgroups take the
    one-(sequence, key/value head)-at-a-time order; every row must still be
    produced once."""
    _varlen_compare([300, 1000], 16, 8, 128, True, seed=21)


def test_varlen_mha_and_mqa():
    _varlen_compare([200, 33, 0, 700], 4, 4, 128, True, seed=11)
    _varlen_compare([200, 33, 0, 700], 8, 1, 64, False, seed=12)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_forward_fp32(causal):
    _varlen_compare([90, 0, 1, 40], 2, 1, 64, causal, dtype="f32", with_bwd=False, seed=13)


def test_varlen_single_sequence_matches_dense():
    """One packed sequence is the dense [1, H, N, d] problem in another layout."""
    cu, q, k, v = workloads.varlen_inputs([777], 4, 4, 128, seed=14)
    cud, qd, kd, vd = cuda(cu, q, k, v)
    o, lse = fa().forward_varlen(qd, kd, vd, cud, 777, causal=True)
    dense = [x.permute(1, 0, 2).unsqueeze(0).contiguous() for x in (qd, kd, vd)]
    od, lsed = fa().forward(*dense, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, od[0].permute(1, 0, 2))
    assert torch.equal(lse, lsed[0])


def test_varlen_all_empty_is_noop():
    cu = torch.zeros(4, dtype=torch.int32, device=DEV)
    z = torch.zeros(0, 2, 64, dtype=torch.bfloat16, device=DEV)
    o, lse = fa().forward_varlen(z, z, z, cu, 0, causal=True)
    assert o.shape == (0, 2, 64) and lse.shape == (2, 0)


# ------------------------------------------------- paged decode, grouped heads
def _decode_compare(name, p):
    d = p.q.shape[-1]
    qd, pool, bt, sl = cuda(p.q, p.kv_pool, p.block_table, p.seq_lens)
    o, lse = fa().decode_paged(qd, pool, bt, sl)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_paged(p.q, p.kv_pool, p.block_table, p.seq_lens, scale=1 / math.sqrt(d),
                                 page_size=p.page_size)
    check(f"{name} O", to64(o), ro, BF16_MAX, BF16_MEAN)
    check(f"{name} LSE", to64(lse), rl, LSE_MAX)
    assert torch.isfinite(o.float()).all()
    return o, lse


@pytest.mark.parametrize("Hkv", [1, 4, 8, 16])
def test_decode_gqa_c4_shape(Hkv):
    """The paged-decode configuration (8 sequences, 32 query heads, d=128,
    lengths 1024..8192) with the pool holding Hkv key/value heads, poisoned
    tails and spare pages."""
    w = workloads.CONFIGS["c4"]
    print(f"[decode gqa] H=32 Hkv={Hkv}", flush=True)
    p = workloads.workload_inputs(w, Hkv=Hkv, poison=True, spare_pages=8)
    _decode_compare(f"decode H=32 Hkv={Hkv}", p)


@pytest.mark.parametrize("H,Hkv,d", [(8, 2, 64), (64, 1, 128), (48, 1, 64), (6, 3, 128)])
def test_decode_gqa_shapes(H, Hkv, d):
    lens = [1, 63, 64, 65, 255, 256, 257, 1000]
    p = workloads.paged_inputs(num_seqs=len(lens), H=H, Hkv=Hkv, d=d, max_blocks=5, seed=H + Hkv + d,
                               seq_lens=lens, poison=True, spare_pages=3)
    print(f"[decode gqa] H={H} Hkv={Hkv} d={d}", flush=True)
    _decode_compare(f"decode H={H} Hkv={Hkv} d={d}", p)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_gqa_page_splits(d):
    """A block table wide enough (8 sequences x 32 pages x 4 key/value heads)
    that each wavefront takes a whole page: lengths on, just before and just
    after page boundaries, a one-token sequence and a nearly full table."""
    lens = [1, 255, 256, 257, 511, 513, 4000, 8191]
    p = workloads.paged_inputs(num_seqs=len(lens), H=16, Hkv=4, d=d, max_blocks=32, seed=40 + d,
                               seq_lens=lens, poison=True, spare_pages=5)
    print(f"[decode gqa pages] H=16 Hkv=4 d={d}", flush=True)
    _decode_compare(f"decode pages H=16 Hkv=4 d={d}", p)


def test_decode_gqa_is_deterministic():
    p = workloads.paged_inputs(num_seqs=4, H=32, Hkv=8, d=128, len_lo=300, len_hi=3000, max_blocks=12, seed=4)
    args = cuda(p.q, p.kv_pool, p.block_table, p.seq_lens)
    a = fa().decode_paged(*args)
    b = fa().decode_paged(*args)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("Hkv", [8, 2])
def test_decode_empty_sequence(Hkv):
    """A sequence with no cached token: O = 0 and LSE = -inf, neighbours unaffected."""
    p = workloads.paged_inputs(num_seqs=3, H=8, Hkv=Hkv, d=128, max_blocks=3, seed=21, seq_lens=[300, 1, 2])
    p.seq_lens[1] = 0
    qd, pool, bt, sl = cuda(p.q, p.kv_pool, p.block_table, p.seq_lens)
    o, lse = fa().decode_paged(qd, pool, bt, sl)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_paged(p.q, p.kv_pool, p.block_table, p.seq_lens, page_size=p.page_size)
    assert (o[1] == 0).all() and torch.isneginf(lse[1]).all() and np.isneginf(rl[1]).all()
    keep = [0, 2]
    check("decode empty neighbours O", to64(o)[keep], ro[keep], BF16_MAX, BF16_MEAN)
    check("decode empty neighbours LSE", to64(lse)[keep], rl[keep], LSE_MAX)


# ------------------------------------------------------ paged chunked prefill
def _prefill_compare(name, p, causal):
    d = p.q.shape[-1]
    qd, pool, bt, sl, cu = cuda(p.q, p.kv_pool, p.block_table, p.seq_lens_k, p.cu_seqlens_q)
    mx = int((p.cu_seqlens_q[1:] - p.cu_seqlens_q[:-1]).max())
    o, lse = fa().prefill_paged(qd, pool, bt, sl, cu, mx, causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_paged(p.q, p.kv_pool, p.block_table, p.seq_lens_k, p.cu_seqlens_q, causal=causal,
                                  scale=1 / math.sqrt(d), page_size=p.page_size)
    o64, l64 = to64(o), to64(lse)
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(l64), empty), "rows that see no key must give LSE = -inf"
    check(f"{name} O", o64, ro, BF16_MAX, BF16_MEAN)
    check(f"{name} LSE", l64[~empty], rl[~empty], LSE_MAX)
    return o, lse


PREFILL = {
    # chunk lengths, cached keys (prefix + chunk)
    "prefix": ([300, 1, 64, 257, 513], [1000, 513, 64, 300, 2048]),
    "no_prefix": ([200, 77, 256], [200, 77, 256]),
    "decode_like": ([1, 1, 1], [1, 255, 4097]),
}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("case", sorted(PREFILL))
def test_prefill_paged(case, causal, d):
    chunks, ctx = PREFILL[case]
    print(f"[prefill] {case} causal={causal} d={d}", flush=True)
    p = workloads.prefill_inputs(chunks, ctx, H=8, Hkv=2, d=d, seed=len(chunks) + d, poison=True, spare_pages=3)
    _prefill_compare(f"prefill {case}", p, causal)


@pytest.mark.parametrize("Hkv", [8, 1])
def test_prefill_paged_heads(Hkv):
    p = workloads.prefill_inputs([130, 40], [900, 40], H=8, Hkv=Hkv, d=128, seed=Hkv)
    _prefill_compare(f"prefill Hkv={Hkv}", p, True)


def test_prefill_blocks_ordered_per_kv_head():
    """B=2, H=32, Hkv=8 (groups of 4): the paged prefill's workgroups take the
    one-(sequence, key/value head)-at-a-time order."""
    p = workloads.prefill_inputs([300, 70], [1000, 70], H=32, Hkv=8, d=128, seed=22, poison=True, spare_pages=3)
    _prefill_compare("prefill ordered blocks", p, True)


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_more_queries_than_keys(d):
    """Causal rows before the first cached key are empty: O = 0, LSE = -inf
    (at d = 128 a whole 64-query wavefront of the first sequence, and part of
    the next, see no key)."""
    p = workloads.prefill_inputs([300, 70, 5], [40, 40, 5], H=4, Hkv=4, d=d, seed=3 + d)
    o, lse = _prefill_compare(f"prefill n > L d={d}", p, True)
    assert (o[:260] == 0).all() and torch.isneginf(lse[:, :260]).all()
    assert (o[300:330] == 0).all() and torch.isneginf(lse[:, 300:330]).all()


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_sequence_without_keys(d):
    """A sequence with no cached key at all: its queries get O = 0 and
    LSE = -inf; the other sequence of the batch is unaffected."""
    p = workloads.prefill_inputs([300, 3], [0, 3], H=4, Hkv=2, d=d, seed=11 + d)
    for causal in (True, False):
        o, lse = _prefill_compare(f"prefill L=0 d={d} causal={causal}", p, causal)
        assert (o[:300] == 0).all() and torch.isneginf(lse[:, :300]).all()


def test_prefill_without_prefix_matches_varlen_forward():
    """With no cached prefix the paged prefill is the packed causal forward."""
    p = workloads.prefill_inputs([333, 64], [333, 64], H=4, Hkv=4, d=128, seed=17)
    qd, pool, bt, sl, cu = cuda(p.q, p.kv_pool, p.block_table, p.seq_lens_k, p.cu_seqlens_q)
    o, lse = fa().prefill_paged(qd, pool, bt, sl, cu, 333, causal=True)
    # the same keys/values gathered into the packed layout
    pool_c = p.kv_pool
    ks, vs = [], []
    for b, L in enumerate(p.seq_lens_k.tolist()):
        for t in range(L):
            pg = int(p.block_table[b, t // 256])
            ks.append(pool_c[pg, 0, t % 256])
            vs.append(pool_c[pg, 1, t % 256])
    k, v = torch.stack(ks).to(DEV), torch.stack(vs).to(DEV)
    o2, lse2 = fa().forward_varlen(qd, k, v, cu, 333, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


# ------------------------------------------------------------ fused rotary
@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_rope_dense(causal, d, interleaved):
    B, H, Hkv, N = 2, 4, 2, 300
    q, k, v = workloads.gqa_inputs(B, H, Hkv, N, d, "bf16", seed=d + int(causal) + 2 * int(interleaved))
    c, s = workloads.rope_tables(N + 5, d)
    print(f"[rope] causal={causal} d={d} interleaved={interleaved}", flush=True)
    o, lse = fa().forward_rope(*cuda(q, k, v, c, s), causal=causal, interleaved=interleaved)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward_rope(q, k, v, c, s, causal=causal, interleaved=interleaved)
    check("rope O", to64(o), ro, BF16_MAX, BF16_MEAN)
    check("rope LSE", to64(lse), rl, LSE_MAX)


def test_forward_rope_long_positions():
    """16K positions: angles up to 16383 rad in the fp32 tables."""
    q, k, v = workloads.gqa_inputs(1, 2, 2, 16384, 128, "bf16", seed=31)
    c, s = workloads.rope_tables(16384, 128)
    o, lse = fa().forward_rope(*cuda(q, k, v, c, s), causal=True)
    torch.cuda.synchronize()
    rows = sorted(set([0, 1, 255, 256, 8191, 16383] + list(np.random.default_rng(3).integers(0, 16384, 24))))
    pos = np.arange(16384)
    qr = oracle.apply_rope_bf16(q, pos, c, s)
    kr = oracle.apply_rope_bf16(k, pos, c, s)
    for h in range(2):
        ro, rl = oracle.attention_forward_rows(qr[0, h], kr[0, h], v[0, h], rows, causal=True)
        check(f"rope 16K head {h} O", to64(o[0, h].cpu())[rows], ro, BF16_MAX, BF16_MEAN)
        check(f"rope 16K head {h} LSE", to64(lse[0, h].cpu())[rows], rl, LSE_MAX)


def test_forward_rope_varlen():
    cu, q, k, v = workloads.varlen_inputs([300, 0, 1, 129, 64], 4, 1, 128, seed=41)
    c, s = workloads.rope_tables(300, 128)
    o, lse = fa().forward_rope(*cuda(q, k, v, c, s), causal=True, cu_seqlens=cu.to(DEV), max_seqlen=300)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward_rope(q, k, v, c, s, causal=True, cu_seqlens=cu)
    check("rope varlen O", to64(o), ro, BF16_MAX, BF16_MEAN)
    check("rope varlen LSE", to64(lse), rl, LSE_MAX)


@pytest.mark.parametrize("interleaved", [False, True])
def test_prefill_paged_rope(interleaved):
    p = workloads.prefill_inputs([300, 1, 64], [1000, 513, 64], H=8, Hkv=2, d=128, seed=5, poison=True,
                                 spare_pages=2)
    c, s = workloads.rope_tables(1024, 128)
    qd, pool, bt, sl, cu = cuda(p.q, p.kv_pool, p.block_table, p.seq_lens_k, p.cu_seqlens_q)
    o, lse = fa().prefill_paged(qd, pool, bt, sl, cu, 300, causal=True, rope_cos=c.to(DEV), rope_sin=s.to(DEV),
                                rope_interleaved=interleaved)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_paged(p.q, p.kv_pool, p.block_table, p.seq_lens_k, p.cu_seqlens_q, causal=True,
                                  rope=(c, s, interleaved))
    check("prefill rope O", to64(o), ro, BF16_MAX, BF16_MEAN)
    check("prefill rope LSE", to64(lse), rl, LSE_MAX)

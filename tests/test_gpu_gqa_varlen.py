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
from tests.parity import BF16_MAX, BF16_MEAN, F32_MAX, LSE_MAX, check, check_rounded, to64

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
    grad_check = check if H == Hkv else check_rounded  # dK, dV sum H / Hkv query heads
    grad_check("gqa dk", to64(dk), rk, BF16_MAX, BF16_MEAN)
    grad_check("gqa dv", to64(dv), rv, BF16_MAX, BF16_MEAN)


def test_gqa_forward_16k_full_size():
    """The grouped-head 16K causal forward the bench times ([1, 32 query heads,
    8 key/value heads, 16384, 128], same seed), run at full size in that launch
    configuration: two whole heads compared element by element plus sampled
    rows of three more heads, each against the fp64 oracle on the shared
    key/value head h // 4."""
    w = workloads.CONFIGS["c2a"]
    Hkv = 8
    print(f"[gqa 16k] generating 1x32q{Hkv}kv x {w.N}x{w.d}", flush=True)
    q, k, v = workloads.gqa_inputs(w.B, w.H, Hkv, w.N, w.d, "bf16", seed=w.seed)
    o, lse = fa().forward(*cuda(q, k, v), causal=True, scale=w.scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    g = w.H // Hkv
    rng = np.random.default_rng(77)
    fixed = [0, 1, 63, 64, 255, 256, 8191, w.N - 257, w.N - 256, w.N - 2, w.N - 1]
    rows = sorted(set(fixed + rng.integers(0, w.N, 40).tolist()))
    got_o, ref_o, got_l, ref_l = [], [], [], []
    for h in (0, w.H - 1):
        ro, rl = oracle.attention_forward(q[0, h], k[0, h // g], v[0, h // g], causal=True, scale=w.scale)
        got_o.append(to64(o[0, h]).ravel()), ref_o.append(ro.ravel())
        got_l.append(to64(lse[0, h]).ravel()), ref_l.append(rl.ravel())
    for h in (1, 13, w.H - 2):
        ro, rl = oracle.attention_forward_rows(q[0, h], k[0, h // g], v[0, h // g], rows, causal=True,
                                               scale=w.scale)
        got_o.append(to64(o[0, h])[rows].ravel()), ref_o.append(ro.ravel())
        got_l.append(to64(lse[0, h])[rows].ravel()), ref_l.append(rl.ravel())
    check("gqa 16k O", np.concatenate(got_o), np.concatenate(ref_o), BF16_MAX, BF16_MEAN)
    check("gqa 16k LSE", np.concatenate(got_l), np.concatenate(ref_l), LSE_MAX)


def test_gqa_backward_full_size():
    """The grouped-head 8K causal backward the bench times ([2, 16 query heads,
    4 key/value heads, 8192, 128], same seed), at full size in that launch
    configuration: dK, dV of two whole key/value heads (one per batch entry,
    each the sum over its four query heads) and dQ of those eight query heads,
    element by element against the fp64 oracle."""
    w = workloads.CONFIGS["c3"]
    Hkv = 4
    g = w.H // Hkv
    print(f"[gqa bwd 8k] generating {w.B}x{w.H}q{Hkv}kv x {w.N}x{w.d}", flush=True)
    q, k, v, do = workloads.gqa_inputs(w.B, w.H, Hkv, w.N, w.d, "bf16", seed=w.seed, with_dout=True)
    qd, kd, vd, dod = cuda(q, k, v, do)
    o, lse = fa().forward(qd, kd, vd, causal=True, scale=w.scale)
    dq, dk, dv = fa().backward(qd, kd, vd, o, dod, lse, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    got = {n: [] for n in ("dq", "dk", "dv")}
    ref = {n: [] for n in ("dq", "dk", "dv")}
    for b, j in ((0, 0), (1, Hkv - 1)):
        rk = np.zeros((w.N, w.d))
        rv = np.zeros((w.N, w.d))
        for h in range(j * g, (j + 1) * g):
            rq, rk_h, rv_h = oracle.attention_backward(q[b, h], k[b, j], v[b, j], do[b, h], causal=True,
                                                       scale=w.scale)
            got["dq"].append(to64(dq[b, h]).ravel()), ref["dq"].append(rq.ravel())
            rk += rk_h
            rv += rv_h
        got["dk"].append(to64(dk[b, j]).ravel()), ref["dk"].append(rk.ravel())
        got["dv"].append(to64(dv[b, j]).ravel()), ref["dv"].append(rv.ravel())
    check("gqa bwd 8k dq", np.concatenate(got["dq"]), np.concatenate(ref["dq"]), BF16_MAX, BF16_MEAN)
    check_rounded("gqa bwd 8k dk", np.concatenate(got["dk"]), np.concatenate(ref["dk"]), BF16_MAX, BF16_MEAN)
    check_rounded("gqa bwd 8k dv", np.concatenate(got["dv"]), np.concatenate(ref["dv"]), BF16_MAX, BF16_MEAN)


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
    grad_check = check if H == Hkv else check_rounded  # dK, dV sum H / Hkv query heads
    grad_check("varlen dk", to64(dk), rk, BF16_MAX, BF16_MEAN)
    grad_check("varlen dv", to64(dv), rv, BF16_MAX, BF16_MEAN)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lens", ["mixed", "one", "tiny", "tiles"])
def test_varlen_forward_backward(lens, causal, d):
    _varlen_compare(LENS[lens], 4, 2, d, causal, seed=len(LENS[lens]) + d)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_spiked_sequence(causal):
    """A packed batch where only keys 500..519 of the first sequence score far
    above the rest (about 130 powers of two, within one key tile): the
    workgroups of that sequence's rows that see them must take the d = 128
    forward's exact-max loop, the others not, and every row must still match
    the oracle."""
    lens = [700, 300, 900]
    cu, q, k, v = workloads.varlen_inputs(lens, 4, 2, 128, seed=77)
    q, k = workloads.add_spike(q, k, list(range(500, 520)), workloads.spike_direction(128, 78))
    print(f"[varlen spike] lens={lens} causal={causal}", flush=True)
    cud, qd, kd, vd = cuda(cu, q, k, v)
    o, lse = fa().forward_varlen(qd, kd, vd, cud, max(lens), causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward_varlen(q, k, v, cu, causal=causal, scale=1 / math.sqrt(128))
    check("varlen spike O", to64(o), ro, BF16_MAX, BF16_MEAN)
    check("varlen spike LSE", to64(lse), rl, LSE_MAX)


def test_varlen_full_size():
    """The packed causal batch the bench times (16 sequences of 527 .. 7723
    tokens, 80 620 rows, H = 32, d = 128, same seed), forward and backward at
    full size in that launch configuration.  Forward: two whole (sequence,
    head) pairs, the longest and the shortest sequence, plus sampled rows of two
    more; backward: dQ, dK, dV of two whole pairs; all against the fp64 oracle
    on the sequence cut out of the packed rows."""
    lens = workloads.varlen_lengths()
    H, d = 32, 128
    scale = 1 / math.sqrt(d)
    print(f"[varlen full] lens={lens} H={H} d={d}", flush=True)
    cu, q, k, v, do = workloads.varlen_inputs(lens, H, H, d, "bf16", seed=workloads.VARLEN_SEED, with_dout=True)
    cud, qd, kd, vd, dod = cuda(cu, q, k, v, do)
    mx = max(lens)
    o, lse = fa().forward_varlen(qd, kd, vd, cud, mx, causal=True)
    dq, dk, dv = fa().backward_varlen(qd, kd, vd, o, dod, lse, cud, mx, causal=True)
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (t.cpu() for t in (o, lse, dq, dk, dv))
    cut = lambda x, s, h: x[int(cu[s]):int(cu[s + 1]), h]  # noqa: E731
    longest, shortest = int(np.argmax(lens)), int(np.argmin(lens))
    got_o, ref_o, got_l, ref_l = [], [], [], []
    for s_, h in ((longest, 0), (shortest, H - 1)):
        ro, rl = oracle.attention_forward(cut(q, s_, h), cut(k, s_, h), cut(v, s_, h), causal=True, scale=scale)
        got_o.append(to64(cut(o, s_, h)).ravel()), ref_o.append(ro.ravel())
        got_l.append(to64(cut(lse.T, s_, h)).ravel()), ref_l.append(rl.ravel())
    rng = np.random.default_rng(5)
    for s_, h in ((0, 13), (12, 20)):
        L = lens[s_]
        rows = sorted(set([0, 1, 63, 64, L - 65, L - 64, L - 2, L - 1] + rng.integers(0, L, 24).tolist()))
        ro, rl = oracle.attention_forward_rows(cut(q, s_, h), cut(k, s_, h), cut(v, s_, h), rows, causal=True,
                                               scale=scale)
        got_o.append(to64(cut(o, s_, h))[rows].ravel()), ref_o.append(ro.ravel())
        got_l.append(to64(cut(lse.T, s_, h))[rows].ravel()), ref_l.append(rl.ravel())
    check("varlen full O", np.concatenate(got_o), np.concatenate(ref_o), BF16_MAX, BF16_MEAN)
    check("varlen full LSE", np.concatenate(got_l), np.concatenate(ref_l), LSE_MAX)
    got = {n: [] for n in ("dq", "dk", "dv")}
    ref = {n: [] for n in ("dq", "dk", "dv")}
    for s_, h in ((shortest, 5), (longest, 17)):
        r = oracle.attention_backward(cut(q, s_, h), cut(k, s_, h), cut(v, s_, h), cut(do, s_, h), causal=True,
                                      scale=scale)
        for n_, g_, r_ in zip(("dq", "dk", "dv"), (dq, dk, dv), r):
            got[n_].append(to64(cut(g_, s_, h)).ravel()), ref[n_].append(r_.ravel())
    for n_ in ("dq", "dk", "dv"):
        check(f"varlen full {n_}", np.concatenate(got[n_]), np.concatenate(ref[n_]), BF16_MAX, BF16_MEAN)


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


@pytest.mark.parametrize("H,Hkv,d,max_blocks", [(16, 4, 64, 12), (32, 8, 128, 32)])
def test_decode_gqa_drifting_scores(H, Hkv, d, max_blocks):
    """Grouped-head decode on scores that grow along every sequence (drift as
    in drifting_inputs): the per-tile rescale inside each split and the merge
    of splits whose maxima lie far apart, with half-page splits (a small block
    table) and whole-page splits (8 sequences x 32 pages x 8 key/value heads)."""
    lens = [1, 257, 700, 3000] if max_blocks == 12 else [1, 255, 256, 257, 700, 3000, 6001, 8191]
    p = workloads.paged_inputs(num_seqs=len(lens), H=H, Hkv=Hkv, d=d, max_blocks=max_blocks, seed=70 + d,
                               seq_lens=lens, poison=True, spare_pages=2, drift=16.0)
    print(f"[decode gqa drift] H={H} Hkv={Hkv} d={d} max_blocks={max_blocks}", flush=True)
    _decode_compare(f"decode drift H={H} Hkv={Hkv} d={d}", p)


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


@pytest.mark.parametrize("Hkv", [8, 2])
def test_decode_stale_workspace(Hkv):
    """A caller's workspace that holds NaN in every word (as left by other
    work): partials past each sequence's last split are never used."""
    lens = [1, 255, 700, 2000, 1]
    p = workloads.paged_inputs(num_seqs=len(lens), H=8, Hkv=Hkv, d=128, max_blocks=12, seed=23, seq_lens=lens,
                               poison=True, spare_pages=2)
    p.seq_lens[4] = 0
    qd, pool, bt, sl = cuda(p.q, p.kv_pool, p.block_table, p.seq_lens)
    need = fa().decode_workspace_bytes(len(lens), 8, 128, 12)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)  # every fp32 word is a NaN
    o, lse = fa().decode_paged(qd, pool, bt, sl, workspace=ws)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_paged(p.q, p.kv_pool, p.block_table, p.seq_lens, page_size=p.page_size)
    assert (o[4] == 0).all() and torch.isneginf(lse[4]).all()
    keep = [0, 1, 2, 3]
    assert torch.isfinite(o[keep].float()).all()
    check(f"decode stale workspace Hkv={Hkv} O", to64(o)[keep], ro[keep], BF16_MAX, BF16_MEAN)
    check(f"decode stale workspace Hkv={Hkv} LSE", to64(lse)[keep], rl[keep], LSE_MAX)


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


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_paged_spiked_prefix(causal):
    """Chunked prefill where cached keys 600..619 of the first sequence (in
    its prefix) score far above the rest: that sequence's workgroups take the
    d = 128 forward's exact-max loop through the block table, the second
    sequence's do not."""
    chunks, ctx = [300, 200], [1000, 700]
    p = workloads.prefill_inputs(chunks, ctx, H=8, Hkv=2, d=128, seed=91)
    q, pool = workloads.add_pool_spike(p.q, p.kv_pool, p.block_table, 0, range(600, 620),
                                       workloads.spike_direction(128, 92))
    p = workloads.PrefillInputs(q, p.cu_seqlens_q, pool, p.block_table, p.seq_lens_k, p.page_size)
    print(f"[prefill spike] causal={causal}", flush=True)
    _prefill_compare("prefill spike", p, causal)


def test_prefill_paged_full_size():
    """The chunked prefill the bench times (8 chunks of 2048 queries on 3875 ..
    7530 cached keys, 32 query heads on 8 key/value heads, 256-token pages,
    same seed), at full size in that launch configuration; every query head
    of two key/value groups of two sequences (the longest and the shortest
    cache) is compared element by element with the oracle run on that
    sequence and group alone."""
    chunks, ctx = workloads.prefill_shapes()
    H, Hkv, d = 32, 8, 128
    g = H // Hkv
    print(f"[prefill full] chunks={chunks} ctx={ctx}", flush=True)
    p = workloads.prefill_inputs(chunks, ctx, H=H, Hkv=Hkv, d=d, seed=workloads.PREFILL_SEED)
    qd, pool, bt, sl, cu = cuda(p.q, p.kv_pool, p.block_table, p.seq_lens_k, p.cu_seqlens_q)
    o, lse = fa().prefill_paged(qd, pool, bt, sl, cu, max(chunks), causal=True)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    cuq = p.cu_seqlens_q.tolist()
    got_o, ref_o, got_l, ref_l = [], [], [], []
    for b, j in ((int(np.argmax(ctx)), 0), (int(np.argmin(ctx)), Hkv - 1)):
        t0, t1 = cuq[b], cuq[b + 1]
        heads = slice(g * j, g * (j + 1))
        ro, rl = oracle.prefill_paged(p.q[t0:t1, heads], p.kv_pool[:, :, :, j:j + 1], p.block_table[b:b + 1],
                                      p.seq_lens_k[b:b + 1], torch.tensor([0, t1 - t0], dtype=torch.int32),
                                      causal=True, scale=1 / math.sqrt(d), page_size=p.page_size)
        got_o.append(to64(o[t0:t1, heads]).ravel()), ref_o.append(ro.ravel())
        got_l.append(to64(lse[heads, t0:t1]).ravel()), ref_l.append(rl.ravel())
    check("prefill full O", np.concatenate(got_o), np.concatenate(ref_o), BF16_MAX, BF16_MEAN)
    check("prefill full LSE", np.concatenate(got_l), np.concatenate(ref_l), LSE_MAX)


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


def test_forward_rope_full_size():
    """The timed RoPE launch: causal [1,32,16384,128] with tables for positions
    0..16383; two whole heads (first and last) and sampled rows of three more."""
    w = workloads.CONFIGS["c2a"]
    q, k, v = workloads.workload_inputs(w)
    c, s = workloads.rope_tables(w.N, w.d)
    print("[rope full] 1x32x16384x128 causal", flush=True)
    o, lse = fa().forward_rope(*cuda(q, k, v, c, s), causal=True, scale=w.scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    pos = np.arange(w.N)
    rng = np.random.default_rng(5)
    rows = sorted(set([0, 1, 63, 64, 255, 256, 8191, w.N - 129, w.N - 1] + rng.integers(0, w.N, 40).tolist()))
    got_o, ref_o, got_l, ref_l = [], [], [], []
    for h in (0, 1, w.H // 2, w.H - 2, w.H - 1):
        qr = oracle.apply_rope_bf16(q[0, h], pos, c, s)
        kr = oracle.apply_rope_bf16(k[0, h], pos, c, s)
        if h in (0, w.H - 1):
            ro, rl = oracle.attention_forward(qr, kr, v[0, h], causal=True, scale=w.scale)
            go, gl = to64(o[0, h]), to64(lse[0, h])
        else:
            ro, rl = oracle.attention_forward_rows(qr, kr, v[0, h], rows, causal=True, scale=w.scale)
            go, gl = to64(o[0, h])[rows], to64(lse[0, h])[rows]
        got_o.append(go.ravel()), ref_o.append(ro.ravel()), got_l.append(gl.ravel()), ref_l.append(rl.ravel())
    check("rope full O", np.concatenate(got_o), np.concatenate(ref_o), BF16_MAX, BF16_MEAN)
    check("rope full LSE", np.concatenate(got_l), np.concatenate(ref_l), LSE_MAX)


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


def test_varlen_too_small_max_seqlen_is_flagged():
    """A max_seqlen below a packed sequence's length cannot be seen on the host
    (cu_seqlens lives on the device): the kernels then compute that sequence
    only up to max_seqlen and write NaN into its rows, forward and backward,
    while the other sequences stay exact."""
    lens, H, Hkv, d = [300, 700], 4, 2, 128
    cu, q, k, v, do = workloads.varlen_inputs(lens, H, Hkv, d, seed=23, with_dout=True)
    cud, qd, kd, vd, dod = cuda(cu, q, k, v, do)
    o, lse = fa().forward_varlen(qd, kd, vd, cud, 500, causal=True)
    torch.cuda.synchronize()
    assert torch.isnan(o[300:800].float()).all() and torch.isnan(lse[:, 300:800]).all()
    ro, rl = oracle.attention_forward_varlen(q, k, v, cu, causal=True, scale=1 / math.sqrt(d))
    check("short sequence O", to64(o[:300]), ro[:300], BF16_MAX, BF16_MEAN)
    check("short sequence LSE", to64(lse[:, :300]), rl[:, :300], LSE_MAX)
    o2, lse2 = fa().forward_varlen(qd, kd, vd, cud, 700, causal=True)
    dq, dk, dv = fa().backward_varlen(qd, kd, vd, o2, dod, lse2, cud, 500, causal=True)
    torch.cuda.synchronize()
    for g_ in (dq, dk, dv):
        assert torch.isnan(g_[300:800].float()).all()
        assert torch.isfinite(g_[:300].float()).all()


def test_rope_operands_are_the_exact_rotation_rounded():
    """One key per head (N = 1), so the logsumexp is scale·q_rot·k_rot: with
    random (not unit-norm) fp32 table entries over 2048 heads, about 500k
    features are rotated, a few of them within fp32 error of a bf16 rounding
    boundary.  A feature rounded to the other bf16 neighbour than the exact
    rotation moves its head's logsumexp by ~1e-3; exact rounding leaves only
    the fp32 accumulation of the products (~1e-6)."""
    H, d = 2048, 128
    g = torch.Generator().manual_seed(61)
    q = torch.randn(1, H, 1, d, generator=g).to(torch.bfloat16)
    k = torch.randn(1, H, 1, d, generator=g).to(torch.bfloat16)
    v = torch.randn(1, H, 1, d, generator=g).to(torch.bfloat16)
    c = torch.randn(1, d // 2, generator=g)
    s = torch.randn(1, d // 2, generator=g)
    for interleaved in (False, True):
        o, lse = fa().forward_rope(*cuda(q, k, v, c, s), causal=True, interleaved=interleaved)
        torch.cuda.synchronize()
        ro, rl = oracle.attention_forward_rope(q, k, v, c, s, causal=True, interleaved=interleaved)
        check(f"rope exact rounding LSE interleaved={interleaved}", to64(lse), rl, 1e-4)
        assert torch.equal(o.cpu(), v)  # one key: O is its V row


# ------------------------------------------------------- seeded random sweeps
def _random_dense_cases(count=16, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        hkv = int(rng.choice([1, 2, 4]))
        cases.append((int(rng.integers(1, 3)), hkv * int(rng.choice([1, 2, 4])), hkv, int(rng.integers(1, 900)),
                      int(rng.choice([64, 128])), bool(rng.integers(0, 2)), 300 + i))
    return cases


@pytest.mark.parametrize("case", _random_dense_cases(), ids=lambda c: "B%d_H%d_kv%d_N%d_d%d_%s" % (
    c[0], c[1], c[2], c[3], c[4], "causal" if c[5] else "full"))
def test_forward_random_shapes(case):
    """Seeded random shapes through the forward (batch 1-2, 1-16 query heads on
    1-4 key/value heads, 1-899 queries, d = 64 or 128, causal or not), every
    output element against the fp64 oracle: lengths that are not multiples of
    the 16-, 32- and 64-row blocks of either forward kernel."""
    B, H, Hkv, N, d, causal, seed = case
    print(f"[random fwd] B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal}", flush=True)
    q, k, v = workloads.gqa_inputs(B, H, Hkv, N, d, "bf16", seed=seed)
    o, lse = fa().forward(*cuda(q, k, v), causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward_gqa(q, k, v, causal=causal, scale=1 / math.sqrt(d))
    check("random O", to64(o), ro, BF16_MAX, BF16_MEAN)
    check("random LSE", to64(lse), rl, LSE_MAX)


def _random_varlen_cases(count=6, seed=2027):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        n = int(rng.integers(1, 6))
        lens = [int(x) for x in rng.integers(0, 700, n)]
        lens[int(rng.integers(0, n))] = max(lens[0], 1)  # at least one non-empty sequence
        hkv = int(rng.choice([1, 2, 4]))
        cases.append((lens, hkv * int(rng.choice([1, 2])), hkv, int(rng.choice([64, 128])), bool(rng.integers(0, 2)),
                      400 + i))
    return cases


@pytest.mark.parametrize("case", _random_varlen_cases(), ids=lambda c: "n%d_H%d_kv%d_d%d_%s" % (
    len(c[0]), c[1], c[2], c[3], "causal" if c[4] else "full"))
def test_varlen_random_batches(case):
    """Seeded random packed batches (1-5 sequences of 0-699 tokens, grouped or
    not, d = 64 or 128, causal or not): forward and backward, every element
    against the oracle."""
    lens, H, Hkv, d, causal, seed = case
    _varlen_compare(lens, H, Hkv, d, causal, seed=seed)

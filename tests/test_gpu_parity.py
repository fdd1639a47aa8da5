"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle on
the same seeded inputs.

Small shapes are compared element by element over every output; the full
configurations (16K and 32K forward, the 8K backward) are run on the GPU at
full size, in the launch configuration the bench times, and compared on
whole heads plus sampled rows that the oracle computes one by one.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import (BF16_MAX, BF16_MEAN, F32_MAX, LSE_MAX, bf16_rounding_var, check,
                          check_operand_rounded, to64)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X")
    import exact_attention_fwd_amd as fa  # noqa: F401  (fails loudly if libfa.so is missing)
    assert "gfx950" in torch.cuda.get_device_properties(0).gcnArchName
    yield


def fa():
    import exact_attention_fwd_amd
    return exact_attention_fwd_amd


def cuda(*ts):
    return [t.to(DEV) for t in ts]


def _fwd_compare(name, q, k, v, causal, scale, heads=None, rows=None, f32=False):
    """Run the GPU forward on full inputs; compare selected heads fully and
    (optionally) sampled rows of other heads."""
    qd, kd, vd = cuda(q, k, v)
    o, lse = fa().forward(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    B, H, N, d = q.shape
    qf, kf, vf = (x.reshape(B * H, N, d) for x in (q, k, v))
    of, lf = o.reshape(B * H, N, d), lse.reshape(B * H, N)
    heads = range(B * H) if heads is None else heads
    got_o, ref_o, got_l, ref_l = [], [], [], []
    for h in heads:
        ro, rl = oracle.attention_forward(qf[h], kf[h], vf[h], causal=causal, scale=scale)
        got_o.append(to64(of[h])), ref_o.append(ro), got_l.append(to64(lf[h])), ref_l.append(rl)
    if rows:
        for h, rr in rows.items():
            ro, rl = oracle.attention_forward_rows(qf[h], kf[h], vf[h], rr, causal=causal, scale=scale)
            got_o.append(to64(of[h][rr])), ref_o.append(ro), got_l.append(to64(lf[h][rr])), ref_l.append(rl)
    go, ro = np.concatenate([x.ravel() for x in got_o]), np.concatenate([x.ravel() for x in ref_o])
    gl, rl = np.concatenate([x.ravel() for x in got_l]), np.concatenate([x.ravel() for x in ref_l])
    if f32:
        check(f"{name} O", go, ro, F32_MAX)
    else:
        check(f"{name} O", go, ro, BF16_MAX, BF16_MEAN)
    check(f"{name} LSE", gl, rl, LSE_MAX)


def test_c0_fp32_forward():
    w = workloads.CONFIGS["c0"]
    q, k, v = workloads.workload_inputs(w)
    _fwd_compare("c0", q, k, v, w.causal, w.scale, f32=True)


def test_c1_causal_forward_all_heads():
    w = workloads.CONFIGS["c1"]
    q, k, v = workloads.workload_inputs(w)
    _fwd_compare("c1", q, k, v, w.causal, w.scale)


def _sample_rows(N, seed, count=48):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 63, 64, 127, 128, 129, N // 2, N - 129, N - 128, N - 65, N - 64, N - 2, N - 1]
    return sorted(set([r for r in fixed if 0 <= r < N] + rng.integers(0, N, count).tolist()))


@pytest.mark.parametrize("cfg", ["c2a", "c2b", "c2c"])
def test_c2_long_forward_full_size(cfg):
    w = workloads.CONFIGS[cfg]
    print(f"[{cfg}] generating {w.B}x{w.H}x{w.N}x{w.d}", flush=True)
    q, k, v = workloads.workload_inputs(w)
    BH = w.B * w.H
    full = [0, BH - 1]
    rows = {h: _sample_rows(w.N, 17 + h) for h in (1, BH // 2, BH - 2)}
    _fwd_compare(cfg, q, k, v, w.causal, w.scale, heads=full, rows=rows)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 7, 63, 64, 100, 129, 255, 257, 1000])
def test_odd_lengths_bf16(N, causal, d):
    q, k, v = workloads.attention_inputs(1, 3, N, d, "bf16", seed=N * 7 + d + int(causal))
    _fwd_compare(f"bf16 N={N} d={d} causal={causal}", q, k, v, causal, 1 / math.sqrt(d))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 33, 200])
def test_odd_lengths_fp32(N, d):
    for causal in (False, True):
        q, k, v = workloads.attention_inputs(2, 1, N, d, "f32", seed=N + d)
        _fwd_compare(f"f32 N={N} d={d} causal={causal}", q, k, v, causal, 1 / math.sqrt(d), f32=True)


def test_batch_and_explicit_scale():
    q, k, v = workloads.attention_inputs(3, 5, 300, 128, "bf16", seed=99)
    _fwd_compare("B=3 H=5 scale=0.3", q, k, v, True, 0.3)
    qd, kd, vd = cuda(q, k, v)
    a = fa().forward(qd, kd, vd, causal=False)
    b = fa().forward(qd, kd, vd, causal=False, scale=1 / math.sqrt(128))
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [300, 1000])
def test_drifting_scores_forward(N, causal, d):
    """Scores that grow along the key axis (about 8 rescales of the running
    maximum per row over the sequence): the lazy-rescale path of the online
    softmax, taken tile after tile, against the two-pass definition."""
    q, k, v = workloads.drifting_inputs(1, 2, N, d, drift=4.0, seed=11 * N + d)
    _fwd_compare(f"drift N={N} d={d} causal={causal}", q, k, v, causal, 1 / math.sqrt(d))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("drift", [12.0, 40.0])
def test_steep_scores_forward(drift, causal):
    """Scores that climb by about 40 (drift 12) or 130 (drift 40) powers of
    two per 64-key tile: far past what the d = 128 forward bounds with its
    row-sum check, so its workgroups must fall back to the exact running max
    (with drift 40, 2^(s - m) against an earlier tile's reference is not even
    finite in fp32)."""
    q, k, v = workloads.drifting_inputs(1, 2, 300, 128, drift=drift, seed=int(drift))
    _fwd_compare(f"steep drift={drift} causal={causal}", q, k, v, causal, 1 / math.sqrt(128))


@pytest.mark.parametrize("height", [3.0, 8.0])
@pytest.mark.parametrize("causal", [False, True])
def test_spiked_keys_forward(causal, height):
    """A band of keys (700..719 of 1000) scoring about height·128 above the
    rest: with height 3 a one-tile jump of ~50 powers of two, with height 8
    ~130.  Causal rows before the band never see it, the others do, so some
    workgroups of one launch keep the row-sum check and others fall back."""
    for d in (64, 128):
        q, k, v = workloads.spiked_inputs(1, 2, 1000, d, 700, 720, height=height, seed=int(height) + d)
        _fwd_compare(f"spike d={d} height={height} causal={causal}", q, k, v, causal, 1 / math.sqrt(d))


def test_forward_is_deterministic_and_n0_is_noop():
    q, k, v = cuda(*workloads.attention_inputs(1, 8, 2000, 128, "bf16", seed=5))
    a = fa().forward(q, k, v, causal=True)
    b = fa().forward(q, k, v, causal=True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    z = torch.zeros(1, 2, 0, 128, dtype=torch.bfloat16, device=DEV)
    o, lse = fa().forward(z, z, z, causal=True)
    assert o.shape == z.shape and lse.shape == (1, 2, 0)


# ------------------------------------------------------------------ backward
def _bwd_compare(name, q, k, v, do, causal, scale, heads=None):
    qd, kd, vd, dod = cuda(q, k, v, do)
    o, lse = fa().forward(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa().backward(qd, kd, vd, o, dod, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    B, H, N, d = q.shape
    flat = lambda x: x.reshape(B * H, N, d)
    heads = range(B * H) if heads is None else heads
    got = {n: [] for n in ("dq", "dk", "dv")}
    ref = {n: [] for n in ("dq", "dk", "dv")}
    for h in heads:
        r = oracle.attention_backward(flat(q)[h], flat(k)[h], flat(v)[h], flat(do)[h], causal=causal, scale=scale)
        for n_, g_, r_ in zip(("dq", "dk", "dv"), (dq, dk, dv), r):
            got[n_].append(to64(flat(g_.cpu())[h]).ravel())
            ref[n_].append(r_.ravel())
    for n_ in ("dq", "dk", "dv"):
        check(f"{name} {n_}", np.concatenate(got[n_]), np.concatenate(ref[n_]), BF16_MAX, BF16_MEAN)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 7, 100, 257, 300, 700])
def test_backward_small(N, causal, d):
    q, k, v, do = workloads.attention_inputs(1, 2, N, d, "bf16", seed=3 * N + d, with_dout=True)
    _bwd_compare(f"bwd N={N} d={d} causal={causal}", q, k, v, do, causal, 1 / math.sqrt(d))


def _operand_sigma(q, k, v, do, o_saved, lse, causal, scale):
    """Per-element standard deviations that rounding the gradient products'
    operands to bf16 implies, from the exact P and dS of one head (fp64):
    P in dV = Pᵀ dO; dS = P ∘ (dP − D) in dK = scale·dSᵀ Q and dQ = scale·dS K
    (D from the saved output, as both sides take it)."""
    n = q.shape[0]
    p = np.exp(scale * (q @ k.T) - lse[:, None])
    if causal:
        p = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], 0.0, p)
    ds = p * (do @ v.T - (do * o_saved).sum(axis=1)[:, None])
    vp, vs = bf16_rounding_var(p), bf16_rounding_var(ds)
    return (np.sqrt(scale ** 2 * (vs @ (k * k))), np.sqrt(scale ** 2 * (vs.T @ (q * q))),
            np.sqrt(vp.T @ (do * do)))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_drifting_scores_backward(causal, d):
    """The backward on scores that grow along the key axis: most rows'
    probabilities P = 2^(s·scale·log2e − LSE·log2e) span many orders of
    magnitude and the last keys collect the attention of nearly every query
    (|dK|, |dV| up to ≈ 15).  Both sides take the same saved forward (the
    oracle's O rounded to bf16, its LSE in fp32) and the oracle forms D from
    that O.  Bound: the stated one beyond each element's output rounding and
    6 standard deviations of the bf16 rounding of the products' operands
    (P, dS), which for keys holding hundreds of probabilities near 1 exceeds
    2e-2 by itself; mean-abs as stated."""
    scale = 1 / math.sqrt(d)
    q, k, v = workloads.drifting_inputs(1, 2, 300, d, drift=4.0, seed=600 + d + causal)
    do = workloads.attention_inputs(1, 2, 300, d, "bf16", seed=610 + d, with_dout=True)[3]
    ro, rl = oracle.attention_forward(q, k, v, causal=causal, scale=scale)
    o_saved = torch.from_numpy(ro).to(torch.bfloat16)
    lse_saved = torch.from_numpy(rl).to(torch.float32)
    qd, kd, vd, dod, od, ld = cuda(q, k, v, do, o_saved, lse_saved)
    dq, dk, dv = fa().backward(qd, kd, vd, od, dod, ld, causal=causal, scale=scale)
    torch.cuda.synchronize()
    r = oracle.attention_backward(q, k, v, do, causal=causal, scale=scale, out=o_saved)
    sig = [[], [], []]
    for h in range(2):
        s3 = _operand_sigma(to64(q[0, h]), to64(k[0, h]), to64(v[0, h]), to64(do[0, h]), to64(o_saved[0, h]),
                            rl[0, h], causal, scale)
        for i in range(3):
            sig[i].append(s3[i])
    name = f"bwd drift d={d} causal={causal}"
    for i, (nm, g) in enumerate(zip(("dq", "dk", "dv"), (dq, dk, dv))):
        check_operand_rounded(f"{name} {nm}", to64(g.cpu())[0], r[i][0], np.stack(sig[i]))


@pytest.mark.parametrize("d", [64, 128])
def test_many_units(d):
    """B=16, H=32: 512 (batch, head) units, 64 per XCD, so every kernel maps
    its blocks through the grouped order (groups of units, rank by rank)
    rather than rank by rank over all units; every head is compared."""
    q, k, v, do = workloads.attention_inputs(16, 32, 130, d, "bf16", seed=500 + d, with_dout=True)
    _fwd_compare(f"B=16 H=32 N=130 d={d}", q, k, v, True, 1 / math.sqrt(d))
    _bwd_compare(f"bwd B=16 H=32 N=130 d={d}", q, k, v, do, True, 1 / math.sqrt(d))


def test_c3_backward_full_size():
    w = workloads.CONFIGS["c3"]
    print(f"[c3] generating {w.B}x{w.H}x{w.N}x{w.d}", flush=True)
    q, k, v, do = workloads.workload_inputs(w)
    # four whole heads, two of each batch entry (flattened index b·H + h)
    _bwd_compare("c3", q, k, v, do, w.causal, w.scale, heads=[0, 9, w.H, w.B * w.H - 1])


def test_backward_is_deterministic():
    q, k, v, do = cuda(*workloads.attention_inputs(1, 4, 1500, 128, "bf16", seed=8, with_dout=True))
    o, lse = fa().forward(q, k, v, causal=True)
    a = fa().backward(q, k, v, o, do, lse, causal=True)
    b = fa().backward(q, k, v, o, do, lse, causal=True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# -------------------------------------------------------------------- decode
def _decode_compare(name, p, scale=None):
    d = p.q.shape[-1]
    scale = 1 / math.sqrt(d) if scale is None else scale
    qd, pool, bt, sl = cuda(p.q, p.kv_pool, p.block_table, p.seq_lens)
    o, lse = fa().decode_paged(qd, pool, bt, sl, scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_paged(p.q, p.kv_pool, p.block_table, p.seq_lens, scale=scale, page_size=p.page_size)
    check(f"{name} O", to64(o.cpu()), ro, BF16_MAX, BF16_MEAN)
    check(f"{name} LSE", to64(lse.cpu()), rl, LSE_MAX)
    return o, lse


def test_c4_decode_full():
    w = workloads.CONFIGS["c4"]
    _decode_compare("c4", workloads.workload_inputs(w))


def test_c4_decode_poisoned_tails_and_spare_pages():
    w = workloads.CONFIGS["c4"]
    p = workloads.workload_inputs(w, poison=True, spare_pages=16)
    o, _ = _decode_compare("c4 poisoned", p)
    assert torch.isfinite(o.float()).all()


@pytest.mark.parametrize("H,d", [(12, 128), (8, 64), (3, 64)])
def test_decode_shapes(H, d):
    lens = [1, 255, 256, 257, 1000, 2048]
    p = workloads.paged_inputs(num_seqs=len(lens), H=H, d=d, max_blocks=9, seed=H + d, seq_lens=lens,
                               poison=True, spare_pages=3)
    _decode_compare(f"decode H={H} d={d}", p)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_drifting_scores(d):
    """Scores that grow along every cached sequence (about 40 in log2 units per
    500 tokens, as drifting_inputs): each split raises its running maximum tile
    after tile, and the splits of one sequence end with maxima up to ~200 apart,
    so most merge weights 2^(m_j − m) underflow to zero."""
    lens = [1, 257, 700, 3000]
    p = workloads.paged_inputs(num_seqs=len(lens), H=8, d=d, max_blocks=12, seed=50 + d, seq_lens=lens,
                               poison=True, spare_pages=2, drift=16.0)
    o, _ = _decode_compare(f"decode drift d={d}", p)
    assert torch.isfinite(o.float()).all()


def test_decode_is_deterministic():
    p = workloads.paged_inputs(num_seqs=4, H=32, d=128, len_lo=300, len_hi=3000, max_blocks=12, seed=4)
    args = cuda(p.q, p.kv_pool, p.block_table, p.seq_lens)
    a = fa().decode_paged(*args)
    b = fa().decode_paged(*args)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_errors_raise():
    x = torch.zeros(1, 1, 8, 128, dtype=torch.float32, device=DEV)
    lse = torch.zeros(1, 1, 8, dtype=torch.float32, device=DEV)
    with pytest.raises(fa().FaError):
        fa().backward(x, x, x, x, x, lse)  # fp32 backward is not provided

"""Pins of the oracle's rotary position embedding: an independent complex-
number formulation, the identity at position 0, pair norms, the relative-
position property of the standard tables, and the reduction of the rotated
forward to the plain forward on pre-rotated inputs."""
import numpy as np
import pytest

import oracle
import workloads


def _tables(rows, d):
    c, s = workloads.rope_tables(rows, d)
    return c.double().numpy(), s.double().numpy()


@pytest.mark.parametrize("interleaved", [False, True])
def test_rope_is_complex_multiplication(rng, interleaved):
    d, n = 8, 11
    c, s = _tables(40, d)
    x = rng.standard_normal((2, n, d))
    pos = rng.integers(0, 40, n)
    got = oracle.apply_rope(x, pos, c, s, interleaved)
    if interleaved:
        z = x[..., 0::2] + 1j * x[..., 1::2]
    else:
        z = x[..., : d // 2] + 1j * x[..., d // 2:]
    w = z * (c[pos] + 1j * s[pos])
    want = np.empty_like(x)
    if interleaved:
        want[..., 0::2], want[..., 1::2] = w.real, w.imag
    else:
        want[..., : d // 2], want[..., d // 2:] = w.real, w.imag
    np.testing.assert_allclose(got, want, atol=1e-15)


def test_position_zero_is_identity_and_pairs_keep_their_norm(rng):
    d = 16
    c, s = _tables(64, d)
    x = rng.standard_normal((5, d))
    np.testing.assert_array_equal(oracle.apply_rope(x, np.zeros(5, int), c, s), x)
    y = oracle.apply_rope(x, np.arange(5) * 7, c, s)
    np.testing.assert_allclose(y[:, :8] ** 2 + y[:, 8:] ** 2, x[:, :8] ** 2 + x[:, 8:] ** 2, atol=1e-12)


@pytest.mark.parametrize("interleaved", [False, True])
def test_scores_depend_only_on_relative_position(rng, interleaved):
    d = 8
    c, s = _tables(200, d)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    def score(i, j):
        return oracle.apply_rope(q[None], [i], c, s, interleaved)[0] @ oracle.apply_rope(k[None], [j], c, s, interleaved)[0]
    for i, j, shift in [(5, 2, 30), (17, 17, 100), (3, 40, 90)]:
        assert abs(score(i, j) - score(i + shift, j + shift)) < 1e-5  # fp32 tables: ~1e-7 per angle


def test_rotated_forward_is_forward_of_rotated_inputs(rng):
    B, H, Hkv, N, d = 1, 4, 2, 9, 8
    c, s = _tables(N, d)
    q, k, v = rng.standard_normal((B, H, N, d)), rng.standard_normal((B, Hkv, N, d)), rng.standard_normal((B, Hkv, N, d))
    o, lse = oracle.attention_forward_rope(q, k, v, c, s, causal=True, rotate=oracle.apply_rope)
    pos = np.arange(N)
    o2, lse2 = oracle.attention_forward_gqa(oracle.apply_rope(q, pos, c, s), oracle.apply_rope(k, pos, c, s), v,
                                            causal=True)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, atol=1e-14)
    # packed form, positions restart per sequence
    cu = np.array([0, 4, 9])
    qp = np.concatenate([q[0, :, :4].transpose(1, 0, 2), q[0, :, :5].transpose(1, 0, 2)])
    kp = np.concatenate([k[0, :, :4].transpose(1, 0, 2), k[0, :, :5].transpose(1, 0, 2)])
    vp = np.concatenate([v[0, :, :4].transpose(1, 0, 2), v[0, :, :5].transpose(1, 0, 2)])
    op, _ = oracle.attention_forward_rope(qp, kp, vp, c, s, causal=True, cu_seqlens=cu, rotate=oracle.apply_rope)
    o4, _ = oracle.attention_forward_rope(q[:, :, :4], k[:, :, :4], v[:, :, :4], c, s, causal=True,
                                          rotate=oracle.apply_rope)
    np.testing.assert_allclose(op[:4], o4[0].transpose(1, 0, 2), atol=1e-14)


# ----------------------------------------------- rotation stored as bf16
def test_bf16_rounding_is_nearest_even_on_ties():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: the even one (1) wins;
    # 1 + 3·2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: the even one (1 + 2^-6) wins;
    # just above a tie rounds up, just below rounds down.
    x = np.array([1 + 2.0**-8, 1 + 3 * 2.0**-8, 1 + 2.0**-8 + 2.0**-20, 1 + 2.0**-8 - 2.0**-20, -(1 + 2.0**-8)],
                 dtype=np.float32)
    want = [1.0, 1 + 2.0**-6, 1 + 2.0**-7, 1.0, -1.0]
    cos = np.zeros((1, 1))
    sin = np.zeros((1, 1))
    # through the rotation: x=1 at an angle with cos = the fp32 value above, sin = 0
    for val, w in zip(x, want):
        cos[0, 0], sin[0, 0] = val, 0.0
        got = oracle.apply_rope_bf16(np.array([[1.0, 0.0]]), [0], cos, sin)
        assert got[0, 0] == w and got[0, 1] == 0.0


def test_bf16_rounding_of_fp32_values_matches_torch(rng):
    # torch rounds an fp32 value to bf16 in one step, so on fp32 inputs it is an
    # independent implementation of the same rounding
    import torch
    from oracle.attention import _bf16_rne
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ties = ((np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000) + 0x3F800000).view(np.float32)  # exact halfway values
    for v in (x, ties):
        want = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
        np.testing.assert_array_equal(_bf16_rne(v), want)


def _bf16_neighbours(x):
    """The two bf16 values bracketing each fp64 x (x > 0), found by stepping
    the 8-bit significand of 2^floor(log2 x) — independent of the bit
    arithmetic under test."""
    e = np.floor(np.log2(x))
    ulp = 2.0 ** (e - 7)
    lo = np.floor(x / ulp) * ulp
    return lo, lo + ulp, ulp


def test_bf16_rounding_of_fp64_values_is_nearest_even(rng):
    # values with more than 24 significant bits (not fp32-representable), including
    # ones just off a tie by less than an fp32 ulp, where rounding through fp32 first
    # would land on the tie and could round the other way
    x = np.abs(rng.standard_normal(200000)) * np.exp(rng.uniform(-30, 30, 200000))
    base = (np.arange(1, 3000, dtype=np.uint64) << np.uint64(45)) | np.uint64(1 << 44)  # exact ties
    ties = (base | (np.uint64(0x3FF) << np.uint64(52))).view(np.float64)
    near = np.concatenate([ties + 2.0 ** -40, ties - 2.0 ** -40])
    for v in (x, ties, near):
        got = oracle.attention._bf16_rne(v)
        lo, hi, ulp = _bf16_neighbours(v)
        assert np.all((got == lo) | (got == hi))
        dlo, dhi = v - lo, hi - v
        pick_lo = (dlo < dhi) | ((dlo == dhi) & (np.mod(lo / ulp, 2) == 0))
        np.testing.assert_array_equal(got, np.where(pick_lo, lo, hi))
        np.testing.assert_array_equal(oracle.attention._bf16_rne(-v), -got)
    # one step from fp64, not through fp32: 1 + 2^-8 + 2^-40 is above the tie, so it
    # rounds up, although its nearest fp32 value is the tie itself (which rounds down)
    assert oracle.attention._bf16_rne(np.array([1 + 2.0**-8 + 2.0**-40]))[0] == 1 + 2.0**-7
    with pytest.raises(ValueError):
        oracle.attention._bf16_rne(np.array([2.0**-130]))


def test_bf16_rotation_is_one_rounding_of_the_exact_rotation():
    # x = 1 + 2^-7, cos = 1 + 2^-23, y = 1, sin = 1 + 2^-7 + 2^-23: the exact first feature
    # (1 + 2^-7)(1 + 2^-23) - (1 + 2^-7 + 2^-23) is 2^-30, a bf16 value; products rounded to
    # fp32 one by one would cancel to 0 instead
    c32 = np.float32(1 + 2.0**-23)
    s32 = np.float32(1 + 2.0**-7 + 2.0**-23)
    x = np.array([[1 + 2.0**-7, 1.0]])
    got = oracle.apply_rope_bf16(x, [0], np.array([[c32]]), np.array([[s32]]))
    assert got[0, 0] == 2.0**-30
    # second feature: 2 + 2^-6 + 2^-14 + 2^-22 + 2^-30 exactly, which rounds to 2 + 2^-6 in bf16
    assert got[0, 1] == 2 + 2.0**-6


@pytest.mark.parametrize("interleaved", [False, True])
def test_bf16_rotation_is_the_exact_rotation_rounded(rng, interleaved):
    import torch
    d, n = 64, 300
    c, s = _tables(n, d)
    x = torch.randn(3, n, d, dtype=torch.float32).to(torch.bfloat16).double().numpy()
    pos = np.arange(n)
    exact = oracle.apply_rope(x, pos, c, s, interleaved)
    got = oracle.apply_rope_bf16(x, pos, c, s, interleaved)
    # representable in bf16
    assert np.array_equal(torch.from_numpy(got).to(torch.bfloat16).double().numpy(), got)
    # within half a bf16 ulp (at most 2^-8 of the value: 8 significant bits) of the exact
    # value; and not within 2^-10 everywhere (it is rounded)
    assert np.all(np.abs(got - exact) <= 2.0**-8 * np.abs(exact))
    assert np.any(np.abs(got - exact) > 2.0**-10 * np.abs(exact))
    # position 0 (cos 1, sin 0) leaves the stored bf16 rows unchanged
    np.testing.assert_array_equal(oracle.apply_rope_bf16(x[:, :1], [0], c, s, interleaved), x[:, :1])


def test_default_rotated_forward_uses_the_bf16_rotation(rng):
    B, H, Hkv, N, d = 1, 2, 1, 7, 8
    c, s = _tables(N, d)
    q, k, v = rng.standard_normal((B, H, N, d)), rng.standard_normal((B, Hkv, N, d)), rng.standard_normal((B, Hkv, N, d))
    o, lse = oracle.attention_forward_rope(q, k, v, c, s, causal=False)
    pos = np.arange(N)
    o2, lse2 = oracle.attention_forward_gqa(oracle.apply_rope_bf16(q, pos, c, s), oracle.apply_rope_bf16(k, pos, c, s),
                                            v, causal=False)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


# ------------------------------------------ planted mistakes in the rotation
def _rope_pins():
    """The pins above as one predicate (used to show they catch planted mistakes)."""
    rng = np.random.default_rng(9)
    try:
        for inter in (False, True):
            test_rope_is_complex_multiplication(rng, inter)
        test_bf16_rounding_of_fp64_values_is_nearest_even(rng)
        test_bf16_rotation_is_one_rounding_of_the_exact_rotation()
    except AssertionError:
        return False
    return True


def _truncate_bf16(x):
    u = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64) & ~np.uint64((1 << 45) - 1)
    return u.view(np.float64)


def _through_fp32(x):
    import torch
    return torch.from_numpy(np.asarray(x, dtype=np.float64).astype(np.float32)).to(torch.bfloat16).double().numpy()


_exact_rope = oracle.attention.apply_rope


def _sin_sign_flipped(x, positions, cos, sin, interleaved=False):
    return _exact_rope(x, positions, cos, -np.asarray(sin, dtype=np.float64), interleaved)


def _pairs_swapped(x, positions, cos, sin, interleaved=False):
    return _exact_rope(x, positions, cos, sin, not interleaved)


ROPE_MUTATIONS = {
    "bf16 truncation": ("_bf16_rne", _truncate_bf16),
    "rounded through fp32 first": ("_bf16_rne", _through_fp32),
    "sine sign flipped": ("apply_rope", _sin_sign_flipped),
    "half-split and interleaved pairs swapped": ("apply_rope", _pairs_swapped),
}


def test_unmutated_rope_passes_pins():
    assert _rope_pins()


@pytest.mark.parametrize("name", sorted(ROPE_MUTATIONS))
def test_rope_pins_catch_mutation(monkeypatch, name):
    attr, fn = ROPE_MUTATIONS[name]
    monkeypatch.setattr(oracle.attention, attr, fn)
    monkeypatch.setattr(oracle, attr, fn, raising=False)
    assert not _rope_pins(), f"mutation '{name}' slipped past the rotation pins"

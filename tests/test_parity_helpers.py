"""CPU checks of the tolerance helpers the GPU parity tests use."""
import numpy as np
import torch

from tests.parity import bf16_half_ulp, check_rounded


def test_half_ulp_is_half_the_bf16_spacing(rng):
    x = rng.standard_normal(5000) * np.exp(rng.uniform(-10, 10, 5000))
    b = torch.from_numpy(x).to(torch.bfloat16)
    up = torch.nextafter(b.abs(), torch.full_like(b, float("inf"))).double().numpy()
    spacing = up - b.abs().double().numpy()  # bf16 spacing just above |rounded x|
    # same binade as |x| except when rounding carried into the next power of two
    same = np.floor(np.log2(np.abs(x))) == np.floor(np.log2(b.abs().double().numpy()))
    np.testing.assert_array_equal(bf16_half_ulp(x)[same], spacing[same] / 2)
    assert bf16_half_ulp(np.array([0.0]))[0] == 0.0


def test_check_rounded_accepts_the_rounded_exact_value_and_rejects_more(rng):
    ref = rng.standard_normal(2000)
    ref[:20] *= 12.0  # a few values past 8, where half an ulp exceeds 2e-2
    rounded = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    check_rounded("exact rounded", rounded, ref)            # the best a bf16 output can do passes
    bad = rounded.copy()
    bad[7] += 0.05 + bf16_half_ulp(ref[7:8])[0]             # 5e-2 beyond the output rounding
    try:
        check_rounded("too far", bad, ref)
    except AssertionError:
        pass
    else:
        raise AssertionError("an error of 5e-2 beyond half an ulp was accepted")


def test_rounding_variance_matches_bf16_rounding(rng):
    """bf16_rounding_var: the variance of the RNE rounding error, binade by
    binade (ulp^2 / 12), against the error of torch's own rounding of many
    values spread uniformly inside one binade, and exactly 0 at 0."""
    from tests.parity import bf16_rounding_var
    for e in (-12, -1, 0, 3):
        x = np.exp2(e) * (1.0 + rng.uniform(0.0, 1.0, 200000))
        err = torch.from_numpy(x).to(torch.bfloat16).double().numpy() - x
        want = bf16_rounding_var(x)
        assert np.allclose(want, want[0])               # one binade: one ulp
        assert want[0] == 2.0 ** (2 * (e - 7)) / 12.0
        assert abs(err.var() / want[0] - 1.0) < 0.02
    assert bf16_rounding_var(np.array([0.0]))[0] == 0.0

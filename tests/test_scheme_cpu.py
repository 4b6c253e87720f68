"""CPU checks of the precision-scheme helper the bit-exact GPU tests use
(tests/scheme.py), and of the per-j bar of the partial-permutation check."""
import numpy as np
import pytest

from scheme import P6_GPU_BAR, p_compose, scheme_scalar

# p^5(2^-j) for j = 3..6: the signed-permutation closed form of the synthesis
# note's quintic (section 4) with its tuned coefficients, as the pins table
# lists them.
P5_VALUES = {3: 0.688140, 4: 1.070524, 5: 1.132924, 6: 0.902526}


@pytest.mark.parametrize("j", sorted(P5_VALUES))
def test_p_compose_closed_form_values(j):
    assert abs(p_compose(2.0 ** -j, 5) - P5_VALUES[j]) < 5e-7


@pytest.mark.parametrize("j", sorted(P6_GPU_BAR))
def test_partial_permutation_bar_fits_the_scheme(j):
    """Each bar holds the scheme's own value, and is the pins' 1e-2 wherever
    the scheme meets 1e-2 (the Newton-Schulz bar 2e-2 only where it cannot)."""
    exact = p_compose(2.0 ** -j, 5)
    dev = max(abs(float(scheme_scalar(2.0 ** -j, 5, fused)) - exact) / exact for fused in (False, True))
    assert dev <= P6_GPU_BAR[j]
    assert (P6_GPU_BAR[j] == 1e-2) == (dev <= 1e-2)
    assert P6_GPU_BAR[j] <= 2e-2


def test_scheme_zero_and_power_of_two_scaling():
    """Zero stays zero; every rounding the scheme makes commutes with a
    power-of-two scale of the input that keeps the values normal, so the
    first step on 2^-k x equals 2^-k times a step whose products are scaled
    alike (checked through the linear term: for tiny x the step is a*x)."""
    assert scheme_scalar(0.0, 5) == 0.0
    x = np.float32(2.0 ** -40)
    assert scheme_scalar(x, 1, fused=True) == np.float32(np.float64(np.float32(3.4445)) * np.float64(x))

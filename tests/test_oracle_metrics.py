"""Pins of the two error measures every float parity test uses, by values worked out by
hand: the normwise max |got - ref| / max |ref|, and the elementwise
max |got - ref| / (|ref| + rms(ref)). A plausible slip (a mean instead of a max, the
scale taken from `got`, a missing absolute value, an rms over the differences) changes
one of the values below."""
import math

import numpy as np

import oracle


def test_normwise_hand_values():
    ref = np.array([1.0, 2.0, -4.0])
    got = np.array([1.0, 2.5, -3.0])
    # differences 0, 0.5, 1; max |ref| = 4
    assert oracle.normwise_rel_err(got, ref) == 0.25
    # the scale comes from ref, not from got: swapping the two changes it (max |got| = 3)
    assert math.isclose(oracle.normwise_rel_err(ref, got), 1.0 / 3.0, rel_tol=0, abs_tol=1e-15)
    # sign of the difference and of ref do not matter
    assert oracle.normwise_rel_err(-got, -ref) == 0.25
    # 2-D input: the max runs over all elements
    assert oracle.normwise_rel_err(np.array([[0.0, 3.0], [1.0, 1.0]]),
                                   np.array([[0.0, 2.0], [-8.0, 1.0]])) == 9.0 / 8.0
    # degenerate cases: equal arrays, an all-zero reference (absolute difference), empty
    assert oracle.normwise_rel_err(ref, ref) == 0.0
    assert oracle.normwise_rel_err(np.array([0.5, -1.5]), np.zeros(2)) == 1.5
    assert oracle.normwise_rel_err(np.zeros(0), np.zeros(0)) == 0.0


def test_elementwise_hand_values():
    ref = np.array([1.0, 2.0, -4.0])
    got = np.array([1.0, 2.5, -3.0])
    rms = math.sqrt((1.0 + 4.0 + 16.0) / 3.0)          # sqrt(7)
    # per element: 0 / (1 + rms), 0.5 / (2 + rms), 1 / (4 + rms); the last is largest
    want = 1.0 / (4.0 + rms)
    assert math.isclose(oracle.elementwise_rel_err(got, ref), want, rel_tol=1e-15)
    assert math.isclose(want, 0.150471, rel_tol=1e-5)
    # a large error on a small output: 0.1 / (0.01 + rms([0.01, 10])) with
    # rms = sqrt((1e-4 + 100) / 2)
    ref2 = np.array([0.01, 10.0])
    got2 = np.array([0.11, 10.0])
    rms2 = math.sqrt((1e-4 + 100.0) / 2.0)
    assert math.isclose(oracle.elementwise_rel_err(got2, ref2), 0.1 / (0.01 + rms2), rel_tol=1e-12)
    # ... which the normwise measure reports as 0.1 / 10
    assert math.isclose(oracle.normwise_rel_err(got2, ref2), 0.01, rel_tol=1e-12)
    assert oracle.elementwise_rel_err(ref, ref) == 0.0
    assert oracle.elementwise_rel_err(np.array([0.25, 0.0]), np.zeros(2)) == 0.25
    assert oracle.elementwise_rel_err(np.zeros(0), np.zeros(0)) == 0.0


def test_bars_against_bf16_rounding():
    """What one bf16 rounding of the output costs under each measure: at most half a
    unit in the last place of an 8-bit significand, 2^-8 relative, inside the 2e-2 bar."""
    rng = np.random.default_rng(0)
    ref = rng.standard_normal(4096)
    import torch
    got = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    assert oracle.normwise_rel_err(got, ref) <= 2.0 ** -8
    assert oracle.elementwise_rel_err(got, ref) <= 2.0 ** -8
    assert oracle.elementwise_rel_err(got, ref) > 0.0

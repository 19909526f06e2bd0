"""Pins for the oracle's tables: PRNG, Hadamard, rotation, codebook, JL matrix.

Every check compares the oracle with something other than itself: published
values (tests/golden), closed forms, brute force or an independent
construction.
"""

import math

import numpy as np
import pytest

from oracle import tables


def test_splitmix64_published_sequence(golden):
    g = golden("splitmix64.txt")
    gen = tables.splitmix64(1234567)
    assert [next(gen) for _ in range(5)] == g["seed_1234567"]


def test_same_seed_same_rotation_and_sketch():
    # same seed -> same matrix (TQ+ guide §3: the deterministic-rotation test)
    for seed in (0, 1, 12345, 2**63 + 7):
        a1, a2 = tables.rotation_signs(seed, 128)
        b1, b2 = tables.rotation_signs(seed, 128)
        assert np.array_equal(a1, b1) and np.array_equal(a2, b2)
        assert np.array_equal(tables.gaussian_matrix(seed, 16, 32), tables.gaussian_matrix(seed, 16, 32))
    r0 = tables.rotation_matrix(0, 64)
    r1 = tables.rotation_matrix(1, 64)
    assert not np.allclose(r0, r1)
    assert not np.array_equal(tables.gaussian_matrix(0, 8, 32), tables.gaussian_matrix(1, 8, 32))


def test_signs_are_balanced_and_both_diagonals_differ():
    d1, d2 = tables.rotation_signs(0, 4096)
    assert set(np.unique(d1)) == {-1, 1}
    assert abs(d1.mean()) < 0.1 and abs(d2.mean()) < 0.1
    assert not np.array_equal(d1, d2)


def _sylvester(d):
    # independent construction: H_{2n} = [[H, H], [H, -H]]
    h = np.array([[1.0]])
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


@pytest.mark.parametrize("d", [2, 4, 8, 16, 32, 128, 256])
def test_hadamard_matches_sylvester_recursion(d):
    assert np.array_equal(tables.hadamard(d), _sylvester(d))


@pytest.mark.parametrize("d", [2, 4, 8, 16])
def test_fwht_matches_brute_force_dense_h(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((5, d))
    brute = np.zeros_like(x)
    for r in range(5):
        for i in range(d):
            acc = 0.0
            for j in range(d):
                acc += (-1.0) ** bin(i & j).count("1") * x[r, j]
            brute[r, i] = acc
    assert np.max(np.abs(tables.fwht(x) - brute)) < 1e-12


@pytest.mark.parametrize("d", [32, 128, 256])
def test_rotation_orthogonal_and_norm_preserving(d):
    R = tables.rotation_matrix(7, d)
    assert np.max(np.abs(R.T @ R - np.eye(d))) < 1e-12
    rng = np.random.default_rng(1)
    x = rng.standard_normal((100, d)) * np.exp(rng.standard_normal(d))
    rx = x @ R.T
    rel = np.abs(np.linalg.norm(rx, axis=1) / np.linalg.norm(x, axis=1) - 1.0)
    assert rel.max() < 1e-6
    # fast structured form D1 * FWHT(D2 * x) / sqrt(d) equals the dense R
    d1, d2 = tables.rotation_signs(7, d)
    fast = d1 * tables.fwht(x * d2) / math.sqrt(d)
    assert np.max(np.abs(fast - rx)) < 1e-12
    # R^T R x = x
    assert np.max(np.abs(rx @ R - x)) < 1e-12


def test_gaussian_matrix_moments():
    S = tables.gaussian_matrix(3, 256, 256)
    assert abs(S.mean()) < 0.01
    assert abs(S.var() - 1.0) < 0.02
    # values are float32-representable
    assert np.array_equal(S, S.astype(np.float32).astype(np.float64))
    # the two Box-Muller outputs of a pair are uncorrelated
    flat = S.ravel()
    assert abs(np.corrcoef(flat[0::2], flat[1::2])[0, 1]) < 0.01


def test_lloyd_max_one_bit_closed_form():
    c = tables.lloyd_max_gaussian(1)
    assert np.allclose(c, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], atol=1e-14)
    assert abs(tables.gaussian_distortion(c) - (1 - 2 / math.pi)) < 1e-12


@pytest.mark.parametrize("bits,key", [(1, 2), (2, 4), (3, 8), (4, 16)])
def test_lloyd_max_matches_max_1960_table(golden, bits, key):
    g = golden("lloyd_max_gaussian.txt")
    c = tables.lloyd_max_gaussian(bits)
    half = c[len(c) // 2:]
    printed = np.array(g[f"levels_{key}"])
    assert np.max(np.abs(half - printed) / printed) < 6e-4
    if f"cuts_{key}" in g:
        cuts = (c[len(c) // 2:-1] + c[len(c) // 2 + 1:]) / 2
        assert np.max(np.abs(cuts - np.array(g[f"cuts_{key}"])) / np.array(g[f"cuts_{key}"])) < 6e-4
    assert abs(tables.gaussian_distortion(c) / g[f"mse_{key}"][0] - 1) < 5e-4


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_lloyd_max_conditions_hold(bits):
    c = tables.lloyd_max_gaussian(bits)
    # symmetric, sorted, and each centroid is the mean of its cell
    assert np.allclose(c, -c[::-1], atol=1e-13)
    assert np.all(np.diff(c) > 0)
    t = [-math.inf] + list((c[:-1] + c[1:]) / 2) + [math.inf]
    for k in range(len(c)):
        a, b = t[k], t[k + 1]
        # conditional mean by numerical integration (independent of the pdf
        # difference formula used inside the iteration)
        lo = max(a, -12.0)
        hi = min(b, 12.0)
        xs = np.linspace(lo, hi, 200001)
        w = np.exp(-0.5 * xs * xs)
        mean = np.trapezoid(xs * w, xs) / np.trapezoid(w, xs)
        assert abs(mean - c[k]) < 1e-8


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_codebook_fp16_and_distortion_targets(golden, bits):
    g = golden("lloyd_max_gaussian.txt")
    c = tables.codebook(bits)
    assert np.array_equal(c, c.astype(np.float16).astype(np.float64))
    assert len(c) == 1 << bits and np.all(np.diff(c) > 0)
    assert np.array_equal(c, -c[::-1])
    tau = tables.thresholds(bits)
    assert np.array_equal(tau, tau.astype(np.float32).astype(np.float64))
    assert tau[len(tau) // 2] == 0.0
    target = g[f"target_mse_bits_{bits}"][0]
    assert abs(tables.gaussian_distortion(c) / target - 1) < 0.02
    # Monte Carlo through the threshold rule
    rng = np.random.default_rng(bits)
    x = rng.standard_normal(2_000_000)
    code = np.searchsorted(tau, x, side="left")  # #(tau < x)
    mse = np.mean((x - c[code]) ** 2)
    assert abs(mse / tables.gaussian_distortion(c) - 1) < 0.01

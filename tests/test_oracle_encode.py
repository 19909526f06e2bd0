"""Pins for the oracle's encoder: packing, norm, quantiser, QJL."""

import math

import numpy as np
import pytest

from oracle import decode, encode, tables
from oracle.encode import Config


def test_fp16_norm_rounds_once_from_float64():
    # 1 + 2^-11 + 2^-40 lies just above the midpoint of fp16 neighbours 1 and
    # 1 + 2^-10.  Rounded directly it goes up; rounded via float32 first it
    # would land exactly on the midpoint and tie-break down to 1.
    v = 1.0 + 2.0 ** -11 + 2.0 ** -40
    assert encode.fp16_bits(v) == np.float16(1.0 + 2.0 ** -10).view(np.uint16)
    assert np.float16(np.float32(v)).view(np.uint16) == np.float16(1.0).view(np.uint16)


@pytest.mark.parametrize("width", [1, 2, 3, 4])
def test_pack_unpack_roundtrip_every_value_every_position(width):
    count = 64
    rng = np.random.default_rng(width)
    vals = rng.integers(0, 1 << width, size=(50, count))
    # every code value at every position
    for v in range(1 << width):
        vals[v % 50, :] = v
    packed = encode.pack_bits_lsb(vals, width)
    assert packed.shape == (50, count * width // 8)
    assert np.array_equal(encode.unpack_bits_lsb(packed, width, count), vals)


def test_pack_layout_by_hand():
    # 3-bit codes 1..8 (mod 8) LSB-first: bit stream 100 010 110 001 101 011 111 000
    codes = np.array([[1, 2, 3, 4, 5, 6, 7, 0]])
    stream = "".join(format(c, "03b")[::-1] for c in codes[0])  # LSB first
    expect = [int(stream[8 * k: 8 * k + 8][::-1], 2) for k in range(3)]
    assert list(encode.pack_bits_lsb(codes, 3)[0]) == expect


def test_sign_packing_matches_pseudocode(golden):
    g = golden("sign_packing.txt")
    bits = np.zeros(16, dtype=np.uint8)
    bits[g["positive_rows"]] = 1
    assert list(encode.pack_bits_lsb(bits[None], 1)[0]) == g["bytes"]
    # and the literal loop of the sketch: sign_bits[i/8] |= (r > 0) << (i % 8)
    rng = np.random.default_rng(0)
    r = rng.standard_normal(128)
    lit = [0] * 16
    for i in range(128):
        lit[i // 8] |= (1 if r[i] > 0 else 0) << (i % 8)
    assert list(encode.pack_bits_lsb((r > 0).astype(np.uint8)[None], 1)[0]) == lit


def test_bits_per_value_arithmetic():
    # one fp16 norm per 128-vector: turbo3 = 3.125 bits/value = 5.12x vs fp16,
    # the compression the TQ+ guide (§5.2) reports for the block-128 layout
    c3 = Config(bits=3)
    assert c3.code_bytes + 2 == 50
    assert 16 * 128 / ((c3.code_bytes + 2) * 8) == pytest.approx(5.12)
    c4q = Config(bits=4, qjl=True)
    assert c4q.code_bytes + 2 + c4q.sign_bytes + 2 == 84


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_zero_vector_and_scale_invariance(bits):
    cfg = Config(seed=5, head_dim=64, bits=bits)
    out = encode.encode(np.zeros((1, 64)), cfg)
    assert out["norms"][0] == 0
    assert np.all(out["code"] == (1 << (bits - 1)) - 1)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((20, 64))
    a = encode.encode(x, cfg)
    b = encode.encode(x * 4.0, cfg)  # exact power-of-two scale
    assert np.array_equal(a["codes"], b["codes"])


def test_quantizer_matches_searchsorted_and_ties():
    tau = tables.thresholds(3)
    z = np.concatenate([tau, np.linspace(-4, 4, 1001)])
    ref = np.searchsorted(tau, z, side="left")
    assert np.array_equal(encode.quantize(z, tau), ref)
    # exact tie goes to the lower code
    assert encode.quantize(np.array([tau[4]]), tau)[0] == 4


def test_quantizer_brute_force_nearest_centroid():
    # midpoint thresholds make the rule "nearest centroid"
    c = tables.codebook(4)
    tau = tables.thresholds(4)
    z = np.random.default_rng(1).standard_normal(20000) * 1.5
    near = np.argmin(np.abs(z[:, None] - c[None, :]), axis=1)
    assert np.array_equal(encode.quantize(z, tau), near)


@pytest.mark.parametrize("bits,target", [(2, 0.1175), (3, 0.0345), (4, 0.0095)])
def test_full_pipeline_mse_on_gaussian_input(bits, target):
    # per-coordinate MSE of dequant(encode(x)) on N(0,1) vectors, d=128,
    # within 2% of the Lloyd-Max Gaussian distortion
    cfg = Config(seed=11, head_dim=128, bits=bits)
    rng = np.random.default_rng(100 + bits)
    x = rng.standard_normal((100_000, 128)).astype(np.float32).astype(np.float64)
    planes = encode.encode(x, cfg)
    xh = decode.dequant(planes, cfg)
    mse = np.mean((x - xh) ** 2)
    assert abs(mse / target - 1) < 0.02, mse


def test_outlier_channel_error_stays_bounded():
    # an input with one huge channel: after the rotation the relative error
    # stays at (or below) the Gaussian figure instead of blowing up
    cfg = Config(seed=0, head_dim=128, bits=3)
    rng = np.random.default_rng(9)
    x = rng.standard_normal((20000, 128))
    x[:, 5] *= 20.0
    planes = encode.encode(x, cfg)
    z = planes["z"]
    assert abs(np.mean(z ** 2) - 1.0) < 1e-9  # unit vector scaled by sqrt(d)
    rel = np.sum((x - decode.dequant(planes, cfg)) ** 2, axis=1) / np.sum(x * x, axis=1)
    assert 0.5 * 0.0345 < rel.mean() < 1.05 * 0.0345


def test_qjl_estimate_unbiased_over_seeds():
    # E_S[estimate] = <q, x>: mean over 10^4 seeds within 3 standard errors
    d = 32
    rng = np.random.default_rng(42)
    x = rng.standard_normal(d)
    q = rng.standard_normal(d)
    truth = float(q @ x)
    est = []
    for s in range(10_000):
        cfg = Config(seed=s, head_dim=d, bits=2, qjl=True)
        planes = encode.encode(x[None], cfg)
        est.append(decode.scores(q[None], planes, cfg)[0, 0])
    est = np.array(est)
    se = est.std(ddof=1) / math.sqrt(len(est))
    assert abs(est.mean() - truth) <= 3 * se, (est.mean(), truth, se)


def test_qjl_variance_matches_theory():
    # Var over S of the estimate ~ n^2 ((pi/2) ||Rq||^2 gamma^2 - <Rq, rho>^2) / m
    d = 32
    rng = np.random.default_rng(7)
    x = rng.standard_normal(d)
    q = rng.standard_normal(d)
    cfg0 = Config(seed=0, head_dim=d, bits=3, qjl=True)
    base = encode.encode(x[None], cfg0)
    n = np.linalg.norm(x)
    t0 = encode.get_tables(cfg0)
    u = t0.R @ q
    rho = base["rho"][0]
    theory = n * n * ((math.pi / 2) * (u @ u) * (rho @ rho) - (u @ rho) ** 2) / d
    # vary only S: rebuild S per draw with the rotation and codes fixed
    est = []
    for s in range(3000):
        S = tables.gaussian_matrix(10_000 + s, d, d)
        sigma = np.where(S @ rho > 0, 1.0, -1.0)
        est.append(n * np.linalg.norm(rho) * math.sqrt(math.pi / 2) / d * ((S @ u) @ sigma))
    var = np.var(est, ddof=1)
    assert abs(var / theory - 1) < 0.1, (var, theory)


def test_boundary_window_fraction_small():
    cfg = Config(seed=0, head_dim=128, bits=4)
    x = np.random.default_rng(5).standard_normal((20000, 128))
    out = encode.encode(x, cfg)
    frac = encode.boundary_window(out["z"], encode.get_tables(cfg).tau).mean()
    assert frac < 1e-4

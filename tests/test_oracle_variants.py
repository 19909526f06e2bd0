"""Pins for the oracle's layout variants: the dense Haar rotation, one norm
per 32-block, and norm correction ([TQ+ guide] §1.2, §3, §4, §5.2, §11)."""

import math

import numpy as np
import pytest

from oracle import decode, encode, tables
from oracle.encode import Config


# ---------------------------------------------------------------- Haar rotation

@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_haar_is_a_proper_rotation(d):
    q = tables.haar_rotation(7, d)
    assert np.abs(q.T @ q - np.eye(d)).max() < 1e-12
    sign, logdet = np.linalg.slogdet(q)
    assert sign == 1.0 and abs(logdet) < 1e-10


def test_haar_same_seed_same_matrix():
    # [TQ+ guide] §3: one seed gives one matrix; another seed another
    a, b = tables.haar_rotation(123, 64), tables.haar_rotation(123, 64)
    assert np.array_equal(a, b)
    assert np.abs(a - tables.haar_rotation(124, 64)).max() > 0.1


@pytest.mark.parametrize("seed", range(6))
def test_haar_is_the_qr_factor_of_its_gaussian(seed):
    # Q^T G must be upper triangular with a positive diagonal (the unique QR
    # factor), except that the determinant fix may have negated column 0, so
    # row 0 of Q^T G may be negative.  A transposed Q, a missed sign fix or a
    # different stream fails this.
    d = 32
    g = tables._gaussian_stream(seed ^ tables.HAAR_STREAM_XOR, d, d)
    q = tables.haar_rotation(seed, d)
    r = q.T @ g
    assert np.abs(np.tril(r, -1)).max() < 1e-10
    assert np.all(np.diag(r)[1:] > 0)
    # G itself is a standard Gaussian sample (float32-rounded)
    assert np.array_equal(g, g.astype(np.float32).astype(np.float64))


def test_haar_entries_have_haar_moments():
    # over many seeds, entries of a Haar rotation have mean 0 and variance
    # 1/d, and distinct entries of one column are uncorrelated
    d, n = 8, 3000
    qs = np.stack([tables.haar_rotation(s, d) for s in range(n)])
    se = math.sqrt(1.0 / d / n)
    assert np.abs(qs.mean(axis=0)).max() < 5 * se
    var = (qs ** 2).mean(axis=0)
    assert np.abs(var - 1.0 / d).max() < 0.15 / d
    cov = (qs[:, 0, :] * qs[:, 1, :]).mean(axis=0)
    assert np.abs(cov).max() < 5 * se


@pytest.mark.parametrize("bits,target", [(2, 0.117482), (3, 0.034548), (4, 0.009501)])
def test_haar_pipeline_distortion_matches_lloyd_max(bits, target):
    # the dense rotation gives the same per-coordinate MSE on N(0,1) vectors
    # as the structured one: within 2% of the Gaussian Lloyd-Max distortion
    # (the sphere law sits 1.3-1.9% below it at d = 128)
    cfg = Config(seed=1, head_dim=128, bits=bits, rotation="haar")
    rng = np.random.default_rng(bits)
    x = rng.standard_normal((20000, 128))
    out = encode.encode(x, cfg)
    c = tables.codebook(bits)
    mse = np.mean((out["z"] - c[out["code"]]) ** 2)
    assert abs(mse / target - 1) < 0.02, mse


def test_haar_dequant_brute_force_tiny():
    # d = 32 by explicit loops: y = Q x, z = sqrt(d) y / ||x||, nearest
    # centroid by a full search, x_hat = (N16/sqrt(d)) Q^T c
    cfg = Config(seed=9, head_dim=32, bits=3, rotation="haar")
    q = tables.haar_rotation(9, 32)
    c = tables.codebook(3)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 32))
    planes = encode.encode(x, cfg)
    got = decode.dequant(planes, cfg)
    for r in range(4):
        n = math.sqrt(sum(v * v for v in x[r]))
        codes = []
        for i in range(32):
            zi = math.sqrt(32) * sum(q[i, j] * x[r, j] for j in range(32)) / n
            codes.append(min(range(8), key=lambda k: (abs(zi - c[k]), k)))
        assert planes["code"][r].tolist() == codes
        n16 = float(np.float16(n))
        for j in range(32):
            want = n16 / math.sqrt(32) * sum(q[i, j] * c[codes[i]] for i in range(32))
            assert abs(got[r, j] - want) < 1e-12


# ---------------------------------------------------------------- block norms

def _bits_per_value(cfg):
    return 8 * (cfg.code_bytes + 2 * cfg.norms_per_vector) / cfg.head_dim


@pytest.mark.parametrize("bits,group,bpv,ratio", [
    (3, 32, 3.5, 4.6),     # [TQ+ guide] §1.2: turbo3 4.6x against fp16
    (3, 0, 3.125, 5.12),   # [TQ+ guide] §5.2: block-128 5.12x
    (4, 32, 4.5, 3.56),
    (4, 0, 4.125, 3.88),
])
def test_layout_bits_per_value_match_the_pages(bits, group, bpv, ratio):
    cfg = Config(head_dim=128, bits=bits, norm_group=group)
    assert _bits_per_value(cfg) == bpv
    assert round(16 / bpv, 2 if ratio != 4.6 else 1) == ratio
    planes = encode.encode(np.random.default_rng(0).standard_normal((3, 128)), cfg)
    assert planes["codes"].shape == (3, cfg.code_bytes)
    assert planes["norms"].shape == ((3, 4) if group else (3,))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_block_norms_reduce_to_vector_norm_when_blocks_are_balanced(bits):
    # if every 32-block of y = R x has the same norm n / sqrt(d/32), block
    # normalisation is exactly vector normalisation: same z, same codes, and
    # each block norm is n / 2 at d = 128
    d = 128
    cfg_v = Config(seed=4, head_dim=d, bits=bits)
    cfg_b = Config(seed=4, head_dim=d, bits=bits, norm_group=32)
    R = encode.get_tables(cfg_v).R
    rng = np.random.default_rng(bits)
    y = rng.standard_normal((50, 4, 32))
    y /= np.linalg.norm(y, axis=-1, keepdims=True)
    y *= rng.uniform(0.5, 3.0, size=(50, 1, 1))          # equal block norms per vector
    x = y.reshape(50, d) @ R                              # x = R^T y
    ov, ob = encode.encode(x, cfg_v), encode.encode(x, cfg_b)
    assert np.abs(ov["z"] - ob["z"]).max() < 1e-12
    win = encode.boundary_window(ov["z"], encode.get_tables(cfg_v).tau, 1e-9)
    assert np.array_equal(ov["code"][~win], ob["code"][~win])
    nb = decode.fp16_value(ob["norms"])
    assert np.array_equal(nb, np.repeat(decode.fp16_value(encode.fp16_bits(np.linalg.norm(x, axis=-1) / 2))[:, None], 4, 1))


def test_block_norm_encode_brute_force_tiny():
    # d = 64, two blocks, by explicit loops over the pages' steps
    cfg = Config(seed=2, head_dim=64, bits=3, norm_group=32)
    R = tables.rotation_matrix(2, 64)
    c = tables.codebook(3)
    rng = np.random.default_rng(8)
    x = rng.standard_normal((3, 64)) * rng.uniform(0.1, 10, size=(3, 1))
    out = encode.encode(x, cfg)
    got = decode.dequant(out, cfg)
    for r in range(3):
        y = [sum(R[i, j] * x[r, j] for j in range(64)) for i in range(64)]
        xh = [0.0] * 64
        for b in range(2):
            blk = y[32 * b: 32 * b + 32]
            nb = math.sqrt(sum(v * v for v in blk))
            assert out["norms"][r, b] == np.float16(nb).view(np.uint16)
            for i, v in enumerate(blk):
                zi = math.sqrt(32) * v / nb
                k = min(range(8), key=lambda k: (abs(zi - c[k]), k))
                assert out["code"][r, 32 * b + i] == k
                yh = float(np.float16(nb)) / math.sqrt(32) * c[k]
                for j in range(64):
                    xh[j] += R[32 * b + i, j] * yh
        assert np.abs(np.array(xh) - got[r]).max() < 1e-12


def test_block_norms_fit_blocks_of_different_scale():
    # a rotated vector whose blocks differ widely in scale: per-block norms
    # keep every block's relative error at the codebook's level, one norm
    # per vector lets the small blocks collapse to their smallest centroids
    d = 128
    cfg_v = Config(seed=6, head_dim=d, bits=3)
    cfg_b = Config(seed=6, head_dim=d, bits=3, norm_group=32)
    R = encode.get_tables(cfg_v).R
    rng = np.random.default_rng(6)
    y = rng.standard_normal((400, 4, 32)) * np.array([1.0, 0.05, 0.01, 3.0])[None, :, None]
    x = y.reshape(400, d) @ R
    err_v = np.linalg.norm(decode.dequant(encode.encode(x, cfg_v), cfg_v) - x, axis=-1)
    err_b = np.linalg.norm(decode.dequant(encode.encode(x, cfg_b), cfg_b) - x, axis=-1)
    assert np.mean(err_b) < 0.8 * np.mean(err_v)


# ---------------------------------------------------------------- norm correction

@pytest.mark.parametrize("group,rotation", [(0, "wht"), (32, "wht"), (0, "haar")])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_norm_correction_keeps_each_group_norm(group, rotation, bits):
    # with correction the dequantised vector (per-vector norm) or each
    # dequantised block of the rotated vector (per-block norms) has the
    # original norm, up to the fp16 rounding of the stored norm (2^-11)
    d = 128
    cfg = Config(seed=3, head_dim=d, bits=bits, norm_group=group, norm_correction=True, rotation=rotation)
    rng = np.random.default_rng(bits + group)
    x = rng.standard_normal((500, d)) * np.exp(rng.standard_normal((500, 1)))
    xh = decode.dequant(encode.encode(x, cfg), cfg)
    if group == 0:
        rel = np.abs(np.linalg.norm(xh, axis=-1) / np.linalg.norm(x, axis=-1) - 1)
    else:
        R = encode.get_tables(cfg).R
        yb = (x @ R.T).reshape(500, 4, 32)
        yhb = (xh @ R.T).reshape(500, 4, 32)
        rel = np.abs(np.linalg.norm(yhb, axis=-1) / np.linalg.norm(yb, axis=-1) - 1)
    assert rel.max() <= 2.0 ** -11
    # without correction the reconstruction's norm is off by the codebook's
    # relative error (the pages' reason for the correction)
    plain = Config(seed=3, head_dim=d, bits=bits, norm_group=group, rotation=rotation)
    xp = decode.dequant(encode.encode(x, plain), plain)
    assert np.mean(np.abs(np.linalg.norm(xp, axis=-1) / np.linalg.norm(x, axis=-1) - 1)) > 4 * 2.0 ** -11


def test_norm_correction_changes_only_the_stored_norm():
    cfg = Config(seed=5, head_dim=64, bits=4, norm_correction=True)
    plain = Config(seed=5, head_dim=64, bits=4)
    x = np.random.default_rng(1).standard_normal((40, 64))
    a, b = encode.encode(x, cfg), encode.encode(x, plain)
    assert np.array_equal(a["codes"], b["codes"])
    c = tables.codebook(4)[a["code"]]
    n = np.linalg.norm(x, axis=-1)
    assert np.array_equal(a["norms"], encode.fp16_bits(n * 8.0 / np.linalg.norm(c, axis=-1)))


def test_qjl_takes_plain_vector_norms():
    with pytest.raises(ValueError):
        Config(qjl=True, norm_group=32).check()
    with pytest.raises(ValueError):
        Config(qjl=True, norm_correction=True).check()

"""Pins for the oracle's decode side: dequant, scores, attention, top-k."""

import math

import numpy as np
import pytest

from oracle import decode, encode, tables
from oracle.encode import Config


def _planes_bhtd(x, cfg):
    """Encode x[B, H, T, d] into planes shaped [B, H, T, ...]."""
    out = encode.encode(x, cfg)
    return {k: out[k] for k in ("codes", "norms", "signs", "rnorms") if k in out}


def test_pre_rotation_identity():
    # <q, R^T c[idx]> = <R q, c[idx]>: the rotated-query score equals the
    # explicit dequant-then-dot score (TQ+ guide §5.3, pre-rotate-queries)
    cfg = Config(seed=3, head_dim=128, bits=3)
    t = encode.get_tables(cfg)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((64, 128))
    q = rng.standard_normal((5, 128))
    planes = encode.encode(x, cfg)
    explicit = decode.scores(q, planes, cfg)
    code = decode.codes_of(planes, cfg)
    n16 = decode.fp16_value(planes["norms"])
    d1, d2 = tables.rotation_signs(3, 128)
    rq = d1 * tables.fwht(q * d2) / math.sqrt(128)   # rotate each query once
    fused = (rq @ t.c[code].T) * n16[None, :] / math.sqrt(128)
    assert np.max(np.abs(explicit - fused)) < 1e-12


@pytest.mark.parametrize("bits,qjl,d", [(3, False, 128), (4, True, 256), (2, True, 32)])
def test_rotated_scores_equal_plain_definition(bits, qjl, d):
    # the rotated-domain form (used on large key sets) against explicit
    # dequantisation of every key followed by a plain dot product
    cfg = Config(seed=5, head_dim=d, bits=bits, qjl=qjl)
    rng = np.random.default_rng(d + bits)
    x = rng.standard_normal((300, d)) * np.exp(0.5 * rng.standard_normal(d))
    q = rng.standard_normal((7, d))
    planes = encode.encode(x, cfg)
    plain = decode.scores(q, planes, cfg, scale=0.3)
    fused = decode.scores_rotated(q, planes, cfg, scale=0.3)
    assert fused.shape == plain.shape == (7, 300)
    assert np.max(np.abs(fused - plain)) <= 1e-12 * np.max(np.abs(plain))


def test_dequant_brute_force_tiny():
    # d=32 by explicit loops: x_hat_i = N/sqrt(d) * sum_k R_ki c[code_k]
    cfg = Config(seed=1, head_dim=32, bits=2)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 32))
    planes = encode.encode(x, cfg)
    R = tables.rotation_matrix(1, 32)
    c = tables.codebook(2)
    codes = planes["code"]
    got = decode.dequant(planes, cfg)
    for r in range(3):
        n = float(np.float16(np.linalg.norm(x[r])))
        for i in range(32):
            acc = sum(R[k, i] * c[codes[r, k]] for k in range(32))
            assert abs(got[r, i] - n / math.sqrt(32) * acc) < 1e-12


def _brute_attend(q, K, V, seq_lens, Hkv, scale):
    B, Hq, d = q.shape
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            L = seq_lens[b]
            if L == 0:
                continue
            s = [scale * sum(q[b, h, i] * K[b, g, j, i] for i in range(d)) for j in range(L)]
            m = max(s)
            e = [math.exp(v - m) for v in s]
            tot = sum(e)
            for i in range(d):
                out[b, h, i] = sum(e[j] / tot * V[b, g, j, i] for j in range(L))
    return out


@pytest.mark.parametrize("qjl", [False, True])
def test_attend_brute_force_tiny(qjl):
    B, Hkv, Hq, T, d = 2, 2, 4, 8, 32
    kc = Config(seed=2, head_dim=d, bits=4, qjl=qjl)
    vc = Config(seed=2, head_dim=d, bits=3)
    rng = np.random.default_rng(12)
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    q = rng.standard_normal((B, Hq, d))
    kp = _planes_bhtd(k, kc)
    vp = _planes_bhtd(v, vc)
    lens = [8, 5]
    got = decode.attend_decode(q, kp, vp, kc, vc, lens)
    K = decode.dequant(kp, kc)
    V = decode.dequant(vp, vc)
    ref = _brute_attend(q, K, V, lens, Hkv, 1 / math.sqrt(d))
    assert np.max(np.abs(got - ref)) < 1e-12


def test_attend_special_cases():
    B, Hkv, Hq, T, d = 1, 1, 2, 6, 64
    cfg = Config(seed=0, head_dim=d, bits=3)
    rng = np.random.default_rng(1)
    v = rng.standard_normal((B, Hkv, T, d))
    q = rng.standard_normal((B, Hq, d))
    # all keys identical -> uniform weights -> mean of the values
    k = np.repeat(rng.standard_normal((1, 1, 1, d)), T, axis=2)
    kp, vp = _planes_bhtd(k, cfg), _planes_bhtd(v, cfg)
    V = decode.dequant(vp, cfg)
    out = decode.attend_decode(q, kp, vp, cfg, cfg, [T])
    assert np.allclose(out[0, 0], V[0, 0].mean(axis=0), atol=1e-12)
    # seq_len 1 -> exactly the first value; seq_len 0 -> zeros
    out1 = decode.attend_decode(q, kp, vp, cfg, cfg, [1])
    assert np.allclose(out1[0, 1], V[0, 0, 0], atol=1e-12)
    out0 = decode.attend_decode(q, kp, vp, cfg, cfg, [0])
    assert np.all(out0 == 0)


def test_attend_output_is_convex_combination():
    B, Hkv, Hq, T, d = 1, 2, 8, 50, 64
    cfg = Config(seed=4, head_dim=d, bits=3)
    rng = np.random.default_rng(2)
    k = rng.standard_normal((B, Hkv, T, d)) * 3
    v = rng.standard_normal((B, Hkv, T, d))
    q = rng.standard_normal((B, Hq, d))
    kp, vp = _planes_bhtd(k, cfg), _planes_bhtd(v, cfg)
    out = decode.attend_decode(q, kp, vp, cfg, cfg, [T])
    V = decode.dequant(vp, cfg)
    for h in range(Hq):
        g = h // 4
        lo, hi = V[0, g].min(axis=0), V[0, g].max(axis=0)
        assert np.all(out[0, h] >= lo - 1e-12) and np.all(out[0, h] <= hi + 1e-12)


def test_top_k_ties_and_order():
    s = np.array([[1.0, 3.0, 3.0, 2.0, 3.0, -1.0]])
    vals, idx = decode.top_k(s, 4)
    assert idx.tolist() == [[1, 2, 4, 3]]
    assert vals.tolist() == [[3.0, 3.0, 3.0, 2.0]]
    rng = np.random.default_rng(0)
    s = rng.integers(0, 5, size=(7, 40)).astype(float)
    vals, idx = decode.top_k(s, 10)
    for r in range(7):
        ref = sorted(range(40), key=lambda j: (-s[r, j], j))[:10]
        assert idx[r].tolist() == ref


def test_prefill_single_query_equals_decode():
    # one new position (Tq = 1) is exactly a decode step over the cache
    B, Hkv, Hq, T, d = 2, 2, 8, 40, 64
    kc = Config(seed=3, head_dim=d, bits=4, qjl=True)
    vc = Config(seed=3, head_dim=d, bits=3)
    rng = np.random.default_rng(7)
    kp = _planes_bhtd(rng.standard_normal((B, Hkv, T, d)), kc)
    vp = _planes_bhtd(rng.standard_normal((B, Hkv, T, d)), vc)
    q = rng.standard_normal((B, Hq, d))
    lens = [T, 17]
    pre = decode.attend_prefill(q[:, :, None, :], kp, vp, kc, vc, lens)
    dec = decode.attend_decode(q, kp, vp, kc, vc, lens)
    assert np.abs(pre[:, :, 0] - dec).max() < 1e-13


def test_prefill_brute_force_tiny():
    # explicit loops: query i of batch b at position L - Tq + i sees j <= p
    B, Hkv, Hq, T, Tq, d = 2, 1, 2, 7, 4, 32
    cfg = Config(seed=1, head_dim=d, bits=3)
    rng = np.random.default_rng(3)
    kp = _planes_bhtd(rng.standard_normal((B, Hkv, T, d)), cfg)
    vp = _planes_bhtd(rng.standard_normal((B, Hkv, T, d)), cfg)
    K, V = decode.dequant(kp, cfg), decode.dequant(vp, cfg)
    q = rng.standard_normal((B, Hq, Tq, d))
    lens = [7, 2]                                  # batch 1: positions -2, -1, 0, 1
    got = decode.attend_prefill(q, kp, vp, cfg, cfg, lens)
    sc = 1 / math.sqrt(d)
    for b in range(B):
        for h in range(Hq):
            for i in range(Tq):
                p = lens[b] - Tq + i
                if p < 0:
                    assert np.all(got[b, h, i] == 0)
                    continue
                s = [sc * sum(q[b, h, i, e] * K[b, 0, j, e] for e in range(d)) for j in range(p + 1)]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                for e in range(d):
                    want = sum(w[j] * V[b, 0, j, e] for j in range(p + 1)) / sum(w)
                    assert abs(got[b, h, i, e] - want) < 1e-12


def test_prefill_is_causal():
    # changing the keys and values after a position leaves every earlier
    # query's output unchanged, and changes the later ones
    B, Hkv, Hq, T, d = 1, 1, 1, 30, 32
    cfg = Config(seed=2, head_dim=d, bits=2)
    rng = np.random.default_rng(4)
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    q = rng.standard_normal((B, Hq, T, d))
    a = decode.attend_prefill(q, _planes_bhtd(k, cfg), _planes_bhtd(v, cfg), cfg, cfg, [T])
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 20:] = rng.standard_normal((B, Hkv, 10, d))
    v2[:, :, 20:] = rng.standard_normal((B, Hkv, 10, d))
    b = decode.attend_prefill(q, _planes_bhtd(k2, cfg), _planes_bhtd(v2, cfg), cfg, cfg, [T])
    assert np.array_equal(a[:, :, :20], b[:, :, :20])
    assert np.abs(a[:, :, 20:] - b[:, :, 20:]).min(axis=-1).max() > 0


def test_prefill_identical_keys_average_the_prefix():
    # with every key equal, query i weighs its visible prefix uniformly
    B, Hkv, Hq, T, d = 1, 1, 2, 12, 64
    cfg = Config(seed=0, head_dim=d, bits=3)
    rng = np.random.default_rng(9)
    k = np.repeat(rng.standard_normal((1, 1, 1, d)), T, axis=2)
    v = rng.standard_normal((B, Hkv, T, d))
    kp, vp = _planes_bhtd(k, cfg), _planes_bhtd(v, cfg)
    V = decode.dequant(vp, cfg)
    out = decode.attend_prefill(rng.standard_normal((B, Hq, 5, d)), kp, vp, cfg, cfg, [T])
    for i in range(5):
        p = T - 5 + i
        assert np.abs(out[0, :, i] - V[0, 0, :p + 1].mean(axis=0)).max() < 1e-12

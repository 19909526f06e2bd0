"""GPU parity: libtq (through its C ABI) against the float64 oracle.

Encode parity compares codes / norms / QJL planes element by element.  Decode
and score parity run both sides on identical packed inputs (planes made by
the oracle, uploaded), so one legitimately different code cannot move a logit
by a whole centroid gap.
"""

import math

import numpy as np
import pytest
import torch

from kv_cache_quantization_05_amd import binding as tq
from kv_cache_quantization_05_amd import workloads as wl
from oracle import decode as odec
from oracle import encode as oenc

from _parity import assert_attend_close, assert_topk_valid, compare_encode, oracle_config, LOGIT_ATOL

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(*a):
    print("[gpu-test]", *a, flush=True)


def _x(shape, dtype, seed, scale_ch=True):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g)
    if scale_ch:
        x = x * torch.exp(0.5 * torch.randn(shape[-1], generator=g))
    return x.to(dtype)


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("qjl", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_encode_matches_oracle(d, bits, qjl, dtype):
    _say("encode", d, bits, qjl, dtype)
    ctx = tq.Context(seed=7 + d, head_dim=d, bits=bits, qjl=qjl)
    x = _x((3, 5, 67, d), dtype, seed=d * 10 + bits)   # 1005 vectors, ragged vs any lane grouping
    x[0, 0, 0] = 0                                       # zero vector
    x[0, 0, 1] *= 1e-3
    x[1, 2, 3] *= 1e4
    xg = x.reshape(15, 67, d).to(DEV)
    planes = tq.encode(ctx, xg)
    torch.cuda.synchronize()
    cfg = oracle_config(ctx)
    ref = oenc.encode(x.reshape(15, 67, d).float().numpy().astype(np.float64), cfg)
    rep = compare_encode(planes.numpy(), ref, cfg)
    _say(rep)


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("qjl", [False, True])
def test_encode_extreme_magnitudes(bits, dtype, qjl):
    # vectors far outside fp32's comfortable range for a 128-point transform
    # (norms from ~1e-35 to ~1e35), including subnormal coordinates
    _say("encode extreme", bits, dtype, qjl)
    ctx = tq.Context(seed=11, head_dim=128, bits=bits, qjl=qjl)
    scales = [1e-35, 1e-20, 2.0 ** -61, 2.0 ** -59, 1.0, 2.0 ** 59, 2.0 ** 61, 1e20, 1e35]
    x = _x((len(scales), 40, 128), torch.float32, seed=99 + bits)
    x = x * torch.tensor(scales).view(-1, 1, 1)
    x = x.to(dtype)
    planes = tq.encode(ctx, x.to(DEV))
    torch.cuda.synchronize()
    cfg = oracle_config(ctx)
    ref = oenc.encode(x.float().numpy().astype(np.float64), cfg)
    _say(compare_encode(planes.numpy(), ref, cfg))


def test_encode_strided_grid_into_cache_layout():
    # x laid out [B, T, Hkv, d] (prefill order) written into planes [B, Hkv, Tcap]
    ctx = tq.Context(seed=0, head_dim=128, bits=3)
    B, T, Hkv, Tcap = 2, 100, 4, 160
    x = _x((B, T, Hkv, 128), torch.bfloat16, seed=3).to(DEV)
    planes = ctx.new_planes((B, Hkv, Tcap))
    planes.codes.zero_()
    planes.norms.zero_()
    view = tq.PackedPlanes(planes.codes[:, :, :T], planes.norms[:, :, :T], None, None)
    tq.encode(ctx, x.permute(0, 2, 1, 3), view)  # strided grid [B, Hkv, T]
    torch.cuda.synchronize()
    ref = oenc.encode(x.permute(0, 2, 1, 3).float().cpu().numpy().astype(np.float64), oracle_config(ctx))
    got = planes.numpy()
    sub = {"codes": got["codes"][:, :, :T], "norms": got["norms"][:, :, :T]}
    compare_encode(sub, ref, oracle_config(ctx))
    assert np.all(got["codes"][:, :, T:] == 0) and np.all(got["norms"][:, :, T:] == 0)


@pytest.mark.parametrize("d", [64, 128])
def test_encode_qjl_strided_grid_into_cache_layout(d):
    # bf16 QJL keys laid out [B, T, Hkv, d] (prefill order), read as a strided
    # [B, Hkv, T] grid and written into [B, Hkv, Tcap] planes: the grid
    # cannot be folded, and codes, norms, signs and residual norms land at
    # strided plane positions; the rest of the planes stays untouched
    _say("encode qjl strided", d)
    ctx = tq.Context(seed=2, head_dim=d, bits=4, qjl=True)
    B, T, Hkv, Tcap = 2, 100, 4, 160
    x = _x((B, T, Hkv, d), torch.bfloat16, seed=30 + d).to(DEV)
    planes = ctx.new_planes((B, Hkv, Tcap))
    for t in (planes.codes, planes.norms, planes.signs, planes.rnorms):
        t.zero_()
    view = tq.PackedPlanes(planes.codes[:, :, :T], planes.norms[:, :, :T], planes.signs[:, :, :T],
                           planes.rnorms[:, :, :T])
    tq.encode(ctx, x.permute(0, 2, 1, 3), view)
    torch.cuda.synchronize()
    cfg = oracle_config(ctx)
    ref = oenc.encode(x.permute(0, 2, 1, 3).float().cpu().numpy().astype(np.float64), cfg)
    got = planes.numpy()
    sub = {k: got[k][:, :, :T] for k in ("codes", "norms", "signs", "rnorms")}
    _say(compare_encode(sub, ref, cfg))
    for k in ("codes", "norms", "signs", "rnorms"):
        assert np.all(got[k][:, :, T:] == 0), k


@pytest.mark.parametrize("d,bits,strided", [(64, 4, False), (128, 3, False), (128, 3, True)])
def test_encode_many_vectors(d, bits, strided):
    # more vectors than a few rounds of resident blocks cover, so the encoder
    # takes its grid-striding loop; contiguous and strided ([B, T, H, d]
    # read as a [B, H, T] grid) inputs
    _say("encode many", d, bits, strided)
    ctx = tq.Context(seed=5, head_dim=d, bits=bits)
    B, H = 2, 8
    T = 600_000 // (B * H) if d == 64 else 400_000 // (B * H)
    if strided:
        xs = _x((B, T, H, d), torch.bfloat16, seed=d + 1, scale_ch=False)
        x = xs.permute(0, 2, 1, 3)
    else:
        x = _x((B, H, T, d), torch.bfloat16, seed=d + 2, scale_ch=False)
        xs = x
    xg = xs.to(DEV)
    planes = tq.encode(ctx, xg.permute(0, 2, 1, 3) if strided else xg)
    torch.cuda.synchronize()
    cfg = oracle_config(ctx)
    ref = oenc.encode(x.float().numpy().astype(np.float64), cfg)
    _say(compare_encode(planes.numpy(), ref, cfg))


def _integer_rows(d, n, seed):
    """Integer-valued vectors whose rotated coordinates are often exactly 0:
    all ones, pairs of unit vectors, and sparse or small random integers."""
    rng = np.random.default_rng(seed)
    rows = [np.ones(d), np.eye(d)[0] + np.eye(d)[1], np.eye(d)[0] - np.eye(d)[3]]
    while len(rows) < n:
        k = len(rows) % 3
        if k == 0:
            rows.append(rng.choice([-1.0, 0.0, 1.0], size=d, p=[0.25, 0.5, 0.25]))
        elif k == 1:
            rows.append(rng.integers(-3, 4, size=d).astype(np.float64))
        else:
            v = np.zeros(d)
            v[rng.choice(d, size=2, replace=False)] = rng.choice([-1.0, 1.0], size=2)
            rows.append(v)
    return np.stack(rows)


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("bits,qjl", [(2, False), (3, False), (4, False), (3, True)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_encode_exact_ties_at_zero(d, bits, qjl, dtype):
    # An integer vector's rotated coordinate D1 H D2 x is an exact integer,
    # often 0.  z = 0 lies exactly on the middle threshold: the centroids
    # -c and +c either side of it are equally near, so codes 2^(b-1) - 1
    # and 2^(b-1) are both nearest-centroid codes there (the oracle's
    # float64 product lands a rounding error either side of 0).  Everywhere
    # else the codes must match as usual; norms are exact.
    _say("encode ties", d, bits, qjl, dtype)
    ctx = tq.Context(seed=13, head_dim=d, bits=bits, qjl=qjl)
    cfg = oracle_config(ctx)
    xi = _integer_rows(d, 96, seed=d + bits)
    xi = np.concatenate([xi, 0.375 * xi[:32]])              # exact in bf16 too
    x = torch.from_numpy(xi).to(dtype)
    planes = tq.encode(ctx, x.to(DEV)).numpy()
    torch.cuda.synchronize()
    ref = oenc.encode(x.float().numpy().astype(np.float64), cfg)
    signs = np.sign(oenc.get_tables(cfg).R)                # D1 H D2 entries, +-1
    y_exact = xi @ signs.T                                   # exact integers
    tie = y_exact == 0
    assert tie.sum() > xi.shape[0], "inputs must produce many exact zeros"
    g_code = oenc.unpack_bits_lsb(planes["codes"], bits, d)
    half = 1 << (bits - 1)
    assert np.all((g_code[tie] == half - 1) | (g_code[tie] == half))
    assert np.array_equal(planes["norms"], ref["norms"])
    # every entry off the exact ties is compared, in every vector; for QJL
    # contexts gamma and the signs are compared on the vectors whose tie
    # choices agree (the residual depends on the chosen centroid)
    rep = compare_encode(planes, ref, cfg, tie_ok=tie)
    _say("tie entries", int(tie.sum()), "tie choices that differ", int(((g_code != ref["code"]) & tie).sum()), rep)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_encode_qjl_wide_dynamic_range(d, bits):
    # bf16 QJL keys whose coordinates reach more than 2^19 below their
    # largest one (most of the 40,000 vectors, more than one round of the
    # resident grid): the matrix-core rotation then needs its third exponent
    # band, and a few residual norms per case lie close enough to an fp16
    # rounding midpoint that the float64 butterflies decide them.  Everything
    # is compared with the oracle.
    _say("encode wide range", d, bits)
    ctx = tq.Context(seed=21 + d, head_dim=d, bits=bits, qjl=True)
    g = torch.Generator().manual_seed(500 + d + bits)
    n = 40_000
    x = torch.randn((n, d), generator=g)
    big = torch.rand((n, d), generator=g) < 0.04          # a few large coordinates
    x = torch.where(big, x * 2.0 ** 12, x)
    tiny = torch.rand((n, d), generator=g) < 0.02         # and some far below them
    x = torch.where(tiny, x * 2.0 ** -10, x)
    x[:50] = torch.randn((50, d), generator=g) * 1e-3    # and some ordinary vectors
    x = x.to(torch.bfloat16)
    planes = tq.encode(ctx, x.to(DEV))
    torch.cuda.synchronize()
    cfg = oracle_config(ctx)
    ref = oenc.encode(x.float().numpy().astype(np.float64), cfg)
    _say(compare_encode(planes.numpy(), ref, cfg))


def test_encode_empty_grid_is_noop():
    ctx = tq.Context(seed=0, head_dim=128, bits=3)
    x = torch.zeros((0, 128), device=DEV)
    planes = ctx.new_planes((0,))
    tq.encode(ctx, x, planes)
    torch.cuda.synchronize()


def _oracle_planes(x, cfg):
    out = oenc.encode(x, cfg)
    return {k: out[k] for k in ("codes", "norms", "signs", "rnorms") if k in out}


@pytest.mark.parametrize("kb,vb,qjl,G", [(3, 3, False, 4), (4, 4, True, 4), (2, 4, False, 1),
                                         (4, 4, False, 1), (4, 3, False, 8), (3, 2, True, 2)])
@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_attend_matches_oracle(kb, vb, qjl, G, d):
    _say("attend", kb, vb, qjl, G, d)
    B, Hkv, T = 3, 2, 2600
    Hq = Hkv * G
    kc = oenc.Config(seed=11, head_dim=d, bits=kb, qjl=qjl)
    vc = oenc.Config(seed=11, head_dim=d, bits=vb)
    rng = np.random.default_rng(kb * 100 + vb * 10 + d)
    k = rng.standard_normal((B, Hkv, T, d)) * 2.0
    v = rng.standard_normal((B, Hkv, T, d))
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    kp, vp = _oracle_planes(k, kc), _oracle_planes(v, vc)
    lens = np.array([T, 1, 1029], dtype=np.int32)
    ref = odec.attend_decode(q.astype(np.float64), kp, vp, kc, vc, lens)
    kctx = tq.Context(seed=11, head_dim=d, bits=kb, qjl=qjl)
    vctx = tq.Context(seed=11, head_dim=d, bits=vb)
    out = tq.attend_decode(kctx, vctx, torch.from_numpy(q).to(DEV), tq.PackedPlanes.from_numpy(kp),
                           tq.PackedPlanes.from_numpy(vp), torch.from_numpy(lens).to(DEV))
    torch.cuda.synchronize()
    worst = assert_attend_close(out.cpu().numpy().astype(np.float64), ref)
    _say("max rel / abs", worst)


@pytest.mark.parametrize("kb", [2, 3, 4])
@pytest.mark.parametrize("vb", [2, 3, 4])
@pytest.mark.parametrize("qjl", [False, True])
def test_attend_matrix_core_bit_widths(kb, vb, qjl):
    """Every (key bits, value bits, QJL) instantiation of the d = 128, GQA 4
    matrix-core path: pair-table and byte-permute decoders, ragged lengths."""
    _say("attend mfma", kb, vb, qjl)
    d, B, Hkv, G, T = 128, 2, 2, 4, 1500
    kc = oenc.Config(seed=5, head_dim=d, bits=kb, qjl=qjl)
    vc = oenc.Config(seed=5, head_dim=d, bits=vb)
    rng = np.random.default_rng(1000 + kb * 100 + vb * 10 + qjl)
    k = rng.standard_normal((B, Hkv, T, d)) * 1.5
    v = rng.standard_normal((B, Hkv, T, d))
    q = rng.standard_normal((B, Hkv * G, d)).astype(np.float32)
    kp, vp = _oracle_planes(k, kc), _oracle_planes(v, vc)
    lens = np.array([T, 777], dtype=np.int32)
    ref = odec.attend_decode(q.astype(np.float64), kp, vp, kc, vc, lens)
    kctx = tq.Context(seed=5, head_dim=d, bits=kb, qjl=qjl)
    vctx = tq.Context(seed=5, head_dim=d, bits=vb)
    out = tq.attend_decode(kctx, vctx, torch.from_numpy(q).to(DEV), tq.PackedPlanes.from_numpy(kp),
                           tq.PackedPlanes.from_numpy(vp), torch.from_numpy(lens).to(DEV))
    torch.cuda.synchronize()
    _say("max rel / abs", assert_attend_close(out.cpu().numpy().astype(np.float64), ref))


def test_attend_zero_and_clamped_lengths():
    d, B, Hkv, G, T = 128, 4, 1, 4, 300
    kc = vc = oenc.Config(seed=0, head_dim=d, bits=3)
    rng = np.random.default_rng(1)
    kp = _oracle_planes(rng.standard_normal((B, Hkv, T, d)), kc)
    vp = _oracle_planes(rng.standard_normal((B, Hkv, T, d)), vc)
    q = rng.standard_normal((B, Hkv * G, d)).astype(np.float32)
    lens = np.array([0, T, 5000, -3], dtype=np.int32)      # clamped to [0, t_max]
    ref = odec.attend_decode(q.astype(np.float64), kp, vp, kc, vc, np.clip(lens, 0, T))
    ctx = tq.Context(seed=0, head_dim=d, bits=3)
    out = tq.attend_decode(ctx, ctx, torch.from_numpy(q).to(DEV), tq.PackedPlanes.from_numpy(kp),
                           tq.PackedPlanes.from_numpy(vp), torch.from_numpy(lens).to(DEV), t_max=T)
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    assert np.all(o[0] == 0) and np.all(o[3] == 0)
    assert_attend_close(o, ref)


@pytest.mark.parametrize("kb,vb,qjl", [(3, 3, False), (4, 4, True)])
def test_attend_ignores_slots_past_each_length(kb, vb, qjl):
    # cache slots at or past a sequence's length hold garbage (0xFF bytes:
    # NaN fp16 norms); they must not reach the output
    d, B, Hkv, G, Tcap = 128, 3, 2, 4, 1500
    kc = oenc.Config(seed=4, head_dim=d, bits=kb, qjl=qjl)
    vc = oenc.Config(seed=4, head_dim=d, bits=vb)
    rng = np.random.default_rng(5)
    kp = _oracle_planes(rng.standard_normal((B, Hkv, Tcap, d)), kc)
    vp = _oracle_planes(rng.standard_normal((B, Hkv, Tcap, d)), vc)
    lens = np.array([1, 700, 1299], dtype=np.int32)
    for planes in (kp, vp):
        for name, arr in planes.items():
            for b_, L in enumerate(lens):
                arr[b_, :, L:] = np.iinfo(arr.dtype).max
    q = rng.standard_normal((B, Hkv * G, d)).astype(np.float32)
    ref = odec.attend_decode(q.astype(np.float64), kp, vp, kc, vc, lens)
    kctx = tq.Context(seed=4, head_dim=d, bits=kb, qjl=qjl)
    vctx = tq.Context(seed=4, head_dim=d, bits=vb)
    out = tq.attend_decode(kctx, vctx, torch.from_numpy(q).to(DEV), tq.PackedPlanes.from_numpy(kp),
                           tq.PackedPlanes.from_numpy(vp), torch.from_numpy(lens).to(DEV), t_max=Tcap)
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o))
    _say("garbage past length", kb, vb, qjl, assert_attend_close(o, ref))


def test_attend_reuses_one_workspace():
    # one workspace serves successive calls of different lengths
    d, B, Hkv, G, T = 128, 2, 2, 4, 3000
    kc = vc = oenc.Config(seed=9, head_dim=d, bits=3)
    rng = np.random.default_rng(9)
    kp = _oracle_planes(rng.standard_normal((B, Hkv, T, d)), kc)
    vp = _oracle_planes(rng.standard_normal((B, Hkv, T, d)), vc)
    q = rng.standard_normal((B, Hkv * G, d)).astype(np.float32)
    ctx = tq.Context(seed=9, head_dim=d, bits=3)
    kg, vg = tq.PackedPlanes.from_numpy(kp), tq.PackedPlanes.from_numpy(vp)
    ws = torch.zeros(tq.attend_workspace_bytes(ctx, ctx, B, Hkv * G, Hkv, T), dtype=torch.uint8, device=DEV)
    # successive calls whose t_max (and so chunk split) differs share the
    # workspace: nothing a call leaves in it may leak into the next
    for lens, t_max in (([T, 17], T), ([1, 2999], T), ([0, 64], T), ([T, T], T), ([40, 700], 700),
                        ([300, 2], 300), ([T, 1000], T)):
        lens = np.array(lens, dtype=np.int32)
        ref = odec.attend_decode(q.astype(np.float64), kp, vp, kc, vc, lens)
        out = tq.attend_decode(ctx, ctx, torch.from_numpy(q).to(DEV), kg, vg, torch.from_numpy(lens).to(DEV),
                               t_max=t_max, workspace=ws)
        torch.cuda.synchronize()
        _say("workspace reuse", lens.tolist(), assert_attend_close(out.cpu().numpy().astype(np.float64), ref))


@pytest.mark.parametrize("kb,vb,qjl", [(3, 3, False), (4, 4, True), (2, 4, False)])
def test_attend_token_strided_planes(kb, vb, qjl):
    """Caches laid out [B, T, Hkv] (heads interleaved per token), passed as
    [B, Hkv, T] views: the token stride is Hkv vectors, not one."""
    d, B, Hkv, G, T = 128, 2, 2, 4, 1500
    kc = oenc.Config(seed=6, head_dim=d, bits=kb, qjl=qjl)
    vc = oenc.Config(seed=6, head_dim=d, bits=vb)
    rng = np.random.default_rng(60 + kb)
    k = rng.standard_normal((B, T, Hkv, d)) * 1.5
    v = rng.standard_normal((B, T, Hkv, d))
    q = rng.standard_normal((B, Hkv * G, d)).astype(np.float32)
    kp, vp = _oracle_planes(k, kc), _oracle_planes(v, vc)   # planes over [B, T, Hkv]
    lens = np.array([T, 901], dtype=np.int32)
    to_bht = lambda pl: {n: np.ascontiguousarray(np.swapaxes(a, 1, 2)) for n, a in pl.items()}  # noqa: E731
    ref = odec.attend_decode(q.astype(np.float64), to_bht(kp), to_bht(vp), kc, vc, lens)

    def view(pl):
        g = tq.PackedPlanes.from_numpy(pl)
        sw = lambda t: t.transpose(1, 2) if t is not None else None  # noqa: E731
        return tq.PackedPlanes(sw(g.codes), sw(g.norms), sw(g.signs), sw(g.rnorms))

    kg, vg = view(kp), view(vp)
    assert kg.norms.stride(2) == Hkv
    kctx = tq.Context(seed=6, head_dim=d, bits=kb, qjl=qjl)
    vctx = tq.Context(seed=6, head_dim=d, bits=vb)
    out = tq.attend_decode(kctx, vctx, torch.from_numpy(q).to(DEV), kg, vg, torch.from_numpy(lens).to(DEV))
    torch.cuda.synchronize()
    _say("token-strided planes", kb, vb, qjl, assert_attend_close(out.cpu().numpy().astype(np.float64), ref))


@pytest.mark.parametrize("kb,vb,qjl", [(3, 3, False), (4, 4, True)])
def test_attend_long_context_counts_every_token_once(kb, vb, qjl):
    """At long contexts each (batch, KV head) is split over many blocks and
    waves.  Every cached token must be counted exactly once: with one key
    repeated over the context (equal weights) and values +v for
    the first half of each sequence and the mirrored codes for the second half
    (-v: mirroring every b-bit code is a bitwise NOT of the packed bytes, and
    the Lloyd-Max codebook of a symmetric density is symmetric), the exact
    output is zero, while one 64-token step counted twice or skipped leaves
    at least 64 |v| / L."""
    d, B, Hkv, G, T = 128, 4, 8, 4, 32768
    kctx = tq.Context(seed=3, head_dim=d, bits=kb, qjl=qjl)
    vctx = tq.Context(seed=3, head_dim=d, bits=vb)
    gen = torch.Generator().manual_seed(77)

    def rand_bytes(n):
        return torch.randint(0, 256, (B, Hkv, 1, n), generator=gen, dtype=torch.uint8)

    kp = tq.PackedPlanes.empty(kctx, (B, Hkv, T), DEV)
    kp.codes.copy_(rand_bytes(kctx.code_bytes).expand(B, Hkv, T, kctx.code_bytes))
    kp.norms.fill_(0x3C00)                      # fp16 1.0
    if qjl:
        kp.signs.copy_(rand_bytes(kctx.sign_bytes).expand(B, Hkv, T, kctx.sign_bytes))
        kp.rnorms.fill_(0x3400)                 # fp16 0.25
    lens = [T, T - 2 * 4321, 2 * 6000, 2 * 777]  # even lengths
    cv = rand_bytes(vctx.code_bytes)
    codes = torch.full((B, Hkv, T, vctx.code_bytes), 0xFF, dtype=torch.uint8)
    norms = torch.full((B, Hkv, T), -1, dtype=torch.int16)   # NaN fp16 past each length
    for b, L in enumerate(lens):
        codes[b, :, :L // 2] = cv[b]
        codes[b, :, L // 2:L] = ~cv[b]
        norms[b, :, :L] = 0x3C00
    vp = tq.PackedPlanes.empty(vctx, (B, Hkv, T), DEV)
    vp.codes.copy_(codes)
    vp.norms.copy_(norms)
    q = torch.randn((B, Hkv * G, d), generator=gen).to(DEV)
    out = tq.attend_decode(kctx, vctx, q, kp, vp, torch.tensor(lens, dtype=torch.int32, device=DEV), t_max=T)
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    worst = float(np.abs(o).max())
    _say("long-context token coverage", kb, vb, qjl, "max |out|", worst, "one step of the shortest:", 64 / min(lens))
    assert np.all(np.isfinite(o))
    assert worst <= 1e-4


@pytest.mark.parametrize("d,bits,qjl", [(128, 4, False), (128, 3, True), (256, 4, True), (32, 2, False),
                                        (256, 3, False), (128, 2, True)])
def test_scores_full_matrix_matches_oracle(d, bits, qjl):
    cfg = oenc.Config(seed=3, head_dim=d, bits=bits, qjl=qjl)
    rng = np.random.default_rng(d + bits)
    x = rng.standard_normal((1000, d)) * np.exp(0.5 * rng.standard_normal(d))
    q = rng.standard_normal((19, d)).astype(np.float32)
    kp = _oracle_planes(x, cfg)
    ref = odec.scores(q.astype(np.float64), kp, cfg, scale=1 / math.sqrt(d))
    ctx = tq.Context(seed=3, head_dim=d, bits=bits, qjl=qjl)
    got = tq.scores(ctx, torch.from_numpy(q).to(DEV), tq.PackedPlanes.from_numpy(kp), top_k=0,
                    scale=1 / math.sqrt(d))
    torch.cuda.synchronize()
    err = np.abs(got.cpu().numpy() - ref).max()
    _say("scores max abs err", err)
    assert err <= LOGIT_ATOL


@pytest.mark.parametrize("k", [1, 10, 64])
def test_scores_topk_matches_oracle(k):
    w = wl.WORKLOADS["search_1m"]
    db, qs = wl.search_set(w, n=20000, n_queries=40)
    cfg = oenc.Config(seed=0, head_dim=256, bits=4, qjl=True)
    kp = _oracle_planes(db.double().numpy(), cfg)
    ref = odec.scores(qs.double().numpy(), kp, cfg)
    ctx = tq.Context(seed=0, head_dim=256, bits=4, qjl=True)
    s, i = tq.scores(ctx, qs.to(DEV), tq.PackedPlanes.from_numpy(kp), top_k=k)
    torch.cuda.synchronize()
    agree = assert_topk_valid(s.cpu().numpy(), i.cpu().numpy(), ref, k)
    _say("top-k agreement with the oracle's exact list", agree)


@pytest.mark.parametrize("d,bits,qjl,k", [(256, 4, True, 10), (256, 4, True, 16), (128, 3, False, 16),
                                           (256, 4, True, 17)])
def test_scores_topk_ties_pick_lower_indices(d, bits, qjl, k):
    """40 distinct vectors, each stored 300 times at scattered positions: equal
    keys give bit-equal scores, so within the GPU's list every vector's copies
    must be its lowest-indexed ones, whichever wave's range they sit in (the
    32 x 32-tile scorer for k <= 16, the 16 x 16 one for k = 17)."""
    cfg = oenc.Config(seed=5, head_dim=d, bits=bits, qjl=qjl)
    rng = np.random.default_rng(d + k)
    base = rng.standard_normal((40, d))
    ids = rng.permutation(np.repeat(np.arange(40), 300))
    kb = _oracle_planes(base, cfg)
    kp = {n: a[ids] for n, a in kb.items()}
    q = rng.standard_normal((37, d)).astype(np.float32)
    ref = odec.scores(q.astype(np.float64), kp, cfg)
    ctx = tq.Context(seed=5, head_dim=d, bits=bits, qjl=qjl)
    s, i = tq.scores(ctx, torch.from_numpy(q).to(DEV), tq.PackedPlanes.from_numpy(kp), top_k=k)
    torch.cuda.synchronize()
    s, i = s.cpu().numpy(), i.cpu().numpy()
    assert_topk_valid(s, i, ref, k)
    for qi in range(q.shape[0]):
        for v in np.unique(ids[i[qi]]):
            chosen = np.sort(i[qi][ids[i[qi]] == v])
            lowest = np.sort(np.nonzero(ids == v)[0])[:len(chosen)]
            assert np.array_equal(chosen, lowest), (qi, v, chosen[:4], lowest[:4])
    _say("top-k ties: lowest indices chosen", d, bits, qjl, k)


@pytest.mark.parametrize("k", [10, 16])
def test_scores_topk_rising_scores(k):
    """Keys whose scores rise with the index for every query, so each 32-key
    step beats every list's threshold: the insertion path at full load."""
    d = 256
    cfg = oenc.Config(seed=2, head_dim=d, bits=4, qjl=True)
    rng = np.random.default_rng(k)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    n = 30000
    x = np.linspace(0.5, 3.0, n)[:, None] * u[None, :] + 0.01 * rng.standard_normal((n, d))
    q = (u[None, :] + 0.02 * rng.standard_normal((24, d))).astype(np.float32)
    kp = _oracle_planes(x, cfg)
    ref = odec.scores(q.astype(np.float64), kp, cfg)
    ctx = tq.Context(seed=2, head_dim=d, bits=4, qjl=True)
    s, i = tq.scores(ctx, torch.from_numpy(q).to(DEV), tq.PackedPlanes.from_numpy(kp), top_k=k)
    torch.cuda.synchronize()
    agree = assert_topk_valid(s.cpu().numpy(), i.cpu().numpy(), ref, k)
    _say("top-k with rising scores: agreement", agree)


@pytest.mark.parametrize("d,bits,qjl", [(256, 4, True), (128, 3, False)])
@pytest.mark.parametrize("n_k,n_q", [(1, 1), (7, 3), (31, 33), (33, 1), (95, 64)])
def test_scores_tiny_key_sets(d, bits, qjl, n_k, n_q):
    """Key sets shorter than one 32-key step or a few steps long, and one or
    a few queries: most waves of the workgroup have no key range, the first
    step is partly past the end; full matrix and top-k (k up to n_k)."""
    cfg = oenc.Config(seed=4, head_dim=d, bits=bits, qjl=qjl)
    rng = np.random.default_rng(n_k * 131 + n_q + d)
    x = rng.standard_normal((n_k, d))
    q = rng.standard_normal((n_q, d)).astype(np.float32)
    kp = _oracle_planes(x, cfg)
    # attention-logit scale (N(0,1) vectors: logits of order 1)
    scale = 1 / math.sqrt(d)
    ref = odec.scores(q.astype(np.float64), kp, cfg, scale=scale)
    ctx = tq.Context(seed=4, head_dim=d, bits=bits, qjl=qjl)
    planes = tq.PackedPlanes.from_numpy(kp)
    full = tq.scores(ctx, torch.from_numpy(q).to(DEV), planes, top_k=0, scale=scale)
    torch.cuda.synchronize()
    assert np.abs(full.cpu().numpy() - ref).max() <= LOGIT_ATOL
    for k in sorted({1, min(10, n_k), min(16, n_k)}):
        s, i = tq.scores(ctx, torch.from_numpy(q).to(DEV), planes, top_k=k, scale=scale)
        torch.cuda.synchronize()
        assert_topk_valid(s.cpu().numpy(), i.cpu().numpy(), ref, k)
    _say("tiny key sets", d, bits, qjl, n_k, n_q)


def test_same_inputs_give_bit_identical_outputs():
    """Run-to-run determinism: encode, decode attention and the fused top-k,
    each called twice on the same inputs, give bit-identical outputs (no
    atomics or scheduling order may leak into a result)."""
    gen = torch.Generator().manual_seed(21)
    B, Hkv, G, T, d = 2, 8, 4, 9000, 128
    K = torch.randn((B, Hkv, T, d), generator=gen).to(torch.bfloat16).to(DEV)
    V = torch.randn((B, Hkv, T, d), generator=gen).to(torch.bfloat16).to(DEV)
    q = torch.randn((B, Hkv * G, d), generator=gen).to(DEV)
    lens = torch.tensor([T, 5001], dtype=torch.int32, device=DEV)
    for kb, vb, qjl in ((3, 3, False), (4, 4, True)):
        kctx = tq.Context(seed=1, head_dim=d, bits=kb, qjl=qjl)
        vctx = tq.Context(seed=1, head_dim=d, bits=vb)
        runs = []
        for _ in range(2):
            kp, vp = tq.encode(kctx, K), tq.encode(vctx, V)
            o = tq.attend_decode(kctx, vctx, q, kp, vp, lens)
            torch.cuda.synchronize()
            runs.append((kp.numpy(), vp.numpy(), o.cpu().numpy()))
        for name in runs[0][0]:
            assert np.array_equal(runs[0][0][name], runs[1][0][name]), ("k", name)
        for name in runs[0][1]:
            assert np.array_equal(runs[0][1][name], runs[1][1][name]), ("v", name)
        assert np.array_equal(runs[0][2].view(np.uint32), runs[1][2].view(np.uint32)), "decode output"
    w = wl.WORKLOADS["search_1m"]
    db, qs = wl.search_set(w, DEV, n=60000, n_queries=70)
    ctx = tq.Context(seed=0, head_dim=256, bits=4, qjl=True)
    planes = tq.encode(ctx, db)
    r1 = [t.cpu().numpy() for t in tq.scores(ctx, qs, planes, top_k=10)]
    r2 = [t.cpu().numpy() for t in tq.scores(ctx, qs, planes, top_k=10)]
    assert np.array_equal(r1[0].view(np.uint32), r2[0].view(np.uint32)) and np.array_equal(r1[1], r2[1])
    _say("bit-identical across runs: encode, decode, top-k")

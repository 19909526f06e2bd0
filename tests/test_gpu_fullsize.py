"""Decode parity at the benchmark workloads' full sizes, on sampled heads.

Each case builds the whole workload on the GPU (every batch element and KV
head, full context) and calls tq_encode / tq_attend_decode with the sizes,
t_max and workspace the benchmark uses, so the launch configuration (chunk
split, block count) is the one that is timed.  For a few sampled (batch, KV head) pairs the oracle encodes
that head's K and V in float64; the GPU encoding of the head is compared
with it, then replaced by it, so the sampled heads' decode inputs come from
the oracle alone; their query heads' outputs are compared with the oracle's
decode.  Other heads only have to hold a valid encoding.
"""

import numpy as np
import pytest
import torch

from kv_cache_quantization_05_amd import binding as tq
from kv_cache_quantization_05_amd import workloads as wl
from oracle import decode as odec
from oracle import encode as oenc

from _parity import assert_attend_close, compare_encode, oracle_config

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(*a):
    print("[gpu-test]", *a, flush=True)


def _plane_slice(planes, b, g):
    out = {"codes": planes.codes[b, g], "norms": planes.norms[b, g]}
    if planes.signs is not None:
        out["signs"] = planes.signs[b, g]
        out["rnorms"] = planes.rnorms[b, g]
    return out


def _check_and_substitute(ctx, planes, x_head, b, g):
    """Compare the GPU encoding of head (b, g) with the oracle's, then write
    the oracle's planes over it.  Returns the oracle planes with a leading
    [1, 1] grid."""
    cfg = oracle_config(ctx)
    ref = oenc.encode(x_head.float().cpu().numpy().astype(np.float64), cfg)
    got = {k: v.cpu().numpy() for k, v in _plane_slice(planes, b, g).items()}
    for k in ("norms", "rnorms"):
        if k in got:
            got[k] = got[k].view(np.uint16)
    rep = compare_encode(got, ref, cfg)
    dst = _plane_slice(planes, b, g)
    for k in dst:
        src = ref[k] if k in ("codes", "signs") else ref[k].view(np.int16)
        dst[k].copy_(torch.from_numpy(np.ascontiguousarray(src)))
    return {k: ref[k][None, None] for k in ("codes", "norms", "signs", "rnorms") if k in ref}, rep


def _run(name, pairs, lens_fn):
    w = wl.WORKLOADS[name]
    G = w.Hq // w.Hkv
    kctx = tq.Context(seed=w.seed, head_dim=w.d, bits=w.k_bits, qjl=w.k_qjl)
    vctx = tq.Context(seed=w.seed, head_dim=w.d, bits=w.v_bits)
    K, V = wl.kv_pair(w, DEV)
    q = wl.queries(w, DEV)
    kp = kctx.new_planes((w.B, w.Hkv, w.T))
    vp = vctx.new_planes((w.B, w.Hkv, w.T))
    tq.encode(kctx, K, kp)
    tq.encode(vctx, V, vp)
    torch.cuda.synchronize()
    ref_planes = {}
    for b, g in pairs:
        kr, krep = _check_and_substitute(kctx, kp, K[b, g], b, g)
        vr, vrep = _check_and_substitute(vctx, vp, V[b, g], b, g)
        ref_planes[(b, g)] = (kr, vr)
        _say(name, "encode head", (b, g), krep, vrep)
    del K, V
    torch.cuda.synchronize()
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=DEV)
    ws = torch.zeros(tq.attend_workspace_bytes(kctx, vctx, w.B, w.Hq, w.Hkv, w.T), dtype=torch.uint8,
                     device=DEV)
    kc, vc = oracle_config(kctx), oracle_config(vctx)
    qn = q.cpu().numpy().astype(np.float64)
    for lens in lens_fn(w):
        lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
        tq.attend_decode(kctx, vctx, q, kp, vp, lens_t, t_max=w.T, out=out, workspace=ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        for (b, g), (kr, vr) in ref_planes.items():
            ref = odec.attend_decode(qn[b:b + 1, g * G:(g + 1) * G], kr, vr, kc, vc,
                                     np.array([lens[b]], dtype=np.int32))
            _say(name, "decode head", (b, g), "len", lens[b],
                 assert_attend_close(got[b:b + 1, g * G:(g + 1) * G], ref))


def test_fullsize_llama_t32k():
    _run("llama_t32k", [(0, 0), (0, 7)], lambda w: [[w.T]])


@pytest.mark.timeout(600)
def test_fullsize_llama_b4_t128k():
    # one sampled head at the full 128K context (the oracle takes ~1 min)
    _run("llama_b4_t128k", [(3, 5)], lambda w: [[w.T] * w.B])


def test_fullsize_llama_b16_t8k_ragged():
    # full lengths, then ragged ones (every batch element a different length,
    # one of them zero) in the same launch configuration
    def lens(w):
        return [[w.T] * w.B, [max(0, w.T - 613 * b) if b != 9 else 0 for b in range(w.B)]]

    _run("llama_b16_t8k", [(0, 0), (5, 3), (9, 1), (15, 7)], lens)

"""Comparison helpers for GPU-vs-oracle parity tests (test infrastructure)."""

import math

import numpy as np

from oracle import decode as odec
from oracle import encode as oenc

# Tolerances stated for this method: codes bit-exact outside a 1e-5 relative
# window around a threshold (and fewer than 1e-4 of entries inside it), fp16
# norms bit-exact, logits within 2e-3 absolute, attention outputs within 5e-3
# relative (L2 per output row).
CODE_WINDOW = 1e-5
MAX_WINDOW_FRACTION = 1e-4
LOGIT_ATOL = 2e-3
OUT_RTOL = 5e-3


def oracle_config(ctx_like):
    return oenc.Config(seed=ctx_like.seed, head_dim=ctx_like.head_dim, bits=ctx_like.bits,
                       qjl=ctx_like.qjl)


def compare_encode(gpu, ref, cfg, x_for_window=None):
    """gpu, ref: numpy plane dicts for the same vectors.  Returns a report and
    asserts the encode tolerance."""
    d, b = cfg.head_dim, cfg.bits
    g_code = oenc.unpack_bits_lsb(gpu["codes"], b, d)
    r_code = ref["code"]
    diff = g_code != r_code
    win = oenc.boundary_window(ref["z"], oenc.get_tables(cfg).tau, CODE_WINDOW)
    outside = diff & ~win
    rep = {"entries": diff.size, "mismatch": int(diff.sum()), "outside_window": int(outside.sum()),
           "window": int(win.sum())}
    assert rep["outside_window"] == 0, rep
    assert rep["mismatch"] <= max(MAX_WINDOW_FRACTION * diff.size, 0), rep
    assert np.array_equal(gpu["norms"], ref["norms"]), "fp16 norms differ"
    if cfg.qjl:
        same_codes = ~diff.any(axis=-1)
        assert np.array_equal(gpu["rnorms"][same_codes], ref["rnorms"][same_codes]), "fp16 residual norms differ"
        g_bits = oenc.unpack_bits_lsb(gpu["signs"], 1, cfg.m)
        r_bits = (ref["h"] > 0).astype(np.int64)
        sdiff = (g_bits != r_bits) & same_codes[..., None]
        rho_n = np.linalg.norm(ref["rho"], axis=-1, keepdims=True)
        swin = np.abs(ref["h"]) <= CODE_WINDOW * rho_n
        rep["sign_mismatch"] = int(sdiff.sum())
        rep["sign_outside_window"] = int((sdiff & ~swin).sum())
        assert rep["sign_outside_window"] == 0, rep
        assert rep["sign_mismatch"] <= MAX_WINDOW_FRACTION * sdiff.size, rep
    return rep


def rel_l2_rows(got, ref):
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def assert_attend_close(got, ref):
    rel = rel_l2_rows(got, ref)
    zero_rows = np.linalg.norm(ref, axis=-1) == 0
    assert np.all(got[zero_rows] == 0), "rows with no cached tokens must be zero"
    assert rel.max() <= OUT_RTOL, ("max relative L2 error", float(rel.max()))
    return float(rel.max()), float(np.abs(got - ref).max())


def assert_topk_valid(g_s, g_i, ref_scores, k):
    """Top-k parity where near-ties may legitimately reorder: GPU scores match
    the oracle's at the GPU's indices; every chosen index scores at least the
    oracle's k-th best minus twice the logit tolerance; order is descending."""
    n_q = ref_scores.shape[0]
    _, r_i = odec.top_k(ref_scores, k)
    kth = np.take_along_axis(ref_scores, r_i[:, -1:], axis=1)[:, 0]
    for qi in range(n_q):
        idx = g_i[qi]
        assert len(set(idx.tolist())) == k, "duplicate indices"
        assert np.all(np.diff(g_s[qi]) <= 1e-6), "not sorted"
        assert np.max(np.abs(g_s[qi] - ref_scores[qi, idx])) <= LOGIT_ATOL
        assert np.all(ref_scores[qi, idx] >= kth[qi] - 2 * LOGIT_ATOL)
    agree = np.mean([len(set(g_i[q]) & set(r_i[q])) / k for q in range(n_q)])
    return agree


def qjl_coef(cfg):
    return math.sqrt(math.pi / 2) / cfg.m

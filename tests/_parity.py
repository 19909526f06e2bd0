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
                       qjl=ctx_like.qjl, rotation=getattr(ctx_like, "rotation", "wht"),
                       norm_group=getattr(ctx_like, "norm_group", 0),
                       norm_correction=getattr(ctx_like, "norm_correction", False))


def compare_encode(gpu, ref, cfg, tie_ok=None):
    """gpu, ref: numpy plane dicts for the same vectors.  Returns a report and
    asserts the encode tolerance.  tie_ok (optional bool array shaped like the
    codes) marks entries where either of two codes is correct (exact ties);
    there a mismatch is allowed, every other entry of the vector is still
    compared."""
    d, b = cfg.head_dim, cfg.bits
    g_code = oenc.unpack_bits_lsb(gpu["codes"], b, d)
    r_code = ref["code"]
    raw_diff = g_code != r_code
    diff = raw_diff & ~tie_ok if tie_ok is not None else raw_diff
    win = oenc.boundary_window(ref["z"], oenc.get_tables(cfg).tau, CODE_WINDOW)
    outside = diff & ~win
    rep = {"entries": diff.size, "mismatch": int(diff.sum()), "outside_window": int(outside.sum()),
           "window": int(win.sum())}
    assert rep["outside_window"] == 0, rep
    assert rep["mismatch"] <= max(MAX_WINDOW_FRACTION * diff.size, 0), rep
    if cfg.norm_correction:
        # a corrected norm depends on its group's codes: compared where they
        # all match (a code inside the boundary window may differ)
        L = cfg.group_len
        grp_same = ~raw_diff.reshape(raw_diff.shape[:-1] + (cfg.head_dim // L, L)).any(axis=-1)
        if not cfg.norm_group:
            grp_same = grp_same[..., 0]
        rep["norm_groups_compared"] = int(grp_same.sum())
        assert np.array_equal(gpu["norms"][grp_same], ref["norms"][grp_same]), "fp16 norms differ"
    else:
        assert np.array_equal(gpu["norms"], ref["norms"]), "fp16 norms differ"
    if cfg.qjl:
        # the residual (so gamma and the signs) depends on the codes: compared
        # on the vectors whose codes all match
        same_codes = ~raw_diff.any(axis=-1)
        rep["qjl_vectors"] = int(same_codes.sum())
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
    """Attention outputs within 5e-3 relative per (b, h) row, read two ways:
    the row's L2 error against its L2 norm, and its largest elementwise error
    against its largest element (so an error confined to a few dims cannot
    hide in the row norm)."""
    rel = rel_l2_rows(got, ref)
    zero_rows = np.linalg.norm(ref, axis=-1) == 0
    assert np.all(got[zero_rows] == 0), "rows with no cached tokens must be zero"
    assert rel.max() <= OUT_RTOL, ("max relative L2 error", float(rel.max()))
    err = np.abs(got - ref).max(axis=-1)
    scale = np.abs(ref).max(axis=-1)
    elem = np.where(scale > 0, err / np.where(scale > 0, scale, 1.0), err)
    assert elem.max() <= OUT_RTOL, ("max elementwise error relative to the row's max", float(elem.max()))
    return float(rel.max()), float(elem.max()), float(np.abs(got - ref).max())


def assert_topk_valid(g_s, g_i, ref_scores, k, tol=LOGIT_ATOL):
    """Top-k parity where near-ties may legitimately reorder.

    For each query: the indices are distinct and valid; the GPU's scores are
    the oracle's scores of those indices within the logit tolerance; the list
    is in descending order, equal scores by ascending index; at every rank r
    the GPU's r-th score is no worse than the oracle's r-th best minus twice
    the tolerance; and every key the oracle scores above the GPU's k-th
    choice by more than twice the tolerance was chosen.  Returns the mean
    fraction of the oracle's top-k that the GPU chose (a report, not a gate)."""
    n_q, n_k = ref_scores.shape
    r_s, r_i = odec.top_k(ref_scores, k)
    agree = []
    for qi in range(n_q):
        idx = np.asarray(g_i[qi], dtype=np.int64)
        s = np.asarray(g_s[qi], dtype=np.float64)
        assert np.all((idx >= 0) & (idx < n_k)), "index out of range"
        assert len(set(idx.tolist())) == k, "duplicate indices"
        assert np.all(np.diff(s) <= 0), "not sorted"
        eq = np.diff(s) == 0
        assert np.all(np.diff(idx)[eq] > 0), "equal scores not ordered by index"
        assert np.max(np.abs(s - ref_scores[qi, idx])) <= tol, "scores differ from the oracle's"
        assert np.all(s >= r_s[qi] - 2 * tol), "a rank scores below the oracle's rank"
        kth = ref_scores[qi, idx[-1]]
        must = np.nonzero(ref_scores[qi] > kth + 2 * tol)[0]
        missing = set(must.tolist()) - set(idx.tolist())
        assert not missing, ("clearly better keys not chosen", sorted(missing)[:5])
        agree.append(len(set(idx.tolist()) & set(r_i[qi].tolist())) / k)
    return float(np.mean(agree))


def qjl_coef(cfg):
    return math.sqrt(math.pi / 2) / cfg.m

"""Oracle decode: dequantise, attention logits, softmax.V and top-k.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The GPU path never reconstructs keys: it rotates the query once and scores it
against centroids, because <q, R^T c[idx]> = <R q, c[idx]> ([TQ+ guide] §5.3,
pre-rotate-queries), and it rotates the attention output back at the end
([TQ+ guide] §6.1, the inverse-rotation fix).  Both are exact identities, so
this oracle uses the plain definitions instead: it rebuilds every key and
value explicitly in float64 and runs textbook attention
softmax(q K^T * scale) V ([TQ explainer] §4.3) with the query at full
precision ([TQ explainer] §2.2.2, §4.3).

Readings (the pages are silent):
  * MSE dequantisation: x_hat = (N16 / sqrt(d)) * R^T c[code], N16 the stored
    fp16 norm;
  * QJL keys (standard QJL estimator; the pages give no formula): the key
    estimate adds the JL reconstruction of the residual,
        k_hat = N16 * R^T ( c[code] / sqrt(d)
                            + gamma16 * sqrt(pi/2) / m * S^T sigma ),
    sigma_l = 2*bit_l - 1.  <q, k_hat> is unbiased for <q, x> over S because
    E[sign(g.rho) (g.u)] = sqrt(2/pi) <u, rho> / ||rho|| for g ~ N(0, I);
  * grouped-query attention: query head h reads KV head h // (Hq / Hkv);
  * a decode query attends to every cached position j < seq_len (no mask);
    seq_len == 0 gives a zero output row;
  * values are always MSE-only; the output is in the original domain;
  * top-k: descending score, ties to the lower index.
"""

import math

import numpy as np

from .encode import Config, get_tables, unpack_bits_lsb


def fp16_value(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def codes_of(planes, cfg: Config):
    return unpack_bits_lsb(planes["codes"], cfg.bits, cfg.head_dim)


def dequant(planes, cfg: Config, with_qjl=None):
    """Explicit float64 reconstruction of every vector in `planes`.

    with_qjl defaults to cfg.qjl; values (MSE-only) pass with_qjl=False.
    """
    t = get_tables(cfg)
    d = cfg.head_dim
    use_qjl = cfg.qjl if with_qjl is None else with_qjl
    code = codes_of(planes, cfg)
    n16 = fp16_value(planes["norms"])
    if cfg.norm_group:                                # one norm per 32-block:
        L = cfg.group_len                             # y_b = (N_b / sqrt(32)) c[code_b]
        cg = t.c[code].reshape(code.shape[:-1] + (d // L, L))
        y = (n16[..., None] * cg / math.sqrt(L)).reshape(code.shape)
        return y @ t.R                                # R^T y, row-vector form
    u = t.c[code] / math.sqrt(d)                      # rotated-domain unit estimate
    if use_qjl:
        bits = unpack_bits_lsb(planes["signs"], 1, cfg.m)
        sigma = 2.0 * bits - 1.0
        g16 = fp16_value(planes["rnorms"])
        u = u + (g16 * math.sqrt(math.pi / 2.0) / cfg.m)[..., None] * (sigma @ t.S)
    return n16[..., None] * (u @ t.R)                 # R^T u, row-vector form


def scores(q, k_planes, cfg: Config, scale=1.0):
    """Logits s[i, j] = scale * <q_i, k_hat_j> for q[n_q, d] and n_k packed keys."""
    k_hat = dequant(k_planes, cfg)
    return scale * (np.asarray(q, dtype=np.float64) @ k_hat.T)


def scores_rotated(q, k_planes, cfg: Config, scale=1.0):
    """The same logits in the form the pages' fused path reaches them, for
    large key sets: the query is rotated once and scored against the stored
    centroids (<q, R^T c> = <R q, c>, [TQ+ guide] §5.3 pre-rotate-queries),
    and a QJL key adds its sketch term against S R q, so no key is ever
    rebuilt in the original domain:
        s = scale * N * ( <R q, c[code]> / sqrt(d)
                          + gamma * sqrt(pi/2) / m * <S R q, sigma> ).
    Equal to scores() up to float64 rounding (pinned by a test)."""
    t = get_tables(cfg)
    d = cfg.head_dim
    q = np.asarray(q, dtype=np.float64)
    rq = q @ t.R.T                                     # R q, one per query
    code = codes_of(k_planes, cfg)
    n16 = fp16_value(k_planes["norms"])
    if cfg.norm_group:                                 # per-block norms weight each block
        L = cfg.group_len
        cg = t.c[code].reshape(code.shape[:-1] + (d // L, L))
        y = (n16[..., None] * cg / math.sqrt(L)).reshape(code.shape)
        return scale * (y @ rq.T).T
    s = (t.c[code] @ rq.T) / math.sqrt(d)              # [n_k, n_q]
    if cfg.qjl:
        sigma = 2.0 * unpack_bits_lsb(k_planes["signs"], 1, cfg.m) - 1.0
        g16 = fp16_value(k_planes["rnorms"])
        s = s + (g16 * math.sqrt(math.pi / 2.0) / cfg.m)[:, None] * (sigma @ (rq @ t.S.T).T)
    return scale * (s * n16[:, None]).T


def attend_decode(q, k_planes, v_planes, k_cfg: Config, v_cfg: Config, seq_lens, scale=None):
    """Decode attention for q[B, Hq, d] against planes laid out [B, Hkv, T, ...].

    Returns float64 output [B, Hq, d] in the original (unrotated) domain.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = k_planes["norms"].shape[1]
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, Hq, d))
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        for g in range(Hkv):
            kp = {k: v[b, g, :L] for k, v in k_planes.items()}
            vp = {k: v[b, g, :L] for k, v in v_planes.items()}
            K = dequant(kp, k_cfg)
            V = dequant(vp, v_cfg, with_qjl=False)
            for h in range(g * group, (g + 1) * group):
                s = scale * (K @ q[b, h])
                p = np.exp(s - s.max())
                p /= p.sum()
                out[b, h] = p @ V
    return out


def attend_prefill(q, k_planes, v_planes, k_cfg: Config, v_cfg: Config, seq_lens, scale=None):
    """Causal attention of a block of new positions over the packed cache.

    q[B, Hq, Tq, d]: the queries of the last Tq positions of each sequence;
    seq_lens[b] is the sequence's length including them, so query i of
    batch b sits at position p = seq_lens[b] - Tq + i and attends the cached
    positions j <= p (causal, [TQ explainer] §4.3 attention; the pages'
    prefill context scaling, [TQ+ guide] §1.2, §5.3).  A query with p < 0
    (a sequence shorter than the block) has no keys and a zero output.
    Planes are [B, Hkv, T, ...].  Returns float64 [B, Hq, Tq, d] in the
    original domain; keys and values are rebuilt explicitly, as in decode.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, Tq, d = q.shape
    Hkv = k_planes["codes"].shape[1]
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, Hq, Tq, d))
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        pos = L - Tq + np.arange(Tq)                    # position of each query
        for g in range(Hkv):
            kp = {k: v[b, g, :L] for k, v in k_planes.items()}
            vp = {k: v[b, g, :L] for k, v in v_planes.items()}
            K = dequant(kp, k_cfg)
            V = dequant(vp, v_cfg, with_qjl=False)
            visible = np.arange(L)[None, :] <= pos[:, None]          # [Tq, L] causal mask
            for h in range(g * group, (g + 1) * group):
                s = scale * (q[b, h] @ K.T)
                s = np.where(visible, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                rows = np.isfinite(m[:, 0])
                p = np.zeros_like(s)
                p[rows] = np.exp(s[rows] - m[rows])
                p[rows] /= p[rows].sum(axis=1, keepdims=True)
                out[b, h] = p @ V
    return out


def top_k(score_matrix, k):
    """Indices and values of the k largest scores per row; ties -> lower index."""
    s = np.asarray(score_matrix, dtype=np.float64)
    n = s.shape[-1]
    order = np.lexsort((np.broadcast_to(np.arange(n), s.shape), -s), axis=-1)[..., :k]
    return np.take_along_axis(s, order, axis=-1), order

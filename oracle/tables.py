"""Oracle tables: seeded rotation, Hadamard matrix, JL matrix, codebook.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What the pages fix:
  * The rotation is the structured random matrix R = D1 . H . D2: two random
    +-1 diagonals around a normalised Walsh-Hadamard matrix, applied in
    O(d log d) by a fast WHT ([TQ+ guide] §4, the comparison of the dense QR
    rotation and the fast D1.H.D2 rotation).
  * Rotation data is generated deterministically from a seed, never shipped
    as a static table, and the same seed gives the same matrix ([TQ+ guide]
    §3, Codex finding 6 and the same-seed test it names).
  * The rotation is fixed and shared by all vectors ([TQ+ guide] §5.3, the
    pre-rotate-queries notes).
  * QJL projects with a random Gaussian matrix ([TQ explainer] §2.2.1-§2.2.2).
  * Quantisation uses a table of centroids ([TQ+ guide] §5.2, Phase-1 file
    list; §5.3 names an fp16 centroid LUT).

Readings taken where the pages are silent:
  * PRNG: SplitMix64 (Steele, Lea and Flood, OOPSLA 2014).  D1 is the first d
    outputs of a generator seeded with `seed`, D2 the next d outputs; an
    output gives +1 when its top bit is 0, else -1.
  * S (m x d, row-major): a second SplitMix64 stream seeded with
    seed XOR 0x514A4C0000000000; entries are made two at a time by the
    Box-Muller transform from consecutive outputs z1, z2:
        u1 = ((z1 >> 11) + 1) * 2^-53,  u2 = (z2 >> 11) * 2^-53
        g0 = sqrt(-2 ln u1) cos(2 pi u2),  g1 = sqrt(-2 ln u1) sin(2 pi u2)
    computed in double and rounded to float32.
  * H is in Sylvester (natural) order, H_ij = (-1)^popcount(i & j), scaled
    once by 1/sqrt(d).
  * Codebook: the Lloyd-Max (minimum-MSE) quantiser of N(0,1) with 2^b levels
    (Max 1960), rounded to fp16, sorted ascending; thresholds are midpoints of
    adjacent fp16 centroids, exact in float32.
"""

import math
from functools import lru_cache

import numpy as np

MASK64 = (1 << 64) - 1
S_STREAM_XOR = 0x514A4C0000000000
HAAR_STREAM_XOR = 0x4841415200000000


def splitmix64(state):
    """Yield SplitMix64 outputs from a 64-bit state (Steele/Lea/Flood 2014).

    state += golden gamma; z = state; then two xor-shift-multiply rounds and a
    final xor-shift.  Plain Python integers keep every step exact.
    """
    state &= MASK64
    while True:
        state = (state + 0x9E3779B97F4A7C15) & MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        yield z ^ (z >> 31)


def rotation_signs(seed, d):
    """D1 and D2 diagonals as int8 arrays of +-1 (reading: top bit 0 -> +1)."""
    gen = splitmix64(seed)
    out = np.empty(2 * d, dtype=np.int8)
    for i in range(2 * d):
        out[i] = 1 if (next(gen) >> 63) == 0 else -1
    return out[:d].copy(), out[d:].copy()


def hadamard(d):
    """Unnormalised Sylvester Hadamard matrix, H_ij = (-1)^popcount(i & j)."""
    return _hadamard(int(d)).copy()


@lru_cache(maxsize=None)
def _hadamard(d):
    idx = np.arange(d)
    pc = np.vectorize(lambda v: bin(v).count("1"))(idx[:, None] & idx[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def rotation_matrix(seed, d):
    """Dense R = D1 . (H / sqrt(d)) . D2 in float64 ([TQ+ guide] §4)."""
    d1, d2 = rotation_signs(seed, d)
    hn = hadamard(d) / math.sqrt(d)
    return d1.astype(np.float64)[:, None] * hn * d2.astype(np.float64)[None, :]


def fwht(v):
    """Fast Walsh-Hadamard transform along the last axis, unnormalised.

    The O(d log d) butterfly the pages use for the structured rotation
    ([TQ+ guide] §4).  Stage h pairs index i with i + h for i & h == 0.
    """
    y = np.array(v, dtype=np.float64, copy=True)
    d = y.shape[-1]
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y


def gaussian_matrix(seed, m, d):
    """QJL projection S (m x d), float32 values held as float64.

    Box-Muller on SplitMix64 output pairs, row-major fill (reading above).
    math.log / math.cos / math.sin are the C library's, as in a C host.
    """
    return _gaussian_stream(seed ^ S_STREAM_XOR, m, d)


def haar_rotation(seed, d):
    """Dense Haar-random rotation Q (d x d, float64), det(Q) = +1.

    The pages' dense alternative to D1.H.D2 ([TQ+ guide] §3: a rotation
    generated deterministically from a seed by a QR decomposition, with the
    log-determinant used to force det = +1; §4: the O(d^2) dense rotation
    beside the fast structured one).  Readings (the pages give no more):
      * G is d x d from a third SplitMix64 stream seeded with
        seed XOR 0x4841415200000000, filled row-major by the same
        Box-Muller pairs as S (entries rounded to float32);
      * G = Q R (Householder QR in float64), and Q's columns are multiplied
        by the signs of R's diagonal, which makes Q the unique QR factor with
        a positive diagonal in R (Haar-distributed for Gaussian G);
      * if det(Q) = -1, the first column is negated.
    The rotation is y = Q x, as R x for the structured rotation.
    """
    g = _gaussian_stream(seed ^ HAAR_STREAM_XOR, d, d)
    q, r = np.linalg.qr(g)
    q = q * np.where(np.diag(r) < 0, -1.0, 1.0)[None, :]
    sign, _ = np.linalg.slogdet(q)
    if sign < 0:
        q[:, 0] = -q[:, 0]
    return q


def _gaussian_stream(stream_seed, m, d):
    """m x d float32-valued Gaussians from the SplitMix64 stream seeded with
    stream_seed: Box-Muller on consecutive output pairs, row-major."""
    if (m * d) % 2:
        raise ValueError("m*d must be even")
    gen = splitmix64(stream_seed)
    flat = np.empty(m * d, dtype=np.float32)
    two_pi = 2.0 * math.pi
    for k in range(0, m * d, 2):
        z1 = next(gen)
        z2 = next(gen)
        u1 = ((z1 >> 11) + 1) * (2.0 ** -53)
        u2 = (z2 >> 11) * (2.0 ** -53)
        r = math.sqrt(-2.0 * math.log(u1))
        flat[k] = np.float32(r * math.cos(two_pi * u2))
        flat[k + 1] = np.float32(r * math.sin(two_pi * u2))
    return flat.reshape(m, d).astype(np.float64)


# ---------------------------------------------------------------------------
# Lloyd-Max quantiser of N(0,1)


def _pdf(t):
    return 0.0 if math.isinf(t) else math.exp(-0.5 * t * t) / math.sqrt(2.0 * math.pi)


def _mass(a, b):
    """P(a < X <= b) for X ~ N(0,1), via erfc on the side that keeps precision."""
    if a >= 0.0:
        return 0.5 * (math.erfc(a / math.sqrt(2.0)) - math.erfc(b / math.sqrt(2.0)))
    if b <= 0.0:
        return 0.5 * (math.erfc(-b / math.sqrt(2.0)) - math.erfc(-a / math.sqrt(2.0)))
    return 1.0 - 0.5 * math.erfc(-a / math.sqrt(2.0)) - 0.5 * math.erfc(b / math.sqrt(2.0))


@lru_cache(maxsize=None)
def _lloyd_max_cached(bits, tol, max_iter):
    return _lloyd_max(bits, tol, max_iter)


def lloyd_max_gaussian(bits, tol=1e-15, max_iter=100000):
    """Float64 Lloyd-Max centroids for N(0,1) with 2^bits levels, ascending."""
    return np.array(_lloyd_max_cached(int(bits), tol, max_iter))


def _lloyd_max(bits, tol, max_iter):
    """Float64 Lloyd-Max centroids for N(0,1) with 2^bits levels, ascending.

    Lloyd's two conditions alternate until the centroids move by < tol:
    thresholds are midpoints of neighbouring centroids; each centroid is the
    conditional mean of its cell, (pdf(a) - pdf(b)) / P(a < X <= b).
    """
    levels = 1 << bits
    c = [-3.0 + 6.0 * (k + 0.5) / levels for k in range(levels)]
    for _ in range(max_iter):
        t = [-math.inf] + [(c[k] + c[k + 1]) / 2.0 for k in range(levels - 1)] + [math.inf]
        nc = [(_pdf(t[k]) - _pdf(t[k + 1])) / _mass(t[k], t[k + 1]) for k in range(levels)]
        moved = max(abs(x - y) for x, y in zip(c, nc))
        c = nc
        if moved < tol:
            break
    return tuple(c)


def codebook(bits):
    """fp16-exact centroids (as float64), ascending: code 0 is the most negative."""
    c16 = lloyd_max_gaussian(bits).astype(np.float16)  # direct float64 -> fp16 RNE
    return np.sort(c16.astype(np.float64))


def thresholds(bits):
    """Midpoints between neighbouring fp16 centroids (exact in float32)."""
    c = codebook(bits)
    return (c[:-1] + c[1:]) / 2.0


def gaussian_distortion(centroids, cuts=None):
    """E[(X - Q(X))^2] for X ~ N(0,1) and a scalar quantiser, in closed form.

    Cells are (t_{k-1}, t_k] with t the midpoints unless `cuts` is given.  Per
    cell: E[X^2; I] - 2c E[X; I] + c^2 P(I), with E[X; I] = pdf(a) - pdf(b) and
    E[X^2; I] = P(I) + a pdf(a) - b pdf(b).
    """
    c = list(map(float, centroids))
    if cuts is None:
        cuts = [(c[k] + c[k + 1]) / 2.0 for k in range(len(c) - 1)]
    t = [-math.inf] + list(map(float, cuts)) + [math.inf]
    total = 0.0
    for k, ck in enumerate(c):
        a, b = t[k], t[k + 1]
        p = _mass(a, b)
        ex = _pdf(a) - _pdf(b)
        apa = 0.0 if math.isinf(a) else a * _pdf(a)
        bpb = 0.0 if math.isinf(b) else b * _pdf(b)
        ex2 = p + apa - bpb
        total += ex2 - 2.0 * ck * ex + ck * ck * p
    return total

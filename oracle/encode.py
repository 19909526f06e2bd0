"""Oracle encode: rotation -> norm -> scalar codebook -> bit packing -> QJL.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The steps follow the pages' order:
  1. per-vector norm extraction and rescale ([TQ+ guide] §5.1, the norm
     extraction named for the Python reference's PolarQuant module);
  2. the seeded structured rotation D1.H.D2 ([TQ+ guide] §4);
  3. MSE-only scalar quantisation against a centroid table, stored in blocks
     of 32 with the rotation width decoupled from the block size ([TQ+ guide]
     §5.1 "algorithm variant", §5.2, §6.1 commit map);
  4. bit packing of the codes;
  5. optionally, QJL: a Gaussian JL projection of the quantisation residual
     reduced to one sign bit per row ([Orión plan] Fase 3 "Implementación
     conceptual", qjl_residual sketch; [TQ explainer] §2.2), with the query
     kept at full precision.

Readings (the pages are silent):
  * norm: n = ||x||_2 of the input in float64, stored as fp16 rounded once,
    directly from float64 (RNE);
  * z = sqrt(d) * (R x) / n (unit-norm vector scaled so coordinates are about
    N(0,1)); n == 0 gives z = 0;
  * norm per 32-block (the layout behind the pages' 3.5-bit turbo3 figure,
    [TQ+ guide] §1.2, against one norm per 128 values, §5.2): n_b is the
    norm of block b of the rotated vector y = R x, z_b = sqrt(32) y_b / n_b,
    and the norms plane holds d/32 fp16 values per vector;
  * norm correction ([TQ+ guide] §11 names it; no formula is given): the
    stored norm is n sqrt(L) / ||c[code]|| over the L coordinates sharing it,
    so that the dequantised group (N / sqrt(L)) c[code] has exactly the
    original norm n (up to the fp16 rounding of N);
  * rotation "haar": the dense seeded QR rotation of tables.haar_rotation in
    place of D1.H.D2 ([TQ+ guide] §3, §4);
  * code_i = #{k : tau_k < z_i} (a tie goes to the lower code);
  * codes are an LSB-first bit stream: code j of a vector occupies bits
    b*j .. b*j+b-1, bit k of the stream is bit (k % 8) of byte k // 8, so a
    32-code block is 4*b bytes and a d-vector d*b/8 bytes;
  * QJL residual rho = (z - c[code]) / sqrt(d) (the residual of the unit
    vector in the rotated domain), gamma = ||rho||_2 stored as fp16, sign bit
    l = [ (S rho)_l > 0 ], packed as in the pseudocode's sign_bits array:
    byte l // 8, bit l % 8.
"""

import math
from dataclasses import dataclass

import numpy as np

from . import tables


@dataclass(frozen=True)
class Config:
    seed: int = 0
    head_dim: int = 128
    bits: int = 3
    block: int = 32
    qjl: bool = False
    qjl_dim: int = 0  # 0 -> head_dim
    rotation: str = "wht"       # "wht": D1.H.D2; "haar": dense seeded QR rotation
    norm_group: int = 0         # 0: one norm per vector; 32: one per 32-code block
    norm_correction: bool = False

    @property
    def m(self):
        return self.qjl_dim or self.head_dim

    @property
    def code_bytes(self):
        return self.head_dim * self.bits // 8

    @property
    def sign_bytes(self):
        return self.m // 8 if self.qjl else 0

    @property
    def norms_per_vector(self):
        return self.head_dim // self.norm_group if self.norm_group else 1

    @property
    def group_len(self):
        """Coordinates sharing one stored norm."""
        return self.norm_group or self.head_dim

    def check(self):
        d = self.head_dim
        if d < 32 or d > 256 or d & (d - 1):
            raise ValueError("head_dim must be a power of two in [32, 256]")
        if self.bits not in (2, 3, 4):
            raise ValueError("bits must be 2, 3 or 4")
        if self.block != 32:
            raise ValueError("block must be 32")
        if self.qjl and (self.m % 8 or self.m <= 0):
            raise ValueError("qjl_dim must be a positive multiple of 8")
        if self.rotation not in ("wht", "haar"):
            raise ValueError("rotation must be 'wht' or 'haar'")
        if self.norm_group not in (0, 32):
            raise ValueError("norm_group must be 0 (per vector) or 32 (per block)")
        if self.qjl and (self.norm_group or self.norm_correction):
            raise ValueError("QJL keys take one plain norm per vector")


class Tables:
    """All per-config tables, built once from the seed."""

    def __init__(self, cfg: Config):
        cfg.check()
        self.cfg = cfg
        self.d1, self.d2 = tables.rotation_signs(cfg.seed, cfg.head_dim)
        if cfg.rotation == "haar":
            self.R = tables.haar_rotation(cfg.seed, cfg.head_dim)
        else:
            self.R = tables.rotation_matrix(cfg.seed, cfg.head_dim)
        self.c = tables.codebook(cfg.bits)
        self.tau = tables.thresholds(cfg.bits)
        self.S = tables.gaussian_matrix(cfg.seed, cfg.m, cfg.head_dim) if cfg.qjl else None


_CACHE = {}


def get_tables(cfg: Config) -> Tables:
    if cfg not in _CACHE:
        _CACHE[cfg] = Tables(cfg)
    return _CACHE[cfg]


def fp16_bits(v):
    """float64 -> fp16 rounded once (numpy casts float64 to float16 directly)."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def pack_bits_lsb(values, width):
    """Pack unsigned ints of `width` bits, LSB-first, along the last axis."""
    v = np.asarray(values, dtype=np.uint8)
    bits = (v[..., :, None] >> np.arange(width, dtype=np.uint8)) & 1
    bits = bits.reshape(v.shape[:-1] + (v.shape[-1] * width,))
    return np.packbits(bits, axis=-1, bitorder="little")


def unpack_bits_lsb(packed, width, count):
    """Inverse of pack_bits_lsb: `count` fields of `width` bits."""
    bits = np.unpackbits(np.asarray(packed, dtype=np.uint8), axis=-1, bitorder="little")
    bits = bits[..., : count * width].reshape(bits.shape[:-1] + (count, width))
    weights = (1 << np.arange(width)).astype(np.int64)
    return (bits.astype(np.int64) * weights).sum(axis=-1)


def quantize(z, tau):
    """code = number of thresholds strictly below z (elementwise)."""
    return (np.asarray(z)[..., None] > np.asarray(tau)).sum(axis=-1)


def encode(x, cfg: Config):
    """Encode vectors x[..., d] (exact fp32 or bf16 values) into packed planes.

    Returns dict(codes=u8[..., d*b/8], norms=u16[...] fp16 bits,
                 signs=u8[..., m/8], rnorms=u16[...] fp16 bits)  (QJL planes
    only when cfg.qjl).  Intermediate values are returned under "z", "code",
    "rho" and "h" for the tests.
    """
    t = get_tables(cfg)
    d = cfg.head_dim
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] != d:
        raise ValueError("last axis must be head_dim")
    y = x @ t.R.T                                       # step 2: y = R x
    L = cfg.group_len
    if cfg.norm_group:                                  # step 1, per block: norms of the
        yg = y.reshape(y.shape[:-1] + (d // L, L))      # rotated vector's 32-blocks
        n = np.sqrt(np.sum(yg * yg, axis=-1))
    else:                                               # step 1: norm of the input
        yg = y[..., None, :]
        n = np.sqrt(np.sum(x * x, axis=-1))[..., None]
    safe = np.where(n > 0, n, 1.0)
    z = np.where(n[..., None] > 0, math.sqrt(L) * yg / safe[..., None], 0.0).reshape(y.shape)
    code = quantize(z, t.tau)                           # step 3: codebook
    stored = n
    if cfg.norm_correction:
        # the stored norm makes the reconstruction keep the group's norm:
        # ||(N'/sqrt(L)) c[code]|| = n  <=>  N' = n sqrt(L) / ||c[code]||
        cg = t.c[code].reshape(yg.shape)
        stored = n * math.sqrt(L) / np.sqrt(np.sum(cg * cg, axis=-1))
    out = {
        "codes": pack_bits_lsb(code, cfg.bits),         # step 4: packing
        "norms": fp16_bits(stored if cfg.norm_group else stored[..., 0]),
        "z": z,
        "code": code,
    }
    if cfg.qjl:                                         # step 5: QJL
        rho = (z - t.c[code]) / math.sqrt(d)
        gamma = np.sqrt(np.sum(rho * rho, axis=-1))
        h = rho @ t.S.T
        out["signs"] = pack_bits_lsb((h > 0).astype(np.uint8), 1)
        out["rnorms"] = fp16_bits(gamma)
        out["rho"] = rho
        out["h"] = h
    return out


def boundary_window(z, tau, rel=1e-5):
    """True where z lies within rel*max(1,|tau_k|) of its nearest threshold.

    Codes in this window may legitimately differ between two correct
    implementations that evaluate z in different precisions.
    """
    z = np.asarray(z, dtype=np.float64)
    diff = np.abs(z[..., None] - np.asarray(tau))
    tol = rel * np.maximum(1.0, np.abs(np.asarray(tau)))
    return (diff <= tol).any(axis=-1)

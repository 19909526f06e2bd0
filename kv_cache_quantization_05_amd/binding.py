"""ctypes binding of libtq (include/tq.h): argument marshalling only.

Every step of the method runs inside libtq's HIP kernels; this module turns
torch tensors into pointers, sizes and strides, and raises TQError with the
library's message on a non-zero status.  It never computes a result itself
and has no fallback: if libtq.so is missing or cannot be loaded, every call
raises.
"""

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtq.so")

TQ_DTYPE_F32 = 0
TQ_DTYPE_BF16 = 1
TQ_ROTATION_WHT = 0
TQ_ROTATION_HAAR = 1
_ROTATIONS = {"wht": TQ_ROTATION_WHT, "haar": TQ_ROTATION_HAAR}

EXPORTED = (
    "tq_ctx_create", "tq_ctx_free", "tq_tables_export", "tq_rotation_export", "tq_code_bytes",
    "tq_sign_bytes", "tq_norm_count",
    "tq_encode", "tq_scores", "tq_scores_workspace", "tq_attend_decode",
    "tq_attend_decode_workspace", "tq_attend_decode_static", "tq_attend_prefill",
    "tq_attend_prefill_workspace", "tq_last_error", "tq_version",
)


class TQError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"libtq status {status}: {msg}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("head_dim", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("block", ctypes.c_int32), ("qjl", ctypes.c_int32), ("qjl_dim", ctypes.c_int32),
                ("rotation", ctypes.c_int32), ("norm_group", ctypes.c_int32),
                ("norm_correction", ctypes.c_int32)]


class Planes(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("norms", ctypes.c_void_p), ("signs", ctypes.c_void_p),
                ("rnorms", ctypes.c_void_p), ("stride", ctypes.c_int64 * 3)]


_lib = None


def lib():
    """Load libtq.so once; raises if it is absent (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libtq.so not built ({LIB_PATH}); run kv_cache_quantization_05_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        cfgp = ctypes.POINTER(Config)
        L.tq_ctx_create.argtypes = [cfgp, ctypes.POINTER(vp)]
        L.tq_ctx_create.restype = i32
        L.tq_ctx_free.argtypes = [vp]
        L.tq_ctx_free.restype = None
        L.tq_tables_export.argtypes = [cfgp, vp, vp, vp, vp, vp]
        L.tq_tables_export.restype = i32
        L.tq_rotation_export.argtypes = [cfgp, vp]
        L.tq_rotation_export.restype = i32
        L.tq_norm_count.argtypes = [cfgp]
        L.tq_norm_count.restype = i64
        L.tq_code_bytes.argtypes = [cfgp]
        L.tq_code_bytes.restype = i64
        L.tq_sign_bytes.argtypes = [cfgp]
        L.tq_sign_bytes.restype = i64
        L.tq_encode.argtypes = [vp, vp, i32, i64, i64, i64, ctypes.POINTER(i64), Planes, vp]
        L.tq_encode.restype = i32
        L.tq_scores.argtypes = [vp, vp, i64, ctypes.c_float, Planes, i64, i32, vp, vp, vp, i64, vp]
        L.tq_scores.restype = i32
        L.tq_scores_workspace.argtypes = [vp, i64, i64, i32]
        L.tq_scores_workspace.restype = i64
        L.tq_attend_decode.argtypes = [vp, vp, vp, Planes, Planes, vp, i32, i32, i32, i64,
                                       ctypes.c_float, vp, vp, i64, vp]
        L.tq_attend_decode.restype = i32
        L.tq_attend_decode_static.argtypes = [vp, vp, vp, Planes, Planes, vp, i32, i32, i32, i64,
                                              ctypes.c_float, vp, vp]
        L.tq_attend_decode_static.restype = i32
        L.tq_attend_prefill.argtypes = [vp, vp, vp, Planes, Planes, vp, i32, i32, i32, i64, i64,
                                        ctypes.c_float, vp, vp, i64, vp]
        L.tq_attend_prefill.restype = i32
        L.tq_attend_prefill_workspace.argtypes = [vp, vp, i32, i32, i64]
        L.tq_attend_prefill_workspace.restype = i64
        L.tq_attend_decode_workspace.argtypes = [vp, vp, i32, i32, i32, i64]
        L.tq_attend_decode_workspace.restype = i64
        L.tq_last_error.argtypes = []
        L.tq_last_error.restype = ctypes.c_char_p
        L.tq_version.argtypes = []
        L.tq_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise TQError(status, lib().tq_last_error().decode())


def make_config(seed=0, head_dim=128, bits=3, qjl=False, qjl_dim=0, block=32, rotation="wht", norm_group=0,
                norm_correction=False):
    rot = _ROTATIONS[rotation] if isinstance(rotation, str) else int(rotation)
    return Config(seed, head_dim, bits, block, 1 if qjl else 0, qjl_dim, rot, norm_group,
                  1 if norm_correction else 0)


def rotation_export(**cfg_kw):
    """Host-only: the dense rotation R (d x d float64, y = R x) of a config."""
    import numpy as np
    cfg = make_config(**cfg_kw)
    r = np.zeros((cfg.head_dim, cfg.head_dim), np.float64)
    _check(lib().tq_rotation_export(ctypes.byref(cfg), r.ctypes.data))
    return r


def tables_export(seed=0, head_dim=128, bits=3, qjl=False, qjl_dim=0):
    """Host-only copy of the tables libtq builds for a config (no GPU needed)."""
    import numpy as np
    cfg = make_config(seed, head_dim, bits, qjl, qjl_dim)
    m = qjl_dim or head_dim
    d1 = np.zeros(head_dim, np.int8)
    d2 = np.zeros(head_dim, np.int8)
    cb = np.zeros(1 << bits, np.float32)
    th = np.zeros((1 << bits) - 1, np.float32)
    S = np.zeros((m, head_dim), np.float32) if qjl else None
    _check(lib().tq_tables_export(ctypes.byref(cfg), d1.ctypes.data, d2.ctypes.data, cb.ctypes.data,
                                  th.ctypes.data, S.ctypes.data if S is not None else None))
    return {"d1": d1, "d2": d2, "codebook": cb, "thresholds": th, "S": S}


def code_bytes(head_dim, bits):
    return lib().tq_code_bytes(ctypes.byref(make_config(0, head_dim, bits)))


def _stream_ptr(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


class Context:
    """A libtq context (rotation, codebook and QJL tables on the current GPU)."""

    def __init__(self, seed=0, head_dim=128, bits=3, qjl=False, qjl_dim=0, rotation="wht", norm_group=0,
                 norm_correction=False):
        self.cfg = make_config(seed, head_dim, bits, qjl, qjl_dim, rotation=rotation, norm_group=norm_group,
                               norm_correction=norm_correction)
        self.seed, self.head_dim, self.bits, self.qjl = seed, head_dim, bits, bool(qjl)
        self.rotation, self.norm_group, self.norm_correction = rotation, norm_group, bool(norm_correction)
        self.m = qjl_dim or head_dim
        h = ctypes.c_void_p()
        _check(lib().tq_ctx_create(ctypes.byref(self.cfg), ctypes.byref(h)))
        self._h = h

    @property
    def handle(self):
        return self._h

    @property
    def code_bytes(self):
        return self.head_dim * self.bits // 8

    @property
    def sign_bytes(self):
        return self.m // 8 if self.qjl else 0

    @property
    def norm_count(self):
        """fp16 norms per vector: 1, or head_dim / 32 with block norms."""
        return self.head_dim // self.norm_group if self.norm_group else 1

    def close(self):
        if getattr(self, "_h", None):
            lib().tq_ctx_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def new_planes(self, shape, device="cuda"):
        """Caller-owned dense planes for a vector grid `shape` (1 to 3 dims)."""
        return PackedPlanes.empty(self, tuple(shape), device)


@dataclass
class PackedPlanes:
    codes: torch.Tensor    # u8 [..., code_bytes]
    norms: torch.Tensor    # int16 (fp16 bits) [...], or [..., d/32] with block norms
    signs: torch.Tensor    # u8 [..., sign_bytes] or None
    rnorms: torch.Tensor   # int16 [...] or None

    @staticmethod
    def empty(ctx, shape, device):
        codes = torch.empty(shape + (ctx.code_bytes,), dtype=torch.uint8, device=device)
        nc = getattr(ctx, "norm_count", 1)
        norms = torch.empty(shape + ((nc,) if getattr(ctx, "norm_group", 0) else ()), dtype=torch.int16,
                            device=device)
        signs = rnorms = None
        if ctx.qjl:
            signs = torch.empty(shape + (ctx.sign_bytes,), dtype=torch.uint8, device=device)
            rnorms = torch.empty(shape, dtype=torch.int16, device=device)
        return PackedPlanes(codes, norms, signs, rnorms)

    @property
    def grid(self):
        return tuple(self.codes.shape[:-1])

    @property
    def block_norms(self):
        """True when the norms plane holds one norm per 32-code block."""
        return self.norms.dim() == self.codes.dim()

    def c_struct(self):
        """Planes struct; strides in vectors (3-D grid, padded in front).
        Every plane must share one vector layout (each vector's bytes of a
        plane contiguous), since the C ABI carries one set of strides: they
        are taken from the codes plane and checked against the others."""
        cb = self.codes.shape[-1]
        if self.codes.stride(-1) != 1 or any(x % cb for x in self.codes.stride()[:-1]):
            raise ValueError("codes plane: each vector's code bytes must be contiguous")
        st = [x // cb for x in self.codes.stride()[:-1]]
        for name, t in (("norms", self.norms), ("signs", self.signs), ("rnorms", self.rnorms)):
            if t is None:
                continue
            per_vec = name == "signs" or (name == "norms" and self.block_norms)
            per = t.shape[-1] if per_vec else 1
            lead = list(t.stride())[:-1] if per_vec else list(t.stride())
            if (per_vec and t.stride(-1) != 1) or lead != [x * per for x in st] or \
                    tuple(t.shape[:len(st)]) != self.grid:
                raise ValueError(f"{name} plane layout does not match the codes plane's vector strides")
        st = [0] * (3 - len(st)) + st
        p = Planes()
        p.codes = self.codes.data_ptr()
        p.norms = self.norms.data_ptr()
        p.signs = self.signs.data_ptr() if self.signs is not None else None
        p.rnorms = self.rnorms.data_ptr() if self.rnorms is not None else None
        for i in range(3):
            p.stride[i] = st[i]
        return p

    def to(self, device):
        f = lambda t: t.to(device) if t is not None else None  # noqa: E731
        return PackedPlanes(f(self.codes), f(self.norms), f(self.signs), f(self.rnorms))

    def numpy(self):
        out = {"codes": self.codes.cpu().numpy(), "norms": self.norms.cpu().numpy().view("uint16")}
        if self.signs is not None:
            out["signs"] = self.signs.cpu().numpy()
            out["rnorms"] = self.rnorms.cpu().numpy().view("uint16")
        return out

    @staticmethod
    def from_numpy(d, device="cuda"):
        import numpy as np
        t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(device)  # noqa: E731
        return PackedPlanes(t(d["codes"], np.uint8), t(d["norms"], np.int16),
                            t(d["signs"], np.uint8) if "signs" in d else None,
                            t(d["rnorms"], np.int16) if "rnorms" in d else None)


def encode(ctx: Context, x: torch.Tensor, planes: PackedPlanes = None, stream=None):
    """tq_encode over the vector grid x.shape[:-1] (up to 3 dims).

    x: fp32 or bf16 CUDA tensor [..., d] with a contiguous last dim.
    planes: output planes over the same grid (allocated if None).
    """
    grid = tuple(x.shape[:-1])
    if len(grid) > 3 or x.shape[-1] != ctx.head_dim or x.stride(-1) != 1:
        raise ValueError("x must be [..., head_dim] with <= 3 leading dims and unit last stride")
    if x.dtype == torch.float32:
        dt = TQ_DTYPE_F32
    elif x.dtype == torch.bfloat16:
        dt = TQ_DTYPE_BF16
    else:
        raise ValueError("x must be float32 or bfloat16")
    if planes is None:
        planes = ctx.new_planes(grid, x.device)
    if tuple(planes.grid) != grid:
        raise ValueError("planes grid does not match x")
    _check_planes(planes, ctx, grid, "out")
    n = [1] * (3 - len(grid)) + list(grid)
    xs = [0] * (3 - len(grid)) + list(x.stride()[:-1])
    xs_arr = (ctypes.c_int64 * 3)(*xs)
    _check(lib().tq_encode(ctx.handle, _ptr(x), dt, n[0], n[1], n[2], xs_arr, planes.c_struct(),
                           _stream_ptr(stream)))
    return planes


def attend_workspace_bytes(k_ctx, v_ctx, B, Hq, Hkv, t_max):
    return lib().tq_attend_decode_workspace(k_ctx.handle, v_ctx.handle, B, Hq, Hkv, t_max)


def _check_query(q, ctx, ndim, what="q"):
    """The C ABI carries no shapes or dtypes for q: check them here."""
    if not isinstance(q, torch.Tensor) or q.dim() != ndim:
        raise ValueError(f"{what} must be a {ndim}-D tensor")
    if q.dtype != torch.float32:
        raise ValueError(f"{what} must be float32")
    if not q.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if q.shape[-1] != ctx.head_dim:
        raise ValueError(f"{what} has last dim {q.shape[-1]}, the context's head_dim is {ctx.head_dim}")


def _check_planes(p, ctx, grid_prefix, what):
    if p.codes.shape[-1] != ctx.code_bytes or tuple(p.codes.shape[:-1]) != tuple(p.grid):
        raise ValueError(f"{what} planes do not match the context's code bytes per vector")
    nc = getattr(ctx, "norm_count", 1)
    want = tuple(p.grid) + ((nc,) if getattr(ctx, "norm_group", 0) else ())
    if tuple(p.norms.shape) != want:
        raise ValueError(f"{what} norms plane has shape {tuple(p.norms.shape)}, the context needs {want}")
    if ctx.qjl and (p.signs is None or p.rnorms is None or p.signs.shape[-1] != ctx.sign_bytes):
        raise ValueError(f"{what} planes lack the QJL sign/rnorm planes of the context")
    if tuple(p.grid[:len(grid_prefix)]) != tuple(grid_prefix):
        raise ValueError(f"{what} planes have grid {p.grid}, expected leading dims {grid_prefix}")


def _check_on_gpu(*tensors):
    """Every tensor handed to libtq must live on one GPU (checked last, so the
    shape and dtype checks above also run on a host without a GPU)."""
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1 or next(iter(devs)).type != "cuda":
        raise ValueError("q, planes, seq_lens and outputs must all be on the same GPU")


def _plane_tensors(p):
    return (p.codes, p.norms, p.signs, p.rnorms)


def _workspace(ws, need, device):
    """A caller's workspace is passed as (pointer, bytes): it must be a
    contiguous uint8 tensor on the GPU of the other arguments."""
    if ws is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    if ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.device != device:
        raise ValueError("workspace must be a contiguous uint8 tensor on q's device")
    return ws


def attend_decode(k_ctx: Context, v_ctx: Context, q: torch.Tensor, k: PackedPlanes, v: PackedPlanes,
                  seq_lens: torch.Tensor, t_max=None, scale=None, out=None, workspace=None, stream=None):
    """tq_attend_decode.  q: fp32 [B, Hq, d]; k, v: planes over [B, Hkv, Tcap];
    seq_lens: int32 [B] on the GPU; returns fp32 [B, Hq, d]."""
    _check_query(q, k_ctx, 3)
    B, Hq, d = q.shape
    if len(k.grid) != 3 or len(v.grid) != 3:
        raise ValueError("k and v planes must cover a 3-D grid [B, Hkv, Tcap]")
    Hkv = k.grid[1]
    _check_planes(k, k_ctx, (B, Hkv), "k")
    _check_planes(v, v_ctx, (B, Hkv), "v")
    if not isinstance(seq_lens, torch.Tensor) or seq_lens.dtype != torch.int32 or seq_lens.numel() != B \
            or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 tensor of B entries")
    if t_max is None:
        t_max = k.grid[2]
    if t_max > k.grid[2] or t_max > v.grid[2]:
        raise ValueError("t_max exceeds the cache capacity of the planes")
    if scale is None:
        scale = d ** -0.5
    if out is not None and (out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != (B, Hq, d)):
        raise ValueError("out must be a contiguous float32 [B, Hq, d] tensor")
    _check_on_gpu(q, seq_lens, out, *_plane_tensors(k), *_plane_tensors(v))
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    need = attend_workspace_bytes(k_ctx, v_ctx, B, Hq, Hkv, t_max)
    workspace = _workspace(workspace, need, q.device)
    _check(lib().tq_attend_decode(k_ctx.handle, v_ctx.handle, _ptr(q), k.c_struct(), v.c_struct(),
                                  _ptr(seq_lens), B, Hq, Hkv, t_max, ctypes.c_float(scale), _ptr(out),
                                  _ptr(workspace), workspace.numel(), _stream_ptr(stream)))
    return out


def attend_decode_static(k_ctx: Context, v_ctx: Context, q: torch.Tensor, k: PackedPlanes, v: PackedPlanes,
                         seq_lens: torch.Tensor, t_max=None, scale=None, out=None, stream=None):
    """tq_attend_decode_static: as attend_decode, with the library's fixed
    device buffer as workspace (the call allocates nothing when `out` is
    given)."""
    _check_query(q, k_ctx, 3)
    B, Hq, d = q.shape
    if len(k.grid) != 3 or len(v.grid) != 3:
        raise ValueError("k and v planes must cover a 3-D grid [B, Hkv, Tcap]")
    Hkv = k.grid[1]
    _check_planes(k, k_ctx, (B, Hkv), "k")
    _check_planes(v, v_ctx, (B, Hkv), "v")
    if not isinstance(seq_lens, torch.Tensor) or seq_lens.dtype != torch.int32 or seq_lens.numel() != B \
            or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 tensor of B entries")
    if t_max is None:
        t_max = k.grid[2]
    if t_max > k.grid[2] or t_max > v.grid[2]:
        raise ValueError("t_max exceeds the cache capacity of the planes")
    if scale is None:
        scale = d ** -0.5
    if out is not None and (out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != (B, Hq, d)):
        raise ValueError("out must be a contiguous float32 [B, Hq, d] tensor")
    _check_on_gpu(q, seq_lens, out, *_plane_tensors(k), *_plane_tensors(v))
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _check(lib().tq_attend_decode_static(k_ctx.handle, v_ctx.handle, _ptr(q), k.c_struct(), v.c_struct(),
                                         _ptr(seq_lens), B, Hq, Hkv, t_max, ctypes.c_float(scale), _ptr(out),
                                         _stream_ptr(stream)))
    return out


def prefill_workspace_bytes(k_ctx, v_ctx, B, Hq, Tq):
    return lib().tq_attend_prefill_workspace(k_ctx.handle, v_ctx.handle, B, Hq, Tq)


def attend_prefill(k_ctx: Context, v_ctx: Context, q: torch.Tensor, k: PackedPlanes, v: PackedPlanes,
                   seq_lens: torch.Tensor, t_max=None, scale=None, out=None, workspace=None, stream=None):
    """tq_attend_prefill.  q: fp32 [B, Hq, Tq, d] (the last Tq positions of
    each sequence); k, v: planes over [B, Hkv, Tcap] holding those positions;
    seq_lens: int32 [B] lengths including them; returns fp32 [B, Hq, Tq, d]."""
    _check_query(q, k_ctx, 4)
    B, Hq, Tq, d = q.shape
    if len(k.grid) != 3 or len(v.grid) != 3:
        raise ValueError("k and v planes must cover a 3-D grid [B, Hkv, Tcap]")
    Hkv = k.grid[1]
    _check_planes(k, k_ctx, (B, Hkv), "k")
    _check_planes(v, v_ctx, (B, Hkv), "v")
    if not isinstance(seq_lens, torch.Tensor) or seq_lens.dtype != torch.int32 or seq_lens.numel() != B \
            or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 tensor of B entries")
    if t_max is None:
        t_max = k.grid[2]
    if t_max > k.grid[2] or t_max > v.grid[2]:
        raise ValueError("t_max exceeds the cache capacity of the planes")
    if scale is None:
        scale = d ** -0.5
    if out is not None and (out.dtype != torch.float32 or not out.is_contiguous()
                            or tuple(out.shape) != (B, Hq, Tq, d)):
        raise ValueError("out must be a contiguous float32 [B, Hq, Tq, d] tensor")
    _check_on_gpu(q, seq_lens, out, *_plane_tensors(k), *_plane_tensors(v))
    if out is None:
        out = torch.empty((B, Hq, Tq, d), dtype=torch.float32, device=q.device)
    workspace = _workspace(workspace, prefill_workspace_bytes(k_ctx, v_ctx, B, Hq, Tq), q.device)
    _check(lib().tq_attend_prefill(k_ctx.handle, v_ctx.handle, _ptr(q), k.c_struct(), v.c_struct(),
                                   _ptr(seq_lens), B, Hq, Hkv, Tq, t_max, ctypes.c_float(scale), _ptr(out),
                                   _ptr(workspace), workspace.numel(), _stream_ptr(stream)))
    return out


def scores_workspace_bytes(k_ctx, n_q, n_k, top_k):
    return lib().tq_scores_workspace(k_ctx.handle, n_q, n_k, top_k)


def scores(k_ctx: Context, q: torch.Tensor, k: PackedPlanes, top_k=0, scale=1.0, out=None,
           out_idx=None, workspace=None, stream=None):
    """tq_scores.  q: fp32 [n_q, d]; k: planes over a 1-D grid [n_k].

    top_k == 0 returns the full [n_q, n_k] score matrix; otherwise
    (scores [n_q, top_k], indices [n_q, top_k]) best first."""
    _check_query(q, k_ctx, 2)
    n_q = q.shape[0]
    if len(k.grid) != 1:
        raise ValueError("k planes must cover a 1-D grid [n_k]")
    _check_planes(k, k_ctx, (), "k")
    n_k = k.grid[-1]
    shape = (n_q, n_k) if top_k == 0 else (n_q, top_k)
    if out is not None and (out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != shape):
        raise ValueError(f"out must be a contiguous float32 {shape} tensor")
    if top_k > 0 and out_idx is not None and (out_idx.dtype != torch.int64 or not out_idx.is_contiguous()
                                              or tuple(out_idx.shape) != shape):
        raise ValueError(f"out_idx must be a contiguous int64 {shape} tensor")
    _check_on_gpu(q, out, out_idx if top_k > 0 else None, *_plane_tensors(k))
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=q.device)
    if top_k > 0 and out_idx is None:
        out_idx = torch.empty(shape, dtype=torch.int64, device=q.device)
    need = scores_workspace_bytes(k_ctx, n_q, n_k, top_k)
    workspace = _workspace(workspace, need, q.device)
    _check(lib().tq_scores(k_ctx.handle, _ptr(q), n_q, ctypes.c_float(scale), k.c_struct(), n_k, top_k,
                           _ptr(out), _ptr(out_idx), _ptr(workspace), workspace.numel(),
                           _stream_ptr(stream)))
    return out if top_k == 0 else (out, out_idx)

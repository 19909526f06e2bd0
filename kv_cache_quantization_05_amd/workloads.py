"""Seeded synthetic inputs for the TurboQuant hot path.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic, so both the GPU path and the CPU oracle may consume what
it makes.  Every draw comes from a seeded torch.Generator on the requested
device (a CPU generator for small cases, a GPU one for the full-size runs),
in a fixed order, so a (workload, seed, device) triple always yields the same
tensors.

Workloads (Llama-3-8B-shaped KV heads; the quality benchmarks the pages cite
are not available, so these distributions stand in for real K/V):

  single_head      1 head, d=128, T=4096, fp32 K/V ~ N(0,1) * s_c with a
                   per-channel scale s_c = exp(0.5 N(0,1)) drawn independently
                   for K and V; one fp32 N(0,1) query.  turbo4, MSE only.
  llama_t32k       B=1, T=32768, 8 KV heads, 32 query heads, d=128; K/V
                   N(0,1) with 4 outlier channels per head scaled x20 (chosen
                   independently for K and V), rounded to bf16; fp32 N(0,1)
                   queries.  turbo3 keys and values.
  llama_b16_t8k    B=16, T=8192, same distribution; keys turbo4 + QJL (m=128),
                   values turbo4.
  llama_b4_t128k   B=4, T=131072, as llama_t32k plus 1% of the positions of
                   each batch (same for K, V and all heads) scaled x8; turbo3.
  llama_t32k_turbo2, llama_t32k_k4v2  as llama_t32k with 2-bit keys and
                   values, or 4-bit keys and 2-bit values.
  llama_t32k_block32  as llama_t32k with one fp16 norm per 32-code block
                   and norm correction (3.5 bits per value at turbo3).
  llama_t32k_haar  as llama_t32k with the dense seeded Haar rotation.
  llama_prefill_t8k  an 8K prompt of the 32K layer's shape and distribution:
                   its K and V encoded into the cache, then causal prefill
                   attention of all 8192 positions (fp32 N(0,1) queries
                   [B, Hq, Tq, d]).
  search_1m        1,000,000 unit vectors, d=256, from a mixture of 1000
                   normalised N(0,I) centres: x = normalise(centre + 0.3 g /
                   sqrt(256)); 1024 queries drawn the same way; turbo4 + QJL
                   (m=256), top-10 inner-product search.
"""

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    Hkv: int
    Hq: int
    d: int
    k_bits: int
    v_bits: int
    k_qjl: bool
    in_dtype: str              # "f32" or "bf16"
    spike_frac: float = 0.0    # fraction of positions scaled by spike_scale
    spike_scale: float = 8.0
    outliers: int = 0          # outlier channels per head
    outlier_scale: float = 20.0
    lognormal_channels: bool = False
    rotation: str = "wht"      # "wht" (D1.H.D2) or "haar" (dense seeded QR rotation)
    norm_group: int = 0        # 0: one norm per vector; 32: one per 32-code block
    norm_correction: bool = False
    seed: int = 0              # method seed (rotation, S)
    data_seed: int = 0
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def tokens(self):
        return self.B * self.T


WORKLOADS = {
    "single_head": Workload("single_head", 1, 4096, 1, 1, 128, 4, 4, False, "f32",
                            lognormal_channels=True),
    "llama_t32k": Workload("llama_t32k", 1, 32768, 8, 32, 128, 3, 3, False, "bf16",
                           outliers=4),
    "llama_b16_t8k": Workload("llama_b16_t8k", 16, 8192, 8, 32, 128, 4, 4, True, "bf16",
                              outliers=4),
    "llama_b4_t128k": Workload("llama_b4_t128k", 4, 131072, 8, 32, 128, 3, 3, False, "bf16",
                               outliers=4, spike_frac=0.01),
    # bit-width variants of the 32K layer: turbo2, and asymmetric turbo4 keys
    # with turbo2 values
    "llama_t32k_turbo2": Workload("llama_t32k_turbo2", 1, 32768, 8, 32, 128, 2, 2, False, "bf16",
                                  outliers=4),
    "llama_t32k_k4v2": Workload("llama_t32k_k4v2", 1, 32768, 8, 32, 128, 4, 2, False, "bf16",
                                outliers=4),
    # layout and rotation variants of the 32K layer
    "llama_t32k_block32": Workload("llama_t32k_block32", 1, 32768, 8, 32, 128, 3, 3, False, "bf16",
                                   outliers=4, norm_group=32, norm_correction=True),
    "llama_t32k_haar": Workload("llama_t32k_haar", 1, 32768, 8, 32, 128, 3, 3, False, "bf16",
                                outliers=4, rotation="haar"),
    # prefill: a whole 8K prompt encoded into the cache and attended causally
    "llama_prefill_t8k": Workload("llama_prefill_t8k", 1, 8192, 8, 32, 128, 3, 3, False, "bf16",
                                  outliers=4, extra={"Tq": 8192}),
    "search_1m": Workload("search_1m", 1, 1_000_000, 1, 1, 256, 4, 4, True, "f32",
                          extra={"centers": 1000, "sigma": 0.3, "n_queries": 1024, "top_k": 10}),
}


def context_kwargs(w: Workload, which="k"):
    """Keyword arguments of a binding Context (or oracle Config) for the
    workload's keys ("k") or values ("v")."""
    kw = dict(seed=w.seed, head_dim=w.d, bits=w.k_bits if which == "k" else w.v_bits,
              qjl=w.k_qjl if which == "k" else False, rotation=w.rotation, norm_group=w.norm_group,
              norm_correction=w.norm_correction)
    return kw


def scaled(w: Workload, **changes) -> Workload:
    """A copy of workload `w` with some fields replaced (for smaller test cases)."""
    d = {k: getattr(w, k) for k in w.__dataclass_fields__}
    d.update(changes)
    return Workload(**d)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def kv_pair(w: Workload, device="cpu", batches=None):
    """K and V caches [B, Hkv, T, d] in the workload's input dtype.

    Draw order: K channel structure, V channel structure, spike positions,
    then per batch element K then V values.  `batches` selects a subset of
    batch elements while keeping the full draw order (so a slice equals the
    same rows of the full workload).
    """
    g = _gen(device, 1000 + w.data_seed)
    dt = torch.float32
    ch = {}
    for name in ("k", "v"):
        if w.lognormal_channels:
            ch[name] = torch.exp(0.5 * torch.randn(w.d, generator=g, device=device, dtype=dt))
        else:
            scale = torch.ones(w.Hkv, w.d, device=device, dtype=dt)
            for h in range(w.Hkv):
                if w.outliers:
                    idx = torch.randperm(w.d, generator=g, device=device)[: w.outliers]
                    scale[h, idx] = w.outlier_scale
            ch[name] = scale
    spikes = None
    if w.spike_frac > 0:
        n_sp = max(1, int(round(w.spike_frac * w.T)))
        spikes = torch.stack([torch.randperm(w.T, generator=g, device=device)[:n_sp]
                              for _ in range(w.B)])
    out_dtype = torch.bfloat16 if w.in_dtype == "bf16" else torch.float32
    sel = range(w.B) if batches is None else list(batches)
    K = torch.empty((len(sel), w.Hkv, w.T, w.d), dtype=out_dtype, device=device)
    V = torch.empty_like(K)
    j = 0
    for b in range(w.B):
        for name, dst in (("k", K), ("v", V)):
            x = torch.randn((w.Hkv, w.T, w.d), generator=g, device=device, dtype=dt)
            if b not in sel:
                continue
            if w.lognormal_channels:
                x = x * ch[name][None, None, :]
            else:
                x = x * ch[name][:, None, :]
            if spikes is not None:
                x[:, spikes[b], :] *= w.spike_scale
            dst[j] = x.to(out_dtype)
        if b in sel:
            j += 1
    return K, V


def queries(w: Workload, device="cpu"):
    """fp32 N(0,1) decode queries [B, Hq, d], or [B, Hq, Tq, d] for a prefill
    workload."""
    g = _gen(device, 2000 + w.data_seed)
    shape = (w.B, w.Hq, w.extra["Tq"], w.d) if "Tq" in w.extra else (w.B, w.Hq, w.d)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def search_set(w: Workload, device="cpu", n=None, n_queries=None):
    """Database [n, d] and queries [n_queries, d], fp32 unit vectors.

    x = normalise(centre[a] + sigma * g / sqrt(d)), centres normalised N(0,I),
    a uniform over centres.  The database is drawn before the queries.
    """
    n = w.T if n is None else n
    nq = w.extra["n_queries"] if n_queries is None else n_queries
    g = _gen(device, 3000 + w.data_seed)
    C = torch.randn((w.extra["centers"], w.d), generator=g, device=device)
    C = C / C.norm(dim=1, keepdim=True)

    def draw(count):
        a = torch.randint(0, C.shape[0], (count,), generator=g, device=device)
        x = C[a] + w.extra["sigma"] * torch.randn((count, w.d), generator=g, device=device) / (w.d ** 0.5)
        return x / x.norm(dim=1, keepdim=True)

    return draw(n), draw(nq)

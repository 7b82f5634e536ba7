"""Seeded synthetic inputs for the sparse-KV decode path.

This module only draws inputs: it holds none of the method's arithmetic (no
scoring, selection, planning or attention).  Both the HIP path (through the
binding) and the CPU oracle read the arrays it returns.

The shapes follow the five workloads the path is measured on:

  tiny      1 seq, 1 layer, L=4096, 32 q-heads / 8 KV heads, d=128, fp32, K=256
  b1_32k    Llama3.1-8B-shaped step: 1 seq, 32 layers, 32/8 heads, d=128,
            L=32768, bf16, K=2048, target KV in pinned host memory
  b16_grow  16 seqs growing from 2048 + U{0..2047} by one token per step up to
            16384, 32 layers, bf16, K=1024
  mha_64k   2 seqs, 1 layer, 32 q-heads = 32 KV heads, L=65536, K=4096, bf16
  mla_32k   4 seqs, 1 layer, 128 heads, latent 512 + rope 64, L=32768, K=2048

Key distribution (the "topic" reading): per (sequence, KV head) a unit
direction u; positions in the boosted set (4 sinks, a recent window of the
starting length, and a Bernoulli(f) set of heavy hitters) get +3 sigma along u
on top of N(0, I) noise; V ~ N(0, I).  Queries are sqrt(d) u + z_t with
z_{t+1} = 0.9 z_t + 0.44 N(0, I), z_0 ~ N(0, I) (0.44^2 / (1 - 0.9^2) ~ 1, so
z stays near unit variance).  The same query serves the retrieval head and
every target layer.  Values are drawn in float32 with torch's seeded
generators on the requested device and rounded to bfloat16
(round-to-nearest-even) where the workload is bf16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Preset:
    name: str
    kind: str                 # "gqa" | "mha" | "mqa" | "mla"
    batch: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int             # scored dimension (MLA: latent + rope)
    v_dim: int                # value dimension (MLA: latent)
    dtype: str                # "f32" | "bf16"
    max_len: int
    budget: int
    steps: int
    sinks: int = 4
    window: int = 64
    hh_frac: float = 0.05
    start_len: Optional[int] = None   # growth workloads: initial length
    offset_max: int = 0               # growth workloads: per-sequence offset U{0..offset_max}
    nope_dim: int = 0                 # MLA: per-head non-rotary key dim
    rope_dim: int = 0                 # MLA: rotary dim
    latent_dim: int = 0               # MLA: latent dim

    @property
    def n_groups(self) -> int:
        if self.kind == "gqa":
            return self.n_kv_heads
        if self.kind == "mqa":
            return 1
        return self.n_q_heads  # mha, mla: per head

    @property
    def scale(self) -> float:
        if self.kind == "mla":
            return 1.0 / math.sqrt(self.nope_dim + self.rope_dim)
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Preset":
        return replace(self, **kw)


PRESETS: Dict[str, Preset] = {
    "tiny": Preset("tiny", "gqa", batch=1, n_layers=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
                   v_dim=128, dtype="f32", max_len=4096, budget=256, steps=8),
    "b1_32k": Preset("b1_32k", "gqa", batch=1, n_layers=32, n_q_heads=32, n_kv_heads=8, head_dim=128,
                     v_dim=128, dtype="bf16", max_len=32768, budget=2048, steps=64),
    "b16_grow": Preset("b16_grow", "gqa", batch=16, n_layers=32, n_q_heads=32, n_kv_heads=8,
                       head_dim=128, v_dim=128, dtype="bf16", max_len=16384, budget=1024,
                       steps=14336, start_len=2048, offset_max=2047),
    "mha_64k": Preset("mha_64k", "mha", batch=2, n_layers=1, n_q_heads=32, n_kv_heads=32,
                      head_dim=128, v_dim=128, dtype="bf16", max_len=65536, budget=4096, steps=64,
                      window=128, hh_frac=0.02),
    "mla_32k": Preset("mla_32k", "mla", batch=4, n_layers=1, n_q_heads=128, n_kv_heads=1,
                      head_dim=576, v_dim=512, dtype="bf16", max_len=32768, budget=2048, steps=64,
                      nope_dim=128, rope_dim=64, latent_dim=512),
}


def _subseed(seed: int, tag: str) -> int:
    """Independent child seed per array, so one array never shifts another's draws."""
    tag_words = [ord(c) for c in tag]
    ss = np.random.SeedSequence([int(seed)] + tag_words)
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(0x7FFF_FFFF_FFFF_FFFF))


def _gen(device, seed: int, tag: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_subseed(seed, tag))
    return g


def lengths_schedule(p: Preset, steps: int, seed: int) -> np.ndarray:
    """[steps][B] int32 valid lengths per decode step."""
    if p.start_len is None:
        return np.full((steps, p.batch), p.max_len, dtype=np.int32)
    rng = np.random.default_rng(_subseed(seed, "offsets"))
    off = rng.integers(0, p.offset_max + 1, size=p.batch)
    s = np.arange(steps)[:, None]
    return np.minimum(p.start_len + off[None, :] + s, p.max_len).astype(np.int32)


@dataclass
class Workload:
    preset: Preset
    seed: int
    steps: int
    lengths: np.ndarray                     # [steps][B] int32 (host)
    q: torch.Tensor                         # [steps][B][Hq][d]   (GQA/MHA) or [steps][B][H][576] is NOT stored for MLA
    dlm_k: Optional[torch.Tensor] = None    # [B][Hkv][L][d]
    host_kv: Optional[torch.Tensor] = None  # [B][layers][Hkv][L][2][d]  (CPU, pinned if requested)
    boosted: Optional[torch.Tensor] = None  # [B][Hkv][L] bool (CPU), the boosted-position mask
    # MLA
    latent: Optional[torch.Tensor] = None   # [B][L][latent + rope]
    w_uk: Optional[torch.Tensor] = None     # [H][nope][latent]
    w_uv: Optional[torch.Tensor] = None     # [H][v_head][latent]
    q_nope: Optional[torch.Tensor] = None   # [steps][B][H][nope]
    q_rope: Optional[torch.Tensor] = None   # [steps][B][H][rope]
    extra: dict = field(default_factory=dict)


def _boosted_mask(p: Preset, lens0: np.ndarray, heads: int, seed: int) -> torch.Tensor:
    """[B][heads][L] bool: sinks, recent window of the starting length, heavy hitters."""
    B, L = p.batch, p.max_len
    g = _gen("cpu", seed, "heavy")
    m = torch.rand((B, heads, L), generator=g) < p.hh_frac
    m[:, :, :min(p.sinks, L)] = True
    for b in range(B):
        n0 = int(lens0[b])
        m[b, :, max(0, n0 - p.window):n0] = True
    return m


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def _ar1_queries(mean: torch.Tensor, steps: int, device, seed: int, tag: str) -> torch.Tensor:
    """q_t = mean + z_t, z_0 ~ N(0,I), z_{t+1} = 0.9 z_t + 0.44 N(0,I).  Returns [steps][...]"""
    g = _gen(device, seed, tag)
    z = torch.randn(mean.shape, generator=g, device=device)
    out = torch.empty((steps,) + tuple(mean.shape), dtype=torch.float32, device=device)
    for t in range(steps):
        out[t] = mean + z
        z = 0.9 * z + 0.44 * torch.randn(mean.shape, generator=g, device=device)
    return out


def generate(p: Preset | str, device="cpu", seed: int = 0, steps: Optional[int] = None,
             pin_host: bool = False, layers: Optional[int] = None) -> Workload:
    """Draw one workload.  ``layers`` overrides the number of target layers."""
    if isinstance(p, str):
        p = PRESETS[p]
    if layers is not None:
        p = p.with_(n_layers=int(layers))
    steps = p.steps if steps is None else int(steps)
    device = torch.device(device)
    if p.kind == "mla":
        return _generate_mla(p, device, seed, steps)
    B, Hq, Hkv, d, L = p.batch, p.n_q_heads, p.n_kv_heads, p.head_dim, p.max_len
    dt = p.torch_dtype
    lens = lengths_schedule(p, steps, seed)

    u = _unit(torch.randn((B, Hkv, d), generator=_gen("cpu", seed, "u")))          # [B][Hkv][d]
    boosted = _boosted_mask(p, lens[0], Hkv, seed)                                   # [B][Hkv][L]
    u_dev = u.to(device)
    bump = 3.0 * u_dev[:, :, None, :]                                                # [B][Hkv][1][d]
    boost_dev = boosted.to(device)[..., None].to(torch.float32)                      # [B][Hkv][L][1]

    gk = _gen(device, seed, "dlm_k")
    dlm_k = (torch.randn((B, Hkv, L, d), generator=gk, device=device) + bump * boost_dev).to(dt)

    host_kv = torch.empty((B, p.n_layers, Hkv, L, 2, d), dtype=dt, pin_memory=pin_host)
    gkv = _gen(device, seed, "target_kv")
    for layer in range(p.n_layers):
        k = torch.randn((B, Hkv, L, d), generator=gkv, device=device) + bump * boost_dev
        v = torch.randn((B, Hkv, L, d), generator=gkv, device=device)
        kv = torch.stack([k, v], dim=3).to(dt)                                       # [B][Hkv][L][2][d]
        host_kv[:, layer].copy_(kv.to("cpu"))
        del k, v, kv

    per_kv = Hq // Hkv
    head_dir = u_dev.repeat_interleave(per_kv, dim=1)                                # [B][Hq][d]
    q = _ar1_queries(math.sqrt(d) * head_dir, steps, device, seed, "q").to(dt)
    return Workload(p, seed, steps, lens, q=q, dlm_k=dlm_k, host_kv=host_kv, boosted=boosted)


def _generate_mla(p: Preset, device, seed: int, steps: int) -> Workload:
    B, H, L = p.batch, p.n_q_heads, p.max_len
    C, R, dn = p.latent_dim, p.rope_dim, p.nope_dim
    dt = p.torch_dtype
    lens = lengths_schedule(p, steps, seed)
    u = _unit(torch.randn((B, C), generator=_gen("cpu", seed, "u")))                # [B][C]
    boosted = _boosted_mask(p, lens[0], 1, seed)[:, 0]                               # [B][L]
    u_dev = u.to(device)
    g = _gen(device, seed, "latent")
    c = torch.randn((B, L, C), generator=g, device=device) \
        + 3.0 * u_dev[:, None, :] * boosted.to(device)[..., None].to(torch.float32)
    r = torch.randn((B, L, R), generator=g, device=device)
    latent = torch.cat([c, r], dim=-1).to(dt)                                         # [B][L][C+R]
    gw = _gen(device, seed, "weights")
    w_uk = (torch.randn((H, dn, C), generator=gw, device=device) / math.sqrt(C)).to(dt)
    w_uv = (torch.randn((H, dn, C), generator=gw, device=device) / math.sqrt(C)).to(dt)
    # per-head query direction: the head's key image of the sequence direction
    img = torch.matmul(w_uk.float(), u_dev.t().contiguous()).permute(2, 0, 1)      # [B][H][dn]
    q_nope = _ar1_queries(math.sqrt(dn + R) * _unit(img), steps, device, seed, "q_nope").to(dt)
    q_rope = _ar1_queries(torch.zeros((B, H, R), device=device), steps, device, seed, "q_rope").to(dt)
    return Workload(p, seed, steps, lens, q=q_nope, latent=latent, w_uk=w_uk, w_uv=w_uv,
                    q_nope=q_nope, q_rope=q_rope, boosted=boosted)


@dataclass
class FrontWeights:
    """Synthetic retrieval-head front end: embedding table, input-norm gain, Q/K projections,
    rotary parameters.  Random weights: they exercise the path, they carry no meaning."""
    emb: torch.Tensor        # [vocab][hidden]
    gamma: torch.Tensor      # [hidden]
    wq: torch.Tensor         # [H_q * d][hidden]
    wk: torch.Tensor         # [H_kv * d][hidden]
    hidden: int
    eps: float
    rope_base: float
    rope_factor: float
    rope_orig: int
    tokens: np.ndarray       # [steps][B] int32 token ids of the decode steps


def generate_front(p: Preset | str, device="cpu", seed: int = 0, steps: int = 8, vocab: int = 128256,
                   hidden: int = 4096, rope_base: float = 500000.0, rope_orig: int = 2048,
                   eps: float = 1e-5) -> FrontWeights:
    """Front-end weights in the workload's element type.  Embedding rows ~ N(0, 0.02^2) (the scale
    cancels in the input norm), gain ~ 1 + N(0, 0.1^2), projections ~ N(0, 1/hidden).  The rotary
    context scale is max(1, L_max / rope_orig): the distilled model's 2K context extended to the
    workload's length."""
    if isinstance(p, str):
        p = PRESETS[p]
    dt = p.torch_dtype
    device = torch.device(device)
    g = _gen(device, seed, "front")
    emb = (0.02 * torch.randn((vocab, hidden), generator=g, device=device)).to(dt)
    gamma = (1.0 + 0.1 * torch.randn((hidden,), generator=g, device=device)).to(dt)
    wq = (torch.randn((p.n_q_heads * p.head_dim, hidden), generator=g, device=device) / math.sqrt(hidden)).to(dt)
    wk = (torch.randn((p.n_kv_heads * p.head_dim, hidden), generator=g, device=device) / math.sqrt(hidden)).to(dt)
    rng = np.random.default_rng(_subseed(seed, "tokens"))
    tokens = rng.integers(0, vocab, size=(steps, p.batch), dtype=np.int64).astype(np.int32)
    return FrontWeights(emb, gamma, wq, wk, hidden, eps, rope_base, max(1.0, p.max_len / rope_orig), rope_orig,
                        tokens)


# ----------------------------------------------------------------------------
# NumPy views for the oracle (raw bits for bf16, float32 otherwise)
# ----------------------------------------------------------------------------


def to_numpy_raw(t: torch.Tensor) -> np.ndarray:
    """CPU NumPy view of a tensor's stored values: uint16 bits for bf16, else the values."""
    t = t.detach()
    if t.device.type != "cpu":
        t = t.to("cpu")
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def dtype_tag(t: torch.Tensor) -> str:
    return "bf16" if t.dtype == torch.bfloat16 else ("f32" if t.dtype == torch.float32 else "f64")

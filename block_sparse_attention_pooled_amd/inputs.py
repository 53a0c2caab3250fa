"""Seeded synthetic inputs shared by the GPU library's tests/bench and the oracle.

This module only draws random numbers and shapes them; it holds none of the
attention method's arithmetic.  The workloads stand in for the attention
layers the pages measure on (LLaDA-1.5 / LLaDA-8B and Dream-7B-Instruct at 8K
context with 256 denoising steps, and a 64K long-context case), whose weights
and evaluation data are not available:

* Q, K, V ~ N(0, 1) in fp32, rounded to bf16 (round-to-nearest-even) before
  either side sees them.
* Per-query-head concentration: Q[h] *= t_h with t_h log-uniform in [0.5, 4]
  ("different heads concentrate their attention mass to very different
  extents", Step-dLLM abstract).
* Attention sinks: keys 0-3 of every key head scaled by 4.
* Denoising-step drift: after every step Q, K, V += 0.02 * N(0, 1), a fresh draw
  per element (the Step-dLLM abstract: attention patterns stay similar only
  over nearby steps), with a full redraw of Q and K at chosen steps (the same
  abstract: patterns can also change suddenly at some points).
* Block structure (the structured 8K variant only, for the mask-quality
  measurement): each key head g draws a unit direction e[g, j] per key block j;
  every key token of block j gets + a * e[g, j], and every query token of block
  i of head h gets + a * (sum of e[g(h), j] over its target blocks j: its own
  block and 4 random ones), with a = structure * (4 * sqrt(d))^(1/2), so a
  target pair scores about +4 * structure^2 before the head temperature.  The
  targets and directions are redrawn with Q and K.
* Shared query heads (the shared-GQA 8K variant only): the query heads of one
  KV group are one draw shared by the group plus a small draw of their own,
  q_h = sqrt(shared) * base_g + sqrt(1 - shared) * own_h, and the heads of a
  group take one temperature (the group's), so a group's heads keep nearly
  the same blocks: the case sharing K/V tiles across a group's heads is for.
  Redrawn with Q and K.
* Column structure (the column-structured 8K variant only): each key head g
  draws one unit direction e[g] and L/64 heavy key tokens at random positions
  (not block-aligned); each heavy key gets + a * e[g] and every query token of
  a head of group g gets + a * e[g], with a = columns * (4 * sqrt(d))^(1/2),
  so every query scores its group's heavy keys about +4 * columns^2 higher:
  "vertical" attention shared by all queries, the case column sparsity
  ("PulseCol" abstract) is made for.  Redrawn with Q and K.
"""
from dataclasses import dataclass, field
import math

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    H: int                 # query heads
    Hkv: int               # key/value heads
    L: int                 # tokens
    d: int                 # head dim
    B: int                 # block size (tokens)
    sparsities: tuple      # fraction of blocks dropped by the global budget
    steps: int             # denoising steps
    dense_steps: int       # dense warm-up steps before the first mask
    refresh_every: int     # anchor period in steps; 0 = mask built once
    temperatures: bool     # per-head Q temperature
    sinks: bool            # keys 0-3 scaled by 4
    drift: float           # per-step drift std (0 = static)
    resample_steps: tuple = field(default=())
    seed: int = 0
    structure: float = 0.0  # block-affinity strength (0 = i.i.d. inputs)
    columns: float = 0.0    # heavy-column strength (0 = none)
    shared: float = 0.0     # variance a KV group's query heads share (0 = independent heads)

    @property
    def nb(self):
        return self.L // self.B

    @property
    def rows(self):
        return self.H * self.nb


WORKLOADS = {
    "tiny": Workload("tiny", H=2, Hkv=2, L=256, d=64, B=64, sparsities=(0.5,), steps=1,
                     dense_steps=0, refresh_every=0, temperatures=False, sinks=True,
                     drift=0.0, seed=1001),
    "llada_2k": Workload("llada_2k", H=32, Hkv=32, L=2048, d=128, B=64, sparsities=(0.9,),
                         steps=8, dense_steps=0, refresh_every=0, temperatures=True,
                         sinks=False, drift=0.02, seed=1002),
    "stepdllm_8k": Workload("stepdllm_8k", H=32, Hkv=32, L=8192, d=128, B=64,
                            sparsities=(0.9,), steps=256, dense_steps=0, refresh_every=32,
                            temperatures=True, sinks=False, drift=0.02,
                            resample_steps=(64, 160), seed=1003),
    "stepdllm_8k_structured": Workload("stepdllm_8k_structured", H=32, Hkv=32, L=8192, d=128,
                                       B=64, sparsities=(0.9,), steps=256, dense_steps=0,
                                       refresh_every=32, temperatures=True, sinks=False,
                                       drift=0.02, resample_steps=(80, 176), seed=1006,
                                       structure=1.0),
    "stepdllm_8k_columns": Workload("stepdllm_8k_columns", H=32, Hkv=32, L=8192, d=128,
                                    B=64, sparsities=(0.9,), steps=256, dense_steps=0,
                                    refresh_every=32, temperatures=True, sinks=False,
                                    drift=0.02, resample_steps=(80, 176), seed=1007,
                                    columns=1.0),
    "dream_gqa_8k": Workload("dream_gqa_8k", H=28, Hkv=4, L=8192, d=128, B=64,
                             sparsities=(0.7, 0.8, 0.9, 0.95), steps=64, dense_steps=0,
                             refresh_every=16, temperatures=True, sinks=False, drift=0.02,
                             seed=1004),
    "dream_gqa_8k_shared": Workload("dream_gqa_8k_shared", H=28, Hkv=4, L=8192, d=128, B=64,
                                    sparsities=(0.7, 0.8, 0.9, 0.95), steps=64, dense_steps=0,
                                    refresh_every=16, temperatures=True, sinks=False,
                                    drift=0.02, seed=1008, shared=0.99),
    "long_64k": Workload("long_64k", H=32, Hkv=32, L=65536, d=128, B=128, sparsities=(0.95,),
                         steps=128, dense_steps=26, refresh_every=0, temperatures=False,
                         sinks=True, drift=0.0, seed=1005),
}


def head_temperatures(H, seed):
    """t_h = exp(U(ln 0.5, ln 4)) per query head, from a CPU generator."""
    g = torch.Generator().manual_seed(seed)
    u = torch.rand(H, generator=g, dtype=torch.float64)
    return torch.exp(math.log(0.5) + u * (math.log(4.0) - math.log(0.5))).to(torch.float32)


class Trajectory:
    """Q/K/V (bf16) for each denoising step of a workload, generated in order.

    ``next()`` returns the inputs of step 0, 1, 2, ...  The fp32 state drifts
    between steps; the returned tensors are its bf16 rounding.
    """

    def __init__(self, w: Workload, device="cpu"):
        self.w = w
        self.device = torch.device(device)
        if w.temperatures and w.shared:   # one temperature per KV group
            temps = head_temperatures(w.Hkv, w.seed).repeat_interleave(w.H // w.Hkv)
        elif w.temperatures:
            temps = head_temperatures(w.H, w.seed)
        else:
            temps = torch.ones(w.H, dtype=torch.float32)
        self.temps = temps.to(self.device)
        self.gen = torch.Generator(device=self.device).manual_seed(w.seed)
        self.step = 0
        self.q, self.k = self._draw_qk()
        self.v = self._randn(w.Hkv, w.L, w.d)

    def _randn(self, *shape):
        return torch.randn(*shape, generator=self.gen, device=self.device, dtype=torch.float32)

    def _draw_qk(self):
        w = self.w
        q = self._randn(w.H, w.L, w.d)
        k = self._randn(w.Hkv, w.L, w.d)
        if w.sinks:
            k[:, 0:4, :] *= 4.0
        if w.shared:
            base = self._randn(w.Hkv, w.L, w.d)
            g = torch.arange(w.H, device=self.device) // (w.H // w.Hkv)
            q = math.sqrt(w.shared) * base[g] + math.sqrt(1.0 - w.shared) * q
        if w.structure:
            a = w.structure * math.sqrt(4.0 * math.sqrt(w.d))
            e = self._randn(w.Hkv, w.nb, w.d)
            e = e / e.norm(dim=-1, keepdim=True)
            k += a * e.repeat_interleave(w.B, dim=1)
            tgt = torch.randint(0, w.nb, (w.H, w.nb, 4), generator=self.gen, device=self.device)
            own = torch.arange(w.nb, device=self.device).view(1, w.nb, 1).expand(w.H, w.nb, 1)
            tgt = torch.cat([own, tgt], dim=2)                        # [H, nb, 5]
            g = torch.arange(w.H, device=self.device) // (w.H // w.Hkv)
            dirs = e[g.view(-1, 1, 1), tgt]                            # [H, nb, 5, d]
            q += a * dirs.sum(dim=2).repeat_interleave(w.B, dim=1)
        if w.columns:
            a = w.columns * math.sqrt(4.0 * math.sqrt(w.d))
            e = self._randn(w.Hkv, w.d)
            e = e / e.norm(dim=-1, keepdim=True)
            n_heavy = w.L // 64
            heavy = torch.argsort(torch.rand(w.Hkv, w.L, generator=self.gen, device=self.device),
                                  dim=1)[:, :n_heavy]                 # [Hkv, L/64] distinct
            k[torch.arange(w.Hkv, device=self.device).view(-1, 1), heavy] += a * e.view(
                w.Hkv, 1, w.d)
            g = torch.arange(w.H, device=self.device) // (w.H // w.Hkv)
            q += a * e[g].view(w.H, 1, w.d)
        return q * self.temps.view(-1, 1, 1), k

    def next(self):
        """bf16 (q, k, v) for the current step, then advance the state."""
        w = self.w
        if self.step in w.resample_steps:
            self.q, self.k = self._draw_qk()
        out = (self.q.to(torch.bfloat16), self.k.to(torch.bfloat16), self.v.to(torch.bfloat16))
        if w.drift:
            self.q += w.drift * self._randn(*self.q.shape)
            self.k += w.drift * self._randn(*self.k.shape)
            self.v += w.drift * self._randn(*self.v.shape)
        self.step += 1
        return out


def random_qkv(H, Hkv, L, d, seed, device="cpu", q_scale=1.0, sinks=False):
    """Plain seeded bf16 N(0,1) Q/K/V for small parity cases."""
    g = torch.Generator(device=device).manual_seed(seed)
    q = torch.randn(H, L, d, generator=g, device=device) * q_scale
    k = torch.randn(Hkv, L, d, generator=g, device=device)
    v = torch.randn(Hkv, L, d, generator=g, device=device)
    if sinks:
        k[:, 0:4, :] *= 4.0
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def to_host_f32(x):
    """bf16 device/host tensor -> fp32 numpy array holding the same values."""
    return x.detach().to("cpu").to(torch.float32).contiguous().numpy()

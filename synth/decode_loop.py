"""Seeded decode-loop workload for the boundary engine (torch, any device).

A batch of requests starts from equal-length prompts and decodes step by step.  Each
step brings one pre-RoPE query per (request, layer, query head) and one new K/V row per
(request, layer, KV head).  Queries are N(0, I) plus a focus direction per (request,
layer, KV head) that drifts slowly as a random walk on the unit sphere; a request
alternates between focused phases (the focus is present in its queries and new keys)
and diffuse phases (pure noise), which is the concentrated / diffuse swing of attention
sparsity the pages describe (GrowPage review on evolve.pub, "Summary" and Figure 3).
New keys carry the step's focus rotated to their own position (the cache holds
post-RoPE keys); prompt keys are N(0, I) with a fraction of heavy hitters along the
initial focus.  Values are N(0, I).  Everything is stored as bf16.

Input construction only: nothing here computes a summary, a working set, a decision
or a page rewrite.  The page pool is sized so that no grow is ever denied.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

from demand_paged_kv_amd import binding as Bd
from demand_paged_kv_amd import pool as PM
from demand_paged_kv_amd.engine import DeviceState

from . import workloads as SW


@dataclasses.dataclass
class DecodeSpec:
    B: int = 128
    L: int = 36
    Hq: int = 32
    Hkv: int = 8
    d: int = 128
    P: int = 16
    prompt: int = 1024
    steps: int = 4096
    seed: int = 4000
    drift: float = 0.05          # random-walk step of the focus per decode step (radians, rms)
    q_focus: float = 2.0         # focus amplitude in queries, in units of sqrt(d)
    k_focus: float = 1.0         # focus amplitude in new keys, in units of sqrt(d)
    hh_frac: float = 0.1         # fraction of prompt keys along the initial focus
    phase: tuple = (32, 256)     # focused / diffuse phase lengths in steps (uniform)
    stagger: bool = False        # request r starts with r % P rows in its write page
    params: dict = dataclasses.field(default_factory=lambda: dict(SW.PARAMS_DEFAULT))

    @property
    def A0(self) -> int:
        return self.prompt // self.P

    @property
    def max_pages(self) -> int:
        return self.A0 + 1 + (self.steps + self.P - 1) // self.P + 1

    @property
    def num_pages(self) -> int:
        return self.B * self.max_pages

    @property
    def max_pos(self) -> int:
        return self.prompt + self.P + self.steps


def _rotate(u: torch.Tensor, c: torch.Tensor, s: torch.Tensor) -> torch.Tensor:
    h = u.shape[-1] // 2
    x1, x2 = u[..., :h], u[..., h:]
    return torch.cat([x1 * c - x2 * s, x2 * c + x1 * s], dim=-1)


def _phase_table(rng, spec: DecodeSpec) -> np.ndarray:
    """[steps][B] 1.0 in focused phases, 0.0 in diffuse ones."""
    amp = np.zeros((spec.steps, spec.B), np.float32)
    lo, hi = spec.phase
    for b in range(spec.B):
        t, on = 0, bool(rng.integers(0, 2))
        while t < spec.steps:
            ln = int(rng.integers(lo, hi + 1))
            amp[t: t + ln, b] = 1.0 if on else 0.0
            t += ln
            on = not on
    return amp


class DecodeLoopGen:
    """Builds the initial device state and yields each step's queries and K/V rows."""

    def __init__(self, spec: DecodeSpec, device="cuda", contiguous: bool = False):
        self.spec = spec
        self.device = device
        self.contiguous = contiguous   # K/V pools in physically contiguous memory if available
        self.pool_memory = "ordinary"
        rng = np.random.default_rng(spec.seed)
        self.gen = torch.Generator(device=device)
        self.gen.manual_seed(spec.seed)
        self.amp = torch.from_numpy(_phase_table(rng, spec)).to(device)
        self.perm = rng.permutation(spec.num_pages)
        cos, sin = SW.rope_tables(spec.max_pos, spec.d)
        self.cos_np, self.sin_np = cos, sin
        self.cos = torch.from_numpy(cos).to(device)
        self.sin = torch.from_numpy(sin).to(device)
        f = torch.randn((spec.B, spec.L, spec.Hkv, spec.d), generator=self.gen, device=device)
        self.focus = f / f.norm(dim=-1, keepdim=True)
        self.t = 0

    def _randn(self, shape):
        return torch.randn(shape, generator=self.gen, device=self.device, dtype=torch.float32)

    @property
    def fill0(self) -> np.ndarray:
        """Rows in each request's write page before the first decode step."""
        sp = self.spec
        return (np.arange(sp.B) % sp.P) if sp.stagger else np.zeros(sp.B, np.int64)

    def initial_state(self) -> DeviceState:
        """Prompts in A0 = prompt/P shuffled allocation pages plus a write page holding
        fill0 further prompt rows (none unless staggered)."""
        sp, dev = self.spec, self.device
        A0, P = sp.A0, sp.P
        table = np.full((sp.B, sp.max_pages), -1, np.int32)
        used = sp.B * (A0 + 1)
        table[:, : A0 + 1] = self.perm[:used].reshape(sp.B, A0 + 1)
        refcount = np.zeros(sp.num_pages, np.int32)
        refcount[self.perm[:used]] = 1
        free = self.perm[used:]
        stack = np.zeros(sp.num_pages, np.int32)
        stack[: len(free)] = free
        shape = (sp.L, sp.num_pages, sp.Hkv, P, sp.d)
        k_pool, kk = PM.empty(shape, torch.bfloat16, dev, self.contiguous)
        v_pool, vk = PM.empty(shape, torch.bfloat16, dev, self.contiguous)
        k_pool.zero_()
        v_pool.zero_()
        self.pool_memory = "contiguous" if kk == vk == "contiguous" else "ordinary"
        npg = A0 + 1 if sp.stagger else A0                                         # pages holding prompt rows
        pages = torch.from_numpy(table[:, :npg].astype(np.int64)).to(dev)          # [B][npg]
        T = npg * P
        c, s = self.cos[:T], self.sin[:T]
        scale = sp.k_focus * math.sqrt(sp.d)
        for l in range(sp.L):
            k = self._randn((sp.B, sp.Hkv, T, sp.d))
            hh = (torch.rand((sp.B, sp.Hkv, T), generator=self.gen, device=dev) < sp.hh_frac).float()
            dirs = _rotate(self.focus[:, l, :, None, :], c, s)                       # [B][Hkv][T][d]
            k += (scale * hh)[..., None] * dirs
            v = self._randn((sp.B, sp.Hkv, T, sp.d))
            for src, pool in ((k, k_pool), (v, v_pool)):
                blk = src.to(torch.bfloat16).view(sp.B, sp.Hkv, npg, P, sp.d).permute(0, 2, 1, 3, 4)
                pool[l][pages] = blk
            del k, v, dirs, hh
        return DeviceState(
            L=sp.L, Hq=sp.Hq, Hkv=sp.Hkv, d=sp.d, P=P, num_pages=sp.num_pages, dtype=Bd.GP_BF16,
            k_pool=k_pool, v_pool=v_pool, page_table=torch.from_numpy(table).to(dev),
            n_alloc=torch.full((sp.B,), A0, dtype=torch.int32, device=dev),
            fill=torch.from_numpy(self.fill0.astype(np.int32)).to(dev),
            refcount=torch.from_numpy(refcount).to(dev), free_stack=torch.from_numpy(stack).to(dev),
            free_top=torch.tensor([len(free)], dtype=torch.int32, device=dev),
            sum_s=torch.zeros((sp.B, sp.L, sp.Hq, sp.d), dtype=torch.float32, device=dev),
            sum_l=torch.zeros((sp.B, sp.L, sp.Hq, sp.d), dtype=torch.float32, device=dev),
            pos=torch.from_numpy((sp.prompt + self.fill0).astype(np.int32)).to(dev),
            rope_cos=self.cos, rope_sin=self.sin)

    def step(self, out=None):
        """Inputs of the next decode step: q [B][L][Hq][d], k, v [B][L][Hkv][d] (bf16).
        Request r's token (and query) of step t sit at absolute position
        prompt + fill0[r] + t.  With ``out`` = (q, k, v) bf16 buffers the step is written
        into them (and they are returned)."""
        sp = self.spec
        t = self.t
        assert t < sp.steps
        G = sp.Hq // sp.Hkv
        f = self.focus + (sp.drift / math.sqrt(sp.d)) * self._randn(self.focus.shape)
        self.focus = f / f.norm(dim=-1, keepdim=True)
        a = self.amp[t][:, None, None, None]                                          # [B][1][1][1]
        qf = (a * (sp.q_focus * math.sqrt(sp.d))) * self.focus                         # [B][L][Hkv][d]
        q = self._randn((sp.B, sp.L, sp.Hq, sp.d)) + qf.repeat_interleave(G, dim=2)
        p = torch.from_numpy((sp.prompt + self.fill0 + t).astype(np.int64)).to(self.device)   # [B]
        kd = _rotate(self.focus, self.cos[p][:, None, None, :], self.sin[p][:, None, None, :])
        k = self._randn((sp.B, sp.L, sp.Hkv, sp.d)) + (a * (sp.k_focus * math.sqrt(sp.d))) * kd
        v = self._randn((sp.B, sp.L, sp.Hkv, sp.d))
        self.t += 1
        if out is not None:
            for dst, src in zip(out, (q, k, v)):
                dst.copy_(src)
            return out
        return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)

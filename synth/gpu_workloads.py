"""Full-size synthetic workloads generated directly in device memory (torch).

Same recipe as ``workloads.direct_case`` (pre-RoPE summaries b*u + noise, keys N(0, I)
plus a Zipf profile along each head's direction rotated to the request position),
vectorised in torch so that tens of GB of paged K/V can be produced on the GPU.  Input
construction only; the engine's outputs are computed by the library and the oracle.

``boundary_sweep`` is the 32-layer boundary sweep on the 8B GQA shape: 64 requests with
contexts log-uniform in [512, 16384], 32 query / 8 KV heads, head_dim 128, bf16, page 16,
30% of the requests planted as broadening demand, page ids shuffled across a 24,576-page
pool, every request at its capacity boundary (write page full).
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
class GpuWorkload:
    st: DeviceState
    n: np.ndarray            # [B] candidate slots
    A: np.ndarray            # [B] allocation pages
    regime: np.ndarray       # [B] 1 = planted broadening
    pos: np.ndarray
    params: dict
    seed: int
    name: str
    pool_memory: str = "ordinary"   # "contiguous": K/V pools in physically contiguous memory

    @property
    def B(self):
        return len(self.n)

    def total_tokens(self):
        return int(self.n.sum())


def _rotate(u: torch.Tensor, c: torch.Tensor, s: torch.Tensor) -> torch.Tensor:
    h = u.shape[-1] // 2
    x1, x2 = u[..., :h], u[..., h:]
    return torch.cat([x1 * c - x2 * s, x2 * c + x1 * s], dim=-1)


def pool_pair(L, num_pages, Hkv, P, d, layout, device, contiguous=False):
    """K and V pools as [L][num_pages][Hkv][P][d] views: "layer_major" stores them in that
    order; "page_major" stores [num_pages][L][Hkv][P][d] (all layers of a page together).
    With ``contiguous`` each pool is asked for physically contiguous memory.  Returns
    (k, v, kind) with kind "contiguous" when both pools got it."""
    shape = (L, num_pages, Hkv, P, d) if layout == "layer_major" else (num_pages, L, Hkv, P, d)
    assert layout in ("layer_major", "page_major"), layout
    k, kk = PM.empty(shape, torch.bfloat16, device, contiguous)
    v, vk = PM.empty(shape, torch.bfloat16, device, contiguous)
    if layout == "page_major":
        k, v = k.permute(1, 0, 2, 3, 4), v.permute(1, 0, 2, 3, 4)
    return k, v, ("contiguous" if kk == vk == "contiguous" else "ordinary")


def boundary_sweep(seed: int = 3000, B: int = 64, L: int = 32, Hq: int = 32, Hkv: int = 8, d: int = 128,
                   P: int = 16, num_pages: int = 24576, ctx=(512, 16384), grow_frac: float = 0.3,
                   s_zipf: float = 1.1, params: dict | None = None, device="cuda",
                   name: str = "boundary_sweep", layout: str = "layer_major",
                   contiguous: bool = False) -> GpuWorkload:
    rng = np.random.default_rng(seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    G = Hq // Hkv
    c = np.exp(rng.uniform(math.log(ctx[0]), math.log(ctx[1]), size=B))
    A = np.ceil(c / P).astype(np.int64)
    n = (A + 1) * P
    assert int((A + 1).sum()) <= num_pages, "pool too small for the drawn contexts"
    pos = (n + rng.integers(0, 64, size=B)).astype(np.int64)
    regime = np.zeros(B, np.int32)
    regime[rng.choice(B, size=int(round(grow_frac * B)), replace=False)] = 1
    max_pages = int(A.max()) + 8
    perm = rng.permutation(num_pages)
    table = np.full((B, max_pages), -1, np.int32)
    cur = 0
    for b in range(B):
        table[b, : A[b] + 1] = perm[cur: cur + A[b] + 1]
        cur += int(A[b]) + 1
    free = perm[cur:]
    refcount = np.zeros(num_pages, np.int32)
    refcount[perm[:cur]] = 1
    stack = np.zeros(num_pages, np.int32)
    stack[: len(free)] = free

    cos_np, sin_np = SW.rope_tables(int(pos.max()) + 1, d)
    cos = torch.from_numpy(cos_np).to(device)
    sin = torch.from_numpy(sin_np).to(device)
    u = torch.randn((B, L, Hq, d), generator=gen, device=device, dtype=torch.float64)
    u = u / u.norm(dim=-1, keepdim=True)
    reg = torch.from_numpy(regime).to(device).bool()[:, None, None]
    U = lambda lo, hi: lo + (hi - lo) * torch.rand((B, L, Hq), generator=gen, device=device, dtype=torch.float64)
    bs = torch.where(reg, U(0.2, 0.8), U(2.0, 5.0))
    bl = torch.where(reg, U(1.5, 3.0), U(0.5, 1.5))
    sum_s = (bs[..., None] * u + 0.1 * torch.randn((B, L, Hq, d), generator=gen, device=device, dtype=torch.float64)).float()
    sum_l = (bl[..., None] * u + 0.1 * torch.randn((B, L, Hq, d), generator=gen, device=device, dtype=torch.float64)).float()

    k_pool, v_pool, mem = pool_pair(L, num_pages, Hkv, P, d, layout, device, contiguous)
    for l in range(L):           # V and unused K pages: N(0, 1)
        k_pool[l].normal_(generator=gen)
        v_pool[l].normal_(generator=gen)
    scale = s_zipf * math.sqrt(d) / 2.0
    for b in range(B):
        nb = int(n[b])
        dirs = _rotate(u[b], cos[pos[b]].double(), sin[pos[b]].double()).float()     # [L][Hq][d]
        k = torch.randn((L, Hkv, nb, d), generator=gen, device=device, dtype=torch.float32)
        for j in range(G):
            rank = torch.argsort(torch.rand((L, Hkv, nb), generator=gen, device=device), dim=-1).float() + 1.0
            mu = scale * (math.log(nb) - torch.log(rank))                              # [L][Hkv][n]
            k += mu[..., None] * dirs[:, j::G][:, :, None, :]
        pages = torch.from_numpy(table[b, : A[b] + 1].astype(np.int64)).to(device)
        k_pool[:, pages] = k.to(torch.bfloat16).view(L, Hkv, int(A[b]) + 1, P, d).permute(0, 2, 1, 3, 4)
        del k
    st = DeviceState(L=L, Hq=Hq, Hkv=Hkv, d=d, P=P, num_pages=num_pages, dtype=Bd.GP_BF16,
                     k_pool=k_pool, v_pool=v_pool,
                     page_table=torch.from_numpy(table).to(device),
                     n_alloc=torch.from_numpy(A.astype(np.int32)).to(device),
                     fill=torch.full((B,), P, dtype=torch.int32, device=device),
                     refcount=torch.from_numpy(refcount).to(device),
                     free_stack=torch.from_numpy(stack).to(device),
                     free_top=torch.tensor([len(free)], dtype=torch.int32, device=device),
                     sum_s=sum_s.contiguous(), sum_l=sum_l.contiguous(),
                     pos=torch.from_numpy(pos.astype(np.int32)).to(device), rope_cos=cos, rope_sin=sin)
    return GpuWorkload(st, n, A, regime, pos, dict(params or SW.PARAMS_DEFAULT), seed, name, mem)


def prefix_share(seed: int = 5000, B: int = 256, L: int = 36, Hq: int = 32, Hkv: int = 8, d: int = 128,
                 P: int = 32, ctx=(1024, 32768), group: int = 16, prefix_pages: int = 64,
                 pool_frac: float = 0.8, alloc_frac: float = 0.8, grow_frac: float = 0.3, s_range=(0.8, 1.6),
                 free_pages: int | None = None, params: dict | None = None, device="cuda",
                 name: str = "prefix_share", contiguous: bool = False) -> GpuWorkload:
    """Prefix-sharing stress: groups of ``group`` consecutive requests share their first
    ``prefix_pages`` pages (refcount = group), contexts log-uniform in ``ctx``, Zipf
    exponent per request uniform in ``s_range``.  The pool holds ``pool_frac`` of the
    full-KV demand (every request's ceil(c/P) pages, a shared prefix counted once); each
    request's allocation is scaled to A = max(prefix_pages, floor(alloc_frac * c / P)), so
    the free stack starts nearly empty and compactions that reach into a shared prefix
    need copy-on-write pages the stack may not have (``free_pages`` instead sets the
    stack's size directly).  Every request is at its boundary.
    Members of a group share their summary directions (same prompt); prefix keys carry
    the Zipf profile of the group's first request."""
    rng = np.random.default_rng(seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    G = Hq // Hkv
    c = np.exp(rng.uniform(math.log(ctx[0]), math.log(ctx[1]), size=B))
    n_groups = (B + group - 1) // group
    sizes = np.array([min(group, B - g * group) for g in range(n_groups)])
    demand = int(np.ceil(c / P).sum()) - int(((sizes - 1) * prefix_pages).sum())
    num_pages = int(pool_frac * demand)
    A = np.maximum(prefix_pages, np.floor(alloc_frac * c / P)).astype(np.int64)
    n = (A + 1) * P
    used = int((A + 1).sum()) - int(((sizes - 1) * prefix_pages).sum())
    if free_pages is not None:
        num_pages = used + int(free_pages)
    assert used <= num_pages, "pool too small for the drawn contexts"
    s_zipf = rng.uniform(s_range[0], s_range[1], size=B)
    pos = (n + rng.integers(0, 64, size=B)).astype(np.int64)
    regime = np.zeros(B, np.int32)
    regime[rng.choice(B, size=int(round(grow_frac * B)), replace=False)] = 1
    max_pages = int(A.max()) + 8
    perm = rng.permutation(num_pages)
    table = np.full((B, max_pages), -1, np.int32)
    refcount = np.zeros(num_pages, np.int32)
    cur = 0
    for g in range(n_groups):
        pre = perm[cur: cur + prefix_pages]
        cur += prefix_pages
        refcount[pre] = sizes[g]
        for b in range(g * group, g * group + sizes[g]):
            table[b, :prefix_pages] = pre
            k = int(A[b]) + 1 - prefix_pages
            table[b, prefix_pages: A[b] + 1] = perm[cur: cur + k]
            refcount[perm[cur: cur + k]] = 1
            cur += k
    free = perm[cur:]
    stack = np.zeros(num_pages, np.int32)
    stack[: len(free)] = free

    cos_np, sin_np = SW.rope_tables(int(pos.max()) + 1, d)
    cos = torch.from_numpy(cos_np).to(device)
    sin = torch.from_numpy(sin_np).to(device)
    u = torch.randn((n_groups, L, Hq, d), generator=gen, device=device, dtype=torch.float64)
    u = u / u.norm(dim=-1, keepdim=True)
    ug = u[torch.from_numpy(np.arange(B) // group).to(device)]                       # [B][L][Hq][d]
    reg = torch.from_numpy(regime).to(device).bool()[:, None, None]
    U = lambda lo, hi: lo + (hi - lo) * torch.rand((B, L, Hq), generator=gen, device=device, dtype=torch.float64)
    bs = torch.where(reg, U(0.2, 0.8), U(2.0, 5.0))
    bl = torch.where(reg, U(1.5, 3.0), U(0.5, 1.5))
    sum_s = (bs[..., None] * ug + 0.1 * torch.randn((B, L, Hq, d), generator=gen, device=device, dtype=torch.float64)).float()
    sum_l = (bl[..., None] * ug + 0.1 * torch.randn((B, L, Hq, d), generator=gen, device=device, dtype=torch.float64)).float()

    k_pool, v_pool, mem = pool_pair(L, num_pages, Hkv, P, d, "layer_major", device, contiguous)
    for l in range(L):
        k_pool[l].normal_(generator=gen)
        v_pool[l].normal_(generator=gen)
    pre_len = prefix_pages * P

    def plant(b, lo, hi):
        """Keys of slots [lo, hi) of request b: N(0, I) plus b's Zipf profile."""
        nb = int(n[b])
        scale = float(s_zipf[b]) * math.sqrt(d) / 2.0
        dirs = _rotate(ug[b], cos[pos[b]].double(), sin[pos[b]].double()).float()   # [L][Hq][d]
        k = torch.randn((L, Hkv, hi - lo, d), generator=gen, device=device, dtype=torch.float32)
        for j in range(G):
            rank = torch.argsort(torch.rand((L, Hkv, nb), generator=gen, device=device), dim=-1)
            rank = rank[..., lo:hi].float() + 1.0
            mu = scale * (math.log(nb) - torch.log(rank))
            k += mu[..., None] * dirs[:, j::G][:, :, None, :]
        pages = torch.from_numpy(table[b, lo // P: hi // P].astype(np.int64)).to(device)
        k_pool[:, pages] = k.to(torch.bfloat16).view(L, Hkv, (hi - lo) // P, P, d).permute(0, 2, 1, 3, 4)

    for g in range(n_groups):
        plant(g * group, 0, pre_len)
    for b in range(B):
        plant(b, pre_len, int(n[b]))
    st = DeviceState(L=L, Hq=Hq, Hkv=Hkv, d=d, P=P, num_pages=num_pages, dtype=Bd.GP_BF16,
                     k_pool=k_pool, v_pool=v_pool,
                     page_table=torch.from_numpy(table).to(device),
                     n_alloc=torch.from_numpy(A.astype(np.int32)).to(device),
                     fill=torch.full((B,), P, dtype=torch.int32, device=device),
                     refcount=torch.from_numpy(refcount).to(device),
                     free_stack=torch.from_numpy(stack).to(device),
                     free_top=torch.tensor([len(free)], dtype=torch.int32, device=device),
                     sum_s=sum_s.contiguous(), sum_l=sum_l.contiguous(),
                     pos=torch.from_numpy(pos.astype(np.int32)).to(device), rope_cos=cos, rope_sin=sin)
    return GpuWorkload(st, n, A, regime, pos, dict(params or SW.PARAMS_DEFAULT), seed, name, mem)


class StateBackup:
    """Device copy of everything a boundary batch mutates, to replay the same batch."""

    FIELDS = ("k_pool", "v_pool", "page_table", "n_alloc", "fill", "refcount", "free_stack", "free_top")

    def __init__(self, st: DeviceState):
        self.st = st
        self.saved = {f: getattr(st, f).clone() for f in self.FIELDS}

    def restore(self):
        for f in self.FIELDS:
            getattr(self.st, f).copy_(self.saved[f])


def to_host_workload(gw: GpuWorkload, batch_idx, page_state=None) -> SW.Workload:
    """Host (oracle) view of the requests ``batch_idx``: their rows gathered through the page
    table, their summaries and positions, and the device page state (copied as is)."""
    from .device import read_rows
    st = gw.st
    idx = list(batch_idx)
    table = st.page_table.cpu().numpy()
    k_rows, v_rows = [], []
    for b in idx:
        kr, vr = read_rows(st, table[b], int(gw.n[b]), "bf16")
        k_rows.append(kr)
        v_rows.append(vr)
    ps = page_state or dict(refcount=st.refcount.cpu().numpy(), free_stack=st.free_stack.cpu().numpy(),
                            free_top=int(st.free_top.item()))
    return SW.Workload(gw.name, st.L, st.Hq, st.Hkv, st.d, st.P, "bf16", st.num_pages, table.shape[1],
                       table[idx].copy(), st.n_alloc.cpu().numpy()[idx].copy(),
                       st.fill.cpu().numpy()[idx].copy(), gw.pos[idx].astype(np.int32), ps["refcount"].copy(),
                       ps["free_stack"].copy(), int(ps["free_top"]), k_rows, v_rows,
                       st.sum_s.cpu().numpy()[idx], st.sum_l.cpu().numpy()[idx], None, "f32",
                       st.rope_cos.cpu().numpy(), st.rope_sin.cpu().numpy(), dict(gw.params), gw.seed,
                       regime=gw.regime[idx].copy())

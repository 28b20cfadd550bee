"""Place a synthetic workload in device memory (torch) and read pages back.

Input plumbing only: rows are scattered into pool pages through the page table and the
page state is copied as is.  Nothing here computes an output of the engine.
"""
from __future__ import annotations

import numpy as np
import torch

from demand_paged_kv_amd import binding as B
from demand_paged_kv_amd.engine import DeviceState

from .workloads import Workload


def torch_rows(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Stored rows (float32 or bf16 bit patterns) as a CPU torch tensor of the storage dtype."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))


def numpy_rows(t: torch.Tensor, dtype: str) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def upload(wl: Workload, device="cuda", max_req: int | None = None, slots=None,
           sum_s: np.ndarray | None = None, sum_l: np.ndarray | None = None) -> DeviceState:
    """Device state for ``wl``; batch entry b lives in request slot ``slots[b]``."""
    B_ = wl.B
    slots = np.arange(B_) if slots is None else np.asarray(slots)
    max_req = int(max_req or (slots.max() + 1))
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    k_pool = torch.zeros((wl.L, wl.num_pages, wl.Hkv, wl.P, wl.d), dtype=tdt, device=device)
    v_pool = torch.zeros_like(k_pool)
    for b in range(B_):
        n = wl.n(b)
        npg = int(wl.n_alloc[b]) + 1
        pages = torch.as_tensor(wl.page_table[b, :npg].astype(np.int64), device=device)
        for rows, pool in ((wl.k_rows[b], k_pool), (wl.v_rows[b], v_pool)):
            t = torch_rows(rows, wl.dtype).to(device)                 # [L][Hkv][n][d]
            full = torch.zeros((wl.L, wl.Hkv, npg * wl.P, wl.d), dtype=tdt, device=device)
            full[:, :, :n] = t
            full = full.view(wl.L, wl.Hkv, npg, wl.P, wl.d).permute(0, 2, 1, 3, 4)
            pool[:, pages] = full
    table = torch.full((max_req, wl.max_pages), -1, dtype=torch.int32)
    n_alloc = torch.zeros(max_req, dtype=torch.int32)
    fill = torch.zeros(max_req, dtype=torch.int32)
    pos = torch.zeros(max_req, dtype=torch.int32)
    ss = torch.zeros((max_req, wl.L, wl.Hq, wl.d), dtype=torch.float32)
    sl = torch.zeros_like(ss)
    s_src = wl.sum_s if sum_s is None else sum_s
    l_src = wl.sum_l if sum_l is None else sum_l
    for b in range(B_):
        r = int(slots[b])
        table[r] = torch.from_numpy(wl.page_table[b].astype(np.int32))
        n_alloc[r] = int(wl.n_alloc[b])
        fill[r] = int(wl.fill[b])
        pos[r] = int(wl.pos[b])
        if s_src is not None:
            ss[r] = torch.from_numpy(np.asarray(s_src[b], np.float32))
            sl[r] = torch.from_numpy(np.asarray(l_src[b], np.float32))
    cos = sin = None
    if wl.rope_cos is not None:
        cos = torch.from_numpy(wl.rope_cos).to(device)
        sin = torch.from_numpy(wl.rope_sin).to(device)
    return DeviceState(
        L=wl.L, Hq=wl.Hq, Hkv=wl.Hkv, d=wl.d, P=wl.P, num_pages=wl.num_pages,
        dtype=B.GP_BF16 if wl.dtype == "bf16" else B.GP_F32,
        k_pool=k_pool, v_pool=v_pool, page_table=table.to(device), n_alloc=n_alloc.to(device),
        fill=fill.to(device), refcount=torch.from_numpy(wl.refcount.astype(np.int32)).to(device),
        free_stack=torch.from_numpy(wl.free_stack.astype(np.int32)).to(device),
        free_top=torch.tensor([wl.free_top], dtype=torch.int32, device=device),
        sum_s=ss.to(device), sum_l=sl.to(device), pos=pos.to(device), rope_cos=cos, rope_sin=sin)


def read_rows(st: DeviceState, page_ids: np.ndarray, n: int, dtype: str):
    """Rows of slots [0, n) stored in ``page_ids`` (in order): K, V as [L][Hkv][n][d]."""
    npg = (n + st.P - 1) // st.P
    idx = torch.as_tensor(np.asarray(page_ids[:npg], np.int64), device=st.k_pool.device)
    out = []
    for pool in (st.k_pool, st.v_pool):
        t = pool[:, idx].permute(0, 2, 1, 3, 4).reshape(st.L, st.Hkv, npg * st.P, st.d)[:, :, :n]
        out.append(numpy_rows(t, dtype))
    return out[0], out[1]


def read_page(st: DeviceState, page: int, dtype: str):
    """Whole page (all layers and heads): K, V as [L][Hkv][P][d]."""
    return numpy_rows(st.k_pool[:, page], dtype), numpy_rows(st.v_pool[:, page], dtype)

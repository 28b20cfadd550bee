"""Decode-loop runs on the GPU beside the oracle (helpers for the decode-loop tests)."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from synth import device as SD


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host)."""
    return SD.numpy_rows(t, "bf16")


def oracle_state(st, req: np.ndarray, sum_s=None, sum_l=None) -> O.LoopState:
    """Oracle view of device requests ``req`` read back right after generation: rows through
    the page table, page state copied as is (pool-wide state only when req covers it)."""
    table = st.page_table.cpu().numpy()[req].copy()
    n_alloc = st.n_alloc.cpu().numpy()[req].astype(np.int64)
    fill = st.fill.cpu().numpy()[req].astype(np.int64)
    k_rows, v_rows = [], []
    for i, r in enumerate(req):
        n = int(n_alloc[i]) * st.P + int(fill[i])
        kr, vr = SD.read_rows(st, table[i], n, "bf16")
        k_rows.append(kr)
        v_rows.append(vr)
    ss = st.sum_s.cpu().numpy()[req] if sum_s is None else sum_s
    sl = st.sum_l.cpu().numpy()[req] if sum_l is None else sum_l
    return O.LoopState(st.L, st.Hq, st.Hkv, st.d, st.P, "bf16", st.num_pages, table, n_alloc, fill,
                       st.refcount.cpu().numpy().astype(np.int64), st.free_stack.cpu().numpy().astype(np.int64),
                       int(st.free_top.item()), k_rows, v_rows, ss.copy(), sl.copy(),
                       st.pos.cpu().numpy()[req].astype(np.int64), st.rope_cos.cpu().numpy(),
                       st.rope_sin.cpu().numpy())

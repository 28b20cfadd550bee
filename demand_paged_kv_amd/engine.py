"""Device state and one boundary batch through the C ABI.

PyTorch is used for device memory and the stream only; every step of the boundary
path (scan, working sets, decision, grow, keep-set, copy-on-write, compaction) runs in
the HIP kernels of libgrowpage.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import binding as B


@dataclasses.dataclass
class DeviceState:
    """Caller-owned device memory the library works on."""
    L: int
    Hq: int
    Hkv: int
    d: int
    P: int
    num_pages: int
    dtype: int                  # binding.GP_F32 / GP_BF16
    k_pool: torch.Tensor        # [L][num_pages][Hkv][P][d]
    v_pool: torch.Tensor
    page_table: torch.Tensor    # [max_req][max_pages] int32
    n_alloc: torch.Tensor       # [max_req] int32
    fill: torch.Tensor          # [max_req] int32
    refcount: torch.Tensor      # [num_pages] int32
    free_stack: torch.Tensor    # [num_pages] int32
    free_top: torch.Tensor      # [1] int32
    sum_s: torch.Tensor         # [max_req][L][Hq][d] float32
    sum_l: torch.Tensor
    pos: torch.Tensor           # [max_req] int32
    rope_cos: Optional[torch.Tensor] = None   # [max_pos][d/2] float32
    rope_sin: Optional[torch.Tensor] = None

    def kv(self) -> B.KV:
        """The pools as [L][num_pages][Hkv][P][d] views (any strides, d contiguous)."""
        k, v = self.k_pool, self.v_pool
        assert k.shape == v.shape and k.stride() == v.stride() and k.stride(4) == 1
        return B.make_kv(k, v, self.L, self.Hq, self.Hkv, self.d, self.P, self.num_pages, self.dtype,
                         strides=k.stride()[:4])

    def pages(self) -> B.Pages:
        return B.make_pages(self.page_table, self.n_alloc, self.fill, self.refcount,
                            self.free_stack, self.free_top)


@dataclasses.dataclass
class StepOutputs:
    ws: torch.Tensor          # [n][L][Hq][2] int32
    stats: torch.Tensor       # [n][L][Hq][2][2] float32 (max logit, sum exp)
    decision: torch.Tensor    # [n] uint8
    delta: torch.Tensor       # [n] int32
    status: torch.Tensor      # [n] int32
    evicted: torch.Tensor     # [n][L][Hkv][P] int32 ([..][2P] under the SHRINK policy)
    counters: torch.Tensor    # [GP_NUM_COUNTERS] int32


class BoundaryEngine:
    """Runs scan -> decide -> compact for batches of requests on one device state.

    Output and scratch buffers are allocated once for a maximum batch and token count
    and reused, so a step launches kernels only.
    """

    def __init__(self, st: DeviceState, max_batch: int, max_total_tokens: int, prm: B.Params):
        self.st = st
        self.prm = prm
        self.max_total_tokens = int(max_total_tokens)
        self.kv = st.kv()
        self.pages = st.pages()
        dev = st.k_pool.device
        self.scratch_nbytes = B.scratch_bytes(self.kv, max_batch, self.max_total_tokens)
        self.scratch = torch.empty(self.scratch_nbytes, dtype=torch.uint8, device=dev)
        n = max_batch
        self.out = StepOutputs(
            ws=torch.empty((n, st.L, st.Hq, 2), dtype=torch.int32, device=dev),
            stats=torch.empty((n, st.L, st.Hq, 2, 2), dtype=torch.float32, device=dev),
            decision=torch.empty(n, dtype=torch.uint8, device=dev),
            delta=torch.empty(n, dtype=torch.int32, device=dev),
            status=torch.empty(n, dtype=torch.int32, device=dev),
            evicted=torch.empty(0, dtype=torch.int32, device=dev),
            counters=torch.zeros(B.GP_NUM_COUNTERS, dtype=torch.int32, device=dev),
        )
        self.max_batch = n
        self._ev_store = torch.empty(n * st.L * st.Hkv * 2 * st.P, dtype=torch.int32, device=dev)
        self.policy, self.rand_u, self.grow_prob = ("shrink" if prm.shrink else "growpage"), None, 0.0
        self._view_evicted()

    def _view_evicted(self):
        """Evicted-slot rows are P wide, 2P under SHRINK (gp_compact's evicted_out)."""
        st, n = self.st, self.max_batch
        E = (2 if self.prm.shrink else 1) * st.P
        self.out.evicted = self._ev_store[: n * st.L * st.Hkv * E].view(n, st.L, st.Hkv, E)

    def scan(self, req_ids: torch.Tensor, stream=None):
        st, o, nb = self.st, self.out, int(req_ids.numel())
        max_pos = 0 if st.rope_cos is None else int(st.rope_cos.shape[0])
        B.boundary_scan(self.kv, self.pages, req_ids, nb, st.sum_s, st.sum_l, st.rope_cos,
                        st.rope_sin, max_pos, st.pos if st.rope_cos is not None else None, self.prm,
                        o.ws, o.stats, self.scratch, self.scratch_nbytes, self.max_total_tokens,
                        stream)

    def decide(self, req_ids: torch.Tensor, stream=None):
        st, o, nb = self.st, self.out, int(req_ids.numel())
        if self.policy == "growpage":
            B.decide(o.ws, req_ids, nb, st.L, st.Hq, st.P, self.prm, self.pages, o.decision, o.delta,
                     o.status, o.counters, stream)
        else:
            B.decide_policy(o.ws, req_ids, nb, st.L, st.Hq, st.P, self.prm, self.policy, self.rand_u,
                            self.grow_prob, self.pages, o.decision, o.delta, o.status, o.counters,
                            stream)

    def set_policy(self, policy: str = "growpage", rand_u: Optional[torch.Tensor] = None,
                   grow_prob: float = 0.0):
        """Decision policy of later decide() calls; rand_u: [batch] float32 uniform draws
        (device), read at the time of each decide() (policy "random" only)."""
        assert policy in B.POLICIES
        assert policy != "random" or (rand_u is not None and rand_u.dtype == torch.float32)
        self.policy, self.rand_u, self.grow_prob = policy, rand_u, float(grow_prob)
        self.prm.shrink = 1 if policy == "shrink" else 0  # the scan sizes keep-sets by it
        self._view_evicted()

    def compact(self, req_ids: torch.Tensor, stream=None):
        o, nb = self.out, int(req_ids.numel())
        B.compact(self.kv, self.pages, req_ids, o.decision, nb, self.prm, o.evicted, o.status,
                  o.counters, self.scratch, self.scratch_nbytes, self.max_total_tokens, stream)

    def compact_prepare(self, req_ids: torch.Tensor, stream=None):
        o, nb = self.out, int(req_ids.numel())
        B.compact_prepare(self.kv, self.pages, req_ids, o.decision, nb, self.prm, o.evicted, o.status,
                          self.scratch, self.scratch_nbytes, self.max_total_tokens, stream)

    def compact_move(self, req_ids: torch.Tensor, stream=None):
        nb = int(req_ids.numel())
        B.compact_move(self.kv, self.pages, req_ids, nb, self.out.counters, self.scratch,
                       self.scratch_nbytes, self.max_total_tokens, stream)

    def step(self, req_ids: torch.Tensor, stream=None) -> StepOutputs:
        """One boundary batch: scan, decide (+grow), compact.  Asynchronous."""
        assert req_ids.dtype == torch.int32 and req_ids.is_cuda
        assert int(req_ids.numel()) <= self.max_batch
        self.scan(req_ids, stream)
        self.decide(req_ids, stream)
        self.compact(req_ids, stream)
        return self.out

    def update_summaries(self, q: torch.Tensor, req_ids: torch.Tensor, stream=None):
        """q: [n][L][Hq][d] float32 or bfloat16 (d contiguous)."""
        st = self.st
        qd = B.GP_BF16 if q.dtype == torch.bfloat16 else B.GP_F32
        B.update_summaries(q, qd, (q.stride(0), q.stride(1), q.stride(2)), req_ids,
                           int(req_ids.numel()), st.L, st.Hq, st.d, st.sum_s, st.sum_l, self.prm,
                           stream)

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor, req_ids: torch.Tensor,
               status_out: Optional[torch.Tensor] = None, stream=None):
        """k_new, v_new: [n][L][Hkv][d] of the pool dtype, contiguous."""
        assert k_new.is_contiguous() and v_new.is_contiguous()
        B.append_kv(self.kv, self.pages, k_new, v_new, req_ids, int(req_ids.numel()), status_out,
                    stream)

    def decode_attention(self, q: torch.Tensor, req_ids: torch.Tensor, out: torch.Tensor, stream=None):
        """out[b][l][h] = attention of q[b][l][h] (pre-RoPE, rotated to st.pos) over the
        request's retained slots; q [n][L][Hq][d] bf16/float32, out float32 contiguous."""
        st = self.st
        qd = B.GP_BF16 if q.dtype == torch.bfloat16 else B.GP_F32
        max_pos = 0 if st.rope_cos is None else int(st.rope_cos.shape[0])
        assert out.dtype == torch.float32 and out.is_contiguous()
        B.decode_attention(self.kv, self.pages, q, qd, (q.stride(0), q.stride(1), q.stride(2)), req_ids,
                           int(req_ids.numel()), st.rope_cos, st.rope_sin, max_pos,
                           st.pos if st.rope_cos is not None else None, out, stream)

    def decode_step(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                    req_ids: torch.Tensor, boundary_ids: Optional[torch.Tensor] = None,
                    stream=None) -> Optional[StepOutputs]:
        """One decode step: summaries absorb q, the step's K/V row is appended, then the
        entries in ``boundary_ids`` (those whose write page just filled) run one boundary
        batch.  The caller keeps ``st.pos`` at the step's absolute position."""
        self.update_summaries(q, req_ids, stream)
        self.append(k_new, v_new, req_ids, None, stream)
        if boundary_ids is None or boundary_ids.numel() == 0:
            return None
        return self.step(boundary_ids, stream)


class DecodeGraph:
    """A decode step of an engine as HIP graphs, replayed with one launch each: ``plain``
    (summaries absorb q, the K/V row is appended) and ``boundary`` (the same, then one
    boundary batch over the requests in ``bids``).  Inputs are read from the static
    buffers ``q``, ``k``, ``v`` and ``bids`` that the caller fills before each replay;
    outputs land in the engine's buffers exactly as with eager calls.  The captured
    kernels allocate nothing and synchronize nothing; capturing runs no kernel, so the
    state is untouched until the first replay."""

    def __init__(self, eng: "BoundaryEngine", req_ids: torch.Tensor, n_boundary: int,
                 q_dtype=torch.bfloat16):
        st = eng.st
        dev = st.k_pool.device
        n = int(req_ids.numel())
        assert 0 < n_boundary <= eng.max_batch
        kv_dtype = torch.bfloat16 if st.dtype == B.GP_BF16 else torch.float32
        self.eng, self.req = eng, req_ids
        self.q = torch.zeros((n, st.L, st.Hq, st.d), dtype=q_dtype, device=dev)
        self.k = torch.zeros((n, st.L, st.Hkv, st.d), dtype=kv_dtype, device=dev)
        self.v = torch.zeros_like(self.k)
        self.bids = torch.zeros(n_boundary, dtype=torch.int32, device=dev)
        self.plain = torch.cuda.CUDAGraph()
        self.boundary = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.plain):
            eng.update_summaries(self.q, req_ids)
            eng.append(self.k, self.v, req_ids)
        with torch.cuda.graph(self.boundary):
            eng.update_summaries(self.q, req_ids)
            eng.append(self.k, self.v, req_ids)
            eng.step(self.bids)

    def replay(self, boundary: bool) -> Optional[StepOutputs]:
        """One decode step from the static buffers; returns the engine's outputs after a
        boundary batch, None otherwise."""
        (self.boundary if boundary else self.plain).replay()
        return self.eng.out if boundary else None

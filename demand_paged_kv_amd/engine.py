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


def _as_stream(stream):
    """``stream`` as a torch stream object (None: the current stream)."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream) if stream else torch.cuda.default_stream()
    return stream


class BoundaryEngine:
    """Runs scan -> decide -> compact for batches of requests on one device state.

    Output and scratch buffers are allocated once for a maximum batch and token count
    and reused, so a step launches kernels only.

    Lifetimes.  Every call is asynchronous: the kernels read and write the tensors they
    are given after the call has returned.  When a method runs on a ``stream`` other
    than the current one, it marks every tensor of the launch -- the caller's (request
    ids, queries, rows, outputs, draws) and the engine's and state's own -- as used on
    that stream (``Tensor.record_stream``), so torch's caching allocator does not hand
    their memory to other work before that stream's queued work is done, even if Python
    drops them right after the call.  On the current stream the allocator's own stream
    order gives the same guarantee.
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

    def _tie(self, stream, *tensors):
        """Mark the launch's tensors (plus the engine's and the state's) as used on a
        stream other than the current one (see the class docstring)."""
        if stream is None:
            return
        s = _as_stream(stream)
        if s == torch.cuda.current_stream():
            return
        st, o = self.st, self.out
        own = (st.k_pool, st.v_pool, st.page_table, st.n_alloc, st.fill, st.refcount, st.free_stack,
               st.free_top, st.sum_s, st.sum_l, st.pos, st.rope_cos, st.rope_sin, self.scratch, o.ws,
               o.stats, o.decision, o.delta, o.status, o.counters, self._ev_store, self.rand_u)
        for t in own + tensors:
            if t is not None and t.is_cuda:
                t.record_stream(s)

    def _ids(self, req_ids: torch.Tensor) -> int:
        """Host-side check of a request-id tensor (the kernels index the page table with
        its entries unchecked): int32, contiguous, on the state's device, at most the
        engine's batch.  Returns its length."""
        dev = self.st.k_pool.device
        if not (isinstance(req_ids, torch.Tensor) and req_ids.dtype == torch.int32 and req_ids.dim() == 1
                and req_ids.is_contiguous() and req_ids.device == dev):
            raise ValueError(f"request ids must be a contiguous 1-D int32 tensor on {dev}")
        nb = int(req_ids.numel())
        if nb > self.max_batch:
            raise ValueError(f"batch of {nb} requests exceeds the engine's maximum of {self.max_batch}")
        return nb

    def _rows(self, x: torch.Tensor, nb: int, heads: int, what: str):
        """Host-side shape and device check of a per-request [n][L][heads][d] tensor."""
        st = self.st
        if tuple(x.shape) != (nb, st.L, heads, st.d) or x.device != st.k_pool.device or x.stride(3) != 1:
            raise ValueError(f"{what} must be [{nb}][{st.L}][{heads}][{st.d}] with d contiguous on "
                             f"{st.k_pool.device}, got {tuple(x.shape)}")

    @staticmethod
    def _qdtype(q: torch.Tensor) -> int:
        if q.dtype == torch.bfloat16:
            return B.GP_BF16
        if q.dtype == torch.float32:
            return B.GP_F32
        raise ValueError(f"queries must be bfloat16 or float32, got {q.dtype}")

    def _view_evicted(self):
        """Evicted-slot rows are P wide, 2P under SHRINK (gp_compact's evicted_out)."""
        st, n = self.st, self.max_batch
        E = (2 if self.prm.shrink else 1) * st.P
        self.out.evicted = self._ev_store[: n * st.L * st.Hkv * E].view(n, st.L, st.Hkv, E)

    def scan(self, req_ids: torch.Tensor, stream=None):
        st, o, nb = self.st, self.out, self._ids(req_ids)
        max_pos = 0 if st.rope_cos is None else int(st.rope_cos.shape[0])
        B.boundary_scan(self.kv, self.pages, req_ids, nb, st.sum_s, st.sum_l, st.rope_cos,
                        st.rope_sin, max_pos, st.pos if st.rope_cos is not None else None, self.prm,
                        o.ws, o.stats, self.scratch, self.scratch_nbytes, self.max_total_tokens,
                        stream)
        self._tie(stream, req_ids)
        self._scan_batch = nb

    def scan_logits(self, entry: int, n: int, stream=None) -> torch.Tensor:
        """The last scan's logits of batch entry ``entry`` (n candidate slots) as a new
        [L][Hkv][n][8] float32 tensor, row 2*j + s = query head G*g + min(j, G-1) of KV head g
        (G = Hq / Hkv), summary s."""
        st = self.st
        out = torch.empty((st.L, st.Hkv, int(n), 8), dtype=torch.float32, device=st.k_pool.device)
        B.scan_logits(self.kv, self._scan_batch, self.max_total_tokens, self.scratch, self.scratch_nbytes,
                      int(entry), int(n), out, stream)
        self._tie(stream, out)
        return out

    def decide(self, req_ids: torch.Tensor, stream=None):
        st, o, nb = self.st, self.out, self._ids(req_ids)
        if self.policy == "growpage":
            B.decide(o.ws, req_ids, nb, st.L, st.Hq, st.P, self.prm, self.pages, o.decision, o.delta,
                     o.status, o.counters, stream)
        else:
            B.decide_policy(o.ws, req_ids, nb, st.L, st.Hq, st.P, self.prm, self.policy, self.rand_u,
                            self.grow_prob, self.pages, o.decision, o.delta, o.status, o.counters,
                            stream)
        self._tie(stream, req_ids)

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
        o, nb = self.out, self._ids(req_ids)
        B.compact(self.kv, self.pages, req_ids, o.decision, nb, self.prm, o.evicted, o.status,
                  o.counters, self.scratch, self.scratch_nbytes, self.max_total_tokens, stream)
        self._tie(stream, req_ids)

    def compact_prepare(self, req_ids: torch.Tensor, stream=None):
        o, nb = self.out, self._ids(req_ids)
        B.compact_prepare(self.kv, self.pages, req_ids, o.decision, nb, self.prm, o.evicted, o.status,
                          self.scratch, self.scratch_nbytes, self.max_total_tokens, stream)
        self._tie(stream, req_ids)

    def compact_move(self, req_ids: torch.Tensor, stream=None):
        nb = self._ids(req_ids)
        B.compact_move(self.kv, self.pages, req_ids, nb, self.out.counters, self.scratch,
                       self.scratch_nbytes, self.max_total_tokens, stream)
        self._tie(stream, req_ids)

    def step(self, req_ids: torch.Tensor, stream=None) -> StepOutputs:
        """One boundary batch: scan, decide (+grow), compact.  Asynchronous."""
        self._ids(req_ids)
        self.scan(req_ids, stream)
        self.decide(req_ids, stream)
        self.compact(req_ids, stream)
        return self.out

    def update_summaries(self, q: torch.Tensor, req_ids: torch.Tensor, stream=None):
        """q: [n][L][Hq][d] float32 or bfloat16 (d contiguous)."""
        st = self.st
        nb = self._ids(req_ids)
        self._rows(q, nb, st.Hq, "q")
        qd = self._qdtype(q)
        B.update_summaries(q, qd, (q.stride(0), q.stride(1), q.stride(2)), req_ids,
                           nb, st.L, st.Hq, st.d, st.sum_s, st.sum_l, self.prm,
                           stream)
        self._tie(stream, q, req_ids)

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor, req_ids: torch.Tensor,
               status_out: Optional[torch.Tensor] = None, stream=None):
        """k_new, v_new: [n][L][Hkv][d] of the pool dtype, contiguous."""
        nb = self._ids(req_ids)
        for x, what in ((k_new, "k_new"), (v_new, "v_new")):
            self._rows(x, nb, self.st.Hkv, what)
            if not x.is_contiguous() or x.dtype != self.st.k_pool.dtype:
                raise ValueError(f"{what} must be contiguous and of the pool's dtype {self.st.k_pool.dtype}")
        B.append_kv(self.kv, self.pages, k_new, v_new, req_ids, nb, status_out,
                    stream)
        self._tie(stream, k_new, v_new, req_ids, status_out)

    def decode_attention(self, q: torch.Tensor, req_ids: torch.Tensor, out: torch.Tensor, stream=None):
        """out[b][l][h] = attention of q[b][l][h] (pre-RoPE, rotated to st.pos) over the
        request's retained slots; q [n][L][Hq][d] bf16/float32, out float32 contiguous."""
        st = self.st
        nb = self._ids(req_ids)
        self._rows(q, nb, st.Hq, "q")
        qd = self._qdtype(q)
        max_pos = 0 if st.rope_cos is None else int(st.rope_cos.shape[0])
        if out.dtype != torch.float32 or not out.is_contiguous() or out.shape[0] < nb:
            raise ValueError("out must be a contiguous float32 [n][L][Hq][d] tensor")
        self._rows(out[:nb], nb, st.Hq, "out")
        B.decode_attention(self.kv, self.pages, q, qd, (q.stride(0), q.stride(1), q.stride(2)), req_ids,
                           nb, st.rope_cos, st.rope_sin, max_pos,
                           st.pos if st.rope_cos is not None else None, out, stream)
        self._tie(stream, q, req_ids, out)

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


class OverlapSchedule:
    """A decode step with the boundary batch on a second stream, beside the other requests'
    decode attention (the background compression the pages keep from Zipage: GrowPage
    review, FAQ "How does GrowPage differ from Zipage?").

    Per step, on the current stream: the summaries absorb q and the K/V rows are appended
    for every request (after the previous step's boundary batch has finished); then the
    attention of the requests at a boundary (``bids``) runs first, over their pages as
    they stand; the boundary batch of those requests is queued on the side stream, and
    the attention of the other requests (``oids``) runs on the current stream at the same
    time.  Requests at a boundary and the others touch disjoint pages (a shared page is
    never changed in place), so the two streams do not race; the next step waits for the
    side stream.  Attention outputs go to ``out`` in the order (bids, oids): row i holds
    request ``order[i]``.  The result equals the serial schedule's (attention of every
    request, then the boundary batch) bit for bit.  Request-id tensors may be
    temporaries: the engine ties every tensor it launches on the side stream to it."""

    def __init__(self, eng: "BoundaryEngine", side: Optional[torch.cuda.Stream] = None):
        self.eng = eng
        self.side = side if side is not None else torch.cuda.Stream()
        self.done = torch.cuda.Event()
        self.pending = False

    def step(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, req_ids: torch.Tensor,
             bids: torch.Tensor, oids: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
        """One decode step (see the class docstring); ``q``, ``k_new``, ``v_new`` are
        indexed like ``req_ids`` (request slot == batch position); returns ``order``."""
        eng = self.eng
        main = torch.cuda.current_stream()
        if self.pending:
            main.wait_event(self.done)
        eng.update_summaries(q, req_ids)
        eng.append(k_new, v_new, req_ids)
        nb = int(bids.numel())
        if nb == 0:
            eng.decode_attention(q, req_ids, out)
            self.pending = False
            return req_ids
        eng.decode_attention(q[bids.long()], bids, out[:nb])
        ready = torch.cuda.Event()
        ready.record(main)
        self.side.wait_event(ready)
        eng.step(bids, stream=self.side)
        self.done.record(self.side)
        self.pending = True
        eng.decode_attention(q[oids.long()], oids, out[nb:])
        return torch.cat([bids, oids])

    def finish(self):
        """Make the current stream wait for the last boundary batch."""
        if self.pending:
            torch.cuda.current_stream().wait_event(self.done)
            self.pending = False

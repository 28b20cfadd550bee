"""The boundary batch on a second stream beside decode attention (engine.OverlapSchedule)
against the serial schedule on a twin state, and sampled attention outputs against the
oracle.

Decode loop on the 8B head shape (32 query / 8 KV heads, d 128, bf16, page 16), 64
requests x 8 layers from 1024-token prompts, boundaries staggered so that 4 requests
reach theirs on every step; 160 serial steps first (the slow summary needs about a
hundred steps before any request grows), then the state is cloned and 96 steps run
under both schedules side by side (the background compression the pages keep from
Zipage: GrowPage review, FAQ "How does GrowPage differ from Zipage?"; the engine inside
PagedAttention serving: the abstract).  Request-id tensors are built afresh on each
step and dropped right after it, as a caller would: the engine ties what it launches on
the side stream to that stream.  After every step (both schedules synchronised) the
attention outputs and the boundary batch's outputs match bit for bit; every 16 steps and
at the end the summaries, the page state and every pool byte match."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
from synth import device as SD
from tests import decode_util as DU

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-4, 1e-4   # decode attention against float64 (tests/test_attention_gpu.py)


def _clone(st):
    return dataclasses.replace(st, **{f.name: getattr(st, f.name).clone()
                                      for f in dataclasses.fields(st)
                                      if isinstance(getattr(st, f.name), torch.Tensor)})


def _same(a, b, what, t):
    assert torch.equal(a, b), (what, t)


def test_overlap_schedule_matches_serial_and_oracle():
    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine, OverlapSchedule
    from synth.decode_loop import DecodeLoopGen, DecodeSpec

    warm = 160
    spec = DecodeSpec(B=64, L=8, steps=warm + 96, seed=4200, stagger=True)
    gen = DecodeLoopGen(spec, "cuda")
    st_s = gen.initial_state()          # serial schedule
    st_o = eng_o = sched = None         # overlapped schedule, from a clone after the warm-up
    max_tokens = spec.B * (spec.prompt + spec.steps + 2 * spec.P)
    eng_s = BoundaryEngine(st_s, spec.B, max_tokens, Bd.params_from(spec.params))
    req = torch.arange(spec.B, dtype=torch.int32, device="cuda")
    out_s = torch.empty((spec.B, spec.L, spec.Hq, spec.d), dtype=torch.float32, device="cuda")
    out_o = torch.empty_like(out_s)
    pos0 = torch.from_numpy((spec.prompt + gen.fill0).astype(np.int32)).cuda()
    fill = gen.fill0.copy()
    rng = np.random.default_rng(4201)
    boundaries = grows = checked = 0
    for t in range(spec.steps):
        q, k, v = gen.step()
        torch.add(pos0, t, out=st_s.pos)
        fill += 1
        bmask = fill == spec.P
        fill[bmask] = 0
        bids = torch.as_tensor(np.flatnonzero(bmask).astype(np.int32), device="cuda")
        oids = torch.as_tensor(np.flatnonzero(~bmask).astype(np.int32), device="cuda")
        nb = int(bids.numel())
        if t == warm:
            torch.cuda.synchronize()
            st_o = _clone(st_s)
            eng_o = BoundaryEngine(st_o, spec.B, max_tokens, Bd.params_from(spec.params))
            sched = OverlapSchedule(eng_o)
        # serial: everything on the current stream
        eng_s.update_summaries(q, req)
        eng_s.append(k, v, req)
        eng_s.decode_attention(q, req, out_s)
        if nb:
            eng_s.step(bids)
        if t < warm:
            continue
        torch.add(pos0, t, out=st_o.pos)
        # overlapped: the boundary batch on the side stream beside the other attention
        order = sched.step(q, k, v, req, bids, oids, out_o)
        sched.finish()
        torch.cuda.synchronize()
        order = order.long()
        _same(out_o.view(torch.int32), out_s[order].view(torch.int32), "attention outputs", t)
        if nb:
            boundaries += 1
            for f in ("ws", "stats", "decision", "delta", "status", "evicted", "counters"):
                a, b = getattr(eng_o.out, f), getattr(eng_s.out, f)
                if f != "counters":
                    a, b = a[:nb], b[:nb]
                _same(a, b, f, t)
            grows += int((eng_s.out.decision[:nb] == 1).sum().item())
        del bids, oids     # dropped while nothing else holds them (the side stream is done)
        if (t + 1) % 16 == 0 or t == spec.steps - 1:
            for f in ("sum_s", "sum_l"):
                _same(getattr(st_s, f).view(torch.int32), getattr(st_o, f).view(torch.int32), f, t)
            for f in ("fill", "n_alloc", "page_table", "refcount", "free_top"):
                _same(getattr(st_s, f), getattr(st_o, f), f, t)
            top = int(st_s.free_top.item())
            _same(st_s.free_stack[:top], st_o.free_stack[:top], "free stack", t)
            _same(st_s.k_pool.view(torch.int16), st_o.k_pool.view(torch.int16), "K pool", t)
            _same(st_s.v_pool.view(torch.int16), st_o.v_pool.view(torch.int16), "V pool", t)
            # oracle: attention of two requests not at a boundary this step (their pages as
            # the attention saw them), from the overlapped state
            cand = np.flatnonzero(~bmask)
            for r in rng.choice(cand, 2, replace=False):
                ost = DU.oracle_state(st_o, np.array([r]))
                p = int(pos0[r].item()) + t
                want = O.decode_attention(ost.k_rows[0], ost.v_rows[0], "bf16", DU.bits(q[r]), "bf16",
                                          ost.rope_cos[p], ost.rope_sin[p])
                got = out_o[int(np.flatnonzero(order.cpu().numpy() == r)[0])].cpu().numpy()
                err = np.abs(got - want) - (ATOL + RTOL * np.abs(want))
                assert (err <= 0).all(), (t, r, float(np.abs(got - want).max()))
                checked += 1
            print(f"[overlap] step {t}: {boundaries} boundary batches equal to the serial twin, "
                  f"grows {grows}, oracle attention checks {checked}", flush=True)
    assert boundaries == spec.steps - warm
    assert 0 < grows < boundaries * 4, "both decisions should occur"

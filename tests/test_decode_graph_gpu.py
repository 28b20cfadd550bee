"""The decode step replayed from HIP graphs (engine.DecodeGraph) matches eager calls on a
twin state, step by step: 256 steps (16 boundary batches) with the generator's eager work and
a synchronization between replays; summaries bit-exact, page state, outputs and every pool
byte equal after each step."""
import dataclasses

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _clone(st):
    return dataclasses.replace(st, **{f.name: getattr(st, f.name).clone()
                                      for f in dataclasses.fields(st)
                                      if isinstance(getattr(st, f.name), torch.Tensor)})


def _same(a, b, what, t):
    assert torch.equal(a, b), (what, t)


def test_decode_graph_replays_match_eager():
    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine, DecodeGraph
    from synth.decode_loop import DecodeLoopGen, DecodeSpec

    spec = DecodeSpec(B=8, L=4, steps=256, seed=4000)
    gen = DecodeLoopGen(spec, "cuda")
    st_e = gen.initial_state()
    st_g = _clone(st_e)
    max_tokens = spec.B * (spec.prompt + spec.steps + spec.P)
    eng_e = BoundaryEngine(st_e, spec.B, max_tokens, Bd.params_from(spec.params))
    eng_g = BoundaryEngine(st_g, spec.B, max_tokens, Bd.params_from(spec.params))
    req = torch.arange(spec.B, dtype=torch.int32, device="cuda")
    graph = DecodeGraph(eng_g, req, spec.B)
    graph.bids.copy_(req)
    torch.cuda.synchronize()
    _same(st_e.k_pool, st_g.k_pool, "capture left the pools untouched", -1)
    fill = boundaries = grows = 0
    for t in range(spec.steps):
        q, k, v = gen.step()
        st_e.pos.fill_(spec.prompt + t)
        st_g.pos.fill_(spec.prompt + t)
        fill += 1
        boundary = fill == spec.P
        out_e = eng_e.decode_step(q, k, v, req, req if boundary else None)
        graph.q.copy_(q)
        graph.k.copy_(k)
        graph.v.copy_(v)
        out_g = graph.replay(boundary)
        torch.cuda.synchronize()
        for f in ("sum_s", "sum_l"):
            _same(getattr(st_e, f).view(torch.int32), getattr(st_g, f).view(torch.int32), f, t)
        for f in ("fill", "n_alloc", "page_table", "refcount", "free_top"):
            _same(getattr(st_e, f), getattr(st_g, f), f, t)
        top = int(st_e.free_top.item())
        _same(st_e.free_stack[:top], st_g.free_stack[:top], "free stack", t)
        if boundary:
            fill = 0
            boundaries += 1
            for f in ("ws", "stats", "decision", "delta", "status", "evicted", "counters"):
                _same(getattr(out_e, f)[: spec.B] if f != "counters" else out_e.counters,
                      getattr(out_g, f)[: spec.B] if f != "counters" else out_g.counters, f, t)
            grows += int((out_e.decision[: spec.B] == 1).sum().item())
            _same(st_e.k_pool.view(torch.int16), st_g.k_pool.view(torch.int16), "K pool", t)
            _same(st_e.v_pool.view(torch.int16), st_g.v_pool.view(torch.int16), "V pool", t)
            print(f"[graph] step {t}: boundary {boundaries} matches eager "
                  f"(decisions {out_g.decision[: spec.B].tolist()})", flush=True)
    assert boundaries == spec.steps // spec.P
    assert 0 < grows < boundaries * spec.B, "both decisions should occur"

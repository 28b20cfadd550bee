"""Decode-loop parity on the Qwen3-8B shape (36 layers, 32 query / 8 KV heads, d 128, bf16,
page 16, 1024-token prompts): every decode step updates both summaries and appends one
K/V row per request; every 16 steps all write pages fill and the batch runs a boundary.

* end to end at reduced size (4 requests x 4 layers x 512 steps): the oracle runs the
  whole loop on its own from the same generated inputs; summaries are compared bit for
  bit after every step and each of the 32 boundary batches element by element (working
  sets, statistics, decisions, keep-sets, page table, refcounts, free stack, page bytes);
* at the full batch shape (128 requests x 36 layers, 256 steps): three sampled requests are
  tracked by the oracle from their own inputs; the whole batch is checked by pool
  invariants at every boundary.

A keep-set near-tie that the GPU resolves the other way (allowed, and validated) makes
the two trajectories differ from then on; the request's comparison stops there and the
test says so.
"""
import numpy as np
import pytest
import torch

import oracle as O
from tests import decode_util as DU
from tests.parity_util import check_pool, compare_requests, compare_step, snapshot

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _engine(spec, st):
    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine
    max_tokens = spec.B * (spec.prompt + spec.steps + spec.P)
    return BoundaryEngine(st, spec.B, max_tokens, Bd.params_from(spec.params))


def _gpu_step(eng, st, spec, t, q, k, v, fill, req):
    """One GPU decode step; ``fill`` is the host's count of rows in each write page."""
    st.pos.fill_(spec.prompt + t)
    fill += 1
    bids = np.flatnonzero(fill == spec.P).astype(np.int32)
    bt = torch.as_tensor(bids, device="cuda") if bids.size else None
    out = eng.decode_step(q, k, v, req, bt)
    torch.cuda.synchronize()
    if out is not None:
        deferred = (out.status[: bids.size].cpu().numpy() & 2) != 0
        fill[bids[~deferred]] = 0
    return bids, out


@pytest.mark.parametrize("policy", ["growpage", "shrink"])
def test_decode_loop_end_to_end_reduced(policy):
    from synth.decode_loop import DecodeLoopGen, DecodeSpec
    spec = DecodeSpec(B=4, L=4, steps=512, seed=4000)
    spec.params = dict(spec.params, policy=policy)
    gen = DecodeLoopGen(spec, "cuda")
    st = gen.initial_state()
    ost = DU.oracle_state(st, np.arange(spec.B))
    eng = _engine(spec, st)
    req = torch.arange(spec.B, dtype=torch.int32, device="cuda")
    fill = np.zeros(spec.B, np.int64)
    n_local = spec.params["n_local"]
    boundaries = compared = 0
    decisions = []
    diverged_at = None
    for t in range(spec.steps):
        q, k, v = gen.step()
        bids, out = _gpu_step(eng, st, spec, t, q, k, v, fill, req)
        app, idx, sub, res = O.decode_step(ost, DU.bits(q), "bf16", DU.bits(k), DU.bits(v), spec.params)
        assert app.all()
        assert np.array_equal(st.sum_s.cpu().numpy().view(np.uint32), ost.sum_s.view(np.uint32)), t
        assert np.array_equal(st.sum_l.cpu().numpy().view(np.uint32), ost.sum_l.view(np.uint32)), t
        assert np.array_equal(idx, bids), (t, idx, bids)
        if res is None:
            continue
        boundaries += 1
        if diverged_at is None:
            rep = compare_step(sub, idx, st, out, res, n_local)
            compared += 1
            decisions.append(res.decision.copy())
            if rep.ev_near_differs:
                diverged_at = t
                _say(f"[decode] step {t}: a keep-set near-tie resolved the other way; "
                     f"page comparison stops here")
        if boundaries % 8 == 0:
            _say(f"[decode] step {t}: {boundaries} boundaries, {compared} compared")
    dec = np.concatenate(decisions)
    grows = int((dec == 1).sum())
    _say(f"[decode] {policy}: {boundaries} boundaries, {compared} compared, grows {grows} of {dec.size}")
    assert boundaries == spec.steps // spec.P
    assert compared >= boundaries // 2
    assert 0 < grows < dec.size, "both decisions should occur"
    if policy == "shrink":
        assert (dec == 2).any() and int(st.n_alloc[: spec.B].min().item()) < spec.A0


def test_decode_loop_full_shape_sampled():
    from synth.decode_loop import DecodeLoopGen, DecodeSpec
    spec = DecodeSpec(B=128, L=36, steps=256, seed=4001)
    gen = DecodeLoopGen(spec, "cuda")
    st = gen.initial_state()
    track = np.array([5, 77, 126])
    ost = DU.oracle_state(st, track)
    eng = _engine(spec, st)
    req = torch.arange(spec.B, dtype=torch.int32, device="cuda")
    fill = np.zeros(spec.B, np.int64)
    n_local = spec.params["n_local"]
    live = np.ones(track.size, bool)
    boundaries = 0
    grows = 0
    _say(f"[decode-full] generated {spec.B} requests x {spec.L} layers; tracking {track.tolist()}")
    for t in range(spec.steps):
        q, k, v = gen.step()
        before = snapshot(st) if fill[0] + 1 == spec.P else None
        bids, out = _gpu_step(eng, st, spec, t, q, k, v, fill, req)
        app, idx, sub, res = O.decode_step(ost, DU.bits(q[track]), "bf16", DU.bits(k[track]),
                                           DU.bits(v[track]), spec.params)
        assert app.all()
        s_gpu = st.sum_s[torch.as_tensor(track, device="cuda")].cpu().numpy()
        l_gpu = st.sum_l[torch.as_tensor(track, device="cuda")].cpu().numpy()
        assert np.array_equal(s_gpu.view(np.uint32), ost.sum_s.view(np.uint32)), t
        assert np.array_equal(l_gpu.view(np.uint32), ost.sum_l.view(np.uint32)), t
        if out is None:
            assert res is None
            continue
        assert bids.size == spec.B and idx.size == track.size
        boundaries += 1
        dec = out.decision[: spec.B].cpu().numpy()
        grows += int(dec.sum())
        assert not out.status[: spec.B].cpu().numpy().any()
        check_pool(st, before, dec, np.arange(spec.B))
        keep = np.flatnonzero(live)
        if keep.size == track.size:
            rep = compare_requests(sub, track, st, out, res, n_local)
        elif keep.size:
            sub_live = sub.subset(keep)
            res_live = O.boundary_step(sub_live, sub_live.sum_s, sub_live.sum_l, spec.params)
            rep = compare_requests(sub_live, track[keep], st, out, res_live, n_local)
        for i in rep.diverged if keep.size else []:
            _say(f"[decode-full] step {t}: request {track[keep[i]]} took the other side of a "
                 f"keep-set near-tie; its comparison ends here")
            live[keep[i]] = False
        _say(f"[decode-full] step {t}: boundary {boundaries}, grows so far {grows}, "
             f"tracked {int(live.sum())}")
    assert boundaries == spec.steps // spec.P
    assert live.sum() >= 2


def test_decode_loop_full_length_snapshots():
    """The whole decode loop at its full size (128 requests x 36 layers x 4096 steps, 256
    boundary batches).  The first, the last and every 16th boundary batch is checked from
    a snapshot: four requests drawn afresh for that batch are read back just before the
    step and the oracle runs the step on them alone (summary update, append, boundary),
    which works at any distance from the start because the summaries are bit-exact.  Pool
    invariants are checked at every boundary.  A request whose decision the oracle finds
    ambiguous (delta within rounding of tau) is checked for a delta inside the oracle's
    range and left out of the element-wise comparison."""
    from synth.decode_loop import DecodeLoopGen, DecodeSpec
    spec = DecodeSpec(B=128, L=36, steps=4096, seed=4000)  # bench.py --workload decode_loop's loop
    gen = DecodeLoopGen(spec, "cuda", contiguous=True)
    st = gen.initial_state()
    eng = _engine(spec, st)
    req = torch.arange(spec.B, dtype=torch.int32, device="cuda")
    fill = np.zeros(spec.B, np.int64)
    n_local = spec.params["n_local"]
    n_batches = spec.steps // spec.P
    sampled = set(range(0, n_batches, 16)) | {n_batches - 1}
    rng = np.random.default_rng(spec.seed)
    boundaries = grows = checked = 0
    _say(f"[decode-length] {spec.B} requests x {spec.L} layers x {spec.steps} steps; "
         f"snapshots at batches {sorted(sampled)}")
    for t in range(spec.steps):
        q, k, v = gen.step()
        at_boundary = fill[0] + 1 == spec.P
        snap = at_boundary and boundaries in sampled
        before = snapshot(st) if at_boundary else None
        if snap:
            track = np.sort(rng.choice(spec.B, 4, replace=False))
            ost = DU.oracle_state(st, track)
            ost.pos[:] = spec.prompt + t  # the step's position (the device's is set by the step)
        bids, out = _gpu_step(eng, st, spec, t, q, k, v, fill, req)
        if out is None:
            assert not at_boundary
            continue
        assert bids.size == spec.B
        dec = out.decision[: spec.B].cpu().numpy()
        assert not out.status[: spec.B].cpu().numpy().any()
        check_pool(st, before, dec, np.arange(spec.B))
        grows += int(dec.sum())
        if snap:
            app, idx, sub, res = O.decode_step(ost, DU.bits(q[track]), "bf16", DU.bits(k[track]),
                                               DU.bits(v[track]), spec.params)
            assert app.all() and idx.size == track.size
            s_gpu = st.sum_s[torch.as_tensor(track, device="cuda")].cpu().numpy()
            assert np.array_equal(s_gpu.view(np.uint32), ost.sum_s.view(np.uint32)), t
            keep = np.flatnonzero(~res.ambiguous)
            delta = out.delta[: spec.B].cpu().numpy()
            for i in np.flatnonzero(res.ambiguous):
                assert res.delta_lo[i] <= delta[track[i]] <= res.delta_hi[i], (t, track[i])
                _say(f"[decode-length] step {t}: request {track[i]} has an ambiguous decision")
            if keep.size == track.size:
                rep = compare_requests(sub, track, st, out, res, n_local)
            elif keep.size:
                sub_k = sub.subset(keep)
                res_k = O.boundary_step(sub_k, sub_k.sum_s, sub_k.sum_l, spec.params)
                rep = compare_requests(sub_k, track[keep], st, out, res_k, n_local)
            checked += int(keep.size)
            _say(f"[decode-length] step {t}: batch {boundaries} checked requests "
                 f"{track[keep].tolist()} (keep-set near-ties {rep.ev_near if keep.size else 0}); "
                 f"grows so far {grows}")
        boundaries += 1
    assert boundaries == n_batches
    assert checked >= len(sampled)
    assert 0 < grows < boundaries * spec.B


def test_decode_loop_paper_point_reduced():
    """The decode loop at the pages' operating point (KV block 256, p 0.99, local quota 64;
    GrowPage review, FAQ "Is GrowPage's code available?") on the Qwen3-8B head shape: 6
    requests x 2 layers from 1024-token prompts (4 pages), 1024 steps, so 4 boundary
    batches.  The oracle runs the whole loop from the same inputs; summaries are compared
    bit for bit after every step and every boundary batch element by element.  Where the
    GPU resolves a keep-set near-tie the other way (allowed and validated), the oracle's
    state is re-read from the GPU after that batch, so later batches are still compared
    from identical inputs."""
    from synth import workloads as SW
    from synth.decode_loop import DecodeLoopGen, DecodeSpec
    spec = DecodeSpec(B=6, L=2, P=256, prompt=1024, steps=1024, seed=4100, params=dict(SW.PARAMS_PAPER))
    gen = DecodeLoopGen(spec, "cuda")
    st = gen.initial_state()
    ost = DU.oracle_state(st, np.arange(spec.B))
    eng = _engine(spec, st)
    req = torch.arange(spec.B, dtype=torch.int32, device="cuda")
    fill = np.zeros(spec.B, np.int64)
    n_local = spec.params["n_local"]
    boundaries = resyncs = 0
    decisions = []
    for t in range(spec.steps):
        q, k, v = gen.step()
        bids, out = _gpu_step(eng, st, spec, t, q, k, v, fill, req)
        app, idx, sub, res = O.decode_step(ost, DU.bits(q), "bf16", DU.bits(k), DU.bits(v), spec.params)
        assert app.all()
        assert np.array_equal(st.sum_s.cpu().numpy().view(np.uint32), ost.sum_s.view(np.uint32)), t
        assert np.array_equal(st.sum_l.cpu().numpy().view(np.uint32), ost.sum_l.view(np.uint32)), t
        assert np.array_equal(idx, bids), (t, idx, bids)
        if res is None:
            continue
        boundaries += 1
        rep = compare_step(sub, idx, st, out, res, n_local)
        decisions.append(res.decision.copy())
        _say(f"[decode-p256] step {t}: boundary {boundaries}, decisions {res.decision.tolist()}, {rep}")
        if rep.ev_near_differs:
            ost = DU.oracle_state(st, np.arange(spec.B))
            ost.pos[:] = spec.prompt + t + 1
            resyncs += 1
    dec = np.concatenate(decisions)
    _say(f"[decode-p256] {boundaries} boundaries compared, {resyncs} re-reads, grows {int((dec == 1).sum())} "
         f"of {dec.size}")
    assert boundaries == spec.steps // spec.P == 4
    assert 0 < int((dec == 1).sum()) < dec.size, "both decisions should occur"

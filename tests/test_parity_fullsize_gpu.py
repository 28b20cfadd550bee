"""Full-size parity on the benchmark workload (32-layer boundary sweep on the 8B GQA
shape, generated on the GPU), in the launch configuration bench.py times: the oracle
recomputes every request of the default batch (a sample at the other operating points)
end to end -- working sets, statistics, decision, keep-sets, compacted page bytes --
and the whole batch is checked by pool invariants."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
from tests.parity_util import check_pool, compare_requests, snapshot

pytestmark = pytest.mark.gpu


def _bench_step(eng, req):
    """One boundary batch with the calls bench.py times: scan, decide, compact_prepare,
    compact_move (the split form of gp_compact)."""
    eng.scan(req)
    eng.decide(req)
    eng.compact_prepare(req)
    eng.compact_move(req)
    torch.cuda.synchronize()
    return eng.out


def _pre_step_view(gw, backup):
    """The workload as it was before the step: the same requests over the state copy."""
    pre = dataclasses.replace(gw.st, **backup.saved)
    return dataclasses.replace(gw, st=pre)


def test_boundary_sweep_full_size_all_requests():
    """All 64 requests of the benchmark batch against the oracle, in the launch
    configuration bench.py times.  The oracle runs on chunks of 8 requests read from a
    device copy of the state taken before the step (pops of new pages depend on the whole
    batch and are checked by the pool invariants); logits and probabilities are compared
    element by element on four requests (longest, shortest, a grow and a compaction)."""
    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine
    from synth import gpu_workloads as GW
    from tests.parity_util import compare_logits

    gw = GW.boundary_sweep(seed=3000, contiguous=True)  # the bench's pools
    st = gw.st
    print(f"[fullsize] generated {gw.B} requests, {gw.total_tokens()} tokens", flush=True)
    backup = GW.StateBackup(st)
    before = snapshot(st)
    eng = BoundaryEngine(st, gw.B, gw.total_tokens(), Bd.params_from(gw.params))
    req = torch.arange(gw.B, dtype=torch.int32, device="cuda")
    out = _bench_step(eng, req)
    print(f"[fullsize] step done ({gw.pool_memory} pools)", flush=True)
    dec = out.decision.cpu().numpy()
    check_pool(st, before, dec, np.arange(gw.B))
    # planted regimes come out as planted
    assert np.array_equal(dec, gw.regime.astype(np.uint8)), (dec, gw.regime)
    pre = _pre_step_view(gw, backup)
    totals = dict(ws=0, ws_near=0, ev_units=0, ev_near=0, ev_near_differs=0)
    for chunk in np.array_split(np.arange(gw.B), 8):
        chunk = [int(b) for b in chunk]
        wl = GW.to_host_workload(pre, chunk)
        res = O.boundary_step(wl, wl.sum_s, wl.sum_l, gw.params)
        rep = compare_requests(wl, chunk, st, out, res, gw.params["n_local"])
        totals["ws"] += rep.ws_total
        totals["ws_near"] += rep.ws_near
        totals["ev_units"] += rep.ev_units
        totals["ev_near"] += rep.ev_near
        totals["ev_near_differs"] += rep.ev_near_differs
        print(f"[fullsize] requests {chunk[0]}-{chunk[-1]} match: {rep}", flush=True)
    order = np.argsort(-gw.n)
    sample = sorted({int(order[0]), int(order[-1]), int(np.flatnonzero(dec == 1)[0]),
                     int(np.flatnonzero(dec == 0)[0])})
    wl = GW.to_host_workload(pre, sample)
    errs = compare_logits(eng, wl, sample, range(len(sample)))
    print("[fullsize] all", gw.B, "requests:", totals, "logit/probability errors on", sample, errs, flush=True)


def test_paper_operating_point_full_size_sampled():
    """The sweep's shape at the pages' operating point: KV block 256, p 0.99, quota 64
    (bench.py --paper's batch, pools and calls)."""
    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine
    from synth import gpu_workloads as GW
    from synth import workloads as SW

    gw = GW.boundary_sweep(seed=3100, P=256, num_pages=1536, params=dict(SW.PARAMS_PAPER), name="paper_sweep",
                           contiguous=True)
    st = gw.st
    print(f"[paper] generated {gw.B} requests, {gw.total_tokens()} tokens", flush=True)
    order = np.argsort(-gw.n)
    sample = sorted({int(order[0]), int(order[-1]), int(np.flatnonzero(gw.regime == 1)[0]),
                     int(np.flatnonzero(gw.regime == 0)[0])})
    wl = GW.to_host_workload(gw, sample)
    before = snapshot(st)
    eng = BoundaryEngine(st, gw.B, gw.total_tokens(), Bd.params_from(gw.params))
    out = _bench_step(eng, torch.arange(gw.B, dtype=torch.int32, device="cuda"))
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, gw.params)
    rep = compare_requests(wl, sample, st, out, res, gw.params["n_local"])
    dec = out.decision.cpu().numpy()
    check_pool(st, before, dec, np.arange(gw.B))
    print("[paper]", rep, "grows", int(dec.sum()), flush=True)


def test_boundary_sweep_full_size_shrink():
    """The benchmark batch under the SHRINK policy: sampled requests against the oracle's
    SHRINK step, the whole batch's page state replayed from the GPU's own decisions."""
    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine
    from synth import gpu_workloads as GW
    from tests.parity_util import check_pool_shared

    gw = GW.boundary_sweep(seed=3000)
    st = gw.st
    params = dict(gw.params, policy="shrink")
    order = np.argsort(-gw.n)
    sample = sorted({int(order[0]), int(order[-1]), int(np.flatnonzero(gw.regime == 1)[0]),
                     int(np.flatnonzero(gw.regime == 0)[0]), int(np.flatnonzero(gw.regime == 0)[-1])})
    wl = GW.to_host_workload(gw, sample)
    before = snapshot(st)
    eng = BoundaryEngine(st, gw.B, gw.total_tokens(), Bd.params_from(params))
    out = eng.step(torch.arange(gw.B, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    print("[fullsize-shrink] step done; oracle on sample", sample, flush=True)
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, params)
    rep = compare_requests(wl, sample, st, out, res, gw.params["n_local"])
    summary = check_pool_shared(st, before, out, gw.B, st.P, int(gw.params["tau"]), shrink=True)
    dec = out.decision.cpu().numpy()[: gw.B]
    assert np.array_equal(dec == 1, gw.regime == 1), (dec, gw.regime)
    assert np.all(dec[gw.regime == 0] == 2)
    c = dict(zip(Bd.COUNTER_NAMES, out.counters.cpu().numpy().tolist()))
    assert c["shrinks"] == int((gw.regime == 0).sum()) == summary["freed"]
    print("[fullsize-shrink]", rep, c, flush=True)

"""Prefix-sharing stress on the 36-layer 8B shape with page size 32: groups of 16
requests share a 2048-token (64-page) refcounted prefix, contexts log-uniform from 1024
to 32768 tokens, Zipf exponent per request in [0.8, 1.6], and a pool of 80% of the
full-KV demand, so compactions that reach into a shared prefix need copy-on-write pages
the free stack mostly lacks (deferrals).

* reduced (2-3 layers, 8-32 requests, same page and prefix structure): the oracle runs
  the whole batch; everything is compared element by element, including copy-on-write
  pops, deferrals, pushes and the bytes of every page;
* full size (256 requests x 36 layers, about 217 GB of K/V): single shot; 32 sampled
  requests are recomputed by the oracle one at a time, each on its own; the whole batch
  is checked by the page-state replay and shared pages are compared byte for byte with a
  copy taken before the step.
"""
import numpy as np
import pytest
import torch

import oracle as O
from tests.parity_util import check_pool_shared, compare_sampled, compare_step, snapshot

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


# (generator arguments, counters the case must exercise)
REDUCED = {
    "pool80": (dict(seed=5000, B=32, L=2, ctx=(1024, 8192)), ("cow_pages", "deferred")),
    "pool100": (dict(seed=5001, B=32, L=2, ctx=(1024, 8192), pool_frac=1.0), ("cow_pages", "deferred")),
    "pairs": (dict(seed=5002, B=8, L=3, ctx=(2048, 8192), group=2, pool_frac=1.2), ("cow_pages", "freed_pages")),
    "denied": (dict(seed=5003, B=16, L=2, ctx=(2048, 8192), group=4, free_pages=5, grow_frac=0.5),
               ("grow_denied", "deferred")),
}


@pytest.mark.parametrize("name", list(REDUCED))
def test_prefix_share_reduced(name):
    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine
    from synth import gpu_workloads as GW

    kw, expect = REDUCED[name]
    _say(f"[prefix] {name} {kw}")
    gw = GW.prefix_share(**kw)
    st = gw.st
    wl = GW.to_host_workload(gw, range(gw.B))
    before = snapshot(st)
    eng = BoundaryEngine(st, gw.B, gw.total_tokens(), Bd.params_from(gw.params))
    out = eng.step(torch.arange(gw.B, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, gw.params)
    rep = compare_step(wl, np.arange(gw.B), st, out, res, gw.params["n_local"])
    summary = check_pool_shared(st, before, out, gw.B, st.P, int(gw.params["tau"]))
    c = dict(zip(Bd.COUNTER_NAMES, out.counters.cpu().numpy().tolist()))
    for key in ("grows", "compacts", "grow_denied", "deferred", "cow_pages", "freed_pages"):
        assert c[key] == res.counters[key], (key, c[key], res.counters[key])
    assert all(c[key] > 0 for key in expect), (expect, c)
    _say(f"[prefix] {name}: {res.counters} {summary} {rep}")


def test_prefix_share_full_size_sampled():
    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine
    from synth import gpu_workloads as GW

    free, total = torch.cuda.mem_get_info()
    _say(f"[prefix-full] device memory free {free / 2**30:.1f} GiB of {total / 2**30:.1f} GiB")
    gw = GW.prefix_share(seed=5000, contiguous=True)  # the bench's pools
    st = gw.st
    torch.cuda.synchronize()
    _say(f"[prefix-full] generated {gw.B} requests, {gw.total_tokens()} tokens, pool {st.num_pages} pages, "
         f"free {int(st.free_top.item())}")
    order = np.argsort(gw.n)
    rng = np.random.default_rng(5001)
    sample = {int(order[0]), int(order[-1]), int(order[len(order) // 2]), int(np.flatnonzero(gw.regime == 1)[0]), 17}
    sample |= {int(b) for b in rng.choice(gw.B, 40, replace=False)}
    sample = sorted(sample)[:32] if len(sample) > 32 else sorted(sample)
    assert len(sample) == 32
    # rows of each sampled request from before the step, one host copy per request
    pre = [GW.to_host_workload(gw, [b]) for b in sample]
    _say(f"[prefix-full] host copies of {len(sample)} requests taken")
    before = snapshot(st)
    shared = torch.as_tensor(np.flatnonzero(before["refcount"] > 1), device="cuda")
    k_shared, v_shared = st.k_pool[:, shared].clone(), st.v_pool[:, shared].clone()
    eng = BoundaryEngine(st, gw.B, gw.total_tokens(), Bd.params_from(gw.params))
    req = torch.arange(gw.B, dtype=torch.int32, device="cuda")
    eng.scan(req)  # the calls bench.py times (split compaction)
    eng.decide(req)
    eng.compact_prepare(req)
    eng.compact_move(req)
    torch.cuda.synchronize()
    out = eng.out
    c = dict(zip(Bd.COUNTER_NAMES, out.counters.cpu().numpy().tolist()))
    _say(f"[prefix-full] step done ({gw.pool_memory} pools): {c}; oracle on sample {sample}")
    assert torch.equal(st.k_pool[:, shared], k_shared) and torch.equal(st.v_pool[:, shared], v_shared), \
        "a shared page changed"
    del k_shared, v_shared
    summary = check_pool_shared(st, before, out, gw.B, st.P, int(gw.params["tau"]))
    assert summary["grows"] == c["grows"] and summary["deferred"] == c["deferred"]
    assert summary["freed"] == c["freed_pages"]
    totals = dict(ws=0, ws_near=0, ev_units=0, ev_near=0, ev_near_differs=0, ambiguous=0)
    for k, b in enumerate(sample):   # one request at a time, its host copy dropped after use
        rep = compare_sampled(pre[k], [b], st, out, gw.params)
        pre[k] = None
        totals["ws"] += rep.ws_total
        totals["ws_near"] += rep.ws_near
        totals["ev_units"] += rep.ev_units
        totals["ev_near"] += rep.ev_near
        totals["ev_near_differs"] += rep.ev_near_differs
        totals["ambiguous"] += rep.decisions_ambiguous
    _say(f"[prefix-full] {summary} {len(sample)} requests: {totals}")
    assert c["cow_pages"] > 0 and c["deferred"] > 0

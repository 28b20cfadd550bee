"""The whole-batch page-state check used on full-size GPU runs (``check_pool_shared``)
agrees with the oracle's own boundary step on small prefix-sharing batches: two
independent writings of the allocation rules (grow pops, copy-on-write, deferral,
ascending pushes) must give the same page state."""
import types

import numpy as np
import pytest
import torch

import oracle as O
from synth import gpu_workloads as GW
from tests.parity_util import check_pool_shared, snapshot


@pytest.mark.parametrize("kw,policy", [(dict(seed=11, B=8, group=4, pool_frac=0.8), "growpage"),
                                       (dict(seed=12, B=8, group=2, pool_frac=1.2), "growpage"),
                                       (dict(seed=13, B=6, group=3, pool_frac=1.0), "growpage"),
                                       (dict(seed=23, B=8, group=4, pool_frac=0.78, grow_frac=0.5), "growpage"),
                                       (dict(seed=26, B=8, group=4, pool_frac=0.8), "shrink"),
                                       (dict(seed=24, B=8, group=2, pool_frac=0.9, grow_frac=0.4), "shrink")])
def test_pool_replay_matches_oracle(kw, policy):
    gw = GW.prefix_share(L=1, Hq=4, Hkv=1, d=16, P=8, ctx=(256, 1024), prefix_pages=8, device="cpu", **kw)
    wl = GW.to_host_workload(gw, range(gw.B))
    before = snapshot(gw.st)
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, dict(gw.params, policy=policy))
    B, P = gw.B, gw.st.P
    ev = np.full((B, 1, 1, 2 * P), -1, np.int32)
    for b, e in res.evicted.items():
        ev[b, :, :, : e.shape[-1]] = e
    out = types.SimpleNamespace(delta=torch.from_numpy(res.delta.astype(np.int32)),
                                decision=torch.from_numpy(res.decision.astype(np.uint8)),
                                status=torch.from_numpy(res.status.astype(np.int32)),
                                evicted=torch.from_numpy(ev))
    st = types.SimpleNamespace(page_table=torch.from_numpy(res.page_table.astype(np.int32)),
                               n_alloc=torch.from_numpy(res.n_alloc.astype(np.int32)),
                               fill=torch.from_numpy(res.fill.astype(np.int32)),
                               refcount=torch.from_numpy(res.refcount.astype(np.int32)),
                               free_stack=torch.from_numpy(res.free_stack.astype(np.int32)),
                               free_top=torch.tensor([res.free_top], dtype=torch.int32))
    summary = check_pool_shared(st, before, out, B, P, int(gw.params["tau"]), shrink=policy == "shrink")
    if policy == "shrink":
        assert res.counters["shrinks"] > 0
    assert summary["grows"] == res.counters["grows"]
    assert summary["deferred"] == res.counters["deferred"]
    assert summary["freed"] == res.counters["freed_pages"]

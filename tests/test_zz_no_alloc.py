"""gp_boundary_step_static -- the boundary batch with the library's own per-device scratch,
for callers that cannot allocate -- against the entry points it stands for
(gp_boundary_scan, gp_decide_policy, gp_compact with a caller scratch) on a twin state:
every output, the page state and every pool byte equal, and the oracle's bar on top.
Two calls in a row, the second with a smaller batch (the buffer then holds the first
call's contents); a batch beyond the buffer is refused before any launch."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import device as SD
from synth import workloads as SW
from tests.parity_util import compare_step

pytestmark = pytest.mark.gpu


def _static_step(wl, st, prm, policy):
    from demand_paged_kv_amd import binding as Bd
    dev = "cuda"
    B, L, Hq, Hkv, P = wl.B, wl.L, wl.Hq, wl.Hkv, wl.P
    E = (2 if policy == "shrink" else 1) * P
    out = dict(ws=torch.empty((B, L, Hq, 2), dtype=torch.int32, device=dev),
               stats=torch.empty((B, L, Hq, 2, 2), dtype=torch.float32, device=dev),
               decision=torch.empty(B, dtype=torch.uint8, device=dev),
               delta=torch.empty(B, dtype=torch.int32, device=dev),
               status=torch.empty(B, dtype=torch.int32, device=dev),
               evicted=torch.empty((B, L, Hkv, E), dtype=torch.int32, device=dev),
               counters=torch.zeros(Bd.GP_NUM_COUNTERS, dtype=torch.int32, device=dev))
    req = torch.arange(B, dtype=torch.int32, device=dev)
    max_pos = 0 if st.rope_cos is None else int(st.rope_cos.shape[0])
    Bd.boundary_step_static(st.kv(), st.pages(), req, B, st.sum_s, st.sum_l, st.rope_cos, st.rope_sin, max_pos,
                            st.pos if st.rope_cos is not None else None, prm, wl.total_tokens(), out["ws"],
                            out["stats"], out["decision"], out["delta"], out["status"], out["evicted"],
                            out["counters"])
    return out


def _check_pair(wl, policy):
    from types import SimpleNamespace

    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine
    params = dict(wl.params, policy=policy)
    prm = Bd.params_from(params)
    st_a, st_b = SD.upload(wl, "cuda"), SD.upload(wl, "cuda")
    eng = BoundaryEngine(st_a, wl.B, wl.total_tokens(), Bd.params_from(params))
    eng.set_policy(policy)
    ref = eng.step(torch.arange(wl.B, dtype=torch.int32, device="cuda"))
    got = _static_step(wl, st_b, prm, policy)
    torch.cuda.synchronize()
    for f in ("ws", "stats", "decision", "delta", "status", "evicted"):
        a, b = getattr(ref, f)[: wl.B], got[f]
        assert torch.equal(a.view(torch.int32) if f == "stats" else a,
                           b.view(torch.int32) if f == "stats" else b), f
    assert torch.equal(ref.counters, got["counters"]), (ref.counters, got["counters"])
    for f in ("page_table", "n_alloc", "fill", "refcount", "free_top", "free_stack"):
        assert torch.equal(getattr(st_a, f), getattr(st_b, f)), f
    assert torch.equal(st_a.k_pool.view(torch.int16), st_b.k_pool.view(torch.int16)), "K pool"
    assert torch.equal(st_a.v_pool.view(torch.int16), st_b.v_pool.view(torch.int16)), "V pool"
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, params)
    rep = compare_step(wl, np.arange(wl.B), st_b, SimpleNamespace(**got), res, wl.params["n_local"])
    return res.counters, rep


def test_static_scratch_matches_caller_scratch_two_calls():
    from demand_paged_kv_amd import binding as Bd
    big = SW.direct_case(seed=811, B=8, L=2, Hq=32, Hkv=8, d=128, P=16, ctx=(300, 2000), grow_frac=0.4,
                         prefix_groups=2, prefix_pages=3, spare_pages=40, params=dict(SW.PARAMS_DEFAULT, n_local=16))
    small = SW.direct_case(seed=812, B=3, L=1, Hq=8, Hkv=2, d=64, P=16, ctx=(40, 400), grow_frac=0.3,
                           params=dict(SW.PARAMS_DEFAULT, n_local=8))
    for wl, policy in ((big, "growpage"), (small, "shrink")):
        need = Bd.scratch_bytes(SD.upload(wl, "cuda").kv(), wl.B, wl.total_tokens())
        assert need <= Bd.GP_STATIC_SCRATCH_BYTES
        counters, rep = _check_pair(wl, policy)
        print(f"[static] {wl.B} requests, {wl.total_tokens()} tokens, {policy}: {counters} {rep}", flush=True)


def test_static_scratch_refuses_a_batch_beyond_its_size():
    from demand_paged_kv_amd import binding as Bd
    wl = SW.direct_case(seed=813, B=2, L=1, Hq=8, Hkv=2, d=64, P=16, ctx=(40, 100))
    st = SD.upload(wl, "cuda")
    before = st.page_table.clone()
    prm = Bd.params_from(wl.params)
    too_many = 1 << 24   # candidate-token budget whose scratch exceeds the library's buffer
    assert Bd.scratch_bytes(st.kv(), wl.B, too_many) > Bd.GP_STATIC_SCRATCH_BYTES
    o = torch.empty(64, dtype=torch.int32, device="cuda")
    with pytest.raises(Bd.GrowPageError, match="GP_ERR_SCRATCH"):
        Bd.boundary_step_static(st.kv(), st.pages(), torch.arange(2, dtype=torch.int32, device="cuda"), 2,
                                st.sum_s, st.sum_l, st.rope_cos, st.rope_sin, int(st.rope_cos.shape[0]), st.pos,
                                prm, too_many, o, o, o, o, o)
    torch.cuda.synchronize()
    assert torch.equal(before, st.page_table)

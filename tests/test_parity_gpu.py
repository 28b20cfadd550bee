"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by element."""
import zlib

import numpy as np
import pytest
import torch

import oracle as O
from synth import workloads as SW
from tests.parity_util import compare_logits, compare_step, run_step_gpu

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _ema_gpu(wl):
    """Feed the decode queries through gp_update_summaries; return host summaries."""
    from demand_paged_kv_amd import binding as Bd
    T = wl.queries.shape[0]
    tdt = torch.bfloat16 if wl.q_dtype == "bf16" else torch.float32
    if wl.q_dtype == "bf16":
        q = torch.from_numpy(np.ascontiguousarray(wl.queries).view(np.int16)).view(torch.bfloat16)
    else:
        q = torch.from_numpy(np.ascontiguousarray(wl.queries))
    q = q.to("cuda")
    assert q.dtype == tdt
    S = torch.zeros((wl.B, wl.L, wl.Hq, wl.d), dtype=torch.float32, device="cuda")
    Lg = torch.zeros_like(S)
    req = torch.arange(wl.B, dtype=torch.int32, device="cuda")
    prm = Bd.params_from(wl.params)
    qd = Bd.GP_BF16 if wl.q_dtype == "bf16" else Bd.GP_F32
    for t in range(T):
        qt = q[t]
        Bd.update_summaries(qt, qd, (qt.stride(0), qt.stride(1), qt.stride(2)), req, wl.B, wl.L,
                            wl.Hq, wl.d, S, Lg, prm)
    torch.cuda.synchronize()
    return S.cpu().numpy(), Lg.cpu().numpy()


@pytest.mark.parametrize("cfg", ["config1", "config2"])
def test_ema_bit_exact(cfg):
    wl = getattr(SW, cfg)()
    _say(f"[ema] {cfg} T={wl.queries.shape[0]} B={wl.B}")
    s_gpu, l_gpu = _ema_gpu(wl)
    s_ref, l_ref = O.ema_run(wl.queries, wl.q_dtype, wl.params["beta_s"], wl.params["beta_l"])
    assert np.array_equal(s_gpu.view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(l_gpu.view(np.uint32), l_ref.view(np.uint32))


@pytest.mark.parametrize("beta_s,beta_l", [(0.5, 1.0), (1.0, 0.1), (0.25, 0.99999994)])
@pytest.mark.parametrize("q_dtype", ["f32", "bf16"])
def test_ema_other_betas(beta_s, beta_l, q_dtype):
    """Summary updates at other smoothing factors, from non-zero summaries: beta 1 keeps
    a summary as it was, a factor one float32 ulp below 1 moves it by a rounded 1-beta;
    bit-exact against the oracle's update."""
    from demand_paged_kv_amd import binding as Bd
    rng = np.random.default_rng(11)
    n, L, Hq, d = 3, 2, 8, 128
    qf = rng.standard_normal((n, L, Hq, d)).astype(np.float32)
    if q_dtype == "bf16":
        q = torch.from_numpy(qf).to(torch.bfloat16).cuda()
        qh = q.float().cpu().numpy()
    else:
        q = torch.from_numpy(qf).cuda()
        qh = qf
    s0 = rng.standard_normal((n, L, Hq, d)).astype(np.float32)
    l0 = rng.standard_normal((n, L, Hq, d)).astype(np.float32)
    S, Lg = torch.from_numpy(s0.copy()).cuda(), torch.from_numpy(l0.copy()).cuda()
    prm = Bd.params(beta_s, beta_l)
    qd = Bd.GP_BF16 if q_dtype == "bf16" else Bd.GP_F32
    req = torch.arange(n, dtype=torch.int32, device="cuda")
    for _ in range(3):
        Bd.update_summaries(q, qd, (q.stride(0), q.stride(1), q.stride(2)), req, n, L, Hq, d, S, Lg, prm)
    torch.cuda.synchronize()
    want_s, want_l = s0.copy(), l0.copy()
    for _ in range(3):
        want_s = O.ema_update(want_s, qh, beta_s)
        want_l = O.ema_update(want_l, qh, beta_l)
    assert np.array_equal(S.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(Lg.cpu().numpy().view(np.uint32), want_l.view(np.uint32))
    if beta_l == 1.0:
        assert np.array_equal(Lg.cpu().numpy(), l0)


def test_ema_strided_slots():
    """Strided q and scattered request slots update exactly the named rows."""
    from demand_paged_kv_amd import binding as Bd
    rng = np.random.default_rng(5)
    n, L, Hq, d, max_req = 5, 3, 8, 64, 11
    slots = np.array([7, 0, 3, 10, 5], np.int32)
    big = rng.standard_normal((n, L + 1, Hq, d + 8)).astype(np.float32)
    q = torch.from_numpy(big).cuda()[:, 1:, :, 4:4 + d]
    s0 = rng.standard_normal((max_req, L, Hq, d)).astype(np.float32)
    l0 = rng.standard_normal((max_req, L, Hq, d)).astype(np.float32)
    S, Lg = torch.from_numpy(s0.copy()).cuda(), torch.from_numpy(l0.copy()).cuda()
    prm = Bd.params(0.9, 0.999)
    Bd.update_summaries(q, Bd.GP_F32, (q.stride(0), q.stride(1), q.stride(2)),
                        torch.from_numpy(slots).cuda(), n, L, Hq, d, S, Lg, prm)
    torch.cuda.synchronize()
    want_s, want_l = s0.copy(), l0.copy()
    qh = big[:, 1:, :, 4:4 + d]
    for b, r in enumerate(slots):
        want_s[r] = O.ema_update(s0[r], qh[b], 0.9)
        want_l[r] = O.ema_update(l0[r], qh[b], 0.999)
    assert np.array_equal(S.cpu().numpy(), want_s)
    assert np.array_equal(Lg.cpu().numpy(), want_l)


def test_config1_boundary():
    wl = SW.config1()
    _say("[step] config1")
    s, l_ = O.ema_run(wl.queries, wl.q_dtype, wl.params["beta_s"], wl.params["beta_l"])
    res = O.boundary_step(wl, s, l_, wl.params)
    st, out, eng = run_step_gpu(wl, sum_s=s, sum_l=l_)
    rep = compare_step(wl, np.arange(wl.B), st, out, res, wl.params["n_local"])
    assert res.decision[0] == O.DECISION_COMPACT
    wl.sum_s, wl.sum_l = s, l_
    errs = compare_logits(eng, wl, range(wl.B))
    _say("config1", rep, "logit/probability errors", errs)


def test_config2_boundary():
    wl = SW.config2()
    _say(f"[step] config2 tokens={wl.total_tokens()}")
    s, l_ = O.ema_run(wl.queries, wl.q_dtype, wl.params["beta_s"], wl.params["beta_l"])
    res = O.boundary_step(wl, s, l_, wl.params)
    assert 0 < res.counters["grows"] < wl.B
    st, out, eng = run_step_gpu(wl, sum_s=s, sum_l=l_)
    rep = compare_step(wl, np.arange(wl.B), st, out, res, wl.params["n_local"])
    wl.sum_s, wl.sum_l = s, l_
    errs = compare_logits(eng, wl, range(wl.B))
    _say("config2", rep, res.counters, "logit/probability errors", errs)


CASES = [
    # (name, kwargs)
    ("bf16_d128_p16", dict(B=6, L=2, Hq=32, Hkv=8, d=128, P=16, ctx=(100, 900))),
    ("f32_d64_p16", dict(B=5, L=3, Hq=8, Hkv=2, d=64, P=16, dtype="f32", ctx=(30, 500))),
    ("bf16_d64_p32", dict(B=4, L=2, Hq=8, Hkv=2, d=64, P=32, ctx=(64, 700))),
    ("f32_d128_p8", dict(B=3, L=1, Hq=16, Hkv=4, d=128, P=8, dtype="f32", ctx=(9, 300))),
    ("no_rope", dict(B=4, L=2, Hq=8, Hkv=2, d=64, P=16, rope=False)),
    ("tiny_ctx", dict(B=6, L=1, Hq=8, Hkv=2, d=64, P=16, ctx=(1, 20), params=dict(SW.PARAMS_DEFAULT, n_local=4))),
    ("local_exceeds_k", dict(B=3, L=1, Hq=8, Hkv=2, d=64, P=16, ctx=(10, 60), params=dict(SW.PARAMS_DEFAULT, n_local=1000))),
    ("pool_exhausted", dict(B=8, L=2, Hq=8, Hkv=2, d=64, P=16, grow_frac=0.9, spare_pages=3)),
    ("cow_prefix", dict(B=6, L=2, Hq=8, Hkv=2, d=64, P=16, grow_frac=0.2, prefix_groups=2, prefix_pages=3,
                        ctx=(60, 200), spare_pages=40, params=dict(SW.PARAMS_DEFAULT, n_local=8))),
    ("cow_many", dict(B=24, L=1, Hq=8, Hkv=2, d=64, P=16, grow_frac=0.25, prefix_groups=4, prefix_pages=2,
                      ctx=(40, 160), spare_pages=30, params=dict(SW.PARAMS_DEFAULT, n_local=4))),
    ("cow_shortfall", dict(B=5, L=1, Hq=8, Hkv=2, d=64, P=16, grow_frac=0.0, prefix_groups=1, prefix_pages=2,
                           ctx=(40, 90), spare_pages=1, params=dict(SW.PARAMS_DEFAULT, n_local=4))),
    ("not_at_boundary", dict(B=4, L=1, Hq=8, Hkv=2, d=64, P=16, fill=[16, 3, 16, 0])),
    ("paper_p099", dict(B=4, L=2, Hq=32, Hkv=8, d=128, P=16, ctx=(200, 1500), params=dict(SW.PARAMS_PAPER))),
    ("p_one", dict(B=3, L=1, Hq=8, Hkv=2, d=64, P=16, params=dict(SW.PARAMS_DEFAULT, top_p=1.0))),
    ("p_zero", dict(B=3, L=1, Hq=8, Hkv=2, d=64, P=16, params=dict(SW.PARAMS_DEFAULT, top_p=0.0))),
    ("table_full", dict(B=4, L=1, Hq=8, Hkv=2, d=64, P=16, grow_frac=1.0, ctx=(60, 70), max_pages=6)),
    # the pages' operating point: KV block 256, p 0.99, quota 64
    ("paper_p256", dict(B=6, L=2, Hq=32, Hkv=8, d=128, P=256, ctx=(600, 4000), grow_frac=0.5,
                        params=dict(SW.PARAMS_PAPER))),
    ("p256_cow", dict(B=6, L=1, Hq=8, Hkv=2, d=64, P=256, grow_frac=0.2, prefix_groups=2, prefix_pages=2,
                      ctx=(300, 1500), spare_pages=12, params=dict(SW.PARAMS_PAPER))),
    ("p128_f32", dict(B=4, L=2, Hq=8, Hkv=2, d=128, P=128, dtype="f32", ctx=(100, 2000))),
    # bf16 keys in pages that are not a multiple of 16 tokens: the vector-unit scan
    ("bf16_d128_p24", dict(B=5, L=2, Hq=32, Hkv=8, d=128, P=24, ctx=(50, 1500))),
    ("bf16_d64_p8_cow", dict(B=6, L=2, Hq=8, Hkv=2, d=64, P=8, ctx=(9, 700), grow_frac=0.3, prefix_groups=2,
                             prefix_pages=2, spare_pages=24, params=dict(SW.PARAMS_DEFAULT, n_local=8))),
    # demand thresholds away from 0: positive deltas below tau compact, negative ones above it grow
    ("tau_positive", dict(B=8, L=2, Hq=32, Hkv=8, d=128, P=16, ctx=(100, 1500), grow_frac=0.5,
                          params=dict(SW.PARAMS_DEFAULT, tau=10000))),
    ("tau_negative", dict(B=8, L=2, Hq=32, Hkv=8, d=128, P=16, ctx=(100, 1500), grow_frac=0.5,
                          params=dict(SW.PARAMS_DEFAULT, tau=-16000))),
    # requests holding only their write page (no allocation pages): they grow or keep nothing;
    # the last one is empty (n = 0)
    ("zero_alloc", dict(B=6, L=2, Hq=8, Hkv=2, d=64, P=16, alloc=[0, 0, 0, 1, 3, 0], fill=[16, 16, 16, 16, 16, 0],
                        grow_frac=0.6, params=dict(SW.PARAMS_DEFAULT, n_local=8))),
    # GQA groups below 4 query heads per KV head (multi-head G = 1, G = 2), on the matrix-core
    # scan (bf16, P % 16 == 0) and the vector-unit scan (float32 or P = 24)
    ("gqa1_bf16_d128_p16", dict(B=5, L=2, Hq=8, Hkv=8, d=128, P=16, ctx=(100, 900), grow_frac=0.5)),
    ("gqa2_bf16_d64_p16", dict(B=5, L=2, Hq=4, Hkv=2, d=64, P=16, ctx=(60, 700), grow_frac=0.5)),
    ("gqa2_f32_d128_p8", dict(B=4, L=1, Hq=8, Hkv=4, d=128, P=8, dtype="f32", ctx=(9, 400))),
    ("gqa1_bf16_d64_p24", dict(B=4, L=2, Hq=4, Hkv=4, d=64, P=24, ctx=(30, 800))),
    ("gqa1_p256_cow", dict(B=5, L=1, Hq=2, Hkv=2, d=128, P=256, grow_frac=0.2, prefix_groups=2, prefix_pages=2,
                           ctx=(300, 1500), spare_pages=12, params=dict(SW.PARAMS_PAPER))),
    # 128K-token units: a unit's logits (4 MB) far beyond the selection's LDS buffers
    ("long_unit_128k", dict(B=2, L=1, Hq=32, Hkv=8, d=128, P=16, ctx=(131072, 131072), grow_frac=0.5)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_direct_cases(name, kw):
    wl = SW.direct_case(seed=zlib.crc32(name.encode()) % 10000, name=name, **kw)
    _say(f"[case] {name} B={wl.B} tokens={wl.total_tokens()}")
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, wl.params)
    # scattered request slots inside a larger table
    slots = np.arange(wl.B) * 3 + 1
    st, out, eng = run_step_gpu(wl, slots=slots, max_req=int(slots.max()) + 2)
    rep = compare_step(wl, slots, st, out, res, wl.params["n_local"])
    errs = compare_logits(eng, wl, range(wl.B))
    _say(name, rep, res.counters, "logit/probability errors", errs)


# The same cases on the fused scan kernel: small batches (at most 512 units) take the split
# logit kernel plus a selection kernel, so each bf16 case with pages of a multiple of 16
# tokens is run again with empty requests added until the batch has more units than that.
FUSED_CASES = [c for c in CASES if c[1].get("dtype", "bf16") == "bf16" and c[1].get("P", 16) % 16 == 0]
SPLIT_UNITS = 512


@pytest.mark.parametrize("name,kw", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_direct_cases_fused_kernel(name, kw):
    from tests.parity_util import pad_with_empty
    wl = SW.direct_case(seed=zlib.crc32(name.encode()) % 10000, name=name, **kw)
    b0, per = wl.B, wl.L * wl.Hkv
    wl = pad_with_empty(wl, -(-(SPLIT_UNITS + 1) // per) - b0)
    assert wl.B * per > SPLIT_UNITS
    _say(f"[case] {name} fused: B={wl.B} ({b0} with tokens) tokens={wl.total_tokens()}")
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, wl.params)
    st, out, eng = run_step_gpu(wl)
    rep = compare_step(wl, np.arange(wl.B), st, out, res, wl.params["n_local"])
    errs = compare_logits(eng, wl, range(b0))
    _say(name, "fused", rep, res.counters, "logit/probability errors", errs)


def test_rope_positions_clamped_to_the_table():
    """Positions beyond the caller's rotation table use its last row: the scan on a table
    cut short matches the oracle at the clamped positions (full table, same rows)."""
    import dataclasses
    wl = SW.direct_case(seed=321, B=6, L=2, Hq=32, Hkv=8, d=128, P=16, ctx=(100, 1200), grow_frac=0.5,
                        params=dict(SW.PARAMS_DEFAULT, n_local=16))
    T = int(np.median(wl.pos))
    assert (wl.pos >= T).any() and (wl.pos < T - 1).any()
    wl_gpu = dataclasses.replace(wl, rope_cos=wl.rope_cos[:T].copy(), rope_sin=wl.rope_sin[:T].copy())
    wl_ref = dataclasses.replace(wl, pos=np.minimum(wl.pos, T - 1).astype(np.int32))
    res = O.boundary_step(wl_ref, wl.sum_s, wl.sum_l, wl.params)
    st, out, _ = run_step_gpu(wl_gpu)
    rep = compare_step(wl_ref, np.arange(wl.B), st, out, res, wl.params["n_local"])
    _say("rope clamp", rep, res.counters)


def test_counters_config2():
    wl = SW.config2(seed=2001)
    s, l_ = O.ema_run(wl.queries, wl.q_dtype, wl.params["beta_s"], wl.params["beta_l"])
    res = O.boundary_step(wl, s, l_, wl.params)
    st, out, _ = run_step_gpu(wl, sum_s=s, sum_l=l_)
    c = out.counters.cpu().numpy()
    assert c[0] == res.counters["grows"] and c[1] == res.counters["compacts"]
    assert c[2] == res.counters["grow_denied"] and c[3] == res.counters["deferred"]
    assert c[4] == res.counters["cow_pages"] and c[5] == res.counters["freed_pages"]
    moved = sum(max(0, wl.n(b) - wl.P - int(res.evicted[b][l, g][0]))
                for b in res.k_new for l in range(wl.L) for g in range(wl.Hkv))
    assert c[6] == moved


def test_empty_batch_is_noop():
    from demand_paged_kv_amd import binding as Bd
    wl = SW.direct_case(seed=3, B=2, L=1, Hq=8, Hkv=2, d=64)
    from synth import device as SD
    st = SD.upload(wl)
    prm = Bd.params_from(wl.params)
    kv, pg = st.kv(), st.pages()
    req = torch.zeros(1, dtype=torch.int32, device="cuda")
    Bd.boundary_scan(kv, pg, req, 0, st.sum_s, st.sum_l, None, None, 0, None, prm, req, None, req, 0, 0)
    Bd.decide(req, req, 0, 1, 8, 16, prm, pg, req, req, req)
    Bd.compact(kv, pg, req, req, 0, prm, None, req, None, req, 0, 0)
    torch.cuda.synchronize()


def test_deterministic_repeat():
    """Two runs on the same inputs give identical bytes (integer mass sums, fixed pop order)."""
    wl = SW.direct_case(seed=77, B=6, L=2, Hq=32, Hkv=8, d=128, P=16, ctx=(200, 2000), prefix_groups=2,
                        prefix_pages=2, spare_pages=20, params=dict(SW.PARAMS_DEFAULT, n_local=16))
    outs = []
    for _ in range(2):
        st, out, _ = run_step_gpu(wl)
        outs.append((out.ws.cpu().numpy(), out.stats.cpu().numpy(), out.evicted.cpu().numpy(),
                     st.k_pool.view(torch.int16).cpu().numpy(), st.page_table.cpu().numpy()))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_concurrent_streams():
    """Two independent batches (own pools, page state, scratch and outputs) with their calls
    interleaved on two streams, so their kernels may run side by side: each matches the
    oracle.  The library keeps no state between calls and launches on the caller's stream."""
    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine
    from synth import device as SD
    cases = [SW.direct_case(seed=seed, B=6, L=2, Hq=32, Hkv=8, d=128, P=16, ctx=(300, 4000), grow_frac=0.4,
                            prefix_groups=2, prefix_pages=2, spare_pages=20,
                            params=dict(SW.PARAMS_DEFAULT, n_local=16), name=f"stream{seed}")
             for seed in (91, 92)]
    results = [O.boundary_step(wl, wl.sum_s, wl.sum_l, wl.params) for wl in cases]
    states = [SD.upload(wl, "cuda") for wl in cases]
    engines = [BoundaryEngine(st, wl.B, wl.total_tokens(), Bd.params_from(wl.params)) for st, wl in zip(states, cases)]
    reqs = [torch.arange(wl.B, dtype=torch.int32, device="cuda") for wl in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for call in ("scan", "decide", "compact"):
        for eng, req, s in zip(engines, reqs, streams):
            getattr(eng, call)(req, s)
    torch.cuda.synchronize()
    for wl, st, eng, res in zip(cases, states, engines, results):
        rep = compare_step(wl, np.arange(wl.B), st, eng.out, res, wl.params["n_local"])
        _say(wl.name, rep, res.counters)


PLANTED = [
    # every element in one bin, more than the LDS candidate buffer holds; equal importance
    ("uniform_5k", [(312, lambda rng, n: np.zeros(n))], dict(SW.PARAMS_DEFAULT, n_local=0)),
    # the mass crossing lies beyond the binned range (x > 255/16): whole-row fallback
    ("tail_crossing", [(250, lambda rng, n: np.where(np.arange(n) < 2, 17.0, 0.0)[rng.permutation(n)])],
     dict(SW.PARAMS_DEFAULT, top_p=0.99999, n_local=0)),
    # importance falling with the slot: every new slot enters the keep buffer
    ("falling", [(300, lambda rng, n: -np.arange(n) / 500.0)], dict(SW.PARAMS_DEFAULT, n_local=32)),
    # importance rising with the slot: the oldest slots go
    ("rising", [(200, lambda rng, n: np.arange(n) / 700.0)], dict(SW.PARAMS_DEFAULT, n_local=0)),
    # narrow spread: thousands of elements inside the crossing bin
    ("narrow", [(400, lambda rng, n: 0.02 * rng.standard_normal(n)),
                (40, lambda rng, n: 3.0 * rng.standard_normal(n))], dict(SW.PARAMS_DEFAULT, n_local=16)),
]


def _deep_tail(rng, n, top=-110.0, step=0.5):
    """Logits in [0, 2] except 40 slots 110-130 nats below (0.5 nat apart, never the last
    8): their probabilities lie below float32's range, yet the keep-set must rank them by
    value (the 16 lowest go), not by age."""
    lg = rng.uniform(0.0, 2.0, n)
    deep = rng.choice(n - 8, 40, replace=False)
    lg[deep] = top - step * rng.permutation(40)
    return lg


# planted cases on bf16 keys (the matrix-core scan); logits x sqrt(64) exact in bf16 where it matters
PLANTED_BF16 = [
    # 100-119.5 nats below the maximum (exact bf16 multiples of 4 after scaling by 8)
    ("deep_tail_bf16", [(40, lambda rng, n: _deep_tail(rng, n, top=-100.0)),
                        (64, lambda rng, n: _deep_tail(rng, n, top=-100.0))], dict(SW.PARAMS_DEFAULT, n_local=8)),
]
PLANTED += [
    ("deep_tail", [(40, _deep_tail), (90, lambda rng, n: _deep_tail(rng, n, top=-115.0, step=0.375))],
     dict(SW.PARAMS_DEFAULT, n_local=8)),
]


@pytest.mark.parametrize("name,fns,params,dtype", [c + ("f32",) for c in PLANTED] + [c + ("bf16",) for c in PLANTED_BF16],
                         ids=[c[0] for c in PLANTED] + [c[0] for c in PLANTED_BF16])
def test_planted_logits(name, fns, params, dtype):
    _planted(name, fns, params, dtype, False)


@pytest.mark.parametrize("name,fns,params", PLANTED_BF16, ids=[c[0] for c in PLANTED_BF16])
def test_planted_logits_fused_kernel(name, fns, params):
    """The bf16 planted cases on the fused scan kernel (empty requests added)."""
    _planted(name, fns, params, "bf16", True)


def _planted(name, fns, params, dtype, fused):
    wl = SW.planted_logits_case(zlib.crc32(name.encode()) % 10000, fns, params=params, name=name, dtype=dtype)
    b0 = wl.B
    if fused:
        from tests.parity_util import pad_with_empty
        wl = pad_with_empty(wl, -(-(SPLIT_UNITS + 1) // (wl.L * wl.Hkv)) - wl.B)
    _say(f"[planted] {name} n={[wl.n(b) for b in range(b0)]} batch {wl.B}")
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, wl.params)
    st, out, eng = run_step_gpu(wl)
    rep = compare_step(wl, np.arange(wl.B), st, out, res, wl.params["n_local"])
    errs = compare_logits(eng, wl, range(b0))
    _say(name, rep, res.counters, "W", res.W[:b0, 0, 0].tolist(), "logit/probability errors", errs)


@pytest.mark.parametrize("policy", ["growpage", "random", "inverse", "always_compact", "shrink"])
def test_decision_policies(policy):
    """The ablation policies through gp_decide_policy, the rest of the batch as usual."""
    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine
    from synth import device as SD
    wl = SW.direct_case(seed=911, B=10, L=2, Hq=32, Hkv=8, d=128, P=16, ctx=(100, 900), grow_frac=0.5,
                        spare_pages=6)
    u = np.random.default_rng(912).random(wl.B).astype(np.float32)
    prm = dict(wl.params, policy=policy, rand_u=u, grow_prob=0.4)
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, prm)
    _say(f"[policy] {policy}: decisions {res.decision.tolist()} status {res.status.tolist()}")
    st = SD.upload(wl, "cuda")
    eng = BoundaryEngine(st, wl.B, wl.total_tokens(), Bd.params_from(wl.params))
    eng.set_policy(policy, torch.as_tensor(u, device="cuda"), 0.4)
    out = eng.step(torch.arange(wl.B, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    compare_step(wl, np.arange(wl.B), st, out, res, wl.params["n_local"])


SHRINK_CASES = [
    # shared prefixes: copy-on-write below the released page, shared released pages
    ("shrink_cow_p16", dict(B=8, L=2, Hq=32, Hkv=8, d=128, P=16, ctx=(40, 600), grow_frac=0.3, prefix_groups=2,
                            prefix_pages=3, spare_pages=40, params=dict(SW.PARAMS_DEFAULT, n_local=16))),
    # 2P = 512 evicted slots per unit, the pages' operating point
    ("shrink_p256", dict(B=4, L=1, Hq=32, Hkv=8, d=128, P=256, ctx=(300, 2500), grow_frac=0.3,
                         params=dict(SW.PARAMS_DEFAULT, top_p=0.99, n_local=64))),
    # no allocation pages and one page: both compact in place; two pages shrink
    ("shrink_write_page_only", dict(B=6, L=2, Hq=8, Hkv=2, d=64, P=16, alloc=[0, 0, 1, 2, 3, 1], grow_frac=0.4,
                                    params=dict(SW.PARAMS_DEFAULT, n_local=8))),
    # float32 keys, page 8 (the vector-unit scan), one-page allocations that compact in place
    ("shrink_f32_p8", dict(B=8, L=2, Hq=8, Hkv=2, d=64, P=8, dtype="f32", ctx=(4, 200), grow_frac=0.3,
                           params=dict(SW.PARAMS_DEFAULT, n_local=4))),
]


@pytest.mark.parametrize("name,kw", SHRINK_CASES, ids=[c[0] for c in SHRINK_CASES])
def test_shrink_policy(name, kw):
    """GP_POLICY_SHRINK end to end against the oracle's SHRINK step: keep-sets of (A-1)P
    slots, released pages, write pages moved, pool state and page contents."""
    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine
    from synth import device as SD
    wl = SW.direct_case(seed=zlib.crc32(name.encode()) % 10000, name=name, **kw)
    prm = dict(wl.params, policy="shrink")
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, prm)
    _say(f"[shrink] {name}: A {wl.n_alloc.tolist()} decisions {res.decision.tolist()} counters {res.counters}")
    assert res.counters["shrinks"] > 0
    st = SD.upload(wl, "cuda")
    eng = BoundaryEngine(st, wl.B, wl.total_tokens(), Bd.params_from(prm))
    assert eng.policy == "shrink" and eng.out.evicted.shape[-1] == 2 * wl.P
    out = eng.step(torch.arange(wl.B, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    rep = compare_step(wl, np.arange(wl.B), st, out, res, wl.params["n_local"])
    c = dict(zip(Bd.COUNTER_NAMES, out.counters.cpu().numpy().tolist()))
    for key in ("shrinks", "compacts", "deferred", "cow_pages", "freed_pages"):
        assert c[key] == res.counters[key], (key, c[key], res.counters[key])
    _say(name, rep)


def test_contiguous_pools():
    """Pools in the library's physically contiguous memory (gp_contiguous_malloc through
    torch's pluggable allocator): the allocation is served, and a boundary step on those
    pools matches the oracle like any other memory."""
    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd import pool as PM
    from demand_paged_kv_amd.engine import BoundaryEngine
    from synth import device as SD
    t, kind = PM.empty((3, 1 << 20), torch.float32, "cuda")
    assert kind == "contiguous" and t.data_ptr() % 4096 == 0
    t.copy_(torch.arange(3 << 20, dtype=torch.float32, device="cuda").view(3, 1 << 20))
    assert float(t[2, 5].item()) == float((2 << 20) + 5)
    del t
    name = "contiguous_pools"
    wl = SW.direct_case(seed=zlib.crc32(name.encode()) % 10000, B=6, L=2, Hq=32, Hkv=8, d=128, P=16,
                        ctx=(100, 1500), grow_frac=0.4, prefix_groups=2, prefix_pages=2, spare_pages=30,
                        name=name)
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, wl.params)
    st = SD.upload(wl, "cuda")
    for f in ("k_pool", "v_pool"):
        src = getattr(st, f)
        dst, kind = PM.empty(src.shape, src.dtype, "cuda")
        assert kind == "contiguous"
        dst.copy_(src)
        setattr(st, f, dst)
    eng = BoundaryEngine(st, wl.B, wl.total_tokens(), Bd.params_from(wl.params))
    out = eng.step(torch.arange(wl.B, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    rep = compare_step(wl, np.arange(wl.B), st, out, res, wl.params["n_local"])
    _say(name, rep, res.counters)


@pytest.mark.parametrize("kernel", ["split", "fused"])
def test_token_budget_overflow(kernel):
    """A batch larger than the scratch's token budget: the entries that fit (a prefix in
    batch order) behave as the oracle's step on them alone; the rest are flagged
    GP_REQ_OVERFLOW, report working sets of -1 and are left untouched.  ``fused``: empty
    requests added after them make the batch large enough for the fused scan kernel."""
    import dataclasses
    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine
    from synth import device as SD
    name = "token_overflow"
    wl = SW.direct_case(seed=zlib.crc32(name.encode()) % 10000, B=6, L=2, Hq=8, Hkv=2, d=64, P=16,
                        ctx=(100, 400), grow_frac=0.2, spare_pages=30, name=name)
    b0 = wl.B
    if kernel == "fused":
        from tests.parity_util import pad_with_empty
        wl = pad_with_empty(wl, -(-(SPLIT_UNITS + 1) // (wl.L * wl.Hkv)) - wl.B)
    j = 3   # the fitting prefix holds a grow and two compactions
    budget = sum(wl.n(b) for b in range(j))
    sub = dataclasses.replace(wl, page_table=wl.page_table[:j], n_alloc=wl.n_alloc[:j], fill=wl.fill[:j],
                              pos=wl.pos[:j], k_rows=wl.k_rows[:j], v_rows=wl.v_rows[:j],
                              sum_s=wl.sum_s[:j], sum_l=wl.sum_l[:j])
    res = O.boundary_step(sub, sub.sum_s, sub.sum_l, sub.params)
    st = SD.upload(wl, "cuda")
    eng = BoundaryEngine(st, wl.B, budget, Bd.params_from(wl.params))
    out = eng.step(torch.arange(wl.B, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    rep = compare_step(sub, np.arange(j), st, out, res, wl.params["n_local"])
    ws = out.ws.cpu().numpy()
    status = out.status.cpu().numpy()
    dec = out.decision.cpu().numpy()
    table = st.page_table.cpu().numpy()
    for b in range(j, wl.B):
        # the added empty requests are also not at a boundary
        want = Bd.GP_REQ_OVERFLOW | (Bd.GP_REQ_NOT_AT_BOUNDARY if b >= b0 else 0)
        assert status[b] == want and dec[b] == Bd.GP_DECISION_COMPACT, (b, status[b], dec[b])
        assert np.all(ws[b] == -1)
        assert int(st.n_alloc[b]) == int(wl.n_alloc[b]) and int(st.fill[b]) == int(wl.fill[b])
        assert np.array_equal(table[b], wl.page_table[b])
        gk, gv = SD.read_rows(st, table[b], wl.n(b), wl.dtype)
        assert np.array_equal(gk, wl.k_rows[b]) and np.array_equal(gv, wl.v_rows[b]), ("untouched", b)
    _say(name, rep, res.counters, "status", status.tolist())

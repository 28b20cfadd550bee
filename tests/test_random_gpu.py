"""Seeded random boundary batches against the oracle.

Each case draws, from its own seed, a batch shape (1-8 requests, 1-3 layers, 1/2/8 KV heads
with 1, 2 or 4 query heads each, head_dim 64 or 128), storage (bf16 or float32), page size (8 to
256 tokens, including sizes that are not multiples of 16, which take the vector-unit
scan), contexts, prefix sharing, pool pressure (free pages, full page-table rows),
requests off their boundary, RoPE or none, Top-p, tau, the local quota and a decision
policy; the GPU batch is compared with the oracle element by element (working sets,
statistics, decisions, status, keep-sets, page state, page bytes, logits and
probabilities).  A case whose decision the oracle finds ambiguous (delta within rounding
of tau) is skipped: either answer is right there, and the rest of the batch then
depends on which one the GPU took."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import device as SD
from synth import workloads as SW
from tests.parity_util import compare_logits, compare_step

pytestmark = pytest.mark.gpu

SEEDS = list(range(7100, 7700))


def _draw(seed):
    rng = np.random.default_rng(seed)
    # the group size from a stream of its own, so the other draws do not depend on it
    G = int(np.random.default_rng([seed, 1]).choice([1, 2, 4, 4]))
    Hkv = int(rng.choice([1, 2, 8]))
    d = int(rng.choice([64, 128]))
    P = int(rng.choice([8, 16, 16, 24, 32, 48, 64, 128, 256]))
    dtype = "bf16" if rng.random() < 0.7 else "f32"
    B = int(rng.integers(1, 9))
    L = int(rng.integers(1, 4))
    lo = int(rng.integers(1, 600))
    hi = lo + int(rng.integers(0, 2500))
    prefix_groups = int(rng.integers(0, 3)) if B > 1 and rng.random() < 0.4 else 0
    prefix_pages = int(rng.integers(1, 4)) if prefix_groups else 0
    fill = None
    if rng.random() < 0.3:
        fill = np.where(rng.random(B) < 0.7, P, rng.integers(0, P, B)).astype(np.int32)
    policy = str(rng.choice(["growpage"] * 5 + ["shrink", "inverse", "random", "always_compact"]))
    params = dict(beta_s=0.9, beta_l=0.999, top_p=float(rng.choice([0.5, 0.9, 0.95, 0.99, 0.999])),
                  tau=int(rng.choice([0, 0, 0, 50, -50])), n_local=int(rng.choice([0, 4, 16, 64])))
    kw = dict(B=B, L=L, Hq=G * Hkv, Hkv=Hkv, d=d, P=P, dtype=dtype, ctx=(lo, hi),
              spare_pages=int(rng.integers(0, 40)), grow_frac=float(rng.uniform(0, 1)),
              rope=bool(rng.random() < 0.85), prefix_groups=prefix_groups, prefix_pages=prefix_pages,
              fill=fill, params=params)
    wl = SW.direct_case(seed=seed, name=f"random{seed}", **kw)
    if rng.random() < 0.15:   # page-table rows with no room to grow for the longest requests
        wl.max_pages = int(wl.n_alloc.max()) + 1
        wl.page_table = np.ascontiguousarray(wl.page_table[:, : wl.max_pages])
    u = rng.random(B).astype(np.float32)
    return wl, policy, u, float(rng.uniform(0.1, 0.9))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_batch(seed):
    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine
    wl, policy, u, grow_prob = _draw(seed)
    prm = dict(wl.params, policy=policy, rand_u=u, grow_prob=grow_prob)
    print(f"[random] seed {seed}: B={wl.B} L={wl.L} Hq={wl.Hq} Hkv={wl.Hkv} d={wl.d} P={wl.P} {wl.dtype} "
          f"tokens={wl.total_tokens()} policy={policy} params={wl.params}", flush=True)
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, prm)
    if res.ambiguous.any():
        pytest.skip("the oracle finds a decision ambiguous (delta within rounding of tau)")
    st = SD.upload(wl, "cuda")
    eng = BoundaryEngine(st, wl.B, wl.total_tokens(), Bd.params_from(prm))
    eng.set_policy(policy, torch.as_tensor(u, device="cuda"), grow_prob)
    out = eng.step(torch.arange(wl.B, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    rep = compare_step(wl, np.arange(wl.B), st, out, res, wl.params["n_local"])
    errs = compare_logits(eng, wl, range(wl.B))
    print(f"[random] seed {seed}: {res.counters} {rep} logit/probability errors {errs}", flush=True)


# Larger batches (8-24 requests x 2-4 layers x 8 KV heads: 128-768 units), bf16 keys in pages
# of 16-256 tokens: both forms of the matrix-core scan, a unit's steps split over several
# blocks (at most 512 units) and one fused block per unit (more).
LARGE_SEEDS = list(range(30000, 30040))


def _draw_large(seed):
    rng = np.random.default_rng(seed)
    G = int(rng.choice([1, 2, 4, 4]))
    Hkv = 8
    d = int(rng.choice([64, 128]))
    P = int(rng.choice([16, 16, 32, 64, 128, 256]))
    B = int(rng.integers(8, 25))
    L = int(rng.integers(2, 5))
    lo = int(rng.integers(1, 1500))
    hi = lo + int(rng.integers(0, 3000))
    prefix_groups = int(rng.integers(0, 3)) if rng.random() < 0.4 else 0
    prefix_pages = int(rng.integers(1, 4)) if prefix_groups else 0
    fill = None
    if rng.random() < 0.3:
        fill = np.where(rng.random(B) < 0.7, P, rng.integers(0, P, B)).astype(np.int32)
    policy = str(rng.choice(["growpage"] * 5 + ["shrink", "inverse", "random", "always_compact"]))
    params = dict(beta_s=0.9, beta_l=0.999, top_p=float(rng.choice([0.5, 0.9, 0.95, 0.99, 0.999])),
                  tau=int(rng.choice([0, 0, 0, 50, -50])), n_local=int(rng.choice([0, 4, 16, 64])))
    kw = dict(B=B, L=L, Hq=G * Hkv, Hkv=Hkv, d=d, P=P, dtype="bf16", ctx=(lo, hi),
              spare_pages=int(rng.integers(0, 60)), grow_frac=float(rng.uniform(0, 1)),
              rope=bool(rng.random() < 0.85), prefix_groups=prefix_groups, prefix_pages=prefix_pages,
              fill=fill, params=params)
    wl = SW.direct_case(seed=seed, name=f"large{seed}", **kw)
    u = rng.random(B).astype(np.float32)
    return wl, policy, u, float(rng.uniform(0.1, 0.9))


@pytest.mark.parametrize("seed", LARGE_SEEDS)
def test_random_large_batch(seed):
    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine
    wl, policy, u, grow_prob = _draw_large(seed)
    prm = dict(wl.params, policy=policy, rand_u=u, grow_prob=grow_prob)
    print(f"[random-large] seed {seed}: B={wl.B} L={wl.L} Hq={wl.Hq} d={wl.d} P={wl.P} "
          f"units={wl.B * wl.L * wl.Hkv} tokens={wl.total_tokens()} policy={policy}", flush=True)
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, prm)
    if res.ambiguous.any():
        pytest.skip("the oracle finds a decision ambiguous (delta within rounding of tau)")
    st = SD.upload(wl, "cuda")
    eng = BoundaryEngine(st, wl.B, wl.total_tokens(), Bd.params_from(prm))
    eng.set_policy(policy, torch.as_tensor(u, device="cuda"), grow_prob)
    out = eng.step(torch.arange(wl.B, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    rep = compare_step(wl, np.arange(wl.B), st, out, res, wl.params["n_local"])
    errs = compare_logits(eng, wl, range(min(wl.B, 3)))
    print(f"[random-large] seed {seed}: {res.counters} {rep} logit/probability errors {errs}", flush=True)

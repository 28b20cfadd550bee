"""Property tests of the oracle on tiny inputs (hypothesis; CPU only).

Each property is stated independently of the oracle's own procedure:

* working sets against an exhaustive search over all subsets in exact integer arithmetic
  (masses are small integers, so ties between slots and sums that hit p exactly are
  common);
* keep-sets against their characterisation: the local slots are kept, and every kept
  candidate beats every evicted one in (importance, slot) order;
* whole boundary steps on random small pools (sharing, exhaustion, partial write pages,
  four decision policies) against the pool's bookkeeping: references equal refcounts,
  the free stack holds exactly the unreferenced pages, grows pop the stack top in batch
  order and copy-on-write pages after them, freed pages are pushed in ascending id order,
  a page is copied exactly when it was shared at the start of the step and its rows
  change, compacted rows are the stable gather of the old rows, and requests that are
  deferred or not at their boundary are untouched.
"""
import itertools
from fractions import Fraction

import numpy as np
from hypothesis import HealthCheck, event, given, settings
from hypothesis import strategies as st

import oracle as O
from synth import workloads as SW

FAST = settings(max_examples=300, deadline=None, derandomize=True, database=None)
SLOW = settings(max_examples=250, deadline=None, derandomize=True, database=None,
                suppress_health_check=[HealthCheck.too_slow])


def _smallest_reaching(masses, p: Fraction) -> int:
    total = sum(masses)
    for m in range(1, len(masses) + 1):
        for c in itertools.combinations(range(len(masses)), m):
            if Fraction(sum(masses[i] for i in c), total) >= p:
                return m
    return len(masses)


@FAST
@given(masses=st.lists(st.integers(0, 8), min_size=1, max_size=9).filter(lambda m: sum(m) > 0),
       p_num=st.integers(1, 63), dyadic=st.booleans(), p_float=st.floats(0.001, 0.999))
def test_working_set_is_the_smallest_subset_reaching_p(masses, p_num, dyadic, p_float):
    """R1: W is the size of the smallest subset of slots whose probability mass is at least
    p.  Masses are integers over their total, p a dyadic fraction (exact hits) or a float."""
    p = p_num / 64.0 if dyadic else p_float
    a = np.array(masses, np.float64) / sum(masses)
    best = _smallest_reaching(masses, Fraction(p))
    W, lo, hi = O.working_set(a, p)
    assert lo <= best <= hi, (masses, p, W, lo, hi)
    if lo == hi:
        assert W == best


@FAST
@given(imp=st.lists(st.integers(0, 4), min_size=1, max_size=9), data=st.data())
def test_keep_set_matches_its_characterisation(imp, data):
    """R6: the last min(n_local, k) slots are kept; among the other slots exactly
    k - min(n_local, k) are kept, each ranking above every evicted one by (importance,
    slot index).  Exactly one subset satisfies this; the oracle must return it."""
    n = len(imp)
    k = data.draw(st.integers(1, n))
    n_local = data.draw(st.integers(0, 4))
    imp_a = np.array(imp, np.float64) / 4.0
    nl = min(n_local, k)
    cand = n - nl
    keep_c = k - nl
    valid = []
    for c in itertools.combinations(range(cand), keep_c):
        ev = [e for e in range(cand) if e not in c]
        if all((imp_a[x], x) > (imp_a[e], e) for x in c for e in ev):
            valid.append(sorted(list(c) + list(range(cand, n))))
    assert len(valid) == 1
    kept, evicted, near = O.keep_set(imp_a, k, n_local)
    assert list(kept) == valid[0]
    assert sorted(set(range(n)) - set(kept)) == list(evicted)
    assert O.keep_set_valid(evicted, imp_a, k, n_local)
    if 0 < keep_c < cand:
        tie = min(imp_a[x] for x in kept if x < cand) == max(imp_a[e] for e in evicted)
        assert near == tie


def _references(table, n_alloc, num_pages):
    refs = np.zeros(num_pages, np.int64)
    for r in range(table.shape[0]):
        for j in range(int(n_alloc[r]) + 1):
            if table[r, j] >= 0:
                refs[table[r, j]] += 1
    return refs


@SLOW
@given(seed=st.integers(0, 10_000), B=st.integers(1, 6), P=st.sampled_from([8, 16]),
       spare=st.integers(0, 12), grow_frac=st.floats(0.0, 1.0), share=st.sampled_from([True, True, False]),
       n_local=st.integers(0, 40), policy=st.sampled_from(["growpage", "inverse", "always_compact", "shrink"]),
       data=st.data())
def test_boundary_step_keeps_the_pool_consistent(seed, B, P, spare, grow_frac, share, n_local, policy, data):
    fill = [data.draw(st.sampled_from([P, P, data.draw(st.integers(0, P - 1))])) for _ in range(B)]
    prefix = dict(prefix_groups=max(1, B // 3), prefix_pages=2) if share else {}
    if not share and data.draw(st.booleans()):  # allocations drawn directly, zero pages included
        prefix = dict(alloc=[data.draw(st.integers(0, 3)) for _ in range(B)])
    params = dict(SW.PARAMS_DEFAULT, n_local=n_local, policy=policy)
    wl = SW.direct_case(seed=seed, B=B, L=1, Hq=8, Hkv=2, d=64, P=P, ctx=(1, 120), spare_pages=spare,
                        grow_frac=grow_frac, fill=fill, params=params, **prefix)
    # the generated state is itself consistent
    assert np.array_equal(_references(wl.page_table, wl.n_alloc, wl.num_pages), wl.refcount)
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, params)
    for name in ("grows", "grow_denied", "deferred", "cow_pages", "freed_pages", "shrinks"):
        if res.counters.get(name, 0):
            event(name)

    # references, refcounts and the free stack
    refs = _references(res.page_table, res.n_alloc, wl.num_pages)
    assert np.array_equal(refs, res.refcount)
    free = res.free_stack[: res.free_top]
    assert np.unique(free).size == free.size and np.all(res.refcount[free] == 0)
    assert res.free_top + np.count_nonzero(refs) == wl.num_pages

    top0 = wl.free_top
    rank = 0
    grown = int(sum(1 for b in range(B) if res.decision[b] == O.DECISION_GROW
                    and not res.status[b] & (O.REQ_NOT_AT_BOUNDARY | O.REQ_DEFERRED)))
    cow_rank = 0  # copy-on-write pages pop after every grow, in batch order and page order
    for b in range(B):
        A, n = int(wl.n_alloc[b]), wl.n(b)
        status, dec = int(res.status[b]), int(res.decision[b])
        untouched = (status & (O.REQ_NOT_AT_BOUNDARY | O.REQ_DEFERRED)) != 0
        if fill[b] < P:
            assert status & O.REQ_NOT_AT_BOUNDARY
        if untouched:
            assert np.array_equal(res.page_table[b], wl.page_table[b])
            assert res.n_alloc[b] == A and res.fill[b] == wl.fill[b] and b not in res.k_new
            continue
        assert res.fill[b] == 0
        if status & O.REQ_GROW_DENIED:
            assert dec != O.DECISION_GROW
        if dec == O.DECISION_GROW:
            # the write page joins the allocation; the new write page is the next stack pop
            assert res.n_alloc[b] == A + 1 and b not in res.k_new
            assert np.array_equal(res.page_table[b, : A + 1], wl.page_table[b, : A + 1])
            assert res.page_table[b, A + 1] == wl.free_stack[top0 - 1 - rank]
            rank += 1
            continue
        # R16: only a request holding two or more allocation pages shrinks
        assert dec == O.DECISION_COMPACT or (policy == "shrink" and dec == O.DECISION_SHRINK and A >= 2)
        shrinks = dec == O.DECISION_SHRINK
        k = (A - 1) * P if shrinks else A * P
        assert res.n_alloc[b] == (A - 1 if shrinks else A)
        ev = res.evicted[b]
        assert ev.shape == (1, 2, n - k)
        for g in range(2):
            kept = np.setdiff1d(np.arange(n), ev[0, g])
            assert kept.size == k
            assert np.array_equal(res.k_new[b][0, g], wl.k_rows[b][0, g][kept])
            assert np.array_equal(res.v_new[b][0, g], wl.v_rows[b][0, g][kept])
            # the most recent slots survive
            nl = min(n_local, k)
            assert np.all(np.isin(np.arange(n - nl, n), kept))
        # R7: a page shared at the start of the step (refcount > 1) whose rows the compaction
        # changes gets a fresh page from the stack; every other page keeps its id
        for j in range(int(res.n_alloc[b])):
            rows = slice(j * P, (j + 1) * P)
            changed = not (np.array_equal(res.k_new[b][:, :, rows], wl.k_rows[b][:, :, rows])
                           and np.array_equal(res.v_new[b][:, :, rows], wl.v_rows[b][:, :, rows]))
            old_id = wl.page_table[b, j]
            if changed and wl.refcount[old_id] > 1:
                assert res.page_table[b, j] == wl.free_stack[top0 - 1 - grown - cow_rank], (b, j)
                cow_rank += 1
            else:
                assert res.page_table[b, j] == old_id, (b, j)
        # the write page stays the write page (after the released page under SHRINK)
        assert res.page_table[b, res.n_alloc[b]] == wl.page_table[b, A]
    assert rank == grown
    # pages whose last reference went are pushed in ascending id order after all pops
    freed = np.flatnonzero((wl.refcount > 0) & (res.refcount == 0))
    base = top0 - grown - cow_rank
    assert res.free_top == base + freed.size
    assert np.array_equal(res.free_stack[:base], wl.free_stack[:base])
    assert np.array_equal(res.free_stack[base: res.free_top], freed)

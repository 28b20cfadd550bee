"""Pins of the CPU oracle to things other than itself: closed forms, special cases,
brute force on tiny inputs and invariants.  CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle as O
from synth import workloads as SW

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- EMA (R3)
@pytest.mark.parametrize("beta", [0.9, 0.999, 0.5])
def test_ema_closed_form_constant_query(beta):
    """Constant q from zero gives s_t = (1 - beta^t) q (within the float32 rounding of t steps)."""
    rng = np.random.default_rng(1)
    q = rng.standard_normal(64).astype(np.float32)
    s = np.zeros(64, np.float32)
    for t in range(1, 201):
        s = O.ema_update(s, q, beta)
        b = float(np.float32(beta))
        want = (1.0 - b ** t) * q.astype(np.float64)
        err = np.abs(s.astype(np.float64) - want)
        assert np.all(err <= (t + 1) * 2.0 ** -23 * np.abs(q) * 2), (t, err.max())


def test_ema_special_cases():
    rng = np.random.default_rng(2)
    s0 = rng.standard_normal(32).astype(np.float32)
    q = rng.standard_normal(32).astype(np.float32)
    assert np.array_equal(O.ema_update(s0, q, 0.0), q)          # beta 0: the last query
    assert np.array_equal(O.ema_update(s0, q, 1.0), s0)         # beta 1: frozen
    # beta 1/2 with values whose halves and sums are exact in float32
    assert np.array_equal(O.ema_update(np.float32([1.0, -6.0]), np.float32([3.0, 2.0]), 0.5),
                          np.float32([2.0, -2.0]))
    assert O.ema_update(s0, q, 0.9).dtype == np.float32


def test_ema_one_minus_beta_is_float32_difference():
    """(1 - beta) is formed in float32: with s = 0 and q = 1 the first update is exactly
    1 - float32(beta), which for beta = 0.999 differs from float32(0.001)."""
    one = np.ones(1, np.float32)
    out = O.ema_update(np.zeros(1, np.float32), one, 0.999)[0]
    assert out == np.float32(1.0) - np.float32(0.999)
    assert out != np.float32(0.001)


def test_ema_run_matches_stepwise_and_bias():
    """With beta_S = beta_L the two summaries coincide; the short one forgets faster."""
    rng = np.random.default_rng(3)
    qs = rng.standard_normal((50, 3, 16)).astype(np.float32)
    s, l_ = O.ema_run(qs, "f32", 0.9, 0.9)
    assert np.array_equal(s, l_)
    s, l_ = O.ema_run(np.ones((32, 1, 4), np.float32), "f32", 0.9, 0.999)
    # closed forms 1 - 0.9^32 and 1 - 0.999^32
    assert abs(float(s[0, 0]) - (1 - 0.9 ** 32)) < 1e-5
    assert abs(float(l_[0, 0]) - (1 - 0.999 ** 32)) < 1e-5


# ----------------------------------------------------------------------------- stored values
# bf16 bit patterns with the values IEEE-754 binary16-brain fixes for them: sign, 8
# exponent bits (bias 127), 7 fraction bits; exponent 0 is the subnormal range.
BF16_VALUES = [
    (0x3F80, 1.0),
    (0xC000, -2.0),
    (0x3FC0, 1.5),
    (0x4049, 3.140625),
    (0xBF00, -0.5),
    (0x0001, 2.0 ** -133),                          # smallest subnormal: 2^-126 * 2^-7
    (0x007F, 127 * 2.0 ** -133),                    # largest subnormal
    (0x0080, 2.0 ** -126),                          # smallest normal
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),       # largest finite
    (0xFF7F, -(2.0 - 2.0 ** -7) * 2.0 ** 127),
    (0x0000, 0.0),
]


@pytest.mark.parametrize("fn", ["widen", "query_f32"])
def test_bf16_bit_patterns_decode_to_their_values(fn):
    """Stored bf16 keys and values (widen) and bf16 decode queries (query_f32) decode to the
    values their bit patterns define, subnormals and the extremes included."""
    bits = np.array([b for b, _ in BF16_VALUES], np.uint16)
    want = np.array([v for _, v in BF16_VALUES], np.float64)
    got = getattr(O, fn)(bits, "bf16").astype(np.float64)
    assert np.array_equal(got, want), (got, want)
    neg0 = getattr(O, fn)(np.array([0x8000], np.uint16), "bf16")
    assert neg0[0] == 0.0 and np.signbit(neg0[0])
    inf = getattr(O, fn)(np.array([0x7F80, 0xFF80], np.uint16), "bf16")
    assert inf[0] == np.inf and inf[1] == -np.inf
    assert np.isnan(getattr(O, fn)(np.array([0x7FC0], np.uint16), "bf16")[0])


def test_widen_and_query_keep_float32_values():
    """float32 storage is taken as it is (widen to float64 exactly, queries unchanged)."""
    x = np.array([1.0, -2.5, 2.0 ** -149, 3.4028234663852886e38, 1.0 + 2.0 ** -23], np.float32)
    assert np.array_equal(O.widen(x, "f32"), x.astype(np.float64))
    assert O.widen(x, "f32").dtype == np.float64
    q = O.query_f32(x, "f32")
    assert q.dtype == np.float32 and np.array_equal(q.view(np.uint32), x.view(np.uint32))


def test_bf16_widening_is_the_top_half_of_float32():
    """Every bf16 pattern equals the float32 whose upper 16 bits it is (lower bits zero):
    checked on all 65536 patterns through float32 rounding of the float64 value."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):          # the NaN patterns
        w = O.widen(bits, "bf16")
        q = O.query_f32(bits, "bf16")
    f = w.astype(np.float32)
    ok = ~np.isnan(w)
    assert np.array_equal((f.view(np.uint32)[ok] >> 16).astype(np.uint16), bits[ok])
    assert np.array_equal(f.view(np.uint32)[ok] & 0xFFFF, np.zeros(int(ok.sum()), np.uint32))
    assert np.array_equal(q.view(np.uint32)[ok], f.view(np.uint32)[ok])


@pytest.mark.parametrize("beta", [0.9, 0.999])
def test_ema_run_constant_bf16_query_closed_form(beta):
    """A constant bf16 query from zero gives s_t = (1 - beta^t) q for the query's decoded
    value q (closed form, within the float32 rounding of t steps): pins the bf16 branch
    of the summaries' input."""
    bits = np.array([0x3F80, 0xC040, 0x4049, 0x3D4D, 0xBB80], np.uint16)     # 1, -3, 3.140625, ~0.0501, ~-0.0039
    q = np.array([1.0, -3.0, 3.140625, 0.050048828125, -0.00390625])
    T = 64
    queries = np.broadcast_to(bits, (T, bits.size)).copy()
    s, l_ = O.ema_run(queries, "bf16", beta, 0.5)
    b = float(np.float32(beta))
    want = (1.0 - b ** T) * q
    assert np.all(np.abs(s.astype(np.float64) - want) <= (T + 1) * 2.0 ** -22 * np.abs(q)), (s, want)
    want_l = (1.0 - 0.5 ** T) * q
    assert np.all(np.abs(l_.astype(np.float64) - want_l) <= (T + 1) * 2.0 ** -22 * np.abs(q))


# ----------------------------------------------------------------------------- RoPE (R4)
def test_rope_identity_and_quarter_turn():
    rng = np.random.default_rng(4)
    s = rng.standard_normal(8)
    assert np.array_equal(O.rope_rotate(s, None, None), s)
    assert np.array_equal(O.rope_rotate(s, np.ones(4), np.zeros(4)), s)
    # quarter turn on every pair: (x1, x2) -> (-x2, x1)
    out = O.rope_rotate(s, np.zeros(4), np.ones(4))
    assert np.array_equal(out, np.concatenate([-s[4:], s[:4]]))


def test_rope_norm_and_angle_addition():
    rng = np.random.default_rng(5)
    d = 64
    cos, sin = SW.rope_tables(300, d, theta=10000.0)
    s = rng.standard_normal(d)
    for pos in (0, 1, 17, 299):
        out = O.rope_rotate(s, cos[pos], sin[pos])
        assert abs(np.linalg.norm(out) - np.linalg.norm(s)) < 1e-6 * np.linalg.norm(s)
    assert np.allclose(O.rope_rotate(s, cos[0], sin[0]), s, rtol=0, atol=0)
    # rotating by positions a then b equals rotating by a + b (angles add), which fixes
    # the sign convention of the pair rotation
    a, b = 37, 101
    two = O.rope_rotate(O.rope_rotate(s, cos[a], sin[a]), cos[b], sin[b])
    one = O.rope_rotate(s, cos[a + b], sin[a + b])
    assert np.allclose(two, one, atol=1e-5)


# ----------------------------------------------------------------------------- logits / softmax
def test_logits_scale_and_layout():
    d = 16
    qt = np.zeros((2, d))
    qt[0, 0] = math.sqrt(d)
    qt[1, 3] = 2 * math.sqrt(d)
    k = np.zeros((5, d))
    k[:, 0] = np.arange(5)
    k[:, 3] = -1.0
    lg = O.logits(qt, k)
    assert lg.shape == (2, 5)
    assert np.allclose(lg[0], np.arange(5))
    assert np.allclose(lg[1], -2.0)


def test_softmax_uniform_and_shift():
    M, Z, a = O.softmax_stats(np.full((1, 10), 3.5))
    assert M[0] == 3.5 and Z[0] == 10.0 and np.allclose(a, 0.1)
    rng = np.random.default_rng(6)
    lg = rng.standard_normal((3, 50))
    _, _, a1 = O.softmax_stats(lg)
    _, _, a2 = O.softmax_stats(lg + 100.0)
    assert np.allclose(a1, a2) and np.allclose(a1.sum(-1), 1.0)


# ----------------------------------------------------------------------------- working set (R1)
def test_working_set_uniform_is_ceil_pn():
    for n, p in [(100, 0.905), (80, 0.853), (1000, 0.9004), (37, 0.51)]:
        a = np.full(n, 1.0 / n)
        W, lo, hi = O.working_set(a, p)
        assert W == math.ceil(p * n), (n, p, W)
        assert lo == hi == W          # far from a tie


def test_working_set_uniform_exact_tie_is_flagged():
    """n = 80 and p = float32(0.9): p*n sits on an integer, a near-tie by construction."""
    n = 80
    p = float(np.float32(0.9))
    W, lo, hi = O.working_set(np.full(n, 1.0 / n), p)
    assert lo <= 72 <= hi and lo != hi
    assert W in (72, 73)


def test_working_set_one_hot():
    lg = np.zeros(500)
    lg[123] = 60.0
    _, _, a = O.softmax_stats(lg[None])
    assert O.working_set(a[0], 0.9)[0] == 1
    assert O.working_set(a[0], 0.99)[0] == 1


@pytest.mark.parametrize("s,n,p", [(1.1, 1000, 0.9), (0.8, 500, 0.9), (1.6, 4000, 0.99), (2.0, 64, 0.5)])
def test_working_set_zipf_closed_form(s, n, p):
    """a_i proportional to i^-s: W = min m with H_{m,s} / H_{n,s} >= p (generalised harmonic numbers)."""
    ranks = np.arange(1, n + 1, dtype=np.float64)
    lg = -s * np.log(ranks)
    rng = np.random.default_rng(7)
    lg = lg[rng.permutation(n)]
    _, _, a = O.softmax_stats(lg[None])
    H = [0.0]
    for i in range(1, n + 1):
        H.append(math.fsum([H[-1], i ** -s]))
    Hn = H[n]
    want = next(m for m in range(1, n + 1) if H[m] / Hn >= p)
    W, lo, hi = O.working_set(a[0], p)
    assert lo <= want <= hi
    if lo == hi:
        assert W == want


def test_working_set_brute_force_small():
    """For n <= 10 the smallest subset reaching mass p (over all 2^n subsets) has W elements."""
    rng = np.random.default_rng(8)
    for trial in range(200):
        n = int(rng.integers(1, 11))
        a = rng.exponential(size=n) ** rng.uniform(0.5, 3)
        a /= a.sum()
        p = float(rng.uniform(0.05, 0.999))
        best = n
        for m in range(1, n + 1):
            if any(sum(a[list(c)]) >= p for c in itertools.combinations(range(n), m)):
                best = m
                break
        W, lo, hi = O.working_set(a, p)
        assert lo <= best <= hi, (a, p)
        if lo == hi:
            assert W == best


def test_working_set_mass_exactly_p_counts():
    """R1 asks for the smallest set whose mass reaches p (>=, not >): with dyadic masses
    every partial sum is exact, so a prefix summing to exactly p ends the set there."""
    a = np.array([0.125, 0.5, 0.125, 0.25])
    assert O.working_set(a, 0.75)[0] == 2
    assert O.working_set(a, 0.5)[0] == 1
    assert O.working_set(a, 0.875)[0] == 3


def test_working_set_limits_and_monotone():
    rng = np.random.default_rng(9)
    a = rng.exponential(size=300)
    a /= a.sum()
    assert O.working_set(a, 1.0)[0] == 300
    assert O.working_set(a, 1.5)[0] == 300
    assert O.working_set(a, 0.0)[0] == 1
    ws = [O.working_set(a, p)[0] for p in np.linspace(0.01, 0.999, 60)]
    assert all(x <= y for x, y in zip(ws, ws[1:]))
    assert O.working_set(np.zeros(0), 0.9) == (0, 0, 0)


def test_scan_query_heads_share_their_group_kv_head():
    """Grouped-query attention: query head h reads KV head h // G.  KV head 0 holds equal
    keys (uniform weights, W = ceil(p n)), KV head 1 one dominant key (W = 1), so the
    first G query heads see ceil(p n) and the rest 1."""
    L, Hkv, G, n, d, p = 1, 2, 3, 40, 8, 0.9
    k = np.zeros((L, Hkv, n, d), np.float32)
    k[0, 1, 7, 0] = 1000.0
    summ = np.zeros((L, Hkv * G, d), np.float32)
    summ[..., 0] = 1.0
    W, lo, hi, M, Z, _ = O.scan_request(k, "f32", summ, summ, None, None, p)
    assert (W[0, :G] == 36).all() and (W[0, G:] == 1).all()


# ----------------------------------------------------------------------------- decision (R2)
def test_decide_sign_and_tau():
    ws = np.array([[10, 20], [30, 40]])
    wl = np.array([[10, 20], [30, 39]])
    assert O.decide(ws, wl, 0) == (1, O.DECISION_GROW)
    assert O.decide(ws, wl, 1) == (1, O.DECISION_COMPACT)
    assert O.decide(wl, ws, 0) == (-1, O.DECISION_COMPACT)
    assert O.decide(ws, ws, 0) == (0, O.DECISION_COMPACT)      # a tie compacts


def test_equal_betas_always_compact():
    """beta_S == beta_L makes the two summaries identical, so delta = 0 and every request compacts."""
    wl = SW.config1(seed=1001)
    s, l_ = O.ema_run(wl.queries, wl.q_dtype, 0.9, 0.9)
    res = O.boundary_step(wl, s, l_, wl.params)
    assert res.delta[0] == 0 and res.decision[0] == O.DECISION_COMPACT


def test_delta_range_hand_built():
    """delta = sum(W_S - W_L); the near-tie range pairs each short size's low end with the
    long size's high end and the other way round (hand-computed integers)."""
    # [L=2][Hq=2][2]: (short, long)
    W = np.array([[[5, 3], [7, 4]], [[2, 6], [9, 9]]])
    Wlo = np.array([[[4, 3], [7, 2]], [[2, 5], [8, 9]]])
    Whi = np.array([[[6, 3], [9, 5]], [[3, 6], [9, 10]]])
    d, lo, hi = O.delta_range(W, Wlo, Whi)
    assert d == (5 - 3) + (7 - 4) + (2 - 6) + (9 - 9) == 1
    assert lo == (4 - 3) + (7 - 5) + (2 - 6) + (8 - 10) == -3
    assert hi == (6 - 3) + (9 - 2) + (3 - 5) + (9 - 9) == 8
    # no near-tie anywhere: the range collapses to delta
    assert O.delta_range(W, W, W) == (1, 1, 1)
    # one long working set uncertain by one: the range widens by one on each side
    lo1, hi1 = W.copy(), W.copy()
    lo1[1, 0, 1] -= 1
    hi1[1, 0, 1] += 1
    assert O.delta_range(W, lo1, hi1) == (1, 0, 2)


def test_delta_range_brackets_every_alternative():
    """Every choice of sizes inside [W_lo, W_hi] gives a delta inside the range, and both
    ends are reached (brute force over a small random case)."""
    rng = np.random.default_rng(12)
    W = rng.integers(3, 9, size=(1, 3, 2))
    Wlo = W - rng.integers(0, 2, size=W.shape)
    Whi = W + rng.integers(0, 2, size=W.shape)
    d, lo, hi = O.delta_range(W, Wlo, Whi)
    seen = set()
    for choice in itertools.product(*[range(int(a), int(b) + 1) for a, b in zip(Wlo.ravel(), Whi.ravel())]):
        c = np.array(choice).reshape(W.shape)
        seen.add(int((c[..., 0] - c[..., 1]).sum()))
    assert min(seen) == lo and max(seen) == hi and lo <= d <= hi


def test_importance_orders_deep_tail_by_value():
    """Slots 110-130 nats below the row maximum keep their order: their probabilities
    (about 1e-48 to 1e-57) are far above float64's range end, so keep-sets rank them by
    value, not by age.  One row: ordering by probability is ordering by logit, so the
    evicted slots are exactly the E lowest logits (closed form)."""
    rng = np.random.default_rng(13)
    n, E = 200, 16
    lg = rng.uniform(0.0, 2.0, n)
    deep = rng.choice(n - 8, 40, replace=False)
    lg[deep] = -110.0 - 20.0 * rng.permutation(40) / 40.0   # distinct, 0.5 nat apart
    _, _, a = O.softmax_stats(lg[None])
    imp = O.importance(a)
    assert np.all(imp[deep] > 0) and np.unique(imp[deep]).size == 40
    kept, ev, near = O.keep_set(imp, n - E, 8)
    assert not near
    assert np.array_equal(ev, np.sort(np.argsort(lg)[:E]))
    # the probabilities themselves: exp(l - M) / Z within float64 rounding
    M = lg.max()
    Z = math.fsum(math.exp(v - M) for v in lg)
    for i in deep[:5]:
        assert abs(imp[i] / (math.exp(lg[i] - M) / Z) - 1.0) < 1e-12


# ----------------------------------------------------------------------------- keep-set (R5, R6)
def test_keep_set_invariants_random():
    rng = np.random.default_rng(10)
    for _ in range(100):
        n = int(rng.integers(2, 200))
        k = int(rng.integers(1, n + 1))
        nl = int(rng.integers(0, n + 2))
        imp = rng.exponential(size=n)
        kept, ev, near = O.keep_set(imp, k, nl)
        assert kept.size == k and ev.size == n - k
        assert np.array_equal(np.sort(np.concatenate([kept, ev])), np.arange(n))
        assert np.all(np.diff(kept) > 0)
        local = np.arange(n - min(nl, k), n)
        assert np.all(np.isin(local, kept))
        nonlocal_kept = np.setdiff1d(kept, local)
        if ev.size and nonlocal_kept.size:
            assert imp[nonlocal_kept].min() >= imp[ev].max()
        assert O.keep_set_valid(ev, imp, k, nl)


def test_keep_set_brute_force_small():
    """Top-(k - local) by importance equals the candidate subset with the largest total importance."""
    rng = np.random.default_rng(11)
    for _ in range(100):
        n = int(rng.integers(2, 11))
        k = int(rng.integers(1, n + 1))
        nl = int(rng.integers(0, 3))
        imp = rng.uniform(size=n)
        nle = min(nl, k)
        cand = n - nle
        best = max(itertools.combinations(range(cand), k - nle), key=lambda c: sum(imp[list(c)]))
        want = sorted(list(best) + list(range(cand, n)))
        kept, _, _ = O.keep_set(imp, k, nl)
        assert list(kept) == want


def test_keep_set_ties_keep_recent():
    imp = np.full(40, 0.025)
    kept, ev, near = O.keep_set(imp, 30, 0)
    assert list(ev) == list(range(10))          # the oldest slots go first
    assert list(kept) == list(range(10, 40))
    # equal importance except one old heavy slot, which survives
    imp[2] = 0.5
    kept, ev, _ = O.keep_set(imp, 30, 4)
    assert 2 in kept and list(ev) == [0, 1, 3, 4, 5, 6, 7, 8, 9, 10]


def test_keep_set_valid_rejects_wrong_sets():
    imp = np.array([0.5, 0.1, 0.3, 0.05, 0.05])
    kept, ev, _ = O.keep_set(imp, 3, 0)
    assert list(ev) == [3, 4]
    assert O.keep_set_valid(ev, imp, 3, 0)
    assert not O.keep_set_valid(np.array([1, 4]), imp, 3, 0)
    assert not O.keep_set_valid(np.array([3]), imp, 3, 0)


def test_importance_is_max_over_rows():
    a = np.array([[0.1, 0.7, 0.2], [0.6, 0.1, 0.3]])
    assert np.array_equal(O.importance(a), [0.6, 0.7, 0.3])


def test_importance_uses_probabilities_not_logits():
    """R5: importance is the max over rows of softmax probabilities.  Row 0 peaks on slot 0
    (logit 10/sqrt(8) against 0 elsewhere), row 2 is flat over slots 1..7 with larger raw
    logits (20/sqrt(8)); the other rows are uniform.  In probability slot 0 matters most
    (about 0.83 against 1/7), so keeping n - 1 slots evicts slot 1 (an exact tie among
    slots 1..7 goes to the older slot); ranked by raw logits slot 0 would go."""
    n, d = 8, 8
    k = np.zeros((1, 1, n, d), np.float32)
    k[0, 0, 0, 0] = 10.0
    k[0, 0, 1:, 1] = 20.0
    s = np.zeros((1, 4, d), np.float32)
    l_ = np.zeros((1, 4, d), np.float32)
    s[0, 0, 0] = 1.0      # head 0, short summary: row 0
    s[0, 1, 1] = 1.0      # head 1, short summary: row 2
    probs = O.scan_request(k, "f32", s, l_, None, None, 0.9, keep_logits=True)[5]
    assert np.allclose(probs[0, 0].sum(axis=-1), 1.0)
    imp = O.importance(probs[0, 0])
    kept, ev, near = O.keep_set(imp, n - 1, 0)
    assert ev.tolist() == [1]
    assert imp[0] > 0.8 and abs(imp[1] - 1.0 / 7.0) < 1e-3


def test_compaction_is_stable_gather():
    rows = np.arange(20 * 3).reshape(20, 3)
    kept = np.array([0, 2, 3, 7, 19])
    out = O.compact_rows(rows, kept)
    assert np.array_equal(out, rows[kept])
    # a multiset of original rows, in original order
    assert all(tuple(r) in {tuple(x) for x in rows} for r in out)


# ----------------------------------------------------------------------------- whole step
def _pool_invariants(res, wl):
    """refcount == number of page-table references; free stack and referenced pages
    partition the pool; no duplicates anywhere."""
    refs = np.zeros(wl.num_pages, np.int64)
    for b in range(wl.B):
        for j in range(int(res.n_alloc[b]) + 1):
            refs[res.page_table[b, j]] += 1
    assert np.array_equal(refs, res.refcount)
    free = res.free_stack[: res.free_top]
    assert np.unique(free).size == free.size
    assert np.all(refs[free] == 0)
    assert free.size + np.count_nonzero(refs) == wl.num_pages


def test_config1_planted_compaction():
    wl = SW.config1()
    s, l_ = O.ema_run(wl.queries, wl.q_dtype, wl.params["beta_s"], wl.params["beta_l"])
    res = O.boundary_step(wl, s, l_, wl.params)
    # sharp short summary, flat long one: the recent working set is the smaller
    assert np.all(res.W[0, 0, :, 0] < res.W[0, 0, :, 1])
    assert res.decision[0] == O.DECISION_COMPACT and not res.ambiguous[0]
    assert res.evicted[0].shape == (1, 2, 16)
    assert res.fill[0] == 0 and res.n_alloc[0] == 4
    _pool_invariants(res, wl)
    # the 4 heavy hitters survive
    k = wl.k_rows[0][0, 0]
    hh = [i for i in range(80) if np.linalg.norm(k[i]) > 20]
    assert len(hh) == 4
    for g in range(2):
        assert not set(hh) & set(res.evicted[0][0, g].tolist())


def test_grow_pops_in_batch_order_and_denial():
    wl = SW.direct_case(seed=12, B=6, grow_frac=1.0, spare_pages=3)
    assert wl.free_top == 3
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, wl.params)
    grows = [b for b in range(wl.B) if res.decision_raw[b] == O.DECISION_GROW]
    assert len(grows) >= 4
    popped = [res.page_table[b, wl.n_alloc[b] + 1] for b in grows[:3]]
    assert popped == [wl.free_stack[2], wl.free_stack[1], wl.free_stack[0]]
    for b in grows[3:]:
        assert res.status[b] & O.REQ_GROW_DENIED and res.decision[b] == O.DECISION_COMPACT
    _pool_invariants(res, wl)


def test_copy_on_write_prefix_sharing():
    wl = SW.direct_case(seed=13, B=4, grow_frac=0.0, prefix_groups=1, prefix_pages=3,
                        ctx=(60, 120), spare_pages=40, params=dict(SW.PARAMS_DEFAULT, n_local=8))
    assert wl.refcount[wl.page_table[0, 0]] == 4
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, wl.params)
    assert res.counters["cow_pages"] > 0
    _pool_invariants(res, wl)
    for (b, j, old, new) in res.cow:
        assert res.page_table[b, j] == new and new != old
        assert j >= res.e_req[b] // wl.P
    # kept contents equal the original rows in slot order
    for b, kn in res.k_new.items():
        for l in range(wl.L):
            for g in range(wl.Hkv):
                ev = set(res.evicted[b][l, g].tolist())
                kept = [i for i in range(wl.n(b)) if i not in ev]
                assert np.array_equal(kn[l, g], wl.k_rows[b][l, g][kept])


def test_copy_on_write_shortfall_defers():
    wl = SW.direct_case(seed=14, B=3, grow_frac=0.0, prefix_groups=1, prefix_pages=2,
                        ctx=(40, 80), spare_pages=0, params=dict(SW.PARAMS_DEFAULT, n_local=4))
    assert wl.free_top == 0
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, wl.params)
    deferred = 0
    for b in range(wl.B):
        need = [j for j in range(int(res.e_req[b]) // wl.P, int(wl.n_alloc[b]))
                if wl.refcount[wl.page_table[b, j]] > 1]
        if need:
            deferred += 1
            assert res.status[b] & O.REQ_DEFERRED
            assert b not in res.k_new and res.fill[b] == wl.P
            assert np.array_equal(res.page_table[b], wl.page_table[b])
        else:
            assert b in res.k_new
    assert deferred > 0
    _pool_invariants(res, wl)


def test_not_at_boundary_is_untouched():
    wl = SW.direct_case(seed=15, B=3, fill=[16, 5, 16])
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, wl.params)
    assert res.status[1] & O.REQ_NOT_AT_BOUNDARY
    assert res.fill[1] == 5 and 1 not in res.k_new


def test_paper_hyperparameters_fixture():
    g = json.load(open(os.path.join(GOLDEN, "paper_hparams.json")))
    assert SW.PARAMS_PAPER["beta_s"] == g["beta_s"] and SW.PARAMS_PAPER["beta_l"] == g["beta_l"]
    assert SW.PARAMS_PAPER["top_p"] == g["top_p"] and SW.PARAMS_PAPER["tau"] == g["tau"]
    assert SW.PARAMS_PAPER["n_local"] == g["local_retention_quota"]


# ----------------------------------------------------------------------------- decode loop
def _tiny_loop(P=4, A=2, d=8, Hq=4, beta_s=0.9, top_p=0.9, n_local=0, seed=0):
    """One request, one layer, one KV head, f32 rows; the write page starts empty."""
    rng = np.random.default_rng(seed)
    n = A * P
    k = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    num_pages = 8
    table = np.full((1, 6), -1, np.int64)
    table[0, : A + 1] = np.arange(A + 1)
    rc = np.zeros(num_pages, np.int64)
    rc[: A + 1] = 1
    stack = np.zeros(num_pages, np.int64)
    stack[: num_pages - A - 1] = np.arange(A + 1, num_pages)
    prm = dict(beta_s=beta_s, beta_l=0.999, top_p=top_p, tau=0, n_local=n_local)
    st = O.LoopState(1, Hq, 1, d, P, "f32", num_pages, table, np.array([A]), np.array([0]), rc, stack,
                     num_pages - A - 1, [k], [v], np.zeros((1, 1, Hq, d), np.float32),
                     np.zeros((1, 1, Hq, d), np.float32), np.array([n]), None, None)
    return st, prm


def test_decode_boundary_fires_when_write_page_fills_and_scans_new_token():
    """p = 1 makes W = n exactly (R1), so W tells how many slots the scan saw: the boundary
    comes on the P-th append and its scan includes that step's row (R6)."""
    P, A, d = 4, 2, 8
    st, prm = _tiny_loop(P, A, d, top_p=1.0)
    rng = np.random.default_rng(1)
    for t in range(P):
        q = rng.standard_normal((1, 1, 4, d)).astype(np.float32)
        kn = rng.standard_normal((1, 1, 1, d)).astype(np.float32)[:, :, 0]
        app, idx, sub, res = O.decode_step(st, q, "f32", kn[None], kn[None], prm)
        assert app.all()
        if t < P - 1:
            assert res is None and st.fill[0] == t + 1
    assert list(idx) == [0]
    assert np.all(res.W == (A + 1) * P)
    assert res.decision[0] == O.DECISION_COMPACT          # delta = 0 with W = n on both sides
    assert st.fill[0] == 0 and st.k_rows[0].shape[2] == A * P
    assert st.pos[0] == A * P + P                          # one position per step


def test_decode_summaries_absorb_the_query_before_the_scan():
    """With beta_S = 0 the short summary is the step's query (R3).  The last query points at
    a key planted far out, so the short working set is 1 only if the boundary scan sees the
    summary after this step's update."""
    P, A, d = 4, 2, 8
    st, prm = _tiny_loop(P, A, d, beta_s=0.0, top_p=0.5)
    u = np.zeros(d, np.float32)
    u[0] = 1.0
    st.k_rows[0][0, 0, 3] = 40.0 * u                      # a key along u at slot 3
    zero = np.zeros((1, 1, 1, d), np.float32)
    for t in range(P):
        q = np.zeros((1, 1, 4, d), np.float32)
        if t == P - 1:
            q[:] = 4.0 * u                                 # only the last query points at it
        app, idx, sub, res = O.decode_step(st, q, "f32", zero[:, :, 0][None], zero[:, :, 0][None], prm)
    assert res is not None
    assert np.all(res.W[0, 0, :, 0] == 1)


def test_decode_full_write_page_takes_nothing():
    P, A, d = 4, 2, 8
    st, prm = _tiny_loop(P, A, d)
    st.fill[0] = P
    st.k_rows[0] = np.concatenate([st.k_rows[0], np.zeros((1, 1, P, d), np.float32)], axis=2)
    st.v_rows[0] = np.concatenate([st.v_rows[0], np.zeros((1, 1, P, d), np.float32)], axis=2)
    before = st.k_rows[0].copy()
    assert not O.append_token(st, 0, np.ones((1, 1, d), np.float32), np.ones((1, 1, d), np.float32))
    assert st.fill[0] == P and np.array_equal(st.k_rows[0], before)


def test_decode_compaction_keeps_a_stable_subset():
    P, A, d = 4, 3, 8
    st, prm = _tiny_loop(P, A, d, seed=3)
    rng = np.random.default_rng(4)
    rows_seen = None
    for t in range(P):
        q = rng.standard_normal((1, 1, 4, d)).astype(np.float32) * 3
        kn = rng.standard_normal((1, 1, d)).astype(np.float32)
        if t == P - 1:
            rows_seen = np.concatenate([st.k_rows[0], kn[None, :, :, None, :][0]], axis=2).copy()
        app, idx, sub, res = O.decode_step(st, q, "f32", kn[None], kn[None], prm)
    assert res.decision[0] == O.DECISION_COMPACT or st.n_alloc[0] == A + 1
    if res.decision[0] == O.DECISION_COMPACT:
        kept = np.setdiff1d(np.arange((A + 1) * P), res.evicted[0][0, 0])
        assert np.array_equal(st.k_rows[0][0, 0], rows_seen[0, 0][kept])
        assert st.k_rows[0].shape[2] == A * P


# ----------------------------------------------------------------------------- decision policies
def test_policy_rules():
    """The ablation policies as read: inverse grows iff -delta > tau, random iff its draw is
    below the grow probability (strictly), always_compact never; ties compact throughout."""
    for d in (-5, -1, 0, 1, 7):
        for tau in (0, 2):
            assert O.policy_decision(d, tau, "growpage") == (d > tau)
            assert O.policy_decision(d, tau, "inverse") == (-d > tau)
            assert O.policy_decision(d, tau, "always_compact") == O.DECISION_COMPACT
    assert O.policy_decision(0, 0, "growpage") == O.policy_decision(0, 0, "inverse") == O.DECISION_COMPACT
    for u, rho, want in ((0.0, 0.0, 0), (0.999, 1.0, 1), (0.3, 0.3, 0), (0.29, 0.3, 1)):
        assert O.policy_decision(100, 0, "random", u, rho) == want
    for d in (-5, -1, 0, 1, 7):
        for tau in (0, 2):
            want = O.DECISION_GROW if d > tau else O.DECISION_SHRINK
            assert O.policy_decision(d, tau, "shrink") == want
    with pytest.raises(ValueError):
        O.policy_decision(1, 0, "grow_always")


def test_boundary_step_follows_the_policy():
    wl = SW.direct_case(seed=77, B=6, L=1, Hq=8, Hkv=2, d=64, P=16, grow_frac=0.5, spare_pages=64)
    base = O.boundary_step(wl, wl.sum_s, wl.sum_l, wl.params)
    assert 0 < base.decision.sum() < wl.B
    inv = O.boundary_step(wl, wl.sum_s, wl.sum_l, dict(wl.params, policy="inverse"))
    assert np.array_equal(inv.delta, base.delta)
    assert np.array_equal(inv.decision, (-base.delta > 0).astype(inv.decision.dtype))
    never = O.boundary_step(wl, wl.sum_s, wl.sum_l, dict(wl.params, policy="always_compact"))
    assert never.decision.sum() == 0 and never.counters["compacts"] == wl.B
    u = np.array([0.1, 0.9, 0.5, 0.2, 0.7, 0.05], np.float32)
    rnd = O.boundary_step(wl, wl.sum_s, wl.sum_l, dict(wl.params, policy="random", rand_u=u, grow_prob=0.3))
    assert np.array_equal(rnd.decision, (u < np.float32(0.3)).astype(rnd.decision.dtype))


def _shrink_checks(wl, res, b, n_local):
    """A request that shrank (R16): one allocation page fewer, the write page in the
    released page's table slot, (A-1) P slots kept by the keep-set rule and packed in
    slot order, the local window kept, the write page emptied."""
    A, P, n = int(wl.n_alloc[b]), wl.P, wl.n(b)
    assert res.decision[b] == O.DECISION_SHRINK and res.n_alloc[b] == A - 1 and res.fill[b] == 0
    assert res.page_table[b, A - 1] == wl.page_table[b, A]
    k = (A - 1) * P
    assert res.evicted[b].shape[-1] == n - k and res.k_new[b].shape[2] == k
    for l in range(wl.L):
        for g in range(wl.Hkv):
            ev = res.evicted[b][l, g]
            assert O.keep_set_valid(ev, res.imp[b][l, g], k, n_local)
            assert ev.size == 0 or ev.max() < n - min(n_local, k)
            kept = np.setdiff1d(np.arange(n), ev)
            assert np.array_equal(res.k_new[b][l, g], wl.k_rows[b][l, g][kept])
            assert np.array_equal(res.v_new[b][l, g], wl.v_rows[b][l, g][kept])


def test_shrink_releases_one_page():
    """SHRINK (R16) against GrowPage on the same batch: same deltas and grows; every
    other request at its boundary with two or more allocation pages shrinks by one, and
    a one-page allocation compacts in place; an unshared released page is pushed."""
    n_local = 8
    wl = SW.direct_case(seed=81, B=10, L=2, Hq=8, Hkv=2, d=64, P=16, ctx=(8, 200), grow_frac=0.4,
                        spare_pages=64, params=dict(SW.PARAMS_DEFAULT, n_local=n_local))
    base = O.boundary_step(wl, wl.sum_s, wl.sum_l, wl.params)
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, dict(wl.params, policy="shrink"))
    assert np.array_equal(res.delta, base.delta)
    kinds = set()
    for b in range(wl.B):
        A = int(wl.n_alloc[b])
        if base.decision[b] == O.DECISION_GROW:
            assert res.decision[b] == O.DECISION_GROW and res.n_alloc[b] == A + 1
            kinds.add("grow")
        elif A >= 2:
            _shrink_checks(wl, res, b, n_local)
            released = int(wl.page_table[b, A - 1])
            assert res.refcount[released] == 0 and released in res.free_stack[: res.free_top]
            kinds.add("shrink")
        else:
            assert res.decision[b] == O.DECISION_COMPACT and res.n_alloc[b] == A
            assert res.k_new[b].shape[2] == A * wl.P
            kinds.add("compact")
    assert kinds == {"grow", "shrink", "compact"}
    assert res.counters["shrinks"] == int(np.sum(res.decision == O.DECISION_SHRINK))
    assert res.counters["freed_pages"] == res.counters["shrinks"]
    # pushes come after the pops, in ascending page id
    grows = int(np.sum(res.decision == O.DECISION_GROW))
    pushed = res.free_stack[wl.free_top - grows: res.free_top]
    assert pushed.size == res.counters["shrinks"] and np.all(np.diff(pushed) > 0)
    _pool_invariants(res, wl)


def test_shrink_keeps_shared_pages_alive():
    """Four requests share a 3-page prefix and hold exactly those 3 pages: each shrink
    drops one reference to shared page 2 (pushed only when the last one goes) and copies
    on write the shared pages its compaction changes."""
    wl = SW.direct_case(seed=82, B=4, grow_frac=0.0, prefix_groups=1, prefix_pages=3, ctx=(20, 40),
                        spare_pages=40, params=dict(SW.PARAMS_DEFAULT, n_local=8))
    assert np.all(wl.n_alloc == 3) and wl.refcount[wl.page_table[0, 2]] == 4
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, dict(wl.params, policy="shrink"))
    shared2 = int(wl.page_table[0, 2])
    for b in range(wl.B):
        _shrink_checks(wl, res, b, 8)
        for (bb, j, old, new) in res.cow:
            assert j < 2
    assert res.refcount[shared2] == 0 and shared2 in res.free_stack[: res.free_top]
    assert res.counters["cow_pages"] > 0
    _pool_invariants(res, wl)


def test_shrink_after_a_denied_grow():
    """Under SHRINK a grow the free stack cannot serve shrinks instead (flagged)."""
    wl = SW.direct_case(seed=12, B=6, grow_frac=1.0, spare_pages=3)
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, dict(wl.params, policy="shrink"))
    denied = [b for b in range(wl.B) if res.status[b] & O.REQ_GROW_DENIED]
    assert denied
    for b in denied:
        assert res.decision[b] == (O.DECISION_SHRINK if wl.n_alloc[b] >= 2 else O.DECISION_COMPACT)
    _pool_invariants(res, wl)


# ----------------------------------------------------------------------------- decode attention
def test_decode_attention_closed_forms():
    """Equal scores average the values; one key far ahead returns its value; a shift of
    every score (a query component along a direction all keys share) changes nothing."""
    rng = np.random.default_rng(8)
    n, d = 12, 16
    v = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    k0 = np.zeros((1, 1, n, d), np.float32)
    q = rng.standard_normal((1, 2, d)).astype(np.float32)
    out = O.decode_attention(k0, v, "f32", q, "f32", None, None)
    assert np.allclose(out[0, 0], v[0, 0].mean(axis=0), atol=1e-12)
    k1 = k0.copy()
    k1[0, 0, 5, 0] = 1000.0
    q1 = np.zeros((1, 2, d), np.float32)
    q1[0, :, 0] = 1.0
    out1 = O.decode_attention(k1, v, "f32", q1, "f32", None, None)
    assert np.allclose(out1[0, 1], v[0, 0, 5], atol=1e-9)
    # every key shares the component e_1 = 3; a query along e_1 adds the same score to all
    k2 = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    k2[..., 1] = 3.0
    qa = rng.standard_normal((1, 2, d)).astype(np.float32)
    qa[..., 1] = 0.0
    qb = qa.copy()
    qb[..., 1] = 5.0
    assert np.allclose(O.decode_attention(k2, v, "f32", qa, "f32", None, None),
                       O.decode_attention(k2, v, "f32", qb, "f32", None, None), atol=1e-12)
    assert np.all(O.decode_attention(k2[:, :, :0], v[:, :, :0], "f32", qa, "f32", None, None) == 0)


def test_decode_attention_is_a_convex_combination():
    rng = np.random.default_rng(9)
    k = rng.standard_normal((2, 2, 30, 8)).astype(np.float32)
    v = rng.standard_normal((2, 2, 30, 8)).astype(np.float32)
    q = rng.standard_normal((2, 8, 8)).astype(np.float32) * 3
    out = O.decode_attention(k, v, "f32", q, "f32", None, None)
    for l in range(2):
        for h in range(8):
            g = h // 4
            assert np.all(out[l, h] <= v[l, g].max(axis=0) + 1e-12)
            assert np.all(out[l, h] >= v[l, g].min(axis=0) - 1e-12)


def test_decode_attention_two_keys_closed_form():
    """Two keys whose scores differ by a/sqrt(d): the weights are the logistic of that
    difference, so the output is (e^x v_1 + v_2) / (e^x + 1) with x = a / sqrt(d)."""
    d, a = 16, 3.0
    k = np.zeros((1, 1, 2, d), np.float32)
    k[0, 0, 0, 0] = a
    v = np.random.default_rng(10).standard_normal((1, 1, 2, d)).astype(np.float32)
    q = np.zeros((1, 4, d), np.float32)
    q[0, :, 0] = 1.0
    out = O.decode_attention(k, v, "f32", q, "f32", None, None)
    x = a / math.sqrt(d)
    want = (math.exp(x) * v[0, 0, 0].astype(np.float64) + v[0, 0, 1]) / (math.exp(x) + 1.0)
    assert np.allclose(out[0, 3], want, atol=1e-12)


def test_decode_attention_rotates_the_query_like_the_keys():
    """A key stored rotated to position t scores like an unrotated key when the query is
    rotated to the same position (a rotation preserves dot products), so against a
    second key of score 0 the weights are the logistic of |u|^2 / sqrt(d)."""
    d, t = 16, 37
    cos, sin = SW.rope_tables(64, d)
    u = np.random.default_rng(11).standard_normal(d)
    u /= np.linalg.norm(u)
    u *= 2.0
    h = d // 2
    kr = np.concatenate([u[:h] * cos[t] - u[h:] * sin[t], u[h:] * cos[t] + u[:h] * sin[t]])
    k = np.zeros((1, 1, 2, d), np.float64)
    k[0, 0, 0] = kr
    v = np.random.default_rng(12).standard_normal((1, 1, 2, d))
    q = np.tile(u, (1, 4, 1))
    out = O.decode_attention(k.astype(np.float32), v.astype(np.float32), "f32", q.astype(np.float32), "f32",
                             cos[t], sin[t])
    x = float(np.dot(u.astype(np.float32).astype(np.float64), u.astype(np.float32).astype(np.float64))) / math.sqrt(d)
    v32 = v.astype(np.float32).astype(np.float64)
    want = (math.exp(x) * v32[0, 0, 0] + v32[0, 0, 1]) / (math.exp(x) + 1.0)
    assert np.allclose(out[0, 0], want, atol=1e-5)


def test_empty_request_statistics():
    """Reading R17: a request with no candidate slots has working sets 0, max -inf and
    sum 0 for every row (the identities of max and sum), and is never at a boundary."""
    wl = SW.direct_case(seed=5, B=2, L=1, Hq=8, Hkv=2, d=64, P=16, alloc=[0, 1], fill=[0, 16])
    res = O.boundary_step(wl, wl.sum_s, wl.sum_l, wl.params)
    assert np.all(res.W[0] == 0) and np.all(np.isneginf(res.M[0])) and np.all(res.Z[0] == 0)
    assert res.status[0] & O.REQ_NOT_AT_BOUNDARY and np.all(np.isfinite(res.M[1]))

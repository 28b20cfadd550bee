"""GrowPage capacity-boundary engine: plain CPU oracle in float64.

TEST INFRASTRUCTURE ONLY -- imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.  It shares no code with
the HIP kernels: every step below is written out from the pages' description with
numpy (matmul and sort are the only library primitives), in float64 except where a
reading fixes the precision.

What the pages say (cited by page title and section; the pages carry no formulas):
  [Summary]  GrowPage review on evolve.pub, section "Summary": a request keeps two
             moving averages of its queries (factors 0.9 and 0.999, before RoPE); at
             each capacity boundary of its paged cache each average gets a Top-p
             working-set size; if the fast one's is larger the request receives one
             more physical page, otherwise its older entries are packed into the pages
             it holds, slots ranked by the larger of the two averages' importance.
  [FAQ-impl] Same page, FAQ "Is GrowPage's code available?": beta_S 0.9, beta_L
             0.999, Top-p 0.99, demand threshold tau 0, local retention quota 64,
             KV block 256.
  [Abstract] The paper's abstract (on every page): capacity is a runtime resource;
             at each boundary either compress within the allocation or acquire an
             additional physical page; page-level integration keeps continuous
             batching and prefix caching.

Readings taken where the pages are silent (each repeated where it is used):
  R1  working set W = smallest m whose m largest probabilities sum to >= p;
      p >= 1 gives W = n.
  R2  demand signal: delta = sum over layers and query heads of (W_S - W_L);
      grow iff delta > tau; delta == tau compacts.
  R3  summaries: s <- beta*s + (1-beta)*q from zero, no bias correction, float32,
      multiply and add rounded separately, (1-beta) rounded to float32 first.
  R4  the stored keys are post-RoPE; each pre-RoPE summary is rotated once to the
      request's absolute position (rotate-half pairs i, i+d/2, caller's cos/sin
      table; no table = identity) and scored against every retained key with
      softmax scale 1/sqrt(d).
  R5  importance of a slot for KV head g = max over g's query heads and both
      summaries of the softmax probability.
  R6  write-page model: a request owns A allocation pages plus one write page;
      n = A*P + fill slots are candidates; the boundary is fill == P; grow makes
      the write page part of the allocation and pops a new write page; compact
      keeps k = A*P slots (the last min(n_local, k) always, the rest by importance
      descending, ties to the more recent slot), packs them in slot order into
      slots 0..k-1 and empties the write page.
  R7  pages are shared across layers and heads; a compaction that would change a
      page whose refcount (at the start of the step) exceeds 1 first copies it to
      a fresh page (copy-on-write).  Free pages form a stack: grows pop first in
      batch order, then copy-on-write pages in batch order and ascending page
      index; pages whose refcount reaches zero are pushed in ascending id order at
      the end of the step.  An empty stack turns a grow into a compaction (status
      GROW_DENIED); a request whose copy-on-write demand exceeds the stack is left
      untouched (status DEFERRED).
  R16 SHRINK ablation [same page, "Strengths", item "Frequency-matched causal
      ablations": a policy whose budget can only go down]: grow iff
      delta > tau as GrowPage; every other request at its boundary with A >= 2
      keeps k = (A-1)*P slots by R6's rule in pages 0..A-2, drops its reference to
      allocation page A-1 and moves its write page into that page-table slot; with
      A < 2 it compacts in place.
  R17 Empty request (no allocation pages, empty write page; the pages never meet
      it): its working sets are 0 and each softmax row has max -inf (the max over
      no logits) and sum 0 (the empty sum).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

NEAR_TIE = 1.0e-5          # cumulative-mass / relative-importance band for near-ties
DECISION_COMPACT = 0
DECISION_GROW = 1
DECISION_SHRINK = 2
REQ_GROW_DENIED = 1
REQ_DEFERRED = 2
REQ_NOT_AT_BOUNDARY = 4


# ----------------------------------------------------------------------------- values
def widen(rows: np.ndarray, dtype: str) -> np.ndarray:
    """Stored K/V values as float64: bf16 bit patterns are widened exactly."""
    if dtype == "bf16":
        return (np.asarray(rows, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(rows, np.float32).astype(np.float64)


def query_f32(q: np.ndarray, dtype: str) -> np.ndarray:
    """Decode queries as float32 (bf16 widened exactly)."""
    if dtype == "bf16":
        return (np.asarray(q, np.uint16).astype(np.uint32) << 16).view(np.float32)
    return np.asarray(q, np.float32)


# ----------------------------------------------------------------------------- steps
def ema_update(s: np.ndarray, q: np.ndarray, beta: float) -> np.ndarray:
    """One summary update [Summary: moving averages of the queries; FAQ-impl: factors].

    Reading R3: s <- beta*s + (1-beta)*q in float32, each product and the sum rounded
    on their own; (1-beta) is itself the float32 difference of 1 and float32(beta).
    """
    b = np.float32(beta)
    omb = np.float32(np.float32(1.0) - b)
    prod_s = np.multiply(b, np.asarray(s, np.float32), dtype=np.float32)
    prod_q = np.multiply(omb, np.asarray(q, np.float32), dtype=np.float32)
    return np.add(prod_s, prod_q, dtype=np.float32)


def ema_run(queries: np.ndarray, q_dtype: str, beta_s: float, beta_l: float):
    """Both summaries after feeding ``queries`` [T][...][d] in order from zero (R3)."""
    q = query_f32(queries, q_dtype)
    s = np.zeros(q.shape[1:], np.float32)
    l_ = np.zeros(q.shape[1:], np.float32)
    for t in range(q.shape[0]):
        s = ema_update(s, q[t], beta_s)
        l_ = ema_update(l_, q[t], beta_l)
    return s, l_


def rope_rotate(s: np.ndarray, cos_row: Optional[np.ndarray], sin_row: Optional[np.ndarray]) -> np.ndarray:
    """Rotate pre-RoPE summaries to the request's position [Summary: summaries kept pre-RoPE].

    Reading R4: rotate-half pairs (i, i+d/2): (x1*c - x2*s, x2*c + x1*s), float64.
    """
    s = np.asarray(s, np.float64)
    if cos_row is None:
        return s.copy()
    h = s.shape[-1] // 2
    c = np.asarray(cos_row, np.float64)
    sn = np.asarray(sin_row, np.float64)
    x1, x2 = s[..., :h], s[..., h:]
    return np.concatenate([x1 * c - x2 * sn, x2 * c + x1 * sn], axis=-1)


def logits(qt: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Scores of rotated summaries against every retained key [Summary: working sets
    induced by the summaries]; reading R4: dot product over d, scaled by 1/sqrt(d)."""
    d = k.shape[-1]
    return (np.asarray(qt, np.float64) @ np.asarray(k, np.float64).T) / math.sqrt(d)


def softmax_stats(lg: np.ndarray):
    """Per-row softmax: M = max, Z = sum exp(l - M), a = exp(l - M) / Z."""
    M = lg.max(axis=-1)
    e = np.exp(lg - M[..., None])
    Z = e.sum(axis=-1)
    return M, Z, e / Z[..., None]


def working_set(a: np.ndarray, p: float, band: float = NEAR_TIE):
    """Top-p attention working-set size [Summary: the boundary compares the two
    summaries' Top-p working-set sizes].

    Reading R1: W = min{m >= 1 : sum of the m largest a_i >= p}, full sort, float64
    cumulative sum; p >= 1 gives n.  Also returns the sizes for p -/+ band, which
    bound every answer that differs from W only by rounding at a near-tie.
    """
    n = int(a.size)
    if n == 0:
        return 0, 0, 0
    if p >= 1.0:
        return n, n, n        # R1 fixes this case exactly; no rounding decides it
    c = np.cumsum(np.sort(np.asarray(a, np.float64))[::-1])

    def first(t):
        if t >= 1.0:
            return n
        i = int(np.searchsorted(c, t, side="left"))
        return max(1, min(i + 1, n))

    return first(p), first(p - band), first(p + band)


def decide(ws: np.ndarray, wl: np.ndarray, tau: int) -> tuple:
    """Boundary decision [Summary: a larger recent working set triggers one extra page;
    FAQ-impl: tau 0].  Reading R2: delta = sum(W_S - W_L), grow iff delta > tau."""
    delta = int(np.sum(np.asarray(ws, np.int64) - np.asarray(wl, np.int64)))
    return delta, (DECISION_GROW if delta > tau else DECISION_COMPACT)


POLICIES = ("growpage", "random", "inverse", "always_compact", "shrink")


def policy_decision(delta: int, tau: int, policy: str = "growpage", u: float = 0.0,
                    grow_prob: float = 0.0) -> int:
    """Grow or compact under the decision policies the pages compare [review, "Strengths",
    item "Frequency-matched causal ablations" (Tables 8-9): RANDOM keeps GrowPage's grow
    ratio without its signal, INVERSE reverses the signal's direction; FAQ "How does
    GrowPage differ from Zipage?": a fixed per-request budget never grows].  Readings: growpage grows iff
    delta > tau (R2); inverse grows iff -delta > tau; random grows iff the request's
    uniform draw u (an input, float32) is below grow_prob (float32); always_compact
    never grows.  shrink [same item: SHRINK isolates the cost of irreversible shrinking]:
    reading R16, grows iff delta > tau like GrowPage and otherwise shrinks the allocation
    by one page (boundary_step turns a shrink of a one-page allocation into an in-place
    compaction)."""
    if policy == "growpage":
        return DECISION_GROW if delta > tau else DECISION_COMPACT
    if policy == "shrink":
        return DECISION_GROW if delta > tau else DECISION_SHRINK
    if policy == "inverse":
        return DECISION_GROW if -delta > tau else DECISION_COMPACT
    if policy == "random":
        return DECISION_GROW if np.float32(u) < np.float32(grow_prob) else DECISION_COMPACT
    if policy == "always_compact":
        return DECISION_COMPACT
    raise ValueError(policy)


def importance(a_group: np.ndarray) -> np.ndarray:
    """Max-of-both importance per slot [Summary: compaction ranks slots by the larger of
    the two summaries' importance]; reading R5: max over the KV head's query heads and
    both summaries."""
    return np.asarray(a_group, np.float64).max(axis=0)


def keep_set(imp: np.ndarray, k: int, n_local: int, band: float = NEAR_TIE):
    """Slots kept by a compaction into k slots [Summary; FAQ-impl: local quota 64].

    Reading R6: the last min(n_local, k) slots are always kept; of the others the
    k - min(n_local, k) with the highest importance are kept, an exact tie going to
    the more recent (higher) slot.  Returns (kept ascending, evicted ascending,
    near_tie) where near_tie marks a kept/evicted boundary within relative ``band``.
    """
    n = int(imp.size)
    k = min(k, n)
    nl = min(n_local, k)
    cand = n - nl
    keep_c = k - nl
    slots = np.arange(cand)
    order = np.lexsort((-slots, -imp[:cand]))          # importance desc, then slot desc
    kept = np.sort(np.concatenate([order[:keep_c], np.arange(cand, n)])).astype(np.int64)
    evicted = np.sort(order[keep_c:]).astype(np.int64)
    near = False
    if 0 < keep_c < cand:
        lo_kept = imp[order[keep_c - 1]]
        hi_ev = imp[order[keep_c]]
        near = bool(lo_kept - hi_ev <= band * lo_kept)
    return kept, evicted, near


def keep_set_valid(evicted: np.ndarray, imp: np.ndarray, k: int, n_local: int,
                   band: float = NEAR_TIE) -> bool:
    """True when ``evicted`` is one of the answers a near-tie allows: the right size,
    only evictable slots, and no evicted slot clearly more important than a kept one."""
    n = int(imp.size)
    nl = min(n_local, k)
    cand = n - nl
    ev = np.asarray(evicted, np.int64)
    if ev.size != n - k or np.unique(ev).size != ev.size:
        return False
    if ev.size and (ev.min() < 0 or ev.max() >= cand):
        return False
    if ev.size == 0 or ev.size == cand:
        return True
    kept_c = np.setdiff1d(np.arange(cand), ev)
    return bool(imp[ev].max() <= imp[kept_c].min() * (1.0 + band))


def compact_rows(rows: np.ndarray, kept: np.ndarray) -> np.ndarray:
    """Stable compaction of one (layer, KV head): new slot j holds old slot kept[j]
    [Summary: compacted within the current allocation]; out of place."""
    return np.asarray(rows)[kept].copy()


# ----------------------------------------------------------------------------- one unit / request
def scan_request(k_rows: np.ndarray, dtype: str, sum_s: np.ndarray, sum_l: np.ndarray,
                 cos_row, sin_row, p: float, keep_logits: bool = False):
    """Working sets of every (layer, query head, summary) of one request.

    k_rows [L][Hkv][n][d] stored keys; sum_s/sum_l [L][Hq][d] float32 pre-RoPE.
    Returns W, W_lo, W_hi [L][Hq][2] (index 0 = short, 1 = long), M, Z [L][Hq][2] and
    the probabilities a [L][Hkv][2G][n] (rows h*2 + sigma within the group) when asked.
    """
    L, Hkv, n, d = k_rows.shape
    Hq = sum_s.shape[1]
    G = Hq // Hkv
    W = np.zeros((L, Hq, 2), np.int64)
    Wlo = np.zeros_like(W)
    Whi = np.zeros_like(W)
    M = np.zeros((L, Hq, 2))
    Z = np.zeros((L, Hq, 2))
    probs = np.zeros((L, Hkv, 2 * G, n)) if keep_logits else None
    for l in range(L):
        for g in range(Hkv):
            kf = widen(k_rows[l, g], dtype)
            for j in range(G):
                h = g * G + j
                for sig, summ in enumerate((sum_s, sum_l)):
                    qt = rope_rotate(summ[l, h], cos_row, sin_row)
                    if n == 0:  # reading R17: empty row, max -inf, sum 0, W 0
                        M[l, h, sig] = -np.inf
                        continue
                    lg = logits(qt[None, :], kf)[0]
                    m_, z_, a = softmax_stats(lg)
                    M[l, h, sig], Z[l, h, sig] = m_, z_
                    W[l, h, sig], Wlo[l, h, sig], Whi[l, h, sig] = working_set(a, p)
                    if keep_logits:
                        probs[l, g, 2 * j + sig] = a
    return W, Wlo, Whi, M, Z, probs


def delta_range(W: np.ndarray, Wlo: np.ndarray, Whi: np.ndarray):
    """Delta and the range over near-tie alternatives (short minus long, summed)."""
    d = int(np.sum(W[..., 0] - W[..., 1]))
    lo = int(np.sum(Wlo[..., 0] - Whi[..., 1]))
    hi = int(np.sum(Whi[..., 0] - Wlo[..., 1]))
    return d, lo, hi


# ----------------------------------------------------------------------------- whole step
@dataclasses.dataclass
class StepResult:
    W: np.ndarray
    W_lo: np.ndarray
    W_hi: np.ndarray
    M: np.ndarray
    Z: np.ndarray
    delta: np.ndarray
    delta_lo: np.ndarray
    delta_hi: np.ndarray
    decision_raw: np.ndarray
    decision: np.ndarray
    ambiguous: np.ndarray
    status: np.ndarray
    evicted: Dict[int, np.ndarray]
    evict_near_tie: Dict[int, np.ndarray]
    imp: Dict[int, np.ndarray]
    e_req: np.ndarray
    page_table: np.ndarray
    n_alloc: np.ndarray
    fill: np.ndarray
    refcount: np.ndarray
    free_stack: np.ndarray
    free_top: int
    k_new: Dict[int, np.ndarray]
    v_new: Dict[int, np.ndarray]
    cow: List[tuple]
    counters: Dict[str, int]


def boundary_step(wl, sum_s: np.ndarray, sum_l: np.ndarray, params: dict) -> StepResult:
    """One boundary batch: scan, decide, grow pops, keep-sets, copy-on-write, compaction.

    ``wl`` carries the per-request stored rows and the page state (see synth.Workload);
    sum_s/sum_l [B][L][Hq][d] float32 are the summaries at the boundary.  Follows
    [Summary] and [Abstract] under readings R1-R7.  Inputs are not modified.  Optional
    params "policy", "rand_u" ([B] float32) and "grow_prob" select a decision policy
    (policy_decision); the default is GrowPage's own rule.  Under "shrink" (reading R16)
    a request at its boundary that does not grow -- by decision or because its grow is
    denied -- and holds A >= 2 allocation pages keeps (A - 1) P slots (same keep-set
    rule), compacted into pages 0..A-2; allocation page A-1 loses this request's
    reference (pushed with the other freed pages if that was the last one) and the write
    page takes its place in the page table (index A-1).  With A < 2 it compacts in place.
    """
    B, L, Hq, Hkv, P = wl.B, wl.L, wl.Hq, wl.Hkv, wl.P
    G = Hq // Hkv
    p = float(np.float32(params["top_p"]))
    tau = int(params["tau"])
    n_local = int(params["n_local"])
    policy = params.get("policy", "growpage")
    rand_u = params.get("rand_u")
    grow_prob = params.get("grow_prob", 0.0)
    W = np.zeros((B, L, Hq, 2), np.int64)
    Wlo, Whi = np.zeros_like(W), np.zeros_like(W)
    M = np.zeros((B, L, Hq, 2))
    Z = np.zeros((B, L, Hq, 2))
    delta = np.zeros(B, np.int64)
    dlo, dhi = np.zeros(B, np.int64), np.zeros(B, np.int64)
    raw = np.zeros(B, np.int64)
    amb = np.zeros(B, bool)
    status = np.zeros(B, np.int64)
    probs = {}
    for b in range(B):
        cr = sr = None
        if wl.rope_cos is not None:
            cr, sr = wl.rope_cos[wl.pos[b]], wl.rope_sin[wl.pos[b]]
        res = scan_request(wl.k_rows[b], wl.dtype, sum_s[b], sum_l[b], cr, sr, p, keep_logits=True)
        W[b], Wlo[b], Whi[b], M[b], Z[b], probs[b] = res
        delta[b], dlo[b], dhi[b] = delta_range(W[b], Wlo[b], Whi[b])
        u = 0.0 if rand_u is None else float(rand_u[b])
        raw[b] = policy_decision(int(delta[b]), tau, policy, u, grow_prob)
        lo_d = policy_decision(int(dlo[b]), tau, policy, u, grow_prob)
        hi_d = policy_decision(int(dhi[b]), tau, policy, u, grow_prob)
        amb[b] = lo_d != hi_d

    table = wl.page_table.copy()
    A = wl.n_alloc.astype(np.int64).copy()
    fill = wl.fill.astype(np.int64).copy()
    rc_snap = wl.refcount.astype(np.int64).copy()
    refcount = rc_snap.copy()
    stack = wl.free_stack.astype(np.int64).copy()
    top = int(wl.free_top)
    decision = raw.copy()
    at_boundary = fill == P
    counters = dict(grows=0, compacts=0, grow_denied=0, deferred=0, cow_pages=0, freed_pages=0)

    # Grows pop first, in batch order (R7).
    for b in range(B):
        if not at_boundary[b]:
            status[b] |= REQ_NOT_AT_BOUNDARY
            decision[b] = DECISION_COMPACT
            continue
        if raw[b] != DECISION_GROW:
            continue
        if top > 0 and A[b] + 2 <= table.shape[1]:
            top -= 1
            pg = int(stack[top])
            table[b, A[b] + 1] = pg
            refcount[pg] = 1
            A[b] += 1
            fill[b] = 0
            counters["grows"] += 1
        else:
            decision[b] = DECISION_COMPACT
            status[b] |= REQ_GROW_DENIED
            counters["grow_denied"] += 1
    if policy == "shrink":  # every request at its boundary that does not grow shrinks (R16)
        for b in range(B):
            if at_boundary[b] and decision[b] != DECISION_GROW:
                decision[b] = DECISION_SHRINK if A[b] >= 2 else DECISION_COMPACT
    counters["shrinks"] = 0

    # Keep-sets, copy-on-write and compaction for compacting requests, batch order.
    evicted, near, imps, k_new, v_new, cow = {}, {}, {}, {}, {}, []
    e_req = np.zeros(B, np.int64)
    freed = []
    for b in range(B):
        n = int(wl.n_alloc[b]) * P + int(wl.fill[b])
        e_req[b] = n
        if not at_boundary[b] or decision[b] == DECISION_GROW:
            continue
        shrink = decision[b] == DECISION_SHRINK
        k = (int(wl.n_alloc[b]) - (1 if shrink else 0)) * P
        ev = np.zeros((L, Hkv, n - k), np.int64)
        nt = np.zeros((L, Hkv), bool)
        im = np.zeros((L, Hkv, n))
        kept_all = {}
        for l in range(L):
            for g in range(Hkv):
                im[l, g] = importance(probs[b][l, g])
                kept, evd, nr = keep_set(im[l, g], k, n_local)
                ev[l, g], nt[l, g] = evd, nr
                kept_all[(l, g)] = kept
                if evd.size:
                    e_req[b] = min(e_req[b], int(evd[0]))
        evicted[b], near[b], imps[b] = ev, nt, im
        # Pages of the allocation that change: j < k / P with (j+1)*P > e (R7).
        j0 = int(e_req[b]) // P
        need = [j for j in range(j0, k // P) if rc_snap[table[b, j]] > 1]
        if len(need) > top:
            status[b] |= REQ_DEFERRED
            counters["deferred"] += 1
            continue
        for j in need:
            top -= 1
            new = int(stack[top])
            old = int(table[b, j])
            cow.append((b, j, old, new))
            table[b, j] = new
            refcount[new] = 1
            refcount[old] -= 1
            if refcount[old] == 0:
                freed.append(old)
            counters["cow_pages"] += 1
        kn = np.empty((L, Hkv, k) + wl.k_rows[b].shape[3:], wl.k_rows[b].dtype)
        vn = np.empty_like(kn)
        for (l, g), kept in kept_all.items():
            kn[l, g] = compact_rows(wl.k_rows[b][l, g], kept)
            vn[l, g] = compact_rows(wl.v_rows[b][l, g], kept)
        k_new[b], v_new[b] = kn, vn
        fill[b] = 0
        counters["compacts"] += 1
        if shrink:  # release allocation page A-1; the write page moves into its slot
            a_old = int(A[b])
            old = int(table[b, a_old - 1])
            refcount[old] -= 1
            if refcount[old] == 0:
                freed.append(old)
            table[b, a_old - 1] = table[b, a_old]
            A[b] = a_old - 1
            counters["shrinks"] += 1

    for pg in sorted(freed):
        stack[top] = pg
        top += 1
    counters["freed_pages"] = len(freed)
    return StepResult(W, Wlo, Whi, M, Z, delta, dlo, dhi, raw, decision, amb, status, evicted, near,
                      imps, e_req, table, A, fill, refcount, stack, top, k_new, v_new, cow, counters)


# ----------------------------------------------------------------------------- decode attention
def decode_attention(k_rows: np.ndarray, v_rows: np.ndarray, dtype: str, q: np.ndarray, q_dtype: str,
                     cos_row, sin_row) -> np.ndarray:
    """Attention of one request's decode queries over its retained slots, the reader of the
    pages the engine rewrites [Abstract: the engine works inside PagedAttention serving].
    Standard softmax attention in float64: each query head h of KV head g is rotated to
    the request position (R4), scored against every stored key with scale 1/sqrt(d),
    and the softmax weights average the stored values.  k_rows, v_rows [L][Hkv][n][d],
    q [L][Hq][d]; returns [L][Hq][d] (zeros when n == 0)."""
    L, Hkv, n, d = k_rows.shape
    Hq = q.shape[1]
    G = Hq // Hkv
    qf = query_f32(q, q_dtype).astype(np.float64)
    out = np.zeros((L, Hq, d))
    if n == 0:
        return out
    for l in range(L):
        for g in range(Hkv):
            kf = widen(k_rows[l, g], dtype)
            vf = widen(v_rows[l, g], dtype)
            for j in range(G):
                h = g * G + j
                qt = rope_rotate(qf[l, h], cos_row, sin_row)
                M, Z, a = softmax_stats(logits(qt[None, :], kf))
                out[l, h] = a[0] @ vf
    return out


# ----------------------------------------------------------------------------- decode loop
@dataclasses.dataclass
class LoopState:
    """Requests between decode steps as the oracle tracks them: stored rows in logical
    slot order ([L][Hkv][n][d] per request), the page state and the summaries.  ``pos``
    is the absolute position of the current step's query and token."""
    L: int
    Hq: int
    Hkv: int
    d: int
    P: int
    dtype: str
    num_pages: int
    page_table: np.ndarray
    n_alloc: np.ndarray
    fill: np.ndarray
    refcount: np.ndarray
    free_stack: np.ndarray
    free_top: int
    k_rows: list
    v_rows: list
    sum_s: np.ndarray
    sum_l: np.ndarray
    pos: np.ndarray
    rope_cos: Optional[np.ndarray]
    rope_sin: Optional[np.ndarray]

    @property
    def B(self) -> int:
        return int(self.page_table.shape[0])

    def n(self, b: int) -> int:
        return int(self.n_alloc[b]) * self.P + int(self.fill[b])

    def subset(self, idx) -> "LoopState":
        """The requests ``idx`` (in that order) over the shared pool state."""
        idx = np.asarray(idx, np.int64)
        return LoopState(self.L, self.Hq, self.Hkv, self.d, self.P, self.dtype, self.num_pages,
                         self.page_table[idx].copy(), self.n_alloc[idx].copy(), self.fill[idx].copy(),
                         self.refcount.copy(), self.free_stack.copy(), int(self.free_top),
                         [self.k_rows[b] for b in idx], [self.v_rows[b] for b in idx],
                         self.sum_s[idx], self.sum_l[idx], self.pos[idx].copy(),
                         self.rope_cos, self.rope_sin)


def append_token(state: LoopState, b: int, k_new: np.ndarray, v_new: np.ndarray) -> bool:
    """The step's K/V row [L][Hkv][d] of request b goes to slot A*P + fill, i.e. the next
    slot of the write page (reading R6); a full write page takes nothing (False)."""
    if int(state.fill[b]) >= state.P:
        return False
    state.k_rows[b] = np.concatenate([state.k_rows[b], np.asarray(k_new)[:, :, None, :]], axis=2)
    state.v_rows[b] = np.concatenate([state.v_rows[b], np.asarray(v_new)[:, :, None, :]], axis=2)
    state.fill[b] += 1
    return True


def decode_step(state: LoopState, q: np.ndarray, q_dtype: str, k_new: np.ndarray,
                v_new: np.ndarray, params: dict):
    """One decode step of every request, in place.

    The summaries absorb the step's query first (R3; [Summary]: the summaries smooth the
    decode queries), the step's row is appended (R6), and the requests whose write page
    is now full form one boundary batch in batch order (boundary_step).  Positions then
    advance by one.  Returns (appended [B] bool, boundary request indices, the boundary
    batch's input state, StepResult); the last two are None when no write page filled."""
    qf = query_f32(q, q_dtype)
    state.sum_s = ema_update(state.sum_s, qf, params["beta_s"])
    state.sum_l = ema_update(state.sum_l, qf, params["beta_l"])
    appended = np.array([append_token(state, b, k_new[b], v_new[b]) for b in range(state.B)])
    idx = np.flatnonzero(state.fill == state.P)
    sub = res = None
    if idx.size:
        sub = state.subset(idx)
        res = boundary_step(sub, sub.sum_s, sub.sum_l, params)
        state.page_table[idx] = res.page_table
        state.n_alloc[idx] = res.n_alloc
        state.fill[idx] = res.fill
        state.refcount = res.refcount.copy()
        state.free_stack = res.free_stack.copy()
        state.free_top = int(res.free_top)
        for i, b in enumerate(idx):
            if i in res.k_new:
                state.k_rows[b] = res.k_new[i]
                state.v_rows[b] = res.v_new[i]
    state.pos = state.pos + 1
    return appended, idx, sub, res

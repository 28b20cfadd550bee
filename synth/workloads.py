"""Seeded synthetic workloads for the GrowPage capacity-boundary engine (CPU, numpy).

Everything here builds *inputs*: paged K/V rows, page tables, the free-page stack,
refcounts, RoPE cos/sin tables, pre-RoPE query summaries or the decode queries that
feed them.  Nothing here computes a working set, a decision, a keep-set or a page
rewrite.  The only arithmetic beyond random draws is the construction of planted
attention structure: a key gets a component along a chosen direction in the
post-RoPE frame, so the generator rotates that one direction with the standard
rotate-half RoPE formula (a model convention, not part of the engine's outputs).

Shapes follow the pages' workloads: 8B-class GQA (32 query heads, 8 KV heads,
head_dim 128, bf16), heterogeneous contexts drawn log-uniformly, concentrated vs
diffuse attention regimes (GrowPage review on evolve.pub, "Summary" and
"Strengths": minimum budgets spanning 512 to 8192+ tokens, sparsity swinging
between concentrated and diffuse phases; grow ratio near 30% in Table 9).

Storage conventions (they are the library's interface, restated here):
  * K/V rows per request: [L][Hkv][n][d], float32 or bf16 bit patterns (uint16).
  * page_table[b][j]: allocation pages j < n_alloc[b], the write page at j = n_alloc[b].
  * n[b] = n_alloc[b] * P + fill[b] candidate slots.
  * free stack: free_stack[0:free_top], the top of the stack is free_stack[free_top-1].
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

PARAMS_DEFAULT = dict(beta_s=0.9, beta_l=0.999, top_p=0.9, tau=0, n_local=64)
# Hyper-parameters the pages report for the paper's own runs (GrowPage review on
# evolve.pub, FAQ "Is GrowPage's code available?"): block 256, p 0.99, quota 64.
PARAMS_PAPER = dict(beta_s=0.9, beta_l=0.999, top_p=0.99, tau=0, n_local=64)


# ----------------------------------------------------------------------------- storage
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) & 0xFFFF
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rope_tables(max_pos: int, d: int, theta: float = 1.0e6):
    """Standard rotate-half RoPE tables: cos/sin [max_pos][d/2] float32, angle pos*theta^(-2i/d)."""
    i = np.arange(d // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / d)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _rotate_direction(u: np.ndarray, c: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Rotate a planting direction into the post-RoPE frame (pairs i, i+d/2)."""
    h = u.shape[-1] // 2
    x1, x2 = u[..., :h], u[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def _unit(rng, shape):
    v = rng.standard_normal(shape)
    return v / np.linalg.norm(v, axis=-1, keepdims=True)


# ----------------------------------------------------------------------------- workload
@dataclasses.dataclass
class Workload:
    name: str
    L: int
    Hq: int
    Hkv: int
    d: int
    P: int
    dtype: str                      # "f32" | "bf16"
    num_pages: int
    max_pages: int
    page_table: np.ndarray          # [B][max_pages] int32, -1 where unused
    n_alloc: np.ndarray             # [B] int32
    fill: np.ndarray                # [B] int32
    pos: np.ndarray                 # [B] int32 absolute position the summaries are rotated to
    refcount: np.ndarray            # [num_pages] int32
    free_stack: np.ndarray          # [num_pages] int32
    free_top: int
    k_rows: list                    # per request [L][Hkv][n][d] storage dtype
    v_rows: list
    sum_s: Optional[np.ndarray]     # [B][L][Hq][d] float32 (direct synthesis) or None
    sum_l: Optional[np.ndarray]
    queries: Optional[np.ndarray]   # [T][B][L][Hq][d] storage dtype (EMA-driven) or None
    q_dtype: str
    rope_cos: Optional[np.ndarray]  # [max_pos][d/2] float32 or None (identity)
    rope_sin: Optional[np.ndarray]
    params: dict
    seed: int
    regime: Optional[np.ndarray] = None   # [B] 1 = planted broadening, 0 = concentrating

    @property
    def B(self) -> int:
        return int(self.page_table.shape[0])

    def n(self, b: int) -> int:
        return int(self.n_alloc[b]) * self.P + int(self.fill[b])

    def total_tokens(self) -> int:
        return sum(self.n(b) for b in range(self.B))


def _storage(x: np.ndarray, dtype: str) -> np.ndarray:
    return x.astype(np.float32) if dtype == "f32" else f32_to_bf16_bits(x.astype(np.float32))


def _zipf_plant(rng, n, d, dirs_post, s_zipf, alpha=2.0, n_plant=None):
    """Keys ~ N(0, I) plus, per head direction, a component giving a rank^-s profile.

    A summary whose post-RoPE projection on the direction equals ``alpha`` sees
    logits s*(ln n - ln rank) + noise, i.e. Zipf(s) attention; larger projections
    sharpen it, smaller ones flatten it.
    """
    k = rng.standard_normal((n, d))
    for u in dirs_post:
        rank = rng.permutation(n).astype(np.float64) + 1.0
        mu = s_zipf * (math.log(max(n, 1)) - np.log(rank)) * math.sqrt(d) / alpha  # n = 0: no keys
        if n_plant is not None:
            mu = np.where(rank <= n_plant, mu, 0.0)
        k += mu[:, None] * u[None, :]
    return k


def _pool_layout(rng, A, fill, P, num_pages, max_pages, shared=None):
    """Assign page ids: shuffled pool, each request takes A+1 pages (prefix pages may be shared)."""
    B = len(A)
    perm = list(rng.permutation(num_pages).astype(np.int64))
    table = np.full((B, max_pages), -1, dtype=np.int32)
    refcount = np.zeros(num_pages, dtype=np.int32)
    shared = shared or {}
    group_pages = {}
    for b in range(B):
        need = int(A[b]) + 1
        j0 = 0
        if b in shared:
            grp, npre = shared[b]
            if grp not in group_pages:
                group_pages[grp] = [perm.pop() for _ in range(npre)]
            for j, pg in enumerate(group_pages[grp]):
                table[b, j] = pg
                refcount[pg] += 1
            j0 = npre
        for j in range(j0, need):
            pg = perm.pop()
            table[b, j] = pg
            refcount[pg] += 1
    free = np.array(perm, dtype=np.int32)
    stack = np.zeros(num_pages, dtype=np.int32)
    stack[: len(free)] = free
    return table, refcount, stack, len(free)


# ----------------------------------------------------------------------------- configs
def config1(seed: int = 1000) -> Workload:
    """Tiny CPU-checkable case: 1 request, 1 layer, 8/2 heads, d 64, fp32, P 16, A 4.

    Keys/values N(0,1); 4 heavy-hitter keys set to 4*sqrt(d)*u for a hidden unit
    direction u; 32 decode queries N(0,1) + 2u feed both summaries from zero;
    identity RoPE; p 0.9, no local quota.  The write page is full: n 80, keep 64.
    """
    rng = np.random.default_rng(seed)
    L, Hq, Hkv, d, P, A = 1, 8, 2, 64, 16, 4
    n = (A + 1) * P
    u = _unit(rng, (d,))
    k = rng.standard_normal((L, Hkv, n, d))
    v = rng.standard_normal((L, Hkv, n, d))
    hh = rng.choice(A * P, size=4, replace=False)
    k[:, :, hh, :] = 4.0 * math.sqrt(d) * u
    q = rng.standard_normal((32, 1, L, Hq, d)) + 2.0 * u
    num_pages = 16
    table, rc, stack, top = _pool_layout(rng, [A], [P], P, num_pages, max_pages=8)
    params = dict(PARAMS_DEFAULT, n_local=0)
    return Workload("config1", L, Hq, Hkv, d, P, "f32", num_pages, 8, table,
                    np.array([A], np.int32), np.array([P], np.int32), np.array([n], np.int32),
                    rc, stack, top, [k.astype(np.float32)], [v.astype(np.float32)],
                    None, None, q.astype(np.float32), "f32", None, None, params, seed,
                    regime=np.array([0], np.int32))


def config2(seed: int = 2000, B: int = 16, T: int = 256, num_pages: int = 65536) -> Workload:
    """Llama-8B-shaped single layer: 32/8 heads, d 128, bf16, P 16, 16 requests.

    Contexts log-uniform in [512, 8192]; page ids drawn from a shuffled 64K-page pool;
    keys N(0,1) plus a Zipf(1.1) profile along each head's planted direction; summaries
    come from T bf16 decode queries in two phases: focused (8u + noise) then broad
    (noise).  A long broad tail makes the recent summary flatter than the long one
    (planted broadening); a short one keeps it sharper (planted concentrating).
    """
    rng = np.random.default_rng(seed)
    L, Hq, Hkv, d, P = 1, 32, 8, 128, 16
    G = Hq // Hkv
    ctx = np.exp(rng.uniform(math.log(512), math.log(8192), size=B))
    A = np.ceil(ctx / P).astype(np.int32)
    fill = np.full(B, P, np.int32)
    n = (A + 1) * P
    pos = n.astype(np.int32)
    cos, sin = rope_tables(int(pos.max()) + 1, d)
    regime = (rng.uniform(size=B) < 0.4).astype(np.int32)
    regime[0], regime[1] = 1, 0                      # both outcomes present
    max_pages = int(A.max()) + 4
    table, rc, stack, top = _pool_layout(rng, A, fill, P, num_pages, max_pages)
    u_pre = _unit(rng, (B, L, Hq, d))
    k_rows, v_rows = [], []
    for b in range(B):
        kb = np.empty((L, Hkv, n[b], d), np.float32)
        for l in range(L):
            for g in range(Hkv):
                dirs = [_rotate_direction(u_pre[b, l, g * G + j], cos[pos[b]], sin[pos[b]])
                        for j in range(G)]
                kb[l, g] = _zipf_plant(rng, int(n[b]), d, dirs, 1.1)
        k_rows.append(f32_to_bf16_bits(kb))
        v_rows.append(f32_to_bf16_bits(rng.standard_normal((L, Hkv, n[b], d)).astype(np.float32)))
    q = rng.standard_normal((T, B, L, Hq, d))
    for b in range(B):
        broad = int(rng.integers(48, 128)) if regime[b] else int(rng.integers(0, 4))
        q[: T - broad, b] += 8.0 * u_pre[b]
    return Workload("config2", L, Hq, Hkv, d, P, "bf16", num_pages, max_pages, table, A, fill,
                    pos, rc, stack, top, k_rows, v_rows, None, None,
                    f32_to_bf16_bits(q.astype(np.float32)), "bf16", cos, sin,
                    dict(PARAMS_DEFAULT), seed, regime=regime)


def direct_case(seed: int, B: int = 4, L: int = 2, Hq: int = 8, Hkv: int = 2, d: int = 64,
                P: int = 16, dtype: str = "bf16", ctx=(64, 400), num_pages: Optional[int] = None,
                spare_pages: int = 64, grow_frac: float = 0.3, rope: bool = True,
                prefix_groups: int = 0, prefix_pages: int = 0, fill=None,
                params: Optional[dict] = None, s_zipf=(0.8, 1.6), max_pages: Optional[int] = None,
                name: str = "direct", alloc=None) -> Workload:
    """Generic case with directly synthesised pre-RoPE summaries (the large-config recipe).

    Per (request, layer, query head) a unit direction u is drawn in the pre-RoPE frame;
    S = b_S u + e_S and L = b_L u + e_L with small isotropic noise e.  Planted broadening
    requests draw b_S in [0.2, 0.8] and b_L in [1.5, 3]; concentrating ones b_S in
    [2, 5] and b_L in [0.5, 1.5].  Keys carry a Zipf(s) profile along each head's
    direction rotated to the request's position.  Optional prefix sharing: groups of
    requests share their first ``prefix_pages`` pages (refcounted).  ``alloc`` sets each
    request's allocation pages directly (0 allowed: a request holding only its write
    page) instead of drawing them from ``ctx``.
    """
    rng = np.random.default_rng(seed)
    G = Hq // Hkv
    ctx_tok = np.exp(rng.uniform(math.log(ctx[0]), math.log(ctx[1]), size=B))
    A = np.maximum(np.ceil(ctx_tok / P).astype(np.int32), max(1, prefix_pages))
    if alloc is not None:
        A = np.asarray(alloc, np.int32)
        assert A.shape == (B,) and A.min() >= (prefix_pages if prefix_groups else 0)
    fill = np.full(B, P, np.int32) if fill is None else np.asarray(fill, np.int32)
    n = A * P + fill
    pos = (n + rng.integers(0, 64, size=B)).astype(np.int32)
    cos, sin = rope_tables(int(pos.max()) + 1, d) if rope else (None, None)
    shared = {}
    if prefix_groups and prefix_pages:
        for b in range(B):
            shared[b] = (b % prefix_groups, prefix_pages)
    total_needed = int(np.sum(A + 1))
    if shared:
        total_needed -= len(shared) * prefix_pages - len({g for g, _ in shared.values()}) * prefix_pages
    if num_pages is None:
        num_pages = total_needed + spare_pages
    if max_pages is None:
        max_pages = int(A.max()) + 4
    table, rc, stack, top = _pool_layout(rng, A, fill, P, num_pages, max_pages, shared)
    regime = (rng.uniform(size=B) < grow_frac).astype(np.int32)
    u_pre = _unit(rng, (B, L, Hq, d))
    bs = np.where(regime[:, None, None], rng.uniform(0.2, 0.8, (B, L, Hq)), rng.uniform(2.0, 5.0, (B, L, Hq)))
    bl = np.where(regime[:, None, None], rng.uniform(1.5, 3.0, (B, L, Hq)), rng.uniform(0.5, 1.5, (B, L, Hq)))
    sum_s = bs[..., None] * u_pre + 0.1 * rng.standard_normal((B, L, Hq, d))
    sum_l = bl[..., None] * u_pre + 0.1 * rng.standard_normal((B, L, Hq, d))
    sz = rng.uniform(s_zipf[0], s_zipf[1], size=B)
    # Shared prefix rows must be identical across the requests that share the pages.
    prefix_rows = {}
    k_rows, v_rows = [], []
    for b in range(B):
        nb = int(n[b])
        kb = np.empty((L, Hkv, nb, d), np.float32)
        vb = rng.standard_normal((L, Hkv, nb, d)).astype(np.float32)
        for l in range(L):
            for g in range(Hkv):
                if cos is not None:
                    dirs = [_rotate_direction(u_pre[b, l, g * G + j], cos[pos[b]], sin[pos[b]]) for j in range(G)]
                else:
                    dirs = [u_pre[b, l, g * G + j] for j in range(G)]
                kb[l, g] = _zipf_plant(rng, nb, d, dirs, float(sz[b]))
        if b in shared:
            grp, npre = shared[b]
            m = npre * P
            if grp in prefix_rows:
                kb[:, :, :m], vb[:, :, :m] = prefix_rows[grp]
            else:
                prefix_rows[grp] = (kb[:, :, :m].copy(), vb[:, :, :m].copy())
        k_rows.append(_storage(kb, dtype))
        v_rows.append(_storage(vb, dtype))
    return Workload(name, L, Hq, Hkv, d, P, dtype, int(num_pages), int(max_pages), table, A, fill, pos,
                    rc, stack, top, k_rows, v_rows, sum_s.astype(np.float32), sum_l.astype(np.float32),
                    None, "f32", cos, sin, dict(params or PARAMS_DEFAULT), seed, regime=regime)


def planted_logits_case(seed: int, logit_fns, L: int = 1, Hq: int = 8, Hkv: int = 2, d: int = 64,
                        P: int = 16, params: Optional[dict] = None, spare_pages: int = 8,
                        name: str = "planted", dtype: str = "f32") -> Workload:
    """Requests whose scores are planted exactly: every summary (all heads, both
    timescales) is the unit vector e_0 and key i carries logit_fn(rng, n)[i] * sqrt(d) in
    component 0 (float32 storage, or bf16 by round-to-nearest-even; no RoPE), so each
    softmax row sees those logits (as stored).  Both summaries coincide, so every request
    compacts.  ``logit_fns[b]`` = (n_alloc, fn)."""
    rng = np.random.default_rng(seed)
    B = len(logit_fns)
    A = np.array([a for a, _ in logit_fns], np.int32)
    fill = np.full(B, P, np.int32)
    n = A * P + fill
    num_pages = int(np.sum(A + 1)) + spare_pages
    max_pages = int(A.max()) + 4
    table, rc, stack, top = _pool_layout(rng, A, fill, P, num_pages, max_pages)
    k_rows, v_rows = [], []
    for b, (_, fn) in enumerate(logit_fns):
        lg = np.asarray(fn(rng, int(n[b])), np.float64)
        kb = rng.standard_normal((L, Hkv, int(n[b]), d))
        kb[..., 0] = lg * math.sqrt(d)
        k_rows.append(_storage(kb, dtype))
        v_rows.append(_storage(rng.standard_normal((L, Hkv, int(n[b]), d)), dtype))
    e0 = np.zeros((B, L, Hq, d), np.float32)
    e0[..., 0] = 1.0
    return Workload(name, L, Hq, Hkv, d, P, dtype, num_pages, max_pages, table, A, fill,
                    n.astype(np.int32), rc, stack, top, k_rows, v_rows, e0, e0.copy(), None, "f32",
                    None, None, dict(params or PARAMS_DEFAULT), seed, regime=np.zeros(B, np.int32))

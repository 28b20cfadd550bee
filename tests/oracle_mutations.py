"""Plausible mistakes planted in the CPU oracle (test infrastructure, CPU only).

Each mutation rewrites one line of one oracle function -- a dropped term, a wrong sign,
an off-by-one, a flipped comparison or order -- and re-executes the function in the
oracle's module, so that everything calling it sees the mistake.  The mutation tests run
the pin suite on each and require it to fail: a pin set that passes a planted mistake
would not pin the oracle."""
from __future__ import annotations

import inspect
import textwrap

import oracle
import oracle.growpage_oracle as OM

# name -> (function, text in its source, replacement)
MUTATIONS = {
    "rope_sign": ("rope_rotate", "x1 * c - x2 * sn", "x1 * c + x2 * sn"),
    "logit_scale_dropped": ("logits", ") / math.sqrt(d)", ")"),
    "working_set_strict": ("working_set", 'side="left"', 'side="right"'),
    "working_set_off_by_one": ("working_set", "return max(1, min(i + 1, n))", "return max(1, min(i, n))"),
    "ema_weights_swapped": ("ema_update", "omb = np.float32(np.float32(1.0) - b)",
                            "omb = b; b = np.float32(np.float32(1.0) - omb)"),
    "ema_one_minus_beta_in_float64": ("ema_update", "omb = np.float32(np.float32(1.0) - b)",
                                      "omb = np.float32(1.0 - float(beta))"),
    "importance_min": ("importance", ".max(axis=0)", ".min(axis=0)"),
    "ties_keep_older": ("keep_set", "np.lexsort((-slots, -imp[:cand]))", "np.lexsort((slots, -imp[:cand]))"),
    "local_quota_dropped": ("keep_set", "    nl = min(n_local, k)\n    cand", "    nl = 0\n    cand"),
    "grow_on_tie": ("policy_decision", 'if policy == "growpage":\n        return DECISION_GROW if delta > tau',
                    'if policy == "growpage":\n        return DECISION_GROW if delta >= tau'),
    "delta_sign": ("delta_range", "d = int(np.sum(W[..., 0] - W[..., 1]))", "d = int(np.sum(W[..., 1] - W[..., 0]))"),
    "grow_pops_bottom": ("boundary_step", "            top -= 1\n            pg = int(stack[top])",
                         "            top -= 1\n            pg = int(stack[0])"),
    "cow_unshared_pages": ("boundary_step", "if rc_snap[table[b, j]] > 1]", "if rc_snap[table[b, j]] >= 1]"),
    "pushes_descending": ("boundary_step", "for pg in sorted(freed):", "for pg in sorted(freed)[::-1]:"),
    "compaction_reversed": ("compact_rows", "np.asarray(rows)[kept].copy()", "np.asarray(rows)[kept[::-1]].copy()"),
    "short_summary_not_updated": ("decode_step", 'state.sum_s = ema_update(state.sum_s, qf, params["beta_s"])',
                                  "pass"),
    "gqa_heads_strided": ("scan_request", "                h = g * G + j\n", "                h = j * Hkv + g\n"),
    "append_overfills": ("append_token", "if int(state.fill[b]) >= state.P:", "if int(state.fill[b]) > state.P:"),
    "positions_frozen": ("decode_step", "state.pos = state.pos + 1", "state.pos = state.pos + 0"),
    "shrink_keeps_whole_allocation": ("boundary_step", "k = (int(wl.n_alloc[b]) - (1 if shrink else 0)) * P",
                                      "k = int(wl.n_alloc[b]) * P"),
    "shrink_releases_write_page": ("boundary_step", "old = int(table[b, a_old - 1])", "old = int(table[b, a_old])"),
    "shrink_on_one_page": ("boundary_step", "DECISION_SHRINK if A[b] >= 2 else DECISION_COMPACT",
                           "DECISION_SHRINK if A[b] >= 1 else DECISION_COMPACT"),
    "cow_pages_descending": ("boundary_step", "        for j in need:\n", "        for j in need[::-1]:\n"),
    "importance_of_logits": ("scan_request", "                        probs[l, g, 2 * j + sig] = a",
                             "                        probs[l, g, 2 * j + sig] = lg"),
    "write_page_not_candidate": ("boundary_step", "        n = int(wl.n_alloc[b]) * P + int(wl.fill[b])\n        e_req[b] = n",
                                 "        n = int(wl.n_alloc[b]) * P\n        e_req[b] = n"),
    "cow_checks_current_refcount": ("boundary_step", "if rc_snap[table[b, j]] > 1]", "if refcount[table[b, j]] > 1]"),
    "attention_scale_dropped": ("decode_attention", "softmax_stats(logits(qt[None, :], kf))",
                                "softmax_stats(logits(qt[None, :], kf) * math.sqrt(d))"),
    "attention_query_not_rotated": ("decode_attention", "qt = rope_rotate(qf[l, h], cos_row, sin_row)",
                                    "qt = qf[l, h]"),
    "query_bf16_misaligned": ("query_f32", "astype(np.uint32) << 16)", "astype(np.uint32) << 15)"),
    "widen_bf16_misaligned": ("widen", "astype(np.uint32) << 16)", "astype(np.uint32) << 15)"),
    "query_bf16_as_float16": ("query_f32", "return (np.asarray(q, np.uint16).astype(np.uint32) << 16).view(np.float32)",
                              "return np.asarray(q, np.uint16).view(np.float16).astype(np.float32)"),
    "delta_range_point_bounds": ("delta_range",
                                 "lo = int(np.sum(Wlo[..., 0] - Whi[..., 1]))\n    hi = int(np.sum(Whi[..., 0] - Wlo[..., 1]))",
                                 "lo = d\n    hi = d"),
    "delta_range_same_side": ("delta_range", "lo = int(np.sum(Wlo[..., 0] - Whi[..., 1]))",
                              "lo = int(np.sum(Wlo[..., 0] - Wlo[..., 1]))"),
    "importance_in_float32": ("importance", "np.asarray(a_group, np.float64).max(axis=0)",
                              "np.asarray(a_group, np.float32).max(axis=0).astype(np.float64)"),
}


def apply(name: str) -> None:
    """Plant mutation `name` in the oracle module (for the rest of the process)."""
    fn, old, new = MUTATIONS[name]
    src = textwrap.dedent(inspect.getsource(getattr(OM, fn)))
    assert src.count(old) == 1, (name, fn)
    exec(compile(src.replace(old, new), f"<mutated {fn}>", "exec"), OM.__dict__)
    if hasattr(oracle, fn):  # the package re-exports the module's names
        setattr(oracle, fn, OM.__dict__[fn])

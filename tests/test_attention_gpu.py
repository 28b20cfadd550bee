"""Decode attention over the paged cache (gp_decode_attention) against the oracle's float64
attention, on the same pages and queries.

Tolerance: the kernel accumulates in float32 with an online softmax (running max and
sum per token slot, merged at the end), so each output element carries a relative
error of a few float32 ulps times log2(n) from the running rescales and sums; with
values of magnitude O(1) an absolute 2e-4 plus relative 1e-4 bound is met with a wide
margin, while a wrong index, row or head would be off by O(1).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle as O
from synth import device as SD
from synth import workloads as SW

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-4, 1e-4

CASES = [
    ("bf16_d128_p16", dict(B=5, L=2, Hq=32, Hkv=8, d=128, P=16, ctx=(100, 1500))),
    ("bf16_d64_p32", dict(B=4, L=2, Hq=8, Hkv=2, d=64, P=32, ctx=(40, 700))),
    ("f32_d128_p8", dict(B=3, L=1, Hq=16, Hkv=4, d=128, P=8, dtype="f32", ctx=(9, 300))),
    ("f32_d64_norope", dict(B=3, L=2, Hq=8, Hkv=2, d=64, P=16, dtype="f32", rope=False)),
    ("tiny_partial_pages", dict(B=6, L=1, Hq=8, Hkv=2, d=64, P=16, ctx=(1, 20), fill=[0, 3, 16, 1, 7, 15])),
    ("p256", dict(B=3, L=1, Hq=32, Hkv=8, d=128, P=256, ctx=(300, 2000))),
    ("gqa1_bf16_d128", dict(B=4, L=2, Hq=4, Hkv=4, d=128, P=16, ctx=(50, 900))),
    ("gqa2_f32_d64", dict(B=4, L=1, Hq=4, Hkv=2, d=64, P=16, dtype="f32", ctx=(20, 600))),
    # no allocation pages: an empty request (zeros), a partial and a full write page
    ("write_page_only", dict(B=4, L=2, Hq=8, Hkv=2, d=64, P=16, alloc=[0, 0, 0, 2], fill=[0, 5, 16, 7])),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_decode_attention(name, kw):
    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine
    seed = zlib.crc32(name.encode()) % 10000
    wl = SW.direct_case(seed=seed, name=name, **kw)
    rng = np.random.default_rng(seed + 1)
    qf = (rng.standard_normal((wl.B, wl.L, wl.Hq, wl.d)) * 2.0).astype(np.float32)
    q_bits = SW.f32_to_bf16_bits(qf)
    slots = np.arange(wl.B) * 2 + 1
    st = SD.upload(wl, "cuda", max_req=int(slots.max()) + 1, slots=slots)
    eng = BoundaryEngine(st, wl.B, wl.total_tokens(), Bd.params_from(wl.params))
    req = torch.as_tensor(slots.astype(np.int32), device="cuda")
    q = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).cuda()
    out = torch.empty((wl.B, wl.L, wl.Hq, wl.d), dtype=torch.float32, device="cuda")
    eng.decode_attention(q, req, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    worst = 0.0
    for b in range(wl.B):
        cr = sr = None
        if wl.rope_cos is not None:
            cr, sr = wl.rope_cos[wl.pos[b]], wl.rope_sin[wl.pos[b]]
        want = O.decode_attention(wl.k_rows[b], wl.v_rows[b], wl.dtype, q_bits[b], "bf16", cr, sr)
        err = np.abs(got[b] - want) - (ATOL + RTOL * np.abs(want))
        worst = max(worst, float((np.abs(got[b] - want)).max()))
        assert (err <= 0).all(), (name, b, wl.n(b), float(np.abs(got[b] - want).max()))
    print(f"[attn] {name}: max abs error {worst:.2e}", flush=True)

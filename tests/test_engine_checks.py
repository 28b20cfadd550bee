"""Host-side argument checks of the engine (CPU): tensors the kernels would index unchecked
are refused before any library call (nothing is launched here)."""
import pytest
import torch

from demand_paged_kv_amd import binding as B
from demand_paged_kv_amd.engine import BoundaryEngine
from synth import device as SD
from synth import workloads as SW


@pytest.fixture(scope="module")
def eng():
    B.load()
    wl = SW.direct_case(seed=11, B=2, L=1, Hq=8, Hkv=2, d=64, P=16, ctx=(20, 60))
    st = SD.upload(wl, "cpu")
    return BoundaryEngine(st, 2, wl.total_tokens(), B.params_from(wl.params))


def test_request_ids_are_checked(eng):
    bad = [torch.arange(2, dtype=torch.int64),                 # wrong dtype
           torch.arange(3, dtype=torch.int32),                 # more than the engine's batch
           torch.arange(4, dtype=torch.int32)[::2],            # not contiguous
           torch.zeros((1, 2), dtype=torch.int32),             # not 1-D
           torch.arange(2, dtype=torch.int32, device="meta")]  # another device
    for ids in bad:
        for call in (eng.scan, eng.decide, eng.compact, eng.compact_prepare, eng.compact_move, eng.step):
            with pytest.raises(ValueError):
                call(ids)


def test_rows_are_checked(eng):
    st = eng.st
    ids = torch.arange(2, dtype=torch.int32)
    q_ok = torch.zeros((2, st.L, st.Hq, st.d), dtype=torch.float32)
    with pytest.raises(ValueError):
        eng.update_summaries(q_ok[:1], ids)                                      # one row short
    with pytest.raises(ValueError):
        eng.update_summaries(q_ok.half(), ids)                                   # float16 queries
    with pytest.raises(ValueError):
        eng.update_summaries(q_ok.transpose(2, 3).contiguous().transpose(2, 3), ids)  # d not contiguous
    kv_ok = torch.zeros((2, st.L, st.Hkv, st.d), dtype=st.k_pool.dtype)
    with pytest.raises(ValueError):
        eng.append(kv_ok.double(), kv_ok, ids)                                   # not the pool's dtype
    with pytest.raises(ValueError):
        eng.append(kv_ok, torch.zeros((2, st.L, st.Hq, st.d), dtype=st.k_pool.dtype), ids)
    out = torch.zeros((2, st.L, st.Hq, st.d), dtype=torch.float32)
    with pytest.raises(ValueError):
        eng.decode_attention(q_ok, ids, out.double())
    with pytest.raises(ValueError):
        eng.decode_attention(q_ok, ids, out[:1])

"""The C-ABI library loads and exports every symbol include/growpage.h declares; host-side
argument validation answers without a GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

from demand_paged_kv_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "growpage.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:gp_status|int32_t|size_t|const char\*|void\*|void)\s+(gp_\w+)\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libgrowpage.so is not built; run `python -m demand_paged_kv_amd.build`")
    return B.load()


def test_header_declares_expected_entry_points():
    assert _declared() == sorted(B.EXPORTED)


def test_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {B.LIB_PATH}").read()
    for name in _declared():
        assert re.search(rf"\bT {name}$", out, re.M), name


def test_version_and_status_strings(lib):
    assert lib.gp_abi_version() == 2
    for s in range(5):
        assert lib.gp_status_string(s).decode().startswith("GP_")
    assert b"unknown" in lib.gp_status_string(99)


def _kv(**over):
    kv = B.make_kv(0x1000, 0x2000, 2, 32, 8, 128, 16, 1024, B.GP_BF16)
    for k, v in over.items():
        setattr(kv, k, v)
    return kv


def test_scratch_bytes_grows_with_tokens(lib):
    kv = _kv()
    a = B.scratch_bytes(kv, 4, 1000)
    b = B.scratch_bytes(kv, 4, 2000)
    # logits: 1000 more tokens x L x Hkv x 8 floats, plus importance and copy-on-write slots
    assert b - a >= 1000 * 2 * 8 * 8 * 4
    assert B.scratch_bytes(kv, -1, 10) == 0
    assert lib.gp_scratch_bytes(None, 1, 1) == 0


def test_invalid_arguments_rejected_on_host(lib):
    kv = _kv()
    pg = B.Pages(0x3000, 4, 8, 0x4000, 0x5000, 0x6000, 0x7000, 0x8000)
    prm = B.params()
    P = ctypes.byref
    args = lambda k=kv, p=pg, pr=prm, n=1, scr=0x10000, nb=1 << 40: (
        P(k), P(p), 0x9000, n, 0xa000, 0xb000, None, None, 0, None, P(pr), 0xc000, None, scr, nb, 10, None)
    assert lib.gp_boundary_scan(*args(k=_kv(k=None))) == B.GP_ERR_INVALID
    assert lib.gp_boundary_scan(*args(k=_kv(Hq=24))) == B.GP_ERR_UNSUPPORTED      # group of 3
    assert lib.gp_boundary_scan(*args(k=_kv(Hq=64))) == B.GP_ERR_UNSUPPORTED      # group of 8
    assert lib.gp_boundary_scan(*args(k=_kv(Hq=12))) == B.GP_ERR_UNSUPPORTED      # not a multiple
    assert lib.gp_boundary_scan(*args(k=_kv(Hq=4))) == B.GP_ERR_UNSUPPORTED       # fewer than Hkv
    for hq in (8, 16):                                                             # groups of 1 and 2 pass
        assert lib.gp_boundary_scan(*args(k=_kv(Hq=hq), n=-1)) == B.GP_ERR_INVALID
    assert lib.gp_boundary_scan(*args(k=_kv(d=96))) == B.GP_ERR_UNSUPPORTED
    assert lib.gp_boundary_scan(*args(k=_kv(P=12))) == B.GP_ERR_UNSUPPORTED
    assert lib.gp_boundary_scan(*args(k=_kv(stride_tok=64))) == B.GP_ERR_INVALID
    assert lib.gp_boundary_scan(*args(k=_kv(k=0x1008))) == B.GP_ERR_INVALID
    assert lib.gp_boundary_scan(*args(n=-1)) == B.GP_ERR_INVALID
    assert lib.gp_boundary_scan(*args(n=5)) == B.GP_ERR_INVALID          # > max_req
    assert lib.gp_boundary_scan(*args(nb=16)) == B.GP_ERR_SCRATCH
    assert lib.gp_boundary_scan(*args(scr=0x10010)) == B.GP_ERR_INVALID  # scratch alignment
    bad = B.params(beta_s=0.0)
    assert lib.gp_boundary_scan(*args(pr=bad)) == B.GP_ERR_INVALID
    assert lib.gp_boundary_scan(*args(n=0)) == B.GP_OK                   # empty batch: nothing launched
    # rope table without positions
    a = list(args())
    a[6], a[7], a[8] = 0xd000, 0xe000, 100
    assert lib.gp_boundary_scan(*a) == B.GP_ERR_INVALID
    # decide / compact / ema / append
    assert lib.gp_decide(None, 0x9000, 1, 2, 32, 16, P(prm), P(pg), 1, 2, 3, None, None) == B.GP_ERR_INVALID
    assert lib.gp_decide(0x1, 0x9000, 1, 2, 32, 0, P(prm), P(pg), 1, 2, 3, None, None) == B.GP_ERR_INVALID
    assert lib.gp_decide(0x1, 0x9000, 0, 2, 32, 16, P(prm), P(pg), 1, 2, 3, None, None) == B.GP_OK
    nopool = B.Pages(0x3000, 4, 8, 0x4000, 0x5000, None, None, None)
    assert lib.gp_decide(0x1, 0x9000, 1, 2, 32, 16, P(prm), P(nopool), 1, 2, 3, None, None) == B.GP_ERR_INVALID
    assert lib.gp_compact(P(kv), P(pg), 0x9000, 0xa000, 1, P(prm), None, None, None, 0x10000, 1 << 40, 10, None) == B.GP_ERR_INVALID
    assert lib.gp_compact(P(kv), P(pg), 0x9000, 0xa000, 1, P(prm), None, 0xb000, None, 0x10000, 8, 10, None) == B.GP_ERR_SCRATCH
    assert lib.gp_update_summaries(0x1000, 1, 4, 4, 4, 0x2000, 1, 2, 8, 62, 0x3000, 0x4000, P(prm), None) == B.GP_ERR_INVALID
    assert lib.gp_update_summaries(0x1000, 1, 4, 4, 6, 0x2000, 1, 2, 8, 64, 0x3000, 0x4000, P(prm), None) == B.GP_ERR_INVALID
    assert lib.gp_update_summaries(0x1000, 1, 4, 4, 4, 0x2000, 0, 2, 8, 64, 0x3000, 0x4000, P(prm), None) == B.GP_OK
    assert lib.gp_append_kv(P(kv), P(pg), None, 0x10, 0x9000, 1, None, None) == B.GP_ERR_INVALID
    # decode attention: a rotation table needs both halves and the positions
    att = lambda cos, sin, pos: lib.gp_decode_attention(P(kv), P(pg), 0x9000, B.GP_BF16, 4096, 512, 128,
                                                        0xa000, 1, cos, sin, 100, pos, 0xb000, None)
    assert att(None, 0xd000, 0xe000) == B.GP_ERR_INVALID
    assert att(0xd000, None, 0xe000) == B.GP_ERR_INVALID
    assert att(0xd000, 0xd800, None) == B.GP_ERR_INVALID
    # SHRINK: the flag is 0 or 1, and the keep-sets the scan sized must match the policy
    assert lib.gp_boundary_scan(*args(pr=B.params(shrink=2))) == B.GP_ERR_INVALID
    sh = B.params(shrink=1)
    assert lib.gp_decide(0x1, 0x9000, 1, 2, 32, 16, P(sh), P(pg), 1, 2, 3, None, None) == B.GP_ERR_INVALID
    dp = lambda pr, pol: lib.gp_decide_policy(0x1, 0x9000, 0, 2, 32, 16, P(pr), pol, None, 0.0, P(pg),
                                              1, 2, 3, None, None)
    assert dp(sh, B.POLICIES["shrink"]) == B.GP_OK                   # empty batch: nothing launched
    assert dp(prm, B.POLICIES["shrink"]) == B.GP_ERR_INVALID
    assert dp(sh, B.POLICIES["growpage"]) == B.GP_ERR_INVALID
    assert dp(prm, 5) == B.GP_ERR_INVALID
    # more candidate slots per request (max_pages * P) than the keep-set keys index
    big = B.Pages(0x3000, 4, (1 << 24) // 16 + 1, 0x4000, 0x5000, 0x6000, 0x7000, 0x8000)
    assert lib.gp_boundary_scan(*args(p=big)) == B.GP_ERR_UNSUPPORTED
    # logit read-back: entry inside the batch, the scan's scratch size
    sl = lambda entry=0, n=10, nreq=1, scr=0x10000, nb=1 << 40, out=0xf000: lib.gp_scan_logits(
        P(kv), nreq, 10, scr, nb, entry, n, out, None)
    assert sl(entry=1) == B.GP_ERR_INVALID
    assert sl(entry=-1) == B.GP_ERR_INVALID
    assert sl(n=-1) == B.GP_ERR_INVALID
    assert sl(out=None) == B.GP_ERR_INVALID
    assert sl(scr=0x10010) == B.GP_ERR_INVALID
    assert sl(nb=16) == B.GP_ERR_SCRATCH
    assert sl(n=0) == B.GP_OK                                        # nothing to copy: nothing launched


def test_param_struct_matches_header():
    """The binding's gp_params mirror has the header's fields in the header's order."""
    text = open(HEADER).read()
    body = re.search(r"typedef struct gp_params \{(.*?)\} gp_params;", text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"(?:float|int32_t)\s+([\w\s,]+);", body)
    names = [n.strip() for f in fields for n in f.split(",")]
    assert names == [f[0] for f in B.Params._fields_]


def test_single_hip_runtime_after_load():
    """Loading the library through the binding leaves exactly one HIP runtime in the process
    (torch's), whatever was imported before."""
    import subprocess
    import sys
    code = ("import demand_paged_kv_amd.binding as B; B.load(); import torch; "
            "print(len({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"

"""CPU-only checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any HIP call
(no GPU is touched by these tests)."""

import ctypes
import os
import re

import pytest

from gated_delta_rule_61_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        from gated_delta_rule_61_amd import build
        build.build()
    return binding.lib()


def declared_functions():
    names = []
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if not h.endswith(".h"):
            continue
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"gdn_chunk_fwd", "kda_chunk_fwd", "gdn_decode"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared but not exported"


def test_version_and_status_strings(L):
    assert L.gdn_version().startswith(b"gdn61")
    assert L.gdn_status_string(0) == b"ok"
    assert L.gdn_status_string(1) == b"invalid argument"
    assert L.gdn_status_string(99) == b"unknown status"


def test_status_numbering():
    """The planned numbering (OK 0, invalid argument 1, unsupported 2, launch
    3), with the workspace code appended as 4."""
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "gdn61.h")).read(), flags=re.S)
    codes = dict((n, int(v)) for n, v in re.findall(r"(GDN_(?:OK|ERR_[A-Z_]+))\s*=\s*(\d+)", src))
    assert codes == {"GDN_OK": 0, "GDN_ERR_INVALID_ARGUMENT": 1, "GDN_ERR_UNSUPPORTED": 2,
                     "GDN_ERR_LAUNCH": 3, "GDN_ERR_WORKSPACE": 4}
    L = binding.lib()
    assert L.gdn_status_string(3) == b"kernel launch failed"
    assert L.gdn_status_string(4) == b"workspace too small"


def _chunk(L, **kw):
    a = dict(q=None, k=None, v=None, g=None, gg=None, beta=None, scale=1.0, h0=None, ht=None, hs=None, ss=0, se=1 << 30,
             sdt=0, cu=None, ns=0, B=1, T=64, Hk=2, HV=2, K=64, V=64, cs=64, dt=1, o=None, ws=None, wsb=0, st=None)
    a.update(kw)
    return L.gdn_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["gg"], a["beta"], a["scale"], a["h0"], a["ht"],
                           a["hs"], a["ss"], a["se"], a["sdt"], a["cu"], a["ns"], a["B"], a["T"], a["Hk"], a["HV"],
                           a["K"], a["V"], a["cs"], a["dt"], a["o"], a["ws"], a["wsb"], a["st"])


FAKE = 1 << 20  # a 16-byte-aligned non-null address; never dereferenced (checks fail first)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(cs=32), 2, b"chunk_size"),
    (dict(K=96, V=96), 2, b"head dims"),
    (dict(Hk=3, HV=4), 1, b"multiple"),
    (dict(dt=7), 1, b"dtype"),
    (dict(B=-1), 1, b"sizes"),
    (dict(B=2, cu=FAKE, ns=3), 1, b"B == 1"),
    (dict(), 1, b"required"),
    (dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, o=FAKE), 4, b"workspace"),
    (dict(q=FAKE + 4, k=FAKE, v=FAKE, beta=FAKE, o=FAKE, ws=FAKE, wsb=1 << 40), 1, b"aligned"),
    (dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, o=FAKE, hs=FAKE, ss=96), 1, b"split_size"),
    (dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, o=FAKE, g=FAKE, gg=FAKE, ws=FAKE, wsb=1 << 40), 1, b"not both"),
    (dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, o=FAKE, hs=FAKE, ss=0), 1, b"split_size"),
    (dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, o=FAKE, hs=FAKE + 8, ss=64, ws=FAKE, wsb=1 << 40), 1, b"aligned"),
    # an undersized snapshot buffer (dense: B * ceil(T / split) = 2 * 3 entries needed) is rejected
    (dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, o=FAKE, hs=FAKE, ss=64, se=5, B=2, T=130, ws=FAKE, wsb=1 << 40),
     1, b"6 needed"),
    (dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, o=FAKE, hs=FAKE, ss=64, sdt=5, ws=FAKE, wsb=1 << 40), 1, b"state dtype"),
])
def test_chunk_fwd_rejects(L, kw, status, msg):
    assert _chunk(L, **kw) == status
    assert msg in L.gdn_last_error()


def test_kda_requires_gate(L):
    r = L.kda_chunk_fwd(FAKE, FAKE, FAKE, None, FAKE, 1.0, None, None, None, 0, 0, 0, None, 0, 1, 64, 1, 1, 64, 64,
                        64, 1, FAKE, None, None, FAKE, 1 << 40, None)
    assert r == 1 and b"gk" in L.gdn_last_error()


def test_kda_rejects_planes_past_32_bit_offsets(L):
    # one head's gated planes span B*T*K*2 bytes, addressed with 32-bit offsets: 2^24 tokens at K = 128 is too many
    r = L.kda_chunk_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, None, None, None, 0, 0, 0, None, 0, 1, 1 << 24, 1, 1, 128,
                        128, 64, 1, FAKE, None, None, FAKE, 1 << 44, None)
    assert r == 2 and b"too large for KDA" in L.gdn_last_error()


def test_launch_index_range_is_checked(L):
    """Grids are indexed with 32-bit integers: shapes whose work-group count
    would pass 2^31 are refused before any launch."""
    # 2^28 packed sequences x 8 heads
    assert _chunk(L, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, o=FAKE, cu=FAKE, ns=1 << 28, HV=8, Hk=8,
                  ws=FAKE, wsb=1 << 60) == 2
    assert b"for one launch" in L.gdn_last_error()
    # 2^24 dense sequences of one token x 32 heads
    assert _chunk(L, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, o=FAKE, B=1 << 24, T=1, HV=32, Hk=32,
                  ws=FAKE, wsb=1 << 60) == 2
    assert b"for one launch" in L.gdn_last_error()
    for fwd in (False, True):
        assert _bwd(L, fwd=fwd, cu=FAKE, ns=1 << 27, HV=4, Hk=4) == 2
        assert b"for one launch" in L.gdn_last_error()
    assert _dec(L, B=1 << 25, HV=16, H=16, idx=FAKE) == 2
    assert b"for one launch" in L.gdn_last_error()


def _intra(L, **kw):
    a = dict(k=FAKE, v=FAKE, g=None, gc=0, beta=FAKE, cu=None, ns=0, B=1, T=64, Hk=1, HV=2, K=64, V=64, cs=64,
             dt=1, A=FAKE, w=None, u=None, ws=None, wsb=0)
    a.update(kw)
    return L.gdn_chunk_intra(a["k"], a["v"], a["g"], a["gc"], a["beta"], a["cu"], a["ns"], a["B"], a["T"], a["Hk"],
                             a["HV"], a["K"], a["V"], a["cs"], a["dt"], a["A"], a["w"], a["u"], a["ws"], a["wsb"],
                             None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(cs=32), 2, b"chunk_size"),
    (dict(K=96), 2, b"head dims"),
    (dict(Hk=3, HV=4), 1, b"multiple"),
    (dict(dt=5), 1, b"dtype"),
    (dict(gc=2), 1, b"g_cumulative"),
    (dict(A=None), 1, b"required"),
    (dict(u=FAKE, v=None), 1, b"v is required"),
    (dict(w=FAKE + 8), 1, b"aligned"),
    (dict(cu=FAKE, ns=3), 4, b"workspace"),
    (dict(cu=FAKE, ns=3, ws=FAKE + 16, wsb=1 << 20), 1, b"256-byte"),
    (dict(B=2, cu=FAKE, ns=3), 1, b"B == 1"),
])
def test_chunk_intra_rejects(L, kw, status, msg):
    assert _intra(L, **kw) == status
    assert msg in L.gdn_last_error()


def test_chunk_intra_workspace_query(L):
    assert L.gdn_chunk_intra_workspace_bytes(0) == 256
    assert L.gdn_chunk_intra_workspace_bytes(100) == 1024
    assert L.gdn_chunk_intra_workspace_bytes(-1) == 0


def test_kda_rejects_undersized_snapshots(L):
    r = L.kda_chunk_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, None, None, FAKE, 128, 1, 0, None, 0, 2, 64, 1, 1, 64, 64,
                        64, 1, FAKE, None, None, FAKE, 1 << 40, None)
    assert r == 1 and b"2 needed" in L.gdn_last_error()


def _dec(L, **kw):
    a = dict(ptr=FAKE, idx=None, B=2, T=1, H=1, HV=2, K=128, V=128, pool=2, sb=1.0, thr=20.0, eps=1e-6)
    a.update(kw)
    p = a["ptr"]
    return L.gdn_decode(p, p, p, p, p, p, p, p, a["idx"], p, a["B"], a["T"], a["H"], a["HV"], a["K"],
                        a["V"], a["pool"], 1.0, a["sb"], a["thr"], 1, a["eps"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(T=0), 1, b"T = 1..4"),
    (dict(T=5), 1, b"T = 1..4"),
    (dict(K=64, V=64), 2, b"K = V = 128"),
    (dict(H=3, HV=4), 1, b"multiple"),
    (dict(pool=1), 1, b"pool >= B"),
    (dict(sb=0.0), 1, b"softplus_beta"),
    (dict(ptr=None), 1, b"required"),
    (dict(ptr=FAKE + 2), 1, b"aligned"),
])
def test_decode_rejects(L, kw, status, msg):
    assert _dec(L, **kw) == status
    assert msg in L.gdn_last_error()


def test_workspace_query(L):
    n = L.gdn_chunk_fwd_workspace_bytes(4, 4096, 16, 16, 128, 128, 4, 1)
    assert n >= 2 * 4 * 4096 * 16 * 64 * 2
    assert n % 256 == 0
    assert L.gdn_chunk_fwd_workspace_bytes(1, 64, 1, 1, 64, 64, 1, 9) == 0
    assert L.kda_chunk_fwd_workspace_bytes(1, 64, 1, 1, 64, 64, 1, 1) > 0


def test_binding_raises_without_cuda_tensors():
    import torch
    q = torch.zeros(1, 4, 1, 64)
    with pytest.raises(ValueError):
        binding.gdn_chunk_fwd(q, q, q, None, torch.zeros(1, 4, 1))


def _pool(L, ht=None, idx=None, pool_state=None, N=2, HV=2, K=128, V=128, pool=2, st=None):
    return L.gdn_state_to_pool(ht, idx, pool_state, N, HV, K, V, pool, st)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(N=-1), 1, b"sizes must be positive"),
    (dict(HV=0), 1, b"sizes must be positive"),
    (dict(K=3, V=5, ht=FAKE, pool_state=FAKE), 2, b"multiple of 8"),
    (dict(pool=1, ht=FAKE, pool_state=FAKE), 1, b"pool >= N"),
    (dict(ht=None, pool_state=FAKE), 1, b"required"),
    (dict(ht=FAKE + 4, pool_state=FAKE), 1, b"16-byte aligned"),
])
def test_state_to_pool_rejects(L, kw, status, msg):
    assert _pool(L, **kw) == status
    assert msg in L.gdn_last_error()


def test_state_to_pool_empty_is_a_no_op(L):
    assert _pool(L, N=0, pool=0) == 0


def _bwd(L, q=FAKE, do=FAKE, g=None, gg=None, gk=None, gv=None, hg=0, dht=None, dh=None, ss=64, se=1 << 30, sdt=0,
         vf=1, dh0=FAKE, cu=None, ns=0, B=1, T=64, Hk=1, HV=1, K=64, V=64, cs=64, dt=1, fwd=False):
    f = L.gdn_chunk_fwd_h if fwd else L.gdn_chunk_bwd_dh
    if fwd:
        return f(q, do, g, gg, gk, gv, hg, dht, dh, ss, se, sdt, vf, dh0, cu, ns, B, T, Hk, HV, K, V, cs, dt, None)
    return f(q, do, g, gg, gk, gv, hg, 1.0, dht, dh, ss, se, sdt, vf, dh0, cu, ns, B, T, Hk, HV, K, V, cs, dt, None)


@pytest.mark.parametrize("fwd", [False, True])
@pytest.mark.parametrize("kw,status,msg", [
    (dict(dt=0), 2, b"bf16 io only"),
    (dict(g=FAKE, gk=FAKE), 1, b"at most one"),
    (dict(gk=FAKE, gv=FAKE), 2, b"gk together with gv"),
    (dict(dh=FAKE, ss=0), 1, b"split_size"),
    (dict(K=96, V=96), 2, b"head dims"),
    (dict(q=None), 1, b"required"),
    (dict(do=FAKE + 2), 1, b"aligned"),
    (dict(gv=FAKE + 4), 1, b"aligned"),
    (dict(B=2, cu=FAKE, ns=2), 1, b"B == 1"),
    (dict(HV=4, Hk=4, hg=3), 1, b"gate heads"),
    (dict(dh=FAKE, B=3, T=100, se=5), 1, b"6 needed"),
    (dict(dh=FAKE, sdt=2), 1, b"state dtype"),
    (dict(vf=2), 1, b"state_v_first"),
])
def test_state_scans_reject(L, kw, status, msg, fwd):
    assert _bwd(L, fwd=fwd, **kw) == status
    assert msg in L.gdn_last_error()


@pytest.mark.parametrize("fwd", [False, True])
def test_state_scans_nothing_to_do(L, fwd):
    # no sequences, or no output requested: returns before any HIP call
    assert _bwd(L, fwd=fwd, B=0) == 0
    assert _bwd(L, fwd=fwd, dh0=None) == 0


def test_snapshot_count_reads_no_device_memory(monkeypatch):
    """No binding path synchronises the host: the varlen snapshot count takes
    host boundaries only (a device -- here a meta -- tensor is refused, and
    Tensor.cpu is never called)."""
    import torch

    def no_cpu(*a, **k):
        raise AssertionError("Tensor.cpu called")

    monkeypatch.setattr(torch.Tensor, "cpu", no_cpu)
    assert binding.snapshot_count(2, 130, 64) == 6
    assert binding.snapshot_count(1, 400, 64, [0, 130, 194, 195, 400]) == 3 + 1 + 1 + 4
    assert binding.snapshot_count(1, 400, 128, torch.tensor([0, 130, 194, 195, 400])) == 2 + 1 + 1 + 2
    # invalid boundaries clamp per sequence into [0, T] with the end not below
    # the start, as the device tables do: (0, 300), empty, (0, 300), empty, (0, 300)
    assert binding.snapshot_count(1, 300, 64, [-7, 300, 0, 300, 0, 1000]) == 5 + 0 + 5 + 0 + 5
    with pytest.raises(ValueError):
        binding.snapshot_count(1, 400, 64, torch.zeros(5, dtype=torch.int64, device="meta"))


def test_binding_sources_never_copy_to_host():
    src = open(os.path.join(ROOT, "gated_delta_rule_61_amd", "binding.py")).read()
    for pat in (".cpu(", ".item(", ".tolist(", "numpy("):
        hits = [l for l in src.splitlines() if pat in l and "cu_seqlens_host" not in l]
        assert not hits, hits

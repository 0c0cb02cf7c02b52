"""GPU regression test of the varlen contract for invalid boundaries: values
below 0 or past T, boundaries that go backwards, and sequences that overlap so
that their chunks (15 here) outnumber the ceil(T / 64) + N rows (10) of the
chunk and decay-row tables.  Every entry point must still return OK and keep
every access inside the caller's buffers: the guard cells around each output
and around the workspace stay untouched, stored states past a buffer's
capacity are skipped, and an empty sequence returns its initial state
unchanged.  Other results of such a call are unspecified (overlapping
sequences race on the rows they share), so nothing else is compared."""

import ctypes

import pytest
import torch

from gated_delta_rule_61_amd import binding

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GUARD = 4096             # guard elements on each side of every output
SENT = 7.0               # guard value of float outputs
SENT_BYTE = 0x5A         # guard value of the workspace
T = 300
# after clamping: (0, 300), (300, 300) empty, (0, 300), (300, 300) empty, (0, 300)
CU = [-7, 300, 0, 300, 0, 1000]
N = len(CU) - 1
EMPTY = (1, 3)
HK, HV, K = 2, 4, 64


def _guarded(shape, dtype, fill=SENT):
    n = 1
    for s in shape:
        n *= s
    buf = torch.full((n + 2 * GUARD,), fill, dtype=dtype, device=DEV)
    return buf, buf[GUARD:GUARD + n].view(shape)


def _guards_ok(buf, fill=SENT):
    return bool((buf[:GUARD] == fill).all().item() and (buf[-GUARD:] == fill).all().item())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _inputs(seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=gen, device=DEV)
    q = torch.nn.functional.normalize(r(1, T, HK, K), dim=-1).to(torch.bfloat16)
    k = torch.nn.functional.normalize(r(1, T, HK, K), dim=-1).to(torch.bfloat16)
    v = r(1, T, HV, K).to(torch.bfloat16)
    g = -torch.nn.functional.softplus(r(1, T, HV)) * 0.1
    gk = -torch.nn.functional.softplus(r(1, T, HV, K)) * 0.05
    beta = torch.sigmoid(r(1, T, HV))
    h0 = r(N, HV, K, K) * 0.1
    cu = torch.tensor(CU, dtype=torch.int64, device=DEV)
    return q, k, v, g, gk, beta, h0, cu


@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
def test_prefill_invalid_boundaries_stay_in_bounds(kda):
    print(f"prefill with invalid cu_seqlens {CU}, kda={kda}", flush=True)
    q, k, v, g, gk, beta, h0, cu = _inputs(300 + kda)
    L = binding.lib()
    ob, o = _guarded((1, T, HV, K), torch.bfloat16)
    hb, ht = _guarded((N, HV, K, K), torch.float32)
    sb, hs = _guarded((8, HV, K, K), torch.float32)   # 15 snapshots would be due: 7 are skipped
    nbytes = binding.workspace_bytes(1, T, HK, HV, K, K, N, torch.bfloat16, kda=kda)
    wb, ws = _guarded((nbytes,), torch.uint8, SENT_BYTE)
    common = (ctypes.c_float(K ** -0.5), _p(h0), _p(ht), _p(hs), 64, hs.shape[0], binding.GDN_DTYPE_F32, _p(cu), N,
              1, T, HK, HV, K, K, 64, binding.GDN_DTYPE_BF16, _p(o))
    if kda:
        ab, aqk = _guarded((1, T, HV, 64), torch.bfloat16)
        kb, akk = _guarded((1, T, HV, 64), torch.bfloat16)
        st = L.kda_chunk_fwd(_p(q), _p(k), _p(v), _p(gk), _p(beta), *common, _p(aqk), _p(akk), _p(ws),
                             ctypes.c_size_t(nbytes), _stream())
    else:
        st = L.gdn_chunk_fwd(_p(q), _p(k), _p(v), _p(g), None, _p(beta), *common, _p(ws), ctypes.c_size_t(nbytes),
                             _stream())
    assert st == 0, L.gdn_last_error()
    torch.cuda.synchronize()
    for name, buf in (("o", ob), ("ht", hb), ("h_snap", sb)) + ((("Aqk", ab), ("Akk_inv", kb)) if kda else ()):
        assert _guards_ok(buf), f"{name}: a guard cell was written"
    assert _guards_ok(wb, SENT_BYTE), "workspace: a guard byte was written"
    for n in EMPTY:
        assert torch.equal(ht[n], h0[n]), f"empty sequence {n}: ht differs from h0"


@pytest.mark.parametrize("vf", [1, 0], ids=["v_first", "k_first"])
@pytest.mark.parametrize("fwd", [False, True], ids=["bwd_dh", "fwd_h"])
def test_state_scan_invalid_boundaries_stay_in_bounds(fwd, vf):
    print(f"state scan with invalid cu_seqlens {CU}, forward={fwd}, state_v_first={vf}", flush=True)
    q, k, v, g, gk, beta, h0, cu = _inputs(310 + fwd)
    L = binding.lib()
    sb, hs = _guarded((8, HV, K, K), torch.bfloat16)
    fb, fin = _guarded((N, HV, K, K), torch.float32)
    a, b = (k, v) if fwd else (q, v)
    if fwd:
        st = L.gdn_chunk_fwd_h(_p(a), _p(b), _p(g), None, None, None, HV, _p(h0), _p(hs), 64, hs.shape[0],
                               binding.GDN_DTYPE_BF16, vf, _p(fin), _p(cu), N, 1, T, HK, HV, K, K, 64,
                               binding.GDN_DTYPE_BF16, _stream())
    else:
        st = L.gdn_chunk_bwd_dh(_p(a), _p(b), _p(g), None, None, None, HV, ctypes.c_float(K ** -0.5), _p(h0),
                                _p(hs), 64, hs.shape[0], binding.GDN_DTYPE_BF16, vf, _p(fin), _p(cu), N, 1, T, HK, HV,
                                K, K, 64, binding.GDN_DTYPE_BF16, _stream())
    assert st == 0, L.gdn_last_error()
    torch.cuda.synchronize()
    assert _guards_ok(sb), "stored states: a guard cell was written"
    assert _guards_ok(fb), "final states: a guard cell was written"
    for n in EMPTY:
        assert torch.equal(fin[n], h0[n]), f"empty sequence {n}: final state differs from the initial one"

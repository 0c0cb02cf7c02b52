"""Thin Python binding of ``libgdn61.so`` (ctypes).

Argument marshalling only: the functions below check tensor placement,
dtypes and shapes, allocate outputs and workspace with PyTorch, and pass raw
device pointers plus the current HIP stream to the C ABI declared in
``include/gdn61.h``.  Every step of the computation runs in the library's
gfx950 kernels; there is no fallback path -- if the library is missing or
fails to load, every entry point raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn61.so")

GDN_DTYPE_F32 = 0
GDN_DTYPE_BF16 = 1

_c_void_p = ctypes.c_void_p
_c_int = ctypes.c_int
_c_float = ctypes.c_float
_c_size_t = ctypes.c_size_t
_c_ll = ctypes.c_longlong

_SIGNATURES = {
    "gdn_status_string": (ctypes.c_char_p, [_c_int]),
    "gdn_last_error": (ctypes.c_char_p, []),
    "gdn_version": (ctypes.c_char_p, []),
    "gdn_chunk_fwd_workspace_bytes": (_c_size_t, [_c_int] * 8),
    "kda_chunk_fwd_workspace_bytes": (_c_size_t, [_c_int] * 8),
    "gdn_chunk_fwd": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_float,
                               _c_void_p, _c_void_p, _c_void_p, _c_int, _c_ll, _c_int, _c_void_p, _c_int,
                               _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                               _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "kda_chunk_fwd": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_float,
                               _c_void_p, _c_void_p, _c_void_p, _c_int, _c_ll, _c_int, _c_void_p, _c_int,
                               _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                               _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "gdn_chunk_fwd_noalloc": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                       _c_float, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_ll, _c_int,
                                       _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_int, _c_void_p, _c_void_p]),
    "gdn_chunk_fwd_noalloc_max_bytes": (_c_size_t, []),
    "gdn_profile_enable": (_c_int, [_c_int]),
    "gdn_profile_read": (_c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_c_int)]),
    "gdn_decode": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                            _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                            _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                            _c_float, _c_float, _c_float, _c_int, _c_float, _c_void_p]),
    "gdn_chunk_bwd_dh": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int,
                                  _c_float, _c_void_p, _c_void_p, _c_int, _c_ll, _c_int, _c_int, _c_void_p,
                                  _c_void_p, _c_int,
                                  _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                  _c_void_p]),
    "gdn_chunk_fwd_h": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int,
                                 _c_void_p, _c_void_p, _c_int, _c_ll, _c_int, _c_int, _c_void_p, _c_void_p, _c_int,
                                 _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                 _c_void_p]),
    "gdn_chunk_intra_workspace_bytes": (_c_size_t, [_c_int]),
    "gdn_chunk_intra": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_void_p, _c_void_p, _c_int,
                                 _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                 _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "gdn_state_to_pool": (_c_int, [_c_void_p, _c_void_p, _c_void_p,
                                   _c_int, _c_int, _c_int, _c_int, _c_int, _c_void_p]),
}

_lib = None


class GDNError(RuntimeError):
    """A call into the library returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def lib() -> ctypes.CDLL:
    """Load (once) and return the library; raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m gated_delta_rule_61_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        L = lib()
        raise GDNError(status, f"{L.gdn_status_string(status).decode()}: {L.gdn_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _io_code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return GDN_DTYPE_BF16
    if dtype == torch.float32:
        return GDN_DTYPE_F32
    raise TypeError(f"io dtype must be bfloat16 or float32, got {dtype}")


def _need(t: Optional[torch.Tensor], name: str, dtype: Optional[torch.dtype], shape, device) -> None:
    if t is None:
        return
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


STAGES = ("varlen_tables", "intra", "scan", "decode", "handoff", "bwd_dh", "fwd_h")


def profile_enable(on: bool = True) -> None:
    """Record HIP events around every kernel the library launches."""
    _check(lib().gdn_profile_enable(1 if on else 0))


def profile_read() -> dict:
    """Wait for the recorded events; return {stage: (total_ms, launches)}."""
    ms = (ctypes.c_double * len(STAGES))()
    cnt = (_c_int * len(STAGES))()
    _check(lib().gdn_profile_read(ms, cnt))
    return {name: (ms[i], cnt[i]) for i, name in enumerate(STAGES)}


def workspace_bytes(B: int, T: int, Hk: int, HV: int, K: int, V: int, num_seqs: int,
                    dtype: torch.dtype, kda: bool = False) -> int:
    fn = lib().kda_chunk_fwd_workspace_bytes if kda else lib().gdn_chunk_fwd_workspace_bytes
    return int(fn(B, T, Hk, HV, K, V, num_seqs, _io_code(dtype)))


def _chunk_common(q, k, v, beta, h0, cu_seqlens, chunk_size, gate, gate_shape_tail, gate_name):
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4:
        raise ValueError("q, k must be [B, T, Hk, K] and v [B, T, HV, V]")
    B, T, Hk, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    dev = q.device
    io = q.dtype
    _io_code(io)
    _need(q, "q", io, None, dev)
    _need(k, "k", io, None, dev)
    _need(v, "v", io, (B, T, HV, V), dev)
    _need(beta, "beta", torch.float32, (B, T, HV), dev)
    _need(gate, gate_name, torch.float32, (B, T, HV) + gate_shape_tail, dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int64, None, dev)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    _need(h0, "h0", torch.float32, (N, HV, V, K), dev)
    return B, T, Hk, HV, K, V, N, dev, io


def snapshot_count(B: int, T: int, split_size: int, cu_seqlens_host=None) -> int:
    """Number of stored states of a call: sum over sequences of
    ceil(length / split_size).  Varlen batches need the boundaries on the
    HOST (a list or a CPU tensor): nothing here reads device memory, so no
    call synchronises the host."""
    if cu_seqlens_host is None:
        return B * ((T + split_size - 1) // split_size)
    if isinstance(cu_seqlens_host, torch.Tensor):
        if cu_seqlens_host.device.type != "cpu":
            raise ValueError("snapshot_count needs the boundaries in host memory (a list or CPU tensor)")
        cu_seqlens_host = cu_seqlens_host.tolist()
    cu = [min(max(int(c), 0), T) for c in cu_seqlens_host]
    return sum((max(b - a, 0) + split_size - 1) // split_size for a, b in zip(cu[:-1], cu[1:]))


def _state_dtype(io: torch.dtype, states_in_fp32: bool) -> torch.dtype:
    """Stored states in the input dtype unless ``states_in_fp32``."""
    return torch.float32 if states_in_fp32 else io


def _states(B, T, HV, V, K, N, dev, split_size, buf, name, varlen, cu_seqlens_cpu, dtype):
    """The stored-state buffer of a call: the caller's (any capacity; the
    library writes no entry past it) or a new one.  A varlen call allocates
    only with the host copy of its boundaries."""
    if split_size is None:
        if buf is not None:
            raise ValueError(f"{name} given without split_size")
        return None
    if split_size <= 0 or split_size % 64:
        raise ValueError("split_size must be a positive multiple of 64")
    if buf is None:
        if varlen and cu_seqlens_cpu is None:
            raise ValueError(f"a varlen call with split_size needs a preallocated {name} or cu_seqlens_cpu "
                             f"(the host copy of cu_seqlens); at most ceil(T / split_size) + N entries are used")
        n = snapshot_count(B, T, split_size, cu_seqlens_cpu if varlen else None)
        buf = torch.empty((n, HV, V, K), dtype=dtype, device=dev)
    if buf.dim() != 4:
        raise ValueError(f"{name} must be [S, HV, V, K]")
    _need(buf, name, dtype, (buf.shape[0], HV, V, K), dev)
    return buf


def _dtype_code(dt: torch.dtype) -> int:
    return GDN_DTYPE_BF16 if dt == torch.bfloat16 else GDN_DTYPE_F32


def gdn_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: Optional[torch.Tensor],
                  beta: torch.Tensor, scale: Optional[float] = None,
                  h0: Optional[torch.Tensor] = None, output_final_state: bool = True,
                  cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = 64,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  split_size: Optional[int] = None, h_snap: Optional[torch.Tensor] = None,
                  g_gamma: Optional[torch.Tensor] = None, states_in_fp32: bool = False,
                  cu_seqlens_cpu=None):
    """GDN chunked prefill.  Returns (o [B,T,HV,V], ht [N,HV,V,K] fp32 or None),
    and the state snapshots [S,HV,V,K] as a third element when
    ``split_size`` is given: in the io dtype, or fp32 with
    ``states_in_fp32``.  ``h_snap`` may be passed preallocated (with
    ``cu_seqlens``, either it or ``cu_seqlens_cpu``, the host copy of the
    boundaries, is required).  ``g_gamma`` [HV] (fp32) is a fixed per-head
    log-decay at every token, in place of ``g``."""
    B, T, Hk, HV, K, V, N, dev, io = _chunk_common(q, k, v, beta, h0, cu_seqlens, chunk_size, g, (), "g")
    if g_gamma is not None:
        if g is not None:
            raise ValueError("pass g or g_gamma, not both")
        _need(g_gamma, "g_gamma", torch.float32, (HV,), dev)
    sdt = _state_dtype(io, states_in_fp32)
    hs = _states(B, T, HV, V, K, N, dev, split_size, h_snap, "h_snap", cu_seqlens is not None, cu_seqlens_cpu, sdt)
    if scale is None:
        scale = K ** -0.5
    o = torch.empty((B, T, HV, V), dtype=io, device=dev) if out is None else out
    _need(o, "out", io, (B, T, HV, V), dev)
    ht = torch.empty((N, HV, V, K), dtype=torch.float32, device=dev) if output_final_state else None
    nbytes = workspace_bytes(B, T, Hk, HV, K, V, N, io)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(lib().gdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(g_gamma), _ptr(beta), float(scale),
                               _ptr(h0), _ptr(ht), _ptr(hs), split_size or 0,
                               0 if hs is None else hs.shape[0], _dtype_code(sdt), _ptr(cu_seqlens), N,
                               B, T, Hk, HV, K, V, chunk_size, _io_code(io),
                               _ptr(o), _ptr(workspace), workspace.numel(), _stream(dev)))
    return (o, ht) if hs is None else (o, ht, hs)


def gdn_chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: Optional[torch.Tensor],
                          beta: torch.Tensor, out: torch.Tensor, ht: Optional[torch.Tensor] = None,
                          scale: Optional[float] = None, h0: Optional[torch.Tensor] = None,
                          cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = 64,
                          split_size: Optional[int] = None, h_snap: Optional[torch.Tensor] = None,
                          g_gamma: Optional[torch.Tensor] = None) -> None:
    """``gdn_chunk_fwd`` through the library's no-allocation entry point: the
    caller passes every output (``out`` [B,T,HV,V], optional ``ht`` [N,HV,V,K]
    fp32 and ``h_snap`` with its ``split_size``; the snapshot dtype is
    ``h_snap``'s), and no workspace: the library uses its own per-GPU scratch
    (``noalloc_max_bytes()``).  Allocates nothing."""
    B, T, Hk, HV, K, V, N, dev, io = _chunk_common(q, k, v, beta, h0, cu_seqlens, chunk_size, g, (), "g")
    if g_gamma is not None:
        _need(g_gamma, "g_gamma", torch.float32, (HV,), dev)
    _need(out, "out", io, (B, T, HV, V), dev)
    _need(ht, "ht", torch.float32, (N, HV, V, K), dev)
    if h_snap is not None:
        if split_size is None or split_size <= 0 or split_size % 64:
            raise ValueError("h_snap needs split_size, a positive multiple of 64")
        if h_snap.dim() != 4 or h_snap.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("h_snap must be [S, HV, V, K] fp32 or bf16")
        _need(h_snap, "h_snap", h_snap.dtype, (h_snap.shape[0], HV, V, K), dev)
    if scale is None:
        scale = K ** -0.5
    _check(lib().gdn_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(g_gamma), _ptr(beta), float(scale),
                                       _ptr(h0), _ptr(ht), _ptr(h_snap), split_size or 0,
                                       0 if h_snap is None else h_snap.shape[0],
                                       GDN_DTYPE_F32 if h_snap is None else _dtype_code(h_snap.dtype),
                                       _ptr(cu_seqlens), N, B, T, Hk, HV, K, V, chunk_size, _io_code(io),
                                       _ptr(out), _stream(dev)))


def noalloc_max_bytes() -> int:
    """Scratch bytes of the no-allocation entry point (per GPU)."""
    return int(lib().gdn_chunk_fwd_noalloc_max_bytes())


def kda_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gk: torch.Tensor,
                  beta: torch.Tensor, scale: Optional[float] = None,
                  h0: Optional[torch.Tensor] = None, output_final_state: bool = True,
                  cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = 64,
                  return_intra: bool = True, workspace: Optional[torch.Tensor] = None,
                  split_size: Optional[int] = None, h_snap: Optional[torch.Tensor] = None,
                  states_in_fp32: bool = False, cu_seqlens_cpu=None):
    """KDA chunked prefill.  Returns (o, ht, Aqk, Akk_inv); the last two are
    [B,T,HV,64] in the io dtype (None when ``return_intra`` is False).  With
    ``split_size`` the state snapshots follow as a fifth element (dtype and
    buffer rules as in ``gdn_chunk_fwd``)."""
    if gk is None:
        raise ValueError("gk is required")
    B, T, Hk, HV, K, V, N, dev, io = _chunk_common(q, k, v, beta, h0, cu_seqlens, chunk_size, gk,
                                                   (q.shape[-1],), "gk")
    sdt = _state_dtype(io, states_in_fp32)
    hs = _states(B, T, HV, V, K, N, dev, split_size, h_snap, "h_snap", cu_seqlens is not None, cu_seqlens_cpu, sdt)
    if scale is None:
        scale = K ** -0.5
    o = torch.empty((B, T, HV, V), dtype=io, device=dev)
    ht = torch.empty((N, HV, V, K), dtype=torch.float32, device=dev) if output_final_state else None
    Aqk = Akk = None
    if return_intra:
        Aqk = torch.empty((B, T, HV, chunk_size), dtype=io, device=dev)
        Akk = torch.empty((B, T, HV, chunk_size), dtype=io, device=dev)
    nbytes = workspace_bytes(B, T, Hk, HV, K, V, N, io, kda=True)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(lib().kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(gk), _ptr(beta), float(scale),
                               _ptr(h0), _ptr(ht), _ptr(hs), split_size or 0,
                               0 if hs is None else hs.shape[0], _dtype_code(sdt), _ptr(cu_seqlens), N,
                               B, T, Hk, HV, K, V, chunk_size, _io_code(io),
                               _ptr(o), _ptr(Aqk), _ptr(Akk), _ptr(workspace), workspace.numel(),
                               _stream(dev)))
    return (o, ht, Aqk, Akk) if hs is None else (o, ht, Aqk, Akk, hs)


def gdn_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, a: torch.Tensor, b: torch.Tensor,
               A_log: torch.Tensor, dt_bias: torch.Tensor, state: torch.Tensor,
               state_indices: Optional[torch.Tensor] = None, scale: Optional[float] = None,
               softplus_beta: float = 1.0, softplus_threshold: float = 20.0,
               use_qk_l2norm: bool = True, eps: float = 1e-6,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode T = 1..4 tokens; ``state`` [pool,HV,V,K] bf16 is updated in place.
    Returns o [B,T,HV,V] bf16."""
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, K]")
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    dev = q.device
    bf = torch.bfloat16
    _need(q, "q", bf, None, dev)
    _need(k, "k", bf, (B, T, H, K), dev)
    _need(v, "v", bf, (B, T, HV, V), dev)
    _need(a, "a", bf, (B, T, HV), dev)
    _need(b, "b", bf, (B, T, HV), dev)
    _need(A_log, "A_log", torch.float32, (HV,), dev)
    _need(dt_bias, "dt_bias", torch.float32, (HV,), dev)
    if state.dim() != 4:
        raise ValueError("state must be [pool, HV, V, K]")
    _need(state, "state", bf, (state.shape[0], HV, V, K), dev)
    if state_indices is not None:
        if state_indices.dtype != torch.int32:
            state_indices = state_indices.to(torch.int32)
        _need(state_indices, "state_indices", torch.int32, (B,), dev)
    if scale is None:
        scale = K ** -0.5
    o = torch.empty((B, T, HV, V), dtype=bf, device=dev) if out is None else out
    _need(o, "out", bf, (B, T, HV, V), dev)
    _check(lib().gdn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
                            _ptr(state), _ptr(state_indices), _ptr(o),
                            B, T, H, HV, K, V, state.shape[0],
                            float(scale), float(softplus_beta), float(softplus_threshold),
                            1 if use_qk_l2norm else 0, float(eps), _stream(dev)))
    return o


def gdn_chunk_intra(k: torch.Tensor, v: torch.Tensor, g: Optional[torch.Tensor], beta: torch.Tensor,
                    cu_seqlens: Optional[torch.Tensor] = None, g_cumulative: bool = False,
                    output_wu: bool = True, chunk_size: int = 64,
                    workspace: Optional[torch.Tensor] = None):
    """The scalar-gate intra-chunk step: returns (w [B,T,HV,K], u [B,T,HV,V],
    A [B,T,HV,64]) in the io dtype, w and u None without ``output_wu``.  ``g``
    holds per-token log-gates, or with ``g_cumulative`` their chunk-local
    cumulative sums."""
    if k.dim() != 4 or v.dim() != 4:
        raise ValueError("k must be [B, T, Hk, K] and v [B, T, HV, V]")
    B, T, Hk, K = k.shape
    HV, V = v.shape[2], v.shape[3]
    dev, io = k.device, k.dtype
    _io_code(io)
    _need(k, "k", io, None, dev)
    _need(v, "v", io, (B, T, HV, V), dev)
    _need(g, "g", torch.float32, (B, T, HV), dev)
    _need(beta, "beta", torch.float32, (B, T, HV), dev)
    N = B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int64, None, dev)
        N = cu_seqlens.numel() - 1
    A = torch.empty((B, T, HV, chunk_size), dtype=io, device=dev)
    w = torch.empty((B, T, HV, K), dtype=io, device=dev) if output_wu else None
    u = torch.empty((B, T, HV, V), dtype=io, device=dev) if output_wu else None
    nbytes = int(lib().gdn_chunk_intra_workspace_bytes(N)) if cu_seqlens is not None else 0
    if nbytes and (workspace is None or workspace.numel() < nbytes):
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _check(lib().gdn_chunk_intra(_ptr(k), _ptr(v), _ptr(g), 1 if g_cumulative else 0, _ptr(beta),
                                 _ptr(cu_seqlens), N, B, T, Hk, HV, K, V, chunk_size, _io_code(io),
                                 _ptr(A), _ptr(w), _ptr(u), _ptr(workspace) if nbytes else None,
                                 workspace.numel() if nbytes else 0, _stream(dev)))
    return w, u, A


def state_to_pool(ht: torch.Tensor, pool_state: torch.Tensor,
                  indices: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Write final prefill states ``ht`` [N,HV,V,K] fp32 into the bf16 decode
    pool ``pool_state`` [pool,HV,V,K] (in place) at slots ``indices`` [N]
    (int32; None = slot n), rounded to nearest bf16.  Returns ``pool_state``."""
    if ht.dim() != 4 or pool_state.dim() != 4:
        raise ValueError("ht must be [N, HV, V, K] and pool_state [pool, HV, V, K]")
    N, HV, V, K = ht.shape
    dev = ht.device
    _need(ht, "ht", torch.float32, None, dev)
    _need(pool_state, "pool_state", torch.bfloat16, (pool_state.shape[0], HV, V, K), dev)
    if indices is not None:
        if indices.dtype != torch.int32:
            indices = indices.to(torch.int32)
        _need(indices, "indices", torch.int32, (N,), dev)
    _check(lib().gdn_state_to_pool(_ptr(ht), _ptr(indices), _ptr(pool_state),
                                   N, HV, K, V, pool_state.shape[0], _stream(dev)))
    return pool_state


def _state_scan_args(a, b, an, bn, g, g_gamma, gk, gv, init, init_name, cu_seqlens):
    if a.dim() != 4 or b.dim() != 4:
        raise ValueError(f"{an} must be [B, T, Hk, K] and {bn} [B, T, HV, V]")
    B, T, Hk, K = a.shape
    HV, V = b.shape[2], b.shape[3]
    dev = a.device
    bf = torch.bfloat16
    _need(a, an, bf, None, dev)
    _need(b, bn, bf, (B, T, HV, V), dev)
    # gate heads: taken from whichever gate is given (all must agree)
    heads = {t.shape[2] for t in (g, gk, gv) if t is not None and t.dim() >= 3}
    if g_gamma is not None:
        heads.add(g_gamma.shape[0])
    if len(heads) > 1:
        raise ValueError(f"the gates disagree on their head count: {sorted(heads)}")
    Hg = heads.pop() if heads else HV
    if Hg <= 0 or HV % Hg:
        raise ValueError(f"HV ({HV}) must be a multiple of the gate heads ({Hg})")
    _need(g, "g", torch.float32, (B, T, Hg), dev)
    _need(g_gamma, "g_gamma", torch.float32, (Hg,), dev)
    _need(gk, "gk", torch.float32, (B, T, Hg, K), dev)
    _need(gv, "gv", torch.float32, (B, T, Hg, V), dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int64, None, dev)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    _need(init, init_name, torch.float32, (N, HV, V, K), dev)
    return B, T, Hk, HV, K, V, N, dev, Hg


def chunk_bwd_dh(q: torch.Tensor, dout: torch.Tensor, g: Optional[torch.Tensor] = None,
                 g_gamma: Optional[torch.Tensor] = None, gk: Optional[torch.Tensor] = None,
                 scale: Optional[float] = None, dht: Optional[torch.Tensor] = None,
                 cu_seqlens: Optional[torch.Tensor] = None, split_size: Optional[int] = 64,
                 output_dh0: bool = True, chunk_size: int = 64, gv: Optional[torch.Tensor] = None,
                 states_in_fp32: bool = False, dh: Optional[torch.Tensor] = None,
                 cu_seqlens_cpu=None, state_v_first: bool = True):
    """Backward state-gradient scan (bf16 q / dout).  Returns (dh [S,HV,V,K]
    -- bf16, or fp32 with ``states_in_fp32``; None when ``split_size`` is
    None -- and dh0 [N,HV,V,K] fp32 or None).  The gates may have fewer heads
    than dout (Hg, a divisor of HV: v-head j takes gate head j / (HV / Hg)).
    ``dh`` may be passed preallocated (any capacity; entries past it are not
    written); a varlen call without it needs ``cu_seqlens_cpu``.  With
    ``state_v_first=False`` dht, dh and dh0 are [*, HV, K, V] (V contiguous)
    instead."""
    B, T, Hk, HV, K, V, N, dev, Hg = _state_scan_args(q, dout, "q", "dout", g, g_gamma, gk, gv, dht, "dht",
                                                      cu_seqlens)
    if scale is None:
        scale = K ** -0.5
    sdt = _state_dtype(torch.bfloat16, states_in_fp32)
    dh = _states(B, T, HV, V, K, N, dev, split_size, dh, "dh", cu_seqlens is not None, cu_seqlens_cpu, sdt)
    dh0 = torch.empty((N, HV, V, K), dtype=torch.float32, device=dev) if output_dh0 else None
    _check(lib().gdn_chunk_bwd_dh(_ptr(q), _ptr(dout), _ptr(g), _ptr(g_gamma), _ptr(gk), _ptr(gv), Hg,
                                  float(scale), _ptr(dht), _ptr(dh), split_size or 0,
                                  0 if dh is None else dh.shape[0], _dtype_code(sdt), int(bool(state_v_first)),
                                  _ptr(dh0),
                                  _ptr(cu_seqlens), N, B, T, Hk, HV, K, V, chunk_size,
                                  _io_code(torch.bfloat16), _stream(dev)))
    return dh, dh0


def chunk_fwd_h(k: torch.Tensor, v: torch.Tensor, g: Optional[torch.Tensor] = None,
                g_gamma: Optional[torch.Tensor] = None, gk: Optional[torch.Tensor] = None,
                gv: Optional[torch.Tensor] = None, h0: Optional[torch.Tensor] = None,
                cu_seqlens: Optional[torch.Tensor] = None, split_size: Optional[int] = 64,
                output_final_state: bool = True, chunk_size: int = 64, states_in_fp32: bool = False,
                h: Optional[torch.Tensor] = None, cu_seqlens_cpu=None, state_v_first: bool = True):
    """Forward decay-only chunk-state scan (bf16 k / v).  Returns (h
    [S,HV,V,K], the state at the start of every split -- bf16, or fp32 with
    ``states_in_fp32``; None when ``split_size`` is None -- and ht [N,HV,V,K]
    fp32 or None).  Gate heads, the ``h`` buffer and ``state_v_first`` (h0,
    h, ht as [*, HV, K, V] when False) as in ``chunk_bwd_dh``."""
    B, T, Hk, HV, K, V, N, dev, Hg = _state_scan_args(k, v, "k", "v", g, g_gamma, gk, gv, h0, "h0", cu_seqlens)
    sdt = _state_dtype(torch.bfloat16, states_in_fp32)
    h = _states(B, T, HV, V, K, N, dev, split_size, h, "h", cu_seqlens is not None, cu_seqlens_cpu, sdt)
    ht = torch.empty((N, HV, V, K), dtype=torch.float32, device=dev) if output_final_state else None
    _check(lib().gdn_chunk_fwd_h(_ptr(k), _ptr(v), _ptr(g), _ptr(g_gamma), _ptr(gk), _ptr(gv), Hg,
                                 _ptr(h0), _ptr(h), split_size or 0, 0 if h is None else h.shape[0],
                                 _dtype_code(sdt), int(bool(state_v_first)), _ptr(ht), _ptr(cu_seqlens), N,
                                 B, T, Hk, HV, K, V, chunk_size, _io_code(torch.bfloat16), _stream(dev)))
    return h, ht

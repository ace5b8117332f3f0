"""Thin Python binding over libckda.so (see include/ckda.h).

Argument marshalling only: checks dtypes / devices / contiguity, allocates
outputs with torch (device memory), passes raw pointers and the current HIP
stream.  Every step of the computation runs in the library's HIP kernels;
there is no Python or CPU fallback.  If the library is missing or fails to
load, every entry point raises ``CkdaError``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("CKDA_LIB", os.path.join(_HERE, "libckda.so"))

CKDA_F32 = 0
CKDA_BF16 = 1
CHUNK = 64


class CkdaError(RuntimeError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """Load libckda.so (raises CkdaError if it is missing or broken)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise CkdaError(f"libckda.so not found at {LIB_PATH}: build it with "
                        "`python -m gated_delta_rule_sign_amd.build`")
    try:
        L = ctypes.CDLL(LIB_PATH)
    except OSError as e:  # pragma: no cover - depends on the machine
        raise CkdaError(f"cannot load {LIB_PATH}: {e}") from e
    P, I, F, S, U = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_uint32
    L.ckda_abi_version.restype = I
    L.ckda_status_string.argtypes = [I]
    L.ckda_status_string.restype = ctypes.c_char_p
    L.ckda_last_error.restype = ctypes.c_char_p
    L.ckda_chunk_prep.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, P]
    L.ckda_chunk_prep.restype = I
    L.ckda_fwd_workspace_bytes.argtypes = [I, I, I, I, I, I]
    L.ckda_fwd_workspace_bytes.restype = S
    L.ckda_fwd_varlen_workspace_bytes.argtypes = [I, I, I, I, I, I]
    L.ckda_fwd_varlen_workspace_bytes.restype = S
    L.ckda_fwd_chunked.argtypes = [I, I, I, I, I, I, U, P, P, P, P, P, P, F, P, P, P, P, P, S, P]
    L.ckda_fwd_chunked.restype = I
    L.ckda_fwd_chunked_noalloc.argtypes = [I, I, I, I, I, I, U, P, P, P, P, P, P, F, P, P, P, P, P]
    L.ckda_fwd_chunked_noalloc.restype = I
    L.ckda_fwd_varlen.argtypes = [I, I, P, P, I, I, I, I, U, P, P, P, P, P, P, F, P, P, P, P, P, S, P]
    L.ckda_fwd_varlen.restype = I
    L.ckda_varlen_chunk_slots.argtypes = [I, I]
    L.ckda_varlen_chunk_slots.restype = I
    L.ckda_decode_step.argtypes = [I, I, I, I, I, U, P, P, P, P, P, P, F, P, P, P, P]
    L.ckda_decode_step.restype = I
    L.ckda_bwd_workspace_bytes.argtypes = [I, I, I, I, I]
    L.ckda_bwd_workspace_bytes.restype = S
    L.ckda_bwd_workspace_bytes_given_ckpt.argtypes = [I, I, I, I, I]
    L.ckda_bwd_workspace_bytes_given_ckpt.restype = S
    L.ckda_bwd.argtypes = [I, I, I, I, I, I, U, P, P, P, P, P, P, F, P, P, P, P,
                           P, P, P, P, P, P, P, S, P]
    L.ckda_bwd.restype = I
    L.ckda_bwd_with_records.argtypes = [I, I, I, I, I, I, U, P, P, P, P, P, P, F, P, P, P, S, P, P,
                                        P, P, P, P, P, P, P, S, P]
    L.ckda_bwd_with_records.restype = I
    L.ckda_bwd_varlen_workspace_bytes.argtypes = [I, I, I, I, I]
    L.ckda_bwd_varlen_workspace_bytes.restype = S
    L.ckda_bwd_varlen_workspace_bytes_given_ckpt.argtypes = [I, I, I, I, I]
    L.ckda_bwd_varlen_workspace_bytes_given_ckpt.restype = S
    L.ckda_bwd_varlen.argtypes = [I, I, P, P, I, I, I, I, U, P, P, P, P, P, P, F, P, P, P, P,
                                  P, P, P, P, P, P, P, S, P]
    L.ckda_bwd_varlen.restype = I
    L.ckda_bwd_varlen_with_records.argtypes = [I, I, P, P, I, I, I, I, U, P, P, P, P, P, P, F, P, P, P, S, P, P,
                                               P, P, P, P, P, P, P, S, P]
    L.ckda_bwd_varlen_with_records.restype = I
    L.ckda_set_segment_chunks.argtypes = [I]
    L.ckda_set_segment_chunks.restype = I
    L.ckda_short_conv_fwd.argtypes = [I, I, P, P, I, I, U, P, P, P, P, P, P]
    L.ckda_short_conv_fwd.restype = I
    L.ckda_short_conv_bwd_workspace_bytes.argtypes = [I, I]
    L.ckda_short_conv_bwd_workspace_bytes.restype = S
    L.ckda_short_conv_bwd.argtypes = [I, I, P, P, I, I, U, P, P, P, P, P, P, P, P, S, P]
    L.ckda_short_conv_bwd.restype = I
    L.ckda_short_conv_step.argtypes = [I, I, I, U, P, P, P, P, P]
    L.ckda_short_conv_step.restype = I
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        L = lib()
        raise CkdaError(f"{L.ckda_status_string(status).decode()}: {L.ckda_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t) -> int:
    """Code of a tensor's dtype (or of a torch.dtype)."""
    dt = t if isinstance(t, torch.dtype) else t.dtype
    if dt == torch.bfloat16:
        return CKDA_BF16
    if dt == torch.float32:
        return CKDA_F32
    raise CkdaError(f"q/k/v must be bfloat16 or float32, got {dt}")


def _need(t: Optional[torch.Tensor], name: str, dtype=None, shape=None, device=None):
    if t is None:
        return
    if not t.is_cuda:
        raise CkdaError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise CkdaError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise CkdaError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise CkdaError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise CkdaError(f"{name} must be contiguous")


CKDA_GATE_CHANNEL, CKDA_GATE_HEAD, CKDA_QK_L2NORM, CKDA_GATE_MAP = 0, 1, 2, 4


def _gate_code(g, lead) -> int:
    """CKDA_GATE_HEAD when g is [.., H] (one gate per head), else per channel."""
    return CKDA_GATE_HEAD if g.dim() == len(lead) + 1 else CKDA_GATE_CHANNEL


def _flags(g, lead, qk_norm: bool, gate_map: bool = False) -> int:
    """The flags word: gate layout from g's shape, plus CKDA_QK_L2NORM and
    CKDA_GATE_MAP (g and beta then hold the gate and beta pre-activations and
    s may be None; the backward's dg and dbeta are taken w.r.t. them)."""
    return _gate_code(g, lead) | (CKDA_QK_L2NORM if qk_norm else 0) | (CKDA_GATE_MAP if gate_map else 0)


def _token_inputs(q, k, v, g, s, beta, lead):
    dt = q.dtype
    DK, DV = q.shape[-1], v.shape[-1]
    H = q.shape[-2]
    dev = q.device
    _need(q, "q", dt, lead + (H, DK))
    _need(k, "k", dt, lead + (H, DK), dev)
    _need(v, "v", dt, lead + (H, DV), dev)
    # gate layout from g's shape: [.., H, DK] per channel, [.., H] per head
    gshape = lead + (H,) if g is not None and g.dim() == len(lead) + 1 else lead + (H, DK)
    _need(g, "g", torch.float32, gshape, dev)
    _need(s, "s", torch.int8, gshape, dev)
    _need(beta, "beta", torch.float32, lead + (H,), dev)
    return _dtype_code(q), H, DK, DV, dev


def chunk_prep(q, k, g, s):
    """Gate / sign-fold prep of every 64-token chunk (ckda_chunk_prep).
    Returns (b [B,T,H,DK] f32, p [B,T,H,DK] int8, qf, kf)."""
    B, T, H, DK = q.shape
    dt = _dtype_code(q)
    _need(q, "q", q.dtype, (B, T, H, DK))
    _need(k, "k", q.dtype, (B, T, H, DK), q.device)
    _need(g, "g", torch.float32, (B, T, H, DK), q.device)
    _need(s, "s", torch.int8, (B, T, H, DK), q.device)
    b = torch.empty((B, T, H, DK), dtype=torch.float32, device=q.device)
    p = torch.empty((B, T, H, DK), dtype=torch.int8, device=q.device)
    qf = torch.empty_like(q)
    kf = torch.empty_like(k)
    _check(lib().ckda_chunk_prep(B, T, H, DK, dt, _ptr(q), _ptr(k), _ptr(g), _ptr(s), _ptr(b),
                                 _ptr(p), _ptr(qf), _ptr(kf), _stream()))
    return b, p, qf, kf


def fwd_workspace_bytes(B, T, H, DK, DV, dtype) -> int:
    return int(lib().ckda_fwd_workspace_bytes(B, T, H, DK, DV, _dtype_code(dtype)))


def fwd_varlen_workspace_bytes(N, T_total, H, DK, DV, dtype) -> int:
    return int(lib().ckda_fwd_varlen_workspace_bytes(N, T_total, H, DK, DV, _dtype_code(dtype)))


def _workspace(workspace, need, dev):
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _need(workspace, "workspace", device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return workspace, wsb


def fwd(q, k, v, g, s, beta, scale: float = 1.0, h0=None, want_ht: bool = True,
        want_ckpt: bool = False, o=None, ht=None, h_ckpt=None, workspace=None,
        qk_norm: bool = False, gate_map: bool = False):
    """Chunked forward (ckda_fwd_chunked).  Inputs [B,T,H,D]; returns
    (o [B,T,H,DV] f32, ht [B,H,DK,DV] f32 or None, h_ckpt or None).
    ``workspace`` (uint8 GPU tensor of fwd_workspace_bytes) is allocated per
    call if not given.  ``qk_norm`` L2-normalises q and k per (token, head)
    inside the kernels (every entry point takes it)."""
    B, T = q.shape[0], q.shape[1]
    dt, H, DK, DV, dev = _token_inputs(q, k, v, g, s, beta, (B, T))
    _need(h0, "h0", torch.float32, (B, H, DK, DV), dev)
    NT = (T + CHUNK - 1) // CHUNK
    if o is None:
        o = torch.empty((B, T, H, DV), dtype=torch.float32, device=dev)
    _need(o, "o", torch.float32, (B, T, H, DV), dev)
    if want_ht and ht is None:
        ht = torch.empty((B, H, DK, DV), dtype=torch.float32, device=dev)
    _need(ht, "ht", torch.float32, (B, H, DK, DV), dev)
    if want_ckpt and h_ckpt is None:
        h_ckpt = torch.empty((B, H, NT, DK, DV), dtype=torch.float32, device=dev)
    _need(h_ckpt, "h_ckpt", torch.float32, (B, H, NT, DK, DV), dev)
    workspace, wsb = _workspace(workspace, fwd_workspace_bytes(B, T, H, DK, DV, q.dtype), dev)
    _check(lib().ckda_fwd_chunked(B, T, H, DK, DV, dt, _flags(g, (B, T), qk_norm, gate_map), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(s),
                                  _ptr(beta), float(scale), _ptr(h0), _ptr(o), _ptr(ht),
                                  _ptr(h_ckpt), _ptr(workspace), wsb, _stream()))
    return o, ht, h_ckpt


def fwd_noalloc(q, k, v, g, s, beta, o, ht=None, h0=None, h_ckpt=None, scale: float = 1.0,
                qk_norm: bool = False, gate_map: bool = False):
    """ckda_fwd_chunked_noalloc: the chunked forward with the records in the
    library's fixed device scratch (no workspace, nothing allocated by the
    library or here).  The caller passes every output tensor (o, and ht /
    h_ckpt when wanted); returns (o, ht, h_ckpt)."""
    B, T = q.shape[0], q.shape[1]
    dt, H, DK, DV, dev = _token_inputs(q, k, v, g, s, beta, (B, T))
    _need(h0, "h0", torch.float32, (B, H, DK, DV), dev)
    _need(o, "o", torch.float32, (B, T, H, DV), dev)
    _need(ht, "ht", torch.float32, (B, H, DK, DV), dev)
    _need(h_ckpt, "h_ckpt", torch.float32, (B, H, (T + CHUNK - 1) // CHUNK, DK, DV), dev)
    _check(lib().ckda_fwd_chunked_noalloc(B, T, H, DK, DV, dt, _flags(g, (B, T), qk_norm, gate_map), _ptr(q), _ptr(k),
                                          _ptr(v), _ptr(g), _ptr(s), _ptr(beta), float(scale), _ptr(h0),
                                          _ptr(o), _ptr(ht), _ptr(h_ckpt), _stream()))
    return o, ht, h_ckpt


def set_segment_chunks(G: int) -> None:
    """Segment length of the forward's state pass (ckda_set_segment_chunks):
    0 automatic (default), < 0 whole chains only, >= 16 segments of G chunks
    for every chain longer than that.  Process-wide."""
    _check(lib().ckda_set_segment_chunks(int(G)))


def varlen_chunk_slots(N, T_total) -> int:
    return int(lib().ckda_varlen_chunk_slots(N, T_total))


def fwd_varlen(q, k, v, g, s, beta, cu_seqlens, scale: float = 1.0, h0=None,
               want_ht: bool = True, cu_seqlens_dev=None, o=None, ht=None, workspace=None,
               want_ckpt: bool = False, qk_norm: bool = False, gate_map: bool = False):
    """Packed-document forward (ckda_fwd_varlen).  q etc. are [T_total,H,D]
    (a leading 1 is accepted); cu_seqlens is an int32 CPU tensor [N+1].
    Returns (o, ht), or (o, ht, h_ckpt) with want_ckpt: the chunk-start
    states per chunk slot [varlen_chunk_slots(N, T_total), H, DK, DV]."""
    if q.dim() == 4:
        q, k, v, g, s, beta = (x[0] for x in (q, k, v, g, s, beta))
    Tt = q.shape[0]
    dt, H, DK, DV, dev = _token_inputs(q, k, v, g, s, beta, (Tt,))
    cu = cu_seqlens
    if cu.is_cuda or cu.dtype != torch.int32 or not cu.is_contiguous():
        raise CkdaError("cu_seqlens must be a contiguous int32 CPU tensor")
    N = cu.numel() - 1
    if cu_seqlens_dev is None:
        cu_seqlens_dev = cu.to(dev)
    _need(cu_seqlens_dev, "cu_seqlens_dev", torch.int32, (N + 1,), dev)
    _need(h0, "h0", torch.float32, (N, H, DK, DV), dev)
    if o is None:
        o = torch.empty((Tt, H, DV), dtype=torch.float32, device=dev)
    _need(o, "o", torch.float32, (Tt, H, DV), dev)
    if want_ht and ht is None:
        ht = torch.empty((N, H, DK, DV), dtype=torch.float32, device=dev)
    _need(ht, "ht", torch.float32, (N, H, DK, DV), dev)
    hc = None
    if want_ckpt:
        hc = torch.empty((varlen_chunk_slots(N, Tt), H, DK, DV), dtype=torch.float32, device=dev)
    workspace, wsb = _workspace(workspace, fwd_varlen_workspace_bytes(N, Tt, H, DK, DV, q.dtype), dev)
    _check(lib().ckda_fwd_varlen(N, Tt, _ptr(cu), _ptr(cu_seqlens_dev), H, DK, DV, dt, _flags(g, (Tt,), qk_norm, gate_map),
                                 _ptr(q),
                                 _ptr(k), _ptr(v), _ptr(g), _ptr(s), _ptr(beta), float(scale),
                                 _ptr(h0), _ptr(o), _ptr(ht), _ptr(hc), _ptr(workspace), wsb, _stream()))
    return (o, ht, hc) if want_ckpt else (o, ht)


def decode_step(q, k, v, g, s, beta, state, sign_prod, scale: float = 1.0, o=None, qk_norm: bool = False, gate_map: bool = False):
    """One recurrent step (ckda_decode_step); state [N,H,DK,DV] f32 and
    sign_prod [N,H,DK] int8 are updated in place.  Returns o [N,H,DV] f32."""
    N = q.shape[0]
    dt, H, DK, DV, dev = _token_inputs(q, k, v, g, s, beta, (N,))
    _need(state, "state", torch.float32, (N, H, DK, DV), dev)
    _need(sign_prod, "sign_prod", torch.int8, (N, H, DK), dev)
    if o is None:
        o = torch.empty((N, H, DV), dtype=torch.float32, device=dev)
    _need(o, "o", torch.float32, (N, H, DV), dev)
    _check(lib().ckda_decode_step(N, H, DK, DV, dt, _flags(g, (N,), qk_norm, gate_map), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(s),
                                  _ptr(beta), float(scale), _ptr(state), _ptr(sign_prod), _ptr(o),
                                  _stream()))
    return o


def bwd_workspace_bytes(B, T, H, DK, DV, ckpt_given: bool = False) -> int:
    """Backward workspace; ckpt_given: the caller passes the checkpoints
    (ckda_bwd_workspace_bytes_given_ckpt), else room to recompute them."""
    f = lib().ckda_bwd_workspace_bytes_given_ckpt if ckpt_given else lib().ckda_bwd_workspace_bytes
    return int(f(B, T, H, DK, DV))


def bwd(q, k, v, g, s, beta, h_ckpt, do, scale: float = 1.0, h0=None, dht=None,
        want_dh0: bool = True, workspace=None, qk_norm: bool = False, gate_map: bool = False,
        fwd_workspace=None):
    """Backward (ckda_bwd).  h_ckpt: the checkpoints of fwd(..., want_ckpt=True)
    on the same inputs, or None (the call recomputes them).  fwd_workspace:
    that forward call's workspace, kept unchanged (ckda_bwd_with_records: the
    backward reads its chunk records instead of writing its own).  Returns
    dict dq, dk, dv, dg, dbeta, dh0 (f32)."""
    B, T = q.shape[0], q.shape[1]
    dt, H, DK, DV, dev = _token_inputs(q, k, v, g, s, beta, (B, T))
    NT = (T + CHUNK - 1) // CHUNK
    _need(h_ckpt, "h_ckpt", torch.float32, (B, H, NT, DK, DV), dev)
    _need(do, "do", q.dtype, (B, T, H, DV), dev)
    _need(h0, "h0", torch.float32, (B, H, DK, DV), dev)
    _need(dht, "dht", torch.float32, (B, H, DK, DV), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    gsh = (B, T, H) if _gate_code(g, (B, T)) == CKDA_GATE_HEAD else (B, T, H, DK)
    out = dict(dq=torch.empty((B, T, H, DK), **f32), dk=torch.empty((B, T, H, DK), **f32),
               dv=torch.empty((B, T, H, DV), **f32), dg=torch.empty(gsh, **f32),
               dbeta=torch.empty((B, T, H), **f32),
               dh0=torch.empty((B, H, DK, DV), **f32) if want_dh0 else None)
    need = bwd_workspace_bytes(B, T, H, DK, DV, ckpt_given=h_ckpt is not None)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if fwd_workspace is not None:
        _need(fwd_workspace, "fwd_workspace", device=dev)
        fb = fwd_workspace.numel() * fwd_workspace.element_size()
        _check(lib().ckda_bwd_with_records(
            B, T, H, DK, DV, dt, _flags(g, (B, T), qk_norm, gate_map), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(s),
            _ptr(beta), float(scale), _ptr(h0), _ptr(h_ckpt), _ptr(fwd_workspace), ctypes.c_size_t(fb), _ptr(do),
            _ptr(dht), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]),
            _ptr(out["dh0"]), _ptr(workspace), ctypes.c_size_t(wsb), _stream()))
        return out
    _check(lib().ckda_bwd(B, T, H, DK, DV, dt, _flags(g, (B, T), qk_norm, gate_map), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(s),
                          _ptr(beta), float(scale), _ptr(h0), _ptr(h_ckpt), _ptr(do), _ptr(dht),
                          _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                          _ptr(out["dbeta"]), _ptr(out["dh0"]), _ptr(workspace), wsb, _stream()))
    return out


def bwd_varlen_workspace_bytes(N, T_total, H, DK, DV, ckpt_given: bool = False) -> int:
    f = lib().ckda_bwd_varlen_workspace_bytes_given_ckpt if ckpt_given else lib().ckda_bwd_varlen_workspace_bytes
    return int(f(N, T_total, H, DK, DV))


def bwd_varlen(q, k, v, g, s, beta, cu_seqlens, h_ckpt, do, scale: float = 1.0, h0=None, dht=None,
               want_dh0: bool = True, cu_seqlens_dev=None, workspace=None, qk_norm: bool = False, gate_map: bool = False,
               fwd_workspace=None):
    """Backward of the packed-document forward (ckda_bwd_varlen).  Shapes as
    in fwd_varlen; h_ckpt from fwd_varlen(..., want_ckpt=True), or None
    (recomputed); fwd_workspace: that call's workspace, kept unchanged
    (ckda_bwd_varlen_with_records); do
    [T_total,H,DV]; dht, dh0 [N,H,DK,DV].  Returns dict dq, dk, dv, dg,
    dbeta, dh0 (f32)."""
    if q.dim() == 4:
        q, k, v, g, s, beta = (x[0] for x in (q, k, v, g, s, beta))
        do = do[0] if do.dim() == 4 else do
    Tt = q.shape[0]
    dt, H, DK, DV, dev = _token_inputs(q, k, v, g, s, beta, (Tt,))
    cu = cu_seqlens
    if cu.is_cuda or cu.dtype != torch.int32 or not cu.is_contiguous():
        raise CkdaError("cu_seqlens must be a contiguous int32 CPU tensor")
    N = cu.numel() - 1
    if cu_seqlens_dev is None:
        cu_seqlens_dev = cu.to(dev)
    _need(cu_seqlens_dev, "cu_seqlens_dev", torch.int32, (N + 1,), dev)
    _need(h_ckpt, "h_ckpt", torch.float32, (varlen_chunk_slots(N, Tt), H, DK, DV), dev)
    _need(do, "do", q.dtype, (Tt, H, DV), dev)
    _need(h0, "h0", torch.float32, (N, H, DK, DV), dev)
    _need(dht, "dht", torch.float32, (N, H, DK, DV), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    gsh = (Tt, H) if _gate_code(g, (Tt,)) == CKDA_GATE_HEAD else (Tt, H, DK)
    out = dict(dq=torch.empty((Tt, H, DK), **f32), dk=torch.empty((Tt, H, DK), **f32),
               dv=torch.empty((Tt, H, DV), **f32), dg=torch.empty(gsh, **f32),
               dbeta=torch.empty((Tt, H), **f32),
               dh0=torch.empty((N, H, DK, DV), **f32) if want_dh0 else None)
    workspace, wsb = _workspace(workspace, bwd_varlen_workspace_bytes(N, Tt, H, DK, DV, ckpt_given=h_ckpt is not None),
                                dev)
    if fwd_workspace is not None:
        _need(fwd_workspace, "fwd_workspace", device=dev)
        fb = fwd_workspace.numel() * fwd_workspace.element_size()
        _check(lib().ckda_bwd_varlen_with_records(
            N, Tt, _ptr(cu), _ptr(cu_seqlens_dev), H, DK, DV, dt, _flags(g, (Tt,), qk_norm, gate_map), _ptr(q), _ptr(k),
            _ptr(v), _ptr(g), _ptr(s), _ptr(beta), float(scale), _ptr(h0), _ptr(h_ckpt), _ptr(fwd_workspace),
            ctypes.c_size_t(fb), _ptr(do), _ptr(dht), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
            _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dh0"]), _ptr(workspace), ctypes.c_size_t(wsb), _stream()))
        return out
    _check(lib().ckda_bwd_varlen(N, Tt, _ptr(cu), _ptr(cu_seqlens_dev), H, DK, DV, dt, _flags(g, (Tt,), qk_norm, gate_map),
                                 _ptr(q),
                                 _ptr(k), _ptr(v), _ptr(g), _ptr(s), _ptr(beta), float(scale),
                                 _ptr(h0), _ptr(h_ckpt), _ptr(do), _ptr(dht), _ptr(out["dq"]),
                                 _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]),
                                 _ptr(out["dh0"]), _ptr(workspace), wsb, _stream()))
    return out


# ----------------------------------------------------------------------------
# short convolution (optional width-4 part of the pre-mixer prep)
# ----------------------------------------------------------------------------
CKDA_CONV_SILU = 8
CONV_WIDTH = 4


def _conv_seqs(x, cu_seqlens, cu_seqlens_dev):
    """(N, T_total, C, host cu, device cu) for x [B, T, ...] (B sequences) or
    x [T_total, ...] with cu_seqlens (an int32 CPU tensor [N+1])."""
    if cu_seqlens is None:
        B, T = x.shape[0], x.shape[1]
        C = int(x[0, 0].numel()) if B * T > 0 else int(torch.tensor(x.shape[2:]).prod())
        return B, B * T, C, None, None
    cu = cu_seqlens
    if cu.is_cuda or cu.dtype != torch.int32 or not cu.is_contiguous():
        raise CkdaError("cu_seqlens must be a contiguous int32 CPU tensor")
    N = cu.numel() - 1
    if cu_seqlens_dev is None:
        cu_seqlens_dev = cu.to(x.device)
    _need(cu_seqlens_dev, "cu_seqlens_dev", torch.int32, (N + 1,), x.device)
    C = int(torch.tensor(x.shape[1:]).prod()) if x.dim() > 1 else 1
    return N, x.shape[0], C, cu, cu_seqlens_dev


def short_conv(x, w, cu_seqlens=None, state0=None, silu: bool = False, want_state: bool = False,
               cu_seqlens_dev=None, y=None, state_out=None):
    """Depthwise causal width-4 convolution over tokens (ckda_short_conv_fwd).
    x: [B, T, ...] (B sequences) or [T_total, ...] with cu_seqlens; channels =
    the trailing dims (e.g. H x D); w [C, 4] f32; state0 [N, 3, C] (x's dtype)
    or None.  Returns (y like x, state_out [N, 3, C] or None).  state_out may
    be state0 (updated in place)."""
    N, Tt, C, cu, cud = _conv_seqs(x, cu_seqlens, cu_seqlens_dev)
    dt, dev = _dtype_code(x), x.device
    _need(x, "x", x.dtype)
    _need(w, "w", torch.float32, (C, CONV_WIDTH), dev)
    _need(state0, "state0", x.dtype, (N, CONV_WIDTH - 1, C), dev)
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", x.dtype, tuple(x.shape), dev)
    if want_state and state_out is None:
        state_out = torch.empty((N, CONV_WIDTH - 1, C), dtype=x.dtype, device=dev)
    _need(state_out, "state_out", x.dtype, (N, CONV_WIDTH - 1, C), dev)
    _check(lib().ckda_short_conv_fwd(N, Tt, _ptr(cu), _ptr(cud), C, dt, CKDA_CONV_SILU if silu else 0, _ptr(x),
                                     _ptr(w), _ptr(state0), _ptr(y), _ptr(state_out), _stream()))
    return y, state_out


def short_conv_bwd(x, w, dy, cu_seqlens=None, state0=None, silu: bool = False, want_dstate0: bool = False,
                   cu_seqlens_dev=None, workspace=None):
    """Backward of short_conv (ckda_short_conv_bwd): dy f32 shaped like x.
    Returns dict dx (f32 like x), dw [C, 4] f32, dstate0 [N, 3, C] f32 or None."""
    N, Tt, C, cu, cud = _conv_seqs(x, cu_seqlens, cu_seqlens_dev)
    dt, dev = _dtype_code(x), x.device
    _need(x, "x", x.dtype)
    _need(w, "w", torch.float32, (C, CONV_WIDTH), dev)
    _need(state0, "state0", x.dtype, (N, CONV_WIDTH - 1, C), dev)
    _need(dy, "dy", torch.float32, tuple(x.shape), dev)
    out = dict(dx=torch.empty(tuple(x.shape), dtype=torch.float32, device=dev),
               dw=torch.empty((C, CONV_WIDTH), dtype=torch.float32, device=dev),
               dstate0=torch.empty((N, CONV_WIDTH - 1, C), dtype=torch.float32, device=dev) if want_dstate0 else None)
    workspace, wsb = _workspace(workspace, int(lib().ckda_short_conv_bwd_workspace_bytes(Tt, C)), dev)
    _check(lib().ckda_short_conv_bwd(N, Tt, _ptr(cu), _ptr(cud), C, dt, CKDA_CONV_SILU if silu else 0, _ptr(x),
                                     _ptr(w), _ptr(state0), _ptr(dy), _ptr(out["dx"]), _ptr(out["dw"]),
                                     _ptr(out["dstate0"]), _ptr(workspace), wsb, _stream()))
    return out


def short_conv_step(x, w, window, silu: bool = False, y=None):
    """One decode step (ckda_short_conv_step): x [N, ...] (C channels after
    the first dim), window [N, 3, C] updated in place.  Returns y like x."""
    N = x.shape[0]
    C = int(x[0].numel()) if N > 0 else int(torch.tensor(x.shape[1:]).prod())
    dev = x.device
    _need(x, "x", x.dtype)
    _need(w, "w", torch.float32, (C, CONV_WIDTH), dev)
    _need(window, "window", x.dtype, (N, CONV_WIDTH - 1, C), dev)
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", x.dtype, tuple(x.shape), dev)
    _check(lib().ckda_short_conv_step(N, C, _dtype_code(x), CKDA_CONV_SILU if silu else 0, _ptr(x), _ptr(w),
                                      _ptr(window), _ptr(y), _stream()))
    return y


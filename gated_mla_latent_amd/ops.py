"""Thin ctypes binding over libgmla.so (C ABI in include/gmla.h).

Every function here only marshals arguments: it checks tensor placement,
dtype and contiguity, allocates outputs and workspace with torch when the
caller does not pass them, and hands raw device pointers plus torch's current
HIP stream to the library. All arithmetic runs in the library's HIP kernels.
There is no fallback: if libgmla.so is missing or a call fails, an exception
is raised.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgmla.so")

GMLA_F32, GMLA_BF16 = 0, 1
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small", 4: "HIP error"}

_lib = None


class GmlaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"gmla: {_STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


def _vp(t):
    return C.c_void_p(t.data_ptr()) if t is not None else C.c_void_p(0)


def lib():
    """Load libgmla.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} not found: build it with `python -m gated_mla_latent_amd.build`")
    L = C.CDLL(LIB_PATH)
    vp, i32, f32, sz = C.c_void_p, C.c_int, C.c_float, C.c_size_t
    L.gmla_prefill_workspace_size.argtypes = [i32] * 8
    L.gmla_prefill_workspace_size.restype = sz
    L.gmla_prefill.argtypes = [vp] * 10 + [vp, sz] + [i32] * 9 + [f32, f32, i32, vp]
    L.gmla_prefill.restype = i32
    L.gmla_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    L.gmla_decode_workspace_size.restype = sz
    L.gmla_decode.argtypes = [vp] * 6 + [vp, sz] + [i32] * 4 + [f32, f32, i32, i32, vp]
    L.gmla_decode.restype = i32
    L.gmla_decode_noalloc.argtypes = [vp] * 6 + [i32] * 4 + [f32, f32, i32, i32, vp]
    L.gmla_decode_noalloc.restype = i32
    L.gmla_decode_prepare_workspace_size.argtypes = [i32] * 8
    L.gmla_decode_prepare_workspace_size.restype = sz
    L.gmla_decode_prepare.argtypes = [vp] * 11 + [vp, sz] + [i32] * 7 + [f32, i32, vp]
    L.gmla_decode_prepare.restype = i32
    L.gmla_head_gate_out_workspace_size.argtypes = [i32] * 7
    L.gmla_head_gate_out_workspace_size.restype = sz
    L.gmla_head_gate_out.argtypes = [vp] * 7 + [vp, sz] + [i32] * 5 + [i32, vp]
    L.gmla_head_gate_out.restype = i32
    L.gmla_gate_out_workspace_size.argtypes = [i32] * 7
    L.gmla_gate_out_workspace_size.restype = sz
    L.gmla_gate_out.argtypes = [vp] * 6 + [vp, sz] + [i32] * 5 + [i32, vp]
    L.gmla_gate_out.restype = i32
    L.gmla_status_string.argtypes = [i32]
    L.gmla_status_string.restype = C.c_char_p
    L.gmla_last_error.argtypes = []
    L.gmla_last_error.restype = C.c_char_p
    L.gmla_version.restype = i32
    L.gmla_probe_read.argtypes = [vp, sz, vp, vp]
    L.gmla_probe_read.restype = i32
    L.gmla_trace_begin.argtypes = [i32]
    L.gmla_trace_begin.restype = i32
    L.gmla_trace_end.restype = i32
    L.gmla_trace_summary.argtypes = [C.c_char_p, C.POINTER(C.c_int), C.POINTER(C.c_double)]
    L.gmla_trace_summary.restype = i32
    L.gmla_trace_kernels.restype = C.c_char_p
    L.gmla_trace_reset.restype = None
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise GmlaError(status, lib().gmla_last_error().decode())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GMLA_BF16
    if t.dtype == torch.float32:
        return GMLA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _workspace(nbytes: int, device, ws):
    if nbytes == 0:
        return ws, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


# ------------------------------------------------------------------ prefill
def prefill(x, W_c, W_q, W_uk, W_uv, sm_scale: float, latent_out=None, o_tilde=None, workspace=None, *,
            W_dq=None, W_kr=None, W_qr=None, rope_base: float = 0.0):
    """x [B, L, d_model] -> (cache rows [B, L, d_c + d_r], o_tilde [B, L, H*d_v]).
    W_dq [d_cq, d_model] makes the query low-rank (W_q is then W^UQ);
    W_kr [d_r, d_model] and W_qr [H*d_r, d_in] add decoupled RoPE."""
    _dev(x, W_c, W_dq, W_q, W_kr, W_qr, W_uk, W_uv, latent_out, o_tilde, workspace)
    B, L, D = x.shape
    H, d_k, d_c = W_uk.shape
    d_v = W_uv.shape[1]
    d_cq = 0 if W_dq is None else W_dq.shape[0]
    d_r = 0 if W_kr is None else W_kr.shape[0]
    dt = _dtype_code(x)
    if latent_out is None:
        latent_out = torch.empty((B, L, d_c + d_r), dtype=x.dtype, device=x.device)
    if o_tilde is None:
        o_tilde = torch.empty((B, L, H * d_v), dtype=x.dtype, device=x.device)
    need = lib().gmla_prefill_workspace_size(B, L, H, d_cq, d_k, d_r, d_v, dt)
    workspace, wsb = _workspace(need, x.device, workspace)
    _check(lib().gmla_prefill(_vp(x), _vp(W_c), _vp(W_dq), _vp(W_q), _vp(W_kr), _vp(W_qr), _vp(W_uk), _vp(W_uv),
                              _vp(latent_out), _vp(o_tilde), _vp(workspace), wsb, B, L, D, H, d_c, d_cq, d_k, d_r,
                              d_v, float(sm_scale), float(rope_base), dt, _stream()))
    return latent_out, o_tilde


# ------------------------------------------------------------------ decode
def decode_workspace_bytes(B, H, d_c, num_splits=0, dtype=torch.bfloat16) -> int:
    return lib().gmla_decode_workspace_size(B, H, d_c, num_splits, GMLA_BF16 if dtype == torch.bfloat16 else GMLA_F32)


def decode(q_abs, cache, seq_start, seq_len, d_c: int, d_r: int, rope_base: float, sm_scale: float,
           num_splits: int = 0, o_lat=None, lse=None, workspace=None, want_lse: bool = True):
    """q_abs [B, H, d_c+d_r], cache [rows, d_c+d_r], seq_start int64 [B],
    seq_len int32 [B] -> (o_lat [B, H, d_c], lse [B, H] fp32 or None)."""
    _dev(q_abs, cache, seq_start, seq_len, o_lat, lse, workspace)
    if seq_start.dtype != torch.int64 or seq_len.dtype != torch.int32:
        raise TypeError("seq_start must be int64 and seq_len int32")
    B, H, W = q_abs.shape
    if W != d_c + d_r or cache.shape[-1] != W:
        raise ValueError("q_abs/cache width must be d_c + d_r")
    dt = _dtype_code(q_abs)
    if o_lat is None:
        o_lat = torch.empty((B, H, d_c), dtype=q_abs.dtype, device=q_abs.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q_abs.device)
    need = lib().gmla_decode_workspace_size(B, H, d_c, num_splits, dt)
    workspace, wsb = _workspace(need, q_abs.device, workspace)
    _check(lib().gmla_decode(_vp(q_abs), _vp(cache), _vp(seq_start), _vp(seq_len), _vp(o_lat), _vp(lse),
                             _vp(workspace), wsb, B, H, d_c, d_r, float(rope_base), float(sm_scale), int(num_splits),
                             dt, _stream()))
    return o_lat, lse


def decode_noalloc(q_abs, cache, seq_start, seq_len, d_c: int, d_r: int, rope_base: float, sm_scale: float,
                   num_splits: int = 0, o_lat=None, lse=None):
    """gmla_decode on the library's own scratch (no workspace argument, no
    device allocation by the library); same arguments and results."""
    _dev(q_abs, cache, seq_start, seq_len, o_lat, lse)
    if seq_start.dtype != torch.int64 or seq_len.dtype != torch.int32:
        raise TypeError("seq_start must be int64 and seq_len int32")
    B, H, W = q_abs.shape
    if W != d_c + d_r or cache.shape[-1] != W:
        raise ValueError("q_abs/cache width must be d_c + d_r")
    dt = _dtype_code(q_abs)
    if o_lat is None:
        o_lat = torch.empty((B, H, d_c), dtype=q_abs.dtype, device=q_abs.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q_abs.device)
    _check(lib().gmla_decode_noalloc(_vp(q_abs), _vp(cache), _vp(seq_start), _vp(seq_len), _vp(o_lat), _vp(lse), B, H,
                                     d_c, d_r, float(rope_base), float(sm_scale), int(num_splits), dt, _stream()))
    return o_lat, lse


def decode_prepare(x, W_c, W_kr, W_q, W_qr, W_uk, cache, seq_start, seq_len, rope_base: float, q_abs=None,
                   workspace=None, W_dq=None):
    """x [B, d_model] -> q_abs [B, H, d_c+d_r]; writes the new cache row
    [W_c x ; RoPE(W_kr x, seq_len[b])] at cache[seq_start[b] + seq_len[b]].
    W_kr and W_qr are None when d_r == 0. seq_len is not changed. W_dq
    [d_cq, d_model] makes the query low-rank (W_q and W_qr then read c^Q)."""
    _dev(x, W_c, W_kr, W_dq, W_q, W_qr, W_uk, cache, seq_start, seq_len, q_abs, workspace)
    if seq_start.dtype != torch.int64 or seq_len.dtype != torch.int32:
        raise TypeError("seq_start must be int64 and seq_len int32")
    B, D = x.shape
    H, d_k, d_c = W_uk.shape
    d_r = 0 if W_kr is None else W_kr.shape[0]
    if cache.shape[-1] != d_c + d_r:
        raise ValueError("cache width must be d_c + d_r")
    dt = _dtype_code(x)
    if q_abs is None:
        q_abs = torch.empty((B, H, d_c + d_r), dtype=x.dtype, device=x.device)
    d_cq = 0 if W_dq is None else W_dq.shape[0]
    need = lib().gmla_decode_prepare_workspace_size(B, D, H, d_c, d_cq, d_k, d_r, dt)
    workspace, wsb = _workspace(need, x.device, workspace)
    _check(lib().gmla_decode_prepare(_vp(x), _vp(W_c), _vp(W_kr), _vp(W_dq), _vp(W_q), _vp(W_qr), _vp(W_uk),
                                     _vp(cache), _vp(seq_start), _vp(seq_len), _vp(q_abs), _vp(workspace), wsb, B, D,
                                     H, d_c, d_cq, d_k, d_r, float(rope_base), dt, _stream()))
    return q_abs


# ------------------------------------------------------------------ gate + output
def gate_out(x, o, W_g, W_o, W_uv=None, y=None, workspace=None):
    """y = W_o [Sigmoid(W_g x) * o~]. With W_uv given, `o` is o_lat [T, H, d_c]
    and o~ = W_uv[h] o_lat_h is formed first; else `o` is o~ [T, H*d_v]."""
    _dev(x, o, W_g, W_o, W_uv, y, workspace)
    T, D = x.shape[0], x.shape[-1]
    HV = W_g.shape[0]
    if W_uv is not None:
        H, d_v, d_c = W_uv.shape
    else:
        # without the value up-projection only H*d_v matters
        H, d_v, d_c = 1, HV, 0
    dt = _dtype_code(x)
    if y is None:
        y = torch.empty((T, D), dtype=x.dtype, device=x.device)
    need = lib().gmla_gate_out_workspace_size(T, D, H, d_c, d_v, int(W_uv is not None), dt)
    workspace, wsb = _workspace(need, x.device, workspace)
    _check(lib().gmla_gate_out(_vp(x), _vp(o), _vp(W_uv), _vp(W_g), _vp(W_o), _vp(y), _vp(workspace), wsb,
                               T, D, H, d_c, d_v, dt, _stream()))
    return y


def head_gate_out(x, o, W_g, W_o, b_g=None, W_uv=None, y=None, workspace=None):
    """y = W_o [g_h * o~_h], g = Sigmoid(x W_g^T + b_g) per head (W_g [H, d_model]).
    With W_uv given, `o` is o_lat [T, H, d_c]; else `o` is o~ [T, H*d_v]."""
    _dev(x, o, W_g, W_o, b_g, W_uv, y, workspace)
    T, D = x.shape[0], x.shape[-1]
    H = W_g.shape[0]
    HV = W_o.shape[1]
    d_v = HV // H
    d_c = W_uv.shape[2] if W_uv is not None else 0
    dt = _dtype_code(x)
    if y is None:
        y = torch.empty((T, D), dtype=x.dtype, device=x.device)
    need = lib().gmla_head_gate_out_workspace_size(T, D, H, d_c, d_v, int(W_uv is not None), dt)
    workspace, wsb = _workspace(need, x.device, workspace)
    _check(lib().gmla_head_gate_out(_vp(x), _vp(o), _vp(W_uv), _vp(W_g), _vp(b_g), _vp(W_o), _vp(y), _vp(workspace),
                                    wsb, T, D, H, d_c, d_v, dt, _stream()))
    return y


# ------------------------------------------------------------------ probe
PROBE_BLOCKS = 2048  # GMLA_PROBE_BLOCKS


def probe_read(src, sink=None):
    """Stream the bytes of device tensor `src` (read-bandwidth probe); the
    returned sink holds one word per workgroup."""
    _dev(src, sink)
    nbytes = src.numel() * src.element_size()
    if sink is None:
        sink = torch.empty(PROBE_BLOCKS, dtype=torch.int32, device=src.device)
    _check(lib().gmla_probe_read(_vp(src), nbytes, _vp(sink), _stream()))
    return sink


# ------------------------------------------------------------------ trace
def trace_begin(max_launches: int = 4096):
    _check(lib().gmla_trace_begin(int(max_launches)))


def trace_end():
    _check(lib().gmla_trace_end())


def trace_summary(name: str):
    n = C.c_int(0)
    ms = C.c_double(0.0)
    _check(lib().gmla_trace_summary(name.encode(), C.byref(n), C.byref(ms)))
    return n.value, ms.value


def trace_kernels():
    s = lib().gmla_trace_kernels().decode()
    return [k for k in s.split(";") if k]


def trace_reset():
    lib().gmla_trace_reset()

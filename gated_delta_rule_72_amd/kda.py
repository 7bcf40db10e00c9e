"""Thin ctypes binding of libkda.so (include/kda.h).

Argument marshalling only: every step of the recurrence runs in the HIP
kernels of libkda.so. PyTorch supplies device memory and the current stream.
There is no fallback: if libkda.so is missing or a call fails, this module
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

KDA_OK, KDA_ERR_ARG, KDA_ERR_SHAPE, KDA_ERR_ALIGN, KDA_ERR_WORKSPACE, KDA_ERR_DEVICE = 0, -1, -2, -3, -4, -5
KDA_BF16, KDA_F32 = 0, 1
KDA_GATE_SCALAR, KDA_GATE_PER_KEY = 0, 1
CHUNK = 64


class KdaError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


class KdaShape(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("qkv_dtype", ctypes.c_int32), ("gate", ctypes.c_int32)]


_lib = None


def load() -> ctypes.CDLL:
    """Loads libkda.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run gated_delta_rule_72_amd/build.py "
                          f"(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "kda_abi_version": ([], ctypes.c_int),
        "kda_last_error": ([], ctypes.c_char_p),
        "kda_snapshot_count": ([I32, P, I64, P], ctypes.c_int),
        "kda_prefill_workspace_size": ([P, I32, P, I32, I64, I64, P], ctypes.c_int),
        "kda_prefill_chunked": ([P, I32, P, P, I32, I64, I64, P, P, P, P, P, P, P, P, P, P, SZ, P],
                                ctypes.c_int),
        "kda_prefill_chunked_noalloc": ([P, I32, P, P, I32, I64, P, P, P, P, P, P, P, P, P, P], ctypes.c_int),
        "kda_decode_step": ([P, I32, P, P, P, P, P, P, P, P], ctypes.c_int),
        "kda_decode_tokens": ([P, I32, I32, P, P, P, P, P, P, P, P, P, P], ctypes.c_int),
        "kda_layer_front": ([P, I32, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, P, P, P, P, P],
                            ctypes.c_int),
        "kda_layer_back": ([P, I64, P, P, P, ctypes.c_float, I32, P, P], ctypes.c_int),
        "kda_layer_prefill_workspace_size": ([P, I32, P, I32, I64, I64, P], ctypes.c_int),
        "kda_layer_prefill": ([P, I32, P, P, I32, I64, I64, P, P, P, P, P, P, P, P, ctypes.c_float, I32, P, P, P,
                               P, SZ, P], ctypes.c_int),
        "kda_prefill_backward_workspace_size": ([P, I32, P, P], ctypes.c_int),
        "kda_prefill_backward": ([P, I32, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
                                 ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


EXPORTED = ("kda_abi_version", "kda_last_error", "kda_snapshot_count", "kda_prefill_workspace_size",
            "kda_prefill_chunked", "kda_prefill_chunked_noalloc", "kda_decode_step", "kda_decode_tokens", "kda_layer_front",
            "kda_layer_back", "kda_layer_prefill_workspace_size", "kda_layer_prefill",
            "kda_prefill_backward_workspace_size", "kda_prefill_backward")


def _check(fn: str, rc: int) -> None:
    if rc != KDA_OK:
        raise KdaError(fn, rc, load().kda_last_error().decode(errors="replace"))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def make_shape(num_heads: int, d_k: int, d_v: int, qkv_dtype: torch.dtype, per_key: bool) -> KdaShape:
    dt = {torch.bfloat16: KDA_BF16, torch.float32: KDA_F32}.get(qkv_dtype)
    if dt is None:
        raise TypeError(f"q, k, v must be bfloat16 or float32 (got {qkv_dtype})")
    return KdaShape(num_heads, d_k, d_v, dt, KDA_GATE_PER_KEY if per_key else KDA_GATE_SCALAR)


# ---- the C ABI, name for name ----------------------------------------------
# The library sees raw pointers, so each binding first checks what a pointer
# cannot tell it: dtype, contiguity, device and shape of every tensor passed.

def _args(fn: str, shape: Optional[KdaShape], **named) -> None:
    """named: name=(tensor or None, expected dtype; "qkv" = the shape's q/k/v dtype)."""
    for name, (t, dt) in named.items():
        if t is None:
            continue
        if dt == "qkv":
            dt = torch.bfloat16 if shape.qkv_dtype == KDA_BF16 else torch.float32
        if t.dtype != dt:
            raise TypeError(f"{fn}: {name} must be {dt} (got {t.dtype})")
        if not t.is_contiguous():
            raise ValueError(f"{fn}: {name} must be contiguous")


def _geom(fn: str, device: torch.device, host_ok=(), **named) -> None:
    """named: name=(tensor or None, expected shape tuple). Every tensor must be
    on `device` (the kernels dereference its pointer there); names in host_ok
    may instead be pinned host memory."""
    for name, (t, sh) in named.items():
        if t is not None and tuple(t.shape) != tuple(sh):
            raise ValueError(f"{fn}: {name} has shape {tuple(t.shape)}, expected {tuple(sh)}")
    if device.type != "cuda":
        raise ValueError(f"{fn}: the kernels need GPU tensors (got {device})")
    for name, (t, sh) in named.items():
        if t is None:
            continue
        if t.device != device:
            if name in host_ok and t.device.type == "cpu" and (t.numel() == 0 or t.is_pinned()):
                continue
            raise ValueError(f"{fn}: {name} is on {t.device}, expected {device}")


def _cu_host(fn: str, cu_seqlens_host: torch.Tensor, T: Optional[int] = None) -> torch.Tensor:
    cu = cu_seqlens_host.to("cpu", torch.int64).contiguous()
    if cu.dim() != 1 or cu.numel() < 1:
        raise ValueError(f"{fn}: cu_seqlens must be a 1-D tensor of N+1 offsets")
    if T is not None and int(cu[-1]) != T:
        raise ValueError(f"{fn}: cu_seqlens[-1] = {int(cu[-1])} must equal the token count {T}")
    return cu


def _alpha_shape(shape: KdaShape, lead) -> tuple:
    return tuple(lead) + ((shape.num_heads, shape.d_k) if shape.gate == KDA_GATE_PER_KEY else (shape.num_heads,))


F32, I64, I32_ = torch.float32, torch.int64, torch.int32


def kda_abi_version() -> int:
    return load().kda_abi_version()


def kda_last_error() -> str:
    return load().kda_last_error().decode(errors="replace")


def kda_snapshot_count(cu_seqlens_host: torch.Tensor, interval: int) -> int:
    cu = cu_seqlens_host.to("cpu", torch.int64).contiguous()
    out = ctypes.c_int64(0)
    _check("kda_snapshot_count",
           load().kda_snapshot_count(cu.numel() - 1, _ptr(cu), int(interval), ctypes.byref(out)))
    return out.value


def kda_prefill_workspace_size(shape: KdaShape, cu_seqlens_host: torch.Tensor, chunk: int = CHUNK,
                               snapshot_interval: int = 0, segment_tokens: int = -1) -> int:
    cu = cu_seqlens_host.to("cpu", torch.int64).contiguous()
    out = ctypes.c_size_t(0)
    _check("kda_prefill_workspace_size",
           load().kda_prefill_workspace_size(ctypes.byref(shape), cu.numel() - 1, _ptr(cu), int(chunk),
                                             int(snapshot_interval), int(segment_tokens), ctypes.byref(out)))
    return out.value


def kda_prefill_chunked(shape: KdaShape, cu_seqlens_host: torch.Tensor, cu_seqlens_dev: torch.Tensor,
                        q, k, v, alpha, beta, initial_state, o, final_state, snapshots,
                        workspace: torch.Tensor, chunk: int = CHUNK, snapshot_interval: int = 0,
                        segment_tokens: int = -1, stream=None) -> None:
    """Enqueues the prefill on `stream` (default: torch's current stream). All
    tensors must already be allocated, contiguous, on one device."""
    _args("kda_prefill_chunked", shape, q=(q, "qkv"), k=(k, "qkv"), v=(v, "qkv"), alpha=(alpha, F32),
          beta=(beta, F32), initial_state=(initial_state, F32), o=(o, F32), final_state=(final_state, F32),
          snapshots=(snapshots, F32), cu_seqlens_dev=(cu_seqlens_dev, I64))
    T = q.shape[0]
    cu = _cu_host("kda_prefill_chunked", cu_seqlens_host, T)
    N, H, dk, dv = cu.numel() - 1, shape.num_heads, shape.d_k, shape.d_v
    n_snap = kda_snapshot_count(cu, snapshot_interval)
    dev = q.device
    _geom("kda_prefill_chunked", dev, ("snapshots",), q=(q, (T, H, dk)), k=(k, (T, H, dk)), v=(v, (T, H, dv)),
          alpha=(alpha, _alpha_shape(shape, (T,))), beta=(beta, (T, H)), initial_state=(initial_state, (N, H, dv, dk)),
          o=(o, (T, H, dv)), final_state=(final_state, (N, H, dv, dk)), snapshots=(snapshots, (n_snap, H, dv, dk)),
          cu_seqlens_dev=(cu_seqlens_dev, (N + 1,)))
    if workspace.device != dev:
        raise ValueError(f"kda_prefill_chunked: workspace is on {workspace.device}, expected {dev}")
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream_ptr(dev)
    _check("kda_prefill_chunked", load().kda_prefill_chunked(
        ctypes.byref(shape), cu.numel() - 1, _ptr(cu), _ptr(cu_seqlens_dev), int(chunk),
        int(snapshot_interval), int(segment_tokens), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(initial_state),
        _ptr(o), _ptr(final_state), _ptr(snapshots), _ptr(workspace),
        ctypes.c_size_t(workspace.numel() * workspace.element_size()), s))


def kda_prefill_chunked_noalloc(shape: KdaShape, cu_seqlens_host: torch.Tensor, cu_seqlens_dev: torch.Tensor,
                                q, k, v, alpha, beta, initial_state, o, final_state, snapshots,
                                chunk: int = CHUNK, snapshot_interval: int = 0, stream=None) -> None:
    """kda_prefill_chunked with no workspace (the library's static scratch, never
    segmented). Same tensor checks as kda_prefill_chunked."""
    _args("kda_prefill_chunked_noalloc", shape, q=(q, "qkv"), k=(k, "qkv"), v=(v, "qkv"), alpha=(alpha, F32),
          beta=(beta, F32), initial_state=(initial_state, F32), o=(o, F32), final_state=(final_state, F32),
          snapshots=(snapshots, F32), cu_seqlens_dev=(cu_seqlens_dev, I64))
    T = q.shape[0]
    cu = _cu_host("kda_prefill_chunked_noalloc", cu_seqlens_host, T)
    N, H, dk, dv = cu.numel() - 1, shape.num_heads, shape.d_k, shape.d_v
    n_snap = kda_snapshot_count(cu, snapshot_interval)
    dev = q.device
    _geom("kda_prefill_chunked_noalloc", dev, ("snapshots",), q=(q, (T, H, dk)), k=(k, (T, H, dk)),
          v=(v, (T, H, dv)), alpha=(alpha, _alpha_shape(shape, (T,))), beta=(beta, (T, H)),
          initial_state=(initial_state, (N, H, dv, dk)), o=(o, (T, H, dv)), final_state=(final_state, (N, H, dv, dk)),
          snapshots=(snapshots, (n_snap, H, dv, dk)), cu_seqlens_dev=(cu_seqlens_dev, (N + 1,)))
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream_ptr(dev)
    _check("kda_prefill_chunked_noalloc", load().kda_prefill_chunked_noalloc(
        ctypes.byref(shape), cu.numel() - 1, _ptr(cu), _ptr(cu_seqlens_dev), int(chunk), int(snapshot_interval),
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(initial_state), _ptr(o), _ptr(final_state),
        _ptr(snapshots), s))


def kda_decode_step(shape: KdaShape, batch: int, q, k, v, alpha, beta, state, o, stream=None) -> None:
    _args("kda_decode_step", shape, q=(q, "qkv"), k=(k, "qkv"), v=(v, "qkv"), alpha=(alpha, F32),
          beta=(beta, F32), state=(state, F32), o=(o, F32))
    B, H, dk, dv = int(batch), shape.num_heads, shape.d_k, shape.d_v
    _geom("kda_decode_step", q.device, q=(q, (B, H, dk)), k=(k, (B, H, dk)), v=(v, (B, H, dv)),
          alpha=(alpha, _alpha_shape(shape, (B,))), beta=(beta, (B, H)), state=(state, (B, H, dv, dk)),
          o=(o, (B, H, dv)))
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream_ptr(q.device)
    _check("kda_decode_step", load().kda_decode_step(
        ctypes.byref(shape), int(batch), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
        _ptr(state), _ptr(o), s))


def kda_decode_tokens(shape: KdaShape, batch: int, n_tok: int, q, k, v, alpha, beta, state, o,
                      token_states=None, commit=None, stream=None) -> None:
    _args("kda_decode_tokens", shape, q=(q, "qkv"), k=(k, "qkv"), v=(v, "qkv"), alpha=(alpha, F32),
          beta=(beta, F32), state=(state, F32), o=(o, F32), token_states=(token_states, F32),
          commit=(commit, I32_))
    B, n, H, dk, dv = int(batch), int(n_tok), shape.num_heads, shape.d_k, shape.d_v
    _geom("kda_decode_tokens", q.device, q=(q, (B, n, H, dk)), k=(k, (B, n, H, dk)), v=(v, (B, n, H, dv)),
          alpha=(alpha, _alpha_shape(shape, (B, n))), beta=(beta, (B, n, H)), state=(state, (B, H, dv, dk)),
          o=(o, (B, n, H, dv)), token_states=(token_states, (B, n, H, dv, dk)), commit=(commit, (B,)))
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream_ptr(q.device)
    _check("kda_decode_tokens", load().kda_decode_tokens(
        ctypes.byref(shape), int(batch), int(n_tok), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
        _ptr(state), _ptr(o), _ptr(token_states), _ptr(commit), s))


def kda_layer_front(shape: KdaShape, cu_seqlens_host: torch.Tensor, cu_seqlens_dev: torch.Tensor, xq, xk, xv,
                    conv_w, conv_state_in, alpha_logit, alpha_bias: float, beta_logit, q, k, v, alpha, beta,
                    conv_state_out, stream=None) -> None:
    _args("kda_layer_front", shape, xq=(xq, "qkv"), xk=(xk, "qkv"), xv=(xv, "qkv"), conv_w=(conv_w, F32),
          conv_state_in=(conv_state_in, "qkv"), alpha_logit=(alpha_logit, F32), beta_logit=(beta_logit, F32),
          q=(q, "qkv"), k=(k, "qkv"), v=(v, "qkv"), alpha=(alpha, F32), beta=(beta, F32),
          conv_state_out=(conv_state_out, "qkv"), cu_seqlens_dev=(cu_seqlens_dev, I64))
    T = xq.shape[0]
    cu = _cu_host("kda_layer_front", cu_seqlens_host, T)
    N, H, d = cu.numel() - 1, shape.num_heads, shape.d_k
    td = (T, H, d)
    _geom("kda_layer_front", xq.device, xq=(xq, td), xk=(xk, td), xv=(xv, td), conv_w=(conv_w, (3, H, d, 4)),
          conv_state_in=(conv_state_in, (N, 3, 3, H, d)), alpha_logit=(alpha_logit, _alpha_shape(shape, (T,))),
          beta_logit=(beta_logit, (T, H)), q=(q, td), k=(k, td), v=(v, td), alpha=(alpha, _alpha_shape(shape, (T,))),
          beta=(beta, (T, H)), conv_state_out=(conv_state_out, (N, 3, 3, H, d)), cu_seqlens_dev=(cu_seqlens_dev, (N + 1,)))
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream_ptr(xq.device)
    _check("kda_layer_front", load().kda_layer_front(
        ctypes.byref(shape), cu.numel() - 1, _ptr(cu), _ptr(cu_seqlens_dev), _ptr(xq), _ptr(xk), _ptr(xv),
        _ptr(conv_w), _ptr(conv_state_in), _ptr(alpha_logit), float(alpha_bias), _ptr(beta_logit), _ptr(q),
        _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(conv_state_out), s))


def kda_layer_back(shape: KdaShape, num_tokens: int, o, g_logit, norm_w, eps: float, out_dtype: int, out,
                   stream=None) -> None:
    _args("kda_layer_back", shape, o=(o, F32), g_logit=(g_logit, F32), norm_w=(norm_w, F32),
          out=(out, torch.bfloat16 if out_dtype == KDA_BF16 else F32))
    rows = (int(num_tokens), shape.num_heads, shape.d_v)
    _geom("kda_layer_back", o.device, o=(o, rows), g_logit=(g_logit, rows), norm_w=(norm_w, (shape.d_v,)),
          out=(out, rows))
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream_ptr(o.device)
    _check("kda_layer_back", load().kda_layer_back(
        ctypes.byref(shape), int(num_tokens), _ptr(o), _ptr(g_logit), _ptr(norm_w), float(eps), int(out_dtype),
        _ptr(out), s))


def kda_layer_prefill_workspace_size(shape: KdaShape, cu_seqlens_host: torch.Tensor, chunk: int = CHUNK,
                                     snapshot_interval: int = 0, segment_tokens: int = -1) -> int:
    cu = cu_seqlens_host.to("cpu", torch.int64).contiguous()
    out = ctypes.c_size_t(0)
    _check("kda_layer_prefill_workspace_size",
           load().kda_layer_prefill_workspace_size(ctypes.byref(shape), cu.numel() - 1, _ptr(cu), int(chunk),
                                                   int(snapshot_interval), int(segment_tokens), ctypes.byref(out)))
    return out.value


def kda_layer_prefill(shape: KdaShape, cu_seqlens_host: torch.Tensor, cu_seqlens_dev: torch.Tensor,
                      q, k, v, alpha, beta, initial_state, g_logit, norm_w, eps: float, out_dtype: int, out,
                      final_state, snapshots, workspace: torch.Tensor, chunk: int = CHUNK,
                      snapshot_interval: int = 0, segment_tokens: int = -1, stream=None) -> None:
    """Enqueues the recurrence and the layer back end (out instead of o)."""
    _args("kda_layer_prefill", shape, q=(q, "qkv"), k=(k, "qkv"), v=(v, "qkv"), alpha=(alpha, F32),
          beta=(beta, F32), initial_state=(initial_state, F32), g_logit=(g_logit, "qkv"), norm_w=(norm_w, F32),
          out=(out, torch.bfloat16 if out_dtype == KDA_BF16 else F32), final_state=(final_state, F32),
          snapshots=(snapshots, F32), cu_seqlens_dev=(cu_seqlens_dev, I64))
    T = q.shape[0]
    cu = _cu_host("kda_layer_prefill", cu_seqlens_host, T)
    N, H, dk, dv = cu.numel() - 1, shape.num_heads, shape.d_k, shape.d_v
    n_snap = kda_snapshot_count(cu, snapshot_interval)
    dev = q.device
    _geom("kda_layer_prefill", dev, ("snapshots",), q=(q, (T, H, dk)), k=(k, (T, H, dk)), v=(v, (T, H, dv)),
          alpha=(alpha, _alpha_shape(shape, (T,))), beta=(beta, (T, H)), initial_state=(initial_state, (N, H, dv, dk)),
          g_logit=(g_logit, (T, H, dv)), norm_w=(norm_w, (dv,)), out=(out, (T, H, dv)),
          final_state=(final_state, (N, H, dv, dk)), snapshots=(snapshots, (n_snap, H, dv, dk)),
          cu_seqlens_dev=(cu_seqlens_dev, (N + 1,)))
    if workspace.device != dev:
        raise ValueError(f"kda_layer_prefill: workspace is on {workspace.device}, expected {dev}")
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream_ptr(dev)
    _check("kda_layer_prefill", load().kda_layer_prefill(
        ctypes.byref(shape), cu.numel() - 1, _ptr(cu), _ptr(cu_seqlens_dev), int(chunk), int(snapshot_interval),
        int(segment_tokens), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(initial_state),
        _ptr(g_logit), _ptr(norm_w), float(eps), int(out_dtype), _ptr(out), _ptr(final_state), _ptr(snapshots),
        _ptr(workspace), ctypes.c_size_t(workspace.numel() * workspace.element_size()), s))


def kda_prefill_backward_workspace_size(shape: KdaShape, cu_seqlens_host: torch.Tensor) -> int:
    cu = cu_seqlens_host.to("cpu", torch.int64).contiguous()
    out = ctypes.c_size_t(0)
    _check("kda_prefill_backward_workspace_size",
           load().kda_prefill_backward_workspace_size(ctypes.byref(shape), cu.numel() - 1, _ptr(cu),
                                                      ctypes.byref(out)))
    return out.value


def kda_prefill_backward(shape: KdaShape, cu_seqlens_host: torch.Tensor, cu_seqlens_dev: torch.Tensor,
                         q, k, v, alpha, beta, initial_state, d_o, d_final_state, dq, dk, dv, dalpha, dbeta,
                         d_initial_state, workspace: torch.Tensor, stream=None) -> None:
    _args("kda_prefill_backward", shape, q=(q, "qkv"), k=(k, "qkv"), v=(v, "qkv"), alpha=(alpha, F32),
          beta=(beta, F32), initial_state=(initial_state, F32), d_o=(d_o, F32), d_final_state=(d_final_state, F32),
          dq=(dq, F32), dk=(dk, F32), dv=(dv, F32), dalpha=(dalpha, F32), dbeta=(dbeta, F32),
          d_initial_state=(d_initial_state, F32), cu_seqlens_dev=(cu_seqlens_dev, I64))
    T = q.shape[0]
    cu = _cu_host("kda_prefill_backward", cu_seqlens_host, T)
    N, H, Dk, Dv = cu.numel() - 1, shape.num_heads, shape.d_k, shape.d_v
    a_sh = _alpha_shape(shape, (T,))
    _geom("kda_prefill_backward", q.device, q=(q, (T, H, Dk)), k=(k, (T, H, Dk)), v=(v, (T, H, Dv)),
          alpha=(alpha, a_sh), beta=(beta, (T, H)), initial_state=(initial_state, (N, H, Dv, Dk)),
          d_o=(d_o, (T, H, Dv)), d_final_state=(d_final_state, (N, H, Dv, Dk)), dq=(dq, (T, H, Dk)),
          dk=(dk, (T, H, Dk)), dv=(dv, (T, H, Dv)), dalpha=(dalpha, a_sh), dbeta=(dbeta, (T, H)),
          d_initial_state=(d_initial_state, (N, H, Dv, Dk)), cu_seqlens_dev=(cu_seqlens_dev, (N + 1,)),
          workspace=(workspace, tuple(workspace.shape)))
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream_ptr(q.device)
    _check("kda_prefill_backward", load().kda_prefill_backward(
        ctypes.byref(shape), cu.numel() - 1, _ptr(cu), _ptr(cu_seqlens_dev), _ptr(q), _ptr(k), _ptr(v),
        _ptr(alpha), _ptr(beta), _ptr(initial_state), _ptr(d_o), _ptr(d_final_state), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(dalpha), _ptr(dbeta), _ptr(d_initial_state), _ptr(workspace),
        ctypes.c_size_t(workspace.numel() * workspace.element_size()), s))


# ---- convenience wrappers: allocate outputs with torch, then call the ABI ----

def _cu_pair(cu_seqlens: Optional[torch.Tensor], cu_seqlens_host: Optional[torch.Tensor], T: int,
             dev: torch.device):
    """(device copy, host copy) of the offsets: one is derived from the other
    when only one is given, one sequence of T tokens when neither is."""
    if cu_seqlens_host is None:
        cu_seqlens_host = (cu_seqlens.to("cpu", torch.int64) if cu_seqlens is not None
                           else torch.tensor([0, T], dtype=torch.int64))
    cu_seqlens_host = cu_seqlens_host.to("cpu", torch.int64).contiguous()
    if cu_seqlens is None:
        cu_seqlens = cu_seqlens_host.to(dev)
    cu_seqlens = cu_seqlens.to(dev, torch.int64).contiguous()
    if cu_seqlens.numel() != cu_seqlens_host.numel():
        raise ValueError("cu_seqlens and cu_seqlens_host differ in length")
    if int(cu_seqlens_host[-1]) != T:
        raise ValueError(f"cu_seqlens[-1] = {int(cu_seqlens_host[-1])} must equal the token count {T}")
    return cu_seqlens, cu_seqlens_host


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _shapes(fn: str, **named) -> None:
    """named: name=(tensor or None, expected shape tuple)."""
    for name, (t, sh) in named.items():
        if t is not None and tuple(t.shape) != tuple(sh):
            raise ValueError(f"{fn}: {name} has shape {tuple(t.shape)}, expected {tuple(sh)}")


def prefill_chunked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                    beta: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None,
                    initial_state: Optional[torch.Tensor] = None, snapshot_interval: int = 0,
                    cu_seqlens_host: Optional[torch.Tensor] = None, chunk: int = CHUNK,
                    segment_tokens: int = -1,
                    out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                    snapshots_on_host: bool = False):
    """q, k [T,H,dk], v [T,H,dv] (bf16/fp32), alpha [T,H] or [T,H,dk], beta [T,H]
    (fp32). cu_seqlens: int64 [N+1] (default: one sequence of length T).
    segment_tokens: -1 automatic segment plan, 0 none, > 0 segment length.
    snapshots_on_host: snapshots go to pinned host memory, written by the
    kernels during the prefill.
    Returns (o [T,H,dv] fp32, final_state [N,H,dv,dk], snapshots [S,H,dv,dk])."""
    T, H, dk = q.shape
    dv = v.shape[2]
    _shapes("prefill_chunked", k=(k, (T, H, dk)), v=(v, (T, H, dv)), beta=(beta, (T, H)),
            alpha=(alpha, (T, H, dk) if alpha.dim() == 3 else (T, H)))
    dev = q.device
    cu_seqlens, cu_seqlens_host = _cu_pair(cu_seqlens, cu_seqlens_host, T, dev)
    cu_dev = cu_seqlens
    N = cu_seqlens_host.numel() - 1
    _contig(q, k, v, alpha, beta, initial_state)
    per_key = alpha.dim() == 3
    shape = make_shape(H, dk, dv, q.dtype, per_key)
    n_snap = kda_snapshot_count(cu_seqlens_host, snapshot_interval)
    if out is None:
        o = torch.empty((T, H, dv), dtype=torch.float32, device=dev)
        fin = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
        if snapshots_on_host:
            snaps = torch.empty((n_snap, H, dv, dk), dtype=torch.float32, pin_memory=True)
        else:
            snaps = torch.empty((n_snap, H, dv, dk), dtype=torch.float32, device=dev)
    else:
        o, fin, snaps = out
    if snaps is not None and snaps.numel() and snaps.device.type == "cpu" and not snaps.is_pinned():
        raise ValueError("host snapshots must be pinned memory (pin_memory=True)")
    ws_bytes = kda_prefill_workspace_size(shape, cu_seqlens_host, chunk, snapshot_interval, segment_tokens)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    kda_prefill_chunked(shape, cu_seqlens_host, cu_dev, q, k, v, alpha, beta, initial_state, o, fin,
                        snaps if n_snap > 0 else None, ws, chunk, snapshot_interval, segment_tokens)
    return o, fin, snaps


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                beta: torch.Tensor, state: torch.Tensor, o: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One token per sequence; `state` [B,H,dv,dk] fp32 is updated in place.
    Returns o [B,H,dv] fp32."""
    B, H, dk = q.shape
    dv = v.shape[2]
    _contig(q, k, v, alpha, beta, state)
    shape = make_shape(H, dk, dv, q.dtype, alpha.dim() == 3)
    if o is None:
        o = torch.empty((B, H, dv), dtype=torch.float32, device=q.device)
    kda_decode_step(shape, B, q, k, v, alpha, beta, state, o)
    return o


def decode_tokens(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                  beta: torch.Tensor, state: torch.Tensor, commit: Optional[torch.Tensor] = None,
                  keep_token_states: bool = False, o: Optional[torch.Tensor] = None):
    """Several tokens per sequence: q, k [B,n,H,dk], v [B,n,H,dv], alpha [B,n,H(,dk)],
    beta [B,n,H]; `state` [B,H,dv,dk] fp32 receives the state after the first
    commit[b] tokens (all when commit is None; int32 [B] on the device).
    Returns (o [B,n,H,dv], token_states [B,n,H,dv,dk] or None)."""
    B, n, H, dk = q.shape
    dv = v.shape[3]
    _contig(q, k, v, alpha, beta, state, commit)
    shape = make_shape(H, dk, dv, q.dtype, alpha.dim() == 4)
    if o is None:
        o = torch.empty((B, n, H, dv), dtype=torch.float32, device=q.device)
    ts = torch.empty((B, n, H, dv, dk), dtype=torch.float32, device=q.device) if keep_token_states else None
    if commit is not None and commit.dtype != torch.int32:
        raise TypeError("commit must be int32")
    kda_decode_tokens(shape, B, n, q, k, v, alpha, beta, state, o, ts, commit)
    return o, ts


def layer_front(xq: torch.Tensor, xk: torch.Tensor, xv: torch.Tensor, conv_w: torch.Tensor,
                alpha_logit: torch.Tensor, beta_logit: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None,
                conv_state: Optional[torch.Tensor] = None, alpha_bias: float = 5.0,
                cu_seqlens_host: Optional[torch.Tensor] = None, keep_state: bool = True):
    """KDA layer front end: xq, xk, xv [T,H,d] (bf16/fp32), conv_w [3,H,d,4] fp32,
    alpha_logit [T,H] or [T,H,d], beta_logit [T,H]; conv_state [N,3,3,H,d] or None.
    Returns (q, k, v, alpha, beta, conv_state_out or None), ready for prefill_chunked."""
    T, H, d = xq.shape
    _shapes("layer_front", xk=(xk, (T, H, d)), xv=(xv, (T, H, d)), conv_w=(conv_w, (3, H, d, 4)),
            beta_logit=(beta_logit, (T, H)),
            alpha_logit=(alpha_logit, (T, H, d) if alpha_logit.dim() == 3 else (T, H)))
    dev = xq.device
    cu_dev, cu_seqlens_host = _cu_pair(cu_seqlens, cu_seqlens_host, T, dev)
    N = cu_seqlens_host.numel() - 1
    _contig(xq, xk, xv, conv_w, alpha_logit, beta_logit, conv_state)
    shape = make_shape(H, d, d, xq.dtype, alpha_logit.dim() == 3)
    q, k, v = (torch.empty_like(xq) for _ in range(3))
    alpha = torch.empty_like(alpha_logit, dtype=torch.float32)
    beta = torch.empty_like(beta_logit, dtype=torch.float32)
    st = torch.empty((N, 3, 3, H, d), dtype=xq.dtype, device=dev) if keep_state else None
    kda_layer_front(shape, cu_seqlens_host, cu_dev, xq, xk, xv, conv_w, conv_state, alpha_logit, alpha_bias,
                    beta_logit, q, k, v, alpha, beta, st)
    return q, k, v, alpha, beta, st


def layer_back(o: torch.Tensor, g_logit: torch.Tensor, norm_w: torch.Tensor, eps: float = 1e-6,
               out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """KDA layer back end: RMSNorm(o) * norm_w * sigmoid(g_logit) over d_v; o, g_logit [T,H,dv] fp32."""
    T, H, dv = o.shape
    _shapes("layer_back", g_logit=(g_logit, (T, H, dv)), norm_w=(norm_w, (dv,)))
    _contig(o, g_logit, norm_w)
    shape = make_shape(H, dv, dv, torch.bfloat16, False)
    out = torch.empty((T, H, dv), dtype=out_dtype, device=o.device)
    kda_layer_back(shape, T, o, g_logit, norm_w, eps, KDA_BF16 if out_dtype == torch.bfloat16 else KDA_F32, out)
    return out


def layer_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
                  g_logit: torch.Tensor, norm_w: torch.Tensor, eps: float = 1e-6,
                  cu_seqlens: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
                  snapshot_interval: int = 0, cu_seqlens_host: Optional[torch.Tensor] = None,
                  segment_tokens: int = -1, out_dtype: torch.dtype = torch.bfloat16):
    """The recurrence and the layer back end in one call: inputs as
    prefill_chunked (d_k = d_v) plus g_logit [T,H,d] in the q/k/v dtype and
    norm_w [d] fp32. Returns (out [T,H,d] in out_dtype, final_state, snapshots)."""
    T, H, dk = q.shape
    dv = v.shape[2]
    _shapes("layer_prefill", k=(k, (T, H, dk)), v=(v, (T, H, dv)), beta=(beta, (T, H)),
            alpha=(alpha, (T, H, dk) if alpha.dim() == 3 else (T, H)), g_logit=(g_logit, (T, H, dv)),
            norm_w=(norm_w, (dv,)))
    dev = q.device
    cu_dev, cu_seqlens_host = _cu_pair(cu_seqlens, cu_seqlens_host, T, dev)
    N = cu_seqlens_host.numel() - 1
    _contig(q, k, v, alpha, beta, initial_state, g_logit, norm_w)
    shape = make_shape(H, dk, dv, q.dtype, alpha.dim() == 3)
    n_snap = kda_snapshot_count(cu_seqlens_host, snapshot_interval)
    out = torch.empty((T, H, dv), dtype=out_dtype, device=dev)
    fin = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
    snaps = torch.empty((n_snap, H, dv, dk), dtype=torch.float32, device=dev)
    ws_bytes = kda_layer_prefill_workspace_size(shape, cu_seqlens_host, CHUNK, snapshot_interval, segment_tokens)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    kda_layer_prefill(shape, cu_seqlens_host, cu_dev, q, k, v, alpha, beta, initial_state, g_logit, norm_w, eps,
                      KDA_BF16 if out_dtype == torch.bfloat16 else KDA_F32, out, fin,
                      snaps if n_snap > 0 else None, ws, CHUNK, snapshot_interval, segment_tokens)
    return out, fin, snaps


def prefill_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
                     d_o: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None,
                     initial_state: Optional[torch.Tensor] = None, d_final_state: Optional[torch.Tensor] = None,
                     cu_seqlens_host: Optional[torch.Tensor] = None, want_d_initial: bool = True):
    """Gradients of sum <d_o, o> + sum <d_final_state, final_state> of
    prefill_chunked. Returns (dq, dk, dv, dalpha, dbeta, d_initial_state or
    None), all fp32."""
    T, H, dk_ = q.shape
    dv_ = v.shape[2]
    _shapes("prefill_backward", k=(k, (T, H, dk_)), v=(v, (T, H, dv_)), beta=(beta, (T, H)), d_o=(d_o, (T, H, dv_)),
            alpha=(alpha, (T, H, dk_) if alpha.dim() == 3 else (T, H)))
    dev = q.device
    cu_dev, cu_seqlens_host = _cu_pair(cu_seqlens, cu_seqlens_host, T, dev)
    N = cu_seqlens_host.numel() - 1
    _contig(q, k, v, alpha, beta, d_o, initial_state, d_final_state)
    shape = make_shape(H, dk_, dv_, q.dtype, alpha.dim() == 3)
    f32 = dict(dtype=torch.float32, device=dev)
    dq, dk = torch.empty((T, H, dk_), **f32), torch.empty((T, H, dk_), **f32)
    dv = torch.empty((T, H, dv_), **f32)
    dalpha = torch.empty(alpha.shape, **f32)
    dbeta = torch.empty((T, H), **f32)
    d_init = torch.empty((N, H, dv_, dk_), **f32) if want_d_initial else None
    ws = torch.empty(max(kda_prefill_backward_workspace_size(shape, cu_seqlens_host), 1), dtype=torch.uint8,
                     device=dev)
    kda_prefill_backward(shape, cu_seqlens_host, cu_dev, q, k, v, alpha, beta, initial_state, d_o, d_final_state,
                         dq, dk, dv, dalpha, dbeta, d_init, ws)
    return dq, dk, dv, dalpha, dbeta, d_init

"""Ternary linear layer for MI355X (gfx950): Python binding of libtwl.so.

Three operations, each one call into the C ABI declared in include/twl.h
(argument marshalling only; every step runs in the library's HIP kernels):

  rotate_quant_act(x, sign)              -> (x_i8, a_scale)
  pack_ternary(code, s)                  -> (packed, q, smax)
  ternary_linear(x_i8, a_scale, packed, q, smax) -> y

PyTorch provides device memory and the current stream.  Tensors must be CUDA
(HIP) tensors on the current device, contiguous; x is bf16 (or its int16 bit
pattern), s is fp16 (or int16 bits), code and sign are int8.
"""
from __future__ import annotations

from typing import Optional, Tuple

from . import _lib
from ._lib import (GEMV_MAX_M, GROUP, HBLOCK, MAX_K, PATH_AUTO, PATH_GEMM, PATH_GEMV, PATH_GEMV_DOT4,
                   PATH_GEMV_MFMA, TwlError)

__all__ = [
    "rotate_quant_act", "silu_mul_rotate_quant_act", "pack_ternary", "rotate_act_bf16",
    "reference_linear_bf16", "ternary_linear", "ternary_linear_acc", "ternary_linear_bf16",
    "ternary_linear_noalloc", "rotate_quant_linear", "rotate_quant_linear_fused",
    "workspace_bytes", "packed_bytes", "plan_info", "TwlError", "PATH_AUTO", "PATH_GEMM", "PATH_GEMV", "PATH_GEMV_DOT4",
    "PATH_GEMV_MFMA", "GEMV_MAX_M",
    "HBLOCK", "GROUP", "MAX_K", "library",
]


def library():
    """The loaded ctypes library (raises ImportError if it is not built)."""
    return _lib.load()


def _torch():
    import torch
    return torch


def _stream_handle(stream=None) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dev_ptr(t, name: str, dtypes) -> int:
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def rotate_quant_act(x, sign, out: Optional[Tuple] = None, stream=None):
    """x [M, K] bf16, sign [K] int8 -> (x_i8 [M, K] int8, a_scale [M] fp32)."""
    torch = _torch()
    lib = _lib.load()
    M, K = x.shape
    if out is None:
        x_i8 = torch.empty((M, K), dtype=torch.int8, device=x.device)
        a_scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    else:
        x_i8, a_scale = out
    st = lib.twl_rotate_quant_act(
        _dev_ptr(x, "x", (torch.bfloat16, torch.int16)), _dev_ptr(sign, "sign", (torch.int8,)),
        M, K, _dev_ptr(x_i8, "x_i8", (torch.int8,)), _dev_ptr(a_scale, "a_scale", (torch.float32,)),
        _stream_handle(stream))
    _lib.check(st, "twl_rotate_quant_act")
    return x_i8, a_scale


def silu_mul_rotate_quant_act(gate_up, sign, out: Optional[Tuple] = None, stream=None):
    """gate_up [M, 2K] bf16 (gate | up), sign [K] int8 -> (x_i8, a_scale) of
    rotate_quant_act applied to bf16(SiLU(gate) * up)."""
    torch = _torch()
    lib = _lib.load()
    M, K2 = gate_up.shape
    if K2 % 2:
        raise ValueError(f"gate_up has {K2} columns, expected 2K")
    K = K2 // 2
    if out is None:
        x_i8 = torch.empty((M, K), dtype=torch.int8, device=gate_up.device)
        a_scale = torch.empty((M,), dtype=torch.float32, device=gate_up.device)
    else:
        x_i8, a_scale = out
    st = lib.twl_silu_mul_rotate_quant_act(
        _dev_ptr(gate_up, "gate_up", (torch.bfloat16, torch.int16)), _dev_ptr(sign, "sign", (torch.int8,)),
        M, K, _dev_ptr(x_i8, "x_i8", (torch.int8,)), _dev_ptr(a_scale, "a_scale", (torch.float32,)),
        _stream_handle(stream))
    _lib.check(st, "twl_silu_mul_rotate_quant_act")
    return x_i8, a_scale


def rotate_act_bf16(x, sign, out=None, stream=None):
    """x [M, K] bf16, sign [K] int8 -> r [M, K] bf16: the rotation alone."""
    torch = _torch()
    lib = _lib.load()
    M, K = x.shape
    if out is None:
        out = torch.empty((M, K), dtype=torch.bfloat16, device=x.device)
    st = lib.twl_rotate_act_bf16(
        _dev_ptr(x, "x", (torch.bfloat16, torch.int16)), _dev_ptr(sign, "sign", (torch.int8,)),
        M, K, _dev_ptr(out, "r", (torch.bfloat16, torch.int16)), _stream_handle(stream))
    _lib.check(st, "twl_rotate_act_bf16")
    return out


def reference_linear_bf16(r, packed, s, out=None, stream=None):
    """r [M, K] bf16 (rotate_act_bf16), packed (pack_ternary), s [N, K/128] fp16
    -> y [M, N] fp32 = r . (code * bf16(s))^T, the bf16 reference path."""
    torch = _torch()
    lib = _lib.load()
    M, K = r.shape
    N = s.shape[0]
    if s.dim() != 2 or s.shape[1] * GROUP != K:
        raise ValueError(f"s has shape {tuple(s.shape)}, expected [N, K/128] with K = {K}")
    if N > 0 and packed.numel() != packed_bytes(N, K):
        raise ValueError(f"packed has {packed.numel()} bytes, expected {packed_bytes(N, K)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=r.device)
    st = lib.twl_reference_linear_bf16(
        _dev_ptr(r, "r", (torch.bfloat16, torch.int16)), _dev_ptr(packed, "packed", (torch.uint8,)),
        _dev_ptr(s, "s", (torch.float16, torch.int16)), M, N, K,
        _dev_ptr(out, "y", (torch.float32,)), _stream_handle(stream))
    _lib.check(st, "twl_reference_linear_bf16")
    return out


def packed_bytes(N: int, K: int) -> int:
    """Bytes of the tiled packed weight buffer of an N x K layer."""
    return int(_lib.load().twl_packed_bytes(N, K))


def pack_ternary(code, s, bad_codes=None, stream=None):
    """code [N, K] int8, s [N, K/128] fp16 -> (packed uint8 [packed_bytes(N, K)] in the
    tiled layout of include/twl.h, q [N, K/128] int8, smax [N] fp32)."""
    torch = _torch()
    lib = _lib.load()
    N, K = code.shape
    packed = torch.empty((packed_bytes(N, K),), dtype=torch.uint8, device=code.device)
    q = torch.empty((N, K // GROUP), dtype=torch.int8, device=code.device)
    smax = torch.empty((N,), dtype=torch.float32, device=code.device)
    bad = 0 if bad_codes is None else _dev_ptr(bad_codes, "bad_codes", (torch.int32,))
    st = lib.twl_pack_ternary(
        _dev_ptr(code, "code", (torch.int8,)), _dev_ptr(s, "s", (torch.float16, torch.int16)), N, K,
        _dev_ptr(packed, "packed", (torch.uint8,)), _dev_ptr(q, "q", (torch.int8,)),
        _dev_ptr(smax, "smax", (torch.float32,)), bad or None, _stream_handle(stream))
    _lib.check(st, "twl_pack_ternary")
    return packed, q, smax


def workspace_bytes(M: int, N: int, K: int) -> int:
    return int(_lib.load().twl_workspace_bytes(M, N, K))


def plan_info(M: int, N: int, K: int, path: int = PATH_AUTO) -> dict:
    """The kernels ternary_linear would launch for this shape and path on the
    current device (twl_plan_info): family, tile, K splits, workgroups, waves,
    reduce kernel, workspace bytes."""
    import ctypes
    info = (ctypes.c_int64 * 8)()
    st = _lib.load().twl_plan_info(M, N, K, path, ctypes.cast(info, ctypes.c_void_p))
    _lib.check(st, "twl_plan_info")
    family = {0: "none", 1: "gemm", 2: "decode_rows", 3: "decode_dot4", 4: "decode_mfma"}[info[0]]
    keys = ("tile_rows", "tile_cols", "splits", "workgroups", "waves", "reduce_kernel", "workspace_bytes")
    return {"family": family, **{k: int(v) for k, v in zip(keys, info[1:])}}


# One workspace per (device, stream) for calls that pass none: grown on demand,
# never cleared (the kernels need no initial contents), reused by every later
# call on that stream, so the hot path does not allocate.  Calls on one stream
# run in order, so sharing it there is safe.
_WORKSPACES = {}


def _default_workspace(need: int, device, stream_handle: int):
    torch = _torch()
    key = (device.index if device.index is not None else torch.cuda.current_device(), stream_handle)
    ws = _WORKSPACES.get(key)
    if ws is not None and ws.numel() >= need:
        return ws
    if torch.cuda.is_current_stream_capturing():
        raise RuntimeError(
            f"ternary_linear needs a {need}-byte workspace and none is cached for this stream; "
            "pass workspace= (a uint8 tensor of workspace_bytes(M, N, K) bytes) when capturing a graph")
    ws = torch.empty(need, dtype=torch.uint8, device=device)
    _WORKSPACES[key] = ws
    return ws


def _linear(x_i8, a_scale, packed, q, smax, out_kind: int, path: int, out=None, workspace=None,
            stream=None):
    torch = _torch()
    lib = _lib.load()
    M, K = x_i8.shape
    N = q.shape[0]
    if q.dim() != 2 or q.shape[1] * GROUP != K:
        raise ValueError(f"q has shape {tuple(q.shape)}, expected [N, K/128] with K = {K}")
    if N > 0 and packed.numel() != packed_bytes(N, K):
        raise ValueError(f"packed has {packed.numel()} bytes, expected {packed_bytes(N, K)}")
    out_acc = out_kind == _lib.OUT_ACC_I32
    out_dtype = {_lib.OUT_F32: torch.float32, _lib.OUT_ACC_I32: torch.int32,
                 _lib.OUT_BF16: torch.bfloat16}[out_kind]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x_i8.device)
    need = workspace_bytes(M, N, K)
    ws_ptr, ws_len = None, 0
    stream_handle = _stream_handle(stream)
    if need:
        if workspace is None:
            workspace = _default_workspace(need, x_i8.device, stream_handle)
        ws_ptr, ws_len = _dev_ptr(workspace, "workspace", (torch.uint8,)), workspace.numel()
    st = lib.twl_ternary_linear_ex(
        _dev_ptr(x_i8, "x_i8", (torch.int8,)),
        None if out_acc else _dev_ptr(a_scale, "a_scale", (torch.float32,)),
        _dev_ptr(packed, "packed", (torch.uint8,)), _dev_ptr(q, "q", (torch.int8,)),
        None if out_acc else _dev_ptr(smax, "smax", (torch.float32,)),
        M, N, K, _dev_ptr(out, "out", (out_dtype,)),
        out_kind, path, ws_ptr, ws_len, stream_handle)
    _lib.check(st, "twl_ternary_linear_ex")
    return out


def ternary_linear_noalloc(x_i8, a_scale, packed, q, smax, out, path: int = PATH_AUTO, stream=None):
    """The linear layer into a preallocated `out` (fp32 y, bf16 y or int32 acc,
    by its dtype) through twl_ternary_linear_noalloc: K-split partial sums go
    to the library's per-GPU scratch, so neither this call nor the library
    allocates anything.  Calls that may overlap on one GPU must not be issued
    concurrently (they share that scratch)."""
    torch = _torch()
    lib = _lib.load()
    M, K = x_i8.shape
    N = q.shape[0]
    kinds = {torch.float32: _lib.OUT_F32, torch.int32: _lib.OUT_ACC_I32, torch.bfloat16: _lib.OUT_BF16}
    if out.dtype not in kinds:
        raise TypeError(f"out has dtype {out.dtype}, expected float32, bfloat16 or int32")
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(M, N)}")
    out_kind = kinds[out.dtype]
    out_acc = out_kind == _lib.OUT_ACC_I32
    st = lib.twl_ternary_linear_noalloc(
        _dev_ptr(x_i8, "x_i8", (torch.int8,)),
        None if out_acc else _dev_ptr(a_scale, "a_scale", (torch.float32,)),
        _dev_ptr(packed, "packed", (torch.uint8,)), _dev_ptr(q, "q", (torch.int8,)),
        None if out_acc else _dev_ptr(smax, "smax", (torch.float32,)),
        M, N, K, _dev_ptr(out, "out", (out.dtype,)), out_kind, path, _stream_handle(stream))
    _lib.check(st, "twl_ternary_linear_noalloc")
    return out


def rotate_quant_linear_fused(M: int, N: int, K: int) -> bool:
    """Whether rotate_quant_linear runs this shape as one fused kernel on the
    current device (twl_rotate_quant_linear_fused)."""
    r = int(_lib.load().twl_rotate_quant_linear_fused(M, N, K))
    if r < 0:
        _lib.check(-r, "twl_rotate_quant_linear_fused")
    return r == 1


def rotate_quant_linear(x, sign, packed, q, smax, silu: bool = False, out=None, out_dtype=None,
                        x_i8=None, a_scale=None, workspace=None, stream=None):
    """A whole layer from its bf16 input (twl_rotate_quant_linear):
    rotate_quant_act (silu: of bf16(SiLU(gate) * up), x being [gate | up]
    [M, 2K]) then ternary_linear with the automatic path, as one fused decode
    kernel for small batches.  Returns (out, x_i8, a_scale); out is y in
    out_dtype (float32 unless given: bfloat16, or int32 for the raw
    accumulators) or the given `out`, whose dtype then sets the kind."""
    torch = _torch()
    lib = _lib.load()
    M, KX = x.shape
    if silu and KX % 2:
        raise ValueError(f"x has {KX} columns, expected 2K with silu")
    K = KX // 2 if silu else KX
    N = q.shape[0]
    if q.dim() != 2 or q.shape[1] * GROUP != K:
        raise ValueError(f"q has shape {tuple(q.shape)}, expected [N, K/128] with K = {K}")
    if N > 0 and packed.numel() != packed_bytes(N, K):
        raise ValueError(f"packed has {packed.numel()} bytes, expected {packed_bytes(N, K)}")
    kinds = {torch.float32: _lib.OUT_F32, torch.int32: _lib.OUT_ACC_I32, torch.bfloat16: _lib.OUT_BF16}
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32 if out_dtype is None else out_dtype, device=x.device)
    if out.dtype not in kinds:
        raise TypeError(f"out has dtype {out.dtype}, expected float32, bfloat16 or int32")
    out_kind = kinds[out.dtype]
    if x_i8 is None:
        x_i8 = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if a_scale is None:
        a_scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    stream_handle = _stream_handle(stream)
    ws_ptr, ws_len = None, 0
    if M > 0 and N > 0 and not rotate_quant_linear_fused(M, N, K):
        need = workspace_bytes(M, N, K)
        if need:
            if workspace is None:
                workspace = _default_workspace(need, x.device, stream_handle)
            ws_ptr, ws_len = _dev_ptr(workspace, "workspace", (torch.uint8,)), workspace.numel()
    out_acc = out_kind == _lib.OUT_ACC_I32
    st = lib.twl_rotate_quant_linear(
        _dev_ptr(x, "x", (torch.bfloat16, torch.int16)), _dev_ptr(sign, "sign", (torch.int8,)),
        _dev_ptr(packed, "packed", (torch.uint8,)), _dev_ptr(q, "q", (torch.int8,)),
        None if out_acc else _dev_ptr(smax, "smax", (torch.float32,)),
        M, N, K, 1 if silu else 0, _dev_ptr(x_i8, "x_i8", (torch.int8,)),
        _dev_ptr(a_scale, "a_scale", (torch.float32,)), _dev_ptr(out, "out", (out.dtype,)),
        out_kind, ws_ptr, ws_len, stream_handle)
    _lib.check(st, "twl_rotate_quant_linear")
    return out, x_i8, a_scale


def ternary_linear(x_i8, a_scale, packed, q, smax, path: int = PATH_AUTO, out=None,
                   workspace=None, stream=None):
    """y [M, N] fp32 = (sum_k x_i8 * code * q) * a_scale[t] * smax[n] / 127."""
    return _linear(x_i8, a_scale, packed, q, smax, _lib.OUT_F32, path, out, workspace, stream)


def ternary_linear_bf16(x_i8, a_scale, packed, q, smax, path: int = PATH_AUTO, out=None,
                        workspace=None, stream=None):
    """The same y rounded to bf16 (nearest even) in the kernels' epilogue."""
    return _linear(x_i8, a_scale, packed, q, smax, _lib.OUT_BF16, path, out, workspace, stream)


def ternary_linear_acc(x_i8, packed, q, path: int = PATH_AUTO, out=None, workspace=None,
                       stream=None):
    """The exact int32 accumulators acc [M, N] of the same kernels (no rescale)."""
    return _linear(x_i8, None, packed, q, None, _lib.OUT_ACC_I32, path, out, workspace, stream)

"""MI355X (gfx950) W4A4 rotate / quantize / GEMM path.

Thin Python layer over the C ABI in include/w4a4.h (libw4a4.so): it checks
tensor dtypes and devices, allocates outputs with torch, passes raw device
pointers and the current HIP stream, and turns a non-OK status into an
exception.  Every step of the computation runs in the library's kernels.

    codes, scales, zeros = rotate_quant_act(x, had_block=128, act_mode="sym")
    wq, ws, gsum = quant_weight_offline(w, had_block=128)
    # randomized Hadamard: the same fp16 +-1 vector d (length K) on both sides
    codes, scales, zeros = rotate_quant_act(x, had_block=128, signs=d)
    wq, ws, gsum = quant_weight_offline(w, had_block=128, signs=d)
    y = w4a4_gemm(codes, scales, zeros, wq, ws, act_mode="sym")
    y = w4a4_decode_fused(x_small, wq, ws)      # M <= 16: both steps in one launch
    kc, ks, kz = kv_rotate_quant4(kv)
    o = kv4_attention_decode(q, kc, ks, kz, vc, vs, vz)   # decode attention on the INT4 cache
    o = kv4_attention_decode_split(q, kc, ks, kz, vc, vs, vz)   # the same, tokens split (few heads)
    o = kv4_attention_decode_noalloc(q, kc, ks, kz, vc, vs, vz, out=o)  # split, library's static scratch
    # MXFP4 (E2M1 codes, a power-of-two scale per 32) on the scaled FP4 MFMA
    xc, xe = rotate_quant_mxfp4(x, had_block=128)
    wc, we = rotate_quant_mxfp4(w, had_block=128)
    y = mxfp4_gemm(xc, xe, wc, we)
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import (W4A4_ACT_ASYM_G128, W4A4_ACT_SYM_TOKEN, W4A4_HAD_128, W4A4_HAD_FULL,  # noqa: F401
                   last_error)

__all__ = ["rotate_quant_act", "quant_weight_offline", "w4a4_gemm", "kv_rotate_quant4",
           "kv4_attention_decode", "kv4_attention_decode_split", "kv4_attention_workspace_bytes",
           "kv4_attention_decode_noalloc",
           "rotate_quant_mxfp4", "mxfp4_gemm", "w4a4_decode_fused", "abi_version", "W4A4Error"]

_MODES = {"sym": W4A4_ACT_SYM_TOKEN, "asym": W4A4_ACT_ASYM_G128}


class W4A4Error(RuntimeError):
    pass


def _check(status: int, name: str) -> None:
    if status == _lib.W4A4_OK:
        return
    msg = f"{name}: {_lib.STATUS_NAMES.get(status, status)}: {last_error()}"
    if status == _lib.W4A4_ERR_DEVICE:
        raise W4A4Error(msg)
    raise ValueError(msg)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _signs(signs, n: int, dev):
    """Check an optional randomized-Hadamard sign vector: fp16 [n], contiguous, on dev."""
    if signs is None:
        return None
    _need(signs, torch.float16, "signs")
    if signs.dim() != 1 or signs.shape[0] != n or not signs.is_contiguous():
        raise ValueError(f"signs must be a contiguous fp16 vector of length {n}")
    if signs.device != dev:
        raise ValueError("signs must be on the same device as the data")
    return signs


def abi_version() -> int:
    return int(_lib.load().w4a4_abi_version())


def rotate_quant_act(x: torch.Tensor, had_block: int = 128, act_mode: str = "sym", signs=None):
    """Rotate every row of fp16 X [M, K] and quantize it to packed INT4.

    signs: None, or fp16 [K] of +-1 (randomized Hadamard, diag(signs) H).

    Returns (codes uint8 [M, K/2], scales fp32 [M] or [M, K/128],
    zeros uint8 [M, K/128] or None).
    """
    _need(x, torch.float16, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with contiguous rows")
    M, K = x.shape
    mode = _MODES[act_mode]
    dev = x.device
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    if mode == W4A4_ACT_SYM_TOKEN:
        scales = torch.empty((M,), dtype=torch.float32, device=dev)
        zeros = None
    else:
        scales = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
        zeros = torch.empty((M, K // 128), dtype=torch.uint8, device=dev)
    hb = W4A4_HAD_128 if had_block == 128 else (W4A4_HAD_FULL if had_block in (0, K, "full") else -1)
    sg = _signs(signs, K, dev)
    st = _lib.call("rotate_quant_act", _ptr(x), M, K, x.stride(0), hb, _ptr(sg), mode, _ptr(codes),
                   _ptr(scales), _ptr(zeros), _stream(dev))
    _check(st, "rotate_quant_act")
    return codes, scales, zeros


def quant_weight_offline(w: torch.Tensor, had_block: int = 128, with_gsum: bool = True, signs=None):
    """Rotate and quantize fp16 W [N, K] per output channel.

    signs: None, or the same fp16 [K] +-1 vector the activations use.

    Returns (codes uint8 [N, K/2], scales fp32 [N], gsum int32 [N, K/128] or None).
    """
    _need(w, torch.float16, "w")
    if w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be 2-D with contiguous rows")
    N, K = w.shape
    dev = w.device
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((N,), dtype=torch.float32, device=dev)
    gsum = torch.empty((N, K // 128), dtype=torch.int32, device=dev) if with_gsum else None
    hb = W4A4_HAD_128 if had_block == 128 else (W4A4_HAD_FULL if had_block in (0, K, "full") else -1)
    sg = _signs(signs, K, dev)
    st = _lib.call("quant_weight_offline", _ptr(w), N, K, w.stride(0), hb, _ptr(sg), _ptr(codes),
                   _ptr(scales), _ptr(gsum), _stream(dev))
    _check(st, "quant_weight_offline")
    return codes, scales, gsum


def _gemm_operands(x_codes, x_scales, x_zeros, w_codes, w_scales, w_gsum, mode: int):
    """Dtype, shape and layout of the GEMM operands, checked before any
    device work (the kernels size their reads from M, N and K, not from the
    tensors, so a short scale vector would be read past its end).  Returns
    (M, N, K)."""
    for t, n, dt in ((x_codes, "x_codes", torch.uint8), (w_codes, "w_codes", torch.uint8),
                     (x_scales, "x_scales", torch.float32), (w_scales, "w_scales", torch.float32)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{n} must be a tensor")
        if t.dtype != dt:
            raise TypeError(f"{n} must be {dt}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if x_codes.dim() != 2 or w_codes.dim() != 2:
        raise ValueError("x_codes and w_codes must be 2-D [rows, K/2]")
    M, K2 = x_codes.shape
    N = w_codes.shape[0]
    if w_codes.shape[1] != K2:
        raise ValueError("x_codes and w_codes disagree on K")
    K = 2 * K2
    G = K // 128
    if tuple(w_scales.shape) != (N,):
        raise ValueError(f"w_scales must be [N] = [{N}], got {tuple(w_scales.shape)}")
    if mode == W4A4_ACT_SYM_TOKEN:
        if tuple(x_scales.shape) != (M,):
            raise ValueError(f"symmetric x_scales must be [M] = [{M}], got {tuple(x_scales.shape)}")
        if x_zeros is not None:
            raise ValueError("x_zeros must be None in symmetric mode")
    else:
        if tuple(x_scales.shape) != (M, G):
            raise ValueError(f"asymmetric x_scales must be [M, K/128] = [{M}, {G}], got {tuple(x_scales.shape)}")
        if not isinstance(x_zeros, torch.Tensor):
            raise ValueError("asymmetric mode needs x_zeros [M, K/128]")
        if x_zeros.dtype != torch.uint8:
            raise TypeError(f"x_zeros must be {torch.uint8}, got {x_zeros.dtype}")
        if tuple(x_zeros.shape) != (M, G) or not x_zeros.is_contiguous():
            raise ValueError(f"x_zeros must be a contiguous [M, K/128] = [{M}, {G}] tensor")
    if w_gsum is not None:
        if not isinstance(w_gsum, torch.Tensor) or w_gsum.dtype != torch.int32:
            raise TypeError("w_gsum must be an int32 tensor")
        if tuple(w_gsum.shape) != (N, G) or not w_gsum.is_contiguous():
            raise ValueError(f"w_gsum must be a contiguous [N, K/128] = [{N}, {G}] tensor")
    return M, N, K


def w4a4_gemm(x_codes, x_scales, x_zeros, w_codes, w_scales, w_gsum=None, act_mode: str = "sym",
              out: torch.Tensor | None = None):
    """Y fp32 [M, N] from packed INT4 activations and weights (see include/w4a4.h).

    Symmetric: x_scales [M], x_zeros None.  Asymmetric: x_scales and x_zeros
    [M, K/128].  w_scales [N]; w_gsum (optional) [N, K/128].
    """
    mode = _MODES[act_mode]
    M, N, K = _gemm_operands(x_codes, x_scales, x_zeros, w_codes, w_scales, w_gsum, mode)
    dev = x_codes.device
    for t, n in ((x_codes, "x_codes"), (w_codes, "w_codes"), (x_scales, "x_scales"),
                 (w_scales, "w_scales"), (x_zeros, "x_zeros"), (w_gsum, "w_gsum")):
        if t is not None:
            if not t.is_cuda:
                raise TypeError(f"{n} must be a CUDA (HIP) tensor")
            if t.device != dev:
                raise ValueError(f"{n} must be on the same device as x_codes")
    y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=dev)
    _need(y, torch.float32, "out")
    if y.dim() != 2 or y.shape[0] != M or y.shape[1] != N or y.stride(1) != 1:
        raise ValueError("out must be [M, N] with contiguous rows")
    if y.device != dev:
        raise ValueError("out must be on the same device as x_codes")
    st = _lib.call("w4a4_gemm", _ptr(x_codes), _ptr(x_scales), _ptr(x_zeros), mode, _ptr(w_codes),
                   _ptr(w_scales), _ptr(w_gsum), M, N, K, _ptr(y), y.stride(0), _stream(dev))
    _check(st, "w4a4_gemm")
    return y


def kv_rotate_quant4(kv: torch.Tensor, signs=None):
    """Rotate + asymmetric INT4 of a KV cache [B, H, S, 128] fp16 (last dim contiguous).

    signs: None, or fp16 [128] of +-1 (randomized Hadamard over the head dim).

    Returns (codes uint8 [B, H, S, 64], scales fp32 [B, H, S], zeros uint8 [B, H, S]).
    """
    _need(kv, torch.float16, "kv")
    if kv.dim() != 4 or kv.stride(3) != 1:
        raise ValueError("kv must be [B, H, S, D] with D contiguous")
    B, H, S, D = kv.shape
    dev = kv.device
    codes = torch.empty((B, H, S, D // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    zeros = torch.empty((B, H, S), dtype=torch.uint8, device=dev)
    sb, sh, ss, _ = kv.stride()
    sg = _signs(signs, D, dev)
    st = _lib.call("kv_rotate_quant4", _ptr(kv), B, H, S, D, sb, sh, ss, _ptr(sg), _ptr(codes), _ptr(scales),
                   _ptr(zeros), _stream(dev))
    _check(st, "kv_rotate_quant4")
    return codes, scales, zeros


def kv4_attention_workspace_bytes(B: int, H: int, S: int) -> int:
    """Bytes of workspace kv4_attention_decode_split needs (0: single pass)."""
    n = int(_lib.load().kv4_attention_workspace_bytes(B, H, S))
    if n < 0:
        raise ValueError(f"kv4_attention_workspace_bytes: {last_error()}")
    return n


def kv4_attention_decode_split(q: torch.Tensor, k_codes, k_scales, k_zeros, v_codes, v_scales, v_zeros,
                               softmax_scale: float | None = None, signs=None, out: torch.Tensor | None = None,
                               workspace: torch.Tensor | None = None):
    """kv4_attention_decode with each head's tokens split over workgroups
    (kv4_attention_decode_ws): the same result for caches with few heads,
    faster when B*H is small.  `workspace` (uint8, at least
    kv4_attention_workspace_bytes(B, H, S) bytes) is allocated here if not
    given."""
    return kv4_attention_decode(q, k_codes, k_scales, k_zeros, v_codes, v_scales, v_zeros, softmax_scale, signs,
                                out, _split=True, _workspace=workspace)


def kv4_attention_decode_noalloc(q: torch.Tensor, k_codes, k_scales, k_zeros, v_codes, v_scales, v_zeros,
                                 softmax_scale: float | None = None, signs=None, out: torch.Tensor | None = None):
    """kv4_attention_decode_split with the partial states in the library's
    static device scratch (kv4_attention_decode_noalloc): the library
    allocates nothing.  Pass `out` (fp32 [B, H, 128]) to allocate nothing
    here either.  Calls that overlap in time on one GPU race."""
    return kv4_attention_decode(q, k_codes, k_scales, k_zeros, v_codes, v_scales, v_zeros, softmax_scale, signs,
                                out, _split="static")


def kv4_attention_decode(q: torch.Tensor, k_codes, k_scales, k_zeros, v_codes, v_scales, v_zeros,
                         softmax_scale: float | None = None, signs=None, out: torch.Tensor | None = None,
                         _split: bool | str = False, _workspace: torch.Tensor | None = None):
    """Single-query attention per (batch, head) over a KV cache written by
    kv_rotate_quant4 (rotated asymmetric INT4); q fp16 [B, H, 128].

    softmax_scale defaults to 1/sqrt(128); signs is the fp16 +-1 vector the
    cache was rotated with (None: plain Hadamard).  Returns fp32 [B, H, 128].
    """
    _need(q, torch.float16, "q")
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, H, D] tensor")
    B, H, D = q.shape
    for t, n, dt in ((k_codes, "k_codes", torch.uint8), (v_codes, "v_codes", torch.uint8),
                     (k_scales, "k_scales", torch.float32), (v_scales, "v_scales", torch.float32),
                     (k_zeros, "k_zeros", torch.uint8), (v_zeros, "v_zeros", torch.uint8)):
        _need(t, dt, n)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if k_codes.dim() != 4 or tuple(k_codes.shape[:2]) != (B, H) or tuple(v_codes.shape) != tuple(k_codes.shape):
        raise ValueError("k_codes and v_codes must both be [B, H, S, D/2]")
    S = k_codes.shape[2]
    for t, n in ((k_scales, "k_scales"), (v_scales, "v_scales"), (k_zeros, "k_zeros"), (v_zeros, "v_zeros")):
        if tuple(t.shape) != (B, H, S):
            raise ValueError(f"{n} must be [B, H, S]")
    dev = q.device
    scale = float(softmax_scale) if softmax_scale is not None else 1.0 / (D ** 0.5)
    y = out if out is not None else torch.empty((B, H, D), dtype=torch.float32, device=dev)
    _need(y, torch.float32, "out")
    if tuple(y.shape) != (B, H, D) or not y.is_contiguous():
        raise ValueError("out must be a contiguous [B, H, D] fp32 tensor")
    sg = _signs(signs, D, dev)
    if _split == "static":
        st = _lib.call("kv4_attention_decode_noalloc", _ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(k_zeros),
                       _ptr(v_codes), _ptr(v_scales), _ptr(v_zeros), B, H, S, D, scale, _ptr(sg), _ptr(y),
                       _stream(dev))
        _check(st, "kv4_attention_decode_noalloc")
        return y
    if _split:
        need = kv4_attention_workspace_bytes(B, H, S) if B * H > 0 else 0
        ws = _workspace
        if ws is None and need > 0:
            ws = torch.empty((need,), dtype=torch.uint8, device=dev)
        if ws is not None:
            _need(ws, torch.uint8, "workspace")
            if not ws.is_contiguous() or ws.device != dev:
                raise ValueError("workspace must be a contiguous uint8 tensor on the device of q")
        st = _lib.call("kv4_attention_decode_ws", _ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(k_zeros),
                       _ptr(v_codes), _ptr(v_scales), _ptr(v_zeros), B, H, S, D, scale, _ptr(sg), _ptr(y),
                       _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev))
        _check(st, "kv4_attention_decode_ws")
        return y
    st = _lib.call("kv4_attention_decode", _ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(k_zeros),
                   _ptr(v_codes), _ptr(v_scales), _ptr(v_zeros), B, H, S, D, scale, _ptr(sg), _ptr(y),
                   _stream(dev))
    _check(st, "kv4_attention_decode")
    return y


def _had(had_block, K: int) -> int:
    return W4A4_HAD_128 if had_block == 128 else (W4A4_HAD_FULL if had_block in (0, K, "full") else -1)


def rotate_quant_mxfp4(x: torch.Tensor, had_block: int = 128, signs=None):
    """Rotate every row of fp16 X [M, K] (activations or weights) and quantize
    it to MXFP4: E2M1 codes with one power-of-two scale per 32 values.

    Returns (codes uint8 [M, K/2], scales uint8 [M, K/32] = exponent + 127).
    """
    _need(x, torch.float16, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with contiguous rows")
    M, K = x.shape
    dev = x.device
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
    sg = _signs(signs, K, dev)
    st = _lib.call("rotate_quant_mxfp4", _ptr(x), M, K, x.stride(0), _had(had_block, K), _ptr(sg),
                   _ptr(codes), _ptr(scales), _stream(dev))
    _check(st, "rotate_quant_mxfp4")
    return codes, scales


def mxfp4_gemm(x_codes, x_scales, w_codes, w_scales, out: torch.Tensor | None = None):
    """Y fp32 [M, N] from MXFP4 activations and weights (see include/w4a4.h)."""
    for t, n in ((x_codes, "x_codes"), (w_codes, "w_codes"), (x_scales, "x_scales"),
                 (w_scales, "w_scales")):
        _need(t, torch.uint8, n)
        if not t.is_contiguous() or t.dim() != 2:
            raise ValueError(f"{n} must be a contiguous 2-D tensor")
    M, K2 = x_codes.shape
    N = w_codes.shape[0]
    if w_codes.shape[1] != K2:
        raise ValueError("x_codes and w_codes disagree on K")
    K = 2 * K2
    if tuple(x_scales.shape) != (M, K // 32) or tuple(w_scales.shape) != (N, K // 32):
        raise ValueError("scales must be [rows, K/32]")
    dev = x_codes.device
    y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=dev)
    _need(y, torch.float32, "out")
    if y.dim() != 2 or y.shape[0] != M or y.shape[1] != N or y.stride(1) != 1:
        raise ValueError("out must be [M, N] with contiguous rows")
    st = _lib.call("mxfp4_gemm", _ptr(x_codes), _ptr(x_scales), _ptr(w_codes), _ptr(w_scales), M, N, K,
                   _ptr(y), y.stride(0), _stream(dev))
    _check(st, "mxfp4_gemm")
    return y


def w4a4_decode_fused(x: torch.Tensor, w_codes, w_scales, signs=None, out: torch.Tensor | None = None):
    """Y fp32 [M, N] = w4a4_gemm(rotate_quant_act(x, 128, "sym"), W) for M <= 16
    rows in one launch (bit-identical to the two calls)."""
    _need(x, torch.float16, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with contiguous rows")
    _need(w_codes, torch.uint8, "w_codes")
    _need(w_scales, torch.float32, "w_scales")
    if not w_codes.is_contiguous() or not w_scales.is_contiguous():
        raise ValueError("w_codes and w_scales must be contiguous")
    M, K = x.shape
    N = w_codes.shape[0]
    if w_codes.shape[1] * 2 != K:
        raise ValueError("x and w_codes disagree on K")
    if w_scales.numel() != N:
        raise ValueError("w_scales must hold one scale per output channel")
    dev = x.device
    y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=dev)
    _need(y, torch.float32, "out")
    if y.dim() != 2 or y.shape[0] != M or y.shape[1] != N or y.stride(1) != 1:
        raise ValueError("out must be [M, N] with contiguous rows")
    sg = _signs(signs, K, dev)
    st = _lib.call("w4a4_decode_fused", _ptr(x), M, K, x.stride(0), _ptr(sg), _ptr(w_codes), _ptr(w_scales), N,
                   _ptr(y), y.stride(0), _stream(dev))
    _check(st, "w4a4_decode_fused")
    return y

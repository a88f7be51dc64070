"""MI355X-native LLM.int8-style row-wise quantized linear layer.

Thin Python binding over libint8lin.so (include/int8lin.h). Every step of
the layer runs in the library's HIP kernels; this module only allocates the
tensors the C ABI fills (through PyTorch's device allocator), passes device
pointers and the current HIP stream, and wraps the two calls in an autograd
function. There is no CPU or PyTorch fallback: the import fails if the
library is missing, and the calls reject non-GPU tensors.

Names follow bitsandbytes PR #33 "Memory efficient backward": CB / SCB are the
int8 weights and their per-row scales, CA / SCA the quantized activation,
subA the fp16 outlier columns, threshold the outlier threshold (default 6.0).
"""
from __future__ import annotations

import warnings
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import (I8L_BF16, I8L_F16, I8L_F32, I8L_MAX_K, Int8LinError, check, lib)

__all__ = [
    "int8_quantize_rowwise", "int8_linear_forward", "int8_linear_backward_input", "quantize_weight",
    "quantize_weight_colwise", "int8_linear_backward_input_int8", "backward_int8_workspace",
    "int8_linear_backward_weight", "Int8LinearTrainableFunction", "Int8LinearTrainable",
    "outlier_flags_buffer", "silu_outlier_flags", "int8_linear_forward_flagged",
    "Int8LinearFunction", "Int8Linear", "Int8LinError", "forward_workspace", "forward_layout",
    "forward_check", "default_cap", "int8_linear_forward_noalloc", "DTYPE_CODE", "I8L_MAX_K",
]

DTYPE_CODE = {torch.float32: I8L_F32, torch.float16: I8L_F16, torch.bfloat16: I8L_BF16}


def _code(t: torch.Tensor) -> int:
    try:
        return DTYPE_CODE[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; expected float32, float16 or bfloat16") from None


def _dev(t: Optional[torch.Tensor], name: str) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr() if t.numel() > 0 else 0


def _check_out(t: Optional[torch.Tensor], shape: tuple, dtype: torch.dtype, name: str) -> None:
    """Caller-provided result tensors must have exactly the size the kernels write."""
    if t is not None and (tuple(t.shape) != tuple(shape) or t.dtype != dtype):
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


# ----------------------------------------------------------------------------
# quantizer


def int8_quantize_rowwise(X: torch.Tensor, threshold: float = 6.0, cap: Optional[int] = None,
                          workspace: Optional[torch.Tensor] = None):
    """Row-wise int8 quantization of a 2-D tensor with outlier-column split.

    Returns (codes int8 R x C, row_scale fp32 R, outlier_idx int32 cap,
    outlier_count int32 (1,), sub fp16 R x cap). Only the first
    min(count, cap) outlier entries / sub columns are meaningful.
    workspace: optional uint8 buffer of at least
    int8_quantize_rowwise_workspace_bytes(R, C) bytes, reused across calls."""
    if X.dim() != 2:
        raise ValueError("X must be 2-D (flatten leading dimensions)")
    R, C = X.shape
    cap = C if cap is None else int(cap)
    dev = X.device
    codes = _empty((R, C), torch.int8, dev)
    scale = _empty((R,), torch.float32, dev)
    idx = _empty((max(cap, 1),), torch.int32, dev)
    count = _empty((1,), torch.int32, dev)
    sub = _empty((R, max(cap, 1)), torch.float16, dev)
    wsb = lib.int8_quantize_rowwise_workspace_bytes(R, C)
    if workspace is not None:
        if workspace.dtype != torch.uint8 or workspace.numel() < wsb:
            raise ValueError(f"workspace must be uint8 with at least {wsb} bytes")
        ws, wsb = workspace, workspace.numel()
    else:
        ws = _empty((max(wsb, 1),), torch.uint8, dev)
    check(lib.int8_quantize_rowwise(_dev(X, "X"), _code(X), R, C, float(threshold), _dev(codes, "codes"),
                                    _dev(scale, "scale"), idx.data_ptr(), count.data_ptr(), sub.data_ptr(), cap,
                                    ws.data_ptr(), wsb, _stream(dev)),
          "int8_quantize_rowwise")
    return codes, scale, idx[:cap], count, sub[:, :cap]


def quantize_weight(W: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Offline weight quantization (threshold off): W (N x K) -> (CB int8, SCB fp32)."""
    codes, scale, _, _, _ = int8_quantize_rowwise(W, threshold=0.0, cap=0)
    return codes, scale


def quantize_weight_colwise(W: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Second offline weight copy for the int8 backward: W^T (K x N) quantized row-wise
    (one scale per input feature) -> (CBt int8 K x N, SCBt fp32 K)."""
    return quantize_weight(W.t().contiguous())


# ----------------------------------------------------------------------------
# forward


def forward_layout(M: int, K: int, N: int, cap: int) -> _lib.ForwardLayout:
    L = _lib.ForwardLayout()
    check(lib.int8_linear_forward_workspace_layout(M, K, N, cap, L), "int8_linear_forward_workspace_layout")
    return L


def forward_workspace(M: int, K: int, N: int, cap: int, device) -> torch.Tensor:
    n = lib.int8_linear_forward_workspace_bytes(M, K, N, cap)
    return _empty((max(n, 1),), torch.uint8, device)


DEFAULT_CAP = 256


def default_cap(K: int) -> int:
    """Columns of the forward workspace's fp16 outlier sub-matrix (and, up to
    256, of the weight's dequantized outlier slice): the values of further
    outlier columns are read from the input and the int8 weights by the GEMM
    epilogue, so this only sizes the staging buffers (the output is complete
    for any number of outlier columns)."""
    return min(int(K), DEFAULT_CAP)


def forward_check(ws: torch.Tensor, M: int, K: int, N: int, cap: int) -> int:
    """Synchronise and return the outlier count |O| of the last forward on ws."""
    c = ctypes_int32()
    check(lib.int8_linear_forward_check(ws.data_ptr(), M, K, N, cap, _stream(ws.device), c),
          "int8_linear_forward")
    return int(c.value)


def ctypes_int32():
    import ctypes
    return ctypes.c_int32(0)


def int8_linear_forward(A: torch.Tensor, CB: torch.Tensor, SCB: torch.Tensor, bias: Optional[torch.Tensor] = None,
                        threshold: float = 6.0, cap: Optional[int] = None, out: Optional[torch.Tensor] = None,
                        c32: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """out = A (int8-quantized) @ CB^T (dequantized) + outlier product + bias, in A's dtype.

    A: M x K; CB: N x K int8; SCB: N fp32; bias: N (A's dtype) or None.
    cap: columns of the workspace's outlier staging (default min(K, 256));
    any number of outlier columns is handled whatever its value.
    c32: optional M x N int32 tensor receiving the exact int8 product."""
    if A.dim() != 2 or CB.dim() != 2:
        raise ValueError("A and CB must be 2-D")
    M, K = A.shape
    N = CB.shape[0]
    if CB.shape[1] != K or SCB.shape != (N,) or CB.dtype != torch.int8 or SCB.dtype != torch.float32:
        raise ValueError("CB must be N x K int8 and SCB N fp32")
    if bias is not None and (bias.shape != (N,) or bias.dtype != A.dtype):
        raise ValueError("bias must have shape (N,) and A's dtype")
    cap = default_cap(K) if cap is None else int(cap)
    _check_out(out, (M, N), A.dtype, "out")
    _check_out(c32, (M, N), torch.int32, "c32")
    if out is None:
        out = _empty((M, N), A.dtype, A.device)
    if workspace is None:
        workspace = forward_workspace(M, K, N, cap, A.device)
    check(lib.int8_linear_forward(_dev(A, "A"), _code(A), M, K, _dev(CB, "CB"), _dev(SCB, "SCB"), N,
                                  _dev(bias, "bias"), float(threshold), cap, _dev(out, "out"), _dev(c32, "c32"),
                                  workspace.data_ptr(), workspace.numel(), _stream(A.device)),
          "int8_linear_forward")
    return out


def int8_linear_forward_noalloc(A: torch.Tensor, CB: torch.Tensor, SCB: torch.Tensor,
                                bias: Optional[torch.Tensor] = None, threshold: float = 6.0,
                                out: Optional[torch.Tensor] = None):
    """int8_linear_forward on the library's static per-GPU scratch: the C call
    allocates nothing (pass `out` to allocate nothing here either). Calls that
    overlap on one GPU share the scratch and race; sizes beyond the scratch
    raise Int8LinError (I8L_ESCRATCH)."""
    if A.dim() != 2 or CB.dim() != 2:
        raise ValueError("A and CB must be 2-D")
    M, K = A.shape
    N = CB.shape[0]
    if CB.shape[1] != K or SCB.shape != (N,) or CB.dtype != torch.int8 or SCB.dtype != torch.float32:
        raise ValueError("CB must be N x K int8 and SCB N fp32")
    if bias is not None and (bias.shape != (N,) or bias.dtype != A.dtype):
        raise ValueError("bias must have shape (N,) and A's dtype")
    _check_out(out, (M, N), A.dtype, "out")
    if out is None:
        out = _empty((M, N), A.dtype, A.device)
    check(lib.int8_linear_forward_noalloc(_dev(A, "A"), _code(A), M, K, _dev(CB, "CB"), _dev(SCB, "SCB"), N,
                                          _dev(bias, "bias"), float(threshold), _dev(out, "out"), _stream(A.device)),
          "int8_linear_forward_noalloc")
    return out


def outlier_flags_buffer(rows: int, cols: int, device) -> torch.Tensor:
    """A flag buffer for an input of rows x cols (int32 words)."""
    n = lib.int8_outlier_flags_words(rows, cols)
    return _empty((max(n, 1),), torch.int32, device)


def silu_outlier_flags(H: torch.Tensor, threshold: float = 6.0, A: Optional[torch.Tensor] = None,
                       flags: Optional[torch.Tensor] = None):
    """A = SiLU(H) in H's dtype and A's outlier-column flags for `threshold`, in one pass
    (the activation between two int8 linears, producing the second one's input)."""
    if H.dim() != 2:
        raise ValueError("H must be 2-D (flatten leading dimensions)")
    R, C = H.shape
    _check_out(A, (R, C), H.dtype, "A")
    if A is None:
        A = _empty((R, C), H.dtype, H.device)
    n = lib.int8_outlier_flags_words(R, C)
    if flags is None:
        flags = outlier_flags_buffer(R, C, H.device)
    elif flags.dtype != torch.int32 or flags.numel() < n:
        raise ValueError(f"flags must be int32 with at least {n} elements")
    check(lib.int8_silu_outlier_flags(_dev(H, "H"), _code(H), R, C, float(threshold), _dev(A, "A"),
                                      _dev(flags, "flags"), flags.numel(), _stream(H.device)),
          "int8_silu_outlier_flags")
    return A, flags


def int8_linear_forward_flagged(A: torch.Tensor, flags: torch.Tensor, CB: torch.Tensor, SCB: torch.Tensor,
                                bias: Optional[torch.Tensor] = None, cap: Optional[int] = None,
                                out: Optional[torch.Tensor] = None, c32: Optional[torch.Tensor] = None,
                                workspace: Optional[torch.Tensor] = None):
    """int8_linear_forward with the outlier columns taken from `flags` (from silu_outlier_flags on A's shape)."""
    if A.dim() != 2 or CB.dim() != 2:
        raise ValueError("A and CB must be 2-D")
    M, K = A.shape
    N = CB.shape[0]
    if CB.shape[1] != K or SCB.shape != (N,) or CB.dtype != torch.int8 or SCB.dtype != torch.float32:
        raise ValueError("CB must be N x K int8 and SCB N fp32")
    if bias is not None and (bias.shape != (N,) or bias.dtype != A.dtype):
        raise ValueError("bias must have shape (N,) and A's dtype")
    if flags.dtype != torch.int32 or flags.numel() < lib.int8_outlier_flags_words(M, K):
        raise ValueError("flags must be the int32 flag buffer of an M x K input")
    cap = default_cap(K) if cap is None else int(cap)
    _check_out(out, (M, N), A.dtype, "out")
    _check_out(c32, (M, N), torch.int32, "c32")
    if out is None:
        out = _empty((M, N), A.dtype, A.device)
    if workspace is None:
        workspace = forward_workspace(M, K, N, cap, A.device)
    check(lib.int8_linear_forward_flagged(_dev(A, "A"), _code(A), M, K, _dev(flags, "flags"), flags.numel(),
                                          _dev(CB, "CB"),
                                          _dev(SCB, "SCB"), N, _dev(bias, "bias"), cap, _dev(out, "out"),
                                          _dev(c32, "c32"), workspace.data_ptr(), workspace.numel(),
                                          _stream(A.device)),
          "int8_linear_forward_flagged")
    return out


# ----------------------------------------------------------------------------
# backward


def int8_linear_backward_input(G: torch.Tensor, CB: torch.Tensor, SCB: torch.Tensor, with_grad_bias: bool = True,
                               grad_A: Optional[torch.Tensor] = None, grad_bias: Optional[torch.Tensor] = None,
                               workspace: Optional[torch.Tensor] = None):
    """grad_A = G (fp16) @ dequant(CB) in G's dtype; grad_bias = column sums of G (un-cast)."""
    if G.dim() != 2:
        raise ValueError("G must be 2-D")
    M, N = G.shape
    K = CB.shape[1]
    if CB.dim() != 2 or CB.shape[0] != N or SCB.shape != (N,) or CB.dtype != torch.int8 or SCB.dtype != torch.float32:
        raise ValueError("CB must be N x K int8 and SCB N fp32")
    _check_out(grad_A, (M, K), G.dtype, "grad_A")
    _check_out(grad_bias, (N,), G.dtype, "grad_bias")
    if grad_A is None:
        grad_A = _empty((M, K), G.dtype, G.device)
    if with_grad_bias and grad_bias is None:
        grad_bias = _empty((N,), G.dtype, G.device)
    if not with_grad_bias:
        grad_bias = None
    wsb = lib.int8_linear_backward_workspace_bytes(M, N, int(grad_bias is not None))
    if grad_bias is not None and (workspace is None or workspace.numel() < wsb):
        workspace = _empty((max(wsb, 1),), torch.uint8, G.device)
    check(lib.int8_linear_backward_input(_dev(G, "G"), _code(G), M, N, _dev(CB, "CB"), _dev(SCB, "SCB"), K,
                                         _dev(grad_A, "grad_A"), _dev(grad_bias, "grad_bias"),
                                         workspace.data_ptr() if workspace is not None else 0,
                                         workspace.numel() if workspace is not None else 0, _stream(G.device)),
          "int8_linear_backward_input")
    return grad_A, grad_bias


def backward_int8_workspace(M: int, N: int, with_grad_bias: bool, device) -> torch.Tensor:
    wsb = lib.int8_linear_backward_int8_workspace_bytes(M, N, int(with_grad_bias))
    return _empty((max(wsb, 1),), torch.uint8, device)


def int8_linear_backward_input_int8(G: torch.Tensor, CBt: torch.Tensor, SCBt: torch.Tensor,
                                    with_grad_bias: bool = True, grad_A: Optional[torch.Tensor] = None,
                                    grad_bias: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                                    c32: Optional[torch.Tensor] = None):
    """int8 backward variant: grad_A = D(C32 * SG * SCBt / 127^2), C32 = quantize(G) @ CBt^T in int32;
    grad_bias = column sums of G (un-cast). CBt, SCBt come from quantize_weight_colwise."""
    if G.dim() != 2:
        raise ValueError("G must be 2-D")
    M, N = G.shape
    K = CBt.shape[0]
    if (CBt.dim() != 2 or CBt.shape[1] != N or SCBt.shape != (K,) or CBt.dtype != torch.int8
            or SCBt.dtype != torch.float32):
        raise ValueError("CBt must be K x N int8 and SCBt K fp32")
    _check_out(grad_A, (M, K), G.dtype, "grad_A")
    _check_out(grad_bias, (N,), G.dtype, "grad_bias")
    _check_out(c32, (M, K), torch.int32, "c32")
    if grad_A is None:
        grad_A = _empty((M, K), G.dtype, G.device)
    if with_grad_bias and grad_bias is None:
        grad_bias = _empty((N,), G.dtype, G.device)
    if not with_grad_bias:
        grad_bias = None
    wsb = lib.int8_linear_backward_int8_workspace_bytes(M, N, int(grad_bias is not None))
    if workspace is None or workspace.numel() < wsb:
        workspace = _empty((max(wsb, 1),), torch.uint8, G.device)
    check(lib.int8_linear_backward_input_int8(_dev(G, "G"), _code(G), M, N, _dev(CBt, "CBt"), _dev(SCBt, "SCBt"), K,
                                              _dev(grad_A, "grad_A"), _dev(grad_bias, "grad_bias"),
                                              _dev(c32, "c32"), workspace.data_ptr(), workspace.numel(),
                                              _stream(G.device)),
          "int8_linear_backward_input_int8")
    return grad_A, grad_bias


def int8_linear_backward_weight(G: torch.Tensor, A: torch.Tensor, grad_W: Optional[torch.Tensor] = None):
    """Weight gradient of the trainable-weight mode: grad_W = D(fp16(G)^T @ fp16(A)), fp32 accumulation.

    G: M x N output gradient; A: M x K layer input (same dtype); returns N x K in that dtype."""
    if G.dim() != 2 or A.dim() != 2 or G.shape[0] != A.shape[0]:
        raise ValueError("G (M x N) and A (M x K) must be 2-D with the same number of rows")
    if G.dtype != A.dtype:
        raise ValueError("G and A must have the same dtype")
    M, N = G.shape
    K = A.shape[1]
    _check_out(grad_W, (N, K), G.dtype, "grad_W")
    if grad_W is None:
        grad_W = _empty((N, K), G.dtype, G.device)
    check(lib.int8_linear_backward_weight(_dev(G, "G"), _dev(A, "A"), _code(G), M, N, K, _dev(grad_W, "grad_W"),
                                          _stream(G.device)),
          "int8_linear_backward_weight")
    return grad_W


# ----------------------------------------------------------------------------
# autograd glue (bitsandbytes Linear8bitLt with memory-efficient backward)

_warned_cast = False


class Int8LinearFunction(torch.autograd.Function):
    """Forward in int8 (outlier columns in fp16), memory-efficient backward.

    The int8 weight is frozen: no weight gradient is returned."""

    @staticmethod
    def forward(ctx, A, CB, SCB, bias, threshold):
        global _warned_cast
        if A.dtype != torch.float16 and not _warned_cast:
            warnings.warn(f"int8 linear: input of dtype {A.dtype} is cast to float16 for quantization "
                          "and the result cast back", stacklevel=3)
            _warned_cast = True
        shape = A.shape
        A2 = A.reshape(-1, shape[-1]).contiguous()
        out = int8_linear_forward(A2, CB, SCB, bias, threshold)
        ctx.save_for_backward(CB, SCB)
        ctx.grad_shape = shape
        ctx.has_bias = bias is not None
        return out.reshape(*shape[:-1], CB.shape[0])

    @staticmethod
    def backward(ctx, g):
        CB, SCB = ctx.saved_tensors
        g2 = g.reshape(-1, g.shape[-1]).contiguous()
        need_b = ctx.has_bias and ctx.needs_input_grad[3]
        gA, gb = int8_linear_backward_input(g2, CB, SCB, with_grad_bias=need_b)
        gA = gA.reshape(ctx.grad_shape) if ctx.needs_input_grad[0] else None
        return gA, None, None, gb, None


class Int8LinearTrainableFunction(torch.autograd.Function):
    """Trainable-weight mode (bitsandbytes' has_fp16_weights option): the weight W
    (same dtype as the input) is quantized on each forward; the backward returns
    grad_A through the memory-efficient kernel from this call's int8 weights and
    grad_W = D(fp16(G)^T fp16(A))."""

    @staticmethod
    def forward(ctx, A, W, bias, threshold):
        if W.dtype != A.dtype:
            raise ValueError("the trainable weight must have the input's dtype")
        shape = A.shape
        A2 = A.reshape(-1, shape[-1]).contiguous()
        CB, SCB = quantize_weight(W.detach().contiguous())
        out = int8_linear_forward(A2, CB, SCB, bias, threshold)
        ctx.save_for_backward(A2, CB, SCB)
        ctx.grad_shape = shape
        ctx.has_bias = bias is not None
        return out.reshape(*shape[:-1], CB.shape[0])

    @staticmethod
    def backward(ctx, g):
        A2, CB, SCB = ctx.saved_tensors
        g2 = g.reshape(-1, g.shape[-1]).contiguous()
        need_b = ctx.has_bias and ctx.needs_input_grad[2]
        gA = gb = gW = None
        if ctx.needs_input_grad[0] or need_b:
            gA, gb = int8_linear_backward_input(g2, CB, SCB, with_grad_bias=need_b)
            gA = gA.reshape(ctx.grad_shape) if ctx.needs_input_grad[0] else None
        if ctx.needs_input_grad[1]:
            gW = int8_linear_backward_weight(g2, A2)
        return gA, gW, gb, None


class Int8Linear(torch.nn.Module):
    """Linear layer with int8 row-major weights (quantized once) and a trainable bias."""

    def __init__(self, weight: torch.Tensor, bias: Optional[torch.Tensor] = None, threshold: float = 6.0):
        super().__init__()
        CB, SCB = quantize_weight(weight.detach().contiguous())
        self.register_buffer("CB", CB)
        self.register_buffer("SCB", SCB)
        self.bias = torch.nn.Parameter(bias.detach().clone()) if bias is not None else None
        self.threshold = float(threshold)

    def forward(self, x):
        b = self.bias.to(x.dtype) if self.bias is not None else None
        return Int8LinearFunction.apply(x, self.CB, self.SCB, b, self.threshold)


class Int8LinearTrainable(torch.nn.Module):
    """Linear layer in the trainable-weight mode: W is a parameter (kept in the
    input dtype) that is re-quantized to int8 on every forward."""

    def __init__(self, weight: torch.Tensor, bias: Optional[torch.Tensor] = None, threshold: float = 6.0):
        super().__init__()
        self.weight = torch.nn.Parameter(weight.detach().clone())
        self.bias = torch.nn.Parameter(bias.detach().clone()) if bias is not None else None
        self.threshold = float(threshold)

    def forward(self, x):
        return Int8LinearTrainableFunction.apply(x, self.weight, self.bias, self.threshold)

"""Fused attention KL divergence (StreamKL) for AMD Instinct MI355X.

Thin torch-facing binding over the C ABI in include/streamkl.h: it allocates
outputs with torch, reads device pointers and the current HIP stream, and calls
the library.  All arithmetic runs in the library's HIP kernels.

    kl, lse1, lse2 = streamkl_fwd(q1, k1, q2, k2, causal=True)
    dq1, dk1, dq2, dk2 = streamkl_bwd(q1, k1, q2, k2, kl, lse1, lse2, g, causal=True)
    loss_rows = attention_kl(q1, k1, q2, k2, causal=True)   # autograd

Q tensors are [B, H, NQ, D] and K tensors [B, H, NK, D], contiguous, bf16 or
fp32, on a HIP device; D is 64 or 128.

Packed variable-length batches use head-major tensors, Q [H, TQ, D] and
K [H, TK, D], with cumulative sequence offsets cu_seqlens_q / cu_seqlens_k
(B + 1 int32 values from 0):

    kl, lse1, lse2 = streamkl_fwd_varlen(q1, k1, q2, k2, cu_q, cu_k, causal=True)
    dq1, dk1, dq2, dk2 = streamkl_bwd_varlen(q1, k1, q2, k2, cu_q, cu_k, kl, lse1, lse2, g, causal=True)
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import StreamKLError

__all__ = ["streamkl_fwd", "streamkl_fwd_splitk", "streamkl_fwd_splitk_noalloc", "streamkl_bwd", "streamkl_bwd_prepare", "streamkl_bwd_dk",
           "streamkl_bwd_dq", "attention_kl",
           "streamkl_fwd_varlen", "streamkl_bwd_varlen", "varlen_problem_for", "bwd_varlen_workspace_size",
           "attention_kl_varlen",
           "StreamKLError", "problem_for", "fwd_splitk_workspace_size", "bwd_workspace_size",
           "streamkl_probe_mfma_bf16"]

_DTYPES = {torch.bfloat16: _lib.STREAMKL_BF16, torch.float32: _lib.STREAMKL_FP32}
if hasattr(torch, "float8_e4m3fn"):  # forward entry points only
    _DTYPES[torch.float8_e4m3fn] = _lib.STREAMKL_FP8_E4M3


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def problem_for(q1: torch.Tensor, k1: torch.Tensor, scale: Optional[float], causal: bool) -> _lib.Problem:
    if q1.dim() != 4 or k1.dim() != 4:
        raise ValueError("expected [B, H, N, D] tensors")
    B, H, NQ, D = q1.shape
    NK = k1.shape[2]
    if q1.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q1.dtype}")
    return _lib.Problem(B, H, NQ, NK, D, float(1.0 / math.sqrt(D) if scale is None else scale),
                        1 if causal else 0, _DTYPES[q1.dtype])


def _check_inputs(q1, k1, q2, k2):
    for t in (q1, k1, q2, k2):
        if not t.is_cuda:
            raise ValueError("inputs must live on a HIP device")
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
        if t.dtype != q1.dtype:
            raise TypeError("all inputs must share one dtype")
    if q2.shape != q1.shape or k2.shape != k1.shape:
        raise ValueError("teacher and student shapes differ")
    if k1.shape[:2] != q1.shape[:2] or k1.shape[3] != q1.shape[3]:
        raise ValueError("Q and K disagree on batch, heads or head dim")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _ws_bytes(workspace: Optional[torch.Tensor], device, what: str) -> int:
    """Size in bytes of a caller-supplied workspace, which must be a contiguous
    tensor on the inputs' device (0 for None)."""
    if workspace is None:
        return 0
    if not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous() or workspace.device != device:
        raise ValueError(f"{what}: the workspace must be a contiguous tensor on {device}")
    return workspace.numel() * workspace.element_size()


def _check_out(ts, shapes, device, what: str) -> None:
    """Caller-supplied outputs: contiguous fp32 tensors of the expected shapes on
    the inputs' device (None where the output is skipped).  The library only
    sees pointers, so a smaller or mistyped buffer would be written past its end."""
    if len(ts) != len(shapes):
        raise ValueError(f"{what}: expected {len(shapes)} output tensors, got {len(ts)}")
    for t, shp in zip(ts, shapes):
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{what}: outputs must be contiguous fp32 tensors")
        if tuple(t.shape) != tuple(shp):
            raise ValueError(f"{what}: output of shape {tuple(t.shape)}, expected {tuple(shp)}")
        if t.device != device:
            raise ValueError(f"{what}: output on {t.device}, inputs on {device}")


def streamkl_fwd(q1, k1, q2, k2, scale: Optional[float] = None, causal: bool = False,
                 out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """Per-row KL(P1||P2), LSE1, LSE2 (fp32 [B, H, NQ]) in one online pass."""
    _check_inputs(q1, k1, q2, k2)
    p = problem_for(q1, k1, scale, causal)
    if out is None:
        shp = q1.shape[:3]
        out = tuple(torch.empty(shp, dtype=torch.float32, device=q1.device) for _ in range(3))
    _check_out(tuple(out), (q1.shape[:3],) * 3, q1.device, "streamkl_fwd")
    kl, lse1, lse2 = out
    st = _lib.lib().streamkl_fwd(p, _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(kl), _ptr(lse1),
                                 _ptr(lse2), _stream_handle(q1.device))
    _lib.check(st, "streamkl_fwd")
    return kl, lse1, lse2


def fwd_splitk_workspace_size(q1, k1, num_splits: int, scale=None, causal=False) -> int:
    p = problem_for(q1, k1, scale, causal)
    return int(_lib.lib().streamkl_fwd_splitk_workspace_size(p, int(num_splits)))


def streamkl_fwd_splitk(q1, k1, q2, k2, num_splits: int, scale: Optional[float] = None,
                        causal: bool = False, workspace: Optional[torch.Tensor] = None, out=None):
    """Split-K forward: key range cut into `num_splits` chunks, merged by LSE rescaling."""
    _check_inputs(q1, k1, q2, k2)
    p = problem_for(q1, k1, scale, causal)
    if out is None:
        shp = q1.shape[:3]
        out = tuple(torch.empty(shp, dtype=torch.float32, device=q1.device) for _ in range(3))
    _check_out(tuple(out), (q1.shape[:3],) * 3, q1.device, "streamkl_fwd_splitk")
    kl, lse1, lse2 = out
    need = int(_lib.lib().streamkl_fwd_splitk_workspace_size(p, int(num_splits)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q1.device)
    ws_bytes = _ws_bytes(workspace, q1.device, "streamkl_fwd_splitk")
    st = _lib.lib().streamkl_fwd_splitk(p, _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(kl), _ptr(lse1),
                                        _ptr(lse2), int(num_splits), _ptr(workspace), ws_bytes,
                                        _stream_handle(q1.device))
    _lib.check(st, "streamkl_fwd_splitk")
    return kl, lse1, lse2


def streamkl_fwd_splitk_noalloc(q1, k1, q2, k2, num_splits: int, scale: Optional[float] = None,
                                causal: bool = False, out=None):
    """The split-K forward with its partial states in the library's own device
    scratch (no workspace, no allocation by the library; calls on one GPU
    share the scratch and must not overlap).  Pass `out` to allocate nothing
    here either."""
    _check_inputs(q1, k1, q2, k2)
    p = problem_for(q1, k1, scale, causal)
    if out is None:
        shp = q1.shape[:3]
        out = tuple(torch.empty(shp, dtype=torch.float32, device=q1.device) for _ in range(3))
    _check_out(tuple(out), (q1.shape[:3],) * 3, q1.device, "streamkl_fwd_splitk_noalloc")
    kl, lse1, lse2 = out
    st = _lib.lib().streamkl_fwd_splitk_noalloc(p, _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(kl), _ptr(lse1),
                                                _ptr(lse2), int(num_splits), _stream_handle(q1.device))
    _lib.check(st, "streamkl_fwd_splitk_noalloc")
    return kl, lse1, lse2


def bwd_workspace_size(q1, k1, scale=None, causal=False) -> int:
    return int(_lib.lib().streamkl_bwd_workspace_size(problem_for(q1, k1, scale, causal)))


def bwd_workspace_size_min(q1, k1, scale=None, causal=False) -> int:
    """Smallest workspace streamkl_bwd accepts: sigma, the operand scales and their
    chunk maxima, without the partials of a key-split query pass (which then runs
    unsplit)."""
    return int(_lib.lib().streamkl_bwd_workspace_size_min(problem_for(q1, k1, scale, causal)))


def streamkl_bwd(q1, k1, q2, k2, kl, lse1, lse2, g, scale: Optional[float] = None, causal: bool = False,
                 teacher: bool = True, student: bool = True, workspace: Optional[torch.Tensor] = None,
                 out=None):
    """Gradients (dq1, dk1, dq2, dk2) of sum(g * KL); a skipped pair comes back as None."""
    _check_inputs(q1, k1, q2, k2)
    p = problem_for(q1, k1, scale, causal)
    _check_rowvecs(q1, kl, lse1, lse2, g)
    if out is None:
        def mk(ref, on):
            return torch.empty(ref.shape, dtype=torch.float32, device=ref.device) if on else None
        out = (mk(q1, teacher), mk(k1, teacher), mk(q2, student), mk(k2, student))
    _check_out(tuple(out), (q1.shape, k1.shape, q2.shape, k2.shape), q1.device, "streamkl_bwd")
    dq1, dk1, dq2, dk2 = out
    workspace, ws_bytes = _workspace(p, q1.device, workspace)
    st = _lib.lib().streamkl_bwd(p, _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(kl), _ptr(lse1),
                                 _ptr(lse2), _ptr(g), _ptr(dq1), _ptr(dk1), _ptr(dq2), _ptr(dk2),
                                 _ptr(workspace), ws_bytes, _stream_handle(q1.device))
    _lib.check(st, "streamkl_bwd")
    return dq1, dk1, dq2, dk2


def _check_rowvecs(q1, *ts):
    for t in ts:
        if t.dtype != torch.float32 or not t.is_contiguous() or t.shape != q1.shape[:3]:
            raise ValueError("kl, lse1, lse2, g must be contiguous fp32 [B, H, NQ]")


def _workspace(p, dev, workspace):
    need = int(_lib.lib().streamkl_bwd_workspace_size(p))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    return workspace, _ws_bytes(workspace, dev, "backward")


def streamkl_bwd_prepare(q1, k1, q2, k2, g, scale: Optional[float] = None, causal: bool = False,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-(b,h) dS scale factors and (bf16 inputs) fp16 operand scales for the
    backward passes; returns the workspace."""
    _check_inputs(q1, k1, q2, k2)
    p = problem_for(q1, k1, scale, causal)
    _check_rowvecs(q1, g)
    workspace, nbytes = _workspace(p, q1.device, workspace)
    st = _lib.lib().streamkl_bwd_prepare(p, _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(g), _ptr(workspace),
                                         nbytes, _stream_handle(q1.device))
    _lib.check(st, "streamkl_bwd_prepare")
    return workspace


def _pass(name, q1, k1, q2, k2, kl, lse1, lse2, g, scale, causal, workspace, out, teacher, student, refs):
    _check_inputs(q1, k1, q2, k2)
    p = problem_for(q1, k1, scale, causal)
    _check_rowvecs(q1, kl, lse1, lse2, g)
    if workspace is None:
        raise ValueError(f"{name} needs the workspace filled by streamkl_bwd_prepare")
    nbytes = _ws_bytes(workspace, q1.device, name)
    if out is None:
        out = tuple(torch.empty(r.shape, dtype=torch.float32, device=r.device) if on else None
                    for r, on in zip(refs, (teacher, student)))
    _check_out(tuple(out), tuple(r.shape for r in refs), q1.device, name)
    a, b = out
    st = getattr(_lib.lib(), name)(p, _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(kl), _ptr(lse1),
                                   _ptr(lse2), _ptr(g), _ptr(a), _ptr(b), _ptr(workspace), nbytes,
                                   _stream_handle(q1.device))
    _lib.check(st, name)
    return a, b


def streamkl_bwd_dk(q1, k1, q2, k2, kl, lse1, lse2, g, scale=None, causal=False, workspace=None, out=None,
                    teacher=True, student=True):
    """Key gradients (dk1, dk2); `workspace` must hold streamkl_bwd_prepare's result."""
    return _pass("streamkl_bwd_dk", q1, k1, q2, k2, kl, lse1, lse2, g, scale, causal, workspace, out,
                 teacher, student, (k1, k2))


def streamkl_bwd_dq(q1, k1, q2, k2, kl, lse1, lse2, g, scale=None, causal=False, workspace=None, out=None,
                    teacher=True, student=True):
    """Query gradients (dq1, dq2); `workspace` must hold streamkl_bwd_prepare's result."""
    return _pass("streamkl_bwd_dq", q1, k1, q2, k2, kl, lse1, lse2, g, scale, causal, workspace, out,
                 teacher, student, (q1, q2))


class _AttentionKL(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q1, k1, q2, k2, scale, causal):
        q1, k1, q2, k2 = (t.contiguous() for t in (q1, k1, q2, k2))
        kl, lse1, lse2 = streamkl_fwd(q1, k1, q2, k2, scale, causal)
        ctx.save_for_backward(q1, k1, q2, k2, kl, lse1, lse2)
        ctx.scale, ctx.causal = scale, causal
        return kl

    @staticmethod
    def backward(ctx, g):
        q1, k1, q2, k2, kl, lse1, lse2 = ctx.saved_tensors
        need1 = ctx.needs_input_grad[0] or ctx.needs_input_grad[1]
        need2 = ctx.needs_input_grad[2] or ctx.needs_input_grad[3]
        if not (need1 or need2):
            return None, None, None, None, None, None
        dq1, dk1, dq2, dk2 = streamkl_bwd(q1, k1, q2, k2, kl, lse1, lse2,
                                          g.to(torch.float32).contiguous(), ctx.scale, ctx.causal,
                                          teacher=need1, student=need2)
        cast = lambda d, ref: None if d is None else d.to(ref.dtype)
        return cast(dq1, q1), cast(dk1, k1), cast(dq2, q2), cast(dk2, k2), None, None


def attention_kl(q1, k1, q2, k2, scale: Optional[float] = None, causal: bool = False) -> torch.Tensor:
    """Differentiable per-row KL(P1||P2), [B, H, NQ] fp32."""
    return _AttentionKL.apply(q1, k1, q2, k2, scale, causal)


class _Varlen:
    """A streamkl_varlen_problem together with the host offset arrays it points at."""

    def __init__(self, q1, k1, cu_seqlens_q, cu_seqlens_k, scale, causal):
        if q1.dim() != 3 or k1.dim() != 3:
            raise ValueError("packed tensors are [H, T, D]")
        if q1.dtype not in _DTYPES:
            raise TypeError(f"unsupported dtype {q1.dtype}")
        H, TQ, D = q1.shape
        # The offsets are read on the host (a device tensor is copied, which synchronises).
        self.cu_q = torch.as_tensor(cu_seqlens_q, dtype=torch.int32).to("cpu").contiguous()
        self.cu_k = torch.as_tensor(cu_seqlens_k, dtype=torch.int32).to("cpu").contiguous()
        if self.cu_q.dim() != 1 or self.cu_q.shape != self.cu_k.shape or self.cu_q.numel() < 1:
            raise ValueError("cu_seqlens_q and cu_seqlens_k must be 1-D with B + 1 entries each")
        if int(self.cu_q[-1]) != TQ or int(self.cu_k[-1]) != k1.shape[1]:
            raise ValueError("the last offsets must equal the packed lengths TQ and TK")
        self.p = _lib.VarlenProblem(self.cu_q.numel() - 1, H, D, self.cu_q.data_ptr(), self.cu_k.data_ptr(),
                                    float(1.0 / math.sqrt(D) if scale is None else scale),
                                    1 if causal else 0, _DTYPES[q1.dtype])


def varlen_problem_for(q1, k1, cu_seqlens_q, cu_seqlens_k, scale=None, causal=False) -> _Varlen:
    return _Varlen(q1, k1, cu_seqlens_q, cu_seqlens_k, scale, causal)


def _check_packed(q1, k1, q2, k2):
    for t in (q1, k1, q2, k2):
        if not t.is_cuda:
            raise ValueError("inputs must live on a HIP device")
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
        if t.dtype != q1.dtype:
            raise TypeError("all inputs must share one dtype")
    if q2.shape != q1.shape or k2.shape != k1.shape:
        raise ValueError("teacher and student shapes differ")
    if k1.shape[0] != q1.shape[0] or k1.shape[2] != q1.shape[2]:
        raise ValueError("Q and K disagree on heads or head dim")


def streamkl_fwd_varlen(q1, k1, q2, k2, cu_seqlens_q, cu_seqlens_k, scale: Optional[float] = None,
                        causal: bool = False, out=None):
    """Per-row KL, LSE1, LSE2 (fp32 [H, TQ]) of a packed batch of sequences."""
    _check_packed(q1, k1, q2, k2)
    v = _Varlen(q1, k1, cu_seqlens_q, cu_seqlens_k, scale, causal)
    if out is None:
        out = tuple(torch.empty(q1.shape[:2], dtype=torch.float32, device=q1.device) for _ in range(3))
    _check_out(tuple(out), (q1.shape[:2],) * 3, q1.device, "streamkl_fwd_varlen")
    kl, lse1, lse2 = out
    st = _lib.lib().streamkl_fwd_varlen(v.p, _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(kl), _ptr(lse1),
                                        _ptr(lse2), _stream_handle(q1.device))
    _lib.check(st, "streamkl_fwd_varlen")
    return kl, lse1, lse2


def bwd_varlen_workspace_size(q1, k1, cu_seqlens_q, cu_seqlens_k, scale=None, causal=False) -> int:
    v = _Varlen(q1, k1, cu_seqlens_q, cu_seqlens_k, scale, causal)
    return int(_lib.lib().streamkl_bwd_varlen_workspace_size(v.p))


def streamkl_bwd_varlen(q1, k1, q2, k2, cu_seqlens_q, cu_seqlens_k, kl, lse1, lse2, g,
                        scale: Optional[float] = None, causal: bool = False, teacher: bool = True,
                        student: bool = True, workspace: Optional[torch.Tensor] = None, out=None):
    """Gradients (dq1, dk1, dq2, dk2) of sum(g * KL) over a packed batch; a skipped pair is None."""
    _check_packed(q1, k1, q2, k2)
    v = _Varlen(q1, k1, cu_seqlens_q, cu_seqlens_k, scale, causal)
    for t in (kl, lse1, lse2, g):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.shape != q1.shape[:2]:
            raise ValueError("kl, lse1, lse2, g must be contiguous fp32 [H, TQ]")
    if out is None:
        def mk(ref, on):
            return torch.empty(ref.shape, dtype=torch.float32, device=ref.device) if on else None
        out = (mk(q1, teacher), mk(k1, teacher), mk(q2, student), mk(k2, student))
    _check_out(tuple(out), (q1.shape, k1.shape, q2.shape, k2.shape), q1.device, "streamkl_bwd_varlen")
    dq1, dk1, dq2, dk2 = out
    if workspace is None:
        need = int(_lib.lib().streamkl_bwd_varlen_workspace_size(v.p))
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q1.device)
    nbytes = _ws_bytes(workspace, q1.device, "streamkl_bwd_varlen")
    st = _lib.lib().streamkl_bwd_varlen(v.p, _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(kl), _ptr(lse1),
                                        _ptr(lse2), _ptr(g), _ptr(dq1), _ptr(dk1), _ptr(dq2), _ptr(dk2),
                                        _ptr(workspace), nbytes, _stream_handle(q1.device))
    _lib.check(st, "streamkl_bwd_varlen")
    return dq1, dk1, dq2, dk2


class _AttentionKLVarlen(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q1, k1, q2, k2, cu_seqlens_q, cu_seqlens_k, scale, causal):
        q1, k1, q2, k2 = (t.contiguous() for t in (q1, k1, q2, k2))
        cu_q = torch.as_tensor(cu_seqlens_q, dtype=torch.int32).to("cpu")
        cu_k = torch.as_tensor(cu_seqlens_k, dtype=torch.int32).to("cpu")
        kl, lse1, lse2 = streamkl_fwd_varlen(q1, k1, q2, k2, cu_q, cu_k, scale, causal)
        ctx.save_for_backward(q1, k1, q2, k2, kl, lse1, lse2)
        ctx.cu, ctx.scale, ctx.causal = (cu_q, cu_k), scale, causal
        return kl

    @staticmethod
    def backward(ctx, g):
        q1, k1, q2, k2, kl, lse1, lse2 = ctx.saved_tensors
        need1 = ctx.needs_input_grad[0] or ctx.needs_input_grad[1]
        need2 = ctx.needs_input_grad[2] or ctx.needs_input_grad[3]
        none = (None,) * 4
        if not (need1 or need2):
            return (None,) * 8
        dq1, dk1, dq2, dk2 = streamkl_bwd_varlen(q1, k1, q2, k2, *ctx.cu, kl, lse1, lse2,
                                                 g.to(torch.float32).contiguous(), ctx.scale, ctx.causal,
                                                 teacher=need1, student=need2)
        cast = lambda d, ref: None if d is None else d.to(ref.dtype)
        return (cast(dq1, q1), cast(dk1, k1), cast(dq2, q2), cast(dk2, k2)) + none


def attention_kl_varlen(q1, k1, q2, k2, cu_seqlens_q, cu_seqlens_k, scale: Optional[float] = None,
                        causal: bool = False) -> torch.Tensor:
    """Differentiable per-row KL(P1||P2) of a packed batch ([H, T, D] inputs), [H, TQ] fp32."""
    return _AttentionKLVarlen.apply(q1, k1, q2, k2, cu_seqlens_q, cu_seqlens_k, scale, causal)


def streamkl_probe_mfma_bf16(iters: int, workgroups: int, sink: torch.Tensor) -> None:
    """Enqueue the matrix-rate probe on the current stream (workgroups * 4 *
    iters * 4 * 32768 flop); `sink` is a float32 device tensor of at least
    workgroups * 4 elements.  The caller times it with events."""
    if sink.dtype != torch.float32 or not sink.is_cuda or sink.numel() < 4 * int(workgroups):
        raise ValueError("sink must be a float32 device tensor of at least 4 * workgroups elements")
    st = _lib.lib().streamkl_probe_mfma_bf16(int(iters), int(workgroups), _ptr(sink), _stream_handle(sink.device))
    _lib.check(st, "streamkl_probe_mfma_bf16")

"""FP8 (E4M3) flash-attention forward for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libfp8attn.so`` (include/fp8attn.h):
argument marshalling only, every step of the computation runs in the HIP
kernels.  PyTorch provides device memory and streams.

    import fp8_flash_attention_amd as fa
    out = fa.attention(q, k, v, cu_seqlens=[0, 15104, 30208, 30208, 30271, 30272])

or, with an explicit plan and workspace (no allocation per call):

    plan = fa.Plan(tokens, heads, cu_seqlens, device=0)
    ws = plan.new_workspace()
    fa.quantize(plan, q, k, v, ws)
    fa.forward(plan, ws, out)

The computation, for every segment [a, b) of cu_seqlens and every head h, is
``out[a:b, h] = softmax(q[a:b, h] @ k[a:b, h]^T * softmax_scale) @ v[a:b, h]``
(FlashInfer "minimax_h3_sm120_varlen_attention_nvfp4" page), with Q/K/V
quantized per head to E4M3 and both products on FP8 MFMA.  ``fmt="mxfp4"``
selects the block-scaled FP4 variant (E2M1 operands and probabilities with
one power-of-two scale per 32 elements).  ``q_centre=True`` adds the page's Q
block-mean centring to either format (E4M3: the mean term added back near
exactly from a precomputed table, for Q with large per-channel offsets).
"""
from __future__ import annotations

import ctypes
import math
from collections import OrderedDict
from typing import Dict, Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import Fp8AttnError  # noqa: F401

HEAD_DIM = 128
DEFAULT_SCALE = 1.0 / math.sqrt(HEAD_DIM)

__all__ = ["Plan", "quantize", "quantize_noalloc", "forward", "attention", "get_plan", "clear_plan_cache",
           "varlen_attention_fp8", "varlen_attention_mxfp4", "workspace_bytes",
           "Fp8AttnError", "HEAD_DIM", "DEFAULT_SCALE"]


def _stream_handle(device: torch.device, stream=None) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


class Plan:
    """A validated segment table and work schedule (``fp8attn_plan_ex``).

    ``device=None`` uses the current CUDA/HIP device; ``device=-1`` builds a
    host-only plan that can be inspected but not run.  ``segment_scales=True``
    quantizes every segment with its own per-head scales.  ``fmt`` is
    ``"e4m3"`` (default) or ``"mxfp4"``; ``q_centre`` centres Q by its 128-row
    block means and adds the mean term back (E4M3: its workspace holds one 4-byte mean-term entry per (128-query block, key) of
    every segment and head).  ``causal``: query i of a segment attends to
    the keys j <= i of that segment.  ``head_dim``: 128, or (e4m3 only) any
    multiple of 8 from 8 to 128 (run at the kernel width 64 or 128 with the
    missing channels as zeros).  ``exact_probs`` (e4m3 only): probabilities rounded from the
    FP32 exp2 instead of the default log-linear E4M3 code (slower, a little
    more accurate).
    """

    def __init__(self, tokens: int, heads: int, cu_seqlens: Optional[Sequence[int]] = None,
                 softmax_scale: Optional[float] = None, device=None, segment_scales: bool = False,
                 fmt: str = "e4m3", q_centre: bool = False, causal: bool = False, head_dim: int = HEAD_DIM,
                 exact_probs: bool = False):
        L = _lib.lib()
        if cu_seqlens is None:
            cu_seqlens = [0, tokens]
        cu = [int(x) for x in cu_seqlens]
        if len(cu) < 2:
            raise ValueError("cu_seqlens needs at least two entries")
        if device is None:
            device = torch.cuda.current_device()
        if isinstance(device, torch.device):
            device = device.index if device.index is not None else torch.cuda.current_device()
        self.device_index = int(device)
        self.tokens = int(tokens)
        self.heads = int(heads)
        self.cu_seqlens = tuple(cu)
        if not (8 <= head_dim <= HEAD_DIM and head_dim % 8 == 0):
            raise ValueError(f"head_dim must be a multiple of 8 from 8 to {HEAD_DIM} (got {head_dim})")
        self.softmax_scale = float(1.0 / math.sqrt(head_dim) if softmax_scale is None else softmax_scale)
        self.segment_scales = bool(segment_scales)
        if fmt not in ("e4m3", "mxfp4"):
            raise ValueError(f"fmt must be 'e4m3' or 'mxfp4' (got {fmt!r})")
        self.fmt = fmt
        self.q_centre = bool(q_centre)
        self.causal = bool(causal)
        self.head_dim = int(head_dim)
        self.exact_probs = bool(exact_probs)
        arr = (ctypes.c_int32 * len(cu))(*cu)
        h = ctypes.c_void_p()
        self._h = None
        flags = ((_lib.PLAN_SEGMENT_SCALES if self.segment_scales else 0)
                 | (_lib.PLAN_MXFP4 if fmt == "mxfp4" else 0) | (_lib.PLAN_Q_CENTRE if self.q_centre else 0)
                 | (_lib.PLAN_CAUSAL if self.causal else 0)
                 | (_lib.plan_head_dim(self.head_dim) if self.head_dim != HEAD_DIM else 0)
                 | (_lib.PLAN_EXACT_PROBS if self.exact_probs else 0))
        _lib.check(L.fp8attn_plan_ex(ctypes.byref(h), self.tokens, self.heads, arr, len(cu) - 1,
                                     ctypes.c_float(self.softmax_scale), self.device_index, flags),
                   "fp8attn_plan_ex")
        self._h = h
        self._used = False          # set once work has been enqueued with this plan
        self.workspace_bytes = int(L.fp8attn_workspace_bytes(h))

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h

    @property
    def device(self) -> torch.device:
        return torch.device("cuda", self.device_index)

    def info(self) -> Dict[str, int]:
        buf = (ctypes.c_int64 * _lib.PLAN_INFO_LEN)()
        _lib.check(_lib.lib().fp8attn_plan_info(self._h, buf), "fp8attn_plan_info")
        keys = ["tokens", "heads", "num_segments", "workspace_rows", "work_items", "stat_chunks",
                "query_tile", "key_tile", "segment_scales", "partial_slots", "mxfp4", "q_centre", "causal",
                "head_dim"]
        return dict(zip(keys, list(buf)))

    def work_items(self):
        n = ctypes.c_int64()
        _lib.check(_lib.lib().fp8attn_plan_work_items(self._h, None, 0, ctypes.byref(n)), "work_items")
        buf = (ctypes.c_int32 * (4 * max(1, n.value)))()
        _lib.check(_lib.lib().fp8attn_plan_work_items(self._h, buf, n.value, ctypes.byref(n)), "work_items")
        flat = list(buf)[: 4 * n.value]
        return [tuple(flat[4 * i: 4 * i + 4]) for i in range(n.value)]

    def new_workspace(self) -> torch.Tensor:
        return torch.empty(self.workspace_bytes, dtype=torch.uint8, device=self.device)

    def region(self, workspace: torch.Tensor, which: int) -> torch.Tensor:
        """A typed view of one workspace region (codes, scales or K means)."""
        ptr = ctypes.c_void_p()
        dims = (ctypes.c_int64 * 3)()
        _lib.check(_lib.lib().fp8attn_workspace_region(self._h, ctypes.c_void_p(workspace.data_ptr()), which,
                                                       ctypes.byref(ptr), dims), "fp8attn_workspace_region")
        off = ptr.value - workspace.data_ptr()
        shape = tuple(dims)
        if which in (_lib.REGION_Q, _lib.REGION_K, _lib.REGION_V, _lib.REGION_Q_BSCALES, _lib.REGION_K_BSCALES,
                     _lib.REGION_V_BSCALES, _lib.REGION_QM_CODES, _lib.REGION_QM_SCALES):
            n = shape[0] * shape[1] * shape[2]
            return workspace[off: off + n].view(shape)
        n = shape[0] * shape[1] * shape[2]
        if which == _lib.REGION_SCALES and shape[1] == 1:
            shape = (shape[0], shape[2])          # per-head scales: [3][H]
        if which == _lib.REGION_QM_TERM:          # uint32 entries (two bf16), as int32
            return workspace[off: off + 4 * shape[0] * shape[1]].view(torch.int32).view(shape[0], shape[1])
        return workspace[off: off + 4 * n].view(torch.float32).view(shape)

    def stats_offset(self) -> int:
        """Bytes of workspace before the statistics region (all that ``quantize_noalloc`` and
        ``forward`` need)."""
        ptr = ctypes.c_void_p()
        dims = (ctypes.c_int64 * 3)()
        base = 256
        _lib.check(_lib.lib().fp8attn_workspace_region(self._h, ctypes.c_void_p(base), _lib.REGION_STATS,
                                                       ctypes.byref(ptr), dims), "fp8attn_workspace_region")
        return int(ptr.value - base)

    def close(self):
        """Free the plan.  Work enqueued with it must be complete first (its device
        tables are freed), so a plan that has run waits for its device."""
        if self._h is not None:
            if self._used and self.device_index >= 0:
                torch.cuda.synchronize(self.device_index)
            _lib.lib().fp8attn_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _strides(x: torch.Tensor, name: str, head_dim: int = HEAD_DIM):
    if x.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16 (got {x.dtype})")
    if x.dim() != 3 or x.shape[2] != head_dim:
        raise ValueError(f"{name} must have shape [tokens, heads, {head_dim}] (got {tuple(x.shape)})")
    if x.stride(2) != 1:
        raise ValueError(f"{name} must have unit stride in the head dimension")
    return _lib.i64_array([x.stride(0), x.stride(1)])


def _on_plan_device(plan: Plan, x: torch.Tensor, name: str) -> None:
    """Device pointers handed to the library must live on the plan's GPU."""
    if plan.device_index < 0:
        raise Fp8AttnError(_lib.EINVAL, name, "host-only plan cannot run")
    if not x.is_cuda or x.device.index != plan.device_index:
        raise ValueError(f"{name} must be a tensor on cuda:{plan.device_index} (got {x.device})")


def quantize(plan: Plan, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, workspace: torch.Tensor,
             stream=None) -> None:
    """``fp8attn_quantize``: E4M3 codes and per-head scales of q, k, v into ``workspace``."""
    for name, x in (("q", q), ("k", k), ("v", v)):
        if tuple(x.shape[:2]) != (plan.tokens, plan.heads):
            raise ValueError(f"{name} shape {tuple(x.shape)} does not match the plan")
        _on_plan_device(plan, x, name)
    _on_plan_device(plan, workspace, "workspace")
    D = plan.head_dim
    qs, ks, vs = _strides(q, "q", D), _strides(k, "k", D), _strides(v, "v", D)
    st = _stream_handle(plan.device, stream)
    plan._used = True
    _lib.check(_lib.lib().fp8attn_quantize(plan.handle, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                           ctypes.c_void_p(v.data_ptr()), qs, ks, vs,
                                           ctypes.c_void_p(workspace.data_ptr()),
                                           workspace.numel() * workspace.element_size(), st),
               "fp8attn_quantize")


def quantize_noalloc(plan: Plan, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, workspace: torch.Tensor,
                     stream=None) -> None:
    """``fp8attn_quantize_noalloc``: as ``quantize``, with the statistics in the library's static
    device buffer; ``workspace`` may stop at ``plan.stats_offset()`` bytes."""
    for name, x in (("q", q), ("k", k), ("v", v)):
        if tuple(x.shape[:2]) != (plan.tokens, plan.heads):
            raise ValueError(f"{name} shape {tuple(x.shape)} does not match the plan")
        _on_plan_device(plan, x, name)
    _on_plan_device(plan, workspace, "workspace")
    D = plan.head_dim
    qs, ks, vs = _strides(q, "q", D), _strides(k, "k", D), _strides(v, "v", D)
    st = _stream_handle(plan.device, stream)
    plan._used = True
    _lib.check(_lib.lib().fp8attn_quantize_noalloc(plan.handle, ctypes.c_void_p(q.data_ptr()),
                                                   ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                                   qs, ks, vs, ctypes.c_void_p(workspace.data_ptr()),
                                                   workspace.numel() * workspace.element_size(), st),
               "fp8attn_quantize_noalloc")


def forward(plan: Plan, workspace: torch.Tensor, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """``fp8attn_forward``: BF16 output from the codes in ``workspace``."""
    if out is None:
        out = torch.empty((plan.tokens, plan.heads, plan.head_dim), dtype=torch.bfloat16, device=plan.device)
    if tuple(out.shape) != (plan.tokens, plan.heads, plan.head_dim):
        raise ValueError("out shape does not match the plan")
    _on_plan_device(plan, out, "out")
    _on_plan_device(plan, workspace, "workspace")
    os_ = _strides(out, "out", plan.head_dim)
    lse_ptr = None
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != (plan.heads, plan.tokens) or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 [heads, tokens] tensor")
        _on_plan_device(plan, lse, "lse")
        lse_ptr = ctypes.c_void_p(lse.data_ptr())
    st = _stream_handle(plan.device, stream)
    plan._used = True
    _lib.check(_lib.lib().fp8attn_forward(plan.handle, ctypes.c_void_p(workspace.data_ptr()),
                                          workspace.numel() * workspace.element_size(),
                                          ctypes.c_void_p(out.data_ptr()), os_, lse_ptr, st), "fp8attn_forward")
    return out


# Plans of attention(), least recently used first.  The FlashInfer page caches
# its segment plan per (cu_seqlens, heads, device); the review of the sglang
# PR "[diffusion] attention: add fp8_fa_sm120 FP8 backend for SM120 GPUs" asks
# that retained state stay bounded across shapes, so the cache holds at most
# PLAN_CACHE_SIZE plans (a few hundred KB of device tables each at most) and
# evicts the least recently used one.
PLAN_CACHE_SIZE = 16
_PLANS: "OrderedDict[Tuple, Plan]" = OrderedDict()


def get_plan(tokens: int, heads: int, cu_seqlens: Sequence[int], softmax_scale: float, device: int,
             segment_scales: bool = False, fmt: str = "e4m3", q_centre: bool = False, causal: bool = False,
             head_dim: int = HEAD_DIM, exact_probs: bool = False) -> Plan:
    """The cached plan for (cu_seqlens, heads, scale, device, quantization mode), built on first use."""
    key = (tuple(int(x) for x in cu_seqlens), int(heads), float(softmax_scale), int(device), bool(segment_scales),
           fmt, bool(q_centre), bool(causal), int(head_dim), bool(exact_probs))
    p = _PLANS.get(key)
    if p is not None:
        _PLANS.move_to_end(key)
        return p
    p = Plan(tokens, heads, cu_seqlens, softmax_scale, device, segment_scales=segment_scales, fmt=fmt,
             q_centre=q_centre, causal=causal, head_dim=head_dim, exact_probs=exact_probs)
    _PLANS[key] = p
    while len(_PLANS) > max(1, PLAN_CACHE_SIZE):
        _, old = _PLANS.popitem(last=False)
        old.close()               # waits for the device if the plan has run
    return p


def clear_plan_cache() -> None:
    """Free every cached plan (each waits for its device if it has run)."""
    while _PLANS:
        _, p = _PLANS.popitem(last=False)
        p.close()


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: Optional[Sequence[int]] = None,
              softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
              return_lse: bool = False, causal: bool = False, workspace: Optional[torch.Tensor] = None,
              segment_scales: bool = False, fmt: str = "e4m3", q_centre: bool = False, exact_probs: bool = False):
    """FP8 attention over packed [tokens, heads, D] BF16 q/k/v.

    ``cu_seqlens`` is a host sequence of segment boundaries (None = one segment).
    ``segment_scales`` quantizes every segment with its own per-head scales.
    ``fmt="mxfp4"`` runs the block-scaled FP4 variant; ``q_centre`` adds Q
    block-mean centring (either format).  ``causal=True`` masks keys after each query.  The
    head size D (128, or for E4M3 any multiple of 8 up to 128) is taken from
    the inputs' last dimension.  Batched [B, T, heads, D] inputs (views of
    [B*T, heads, D]) are run as B segments of T tokens and returned as
    [B, T, heads, D] (with the LSE as [heads, B*T]).
    """
    if q.dim() == 4:
        if cu_seqlens is not None:
            raise ValueError("batched [B, T, H, D] input takes no cu_seqlens (each batch entry is one segment)")
        B, T0 = q.shape[0], q.shape[1]
        try:
            flat = [x.view(B * T0, x.shape[2], x.shape[3]) for x in (q, k, v)]
            oflat = None if out is None else out.view(B * T0, out.shape[2], out.shape[3])
        except RuntimeError as e:
            raise ValueError("batched q, k, v (and out) must be viewable as [B*T, H, D]") from e
        res = attention(*flat, cu_seqlens=[T0 * i for i in range(B + 1)], softmax_scale=softmax_scale, out=oflat,
                        return_lse=return_lse, causal=causal, workspace=workspace, segment_scales=segment_scales,
                        fmt=fmt, q_centre=q_centre, exact_probs=exact_probs)
        if return_lse:
            return res[0].view(B, T0, *res[0].shape[1:]), res[1]
        return res.view(B, T0, *res.shape[1:])
    T, H, D = q.shape[0], q.shape[1], q.shape[-1]
    if cu_seqlens is None:
        cu_seqlens = [0, T]
    elif isinstance(cu_seqlens, torch.Tensor):
        cu_seqlens = cu_seqlens.tolist()
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    dev = q.device.index if q.device.index is not None else torch.cuda.current_device()
    plan = get_plan(T, H, cu_seqlens, scale, dev, segment_scales, fmt, q_centre, causal, D, exact_probs)
    ws = workspace if workspace is not None else plan.new_workspace()
    quantize(plan, q, k, v, ws)
    lse = torch.empty((H, T), dtype=torch.float32, device=q.device) if return_lse else None
    out = forward(plan, ws, out, lse)
    return (out, lse) if return_lse else out


# ---------------------------------------------------------------------------
# The pages' varlen entry points (FlashInfer page
# "minimax_h3_sm120_varlen_attention_nvfp4", its signature and parameters):
# q, k, v [tokens, heads, 128], a device cu_seqlens with an optional host copy
# that saves the device-to-host read, an optional preallocated out, the
# softmax scale, and a grow-only per-device workspace shared by the FP8 and
# FP4 forms.  Calls that overlap on one device (several streams or threads)
# share that workspace and must be serialized by the caller.
# ---------------------------------------------------------------------------

_SHARED_WS = {}


def _shared_workspace(device_index: int, nbytes: int) -> torch.Tensor:
    ws = _SHARED_WS.get(device_index)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            torch.cuda.synchronize(device_index)   # work queued on the old buffer finishes first
        ws = torch.empty(nbytes, dtype=torch.uint8, device=torch.device("cuda", device_index))
        _SHARED_WS[device_index] = ws
    return ws


def workspace_bytes(device=None) -> int:
    """Bytes of the shared workspace the varlen entry points hold on a device (0 if none)."""
    if isinstance(device, torch.device):
        device = device.index
    idx = torch.cuda.current_device() if device is None else int(device)
    ws = _SHARED_WS.get(idx)
    return 0 if ws is None else int(ws.numel())


def _varlen(q, k, v, cu_seqlens, out, cu_seqlens_host, softmax_scale, return_lse, fmt, q_centre):
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor [segments + 1]")
    if cu_seqlens.device != q.device:
        raise ValueError("cu_seqlens must be on the device of q")
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError(f"q, k, v must be [tokens, heads, {HEAD_DIM}] (got {tuple(q.shape)})")
    if cu_seqlens_host is not None:
        cu = [int(x) for x in cu_seqlens_host]
        if len(cu) != cu_seqlens.numel():
            raise ValueError("cu_seqlens_host must have as many entries as cu_seqlens")
    else:
        cu = cu_seqlens.tolist()              # one synchronizing device-to-host copy
    T, H = q.shape[0], q.shape[1]
    scale = DEFAULT_SCALE if softmax_scale is None else float(softmax_scale)
    dev = q.device.index if q.device.index is not None else torch.cuda.current_device()
    plan = get_plan(T, H, cu, scale, dev, False, fmt, q_centre, False, HEAD_DIM, False)
    ws = _shared_workspace(dev, plan.workspace_bytes)
    quantize(plan, q, k, v, ws)
    lse = torch.empty((H, T), dtype=torch.float32, device=q.device) if return_lse else None
    out = forward(plan, ws, out, lse)
    return (out, lse) if return_lse else out


def varlen_attention_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                         out: Optional[torch.Tensor] = None, *, cu_seqlens_host: Optional[Sequence[int]] = None,
                         softmax_scale: Optional[float] = None, return_lse: bool = False, q_centre: bool = False):
    """Non-causal packed-varlen self-attention on E4M3 operands: for every
    segment [a, b) of cu_seqlens and head h, out[a:b, h] = softmax(q[a:b, h]
    k[a:b, h]^T softmax_scale) v[a:b, h], BF16 [tokens, heads, 128].  The
    E4M3 path of this library (the recipe of sglang PR "[diffusion] attention:
    add fp8_fa_sm120 FP8 backend for SM120 GPUs", "Modifications"), with the
    calling convention of the FlashInfer page
    "flashinfer.diffusion_ops.minimax_h3_sm120_varlen_attention_nvfp4";
    ``return_lse`` adds the natural-log LSE [heads, tokens]; ``q_centre``
    centres Q by its 128-row block means (the page's Q centring) with the mean
    term added back from a precomputed table."""
    return _varlen(q, k, v, cu_seqlens, out, cu_seqlens_host, softmax_scale, return_lse, "e4m3", q_centre)


def varlen_attention_mxfp4(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                           out: Optional[torch.Tensor] = None, *, cu_seqlens_host: Optional[Sequence[int]] = None,
                           softmax_scale: Optional[float] = None, return_lse: bool = False):
    """The same on block-scaled FP4 operands with Q centred by its 128-row
    block means (the page's recipe in gfx950's MX form: one power-of-two scale
    per 32 elements); several times the E4M3 error."""
    return _varlen(q, k, v, cu_seqlens, out, cu_seqlens_host, softmax_scale, return_lse, "mxfp4", True)

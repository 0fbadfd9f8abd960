"""Fused CSR graph attention for AMD MI355X (gfx950): Python binding.

Every step of the computation runs in the HIP kernels of ``libgraph_attn.so``; this module
only marshals arguments: it takes tensors' device pointers, allocates outputs and
workspaces with torch (the library never allocates device memory) and passes torch's
current HIP stream.  ``capi`` holds the raw C entry points under their C names.

    plan = Plan(indptr, indices)          # host planner: bins, hub chunks, transpose
    plan.upload("cuda")                   # one device copy, caller-owned (torch)
    out, lse = fwd(plan, q, k, v)         # dot score, scale 1/sqrt(d)
    dq, dk, dv = bwd(plan, q, k, v, dout, lse)
    out, lse = fwd(plan, s, t, v, score="gat")
    out, arg, slot = reduce_fwd(plan, x, op="max")  # neighbourhood max pooling, its arg
    dx = reduce_bwd(plan, arg, dout, slot=slot)

Method: "On Efficient Scaling of GNNs via IO-Aware Layers Implementations", Technical
Summary > Methodology, attention-based layers (fused score -> online softmax ->
aggregation; backward recomputes weights from the per-node log-sum-exp) and
reduction-based layers (degree-aware min / max pooling, heavy rows as edge chunks whose
partials combine as (value, index) pairs).
"""
from __future__ import annotations

import ctypes
import math
from ctypes import POINTER, byref, c_int32, c_int64, c_size_t, c_void_p

import numpy as np

from . import capi
from .capi import (GA_BF16, GA_F32, GA_REDUCE_MAX, GA_REDUCE_MIN,  # noqa: F401
                   GA_SCORE_DOT, GA_SCORE_GAT, GraphAttnError,
                   graph_attn_reduce_bwd, graph_attn_reduce_bwd_workspace_bytes,
                   graph_attn_reduce_fwd, graph_attn_reduce_fwd_workspace_bytes,
                   graph_attn_reduce_slot_bytes,
                   graph_attn_bwd, graph_attn_bwd_gatv2, graph_attn_bwd_gatv2_workspace_bytes,
                   graph_attn_bwd_workspace_bytes, graph_attn_copy_probe,
                   graph_attn_fwd, graph_attn_fwd_gatv2, graph_attn_fwd_noalloc,
                   graph_attn_fwd_workspace_bytes,
                   graph_attn_gather_probe, graph_attn_gather_probe_cols,
                   graph_attn_gather_probe_random,
                   graph_attn_plan_array,
                   graph_attn_plan_array_count, graph_attn_plan_array_name,
                   graph_attn_plan_create, graph_attn_plan_destroy,
                   graph_attn_plan_device_bytes, graph_attn_plan_get_info,
                   graph_attn_plan_opts_default, graph_attn_plan_upload,
                   graph_attn_status_string, graph_attn_timer_count, graph_attn_timer_enable,
                   graph_attn_timer_read, graph_attn_timer_reset, graph_attn_version)

__all__ = ["Plan", "fwd", "fwd_noalloc", "fwd_gatv2", "bwd", "bwd_gatv2", "graph_attention",
           "graph_attention_gatv2", "reduce_fwd",
           "reduce_bwd", "reduce_slot_dtype", "graph_reduce", "copy_probe", "gather_probe", "gather_probe_cols",
           "gather_probe_random", "timers", "default_opts",
           "GraphAttnError", "capi"]


def default_opts() -> dict:
    o = capi.ga_plan_opts()
    graph_attn_plan_opts_default(byref(o))
    return {n: int(getattr(o, n)) for n, _ in o._fields_}


class Plan:
    """A graph's cached metadata: degree bins, hub chunks and (optionally) the transpose,
    built on the host by the library's planner; ``upload`` copies it to the GPU.

    Thresholds left as None take the library defaults, except that the column hub
    threshold and chunk, and the column XCD split threshold, follow explicitly given row
    values unless given themselves. ``xcd_split_min_deg_exclusive`` > 0 regroups longer
    rows (columns) by neighbour id mod 8 and schedules their chunks to the matching XCD
    (see graph_attn_plan_opts); 0, the default, leaves the CSR as given."""

    def __init__(self, indptr, indices, *, light_max_deg=None, hub_min_deg_exclusive=None,
                 hub_chunk=None, build_csc=True, feature_slices=None,
                 col_hub_min_deg_exclusive=None, col_hub_chunk=None,
                 xcd_split_min_deg_exclusive=None, col_xcd_split_min_deg_exclusive=None):
        ip = np.ascontiguousarray(indptr, dtype=np.int32)
        ix = np.ascontiguousarray(indices, dtype=np.int32)
        opts = capi.ga_plan_opts()
        graph_attn_plan_opts_default(byref(opts))
        if col_hub_min_deg_exclusive is None:
            col_hub_min_deg_exclusive = hub_min_deg_exclusive
        if col_hub_chunk is None:
            col_hub_chunk = hub_chunk
        if col_xcd_split_min_deg_exclusive is None:
            col_xcd_split_min_deg_exclusive = xcd_split_min_deg_exclusive
        for k, v in (("light_max_deg", light_max_deg),
                     ("hub_min_deg_exclusive", hub_min_deg_exclusive),
                     ("hub_chunk", hub_chunk), ("feature_slices", feature_slices),
                     ("col_hub_min_deg_exclusive", col_hub_min_deg_exclusive),
                     ("col_hub_chunk", col_hub_chunk),
                     ("xcd_split_min_deg_exclusive", xcd_split_min_deg_exclusive),
                     ("col_xcd_split_min_deg_exclusive", col_xcd_split_min_deg_exclusive)):
            if v is not None:
                setattr(opts, k, int(v))
        opts.build_csc = 1 if build_csc else 0
        h = c_void_p()
        graph_attn_plan_create(ip.ctypes.data_as(POINTER(c_int32)),
                               ix.ctypes.data_as(POINTER(c_int32)) if ix.size else None,
                               ip.size - 1, ix.size, byref(opts), byref(h))
        self._h = h
        self.n_nodes = ip.size - 1
        self.n_edges = ix.size
        self.device_buffer = None

    @property
    def handle(self):
        return self._h

    def info(self) -> dict:
        i = capi.ga_plan_info()
        graph_attn_plan_get_info(self._h, byref(i))
        return i.as_dict()

    def array(self, name: str) -> np.ndarray:
        """Copy of one of the plan's host arrays (see graph_attn_plan_array)."""
        p = POINTER(c_int32)()
        n = c_int64()
        graph_attn_plan_array(self._h, name.encode(), byref(p), byref(n))
        if n.value == 0:
            return np.zeros(0, np.int32)
        return np.ctypeslib.as_array(p, shape=(n.value,)).copy()

    def device_bytes(self) -> int:
        b = c_size_t()
        graph_attn_plan_device_bytes(self._h, byref(b))
        return int(b.value)

    def upload(self, device="cuda", stream=None):
        import torch
        nbytes = self.device_bytes()
        buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        with torch.cuda.device(buf.device):
            graph_attn_plan_upload(self._h, c_void_p(buf.data_ptr()), nbytes, _stream(stream))
        self.device_buffer = buf
        return self

    def fwd_workspace_bytes(self, heads: int, dim: int) -> int:
        b = c_size_t()
        graph_attn_fwd_workspace_bytes(self._h, heads, dim, byref(b))
        return int(b.value)

    def bwd_workspace_bytes(self, heads: int, dim: int) -> int:
        b = c_size_t()
        graph_attn_bwd_workspace_bytes(self._h, heads, dim, byref(b))
        return int(b.value)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            try:
                graph_attn_plan_destroy(h)
            except Exception:
                pass
            self._h = None


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return GA_F32
    if t.dtype == torch.bfloat16:
        return GA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _ptr(t):
    return c_void_p(t.data_ptr()) if t is not None else None


def _need(t, name, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must live on {device}")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {tuple(shape)} {dtype}, got "
                         f"{tuple(t.shape)} {t.dtype} contiguous={t.is_contiguous()}")


def _rows_match(plan, n_rows):
    """Feature tensors must have one row per node: the kernels index them by node id."""
    if n_rows != plan.n_nodes:
        raise ValueError(f"tensors have {n_rows} rows, the plan's graph {plan.n_nodes} nodes")


def _workspace(nbytes, device, ws):
    import torch
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def _fwd_args(plan, q_or_s, k_or_t, v, score, scale, out, lse):
    """Checked forward arguments: (score code, scale, out, lse, N, H, d, device)."""
    import torch
    if plan.device_buffer is None:
        raise RuntimeError("plan is not uploaded")
    N, H, d = v.shape
    dev = v.device
    _rows_match(plan, N)
    sc = GA_SCORE_DOT if score == "dot" else GA_SCORE_GAT if score == "gat" else None
    if sc is None:
        raise ValueError(score)
    if sc == GA_SCORE_DOT:
        _need(q_or_s, "q", (N, H, d), v.dtype, dev)
        _need(k_or_t, "k", (N, H, d), v.dtype, dev)
        scale = 1.0 / math.sqrt(d) if scale is None else scale
    else:
        _need(q_or_s, "s", (N, H), torch.float32, dev)
        _need(k_or_t, "t", (N, H), torch.float32, dev)
        scale = 1.0 if scale is None else scale
    _need(v, "v", (N, H, d), v.dtype, dev)
    out = torch.empty_like(v) if out is None else out
    lse = torch.empty((N, H), dtype=torch.float32, device=dev) if lse is None else lse
    _need(out, "out", (N, H, d), v.dtype, dev)
    _need(lse, "lse", (N, H), torch.float32, dev)
    return sc, scale, out, lse, N, H, d, dev


def fwd(plan: Plan, q_or_s, k_or_t, v, *, score="dot", scale=None, neg_slope=0.2, out=None,
        lse=None, workspace=None, stream=None):
    """Forward of the fused layer; returns (out [N,H,d], lse [N,H] fp32).

    dot: q, k, v [N,H,d] (fp32 or bf16), scale defaults to 1/sqrt(d).
    gat: s, t fp32 [N,H], v [N,H,d], scale defaults to 1, neg_slope to 0.2.
    """
    import torch
    sc, scale, out, lse, N, H, d, dev = _fwd_args(plan, q_or_s, k_or_t, v, score, scale, out,
                                                  lse)
    ws, wsb = _workspace(plan.fwd_workspace_bytes(H, d), dev, workspace)
    with torch.cuda.device(dev):
        graph_attn_fwd(plan.handle, sc, _dtype_code(v), H, d, float(scale), float(neg_slope),
                       _ptr(q_or_s), _ptr(k_or_t), _ptr(v), _ptr(out), _ptr(lse), _ptr(ws),
                       wsb, _stream(stream))
    return out, lse


def fwd_noalloc(plan: Plan, q_or_s, k_or_t, v, *, score="dot", scale=None, neg_slope=0.2,
                out=None, lse=None, stream=None):
    """The forward of ``fwd`` through graph_attn_fwd_noalloc: the library takes the hub
    partials from its fixed per-GPU scratch (GA_FWD_NOALLOC_SCRATCH_BYTES) instead of a
    workspace. Pass ``out`` and ``lse`` to allocate nothing at all. Calls that may overlap
    on one GPU share that scratch and must not run concurrently."""
    import torch
    sc, scale, out, lse, N, H, d, dev = _fwd_args(plan, q_or_s, k_or_t, v, score, scale, out,
                                                  lse)
    with torch.cuda.device(dev):
        graph_attn_fwd_noalloc(plan.handle, sc, _dtype_code(v), H, d, float(scale),
                               float(neg_slope), _ptr(q_or_s), _ptr(k_or_t), _ptr(v), _ptr(out),
                               _ptr(lse), _stream(stream))
    return out, lse


def fwd_gatv2(plan: Plan, xd, xs, attn, *, scale=1.0, neg_slope=0.2, out=None, lse=None,
              workspace=None, stream=None):
    """GATv2 forward: e = scale * attn . LeakyReLU(xd_i + xs_j), message xs_j.
    xd, xs [N,H,d] (fp32 or bf16), attn fp32 [H,d]; returns (out [N,H,d], lse [N,H])."""
    import torch
    if plan.device_buffer is None:
        raise RuntimeError("plan is not uploaded")
    N, H, d = xs.shape
    dev = xs.device
    _rows_match(plan, N)
    _need(xd, "xd", (N, H, d), xs.dtype, dev)
    _need(xs, "xs", (N, H, d), xs.dtype, dev)
    _need(attn, "attn", (H, d), torch.float32, dev)
    out = torch.empty_like(xs) if out is None else out
    lse = torch.empty((N, H), dtype=torch.float32, device=dev) if lse is None else lse
    _need(out, "out", (N, H, d), xs.dtype, dev)
    _need(lse, "lse", (N, H), torch.float32, dev)
    ws, wsb = _workspace(plan.fwd_workspace_bytes(H, d), dev, workspace)
    with torch.cuda.device(dev):
        graph_attn_fwd_gatv2(plan.handle, _dtype_code(xs), H, d, float(scale), float(neg_slope),
                             _ptr(xd), _ptr(xs), _ptr(attn), _ptr(out), _ptr(lse), _ptr(ws), wsb,
                             _stream(stream))
    return out, lse


def bwd(plan: Plan, q_or_s, k_or_t, v, dout, lse, *, score="dot", scale=None, neg_slope=0.2,
        dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Backward from the forward's lse.

    dot: returns (dq, dk, dv), each [N,H,d] like q; scale defaults to 1/sqrt(d).
    gat: q_or_s = s, k_or_t = t (fp32 [N,H]); returns (ds, dt fp32 [N,H], dv [N,H,d]);
    scale defaults to 1 and neg_slope to 0.2 (use the forward's values).
    """
    import torch
    if plan.device_buffer is None:
        raise RuntimeError("plan is not uploaded")
    N, H, d = v.shape
    dev = v.device
    _rows_match(plan, N)
    sc = GA_SCORE_DOT if score == "dot" else GA_SCORE_GAT if score == "gat" else None
    if sc is None:
        raise ValueError(score)
    for name, t in (("v", v), ("dout", dout)):
        _need(t, name, (N, H, d), v.dtype, dev)
    if sc == GA_SCORE_DOT:
        _need(q_or_s, "q", (N, H, d), v.dtype, dev)
        _need(k_or_t, "k", (N, H, d), v.dtype, dev)
        dq = torch.empty_like(q_or_s) if dq is None else dq
        dk = torch.empty_like(k_or_t) if dk is None else dk
        scale = 1.0 / math.sqrt(d) if scale is None else scale
    else:
        _need(q_or_s, "s", (N, H), torch.float32, dev)
        _need(k_or_t, "t", (N, H), torch.float32, dev)
        dq = torch.empty((N, H), dtype=torch.float32, device=dev) if dq is None else dq
        dk = torch.empty((N, H), dtype=torch.float32, device=dev) if dk is None else dk
        scale = 1.0 if scale is None else scale
    _need(lse, "lse", (N, H), torch.float32, dev)
    dv = torch.empty_like(v) if dv is None else dv
    ws, wsb = _workspace(plan.bwd_workspace_bytes(H, d), dev, workspace)
    with torch.cuda.device(dev):
        graph_attn_bwd(plan.handle, sc, _dtype_code(v), H, d, float(scale), float(neg_slope),
                       _ptr(q_or_s), _ptr(k_or_t), _ptr(v), _ptr(dout), _ptr(lse), _ptr(dq),
                       _ptr(dk), _ptr(dv), _ptr(ws), wsb, _stream(stream))
    return dq, dk, dv


def bwd_gatv2_workspace_bytes(plan: Plan, dtype, heads: int, dim: int) -> int:
    b = c_size_t()
    graph_attn_bwd_gatv2_workspace_bytes(plan.handle, _dtype_code_of(dtype), heads, dim, byref(b))
    return int(b.value)


def _dtype_code_of(dtype) -> int:
    import torch
    return GA_F32 if dtype == torch.float32 else GA_BF16 if dtype == torch.bfloat16 else -1


def bwd_gatv2(plan: Plan, xd, xs, attn, dout, lse, *, scale=1.0, neg_slope=0.2, dxd=None,
              dxs=None, dattn=None, workspace=None, stream=None):
    """GATv2 backward from the forward's lse; returns (dxd, dxs [N,H,d], dattn fp32 [H,d])."""
    import torch
    if plan.device_buffer is None:
        raise RuntimeError("plan is not uploaded")
    N, H, d = xs.shape
    dev = xs.device
    _rows_match(plan, N)
    for name, t in (("xd", xd), ("xs", xs), ("dout", dout)):
        _need(t, name, (N, H, d), xs.dtype, dev)
    _need(attn, "attn", (H, d), torch.float32, dev)
    _need(lse, "lse", (N, H), torch.float32, dev)
    dxd = torch.empty_like(xd) if dxd is None else dxd
    dxs = torch.empty_like(xs) if dxs is None else dxs
    dattn = torch.empty((H, d), dtype=torch.float32, device=dev) if dattn is None else dattn
    b = c_size_t()
    graph_attn_bwd_gatv2_workspace_bytes(plan.handle, _dtype_code(xs), H, d, byref(b))
    ws, wsb = _workspace(int(b.value), dev, workspace)
    with torch.cuda.device(dev):
        graph_attn_bwd_gatv2(plan.handle, _dtype_code(xs), H, d, float(scale), float(neg_slope),
                             _ptr(xd), _ptr(xs), _ptr(attn), _ptr(dout), _ptr(lse), _ptr(dxd),
                             _ptr(dxs), _ptr(dattn), _ptr(ws), wsb, _stream(stream))
    return dxd, dxs, dattn


def _autograd_fn():
    import torch

    class _GraphAttention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, plan, scale, score, neg_slope):
            out, lse = fwd(plan, q.contiguous(), k.contiguous(), v.contiguous(), score=score,
                           scale=scale, neg_slope=neg_slope)
            ctx.save_for_backward(q, k, v, lse)
            ctx.plan, ctx.scale, ctx.score, ctx.neg_slope = plan, scale, score, neg_slope
            return out

        @staticmethod
        def backward(ctx, g):
            q, k, v, lse = ctx.saved_tensors
            dq, dk, dv = bwd(ctx.plan, q.contiguous(), k.contiguous(), v.contiguous(),
                             g.contiguous(), lse, score=ctx.score, scale=ctx.scale,
                             neg_slope=ctx.neg_slope)
            return dq, dk, dv, None, None, None, None

    class _GraphAttentionV2(torch.autograd.Function):
        @staticmethod
        def forward(ctx, xd, xs, attn, plan, scale, neg_slope):
            out, lse = fwd_gatv2(plan, xd.contiguous(), xs.contiguous(), attn.contiguous(),
                                 scale=scale, neg_slope=neg_slope)
            ctx.save_for_backward(xd, xs, attn, lse)
            ctx.plan, ctx.scale, ctx.neg_slope = plan, scale, neg_slope
            return out

        @staticmethod
        def backward(ctx, g):
            xd, xs, attn, lse = ctx.saved_tensors
            dxd, dxs, dattn = bwd_gatv2(ctx.plan, xd.contiguous(), xs.contiguous(),
                                        attn.contiguous(), g.contiguous(), lse, scale=ctx.scale,
                                        neg_slope=ctx.neg_slope)
            return dxd, dxs, dattn, None, None, None

    return _GraphAttention, _GraphAttentionV2


_FN = None


def graph_attention(plan: Plan, q, k, v, scale=None, *, score="dot", neg_slope=0.2):
    """Graph attention as a differentiable torch op (forward saves lse; backward recomputes
    the weights). score "dot": q, k, v [N,H,d]; "gat": q = s, k = t (fp32 [N,H]) and
    v [N,H,d], with the LeakyReLU slope neg_slope (scale defaults to 1 there)."""
    global _FN
    if _FN is None:
        _FN = _autograd_fn()
    return _FN[0].apply(q, k, v, plan, scale, score, neg_slope)


def graph_attention_gatv2(plan: Plan, xd, xs, attn, scale=1.0, *, neg_slope=0.2):
    """GATv2 attention as a differentiable torch op: xd, xs [N,H,d] (destination and source
    projections; xs is also the message), attn fp32 [H,d]; returns out [N,H,d]."""
    global _FN
    if _FN is None:
        _FN = _autograd_fn()
    return _FN[1].apply(xd, xs, attn, plan, scale, neg_slope)


def _features_view(t, name, device=None):
    """[N, ...] contiguous tensor -> (N, F)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or (device is not None and t.device != device):
        raise ValueError(f"{name} must live on {device or 'a GPU'}")
    if not t.is_contiguous() or t.dim() < 1:
        raise ValueError(f"{name} must be a contiguous [N, ...] tensor")
    return t.shape[0], (t.numel() // t.shape[0] if t.shape[0] else int(np.prod(t.shape[1:])))


def reduce_slot_dtype(plan: Plan):
    """torch dtype holding the plan's slot values (int16 storage of unsigned 16-bit
    positions, or int32)."""
    import torch
    b = c_size_t()
    graph_attn_reduce_slot_bytes(plan.handle, byref(b))
    return torch.int16 if b.value == 2 else torch.int32


def reduce_fwd(plan: Plan, x, *, op="max", out=None, arg=None, slot=None, with_slot=True,
               workspace=None, stream=None):
    """Neighbourhood max (or min) of the source rows, elementwise, and the winning source
    id per element (smallest id on ties; empty rows give 0 and -1).  x: [N, ...] fp32 or
    bf16.  Returns (out like x, arg int32 of x's shape, slot): slot holds each winner's
    position within its row (reduce_slot_dtype; the backward's compact input), None when
    ``with_slot`` is false."""
    import torch
    if plan.device_buffer is None:
        raise RuntimeError("plan is not uploaded")
    code = {"max": GA_REDUCE_MAX, "min": GA_REDUCE_MIN}.get(op)
    if code is None:
        raise ValueError(op)
    N, F = _features_view(x, "x")
    if N != plan.n_nodes:
        raise ValueError(f"x has {N} rows, the graph {plan.n_nodes} nodes")
    out = torch.empty_like(x) if out is None else out
    arg = torch.empty(x.shape, dtype=torch.int32, device=x.device) if arg is None else arg
    _need(out, "out", x.shape, x.dtype, x.device)
    _need(arg, "arg", x.shape, torch.int32, x.device)
    if with_slot:
        sdt = reduce_slot_dtype(plan)
        slot = torch.empty(x.shape, dtype=sdt, device=x.device) if slot is None else slot
        _need(slot, "slot", x.shape, sdt, x.device)
    else:
        slot = None
    b = c_size_t()
    graph_attn_reduce_fwd_workspace_bytes(plan.handle, F, byref(b))
    ws, wsb = _workspace(int(b.value), x.device, workspace)
    with torch.cuda.device(x.device):
        graph_attn_reduce_fwd(plan.handle, code, _dtype_code(x), F, _ptr(x), _ptr(out),
                              _ptr(arg), _ptr(slot), _ptr(ws), wsb, _stream(stream))
    return out, arg, slot


def reduce_bwd(plan: Plan, arg, dout, *, slot=None, dx=None, workspace=None, stream=None):
    """Gradient of reduce_fwd: dx[j] collects dout[i] where arg[i] == j (each destination
    once).  With the forward's ``slot`` the kernels read it instead of arg (half the
    bytes; arg may then be None).  The plan needs the transpose (build_csc=True)."""
    import torch
    if plan.device_buffer is None:
        raise RuntimeError("plan is not uploaded")
    N, F = _features_view(dout, "dout")
    if N != plan.n_nodes:
        raise ValueError(f"dout has {N} rows, the graph {plan.n_nodes} nodes")
    if slot is not None:
        _need(slot, "slot", dout.shape, reduce_slot_dtype(plan), dout.device)
    else:
        _need(arg, "arg", dout.shape, torch.int32, dout.device)
    dx = torch.empty_like(dout) if dx is None else dx
    _need(dx, "dx", dout.shape, dout.dtype, dout.device)
    b = c_size_t()
    graph_attn_reduce_bwd_workspace_bytes(plan.handle, F, byref(b))
    ws, wsb = _workspace(int(b.value), dout.device, workspace)
    with torch.cuda.device(dout.device):
        graph_attn_reduce_bwd(plan.handle, _dtype_code(dout), F,
                              _ptr(arg) if slot is None else None, _ptr(slot), _ptr(dout),
                              _ptr(dx), _ptr(ws), wsb, _stream(stream))
    return dx


def _reduce_fn():
    import torch

    class _GraphReduce(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, plan, op):
            out, arg, slot = reduce_fwd(plan, x.contiguous(), op=op)
            ctx.save_for_backward(slot)
            ctx.plan = plan
            ctx.mark_non_differentiable(arg)
            return out, arg

        @staticmethod
        def backward(ctx, g, _garg):
            (slot,) = ctx.saved_tensors
            return reduce_bwd(ctx.plan, None, g.contiguous(), slot=slot), None, None

    return _GraphReduce


_RFN = None


def graph_reduce(plan: Plan, x, op="max"):
    """Neighbourhood max / min pooling as a differentiable torch op; returns (out, arg)
    (the backward uses the forward's slot array, kept for it)."""
    global _RFN
    if _RFN is None:
        _RFN = _reduce_fn()
    return _RFN.apply(x, plan, op)


def copy_probe(dst, src, stream=None):
    import torch
    nbytes = src.numel() * src.element_size()
    with torch.cuda.device(src.device):
        graph_attn_copy_probe(_ptr(dst), _ptr(src), nbytes, _stream(stream))


def _probe_rows(x, name, N, H, d, dtype, device):
    if x is not None:
        _need(x, name, (N, H, d), dtype, device)
    return _ptr(x)


def gather_probe(plan: Plan, k, v=None, *, row_a=None, row_b=None, sink=None, stream=None):
    """Loads of the forward's (or the dQ pass's) work list without the arithmetic (see
    graph_attn_gather_probe): per work item row_a[i], row_b[i]; per edge k[j] and v[j] (v
    None: one row per edge). Returns the sink tensor."""
    import torch
    N, H, d = k.shape
    _rows_match(plan, N)
    if sink is None:
        sink = torch.zeros(1024, dtype=torch.uint8, device=k.device)
    ptrs = [_probe_rows(x, n, N, H, d, k.dtype, k.device)
            for x, n in ((row_a, "row_a"), (row_b, "row_b"), (k, "k"), (v, "v"))]
    with torch.cuda.device(k.device):
        graph_attn_gather_probe(plan.handle, _dtype_code(k), H, d, *ptrs, _ptr(sink),
                                _stream(stream))
    return sink


def gather_probe_cols(plan: Plan, dout, *, q=None, record=None, k=None, v=None, sink=None,
                      stream=None):
    """Loads of the dK/dV pass's work list over the transpose without the arithmetic (see
    graph_attn_gather_probe_cols): per column k[j], v[j]; per transpose edge dout[i], q[i]
    and record[i] (fp32 [N, H, 2]). Returns the sink tensor."""
    import torch
    N, H, d = dout.shape
    _rows_match(plan, N)
    if record is not None:
        _need(record, "record", (N, H, 2), torch.float32, dout.device)
    if sink is None:
        sink = torch.zeros(1024, dtype=torch.uint8, device=dout.device)
    ptrs = [_probe_rows(x, n, N, H, d, dout.dtype, dout.device)
            for x, n in ((k, "k"), (v, "v"), (q, "q"), (dout, "dout"))]
    with torch.cuda.device(dout.device):
        graph_attn_gather_probe_cols(plan.handle, _dtype_code(dout), H, d, *ptrs, _ptr(record),
                                     _ptr(sink), _stream(stream))
    return sink


def gather_probe_random(table, row_bytes, n_gathers, *, table_rows=None, seed=1, sink=None,
                        stream=None):
    """n_gathers uniformly random rows of row_bytes bytes from the first table_rows rows
    of ``table`` (a device tensor; default: all of it) (graph_attn_gather_probe_random).
    Returns the sink tensor."""
    import torch
    nbytes = table.numel() * table.element_size()
    rows = nbytes // row_bytes if table_rows is None else int(table_rows)
    if not table.is_cuda or not table.is_contiguous() or rows * row_bytes > nbytes:
        raise ValueError("table: a contiguous device tensor of at least table_rows rows")
    if sink is None:
        sink = torch.zeros(1024, dtype=torch.uint8, device=table.device)
    with torch.cuda.device(table.device):
        graph_attn_gather_probe_random(int(row_bytes), _ptr(table), rows, int(n_gathers),
                                       int(seed), _ptr(sink), _stream(stream))
    return sink


def timers(enable=None, reset=False) -> dict:
    """Per-kernel {name: (launches, total_ms)} from the library's event timers.
    ``enable`` switches recording, ``reset`` clears the records (after reading)."""
    if enable is not None:
        graph_attn_timer_enable(1 if enable else 0)
    n = graph_attn_timer_count()
    res = {}
    for i in range(n):
        name = ctypes.c_char_p()
        launches = c_int64()
        ms = ctypes.c_double()
        graph_attn_timer_read(i, byref(name), byref(launches), byref(ms))
        res[name.value.decode()] = (int(launches.value), float(ms.value))
    if reset:
        graph_attn_timer_reset()
    return res

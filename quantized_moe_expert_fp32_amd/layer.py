"""Device-resident MoE layers and the per-step call sequence over the C ABI.

torch allocates device memory and supplies the stream; every step of the layer
(routing, dispatch, expert GEMV/GEMM, combine, RMSNorm) is a call into
libmoe.so. Host arrays come in the canonical storage format documented in
include/moe.h.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import moe

DECODE_MAX_T = 16


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy array -> contiguous device tensor with the same bytes (uint16 -> int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def bits_to_numpy(t: torch.Tensor) -> np.ndarray:
    """int16 device tensor of bf16 bits -> numpy uint16."""
    return t.cpu().numpy().view(np.uint16)


def make_shape(s) -> moe.Shape:
    """moe.Shape from any object with hidden/inter/n_experts/top_k/has_shared/router_fmt
    (and optionally bits: 4 or 8)."""
    return moe.Shape.make(s.hidden, s.inter, s.n_experts, s.top_k, s.has_shared, s.router_fmt,
                          bits=getattr(s, "bits", 4))


class DeviceLayer:
    """One layer's packed expert buffer, packed router and optional logit bias on the GPU;
    with prefill=True (the default) also the prefill layout of the experts that
    moe_experts_prefill reads (experts_prefill, as many bytes again), with fp8=True
    the experts upcast for the FP8 prompt route (experts_fp8)."""

    def __init__(self, shape: moe.Shape, host_layer, device="cuda", fp8: bool = False, prefill: bool = True):
        self.shape = shape
        self.device = device
        nb = moe.moe_experts_packed_bytes(shape)
        if nb == 0:
            raise moe.MoeError(moe.moe_shape_check(shape), "moe_experts_packed_bytes")
        self.experts = torch.empty(nb, dtype=torch.uint8, device=device)
        src = {n: to_device(getattr(host_layer, n), device) for n in
               ("q_gate", "s_gate", "b_gate", "q_up", "s_up", "b_up", "q_down", "s_down", "b_down")}
        moe.moe_pack_experts(shape, src, self.experts)
        self.experts_prefill = None
        if prefill:
            self.experts_prefill = torch.empty(nb, dtype=torch.uint8, device=device)
            moe.moe_pack_experts_prefill(shape, self.experts, self.experts_prefill)
        self.experts_fp8 = None
        if fp8:
            self.experts_fp8 = torch.empty(moe.moe_experts_fp8_bytes(shape), dtype=torch.uint8, device=device)
            moe.moe_pack_experts_fp8(shape, src, self.experts_fp8)
        self.router = torch.empty(moe.moe_router_packed_bytes(shape), dtype=torch.uint8, device=device)
        if shape.router_fmt == moe.ROUTER_F32:
            moe.moe_pack_router(shape, to_device(host_layer.router_f32, device), None, None, self.router)
        else:
            moe.moe_pack_router(shape, to_device(host_layer.router_q, device), to_device(host_layer.router_s, device),
                                to_device(host_layer.router_b, device), self.router)
        lb = getattr(host_layer, "logit_bias", None)
        self.logit_bias = None if lb is None else to_device(lb.astype(np.float32), device)
        torch.cuda.current_stream().synchronize()  # canonical copies may be freed after this
        del src


@dataclass
class StepBuffers:
    T: int
    logits: torch.Tensor
    ids: torch.Tensor
    w: torch.Tensor
    wsh: Optional[torch.Tensor]
    ws: torch.Tensor
    y: torch.Tensor
    out: torch.Tensor


def alloc_buffers(shape: moe.Shape, T: int, path: str, device="cuda") -> StepBuffers:
    R = shape.n_experts + shape.has_shared
    S = shape.slots
    ws_bytes = (moe.moe_decode_workspace_bytes(shape, T) if path in ("decode", "fused")
                else moe.moe_prefill_fp8_workspace_bytes(shape, T) if path == "fp8"
                else moe.moe_prefill_workspace_bytes(shape, T))
    return StepBuffers(
        T=T,
        logits=torch.empty((T, R), dtype=torch.float32, device=device),
        ids=torch.empty((T, shape.top_k), dtype=torch.int32, device=device),
        w=torch.empty((T, shape.top_k), dtype=torch.int16, device=device),
        wsh=torch.empty((T,), dtype=torch.int16, device=device) if shape.has_shared else None,
        ws=torch.zeros(ws_bytes, dtype=torch.uint8, device=device),
        y=torch.empty((T, S, shape.hidden), dtype=torch.float32, device=device),
        out=torch.empty((T, shape.hidden), dtype=torch.int16, device=device),
    )


def pick_path(T: int) -> str:
    return "fused" if T <= DECODE_MAX_T else "prefill"


def layer_step(layer: DeviceLayer, x: torch.Tensor, buf: StepBuffers, path: Optional[str] = None,
               residual: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None, stream=None):
    """One layer on one stream. path "fused" (T <= 16): moe_decode_layer (one launch);
    "decode" / "prefill" / "fp8": moe_route, then moe_experts_decode, moe_experts_prefill
    or moe_experts_prefill_fp8 (the FP8 route; needs a layer built with fp8=True),
    then moe_combine."""
    sh, T = layer.shape, buf.T
    path = path or pick_path(T)
    dst = buf.out if out is None else out
    if path == "fused":
        moe.moe_decode_layer(sh, layer.router, layer.logit_bias, layer.experts, x, T, buf.ws, buf.logits, buf.ids,
                             buf.w, buf.wsh, buf.y, residual, dst, stream)
        return dst
    moe.moe_route(sh, layer.router, layer.logit_bias, x, T, buf.logits, buf.ids, buf.w, buf.wsh, stream)
    if path == "decode":
        moe.moe_experts_decode(sh, layer.experts, x, T, buf.ids, buf.ws, buf.y, stream)
    elif path == "fp8":
        if layer.experts_fp8 is None:
            raise ValueError("the FP8 route needs a DeviceLayer built with fp8=True")
        moe.moe_experts_prefill_fp8(sh, layer.experts_fp8, x, T, buf.ids, buf.ws, buf.y, stream)
    else:
        if layer.experts_prefill is None:
            raise ValueError("the prefill path needs a DeviceLayer built with prefill=True")
        moe.moe_experts_prefill(sh, layer.experts_prefill, x, T, buf.ids, buf.ws, buf.y, stream)
    moe.moe_combine(sh, buf.y, buf.w, buf.wsh, T, residual, dst, stream)
    return dst


def stack_step(layers, x: torch.Tensor, xn: torch.Tensor, buf: StepBuffers, eps: float = 1e-6,
               path: Optional[str] = None, stream=None, keep: Optional[list] = None):
    """x <- bf16(x + MoE(bf16(RMSNorm(x)))) for every layer, in place on x. With
    `keep`, a copy of every layer's output state, normalised input and picks is
    appended to it as (x, xn, ids) (device copies, made on the stream; under graph capture they live in
    the graph's memory and hold the last replay's values)."""
    sh = layers[0].shape
    for L in layers:
        moe.moe_rmsnorm(sh.hidden, x, buf.T, eps, xn, stream)
        layer_step(L, xn, buf, path, residual=x, out=x, stream=stream)
        if keep is not None:
            keep.append((x.clone(), xn.clone(), buf.ids.clone()))
    return x


def stack_step_fused(layers, x: torch.Tensor, x_other: torch.Tensor, buf: StepBuffers, eps: float = 1e-6,
                     stream=None, keep: Optional[list] = None) -> torch.Tensor:
    """The same stack step as stack_step for T <= 16, one launch per layer: each layer
    is moe_decode_block (RMSNorm, the layer and the residual add), reading one state
    buffer and writing the other. Returns the buffer that holds the final state (x
    after an even number of layers). With `keep`, (state, ids) copies per layer."""
    sh = layers[0].shape
    cur, nxt = x, x_other
    for L in layers:
        moe.moe_decode_block(sh, L.router, L.logit_bias, L.experts, cur, buf.T, eps, buf.ws, buf.logits, buf.ids, buf.w,
                             buf.wsh, buf.y, nxt, stream)
        if keep is not None:
            keep.append((nxt.clone(), buf.ids.clone()))
        cur, nxt = nxt, cur
    return cur


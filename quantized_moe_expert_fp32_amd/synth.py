"""Seeded synthetic inputs for the routed int4 MoE layer.

This module only draws random numbers and stores them in the layer's
storage formats. It contains none of the layer's arithmetic (no routing,
no dequantisation, no expert math, no combine): both the CPU oracle and the
HIP path consume what it returns, and neither depends on the other.

Workloads (the shapes of the Qwen3.6-35B-A3B routed-expert block: 256 experts,
8 picked per token plus one shared expert, hidden 2048, expert intermediate 512,
affine 4-bit experts in groups of 64 and 8-bit routers; TensorFold issue #931,
"What it is" and "What I'd build"; R9700 blog part 13, model facts list):

  tiny          T=4,    H=256,  E=16,  k=2, I=64,  fp32 router,          seed 0
  decode        T=1,    H=2048, E=256, k=8, I=512, 8-bit affine router,  seed 1
  prefill512    T=512,  same layer,                                      seed 2
  prefill4096   T=4096, same layer, Zipf(s=1.1) per-expert logit bias,   seed 3
  stack         40 independent layers of the same shape, T=1 or T=16,    seed 4

Storage formats (the "canonical" layout every consumer reads):
  * bf16 values are uint16 bit patterns.
  * int4 matrix [rows, cols]: uint8 [rows, cols/2], element 2j in the low
    nibble of byte j, element 2j+1 in the high nibble. Values q in 0..15.
    scale and bias are bf16 [rows, cols/64]; the weight is scale*q + bias.
  * int8 expert matrix [rows, cols] (8-bit experts): uint8 [rows, cols], q in
    0..255, scale and bias as above.
  * int8 router [E+1, H]: uint8 q in 0..255, scale and bias bf16 [E+1, H/64].
  * fp32 router [E+1, H]: float32.
  * Experts are stacked [E+1, ...]; index E is the shared expert. Router row E
    is the shared-expert gate.

Draw order for one layer, rng = numpy.random.default_rng([seed, 1000 + layer]):
  1. router fp32 N(0, 0.02), shape [E+1, H]
  2. (Zipf workload only) r = rng.permutation(E) + 1; bias_e = -1.1 * ln(r_e)
  3. for each of gate [E+1, I, H], up [E+1, I, H], down [E+1, H, I]:
       packed nibbles  rng.integers(0, 256, rows*cols/2, uint8)
       scale           rng.uniform(0.002, 0.02, rows*cols/64) -> fp32 -> bf16
       bias            -8 * scale (exact in bf16)
     (8-bit experts, shape.bits == 8: codes rng.integers(0, 256, rows*cols, uint8),
     scale rng.uniform(0.002, 0.02, rows*cols/64) / 16 -> fp32 -> bf16, bias
     -128 * scale: the same weight range as the 4-bit matrices)
Activations: numpy.random.default_rng([seed, 1]).standard_normal((T, H)) -> fp32 -> bf16.

bf16 values are produced from fp32 draws by torch's round-to-nearest-even cast
(a library conversion).
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

ROUTER_F32 = 0
ROUTER_AFFINE8 = 1

GROUP = 64


def _to_bf16_bits(a32: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns via torch's round-to-nearest-even cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Shape:
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    has_shared: int = 1
    router_fmt: int = ROUTER_AFFINE8
    group: int = GROUP
    bits: int = 4

    @property
    def slots(self) -> int:
        return self.top_k + (1 if self.has_shared else 0)

    @property
    def n_mats(self) -> int:
        """Expert weight sets stored: E routed plus the shared one."""
        return self.n_experts + (1 if self.has_shared else 0)

    @property
    def router_rows(self) -> int:
        return self.n_experts + (1 if self.has_shared else 0)


@dataclass
class Layer:
    shape: Shape
    router_f32: Optional[np.ndarray] = None  # [R, H] float32 (fp32 router)
    router_q: Optional[np.ndarray] = None  # [R, H] uint8 (8-bit router)
    router_s: Optional[np.ndarray] = None  # [R, H/64] bf16 bits
    router_b: Optional[np.ndarray] = None  # [R, H/64] bf16 bits
    logit_bias: Optional[np.ndarray] = None  # [E] float32 or None
    q_gate: np.ndarray = None  # [M, I, H/2] uint8
    s_gate: np.ndarray = None  # [M, I, H/64] bf16 bits
    b_gate: np.ndarray = None
    q_up: np.ndarray = None
    s_up: np.ndarray = None
    b_up: np.ndarray = None
    q_down: np.ndarray = None  # [M, H, I/2] uint8
    s_down: np.ndarray = None  # [M, H, I/64]
    b_down: np.ndarray = None

    def arrays(self) -> Dict[str, np.ndarray]:
        out = {}
        for k in ("router_f32", "router_q", "router_s", "router_b", "logit_bias",
                  "q_gate", "s_gate", "b_gate", "q_up", "s_up", "b_up",
                  "q_down", "s_down", "b_down"):
            v = getattr(self, k)
            if v is not None:
                out[k] = v
        return out

    def sha256(self) -> Dict[str, str]:
        return {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()
                for k, v in self.arrays().items()}


@dataclass
class Case:
    name: str
    seed: int
    T: int
    shape: Shape
    x: np.ndarray  # [T, H] bf16 bits
    layers: List[Layer] = field(default_factory=list)


WORKLOADS = {
    # name: (T, H, I, E, k, router_fmt, zipf, seed, n_layers)
    "tiny": (4, 256, 64, 16, 2, ROUTER_F32, False, 0, 1),
    "decode": (1, 2048, 512, 256, 8, ROUTER_AFFINE8, False, 1, 1),
    "prefill512": (512, 2048, 512, 256, 8, ROUTER_AFFINE8, False, 2, 1),
    "prefill4096": (4096, 2048, 512, 256, 8, ROUTER_AFFINE8, True, 3, 1),
    "stack": (1, 2048, 512, 256, 8, ROUTER_AFFINE8, False, 4, 40),
}


def quantise_router_affine8(w: np.ndarray):
    """Generator-side encoding of an fp32 router into 8-bit affine groups of 64.

    scale = bf16((max - min) / 255), bias = bf16(min), q = clamp(rint((w - bias) / scale), 0, 255).
    Only (q, scale, bias) define the layer; this is how the synthetic router is drawn.
    """
    R, H = w.shape
    g = w.reshape(R, H // GROUP, GROUP).astype(np.float32)
    mn = g.min(axis=2)
    mx = g.max(axis=2)
    s_bits = _to_bf16_bits((mx - mn) / np.float32(255.0))
    b_bits = _to_bf16_bits(mn)
    s = bf16_bits_to_f32(s_bits)[..., None]
    b = bf16_bits_to_f32(b_bits)[..., None]
    q = np.clip(np.rint((g - b) / s), 0, 255).astype(np.uint8).reshape(R, H)
    return q, s_bits, b_bits


def _int4_matrix(rng: np.random.Generator, n: int, rows: int, cols: int):
    q = rng.integers(0, 256, size=(n, rows, cols // 2), dtype=np.uint8)
    scale32 = rng.uniform(0.002, 0.02, size=(n, rows, cols // GROUP)).astype(np.float32)
    s_bits = _to_bf16_bits(scale32)
    b_bits = _to_bf16_bits(np.float32(-8.0) * bf16_bits_to_f32(s_bits))
    return q, s_bits, b_bits


def _int8_matrix(rng: np.random.Generator, n: int, rows: int, cols: int):
    """8-bit affine codes with the int4 matrices' weight range: q uniform 0..255,
    scale bf16(U(0.002, 0.02) / 16), bias -128 * scale (exact in bf16)."""
    q = rng.integers(0, 256, size=(n, rows, cols), dtype=np.uint8)
    scale32 = (rng.uniform(0.002, 0.02, size=(n, rows, cols // GROUP)) / 16.0).astype(np.float32)
    s_bits = _to_bf16_bits(scale32)
    b_bits = _to_bf16_bits(np.float32(-128.0) * bf16_bits_to_f32(s_bits))
    return q, s_bits, b_bits


def make_layer(shape: Shape, seed: int, layer: int = 0, zipf: bool = False) -> Layer:
    rng = np.random.default_rng([seed, 1000 + layer])
    H, I, E = shape.hidden, shape.inter, shape.n_experts
    R = shape.router_rows
    M = shape.n_mats
    L = Layer(shape=shape)
    w = rng.normal(0.0, 0.02, size=(R, H)).astype(np.float32)
    if shape.router_fmt == ROUTER_F32:
        L.router_f32 = w
    else:
        L.router_q, L.router_s, L.router_b = quantise_router_affine8(w)
    if zipf:
        r = rng.permutation(E) + 1
        L.logit_bias = (-1.1 * np.log(r.astype(np.float64))).astype(np.float32)
    mat = _int8_matrix if shape.bits == 8 else _int4_matrix
    L.q_gate, L.s_gate, L.b_gate = mat(rng, M, I, H)
    L.q_up, L.s_up, L.b_up = mat(rng, M, I, H)
    L.q_down, L.s_down, L.b_down = mat(rng, M, H, I)
    return L


def make_x(seed: int, T: int, H: int) -> np.ndarray:
    rng = np.random.default_rng([seed, 1])
    return _to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))


def workload_shape(name: str, bits: int = 4) -> Shape:
    T, H, I, E, k, rf, zipf, seed, nl = WORKLOADS[name]
    return Shape(hidden=H, inter=I, n_experts=E, top_k=k, has_shared=1, router_fmt=rf, bits=bits)


def make_case(name: str, T: Optional[int] = None, n_layers: Optional[int] = None,
              seed: Optional[int] = None, bits: int = 4) -> Case:
    """Build one named workload. T, n_layers and seed override the defaults; bits = 8
    gives the same workload with 8-bit experts."""
    T0, H, I, E, k, rf, zipf, seed0, nl0 = WORKLOADS[name]
    T = T0 if T is None else T
    seed = seed0 if seed is None else seed
    n_layers = nl0 if n_layers is None else n_layers
    shape = workload_shape(name, bits)
    layers = [make_layer(shape, seed, l, zipf) for l in range(n_layers)]
    return Case(name=name, seed=seed, T=T, shape=shape, x=make_x(seed, T, H), layers=layers)


def random_x(seed: int, T: int, H: int, stream: int = 2) -> np.ndarray:
    """Extra activation draws (independent of make_x) for rotating inputs."""
    rng = np.random.default_rng([seed, stream])
    return _to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))

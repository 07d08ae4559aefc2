"""FP64 CPU oracle for the routed int4 Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the tests, the smoke check of the graft entry point
and the CPU-baseline leg of the benchmark use it. It shares no code with the
HIP library and imports nothing from it.

What it computes follows the routing contract of TensorFold issue #931,
"Qwen3.6-35B-A3B (qwen3_5_moe) on the native Metal engine: proposal and gate",
section "What I'd build":
  * fp32 logits over the routed experts and the shared expert's gate;
  * top-k by logit, ties going to the lower expert id;
  * pick weights exp(l - l_top) over the k picks (normalised over the picks),
    rounded to bf16;
  * the shared expert is one more slot, weighted bf16(sigmoid(bf16(gate)));
  * the weighted sum is rounded once to bf16.
Same section: experts are affine 4-bit in groups of 64, routers 8-bit. Section
"What it is": the routed experts replace the dense MLP (256 experts, 8 picked,
one shared expert). Section "Gate": an FP64 reference per projection class
(router logits, expert gate/up, expert down, combine) on prompt and decode rows;
every stage below is callable on its own so a check can feed it another
implementation's previous-stage output.

Arithmetic: every value is carried in float64; the only roundings are the ones
the contract (or a stated reading) fixes: logits to fp32, pick weights, the
shared weight and its gate to bf16, the SwiGLU intermediate to bf16 (reading),
the combined output to bf16, and (layer stack) the RMSNorm output and the
residual sum to bf16 (reading). Library primitives used as steps: numpy matmul
in float64, numpy.exp, a stable lexicographic sort.

Readings where the pages are silent are listed in the design notes; the ones
that shape this file are repeated at the function that takes them.
"""

from __future__ import annotations

import numpy as np

GROUP = 64


# ---------------------------------------------------------------- number formats

def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_bf16(v) -> np.ndarray:
    """Round float64 values to bf16 with round-to-nearest-even; return bit patterns.

    One rounding, straight from the float64 value (no fp32 step, so no double
    rounding). bf16 has 8 significant bits; normal values have exponents
    -126..127, subnormals are multiples of 2^-133. Values at or beyond
    (2 - 2^-8) * 2^127 become infinity; NaN becomes 0x7FC0.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    with np.errstate(over="ignore", invalid="ignore"):
        _, e = np.frexp(a)  # a = m * 2^e, m in [0.5, 1)
        qexp = np.maximum(e - 8, -133)  # quantum of the bf16 binade holding a
        big = a >= 2.0 ** 128
        n = np.rint(np.ldexp(np.where(big | ~np.isfinite(a), 0.0, a), -qexp))  # half-to-even
        r = np.ldexp(n, qexp)  # exactly a bf16 value, hence exactly an fp32 value
        bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(big | np.isinf(a), np.uint16(0x7F80), bits)
    bits = np.where(np.signbit(v), bits | np.uint16(0x8000), bits)
    bits = np.where(np.isnan(v), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


def round_f32(v) -> np.ndarray:
    """float64 -> fp32 with IEEE round-to-nearest-even (numpy's cast)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32)


# ---------------------------------------------------------------- dequantisation

def dequant_int4(q_packed, scale_bits, bias_bits) -> np.ndarray:
    """Affine 4-bit groups of 64: w = scale * q + bias, exact in float64.

    Storage (TensorFold #931, "What I'd build": MLX affine 4-bit, groups of 64):
    q_packed [..., rows, cols/2] uint8 with element 2j in the low nibble of
    byte j and element 2j+1 in the high nibble; scale and bias are bf16
    [..., rows, cols/64]; group g covers columns 64g..64g+63 of its row.
    """
    q_packed = np.asarray(q_packed, dtype=np.uint8)
    lo = (q_packed & 0x0F).astype(np.float64)
    hi = (q_packed >> 4).astype(np.float64)
    q = np.stack([lo, hi], axis=-1).reshape(*q_packed.shape[:-1], q_packed.shape[-1] * 2)
    s = np.repeat(bf16_to_f64(scale_bits), GROUP, axis=-1)
    b = np.repeat(bf16_to_f64(bias_bits), GROUP, axis=-1)
    return s * q + b


def dequant_int8(q, scale_bits, bias_bits) -> np.ndarray:
    """Affine 8-bit groups of 64 (the router format): w = scale * q + bias."""
    q = np.asarray(q, dtype=np.uint8).astype(np.float64)
    s = np.repeat(bf16_to_f64(scale_bits), GROUP, axis=-1)
    b = np.repeat(bf16_to_f64(bias_bits), GROUP, axis=-1)
    return s * q + b


def dequant_expert(q, scale_bits, bias_bits, bits: int) -> np.ndarray:
    """An expert matrix in its storage format: affine 4-bit (two weights per byte,
    dequant_int4) or affine 8-bit (one weight per byte, dequant_int8), groups of 64.

    TensorFold #931, "What I'd build": experts are affine 4-bit in groups of 64,
    and the 8-bit experts (a second checkpoint of the same layout) store one code
    per byte with the same groups; w = scale * q + bias either way.
    """
    if bits == 4:
        return dequant_int4(q, scale_bits, bias_bits)
    if bits == 8:
        return dequant_int8(q, scale_bits, bias_bits)
    raise ValueError("expert bit width %d" % bits)


def router_matrix(layer) -> np.ndarray:
    """Router [E(+1), H] in float64: fp32 rows, or dequantised 8-bit affine rows."""
    if getattr(layer, "router_f32", None) is not None:
        return np.asarray(layer.router_f32, dtype=np.float32).astype(np.float64)
    return dequant_int8(layer.router_q, layer.router_s, layer.router_b)


# ---------------------------------------------------------------- a1: router logits

def router_logits(x_bits, W, logit_bias=None, n_experts=None) -> np.ndarray:
    """fp32 logits [T, R] = round_fp32(sum_h x[t,h] * W[r,h] (+ bias[r] for r < E)).

    Contract: fp32 logits over the experts and the shared expert's gate. The
    products of bf16 activations and dequantised weights are exact in float64;
    the sum is accumulated in float64 and rounded to fp32 once. The optional
    per-expert logit bias is part of the routed logits only (reading: the shared
    gate is a plain N=1 projection with no bias).
    """
    x = bf16_to_f64(x_bits)
    acc = x @ np.asarray(W, dtype=np.float64).T
    if logit_bias is not None:
        E = len(logit_bias) if n_experts is None else n_experts
        acc[:, :E] = acc[:, :E] + np.asarray(logit_bias, dtype=np.float32).astype(np.float64)
    return round_f32(acc)


# ---------------------------------------------------------------- a2: top-k, weights, shared weight

def topk(logits_routed, k: int) -> np.ndarray:
    """Ids [T, k] of the k largest logits, largest first, ties to the lower id.

    Contract: top-k by logit with ties going to the lower id. IEEE comparison,
    so -0 and +0 tie. NaN logits rank below every number (reading: never picked
    while k non-NaN logits exist).
    """
    l = np.asarray(logits_routed, dtype=np.float32).astype(np.float64)
    T, E = l.shape
    ids = np.broadcast_to(np.arange(E), (T, E))
    nan = np.isnan(l)
    neg = np.where(nan, 0.0, -l)
    out = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        order = np.lexsort((ids[t], neg[t], nan[t]))  # last key is primary
        out[t] = order[:k]
    return out


def pick_weights(logits_routed, ids) -> np.ndarray:
    """bf16 weights [T, k]: w_i = exp(l_i - l_top) / sum_j exp(l_j - l_top) over the k picks.

    Contract: weights exp(l - l_top) over the k picks, rounded to bf16. Reading:
    normalised over the picks (a softmax over the k picked logits), evaluated in
    float64 from the fp32 logits and rounded once to bf16, with no renormalisation
    after rounding. The sum runs over the picks in slot order.
    """
    l = np.asarray(logits_routed, dtype=np.float32)
    T, k = ids.shape
    out = np.empty((T, k), dtype=np.uint16)
    for t in range(T):
        lt = l[t, ids[t]].astype(np.float64)
        e = np.exp(lt - lt[0])
        s = 0.0
        for j in range(k):
            s += e[j]
        out[t] = round_bf16(e / s)
    return out


def sigmoid64(v) -> np.ndarray:
    """1 / (1 + exp(-v)) in float64."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-v))


def shared_weight(gate_logit) -> np.ndarray:
    """bf16(sigmoid(bf16(gate))): the shared expert's slot weight [T].

    Contract: the shared expert is one more slot weighted bf16(sigmoid(bf16(gate))).
    The fp32 gate logit is rounded to bf16, the sigmoid is taken in float64 and
    rounded to bf16.
    """
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen with the invalid flag
        g64 = np.asarray(gate_logit, dtype=np.float32).astype(np.float64)
    g = bf16_to_f64(round_bf16(g64))
    return round_bf16(sigmoid64(g))


# ---------------------------------------------------------------- a3: dispatch

def dispatch(ids, n_experts: int, has_shared: bool):
    """Histogram and expert-sorted order of the picks.

    Returns (counts [E(+1)] int32, offsets [E(+1)+1] int32, order [T*S] int32):
    counts[e] = #{(t, s): ids[t, s] = e}; the shared expert (index E) takes every
    token once. offsets is the exclusive prefix sum. order lists the pick
    indices p = t*S + s grouped by expert (ascending e), and within an expert by
    ascending p. S = k (+1 with the shared slot, whose s is k).
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    S = k + (1 if has_shared else 0)
    nE = n_experts + (1 if has_shared else 0)
    e_of = np.full((T, S), -1, dtype=np.int64)
    e_of[:, :k] = ids
    if has_shared:
        e_of[:, k] = n_experts
    flat = e_of.reshape(-1)
    counts = np.bincount(flat, minlength=nE).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    order = np.argsort(flat, kind="stable").astype(np.int32)
    return counts, offsets, order


# ---------------------------------------------------------------- a4/a5: experts

def silu64(z) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z)) in float64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(x64, q_gate, s_gate, b_gate, q_up, s_up, b_up, q_down, s_down, b_down, bits: int = 4):
    """One expert on rows x64 [n, H]: returns (h bf16 bits [n, I], y float64 [n, H]).

    gate/up pair then down (TensorFold #931, "Gate": "the expert gate/up pair,
    expert down"); SwiGLU: h = silu(x Wg^T) * (x Wu^T). Reading: h is rounded to
    bf16 (the model's activation type) before the down projection; y is kept in
    float64 because the contract rounds only the weighted sum.
    """
    Wg = dequant_expert(q_gate, s_gate, b_gate, bits)
    Wu = dequant_expert(q_up, s_up, b_up, bits)
    Wd = dequant_expert(q_down, s_down, b_down, bits)
    g = x64 @ Wg.T
    u = x64 @ Wu.T
    h = round_bf16(silu64(g) * u)
    y = bf16_to_f64(h) @ Wd.T
    return h, y


def expert_bits(layer) -> int:
    """Bit width of a layer's expert codes, from its storage: 4-bit matrices hold
    two codes per byte along the input dimension ([.., I, H/2] for gate), 8-bit
    one ([.., I, H])."""
    return 8 if layer.q_gate.shape[-1] == layer.q_down.shape[-2] else 4


def expert_outputs(x_bits, ids, layer, n_experts: int, has_shared: bool, fp8: bool = False):
    """Per-slot expert outputs y [T, S, H] (float64) and h [T, S, I] (bf16 bits).

    Slot s < k holds expert ids[t, s]; slot k (when present) the shared expert,
    stored as expert index E. fp8: every expert through the FP8 route
    (fp8_gate_up, fp8_down) instead of expert_ffn.
    """
    x = bf16_to_f64(x_bits)
    ids = np.asarray(ids)
    T, k = ids.shape
    S = k + (1 if has_shared else 0)
    H = x.shape[1]
    I = layer.q_gate.shape[1]
    bits = expert_bits(layer)
    y = np.zeros((T, S, H), dtype=np.float64)
    h = np.zeros((T, S, I), dtype=np.uint16)
    experts = sorted(set(int(e) for e in ids.reshape(-1)))
    if has_shared:
        experts.append(n_experts)
    for e in experts:
        if e == n_experts and has_shared:
            rows_t = np.arange(T)
            rows_s = np.full(T, k)
        else:
            rows_t, rows_s = np.nonzero(ids == e)
        if fp8:
            f8 = fp8_expert(layer, e)
            he = fp8_gate_up(np.asarray(x_bits)[rows_t], f8["gate"], f8["up"])
            ye = fp8_down(he, f8["down"])
        else:
            he, ye = expert_ffn(x[rows_t], layer.q_gate[e], layer.s_gate[e], layer.b_gate[e],
                                layer.q_up[e], layer.s_up[e], layer.b_up[e],
                                layer.q_down[e], layer.s_down[e], layer.b_down[e], bits)
        y[rows_t, rows_s] = ye
        h[rows_t, rows_s] = he
    return y, h


# ---------------------------------------------------------------- a6: combine

def combine(y, w_bits, wsh_bits=None) -> np.ndarray:
    """out[t] = bf16( sum_{s<k} w[t,s] * y[t,s] + wsh[t] * y[t,k] ), one rounding.

    Contract: the shared expert is one more slot; the weighted sum is rounded once
    to bf16. The bf16 weights enter as exact values; the sum is float64.
    """
    y = np.asarray(y, dtype=np.float64)
    w = bf16_to_f64(w_bits)
    k = w.shape[1]
    acc = np.zeros((y.shape[0], y.shape[2]), dtype=np.float64)
    for s in range(k):
        acc += w[:, s:s + 1] * y[:, s]
    if wsh_bits is not None:
        acc += bf16_to_f64(wsh_bits)[:, None] * y[:, k]
    return round_bf16(acc)


# ---------------------------------------------------------------- a7: stack glue (reading)

def rmsnorm_bf16(x_bits, eps: float = 1e-6) -> np.ndarray:
    """Unit-weight RMSNorm: bf16( x / sqrt(mean(x^2) + eps) ) per row, float64 math.

    Reading for the layer stack (the pages give no norm for an MoE-only stack):
    a pre-norm residual block, x <- bf16(x + MoE(bf16(RMSNorm(x)))).
    """
    x = bf16_to_f64(x_bits)
    ms = np.mean(x * x, axis=1, keepdims=True)
    return round_bf16(x / np.sqrt(ms + eps))


def residual_bf16(x_bits, out_bits) -> np.ndarray:
    """bf16(x + out): the residual add between stacked layers."""
    return round_bf16(bf16_to_f64(x_bits) + bf16_to_f64(out_bits))


# ---------------------------------------------------------------- whole layer

def layer_forward(x_bits, layer, top_k: int, has_shared: bool = True, fp8: bool = False):
    """Route -> experts -> combine for one layer; returns every stage's output.
    fp8: the experts take the FP8 route (routing and combine unchanged)."""
    W = router_matrix(layer)
    E = W.shape[0] - (1 if has_shared else 0)
    logits = router_logits(x_bits, W, getattr(layer, "logit_bias", None), E)
    ids = topk(logits[:, :E], top_k)
    w = pick_weights(logits[:, :E], ids)
    wsh = shared_weight(logits[:, E]) if has_shared else None
    y, h = expert_outputs(x_bits, ids, layer, E, has_shared, fp8=fp8)
    out = combine(y, w, wsh)
    return {"logits": logits, "ids": ids, "w": w, "wsh": wsh, "h": h, "y": y, "out": out}


# ---------------------------------------------------------------- FP8 route (prompt experts)
# "R9700: the 35B only one runtime could load" (R9700 vLLM blog, part 13), its
# closing list of kernel work: upcast the experts to FP8 so that the prompt GEMMs
# can run on the FP8 matrix units as well.
# The pages fix neither the FP8 format, the scaling nor the activation side;
# readings:
#   * OCP FP8 E4M3 (4 exponent bits, bias 7, 3 mantissa bits, subnormals, no
#     infinities, largest finite 448), round to nearest even;
#   * every weight row (gate, up, down) is formed as w = fp32(scale * q + bias)
#     (one rounding of the exact value) and stored as E4M3 codes of w * 2^-e with
#     one power-of-two scale 2^e per row, e = floor(log2 max|w|) - 7, so the row's
#     largest magnitude lands in [128, 256) and no code saturates;
#   * the activation rows entering each projection (the bf16 input x for gate/up,
#     the bf16 SwiGLU intermediate h for down) are quantised the same way, one
#     power-of-two scale per row;
#   * a projection is 2^(e_row + e_col) * sum(code products), exact here, rounded
#     nowhere but where the exact route rounds (h to bf16, the combined output).
# The route keeps the exact path's routing, dispatch and combine.

E4M3_BIAS = 7


def e4m3_decode(codes) -> np.ndarray:
    """Values of E4M3 codes (float64): sign bit 7, exponent field E (bits 3..6),
    mantissa m (bits 0..2); (8 + m) 2^(E - 10) for E > 0, m 2^-9 for E = 0 (2^-6 the
    least normal value, m/8 of it below); codes 0x7F and 0xFF are NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    E = (c >> 3) & 15
    m = c & 7
    v = np.where(E > 0, np.ldexp((8 + m).astype(np.float64), E - 3 - E4M3_BIAS), np.ldexp(m.astype(np.float64), -9))
    v = np.where(c & 0x80, -v, v)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def e4m3_encode(v) -> np.ndarray:
    """E4M3 codes of finite values below 256 in magnitude, round to nearest even.

    The quantum of a magnitude a in [2^p, 2^(p+1)) is 2^(p-3) (3 mantissa bits),
    and 2^-9 below the normal range (a < 2^-6); a rounds to the nearest multiple
    of its quantum, ties to the even multiple (numpy.rint). A result of 2^(p+1)
    lands exactly on the next binade's first code, so the code follows from the
    rounded value alone. The route never encodes 256 or more (its scales map every
    row below 256), so saturation at 448 does not arise and is refused.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if not np.isfinite(a).all() or (a >= 256).any():
        raise ValueError("e4m3_encode takes finite magnitudes below 256")
    _, p = np.frexp(a)  # a = f 2^p, f in [0.5, 1): floor(log2 a) = p - 1
    q = np.maximum(p - 1 - 3, -9)
    n = np.rint(np.ldexp(a, -q))
    r = np.ldexp(n, q)  # the rounded magnitude, an E4M3 value
    _, pr = np.frexp(r)
    E = pr - 1 + E4M3_BIAS
    normal = r >= 2.0 ** -6
    mant = np.where(normal, np.ldexp(r, -(pr - 1 - 3)) - 8, 0).astype(np.int64)
    code = np.where(normal, (E.astype(np.int64) << 3) | mant, np.ldexp(r, 9).astype(np.int64))
    code = np.where(np.signbit(v), code | 0x80, code)
    return code.astype(np.uint8)


def fp8_row_exponent(amax) -> np.ndarray:
    """e = floor(log2 amax) - 7 per row (reading above); 0 for an all-zero row."""
    a = np.asarray(amax, dtype=np.float64)
    _, p = np.frexp(a)
    return np.where(a > 0, p - 1 - 7, 0).astype(np.int64)


def fp8_quantise_rows(v):
    """Rows of fp32-representable values -> (E4M3 codes [..., K], exponents [...]).

    Each row's codes encode v * 2^-e (exact: a power-of-two scaling) with its own e.
    """
    v = np.asarray(v, dtype=np.float64)
    e = fp8_row_exponent(np.abs(v).max(axis=-1))
    return e4m3_encode(np.ldexp(v, -e[..., None])), e


def fp8_rows_value(codes, e) -> np.ndarray:
    """The values a quantised row stands for: decode(code) * 2^e."""
    return np.ldexp(e4m3_decode(codes), np.asarray(e)[..., None])


def fp8_weight_rows(q, scale_bits, bias_bits, bits: int):
    """An expert matrix [rows, in] upcast to E4M3 rows: (codes, exponents).

    w = fp32(scale * q + bias): the exact value (scale * q has at most 16
    significant bits) rounded once to fp32, as a fused multiply-add would. The sum
    is checked to be exact in float64 (an error-free two-sum), so that the fp32
    cast is a single rounding.
    """
    zeros = np.zeros_like(np.asarray(scale_bits, dtype=np.uint16))
    sq = dequant_expert(q, scale_bits, zeros, bits)   # scale * q, exact
    b = dequant_expert(q, zeros, bias_bits, bits)     # bias, repeated over each group
    w = sq + b
    bb = w - sq
    err = (sq - (w - bb)) + (b - bb)
    if (err != 0).any():
        raise ValueError("scale * q + bias not exact in float64")
    return fp8_quantise_rows(round_f32(w))


def fp8_gate_up(x_bits, gate, up) -> np.ndarray:
    """h = bf16(silu(g) * u) with g, u the FP8 projections of the rows x (bf16
    bits [n, H]); gate, up: (codes [I, H], exponents [I]) from fp8_weight_rows."""
    xc, xe = fp8_quantise_rows(bf16_to_f64(x_bits))
    xv = e4m3_decode(xc)
    g = np.ldexp(xv @ e4m3_decode(gate[0]).T, xe[:, None] + gate[1][None, :])
    u = np.ldexp(xv @ e4m3_decode(up[0]).T, xe[:, None] + up[1][None, :])
    return round_bf16(silu64(g) * u)


def fp8_down(h_bits, down) -> np.ndarray:
    """y = the FP8 down projection of the rows h (bf16 bits [n, I]), float64."""
    hc, he = fp8_quantise_rows(bf16_to_f64(h_bits))
    return np.ldexp(e4m3_decode(hc) @ e4m3_decode(down[0]).T, he[:, None] + down[1][None, :])


def fp8_expert(layer, e: int):
    """Expert e of a layer upcast: dict of (codes, exponents) for gate, up, down."""
    bits = expert_bits(layer)
    return {"gate": fp8_weight_rows(layer.q_gate[e], layer.s_gate[e], layer.b_gate[e], bits),
            "up": fp8_weight_rows(layer.q_up[e], layer.s_up[e], layer.b_up[e], bits),
            "down": fp8_weight_rows(layer.q_down[e], layer.s_down[e], layer.b_down[e], bits)}


# ---------------------------------------------------------------- comparison helpers (test bars)

def bf16_ulp(v) -> np.ndarray:
    """Spacing of the bf16 values around |v| (float64): 2^(e-8) for |v| in [2^(e-1), 2^e),
    and 2^-133 (the least subnormal step) below the normal range and at zero.

    bf16 keeps 8 significant bits, so the spacing inside the binade [2^(e-1), 2^e)
    is 2^(e-1) * 2^-7 = 2^(e-8); the normal range ends at 2^-126, under which the
    values are multiples of 2^-133.
    """
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(a)
    e = np.where(a == 0.0, -200, e)
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def near_tie_tokens(logits_routed, k: int, gap: float = 1e-5) -> np.ndarray:
    """Tokens whose k-th and (k+1)-th largest routed logits lie less than `gap` apart.

    These are the tokens whose set of picks may change when the logits move by
    less than `gap`: the exemption that the pick bar grants (boolean [T]). Ranks
    are by value; equal values count as a gap of zero.
    """
    l = np.sort(np.asarray(logits_routed, dtype=np.float64), axis=1)[:, ::-1]
    if l.shape[1] <= k:
        return np.zeros(l.shape[0], dtype=bool)
    return (l[:, k - 1] - l[:, k]) < gap


def picks_within_ties(ids, ref_logits_routed, k: int, gap: float = 1e-5):
    """Compares ordered picks `ids` [T, k] with the oracle's picks on ref logits.

    A token passes when, slot by slot, each pick is the oracle's pick or an expert
    whose oracle logit lies within `gap` of that pick's. So a pick may differ from
    the oracle's only across a near tie: at the k-th/(k+1)-th boundary (the set
    changes; near_tie_tokens) or between two ranks inside the top k (the order
    changes). The picks of a token must be k distinct ids in [0, E).
    Returns (ok [T] bool, set_exempt [T] bool, order_exempt [T] bool): the last two
    mark passing tokens that differ from the oracle's picks, with a different set
    or with the same set in another order.
    """
    ids = np.asarray(ids, dtype=np.int64)
    l = np.asarray(ref_logits_routed, dtype=np.float64)
    T, E = l.shape
    ref = topk(ref_logits_routed, k).astype(np.int64)
    valid = ((ids >= 0) & (ids < E)).all(axis=1)
    distinct = np.array([len(set(r.tolist())) == k for r in ids])
    safe = np.clip(ids, 0, E - 1)
    rows = np.arange(T)[:, None]
    close = (ids == ref) | (np.abs(l[rows, safe] - l[rows, ref]) < gap)
    ok = valid & distinct & close.all(axis=1)
    differ = (ids != ref).any(axis=1)
    same_set = np.array([set(a.tolist()) == set(b.tolist()) for a, b in zip(ids, ref)])
    return ok, ok & differ & ~same_set, ok & differ & same_set

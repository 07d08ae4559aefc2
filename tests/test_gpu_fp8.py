"""GPU parity of the FP8 prompt route ("R9700: the 35B only one runtime could load",
its closing list of kernel work: the experts upcast to FP8 for the FP8 matrix
units) against the oracle's FP8 route (fp8_weight_rows, fp8_gate_up, fp8_down).

Inputs of the expert stage (x, the picks, the pick weights) come from the seeded
generators and the oracle's own routing, never from the GPU.

Bars. Both sides hold the same codes of x and of the weights (checked byte for
byte), so they part only where the GPU sums. The FP8 matrix cores do not add
exactly: they keep each product only to 13 bits below its run's operand exponents
(tests._fp8_mfma, measured on MI355X). fp8_expected evaluates the oracle's FP8
route with that summation (the model, from oracle codes only) and lists what the
model leaves open:
  * the fp32 rounding of the run-sum accumulation (_fp8_mfma.fp32_bound), for g, u
    and y;
  * h = bf16(silu(g) u): with g and u within that bound and the GPU's fp32 silu
    within (1e-6 + 1e-7 |g|) relative (an fp32 exp2 argument), an element whose
    interval straddles a bf16 rounding boundary may take either neighbour. Such a
    flip changes y only through the run of 8 down products holding that element,
    so the admissible outputs are y0 plus one choice per affected run.
A GPU row passes when it equals one admissible output within twice its fp32 bound
(y_check picks the choice). Where a flip could move h's row maximum across a power
of two, the row may be re-quantised as a whole; such rows (rare) are held to the
bound of any re-quantisation instead. The combined output must equal the oracle's
combine of the matched rows within their bounds, the fp32 combine's rounding and
one bf16 step. The model's departure from the oracle's exact sums is recorded and
held small (the median row within MODEL_GAP of its rms), so the summation is the
only difference. The upcast buffer (codes, zero padding, row scales) is byte work:
bit-exact.
"""

import itertools

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from quantized_moe_expert_fp32_amd import synth
from tests._fp8_mfma import RUN, fp32_bound, operand_exponent, run_sums
from tests._parity import _L, check_picks, record_stats

pytestmark = pytest.mark.gpu

MODEL_GAP = 1e-3
MAX_COMBOS = 4096  # exhaustive matching up to this many choices, else coordinate descent


def _moe():
    from quantized_moe_expert_fp32_amd import moe

    return moe


def _dev(c, idx=0):
    L = _L()
    return L.DeviceLayer(L.make_shape(c.shape), c.layers[idx], fp8=True)


def _oracle_route(layer, x, E, k):
    logits = O.router_logits(x, O.router_matrix(layer), getattr(layer, "logit_bias", None), E)
    ids = O.topk(logits[:, :E], k)
    return logits, ids, O.pick_weights(logits[:, :E], ids), O.shared_weight(logits[:, E])


def _gpu_experts(dl, x, ids):
    moe, L = _moe(), _L()
    sh = dl.shape
    T = x.shape[0]
    ws = torch.zeros(moe.moe_prefill_fp8_workspace_bytes(sh, T), dtype=torch.uint8, device="cuda")
    y = torch.full((T, sh.slots, sh.hidden), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_experts_prefill_fp8(sh, dl.experts_fp8, L.to_device(x), T,
                                L.to_device(np.ascontiguousarray(ids, dtype=np.int32)), ws, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _gpu_combine(dl, y, w, wsh):
    moe, L = _moe(), _L()
    T = y.shape[0]
    out = torch.empty((T, dl.shape.hidden), dtype=torch.int16, device="cuda")
    moe.moe_combine(dl.shape, L.to_device(np.ascontiguousarray(y, dtype=np.float32)), L.to_device(w),
                    L.to_device(wsh), T, None, out)
    torch.cuda.synchronize()
    return L.bits_to_numpy(out)


def _pad(v, n):
    out = np.zeros(v.shape[:-1] + (n,))
    out[..., :v.shape[-1]] = v
    return out


def _run_sum_direct(c, Dr, eDr):
    from tests._fp8_mfma import KEEP

    r = (eDr + operand_exponent(c)[None, :]).max(axis=1, keepdims=True)
    grid = np.ldexp(1.0, r - KEEP)
    return (np.trunc(Dr * c[None, :] / grid) * grid).sum(axis=1)


class PickModel:
    """The model's outputs for one pick: y0, its fp32 bound dy, the admissible
    per-run changes (options: list of (run, [delta vectors])) and, for a row that
    may be re-quantised, a bound of any re-quantisation (loose, else None)."""

    def __init__(self, y0, dy, options, loose, y_oracle):
        self.y0, self.dy, self.options, self.loose, self.y_oracle = y0, dy, options, loose, y_oracle


def _pick_model(xv, ex, xe_t, mat, x_row, I, Ip):
    f8, G, eG, U, eU, D, eD = mat
    sG, sU = run_sums(xv, G, eG, ex), run_sums(xv, U, eU, ex)
    g = np.ldexp(sG.sum(axis=1), xe_t + f8["gate"][1])
    u = np.ldexp(sU.sum(axis=1), xe_t + f8["up"][1])
    dg = np.ldexp(fp32_bound(sG), xe_t + f8["gate"][1])
    du = np.ldexp(fp32_bound(sU), xe_t + f8["up"][1])
    sg = O.silu64(g)
    P = sg * u
    dP = 1.1 * dg * np.abs(u) + (np.abs(sg) + 1.1 * dg) * du + (1e-6 + 1e-7 * np.abs(g)) * np.abs(P)
    h = O.round_bf16(P)
    lo, hi = O.round_bf16(P - dP), O.round_bf16(P + dP)
    hv, lov, hiv = O.bf16_to_f64(h), O.bf16_to_f64(lo), O.bf16_to_f64(hi)
    b = int(O.fp8_row_exponent(np.abs(hv).max()))
    sd = np.ldexp(1.0, b + f8["down"][1])  # [H] output scales
    c0 = _pad(O.fp8_rows_value(*O.fp8_quantise_rows(hv[None, :]))[0], Ip) * 2.0 ** -b
    s0 = run_sums(c0, D, eD)
    y0 = s0.sum(axis=1) * sd
    dy = fp32_bound(s0) * sd
    amax_hi = np.maximum(np.abs(lov), np.abs(hiv)).max()
    amax_lo = np.where(np.sign(lov) != np.sign(hiv), 0.0, np.minimum(np.abs(lov), np.abs(hiv))).max()
    loose = None
    options = []
    if O.fp8_row_exponent(amax_hi) != b or O.fp8_row_exponent(amax_lo) != b:
        Dv = np.abs(D[:, :I]) * sd[:, None]
        move = np.abs(hiv - lov) + np.abs(hv) / 4 + np.ldexp(1.0, b - 7)  # E4M3 half steps, either scale
        loose = (Dv @ move + 2.0 ** -12 * (Dv @ np.abs(hv))) * 2.0 ** -b
    else:
        flip = np.nonzero((lo != h) | (hi != h))[0]
        for r in sorted(set(int(i) // RUN for i in flip)):
            sl = slice(RUN * r, RUN * r + RUN)
            els = [int(i) for i in flip if int(i) // RUN == r]
            # the codes each flippable element may take (its value and its neighbours)
            choices = [np.unique(O.e4m3_decode(O.e4m3_encode(np.array([hv[i], lov[i], hiv[i]]) * 2.0 ** -b)))
                       for i in els]
            base = _run_sum_direct(c0[sl], D[:, sl], eD[:, sl])
            deltas = []
            for combo in itertools.product(*choices):
                cr = c0[sl].copy()
                for i, v in zip(els, combo):
                    cr[i - RUN * r] = v
                if np.array_equal(cr, c0[sl]):
                    continue
                d = (_run_sum_direct(cr, D[:, sl], eD[:, sl]) - base) * sd
                if not any(np.array_equal(d, q) for q in deltas):
                    deltas.append(d)
            if deltas:
                options.append((r, deltas))
    yo = O.fp8_down(O.fp8_gate_up(x_row, f8["gate"], f8["up"]), f8["down"])[0]
    return PickModel(y0, dy, options, loose, yo)


def fp8_expected(x_bits, ids, layer, E, k):
    """PickModel [n][S] for the rows x (bf16 bits [n, H]) with picks ids [n, k]
    (slot k: the shared expert); picks evaluated on a thread pool."""
    from concurrent.futures import ThreadPoolExecutor

    n, S = ids.shape[0], k + 1
    H, I = layer.q_down.shape[1], layer.q_gate.shape[1]
    Hp, Ip = -(-H // 128) * 128, -(-I // 128) * 128
    xc, xe = O.fp8_quantise_rows(O.bf16_to_f64(x_bits))
    xv = _pad(O.e4m3_decode(xc), Hp)
    ex = operand_exponent(xv)
    experts = [[int(ids[t, s]) if s < k else E for s in range(S)] for t in range(n)]

    def mat(e):
        f8 = O.fp8_expert(layer, e)
        G = _pad(O.e4m3_decode(f8["gate"][0]), Hp)
        U = _pad(O.e4m3_decode(f8["up"][0]), Hp)
        D = _pad(O.e4m3_decode(f8["down"][0]), Ip)
        return e, (f8, G, operand_exponent(G), U, operand_exponent(U), D, operand_exponent(D))

    with ThreadPoolExecutor(max_workers=8) as pool:
        mats = dict(pool.map(mat, sorted({e for row in experts for e in row})))
        futs = [[pool.submit(_pick_model, xv[t], ex[t], int(xe[t]), mats[experts[t][s]], x_bits[t:t + 1], I, Ip)
                 for s in range(S)] for t in range(n)]
        return [[f.result() for f in row] for row in futs]


def _match(res, pm):
    """The admissible output nearest the GPU row res: (y, max |res - y| / (2 dy))."""
    tol = 2 * pm.dy + 1e-300
    best = pm.y0
    score = (np.abs(res - best) / tol).max()
    opts = [[np.zeros_like(pm.y0)] + d for _, d in pm.options]
    if not opts or score <= 1:
        return best, score
    if np.prod([len(o) for o in opts], dtype=np.float64) <= MAX_COMBOS:
        for combo in itertools.product(*opts):
            y = pm.y0 + np.sum(combo, axis=0)
            sc = (np.abs(res - y) / tol).max()
            if sc < score:
                best, score = y, sc
        return best, score
    choice = [0] * len(opts)
    for _ in range(4):  # coordinate descent over the runs
        for j, o in enumerate(opts):
            rest = pm.y0 + sum(opts[q][choice[q]] for q in range(len(opts)) if q != j)
            scores = [(np.abs(res - rest - d) / tol).max() for d in o]
            choice[j] = int(np.argmin(scores))
    best = pm.y0 + sum(opts[q][choice[q]] for q in range(len(opts)))
    return best, (np.abs(res - best) / tol).max()


def y_check(g, models, keep=None, what="y"):
    """Every GPU row equal to one admissible output of the model within twice its fp32
    bound (rows that may be re-quantised: within the loose bound); the model near the
    oracle. Returns (matched y [n, S, H], tolerance [n, S, H]) for out_check."""
    n, S = len(models), len(models[0])
    ym = np.zeros(g.shape)
    tol = np.zeros(g.shape)
    worst, flipped, loose_rows, gaps = 0.0, 0, 0, []
    for t in range(n):
        for s in range(S):
            if keep is not None and not keep[t, s]:
                continue
            pm = models[t][s]
            res = g[t, s].astype(np.float64)
            assert np.isfinite(res).all(), (t, s)
            rms = np.sqrt(np.mean(pm.y_oracle ** 2)) or 1.0
            gaps.append(np.abs(pm.y0 - pm.y_oracle).max() / rms)
            if pm.loose is not None:
                loose_rows += 1
                sc = (np.abs(res - pm.y0) / (pm.loose + 2 * pm.dy)).max()
                ym[t, s], tol[t, s] = pm.y0, pm.loose + 2 * pm.dy
            else:
                y, sc = _match(res, pm)
                flipped += int(not np.array_equal(y, pm.y0))
                ym[t, s], tol[t, s] = y, 2 * pm.dy
            worst = max(worst, float(sc))
    stats = dict(what=what, rows=int(len(gaps)), worst_over_tol=worst, rows_with_flips=flipped,
                 rows_requantisable=loose_rows, median_model_gap=float(np.median(gaps)),
                 max_model_gap=float(np.max(gaps)))
    record_stats(**stats)
    assert worst <= 1.0, stats
    assert stats["median_model_gap"] <= MODEL_GAP, stats
    return ym, tol


def out_check(gpu_bits, y_match, tol_y, w_bits, wsh_bits, what="out"):
    """The GPU's combined output against the oracle's combine of the matched rows:
    within sum_s w_s tol_s, the fp32 combine's rounding and one bf16 step."""
    ref = O.combine(y_match, w_bits, wsh_bits)
    g = O.bf16_to_f64(gpu_bits)
    r = O.bf16_to_f64(ref)
    wts = np.abs(np.concatenate([O.bf16_to_f64(w_bits), O.bf16_to_f64(wsh_bits)[:, None]], axis=1))
    dsum = np.einsum("ts,tsh->th", wts, tol_y)
    dsum += 16 * 2.0 ** -24 * np.einsum("ts,tsh->th", wts, np.abs(y_match) + tol_y)
    tol = dsum + O.bf16_ulp(np.abs(r) + dsum)
    err = np.abs(g - r)
    stats = dict(what=what, n=int(err.size), n_bad=int((err > tol).sum()), frac_exact=float((err == 0).mean()))
    record_stats(**stats)
    assert stats["n_bad"] == 0, stats
    return stats


def _check_fp8_buffer(dl, layer, experts):
    moe = _moe()
    R = moe.fp8_expert_regions(dl.shape)
    buf = dl.experts_fp8.cpu().numpy()
    stride = R["stride"]
    assert buf.size == stride * dl.shape.n_mats
    for m in experts:
        ref = O.fp8_expert(layer, m)
        base = m * stride
        for name in ("gate", "up", "down"):
            off, rows, rowb = R[name]
            codes = buf[base + off:base + off + rows * rowb].reshape(rows, rowb)
            K = ref[name][0].shape[1]
            assert np.array_equal(codes[:, :K], ref[name][0]), (m, name)
            assert not codes[:, K:].any(), (m, name)
        off, cnt = R["scales"]
        sc = buf[base + off:base + off + 4 * cnt].view(np.float32)
        e = np.concatenate([ref["gate"][1], ref["up"][1], ref["down"][1]])
        assert np.array_equal(sc, np.ldexp(1.0, e).astype(np.float32)), m


@pytest.mark.parametrize("name,bits,experts", [("tiny", 4, range(17)), ("tiny", 8, range(17)),
                                               ("prefill512", 4, (0, 77, 255, 256))])
def test_fp8_upcast_bit_exact(gpu, name, bits, experts):
    """The upcast codes, their zero padding and the row scales, byte for byte."""
    c = synth.make_case(name, T=1, bits=bits)
    _check_fp8_buffer(_dev(c), c.layers[0], experts)


@pytest.mark.parametrize("name,T,bits", [("tiny", 1, 4), ("tiny", 200, 4), ("tiny", 700, 4), ("tiny", 300, 8)])
def test_fp8_experts_and_layer(gpu, name, T, bits):
    """Expert outputs and the combined layer on the oracle's picks: one row, partial
    tiles, the shared expert over full 256-row tiles plus a ragged one, 8-bit experts."""
    c = synth.make_case(name, T=T, bits=bits)
    sh, layer = c.shape, c.layers[0]
    E, k = sh.n_experts, sh.top_k
    x = synth.random_x(2000 + T, T, sh.hidden)
    dl = _dev(c)
    _, ids, w, wsh = _oracle_route(layer, x, E, k)
    y = _gpu_experts(dl, x, ids)
    ym, tol = y_check(y, fp8_expected(x, ids, layer, E, k))
    out_check(_gpu_combine(dl, y, w, wsh), ym, tol, w, wsh)


def test_fp8_invalid_picks_zero_rows(gpu):
    """Picks with an id outside [0, E) give zero rows; every other row is unchanged."""
    c = synth.make_case("tiny", T=64)
    sh, layer = c.shape, c.layers[0]
    E, k = sh.n_experts, sh.top_k
    x = synth.random_x(2100, 64, sh.hidden)
    dl = _dev(c)
    _, ids, _, _ = _oracle_route(layer, x, E, k)
    bad = ids.copy()
    bad[3, 1] = -1
    bad[10, 0] = E
    y = _gpu_experts(dl, x, bad)
    assert not y[3, 1].any() and not y[10, 0].any()
    keep = np.ones(y.shape[:2], bool)
    keep[3, 1] = keep[10, 0] = False
    y_check(y, fp8_expected(x, ids, layer, E, k), keep)


def test_fp8_deterministic_and_chunk_invariant(gpu):
    """Each output depends on its own token's row in a fixed order: two calls agree
    bit for bit, and 16 tokens alone give the same bytes as inside 128."""
    c = synth.make_case("prefill512", T=128)
    sh, layer = c.shape, c.layers[0]
    E, k = sh.n_experts, sh.top_k
    x = synth.random_x(2200, 128, sh.hidden)
    dl = _dev(c)
    _, ids, _, _ = _oracle_route(layer, x, E, k)
    y1 = _gpu_experts(dl, x, ids)
    y2 = _gpu_experts(dl, x, ids)
    assert np.array_equal(y1, y2)
    y16 = _gpu_experts(dl, x[:16], ids[:16])
    assert np.array_equal(y16, y1[:16])


@pytest.mark.parametrize("name", ["prefill512", "prefill4096"])
def test_fp8_full_size_sampled(gpu, name):
    """The benchmark's prompt workloads at full size (512 tokens; 4096 tokens with
    Zipf-skewed routing, so the hot experts span several 256-row tiles): the whole
    batch on the GPU, eight sampled tokens in the oracle (a token's outputs depend
    on its own row only)."""
    c = synth.make_case(name)
    sh, layer = c.shape, c.layers[0]
    E, k = sh.n_experts, sh.top_k
    dl = _dev(c)
    _, ids, w, wsh = _oracle_route(layer, c.x, E, k)
    if name == "prefill4096":
        counts = np.bincount(ids.reshape(-1), minlength=E)
        assert counts.max() > 256  # several tiles for the hot experts
    y = _gpu_experts(dl, c.x, ids)
    rows = np.random.default_rng(7).choice(c.T, 6, replace=False)
    ym, tol = y_check(y[rows], fp8_expected(c.x[rows], ids[rows], layer, E, k))
    out_check(_gpu_combine(dl, y[rows], w[rows], wsh[rows]), ym, tol, w[rows], wsh[rows])


def test_fp8_layer_end_to_end(gpu):
    """route -> FP8 experts -> combine through the layer driver on the GPU's own
    routing: picks within the oracle's near ties, and the tokens whose picks equal
    the oracle's within the bar of the module docstring."""
    L = _L()
    c = synth.make_case("prefill512", T=96)
    sh, layer = c.shape, c.layers[0]
    E, k = sh.n_experts, sh.top_k
    dl = _dev(c)
    buf = L.alloc_buffers(dl.shape, c.T, "fp8")
    L.layer_step(dl, L.to_device(c.x), buf, "fp8")
    torch.cuda.synchronize()
    logits, ids, w, wsh = _oracle_route(layer, c.x, E, k)
    gids = buf.ids.cpu().numpy()
    check_picks(gids, logits, k, E)
    same = (gids == ids).all(axis=1)
    assert same.mean() > 0.9
    rows = np.nonzero(same)[0][:8]
    ym, tol = y_check(buf.y.cpu().numpy()[rows], fp8_expected(c.x[rows], ids[rows], layer, E, k))
    out_check(L.bits_to_numpy(buf.out)[rows], ym, tol, w[rows], wsh[rows])


def test_fp8_exact_operands(gpu):
    """Integer weights (scale 1, bias -8: w = q - 8) and inputs that are small
    integers: every gate/up product sits on the summation's grid, so the model's
    g and u are the exact ones, and a wrong row, column, chunk or scale shows as an
    O(1) error."""
    c = synth.make_case("prefill512", T=160)
    sh, layer = c.shape, c.layers[0]
    E, k = sh.n_experts, sh.top_k
    for m in ("gate", "up", "down"):
        getattr(layer, "s_" + m)[...] = 0x3F80
        getattr(layer, "b_" + m)[...] = 0xC100
    rng = np.random.default_rng(2300)
    x = O.round_bf16(rng.integers(-16, 17, (160, sh.hidden)).astype(np.float64))
    dl = _dev(c)
    _, ids, _, _ = _oracle_route(layer, x, E, k)
    y = _gpu_experts(dl, x, ids)
    rows = np.arange(0, 160, 20)
    y_check(y[rows], fp8_expected(x[rows], ids[rows], layer, E, k))

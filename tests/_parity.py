"""Helpers of the GPU parity tests: the comparison bars and the staged checks.

Bars (routing contract of TensorFold issue #931, "What I'd build"; staged
reference per projection class from its "Gate" section):
  * integer work (picks, dispatch) bit-exact; end to end, a pick may differ from
    the oracle's only across a near tie (the two oracle logits less than 1e-5
    apart): at the k-th/(k+1)-th boundary or, with the same set, inside the top k
    (both counted);
  * pick and shared weights bit-exact when computed from the same fp32 logits;
  * logits within 1 fp32 ulp of the oracle's fp32 rounding of the fp64 sum;
  * layer outputs: |gpu - ref| <= max(2 bf16 ulp(ref), 1e-2 |ref|, 1e-2 rms(ref row)),
    and at most FRAC_GT_2ULP of the elements beyond 2 bf16 ulp.
Statistics of every output and pick check are appended as JSON lines to the file
named by MOE_PARITY_STATS when that variable is set.
"""

import functools
import json
import os

import numpy as np
import torch

from oracle import moe_oracle as O
from quantized_moe_expert_fp32_amd import synth


@functools.lru_cache(maxsize=None)
def case(name, T=None):
    return synth.make_case(name, T=T)


def _L():
    from quantized_moe_expert_fp32_amd import layer as L

    return L


def dev_layer(gpu, c, idx=0, shape=None):
    L = _L()
    sh = shape or L.make_shape(c.shape)
    return L.DeviceLayer(sh, c.layers[idx])


def run_path(gpu, dl, x_np, path):
    """route -> experts -> combine on the GPU; returns numpy copies of every stage."""
    L = _L()
    T = x_np.shape[0]
    buf = L.alloc_buffers(dl.shape, T, path)
    x = L.to_device(x_np)
    L.layer_step(dl, x, buf, path)
    torch.cuda.synchronize()
    return dict(logits=buf.logits.cpu().numpy(), ids=buf.ids.cpu().numpy(), w=L.bits_to_numpy(buf.w),
                wsh=None if buf.wsh is None else L.bits_to_numpy(buf.wsh), y=buf.y.cpu().numpy(),
                out=L.bits_to_numpy(buf.out))


# Elements beyond 2 bf16 ulp come from outputs that cancel to far below their
# row's scale (the row-rms term of the bar) and from rounding flips of h between
# fp32 and fp64 accumulation; the bound is asserted on every output check.
FRAC_GT_2ULP = 2e-3


def record_stats(**kw):
    path = os.environ.get("MOE_PARITY_STATS")
    if path:
        kw["test"] = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
        with open(path, "a") as f:
            f.write(json.dumps(kw) + "\n")


def out_tolerance_check(gpu_bits, ref_bits, rows=None, what="out"):
    g = O.bf16_to_f64(gpu_bits)
    r = O.bf16_to_f64(ref_bits)
    if rows is not None:
        g, r = g[rows], r[rows]
    err = np.abs(g - r)
    ulp = O.bf16_ulp(r)
    rms = np.sqrt(np.mean(r * r, axis=1, keepdims=True))
    tol = np.maximum(np.maximum(2 * ulp, 1e-2 * np.abs(r)), 1e-2 * rms)
    bad = err > tol
    stats = dict(what=what, n=int(err.size), max_ulp=float((err / ulp).max()) if err.size else 0.0,
                 frac_gt_2ulp=float((err > 2 * ulp).mean()) if err.size else 0.0,
                 frac_exact=float((err == 0).mean()) if err.size else 1.0, n_bad=int(bad.sum()))
    record_stats(**stats)
    assert stats["n_bad"] == 0, stats
    assert stats["frac_gt_2ulp"] <= FRAC_GT_2ULP, stats
    return stats


def check_logits(gpu_logits, ref_logits, fp64_path=True):
    """fp64-accumulated logits (T <= 16): within 1 fp32 ulp of the oracle's.
    Matrix-core logits (T > 16, fp32 accumulation): within 2e-6 absolute."""
    g = gpu_logits.astype(np.float32)
    r = ref_logits.astype(np.float32)
    if not fp64_path:
        d = np.abs(g.astype(np.float64) - r.astype(np.float64))
        assert d.max() <= 2e-6, d.max()
        return float((d == 0).mean())
    gi = g.view(np.int32).astype(np.int64)
    ri = r.view(np.int32).astype(np.int64)
    diff = np.abs(gi - ri)
    assert diff.max() <= 1, diff.max()
    return float((diff == 0).mean())


def check_picks(gpu_ids, ref_logits, k, E):
    """End-to-end picks against the oracle's on its own logits; returns the counts of
    near-tie tokens at the k/k+1 boundary, of tokens whose set differed across it and
    of tokens whose order differed across a near tie inside the top k."""
    ok, set_ex, order_ex = O.picks_within_ties(gpu_ids, ref_logits[:, :E], k)
    assert ok.all(), np.nonzero(~ok)
    n_tie = int(O.near_tie_tokens(ref_logits[:, :E], k).sum())
    record_stats(what="picks", n=int(len(ok)), near_tie=n_tie, set_differs=int(set_ex.sum()),
                 order_differs=int(order_ex.sum()))
    return n_tie, int(set_ex.sum()), int(order_ex.sum())


def staged_route_check(gpu, res, E, k, has_shared=True):
    """Selection step from the GPU's own logits: ids, weights and shared weight bit-exact."""
    lg = res["logits"]
    ids = O.topk(lg[:, :E], k)
    assert np.array_equal(res["ids"], ids)
    assert np.array_equal(res["w"], O.pick_weights(lg[:, :E], ids))
    if has_shared:
        assert np.array_equal(res["wsh"], O.shared_weight(lg[:, E]))


def staged_layer_check(res, x_np, host_layer, E, has_shared=True):
    """Oracle experts and combine fed the GPU's picks and weights."""
    y, _ = O.expert_outputs(x_np, res["ids"], host_layer, E, has_shared)
    out = O.combine(y, res["w"], res["wsh"] if has_shared else None)
    return out_tolerance_check(res["out"], out), y



"""The 40-layer decode stack (MoE blocks with RMSNorm and the residual add, 40
independent layers of the 35B shape, about 18 GB of weights) at 1 and 16 tokens.
Two call sequences, each captured in a HIP graph and replayed three times (every
replay gives the same states):
  * staged: moe_rmsnorm, then moe_decode_layer with the residual, per layer; every
    layer is checked against the oracle: the GPU's RMSNorm within one bf16 step of
    the oracle's (fp32 against float64 norm arithmetic), and the oracle layer fed
    the GPU's own normalised input - picks within near ties, and the new state
    bf16(x + out) within the output bar on the rows whose picks equal the oracle's;
  * fused (the sequence bench.py times): one moe_decode_block per layer, between two
    state buffers; every layer's state and picks equal the staged sequence's bit for
    bit.
"""

import concurrent.futures as cf

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from quantized_moe_expert_fp32_amd import synth
from tests._parity import _L, out_tolerance_check, record_stats

pytestmark = pytest.mark.gpu

N_LAYERS = 40


def _oracle_layer(args):
    xin, xn, host = args
    st = O.layer_forward(xn, host, 8)
    return st["logits"], st["ids"], O.residual_bf16(xin, st["out"])


def _replays(g, x, x0, keep, T, what):
    """Replays graph g three times from state x0; every replay's kept states are equal."""
    L = _L()
    first = None
    for rep in range(3):
        x.copy_(x0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        states = [tuple(L.bits_to_numpy(a) if a.dtype == torch.int16 else a.cpu().numpy() for a in kept)
                  for kept in keep]
        if first is None:
            first = states
        else:
            for l in range(N_LAYERS):
                for j in range(len(states[l])):
                    assert np.array_equal(first[l][j], states[l][j]), (what, rep, l, j)
        record_stats(what="stack_replay_" + what, T=T, rep=rep)
    return first


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [1, 16])
def test_stack40_graph_replay(gpu, T):
    L = _L()
    c = synth.make_case("stack", T=T, n_layers=N_LAYERS)
    record_stats(what="stack_setup", T=T, layers=len(c.layers))
    sh = L.make_shape(c.shape)
    layers = [L.DeviceLayer(sh, hl, prefill=False) for hl in c.layers]
    x0 = L.to_device(c.x)
    x = x0.clone()
    xn = torch.empty_like(x)
    buf = L.alloc_buffers(sh, T, L.pick_path(T))
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        L.stack_step(layers, x, xn, buf)  # eager warm-up
    torch.cuda.synchronize()
    keep = []
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        L.stack_step(layers, x, xn, buf, keep=keep)
    torch.cuda.synchronize()
    first = _replays(g, x, x0, keep, T, "staged")
    # the fused sequence: one moe_decode_block per layer between two state buffers
    xa, xb = x0.clone(), torch.empty_like(x0)
    with torch.cuda.stream(stream):
        L.stack_step_fused(layers, xa, xb, buf)  # eager warm-up
    torch.cuda.synchronize()
    keep_f = []
    gf = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gf, stream=stream):
        L.stack_step_fused(layers, xa, xb, buf, keep=keep_f)
    torch.cuda.synchronize()
    fused = _replays(gf, xa, x0, keep_f, T, "fused")
    for l in range(N_LAYERS):
        assert np.array_equal(fused[l][0], first[l][0]), ("state", l)
        assert np.array_equal(fused[l][-1], first[l][-1]), ("ids", l)
    assert gpu.moe_decode_layer_check(sh, T, buf.ws) if L.pick_path(T) == "fused" else True
    ins = [c.x] + [first[l][0] for l in range(N_LAYERS - 1)]
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        refs = list(ex.map(_oracle_layer, [(ins[l], first[l][1], c.layers[l]) for l in range(N_LAYERS)]))
    n_set = n_order = 0
    for l in range(N_LAYERS):
        xin, xn_gpu, ids_gpu = ins[l], first[l][1], first[l][2]
        d = np.abs(xn_gpu.astype(np.int32) - O.rmsnorm_bf16(xin).astype(np.int32))
        assert d.max() <= 1 and (d > 0).mean() < 2e-3, l
        logits, ids_ref, ref_state = refs[l]
        ok, set_ex, order_ex = O.picks_within_ties(ids_gpu, logits[:, :256], 8)
        assert ok.all(), (l, np.nonzero(~ok))
        n_set += int(set_ex.sum())
        n_order += int(order_ex.sum())
        rows = (ids_gpu == ids_ref).all(axis=1)
        out_tolerance_check(first[l][0], ref_state, rows=rows, what="stack_layer_%d" % l)
    record_stats(what="stack_picks", T=T, set_differs=n_set, order_differs=n_order)

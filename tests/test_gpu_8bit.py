"""GPU parity of the 8-bit affine experts (TensorFold issue #931, "What I'd build":
the 8-bit expert checkpoint, same groups of 64, same ABI with bits = 8). The
library packs an 8-bit row of K codes as a 4-bit row of 2K codes (high nibbles
with (16 scale, bias), then low nibbles with (scale, 0)); every path is checked
against the oracle's 8-bit dequantisation w = scale * q + bias."""

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from quantized_moe_expert_fp32_amd import synth
from tests._parity import _L, check_logits, check_picks, run_path, staged_layer_check, staged_route_check

pytestmark = pytest.mark.gpu


def _layer(name, seed_shift=0):
    c = synth.make_case(name, bits=8, seed=synth.WORKLOADS[name][7] + 100 + seed_shift)
    assert O.expert_bits(c.layers[0]) == 8
    L = _L()
    return c, L.DeviceLayer(L.make_shape(c.shape), c.layers[0])


def test_pack_8bit_group_words(gpu):
    """The packed (scale, bias) words of an 8-bit gate row: (16 s, b) for the high
    plane's groups, then (s, 0) for the low plane's, in the blocked order."""
    c, dl = _layer("tiny")
    L0 = c.layers[0]
    H, I, M = 256, 64, 17
    p = dl.experts.cpu().numpy()
    stride = p.size // M
    Gw = 2 * H // 64  # groups of a 4-bit row of 2H codes
    gu_sb = 2 * I * (2 * H) // 2 + H * (2 * I) // 2  # after gate/up and down codes
    for m in (0, 16):
        w = p[m * stride + gu_sb:m * stride + gu_sb + 2 * I * Gw * 4].view(np.uint32).reshape(I // 2, Gw, 4)
        for r in (0, 5, 63):
            row = w[r // 2, :, r % 2]  # gate rows sit in slots 0, 1 of their block
            s16 = synth._to_bf16_bits(16 * synth.bf16_bits_to_f32(L0.s_gate[m, r]))
            hi = s16.astype(np.uint32) | (L0.b_gate[m, r].astype(np.uint32) << 16)
            lo = L0.s_gate[m, r].astype(np.uint32)
            assert np.array_equal(row[:Gw // 2], hi) and np.array_equal(row[Gw // 2:], lo)


@pytest.mark.parametrize("name,T", [("tiny", 1), ("tiny", 4), ("decode", 1), ("decode", 16)])
def test_8bit_decode_paths(gpu, name, T):
    """Staged decode, the single-launch decode layer (bit-identical to it) and the
    oracle bar."""
    c, dl = _layer(name)
    x = synth.random_x(1000 + T, T, c.shape.hidden)
    E, k = c.shape.n_experts, c.shape.top_k
    staged = run_path(gpu, dl, x, "decode")
    fused = run_path(gpu, dl, x, "fused")
    for key in ("logits", "ids", "w", "wsh", "y", "out"):
        assert np.array_equal(staged[key], fused[key]), key
    ref = O.router_logits(x, O.router_matrix(c.layers[0]), None, E)
    check_logits(fused["logits"], ref, fp64_path=True)
    check_picks(fused["ids"], ref, k, E)
    staged_route_check(gpu, fused, E, k)
    staged_layer_check(fused, x, c.layers[0], E)


@pytest.mark.parametrize("name,T", [("tiny", 40), ("decode", 64)])
def test_8bit_prefill(gpu, name, T):
    """The grouped GEMMs over the two planes (full and ragged tiles) against the oracle."""
    c, dl = _layer(name)
    x = synth.random_x(1100 + T, T, c.shape.hidden)
    E, k = c.shape.n_experts, c.shape.top_k
    res = run_path(gpu, dl, x, "prefill")
    staged_route_check(gpu, res, E, k)
    staged_layer_check(res, x, c.layers[0], E)


def test_8bit_decode_matches_prefill(gpu):
    """16 tokens through the decode and the prefill path with 8-bit experts: same
    picks, outputs within the bar of each other."""
    c, dl = _layer("decode", 1)
    x = synth.random_x(1200, 16, 2048)
    a = run_path(gpu, dl, x, "fused")
    b = run_path(gpu, dl, x, "prefill")
    assert np.array_equal(a["ids"], b["ids"]) and np.array_equal(a["w"], b["w"])
    from tests._parity import out_tolerance_check

    out_tolerance_check(b["out"], a["out"])

"""moe_experts_decode_noalloc (h rows in the library's device array, no workspace
argument, no allocation) against moe_experts_decode (caller workspace): two calls
in a row, the second with a smaller input, give bit-identical slot outputs."""

import numpy as np
import pytest
import torch

from quantized_moe_expert_fp32_amd import synth
from tests._parity import _L, case, dev_layer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,calls", [("decode", ((16, 901), (3, 902))), ("tiny", ((4, 903), (1, 904)))])
def test_noalloc_decode_matches_workspace_entry(gpu, name, calls):
    c = case(name)
    dl = dev_layer(gpu, c)
    L = _L()
    H = c.shape.hidden
    for T, seed in calls:
        x = L.to_device(synth.random_x(seed, T, H))
        buf = L.alloc_buffers(dl.shape, T, "decode")
        gpu.moe_route(dl.shape, dl.router, dl.logit_bias, x, T, buf.logits, buf.ids, buf.w, buf.wsh)
        y_ref = torch.full_like(buf.y, 3.0)
        y_na = torch.full_like(buf.y, float("nan"))
        gpu.moe_experts_decode(dl.shape, dl.experts, x, T, buf.ids, buf.ws, y_ref)
        gpu.moe_experts_decode_noalloc(dl.shape, dl.experts, x, T, buf.ids, y_na)
        torch.cuda.synchronize()
        a, b = y_ref.cpu().numpy(), y_na.cpu().numpy()
        assert np.isfinite(b).all()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (name, T)


def test_noalloc_decode_refuses_bad_arguments(gpu):
    c = case("decode")
    dl = dev_layer(gpu, c)
    L = _L()
    x = L.to_device(synth.random_x(905, 1, 2048))
    ids = torch.zeros((17, 8), dtype=torch.int32, device="cuda")
    y = torch.empty((17, 9, 2048), dtype=torch.float32, device="cuda")
    from quantized_moe_expert_fp32_amd import moe

    with pytest.raises(moe.MoeError):
        gpu.moe_experts_decode_noalloc(dl.shape, dl.experts, x, 17, ids, y)
    with pytest.raises(moe.MoeError):
        gpu.moe_experts_decode_noalloc(dl.shape, dl.experts, x, 0, ids, y)

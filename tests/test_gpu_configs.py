"""GPU parity of the kernel instances and configurations beyond the served decode
shape, through the C ABI:
  * the single-launch decode layer on other shapes - the generic instance, the
    fp32 router, one and sixteen keys per lane, no shared expert, a logit bias,
    and more h words than one staging pass of a one-token launch holds - each
    bit-identical to the staged calls and within the oracle bar;
  * the fp32 router above 16 tokens, and 8-bit routers of other sizes on the
    matrix cores (both tile shapes byte-equal);
  * the prefill path's dispatch, read back from its workspace, against the
    oracle's histogram and stable expert-sorted order;
  * the prefill path's determinism and chunk invariance: the same tokens in one
    call or in chunks of 128 and 16 rows give byte-equal slot outputs and layer
    outputs (TensorFold issue #931, the slice-1 reply: prompt chunks of 128 and 16
    rows give byte-equal states; "What I'd build": windows of 1 to 16 rows).
"""

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from quantized_moe_expert_fp32_amd import synth
from tests._parity import (_L, case, check_logits, check_picks, dev_layer, run_path, staged_layer_check,
                           staged_route_check)

pytestmark = pytest.mark.gpu

F32, A8 = synth.ROUTER_F32, synth.ROUTER_AFFINE8

# name: (hidden, inter, n_experts, top_k, has_shared, router format, Zipf logit bias, token counts)
FUSED_CASES = {
    "tiny_fp32_router": (256, 64, 16, 2, 1, F32, False, (1, 4)),      # generic instance, one key per lane
    "tiny_no_shared": (256, 64, 16, 2, 0, F32, False, (1, 3)),        # no shared expert
    "served_zipf_bias": (2048, 512, 256, 8, 1, A8, True, (1, 16)),     # the served instance with a logit bias
    "inter1024": (2048, 1024, 64, 8, 1, A8, False, (1, 3)),            # 9 x 512 h words: two staging passes
    "top16": (1024, 512, 128, 16, 1, A8, False, (1, 2)),               # 17 x 256 h words, k = 16
    "experts300": (512, 128, 300, 4, 1, F32, False, (1, 5)),           # five keys per lane (16-key instance)
}


def _fused_case_params():
    return [(n, T) for n, c in FUSED_CASES.items() for T in c[-1]]


@pytest.mark.parametrize("name,T", _fused_case_params())
def test_fused_decode_instances(gpu, name, T):
    H, I, E, k, hs, rf, zipf, _ = FUSED_CASES[name]
    shape = synth.Shape(hidden=H, inter=I, n_experts=E, top_k=k, has_shared=hs, router_fmt=rf)
    host = synth.make_layer(shape, seed=20 + list(FUSED_CASES).index(name), layer=0, zipf=zipf)
    x = synth.random_x(700 + T, T, H)
    L = _L()
    dl = L.DeviceLayer(L.make_shape(shape), host)
    staged = run_path(gpu, dl, x, "decode")
    buf = L.alloc_buffers(dl.shape, T, "fused")
    dx = L.to_device(x)
    for _ in range(2):  # the second launch runs on the control words the first left
        L.layer_step(dl, dx, buf, "fused")
    torch.cuda.synchronize()
    assert gpu.moe_decode_layer_check(dl.shape, T, buf.ws), "a bounded wait timed out"
    fused = dict(logits=buf.logits.cpu().numpy(), ids=buf.ids.cpu().numpy(), w=L.bits_to_numpy(buf.w),
                 wsh=None if buf.wsh is None else L.bits_to_numpy(buf.wsh), y=buf.y.cpu().numpy(),
                 out=L.bits_to_numpy(buf.out))
    for key in ("logits", "ids", "w", "wsh", "y", "out"):
        if fused[key] is not None:
            assert np.array_equal(staged[key], fused[key]), key
    ref = O.router_logits(x, O.router_matrix(host), host.logit_bias, E)
    check_logits(fused["logits"], ref, fp64_path=True)
    check_picks(fused["ids"], ref, k, E)
    staged_route_check(gpu, fused, E, k, has_shared=bool(hs))
    staged_layer_check(fused, x, host, E, has_shared=bool(hs))


@pytest.mark.parametrize("T", [17, 40, 100])
def test_fp32_router_above_16_tokens(gpu, T):
    """The fp32 router keeps fp64 accumulation at any token count (16 tokens per
    launch row), so its logits stay within one fp32 ulp of the oracle's."""
    c = case("tiny")
    dl = dev_layer(gpu, c)
    x = synth.random_x(800 + T, T, 256)
    res = run_path(gpu, dl, x, "prefill")
    ref = O.router_logits(x, O.router_matrix(c.layers[0]), None, 16)
    assert check_logits(res["logits"], ref, fp64_path=True) > 0.999
    check_picks(res["ids"], ref, 2, 16)
    staged_route_check(gpu, res, 16, 2)
    staged_layer_check(res, x, c.layers[0], 16)


def _dispatch_from_ws(gpu, shape, T, ws):
    v = gpu.moe_prefill_dispatch_layout(shape, T)
    b = ws.cpu().numpy()
    M, S = shape.n_mats, shape.slots
    i32 = lambda off, n: b[off:off + 4 * n].view(np.int32).copy()
    ntiles = int(i32(v.ntiles, 1)[0])
    assert 0 < ntiles <= v.max_tiles
    return (i32(v.counts, M), i32(v.offsets, M + 1), i32(v.tiles, 4 * v.max_tiles).reshape(-1, 4)[:ntiles],
            i32(v.order, T * S), v.tile_rows)


def _expected_tiles(counts, offsets, BM=128):
    """The documented tile list: every full tile in expert order, then the partial
    tiles with the most row blocks of 16 first, in expert order within a size."""
    full, part = [], []
    for e, c in enumerate(counts):
        for q in range(c // BM):
            full.append((e, offsets[e] + q * BM, BM, 0))
        if c % BM:
            part.append((8 - (c % BM + 15) // 16, e, (e, offsets[e] + (c // BM) * BM, c % BM, 0)))
    return np.array(full + [t for _, _, t in sorted(part)], dtype=np.int32).reshape(-1, 4)


@pytest.mark.parametrize("name,T", [("prefill512", None), ("prefill4096", None), ("prefill512", 1024),
                                    ("prefill512", 1025)])
def test_prefill_dispatch_readback(gpu, name, T):
    """Counts, offsets and the expert-sorted order that moe_experts_prefill leaves in
    its workspace equal the oracle's bit for bit (ascending pick order within an
    expert); the tile list covers every row once, in the documented order, with
    tiles of 64 rows up to 1024 tokens and 128 above. 1024 tokens are 8192 picks,
    the most that the scatter counts without a count launch; 1025 take the count
    launch, 128-row tiles and the wide router GEMM."""
    c = case(name, T)
    dl = dev_layer(gpu, c)
    L = _L()
    buf = L.alloc_buffers(dl.shape, c.T, "prefill")
    L.layer_step(dl, L.to_device(c.x), buf, "prefill")
    torch.cuda.synchronize()
    counts, offsets, tiles, order, tile_rows = _dispatch_from_ws(gpu, dl.shape, c.T, buf.ws)
    assert tile_rows == (64 if c.T <= 1024 else 128)
    rc, ro, rord = O.dispatch(buf.ids.cpu().numpy(), 256, True)
    assert np.array_equal(counts, rc)
    assert np.array_equal(offsets, ro)
    assert np.array_equal(order, rord)
    assert np.array_equal(tiles, _expected_tiles(rc, ro, tile_rows))


def _prefill_chunks(gpu, dl, x, ids, w, wsh, C):
    """moe_experts_prefill + moe_combine over chunks of C rows with given picks."""
    L = _L()
    T, H = x.shape
    S = dl.shape.slots
    y = torch.empty((T, S, H), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ws = torch.zeros(gpu.moe_prefill_workspace_bytes(dl.shape, C), dtype=torch.uint8, device="cuda")
    for t0 in range(0, T, C):
        n = min(C, T - t0)
        gpu.moe_experts_prefill(dl.shape, dl.experts_prefill, x[t0:t0 + n], n, ids[t0:t0 + n], ws, y[t0:t0 + n])
        gpu.moe_combine(dl.shape, y[t0:t0 + n], w[t0:t0 + n], wsh[t0:t0 + n], n, None, out[t0:t0 + n])
    torch.cuda.synchronize()
    return y.cpu().numpy(), L.bits_to_numpy(out)


def test_prefill_deterministic_and_chunk_invariant(gpu):
    """4096 tokens with skewed routing: two runs are bit-identical, and the slot
    outputs and layer outputs of chunks of 128 and of 16 rows (same picks and
    weights) equal the single call's byte for byte."""
    c = case("prefill4096")
    dl = dev_layer(gpu, c)
    a = run_path(gpu, dl, c.x, "prefill")
    b = run_path(gpu, dl, c.x, "prefill")
    for key in ("logits", "ids", "w", "wsh", "y", "out"):
        assert np.array_equal(a[key], b[key]), key
    L = _L()
    x = L.to_device(c.x)
    ids = torch.from_numpy(a["ids"]).cuda()
    w, wsh = L.to_device(a["w"]), L.to_device(a["wsh"])
    for C in (128, 16):
        y, out = _prefill_chunks(gpu, dl, x, ids, w, wsh, C)
        assert np.array_equal(y.view(np.uint32), a["y"].view(np.uint32)), C
        assert np.array_equal(out, a["out"]), C


def test_prefill_route_chunks_of_128(gpu):
    """Route + experts + combine in chunks of 128 tokens (the router GEMM's smaller
    instance) against one call over 4096 tokens (its larger instance): logits, picks,
    weights, slot outputs and layer outputs are byte-equal."""
    c = case("prefill4096")
    dl = dev_layer(gpu, c)
    full = run_path(gpu, dl, c.x, "prefill")
    for t0 in range(0, c.T, 128):
        part = run_path(gpu, dl, c.x[t0:t0 + 128], "prefill")
        for key in ("logits", "ids", "w", "wsh", "y", "out"):
            assert np.array_equal(part[key], full[key][t0:t0 + 128]), (key, t0)


def _prefill_layout_expected(packed, shape):
    """The prefill layout from the packed buffer, by its documented permutation: in
    every set of 64 consecutive four-row blocks (n blocks in a shorter last set), the
    128-byte line (block j, group g) moves from set + 128 (j G + g) to
    set + 128 (g n + j), and the 16-byte (scale, bias) unit likewise."""
    km = shape.bits // 4
    H, I, M = shape.hidden, shape.inter, shape.n_experts + shape.has_shared
    Hw, Iw = H * km, I * km
    regions = [(0, I // 2, Hw // 64, 128), (I * Hw, H // 4, Iw // 64, 128)]
    sb0 = I * Hw + H * Iw // 2
    regions += [(sb0, I // 2, Hw // 64, 16), (sb0 + (I // 2) * (Hw // 64) * 16, H // 4, Iw // 64, 16)]
    stride = len(packed) // M
    out = packed.copy()
    for m in range(M):
        for base, nblk, G, ub in regions:
            for s0 in range(0, nblk, 64):
                n = min(64, nblk - s0)
                a = m * stride + base + s0 * G * ub
                src = packed[a:a + n * G * ub].reshape(n, G, ub)
                out[a:a + n * G * ub] = src.transpose(1, 0, 2).reshape(-1)
    return out


@pytest.mark.parametrize("name,bits", [("tiny", 4), ("decode", 4), ("tiny", 8)])
def test_prefill_layout_permutation(gpu, name, bits):
    """moe_pack_experts_prefill writes the documented permutation of the packed
    buffer, byte for byte (sets shorter than 64 blocks at 64 intermediate rows,
    several sets at 2048 hidden, 8-bit rows twice as long)."""
    c = synth.make_case(name, bits=bits)
    L = _L()
    dl = L.DeviceLayer(L.make_shape(c.shape), c.layers[0])
    torch.cuda.synchronize()
    packed = dl.experts.cpu().numpy()
    got = dl.experts_prefill.cpu().numpy()
    assert np.array_equal(got, _prefill_layout_expected(packed, c.shape))


# 8-bit routers of other sizes on the matrix cores (T > 16); R = experts + shared gate.
# name: (hidden, n_experts, has_shared)
MC_ROUTER_CASES = {
    "rows17": (256, 16, 1),   # fewer rows than one 32-row block
    "rows49": (512, 48, 1),   # two 16-row blocks past the last whole 32
    "rows64": (512, 64, 0),   # whole 32-row blocks only
    "rows65": (512, 64, 1),   # one 16-row block past the last whole 32, as at 257
}


@pytest.mark.parametrize("name", list(MC_ROUTER_CASES))
def test_matrix_core_router_shapes(gpu, name):
    """The router GEMM's tile shapes (16 tokens x 32 rows up to 1024 tokens, with
    the rows past the last whole 32 in the last row block's workgroup; 32 x 64 and
    32 x 16 above) on routers of other sizes: a token's logits are byte-equal
    between the two, within the matrix-core bar of the oracle's, and the picks and
    weights follow from them."""
    H, E, hs = MC_ROUTER_CASES[name]
    shape = synth.Shape(hidden=H, inter=64, n_experts=E, top_k=2, has_shared=hs, router_fmt=A8)
    host = synth.make_layer(shape, seed=40 + list(MC_ROUTER_CASES).index(name), layer=0)
    L = _L()
    dl = L.DeviceLayer(L.make_shape(shape), host)
    x = synth.random_x(900, 1100, H)
    big = run_path(gpu, dl, x, "prefill")         # above 1024 tokens
    small = run_path(gpu, dl, x[:300], "prefill")  # up to 1024 tokens
    for key in ("logits", "ids", "w", "wsh"):
        if small[key] is not None:
            assert np.array_equal(small[key], big[key][:300]), key
    ref = O.router_logits(x[:300], O.router_matrix(host), host.logit_bias, E)
    check_logits(small["logits"], ref, fp64_path=False)
    check_picks(small["ids"], ref, 2, E)
    staged_route_check(gpu, small, E, 2, has_shared=bool(hs))


@pytest.mark.parametrize("name,T,bits", [("decode", 1, 4), ("decode", 3, 4), ("decode", 16, 4), ("tiny", 1, 4),
                                         ("tiny", 4, 4), ("decode", 2, 8)])
def test_decode_block_equals_norm_then_layer(gpu, name, T, bits):
    """moe_decode_block (RMSNorm folded into the single-launch layer, residual add)
    gives the same bits as moe_rmsnorm followed by moe_decode_layer with residual,
    over repeated launches; x is left unchanged."""
    L = _L()
    c = synth.make_case(name, bits=bits, seed=40 + T)
    dl = L.DeviceLayer(L.make_shape(c.shape), c.layers[0])
    H = c.shape.hidden
    x_np = synth.random_x(1300 + T, T, H)
    x = L.to_device(x_np)
    xn = torch.empty_like(x)
    a = L.alloc_buffers(dl.shape, T, "fused")
    b = L.alloc_buffers(dl.shape, T, "fused")
    staged_out = torch.empty_like(x)
    gpu.moe_rmsnorm(H, x, T, 1e-6, xn)
    L.layer_step(dl, xn, a, "fused", residual=x, out=staged_out)
    x_out = torch.empty_like(x)
    for _ in range(2):
        gpu.moe_decode_block(dl.shape, dl.router, dl.logit_bias, dl.experts, x, T, 1e-6, b.ws, b.logits, b.ids, b.w,
                             b.wsh, b.y, x_out)
    torch.cuda.synchronize()
    assert np.array_equal(L.bits_to_numpy(x), x_np)
    assert np.array_equal(L.bits_to_numpy(x_out), L.bits_to_numpy(staged_out))
    for key in ("logits", "ids", "w", "wsh", "y"):
        assert np.array_equal(getattr(a, key).cpu().numpy(), getattr(b, key).cpu().numpy()), key
    assert gpu.moe_decode_layer_check(dl.shape, T, b.ws)
    with pytest.raises(Exception):
        gpu.moe_decode_block(dl.shape, dl.router, dl.logit_bias, dl.experts, x, T, 1e-6, b.ws, b.logits, b.ids, b.w,
                             b.wsh, b.y, x)  # x_out aliasing x is refused

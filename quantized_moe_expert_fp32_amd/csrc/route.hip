// Router logits and top-k selection (routing contract of TensorFold issue #931,
// "What I'd build"; a wavefront-parallel replacement of a serial top-k softmax as
// in the AGX Orin port's "Phase 1-4").
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------- logits, GEMV form
// One wavefront per router row r and chunk of TT tokens. Lane l reads the four
// router elements [4l + 256i, +4) of the row (coalesced 256-byte lines for the
// 8-bit router) and the matching activations of each token; products are exact
// in fp64 and accumulate in fp64 in a fixed order (lane-sequential, then a
// butterfly), so a token's logits do not depend on T or on the other tokens.
template <int TT, bool AFF8>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint8_t* __restrict__ router,
                                                            const float* __restrict__ logit_bias,
                                                            const uint16_t* __restrict__ x, int T, int H,
                                                            int R, int E, float* __restrict__ logits) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + wave;
    if (r >= R) return;  // wave-uniform; no block barriers below
    const int t0 = blockIdx.y * TT;
    const int nt = min(TT, T - t0);
    double acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.0;

    const uint32_t* sb = reinterpret_cast<const uint32_t*>(router + (size_t)R * H);
    for (int c0 = lane * 4; c0 < H; c0 += 256) {
        double w[4];
        if (AFF8) {
            const uint32_t q = *reinterpret_cast<const uint32_t*>(router + (size_t)r * H + c0);
            const uint32_t g = sb[(size_t)r * (H / 64) + (c0 >> 6)];
            const double s = (double)bf16_to_f32(g & 0xFFFFu), b = (double)bf16_to_f32(g >> 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = s * (double)((q >> (8 * j)) & 0xFFu) + b;  // exact
        } else {
            const float4 v = *reinterpret_cast<const float4*>(
                reinterpret_cast<const float*>(router) + (size_t)r * H + c0);
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        }
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            if (t < nt) {
                const uint2 xv = *reinterpret_cast<const uint2*>(x + (size_t)(t0 + t) * H + c0);
                acc[t] = fma((double)bf16_to_f32(xv.x & 0xFFFFu), w[0], acc[t]);
                acc[t] = fma((double)bf16_to_f32(xv.x >> 16), w[1], acc[t]);
                acc[t] = fma((double)bf16_to_f32(xv.y & 0xFFFFu), w[2], acc[t]);
                acc[t] = fma((double)bf16_to_f32(xv.y >> 16), w[3], acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) acc[t] += __shfl_xor(acc[t], off);
    }
    if (lane == 0) {
        const double bias = (r < E && logit_bias) ? (double)logit_bias[r] : 0.0;
#pragma unroll
        for (int t = 0; t < TT; ++t)
            if (t < nt) logits[(size_t)(t0 + t) * R + r] = (float)(acc[t] + bias);
    }
}

// ---------------------------------------------------------------- selection
// One wavefront per token. Each lane holds VPL keys (ordered logit << 32 | ~id);
// k rounds of a wave-wide max pick the experts in descending logit, ties to the
// lower id. Weights: exp(l_i - l_0) in fp64, summed over the picks in slot order,
// divided and rounded once to bf16. Shared weight: bf16(sigmoid(bf16(gate))) in fp64.
template <int VPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int R, int E, int k,
                                                   int has_shared, int32_t* __restrict__ ids,
                                                   uint16_t* __restrict__ w, uint16_t* __restrict__ wsh) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    const float* lr = logits + (size_t)t * R;
    uint64_t key[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        const int e = lane + 64 * j;
        key[j] = e < E ? ((uint64_t)ordered_logit(lr[e]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e) : 0ull;
    }
    uint32_t my_id = 0;
    for (int i = 0; i < k; ++i) {
        uint64_t best = 0;
#pragma unroll
        for (int j = 0; j < VPL; ++j) best = key[j] > best ? key[j] : best;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const uint64_t o = __shfl_xor(best, off);
            best = o > best ? o : best;
        }
#pragma unroll
        for (int j = 0; j < VPL; ++j)
            if (key[j] == best) key[j] = 0;
        if (lane == i) my_id = 0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull);
    }
    my_id = my_id < (uint32_t)E ? my_id : (uint32_t)(E - 1);  // k <= E valid keys always exist
    const double li = lane < k ? (double)lr[my_id] : 0.0;
    const double l0 = __shfl(li, 0);
    const double ex = lane < k ? exp(li - l0) : 0.0;
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += __shfl(ex, j);
    if (lane < k) {
        ids[(size_t)t * k + lane] = (int32_t)my_id;
        w[(size_t)t * k + lane] = (uint16_t)f64_to_bf16(ex / sum);
    }
    if (has_shared && lane == 0) {
        const double g = (double)bf16_to_f32(f32_to_bf16(lr[E]));
        wsh[t] = (uint16_t)f64_to_bf16(1.0 / (1.0 + exp(-g)));
    }
}

static moe_status launch_topk(const moe_shape& sh, const float* logits, int T, int32_t* ids, uint16_t* w,
                              uint16_t* wsh, hipStream_t st) {
    const int R = router_rows(sh), E = sh.n_experts;
    const int vpl = (E + 63) / 64;
    dim3 grid((T + 3) / 4), block(256);
#define MOE_TOPK(V)                                                                                            \
    hipLaunchKernelGGL(topk_kernel<V>, grid, block, 0, st, logits, T, R, E, sh.top_k, sh.has_shared, ids, w, wsh)
    if (vpl <= 1) MOE_TOPK(1);
    else if (vpl <= 2) MOE_TOPK(2);
    else if (vpl <= 4) MOE_TOPK(4);
    else if (vpl <= 8) MOE_TOPK(8);
    else MOE_TOPK(16);
#undef MOE_TOPK
    return check_launch("topk_kernel");
}

template <int TT>
static void launch_logits_tt(const moe_shape& sh, const uint8_t* router, const float* bias, const uint16_t* x, int T,
                             float* logits, hipStream_t st) {
    const int R = router_rows(sh);
    dim3 grid((R + 3) / 4, (T + TT - 1) / TT), block(256);
    if (sh.router_fmt == MOE_ROUTER_AFFINE8)
        hipLaunchKernelGGL((router_logits_kernel<TT, true>), grid, block, 0, st, router, bias, x, T, sh.hidden, R,
                           sh.n_experts, logits);
    else
        hipLaunchKernelGGL((router_logits_kernel<TT, false>), grid, block, 0, st, router, bias, x, T, sh.hidden, R,
                           sh.n_experts, logits);
}

static moe_status check_route_outputs(const moe_shape& sh, int T, const int32_t* ids, const uint16_t* w,
                                      const uint16_t* wsh) {
    if (T < 1) return fail(MOE_ERR_INVALID_ARG, "T = %d, need T >= 1", T);
    if (!ids || !w) return fail(MOE_ERR_INVALID_ARG, "ids or w is NULL");
    if (sh.has_shared && !wsh) return fail(MOE_ERR_INVALID_ARG, "w_shared is NULL with a shared expert");
    if (!sh.has_shared && wsh) return fail(MOE_ERR_INVALID_ARG, "w_shared given without a shared expert");
    return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_route(const moe_shape* shape, const void* router_packed, const float* logit_bias,
                                const uint16_t* x, int32_t T, float* logits, int32_t* ids, uint16_t* w,
                                uint16_t* w_shared, void* stream) {
    clear_error();
    moe_status st = validate_shape(shape);
    if (st != MOE_OK) return st;
    if ((st = check_route_outputs(*shape, T, ids, w, w_shared)) != MOE_OK) return st;
    if (!router_packed || !x || !logits || !aligned16(router_packed) || !aligned16(x))
        return fail(MOE_ERR_INVALID_ARG, "router, x or logits NULL or unaligned");
    hipStream_t hs = (hipStream_t)stream;
    const uint8_t* r = (const uint8_t*)router_packed;
    if (T <= 1) launch_logits_tt<1>(*shape, r, logit_bias, x, T, logits, hs);
    else if (T <= 2) launch_logits_tt<2>(*shape, r, logit_bias, x, T, logits, hs);
    else if (T <= 4) launch_logits_tt<4>(*shape, r, logit_bias, x, T, logits, hs);
    else if (T <= 8) launch_logits_tt<8>(*shape, r, logit_bias, x, T, logits, hs);
    else launch_logits_tt<16>(*shape, r, logit_bias, x, T, logits, hs);
    if ((st = check_launch("router_logits_kernel")) != MOE_OK) return st;
    return launch_topk(*shape, logits, T, ids, w, w_shared, hs);
}

extern "C" moe_status moe_route_from_logits(const moe_shape* shape, const float* logits, int32_t T, int32_t* ids,
                                            uint16_t* w, uint16_t* w_shared, void* stream) {
    clear_error();
    moe_status st = validate_shape(shape);
    if (st != MOE_OK) return st;
    if ((st = check_route_outputs(*shape, T, ids, w, w_shared)) != MOE_OK) return st;
    if (!logits) return fail(MOE_ERR_INVALID_ARG, "logits is NULL");
    return launch_topk(*shape, logits, T, ids, w, w_shared, (hipStream_t)stream);
}

// Router logits and top-k selection (routing contract of TensorFold issue #931,
// "What I'd build"; a wavefront-parallel replacement of a serial top-k softmax as
// in the AGX Orin port's "Phase 1-4").
#include "moe_internal.h"
#include "route_internal.h"

namespace moe {

// ---------------------------------------------------------------- selection of one token
// One wavefront. Each lane holds VPL keys (ordered logit << 32 | ~id); k rounds of
// a wave-wide max pick the experts in descending logit, ties to the lower id.
// Weights: exp(l_i - l_0) in fp64, summed over the picks in slot order, divided
// and rounded once to bf16. Shared weight: bf16(sigmoid(bf16(gate))) in fp64.
template <int VPL>
__device__ __forceinline__ void select_token(const float* lr, int t, int E, int k, int has_shared, int lane,
                                             int32_t* __restrict__ ids, uint16_t* __restrict__ w,
                                             uint16_t* __restrict__ wsh) {
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

template <int VPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int R, int E, int k,
                                                   int has_shared, int32_t* __restrict__ ids,
                                                   uint16_t* __restrict__ w, uint16_t* __restrict__ wsh) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    select_token<VPL>(logits + (size_t)t * R, t, E, k, has_shared, lane, ids, w, wsh);
}

// ---------------------------------------------------------------- logits, GEMV form
// One wavefront per router row r and chunk of TT tokens. A lane reads 16-byte
// chunks of the row (16 int8 weights, or 4 fp32 weights) at chunk index
// lane + 64 i, so every load instruction covers 1 KiB of the row contiguously.
// Products are exact in fp64 and accumulate in fp64 in a fixed order
// (lane-sequential, then a butterfly), so a token's logits do not depend on T or
// on the other tokens.
//
// FUSE: the launch covers every token (TT >= T); after writing its logits each
// workgroup publishes them (agent-scope fence) and counts itself done on
// `counter`; the last one to finish runs the selection for every token and
// resets the counter to zero. No workgroup ever waits for another.
template <int TT, bool AFF8, bool FUSE>
__global__ __launch_bounds__(256) void router_kernel(const uint8_t* __restrict__ router,
                                                     const float* __restrict__ logit_bias,
                                                     const uint16_t* __restrict__ x, int T, int H, int R, int E,
                                                     float* logits, unsigned int* counter, int k, int has_shared,
                                                     int32_t* __restrict__ ids, uint16_t* __restrict__ w,
                                                     uint16_t* __restrict__ wsh) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + wave;
    const int t0 = blockIdx.y * TT;
    const int nt = min(TT, T - t0);
    if (r < R) {
        double acc[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[t] = 0.0;
        constexpr int EPC = AFF8 ? 16 : 4;  // elements per 16-byte chunk
        const int C = H / EPC;
        const uint32_t* sb = reinterpret_cast<const uint32_t*>(router + (size_t)R * H);
        for (int j = lane; j < C; j += 64) {
            const int c0 = j * EPC;
            double wv[EPC];
            if constexpr (AFF8) {
                const uint4 q = *reinterpret_cast<const uint4*>(router + (size_t)r * H + c0);
                const uint32_t g = sb[(size_t)r * (H / 64) + (c0 >> 6)];
                const double s = (double)bf16_to_f32(g & 0xFFFFu), b = (double)bf16_to_f32(g >> 16);
                const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int i = 0; i < EPC; ++i) wv[i] = s * (double)((qw[i >> 2] >> (8 * (i & 3))) & 0xFFu) + b;
            } else {
                const float4 v = *reinterpret_cast<const float4*>(
                    reinterpret_cast<const float*>(router) + (size_t)r * H + c0);
                wv[0] = v.x; wv[1] = v.y; wv[2] = v.z; wv[3] = v.w;
            }
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                if (t < nt) {
                    const uint16_t* xr = x + (size_t)(t0 + t) * H + c0;
                    uint32_t xw[EPC / 2];
                    if constexpr (AFF8) {
                        const uint4 a = *reinterpret_cast<const uint4*>(xr);
                        const uint4 b = *reinterpret_cast<const uint4*>(xr + 8);
                        xw[0] = a.x; xw[1] = a.y; xw[2] = a.z; xw[3] = a.w;
                        xw[4] = b.x; xw[5] = b.y; xw[6] = b.z; xw[7] = b.w;
                    } else {
                        const uint2 a = *reinterpret_cast<const uint2*>(xr);
                        xw[0] = a.x; xw[1] = a.y;
                    }
#pragma unroll
                    for (int i = 0; i < EPC; ++i) {
                        const uint32_t bits = (i & 1) ? (xw[i >> 1] >> 16) : (xw[i >> 1] & 0xFFFFu);
                        acc[t] = fma((double)bf16_to_f32(bits), wv[i], acc[t]);
                    }
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
    if (FUSE) {
        __shared__ int am_last;
        __threadfence();
        __syncthreads();
        if (threadIdx.x == 0) am_last = atomicAdd(counter, 1u) == gridDim.x * gridDim.y - 1;
        __syncthreads();
        if (!am_last) return;
        __threadfence();
        const int vpl = (E + 63) / 64;
        for (int t = wave; t < T; t += 4) {
            const float* lr = logits + (size_t)t * R;
            if (vpl <= 1) select_token<1>(lr, t, E, k, has_shared, lane, ids, w, wsh);
            else if (vpl <= 2) select_token<2>(lr, t, E, k, has_shared, lane, ids, w, wsh);
            else if (vpl <= 4) select_token<4>(lr, t, E, k, has_shared, lane, ids, w, wsh);
            else if (vpl <= 8) select_token<8>(lr, t, E, k, has_shared, lane, ids, w, wsh);
            else select_token<16>(lr, t, E, k, has_shared, lane, ids, w, wsh);
        }
        if (threadIdx.x == 0) atomicExch(counter, 0u);
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

template <int TT, bool FUSE>
static void launch_router_tt(const moe_shape& sh, const uint8_t* router, const float* bias, const uint16_t* x, int T,
                             float* logits, unsigned int* counter, int32_t* ids, uint16_t* w, uint16_t* wsh,
                             hipStream_t st) {
    const int R = router_rows(sh);
    dim3 grid((R + 3) / 4, (T + TT - 1) / TT), block(256);
    if (sh.router_fmt == MOE_ROUTER_AFFINE8)
        hipLaunchKernelGGL((router_kernel<TT, true, FUSE>), grid, block, 0, st, router, bias, x, T, sh.hidden, R,
                           sh.n_experts, logits, counter, sh.top_k, sh.has_shared, ids, w, wsh);
    else
        hipLaunchKernelGGL((router_kernel<TT, false, FUSE>), grid, block, 0, st, router, bias, x, T, sh.hidden, R,
                           sh.n_experts, logits, counter, sh.top_k, sh.has_shared, ids, w, wsh);
}

template <bool FUSE>
static void launch_router(const moe_shape& sh, const uint8_t* r, const float* bias, const uint16_t* x, int T,
                          float* logits, unsigned int* counter, int32_t* ids, uint16_t* w, uint16_t* wsh,
                          hipStream_t hs) {
    if (T <= 1) launch_router_tt<1, FUSE>(sh, r, bias, x, T, logits, counter, ids, w, wsh, hs);
    else if (T <= 2) launch_router_tt<2, FUSE>(sh, r, bias, x, T, logits, counter, ids, w, wsh, hs);
    else if (T <= 4) launch_router_tt<4, FUSE>(sh, r, bias, x, T, logits, counter, ids, w, wsh, hs);
    else if (T <= 8) launch_router_tt<8, FUSE>(sh, r, bias, x, T, logits, counter, ids, w, wsh, hs);
    else launch_router_tt<16, FUSE>(sh, r, bias, x, T, logits, counter, ids, w, wsh, hs);
}

moe_status check_route_outputs(const moe_shape& sh, int T, const int32_t* ids, const uint16_t* w,
                               const uint16_t* wsh) {
    if (T < 1) return fail(MOE_ERR_INVALID_ARG, "T = %d, need T >= 1", T);
    if (!ids || !w) return fail(MOE_ERR_INVALID_ARG, "ids or w is NULL");
    if (sh.has_shared && !wsh) return fail(MOE_ERR_INVALID_ARG, "w_shared is NULL with a shared expert");
    if (!sh.has_shared && wsh) return fail(MOE_ERR_INVALID_ARG, "w_shared given without a shared expert");
    return MOE_OK;
}

moe_status launch_route_fused(const moe_shape& sh, const void* router_packed, const float* logit_bias,
                              const uint16_t* x, int T, float* logits, unsigned int* counter, int32_t* ids,
                              uint16_t* w, uint16_t* wsh, hipStream_t hs) {
    launch_router<true>(sh, (const uint8_t*)router_packed, logit_bias, x, T, logits, counter, ids, w, wsh, hs);
    return check_launch("router_kernel (fused selection)");
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
    launch_router<false>(*shape, (const uint8_t*)router_packed, logit_bias, x, T, logits, nullptr, ids, w, w_shared,
                         hs);
    if ((st = check_launch("router_kernel")) != MOE_OK) return st;
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

// Router logits and top-k selection (routing contract of TensorFold issue #931,
// "What I'd build"; a wavefront-parallel replacement of a serial top-k softmax as
// in the AGX Orin port's "Phase 1-4").
#include "mfma_common.h"
#include "moe_internal.h"
#include "route_device.h"
#include "route_internal.h"

namespace moe {

template <int VPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int R, int E, int k,
                                                   int has_shared, int32_t* __restrict__ ids,
                                                   uint16_t* __restrict__ w, uint16_t* __restrict__ wsh) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    const LogitSrc src{logits + (size_t)t * R, nullptr, 0u, nullptr, false};
    select_token<VPL>(src, E, k, has_shared, lane, ids + (size_t)t * k, w + (size_t)t * k, wsh ? wsh + t : nullptr);
}

// One wavefront per router row r and chunk of TT tokens (see router_row).
// FUSE: the launch covers every token (TT >= T); after writing its logits each
// workgroup publishes them (coherent stores, completed) and counts itself done on
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
    if (r < R) router_row<TT, AFF8>(router, logit_bias, x, t0, nt, H, R, E, r, lane, logits, FUSE, nullptr, 0u);
    if (FUSE) {
        __shared__ int am_last;
        publish_fence();
        __syncthreads();
        if (threadIdx.x == 0) am_last = atomicAdd(counter, 1u) == gridDim.x * gridDim.y - 1;
        __syncthreads();
        if (!am_last) return;
        for (int t = wave; t < T; t += 4) {
            const LogitSrc src{logits + (size_t)t * R, nullptr, 0u, nullptr, true};
            select_token_any(src, E, k, has_shared, lane, ids + (size_t)t * k, w + (size_t)t * k,
                             wsh ? wsh + t : nullptr);
        }
        if (threadIdx.x == 0) atomicExch(counter, 0u);
    }
}

// ---------------------------------------------------------------- logits, GEMM form (8-bit router, T > 16)
// logits[t][r] = sum_g ( s[r][g] * sum_{k in g} x[t][k] q[r][k] + b[r][g] * sum_{k in g} x[t][k] ) (+ bias[r])
// on the matrix cores: the int8 codes are exact bf16 operands, each 64-wide
// group's partial comes from two v_mfma_f32_16x16x32_bf16, and scale and bias are
// applied in fp32 per group. Grid (ceil(T / 64), ceil(R / 64)); wavefront w owns
// router rows nb*64 + 16w .. +16 for the block's 64 tokens. Activation groups are
// loaded two groups ahead and staged in LDS (double-buffered); weights are
// loaded four groups ahead into a register ring.
__global__ __launch_bounds__(256) void router_gemm_kernel(const uint8_t* __restrict__ router,
                                                          const float* __restrict__ logit_bias,
                                                          const uint16_t* __restrict__ x, int T, int H, int R, int E,
                                                          float* __restrict__ logits) {
    __shared__ __attribute__((aligned(16))) uint16_t a_lds[2][64 * A_STRIDE];
    __shared__ __attribute__((aligned(16))) float x_lds[2][64];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lg = lane >> 4, lc = lane & 15;
    const int m0 = blockIdx.x * 64;
    const int nrows = min(64, T - m0);
    const int n_ms = (nrows + 15) >> 4;
    const int r = blockIdx.y * 64 + wave * 16 + lc;
    const bool r_ok = r < R;
    const uint8_t* qrow = router + (size_t)(r_ok ? r : 0) * H + 8 * lg;
    const uint32_t* sbrow = reinterpret_cast<const uint32_t*>(router + (size_t)R * H) + (size_t)(r_ok ? r : 0) * (H / 64);
    const int srow = tid >> 2, sq = tid & 3;
    const bool srow_ok = srow < nrows;
    const uint16_t* xsrc = x + (size_t)(m0 + (srow_ok ? srow : 0)) * H + 16 * sq;

    f32x4_t acc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int G = H / 64;
    constexpr int PDR = 4;  // weight groups in flight
    uint2 wq[PDR][2];
    uint32_t ws[PDR];
#pragma unroll
    for (int u = 0; u < PDR; ++u) {
        if (u < G) {
            wq[u][0] = *reinterpret_cast<const uint2*>(qrow + 64 * u);
            wq[u][1] = *reinterpret_cast<const uint2*>(qrow + 64 * u + 32);
            ws[u] = sbrow[u];
        }
    }
    uint4 xr[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) xr[i][0] = xr[i][1] = make_uint4(0, 0, 0, 0);
    if (srow_ok) {
        xr[0][0] = *reinterpret_cast<const uint4*>(xsrc);
        xr[0][1] = *reinterpret_cast<const uint4*>(xsrc + 8);
        if (G > 1) {
            xr[1][0] = *reinterpret_cast<const uint4*>(xsrc + 64);
            xr[1][1] = *reinterpret_cast<const uint4*>(xsrc + 72);
        }
    }
    stage_store(a_lds[0], x_lds[0], tid, xr[0][0], xr[0][1]);
    __syncthreads();
    for (int g0 = 0; g0 < G; g0 += PDR) {
#pragma unroll
        for (int u = 0; u < PDR; ++u) {
            const int g = g0 + u;
            if (g >= G) break;  // uniform
            if (g + 2 < G && srow_ok) {
                xr[u & 1][0] = *reinterpret_cast<const uint4*>(xsrc + 64 * (g + 2));
                xr[u & 1][1] = *reinterpret_cast<const uint4*>(xsrc + 64 * (g + 2) + 8);
            }
            const uint4 b0 = int8x8_to_bf16_pairs(wq[u][0].x, wq[u][0].y);
            const uint4 b1 = int8x8_to_bf16_pairs(wq[u][1].x, wq[u][1].y);
            const float sc = bf16_to_f32(ws[u] & 0xFFFFu), bi = bf16_to_f32(ws[u] >> 16);
            if (g + PDR < G) {
                wq[u][0] = *reinterpret_cast<const uint2*>(qrow + 64 * (g + PDR));
                wq[u][1] = *reinterpret_cast<const uint2*>(qrow + 64 * (g + PDR) + 32);
                ws[u] = sbrow[g + PDR];
            }
            const uint16_t* al = a_lds[u & 1];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                if (m < n_ms) {
                    const uint4 a0 = *reinterpret_cast<const uint4*>(al + (16 * m + lc) * A_STRIDE + 8 * lg);
                    const uint4 a1 = *reinterpret_cast<const uint4*>(al + (16 * m + lc) * A_STRIDE + 32 + 8 * lg);
                    const float4 xs = *reinterpret_cast<const float4*>(&x_lds[u & 1][16 * m + 4 * lg]);
                    f32x4_t p = mfma16x16x32(a0, b0, f32x4_t{0.f, 0.f, 0.f, 0.f});
                    p = mfma16x16x32(a1, b1, p);
                    acc[m][0] = fmaf(bi, xs.x, fmaf(sc, p[0], acc[m][0]));
                    acc[m][1] = fmaf(bi, xs.y, fmaf(sc, p[1], acc[m][1]));
                    acc[m][2] = fmaf(bi, xs.z, fmaf(sc, p[2], acc[m][2]));
                    acc[m][3] = fmaf(bi, xs.w, fmaf(sc, p[3], acc[m][3]));
                }
            }
            if (g + 1 < G) stage_store(a_lds[(u + 1) & 1], x_lds[(u + 1) & 1], tid, xr[(u + 1) & 1][0],
                                       xr[(u + 1) & 1][1]);
            __syncthreads();
        }
    }
    if (!r_ok) return;
    const float bias = (r < E && logit_bias) ? logit_bias[r] : 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * m + 4 * lg + i;
            if (row < nrows) logits[(size_t)(m0 + row) * R + r] = acc[m][i] + bias;
        }
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
    if (T > 16 && shape->router_fmt == MOE_ROUTER_AFFINE8) {
        const int R = router_rows(*shape);
        hipLaunchKernelGGL(router_gemm_kernel, dim3((T + 63) / 64, (R + 63) / 64), dim3(256), 0, hs,
                           (const uint8_t*)router_packed, logit_bias, x, T, shape->hidden, R, shape->n_experts, logits);
        if ((st = check_launch("router_gemm_kernel")) != MOE_OK) return st;
    } else {
        launch_router<false>(*shape, (const uint8_t*)router_packed, logit_bias, x, T, logits, nullptr, ids, w,
                             w_shared, hs);
        if ((st = check_launch("router_kernel")) != MOE_OK) return st;
    }
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

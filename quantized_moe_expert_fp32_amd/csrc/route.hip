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
constexpr int RG_TOK = 32;  // tokens per workgroup above 1024 tokens
// logits[t][r] = sum_g ( s[r][g] * sum_{k in g} x[t][k] q[r][k] + b[r][g] * sum_{k in g} x[t][k] ) (+ bias[r])
// on the matrix cores. A workgroup takes 16 MB tokens x 16 NB router rows; wavefront
// w takes the groups [w G/4, (w+1) G/4) of K and its partial sums are added in
// wavefront order at the end, so the result does not depend on timing. Per group,
// 16-token block and 16 rows:
//   * the int8 codes are exact bf16 B operands; lane (row lc, quarter lg) holds
//     codes 16 lg .. 16 lg + 15 of its row, the first 8 for one
//     v_mfma_f32_16x16x32_bf16 and the last 8 for the next, and the A operand
//     carries the matching activations (any assignment of k to MFMA slots gives
//     the same sum), so both operands are single contiguous loads;
//   * the scale multiplies the group's partial in fp32 (one FMA per output);
//   * the bias term b * sum x comes from two more MFMAs whose B operand is b in
//     every slot (exact products, fp32 sums), accumulated in place.
// Every (16-token block, 16-row block) pair goes through the same operations
// whatever MB and NB are, so a logit does not depend on the tile shape.
// Operands come straight from global memory into a ring of PD groups per
// wavefront: no LDS and no barrier in the loop.
//
// Tile shapes. A workgroup's first loads wait on address translation: each 4 KiB
// page it touches for the first time (an activation row is one page, two router
// rows share one) costs it about 0.1 us, and that, not bytes or instructions,
// sets most of its time (a timing-only build whose loads hit three pages per
// workgroup ran 3.9 instead of 7.8 us per workgroup at 512 tokens; one page per
// load instruction but the same pages was as slow as the real one). Up to 1024
// tokens a workgroup takes 16 tokens x 32 rows (about 36 pages with its logit
// stores, against 48 for 32 x 16), and the rows past the last whole 32, the
// shared gate's, join the last row block's workgroup, so 512 tokens take exactly
// 256 workgroups. Thousands of tokens: 32 tokens x 64 rows, which reads the
// activations a quarter as often.
template <int MB, int NB>
__device__ __forceinline__ void router_gemm_tile(const uint8_t* __restrict__ router,
                                                 const float* __restrict__ logit_bias,
                                                 const uint16_t* __restrict__ x, int T, int H, int R, int E,
                                                 float* __restrict__ logits, int t0, int rb0,
                                                 float (*part)[MB][NB][4][64]) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lg = lane >> 4, lc = lane & 15;
    const int rb = rb0 + lc;
    const int G = H / 64, ga = wave * G / 4, gb = (wave + 1) * G / 4;
    const uint8_t* qrow[NB];
    const uint32_t* sbrow[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) {
        const int r = rb + 16 * n, rr = r < R ? r : 0;
        qrow[n] = router + (size_t)rr * H + 16 * lg;
        sbrow[n] = reinterpret_cast<const uint32_t*>(router + (size_t)R * H) + (size_t)rr * G;
    }
    const uint16_t* xrow[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        const int t = t0 + 16 * m + lc;
        xrow[m] = x + (size_t)(t < T ? t : 0) * H + 16 * lg;
    }
    f32x4_t acc[MB][NB];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    constexpr int PD = MB * NB <= 2 ? 4 : 3;  // groups in flight per wavefront
    uint4 wq[PD][NB], xa[PD][MB][2];
    uint32_t ws[PD][NB];
    auto load = [&](int u, int g) {
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            wq[u][n] = *reinterpret_cast<const uint4*>(qrow[n] + 64 * g);
            ws[u][n] = sbrow[n][g];
        }
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            xa[u][m][0] = *reinterpret_cast<const uint4*>(xrow[m] + 64 * g);
            xa[u][m][1] = *reinterpret_cast<const uint4*>(xrow[m] + 64 * g + 8);
        }
    };
#pragma unroll
    for (int u = 0; u < PD; ++u)
        if (ga + u < gb) load(u, ga + u);
    for (int g = ga; g < gb; g += PD) {
#pragma unroll
        for (int u = 0; u < PD; ++u) {
            const int gg = g + u;
            if (gg >= gb) break;  // uniform
            uint4 b0[NB], b1[NB], bb[NB];
            float sc[NB];
#pragma unroll
            for (int n = 0; n < NB; ++n) {
                b0[n] = int8x8_to_bf16_pairs(wq[u][n].x, wq[u][n].y);
                b1[n] = int8x8_to_bf16_pairs(wq[u][n].z, wq[u][n].w);
                sc[n] = bf16_to_f32(ws[u][n] & 0xFFFFu);
                const uint32_t bp = (ws[u][n] >> 16) | (ws[u][n] & 0xFFFF0000u);
                bb[n] = make_uint4(bp, bp, bp, bp);
            }
            uint4 a[MB][2];
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                a[m][0] = xa[u][m][0];
                a[m][1] = xa[u][m][1];
            }
            if (gg + PD < gb) load(u, gg + PD);
#pragma unroll
            for (int m = 0; m < MB; ++m) {
#pragma unroll
                for (int n = 0; n < NB; ++n) {
                    f32x4_t p = mfma16x16x32(a[m][0], b0[n], f32x4_t{0.f, 0.f, 0.f, 0.f});
                    p = mfma16x16x32(a[m][1], b1[n], p);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[m][n][i] = fmaf(sc[n], p[i], acc[m][n][i]);
                    acc[m][n] = mfma16x16x32(a[m][0], bb[n], acc[m][n]);
                    acc[m][n] = mfma16x16x32(a[m][1], bb[n], acc[m][n]);
                }
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) part[wave][m][n][i][lane] = acc[m][n][i];
    __syncthreads();
    // the reduction and stores are spread over the four wavefronts: row block n goes
    // to wavefront n % 4
#pragma unroll
    for (int n = 0; n < NB; ++n) {
        if (wave != (n & 3)) continue;
        const int r = rb + 16 * n;
        if (r >= R) continue;
        const float bias = (r < E && logit_bias) ? logit_bias[r] : 0.f;
#pragma unroll
        for (int m = 0; m < MB; ++m) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + 16 * m + 4 * lg + i;
                const float v = ((part[0][m][n][i][lane] + part[1][m][n][i][lane]) + part[2][m][n][i][lane]) +
                                part[3][m][n][i][lane];
                if (t < T) logits[(size_t)t * R + r] = v + bias;
            }
        }
    }
}

// Up to 1024 tokens: 16 tokens x 32 rows per workgroup; blockIdx.y = n32 - 1 also
// takes the rows past the last whole 32 (one or two more blocks of 16), and with
// fewer than 32 rows one workgroup per token block takes them all.
__global__ __launch_bounds__(256) void router_gemm_narrow_kernel(const uint8_t* __restrict__ router,
                                                                const float* __restrict__ logit_bias,
                                                                const uint16_t* __restrict__ x, int T, int H, int R,
                                                                int E, float* __restrict__ logits) {
    __shared__ float part[4][1][4][4][64];
    const int n32 = R / 32, extra = (R % 32 + 15) / 16;  // extra: blocks of 16 past the last whole 32
    const int t0 = blockIdx.x * 16, y = blockIdx.y, rb0 = 32 * y;
    auto run = [&](auto nb_tag) __attribute__((always_inline)) {
        constexpr int NB = decltype(nb_tag)::value;
        router_gemm_tile<1, NB>(router, logit_bias, x, T, H, R, E, logits, t0, rb0,
                                reinterpret_cast<float (*)[1][NB][4][64]>(&part[0][0][0][0][0]));
    };
    const int nb = y + 1 < n32 ? 2 : (n32 > 0 ? 2 : 0) + extra;  // 1 .. 4
    if (nb == 1) run(std::integral_constant<int, 1>{});
    else if (nb == 2) run(std::integral_constant<int, 2>{});
    else if (nb == 3) run(std::integral_constant<int, 3>{});
    else run(std::integral_constant<int, 4>{});
}

// Thousands of tokens: row blocks of 64 (NB = 4) up to the last whole one, then
// blocks of 16 for the rows left over (the shared gate's at 256 experts), so that a
// block of 64 mostly empty rows does not take a round of workgroups of its own.
__global__ __launch_bounds__(256) void router_gemm_wide_kernel(const uint8_t* __restrict__ router,
                                                              const float* __restrict__ logit_bias,
                                                              const uint16_t* __restrict__ x, int T, int H, int R,
                                                              int E, float* __restrict__ logits) {
    __shared__ float part[4][2][4][4][64];
    const int n64 = R / 64;
    if ((int)blockIdx.y < n64)
        router_gemm_tile<2, 4>(router, logit_bias, x, T, H, R, E, logits, blockIdx.x * RG_TOK, blockIdx.y * 64, part);
    else
        router_gemm_tile<2, 1>(router, logit_bias, x, T, H, R, E, logits, blockIdx.x * RG_TOK,
                               64 * n64 + 16 * ((int)blockIdx.y - n64),
                               reinterpret_cast<float (*)[2][1][4][64]>(&part[0][0][0][0][0]));
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
        if (T <= 1024)
            hipLaunchKernelGGL(router_gemm_narrow_kernel, dim3((T + 15) / 16, R >= 32 ? R / 32 : 1), dim3(256), 0, hs,
                               (const uint8_t*)router_packed, logit_bias, x, T, shape->hidden, R, shape->n_experts,
                               logits);
        else
            hipLaunchKernelGGL(router_gemm_wide_kernel, dim3((T + RG_TOK - 1) / RG_TOK, R / 64 + (R % 64 + 15) / 16),
                               dim3(256), 0, hs, (const uint8_t*)router_packed, logit_bias, x, T, shape->hidden, R,
                               shape->n_experts, logits);
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

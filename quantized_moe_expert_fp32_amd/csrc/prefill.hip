// Prefill path: dispatch of the T*S picks into expert-sorted rows, then two
// grouped GEMMs on the matrix cores (the tensor-core MoE GEMM with int4 dequant
// and dispatch table of the AGX Orin port, "Phase 9b", re-designed for CDNA4).
//
// GEMM operands (exact): activations enter as bf16; each int4 weight q enters the
// MFMA as the bf16 value 1 + q/16 (exact), staged per 64-wide group, so one
// group's MFMA partial is P = sum x*(1 + q/16). With X = sum x over the same
// group the group's contribution is 16*scale*P + (bias - 16*scale)*X, applied in
// fp32 per output element and group. No weight is rounded.
//
// Tiles: BM = 64 expert-sorted rows x 64 output columns per workgroup of four
// wavefronts; each wavefront owns 16 output columns (gate and up for the first
// GEMM) over all 64 rows, using v_mfma_f32_16x16x32_bf16. The activation tile of
// a group is staged once per workgroup in LDS (double-buffered, one barrier per
// group); the weight fragments are read straight from HBM into registers (each
// wavefront reads distinct weight rows, so nothing is fetched twice).
#include "mfma_common.h"
#include "moe_internal.h"

namespace moe {

constexpr int BM = 64;  // rows per tile
constexpr int BN = 64;  // output columns per workgroup

struct Tile {
    int32_t expert, row0, nrows, pad;
};

// Workspace layout for moe_experts_prefill.
struct PrefillWs {
    size_t counts, offsets, cursor, ntiles, tiles, order, h, total;
    int max_tiles;
};

static PrefillWs prefill_ws_layout(const moe_shape& s, int T) {
    PrefillWs w;
    const int M = n_mats(s), S = n_slots(s);
    const long long picks = (long long)T * s.top_k;
    const long long routed_tiles = picks / BM + (picks < s.n_experts ? picks : s.n_experts) + 1;
    const long long shared_tiles = s.has_shared ? (T + BM - 1) / BM : 0;
    w.max_tiles = (int)(routed_tiles + shared_tiles);
    size_t o = 0;
    w.counts = o;  o = align_up(o + 4 * (size_t)M, 256);
    w.offsets = o; o = align_up(o + 4 * (size_t)(M + 1), 256);
    w.cursor = o;  o = align_up(o + 4 * (size_t)M, 256);
    w.ntiles = o;  o = align_up(o + 4, 256);
    w.tiles = o;   o = align_up(o + sizeof(Tile) * (size_t)w.max_tiles, 256);
    w.order = o;   o = align_up(o + 4 * (size_t)T * S, 256);
    w.h = o;       o = align_up(o + 2 * (size_t)T * S * s.inter, 256);
    w.total = o;
    return w;
}

// ---------------------------------------------------------------- dispatch
// One workgroup: LDS histogram of the routed picks (the shared expert takes every
// token), a wavefront scan for the exclusive offsets and the tile offsets, the
// tile list, then a scatter of pick indices p = t*S + s into expert-sorted order.
// Picks with an id outside [0, E) are skipped and their y rows zeroed.
__global__ __launch_bounds__(1024) void dispatch_kernel(const int32_t* __restrict__ ids, int T, int k, int E,
                                                        int has_shared, int H, int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ offsets, int32_t* __restrict__ ntiles,
                                                        Tile* __restrict__ tiles, int32_t* __restrict__ order,
                                                        float* __restrict__ y) {
    __shared__ int cnt[1025];
    __shared__ int off[1026];
    __shared__ int toff[1026];
    const int M = E + has_shared, S = k + has_shared;
    const int tid = threadIdx.x;
    for (int i = tid; i < M; i += blockDim.x) cnt[i] = 0;
    __syncthreads();
    const long long P = (long long)T * k;
    for (long long p = tid; p < P; p += blockDim.x) {
        const int e = ids[p];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    if (has_shared && tid == 0) cnt[E] = T;
    __syncthreads();
    if (tid < 64) {
        const int per = (M + 63) / 64;
        const int beg = tid * per, end = min(M, beg + per);
        int lc = 0, lt = 0;
        for (int i = beg; i < end; ++i) {
            lc += cnt[i];
            lt += (cnt[i] + BM - 1) / BM;
        }
        int ic = lc, it = lt;
        for (int d = 1; d < 64; d <<= 1) {
            const int oc = __shfl_up(ic, d), ot = __shfl_up(it, d);
            if (tid >= d) {
                ic += oc;
                it += ot;
            }
        }
        int rc = ic - lc, rt = it - lt;
        for (int i = beg; i < end; ++i) {
            off[i] = rc;
            toff[i] = rt;
            rc += cnt[i];
            rt += (cnt[i] + BM - 1) / BM;
        }
        if (tid == 63) {
            off[M] = ic;
            toff[M] = it;
            if (ntiles) *ntiles = it;
        }
    }
    __syncthreads();
    for (int e = tid; e < M; e += blockDim.x) {
        counts[e] = cnt[e];
        offsets[e] = off[e];
        const int nt = tiles ? (cnt[e] + BM - 1) / BM : 0;
        for (int j = 0; j < nt; ++j) {
            Tile tl;
            tl.expert = e;
            tl.row0 = off[e] + j * BM;
            tl.nrows = min(BM, cnt[e] - j * BM);
            tl.pad = 0;
            tiles[toff[e] + j] = tl;
        }
    }
    if (tid == 0) offsets[M] = off[M];
    __syncthreads();
    for (int i = tid; i < M; i += blockDim.x) cnt[i] = off[i];  // cursors
    __syncthreads();
    for (long long p = tid; p < P; p += blockDim.x) {
        const int e = ids[p];
        const int t = (int)(p / k), s = (int)(p % k);
        if (e >= 0 && e < E) {
            const int pos = atomicAdd(&cnt[e], 1);
            order[pos] = t * S + s;
        } else if (y) {
            float* yr = y + ((size_t)t * S + s) * H;
            for (int n = 0; n < H; ++n) yr[n] = 0.f;
        }
    }
    if (has_shared)
        for (int t = tid; t < T; t += blockDim.x) order[off[E] + t] = t * S + k;
}

// ---------------------------------------------------------------- pipelining
// Both GEMMs walk K in 64-wide groups. Weight fragments (the HBM stream) are
// loaded PD groups ahead into a register ring; the gathered activation group is
// loaded two groups ahead into registers and staged into a double-buffered LDS
// tile one group ahead; one barrier per group. PD is even so the LDS and register
// slots of group g are g & 1 at every unrolled position.
constexpr int PD_GU = 4;  // gate/up: 6 words per group in flight per lane
constexpr int PD_DN = 8;  // down: 3 words per group

__device__ __forceinline__ uint32_t ld32(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }

// ---------------------------------------------------------------- gate/up + SwiGLU
// Grid: (max_tiles, I / 64). Wavefront w computes gate and up for intermediate
// columns ib*64 + 16w .. +16 over the tile's rows and writes
// h[row][i] = bf16(silu(gate) * up) in expert-sorted row order.
__global__ __launch_bounds__(256) void gateup_gemm_kernel(const uint8_t* __restrict__ packed, ExpertLayout L, int H,
                                                          int I, int S, const uint16_t* __restrict__ x,
                                                          const int32_t* __restrict__ ntiles,
                                                          const Tile* __restrict__ tiles,
                                                          const int32_t* __restrict__ order,
                                                          uint16_t* __restrict__ hbuf) {
    __shared__ __attribute__((aligned(16))) uint16_t a_lds[2][BM * A_STRIDE];
    __shared__ __attribute__((aligned(16))) float x_lds[2][BM];
    if ((int)blockIdx.x >= *ntiles) return;
    const Tile tl = tiles[blockIdx.x];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lg = lane >> 4, lc = lane & 15;
    const int i_col = blockIdx.y * BN + wave * 16 + lc;  // this lane's intermediate column (weight row)
    const int n_ms = (tl.nrows + 15) >> 4;               // active 16-row subtiles (wave-uniform)

    // activation row of this thread's staging slot
    const int srow = tid >> 2, sq = tid & 3;
    const bool srow_ok = srow < tl.nrows;
    const uint16_t* xsrc = x + (size_t)(srow_ok ? order[tl.row0 + srow] / S : 0) * H + 16 * sq;

    const uint8_t* base = packed + (size_t)tl.expert * L.stride;
    const uint8_t* gq = base + L.gate_q + (size_t)i_col * (H / 2) + 4 * lg;
    const uint8_t* uq = base + L.up_q + (size_t)i_col * (H / 2) + 4 * lg;
    const uint32_t* gsb = reinterpret_cast<const uint32_t*>(base + L.gate_sb) + (size_t)i_col * (H / 64);
    const uint32_t* usb = reinterpret_cast<const uint32_t*>(base + L.up_sb) + (size_t)i_col * (H / 64);

    f32x4_t accg[4], accu[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        accg[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        accu[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const int G = H / 64;
    uint32_t bq[PD_GU][4], bs[PD_GU][2];
#pragma unroll
    for (int u = 0; u < PD_GU; ++u) {
        if (u < G) {
            bq[u][0] = ld32(gq + 32 * u);
            bq[u][1] = ld32(gq + 32 * u + 16);
            bq[u][2] = ld32(uq + 32 * u);
            bq[u][3] = ld32(uq + 32 * u + 16);
            bs[u][0] = gsb[u];
            bs[u][1] = usb[u];
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
    for (int g0 = 0; g0 < G; g0 += PD_GU) {
#pragma unroll
        for (int u = 0; u < PD_GU; ++u) {
            const int g = g0 + u;
            if (g >= G) break;  // uniform
            if (g + 2 < G && srow_ok) {
                xr[u & 1][0] = *reinterpret_cast<const uint4*>(xsrc + 64 * (g + 2));
                xr[u & 1][1] = *reinterpret_cast<const uint4*>(xsrc + 64 * (g + 2) + 8);
            }
            const uint4 bg0 = bfrag(bq[u][0]), bg1 = bfrag(bq[u][1]), bu0 = bfrag(bq[u][2]), bu1 = bfrag(bq[u][3]);
            const float sg = 16.f * bf16_to_f32(bs[u][0] & 0xFFFFu), cg = bf16_to_f32(bs[u][0] >> 16) - sg;
            const float su = 16.f * bf16_to_f32(bs[u][1] & 0xFFFFu), cu = bf16_to_f32(bs[u][1] >> 16) - su;
            if (g + PD_GU < G) {
                bq[u][0] = ld32(gq + 32 * (g + PD_GU));
                bq[u][1] = ld32(gq + 32 * (g + PD_GU) + 16);
                bq[u][2] = ld32(uq + 32 * (g + PD_GU));
                bq[u][3] = ld32(uq + 32 * (g + PD_GU) + 16);
                bs[u][0] = gsb[g + PD_GU];
                bs[u][1] = usb[g + PD_GU];
            }
            const uint16_t* al = a_lds[u & 1];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                if (m < n_ms) {
                    const uint4 a0 = *reinterpret_cast<const uint4*>(al + (16 * m + lc) * A_STRIDE + 8 * lg);
                    const uint4 a1 = *reinterpret_cast<const uint4*>(al + (16 * m + lc) * A_STRIDE + 32 + 8 * lg);
                    const float4 xs = *reinterpret_cast<const float4*>(&x_lds[u & 1][16 * m + 4 * lg]);
                    f32x4_t pg = mfma16x16x32(a0, bg0, f32x4_t{0.f, 0.f, 0.f, 0.f});
                    pg = mfma16x16x32(a1, bg1, pg);
                    f32x4_t pu = mfma16x16x32(a0, bu0, f32x4_t{0.f, 0.f, 0.f, 0.f});
                    pu = mfma16x16x32(a1, bu1, pu);
                    accg[m][0] = fmaf(cg, xs.x, fmaf(sg, pg[0], accg[m][0]));
                    accg[m][1] = fmaf(cg, xs.y, fmaf(sg, pg[1], accg[m][1]));
                    accg[m][2] = fmaf(cg, xs.z, fmaf(sg, pg[2], accg[m][2]));
                    accg[m][3] = fmaf(cg, xs.w, fmaf(sg, pg[3], accg[m][3]));
                    accu[m][0] = fmaf(cu, xs.x, fmaf(su, pu[0], accu[m][0]));
                    accu[m][1] = fmaf(cu, xs.y, fmaf(su, pu[1], accu[m][1]));
                    accu[m][2] = fmaf(cu, xs.z, fmaf(su, pu[2], accu[m][2]));
                    accu[m][3] = fmaf(cu, xs.w, fmaf(su, pu[3], accu[m][3]));
                }
            }
            if (g + 1 < G) stage_store(a_lds[(u + 1) & 1], x_lds[(u + 1) & 1], tid, xr[(u + 1) & 1][0],
                                       xr[(u + 1) & 1][1]);
            __syncthreads();
        }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * m + 4 * lg + r;
            if (row < tl.nrows) {
                const float gv = accg[m][r], uv = accu[m][r];
                const float hv = gv / (1.f + expf(-gv)) * uv;
                hbuf[(size_t)(tl.row0 + row) * I + i_col] = (uint16_t)f32_to_bf16(hv);
            }
        }
    }
}

// ---------------------------------------------------------------- down + scatter
// Grid: (max_tiles, H / 64). Wavefront w computes output columns nb*64 + 16w .. +16
// of y for the tile's rows (A = h rows, contiguous in expert-sorted order) and
// writes y[p][n] for the row's pick p = order[row].
__global__ __launch_bounds__(256) void down_gemm_kernel(const uint8_t* __restrict__ packed, ExpertLayout L, int H,
                                                        int I, const int32_t* __restrict__ ntiles,
                                                        const Tile* __restrict__ tiles,
                                                        const int32_t* __restrict__ order,
                                                        const uint16_t* __restrict__ hbuf, float* __restrict__ y) {
    __shared__ __attribute__((aligned(16))) uint16_t a_lds[2][BM * A_STRIDE];
    __shared__ __attribute__((aligned(16))) float x_lds[2][BM];
    if ((int)blockIdx.x >= *ntiles) return;
    const Tile tl = tiles[blockIdx.x];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lg = lane >> 4, lc = lane & 15;
    const int n_col = blockIdx.y * BN + wave * 16 + lc;
    const int n_ms = (tl.nrows + 15) >> 4;

    const int srow = tid >> 2, sq = tid & 3;
    const bool srow_ok = srow < tl.nrows;
    const uint16_t* hsrc = hbuf + (size_t)(tl.row0 + (srow_ok ? srow : 0)) * I + 16 * sq;

    const uint8_t* base = packed + (size_t)tl.expert * L.stride;
    const uint8_t* dq = base + L.down_q + (size_t)n_col * (I / 2) + 4 * lg;
    const uint32_t* dsb = reinterpret_cast<const uint32_t*>(base + L.down_sb) + (size_t)n_col * (I / 64);

    f32x4_t acc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int G = I / 64;
    uint32_t bq[PD_DN][2], bs[PD_DN];
#pragma unroll
    for (int u = 0; u < PD_DN; ++u) {
        if (u < G) {
            bq[u][0] = ld32(dq + 32 * u);
            bq[u][1] = ld32(dq + 32 * u + 16);
            bs[u] = dsb[u];
        }
    }
    uint4 xr[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) xr[i][0] = xr[i][1] = make_uint4(0, 0, 0, 0);
    if (srow_ok) {
        xr[0][0] = *reinterpret_cast<const uint4*>(hsrc);
        xr[0][1] = *reinterpret_cast<const uint4*>(hsrc + 8);
        if (G > 1) {
            xr[1][0] = *reinterpret_cast<const uint4*>(hsrc + 64);
            xr[1][1] = *reinterpret_cast<const uint4*>(hsrc + 72);
        }
    }
    stage_store(a_lds[0], x_lds[0], tid, xr[0][0], xr[0][1]);
    __syncthreads();
    for (int g0 = 0; g0 < G; g0 += PD_DN) {
#pragma unroll
        for (int u = 0; u < PD_DN; ++u) {
            const int g = g0 + u;
            if (g >= G) break;  // uniform
            if (g + 2 < G && srow_ok) {
                xr[u & 1][0] = *reinterpret_cast<const uint4*>(hsrc + 64 * (g + 2));
                xr[u & 1][1] = *reinterpret_cast<const uint4*>(hsrc + 64 * (g + 2) + 8);
            }
            const uint4 b0 = bfrag(bq[u][0]), b1 = bfrag(bq[u][1]);
            const float sc = 16.f * bf16_to_f32(bs[u] & 0xFFFFu), cc = bf16_to_f32(bs[u] >> 16) - sc;
            if (g + PD_DN < G) {
                bq[u][0] = ld32(dq + 32 * (g + PD_DN));
                bq[u][1] = ld32(dq + 32 * (g + PD_DN) + 16);
                bs[u] = dsb[g + PD_DN];
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
                    acc[m][0] = fmaf(cc, xs.x, fmaf(sc, p[0], acc[m][0]));
                    acc[m][1] = fmaf(cc, xs.y, fmaf(sc, p[1], acc[m][1]));
                    acc[m][2] = fmaf(cc, xs.z, fmaf(sc, p[2], acc[m][2]));
                    acc[m][3] = fmaf(cc, xs.w, fmaf(sc, p[3], acc[m][3]));
                }
            }
            if (g + 1 < G) stage_store(a_lds[(u + 1) & 1], x_lds[(u + 1) & 1], tid, xr[(u + 1) & 1][0],
                                       xr[(u + 1) & 1][1]);
            __syncthreads();
        }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * m + 4 * lg + r;
            if (row < tl.nrows) y[(size_t)order[tl.row0 + row] * H + n_col] = acc[m][r];
        }
    }
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_prefill_workspace_bytes(const moe_shape* shape, int32_t T) {
    if (validate_shape(shape) != MOE_OK || T < 1) return 0;
    return prefill_ws_layout(*shape, T).total;
}

extern "C" moe_status moe_dispatch(const moe_shape* shape, const int32_t* ids, int32_t T, int32_t* counts,
                                   int32_t* offsets, int32_t* order, void* stream) {
    clear_error();
    moe_status st = validate_shape(shape);
    if (st != MOE_OK) return st;
    if (T < 1 || !ids || !counts || !offsets || !order) return fail(MOE_ERR_INVALID_ARG, "bad T or NULL pointer");
    hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, ids, T, shape->top_k,
                       shape->n_experts, shape->has_shared, shape->hidden, counts, offsets, (int32_t*)nullptr,
                       (Tile*)nullptr, order, (float*)nullptr);
    return check_launch("dispatch_kernel");
}

extern "C" moe_status moe_experts_prefill(const moe_shape* shape, const void* experts_packed, const uint16_t* x,
                                          int32_t T, const int32_t* ids, void* ws, size_t ws_bytes, float* y,
                                          void* stream) {
    clear_error();
    moe_status st = validate_shape(shape);
    if (st != MOE_OK) return st;
    if (T < 1) return fail(MOE_ERR_INVALID_ARG, "T = %d, need T >= 1", T);
    if (!experts_packed || !x || !ids || !ws || !y || !aligned16(experts_packed) || !aligned16(x) ||
        !aligned16(ws) || !aligned16(y))
        return fail(MOE_ERR_INVALID_ARG, "NULL or unaligned pointer");
    const moe_shape& sh = *shape;
    const PrefillWs W = prefill_ws_layout(sh, T);
    if (ws_bytes < W.total) return fail(MOE_ERR_WORKSPACE, "prefill workspace too small (%zu < %zu)", ws_bytes, W.total);
    const ExpertLayout L = expert_layout(sh);
    const int S = n_slots(sh), H = sh.hidden, I = sh.inter;
    hipStream_t hs = (hipStream_t)stream;
    char* w = (char*)ws;
    int32_t* counts = (int32_t*)(w + W.counts);
    int32_t* offsets = (int32_t*)(w + W.offsets);
    int32_t* ntiles = (int32_t*)(w + W.ntiles);
    Tile* tiles = (Tile*)(w + W.tiles);
    int32_t* order = (int32_t*)(w + W.order);
    uint16_t* hbuf = (uint16_t*)(w + W.h);
    hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(1024), 0, hs, ids, T, sh.top_k, sh.n_experts, sh.has_shared, H,
                       counts, offsets, ntiles, tiles, order, y);
    if ((st = check_launch("dispatch_kernel")) != MOE_OK) return st;
    const uint8_t* p = (const uint8_t*)experts_packed;
    hipLaunchKernelGGL(gateup_gemm_kernel, dim3(W.max_tiles, I / BN), dim3(256), 0, hs, p, L, H, I, S, x, ntiles,
                       tiles, order, hbuf);
    if ((st = check_launch("gateup_gemm_kernel")) != MOE_OK) return st;
    hipLaunchKernelGGL(down_gemm_kernel, dim3(W.max_tiles, H / BN), dim3(256), 0, hs, p, L, H, I, ntiles, tiles, order,
                       hbuf, y);
    return check_launch("down_gemm_kernel");
}

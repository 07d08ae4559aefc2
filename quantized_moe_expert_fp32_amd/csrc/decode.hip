// Decode path: int4 expert GEMVs for 1..16 token rows (the GEMV MoE path at
// batch 1 of the AGX Orin port, "Phase 1-4"; row windows of 1 to 16 of TensorFold
// issue #931, "What I'd build"). Expert gate/up pair with SwiGLU, then down.
//
// Data movement: every weight row is streamed once with 16-byte loads; a
// wavefront covers a row with consecutive lanes (one 1 KiB line per load for a
// 2048-wide row). Each lane keeps its slice of the activation row in registers
// for the whole kernel, so the only HBM traffic is the weights.
//
// Arithmetic (exact weights): a group's weights are scale*q + bias. A lane's 32
// activations x meet the 32 nibbles q of the same group through
//   sum x*(scale*q + bias) = 16*scale * sum x*(1 + q/16) + (bias - 16*scale) * sum x,
// where 1 + q/16 is exactly a bf16 whose mantissa is q (one shift and one
// and-or per two weights) and sum x*(1 + q/16) is a chain of bf16 dot2
// instructions accumulating in fp32.
#include "moe_internal.h"
#include "route_internal.h"

namespace moe {

template <int CPL>
struct XSlice {
    uint32_t p[CPL][16];  // 32 bf16 per chunk, repacked in (0,4),(1,5),(2,6),(3,7) pairs per 8
    float s[CPL];         // plain sum of the chunk's 32 values, in element order
};

// Chunk c of this lane covers elements [32 * (lr + lpr * c), +32) of the row.
template <int CPL>
__device__ __forceinline__ void load_xslice(const uint16_t* __restrict__ row, int lr, int lpr, XSlice<CPL>& xs) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const uint4* src = reinterpret_cast<const uint4*>(row + 32 * (lr + lpr * c));
        float sum = 0.f;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const uint4 v = src[q4];
            const uint32_t in[4] = {v.x, v.y, v.z, v.w};
            bf16x8_to_pair_order(in, &xs.p[c][4 * q4]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sum += bf16_to_f32(in[j] & 0xFFFFu);
                sum += bf16_to_f32(in[j] >> 16);
            }
        }
        xs.s[c] = sum;
    }
}

// One 16-byte chunk of an int4 row and its group's (scale, bias) word.
struct ChunkLoad {
    uint4 q;
    uint32_t sb;
};

__device__ __forceinline__ ChunkLoad load_chunk(const uint8_t* __restrict__ qrow, const uint32_t* __restrict__ sbrow,
                                                int chunk) {
    ChunkLoad c;
    c.q = *reinterpret_cast<const uint4*>(qrow + 16 * chunk);
    c.sb = sbrow[chunk >> 1];
    return c;
}

// This lane's share of one row's dot product: 32 int4 weights against the
// activation chunk xp (pair order) whose plain sum is xsum.
__device__ __forceinline__ float chunk_dot(const ChunkLoad& c, const uint32_t* xp, float xsum) {
    const uint32_t qw[4] = {c.q.x, c.q.y, c.q.z, c.q.w};
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t wp[4];
        int4x8_to_bf16_pairs(qw[j], wp);
        d0 = dot2_bf16(wp[0], xp[4 * j + 0], d0);
        d1 = dot2_bf16(wp[1], xp[4 * j + 1], d1);
        d0 = dot2_bf16(wp[2], xp[4 * j + 2], d0);
        d1 = dot2_bf16(wp[3], xp[4 * j + 3], d1);
    }
    const float s16 = 16.f * bf16_to_f32(c.sb & 0xFFFFu);
    const float b = bf16_to_f32(c.sb >> 16);
    return fmaf(b - s16, xsum, s16 * (d0 + d1));
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.f + expf(-g)); }

// ---------------------------------------------------------------- gate/up + SwiGLU
// Grid: (I / 16, S, T); block 256 = 4 wavefronts, each owning 4 consecutive
// intermediate rows (gate row and up row). Every weight load of a wavefront is
// issued before the first one is consumed (up to 2 x 4 x CPL 16-byte loads per
// lane in flight). Writes h[t][s][i] (bf16).
constexpr int GU_ROWS_PER_WG = 16;
constexpr int GU_IT = 4;  // row iterations per wavefront (rows per iteration = 64 / lanes per row)

template <int CPL>
__global__ __launch_bounds__(256) void decode_gateup_kernel(const uint8_t* __restrict__ packed, ExpertLayout L, int H,
                                                            int I, int E, int k, int has_shared,
                                                            const uint16_t* __restrict__ x,
                                                            const int32_t* __restrict__ ids,
                                                            uint16_t* __restrict__ hbuf) {
    const int t = blockIdx.z, s = blockIdx.y, S = k + has_shared;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int e = s < k ? ids[(size_t)t * k + s] : E;
    const bool valid = s < k ? (e >= 0 && e < E) : true;
    uint16_t* hrow = hbuf + ((size_t)t * S + s) * I;
    const int C = H / 32, lpr = C < 64 ? C : 64, rpw = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    constexpr int per_wave = GU_ROWS_PER_WG / 4;
    const int r0 = blockIdx.x * GU_ROWS_PER_WG + wave * per_wave;
    if (!valid) {
        if (lane < per_wave) hrow[r0 + lane] = 0;
        return;
    }
    const uint8_t* base = packed + (size_t)e * L.stride;
    const uint8_t* gq = base + L.gate_q;
    const uint8_t* uq = base + L.up_q;
    const uint32_t* gsb = reinterpret_cast<const uint32_t*>(base + L.gate_sb);
    const uint32_t* usb = reinterpret_cast<const uint32_t*>(base + L.up_sb);
    const size_t qstride = H / 2, sbstride = H / 64;

    ChunkLoad lg[GU_IT][CPL], lu[GU_IT][CPL];
#pragma unroll
    for (int it = 0; it < GU_IT; ++it) {
        const int rr = it * rpw + rsub;
        const int r = r0 + (rr < per_wave ? rr : 0);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            if (rr < per_wave) {
                lg[it][c] = load_chunk(gq + r * qstride, gsb + r * sbstride, lr + lpr * c);
                lu[it][c] = load_chunk(uq + r * qstride, usb + r * sbstride, lr + lpr * c);
            }
        }
    }
    XSlice<CPL> xs;
    load_xslice(x + (size_t)t * H, lr, lpr, xs);
#pragma unroll
    for (int it = 0; it < GU_IT; ++it) {
        const int rr = it * rpw + rsub;
        if (it * rpw >= per_wave) break;  // wave-uniform
        const bool act = rr < per_wave;
        float g = 0.f, u = 0.f;
        if (act) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                g += chunk_dot(lg[it][c], xs.p[c], xs.s[c]);
                u += chunk_dot(lu[it][c], xs.p[c], xs.s[c]);
            }
        }
        for (int off = lpr >> 1; off >= 1; off >>= 1) {
            g += __shfl_xor(g, off);
            u += __shfl_xor(u, off);
        }
        if (act && lr == 0) hrow[r0 + rr] = (uint16_t)f32_to_bf16(silu_f32(g) * u);
    }
}

// ---------------------------------------------------------------- down (+ combine)
// Grid: (H / 8, T); block 256. A workgroup computes y[t][s][n] for its 8 output
// rows n and every slot s (S*8 row dot products of length I, lpr = I/32 lanes
// each), keeps them in LDS, and optionally writes
//   out[t][n] = bf16(sum_{s<k} w[t][s] * y[t][s][n] + wsh[t] * y[t][k][n])
// (then bf16(residual + out) when a residual is given) with the same fp32
// slot-order arithmetic as moe_combine. Weight loads depend only on ids, so they
// are issued before the h rows produced by the gate/up kernel are read.
constexpr int DN_ROWS_PER_WG = 8;
constexpr int DN_BATCH = 5;  // 9 slots x 8 rows at I = 512: 18 iterations, 4.5 per wavefront

__global__ __launch_bounds__(256) void decode_down_kernel(const uint8_t* __restrict__ packed, ExpertLayout L, int H,
                                                          int I, int E, int k, int has_shared,
                                                          const uint16_t* __restrict__ hbuf,
                                                          const int32_t* __restrict__ ids, float* __restrict__ y,
                                                          const uint16_t* __restrict__ w,
                                                          const uint16_t* __restrict__ wsh, const uint16_t* residual,
                                                          uint16_t* out) {
    __shared__ float ysh[17][DN_ROWS_PER_WG];
    const int t = blockIdx.y, S = k + has_shared;
    const int n0 = blockIdx.x * DN_ROWS_PER_WG;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lpr = I / 32, rpw = 64 / lpr;  // I <= 2048: one chunk per lane
    const int lr = lane % lpr, rsub = lane / lpr;
    const int n_dots = S * DN_ROWS_PER_WG;
    const int n_it = (n_dots + rpw - 1) / rpw;
    const size_t qstride = I / 2, sbstride = I / 64;

    // iterations it = wave + 4 j; processed in batches of DN_BATCH per wavefront with
    // every weight load of a batch issued before the batch is consumed
    for (int j0 = 0; 4 * j0 < n_it; j0 += DN_BATCH) {
        ChunkLoad ld[DN_BATCH];
        int slot[DN_BATCH];
        bool ok[DN_BATCH];
#pragma unroll
        for (int j = 0; j < DN_BATCH; ++j) {
            const int it = wave + 4 * (j0 + j);
            const int q = it * rpw + rsub;
            ok[j] = it < n_it && q < n_dots;
            slot[j] = ok[j] ? q / DN_ROWS_PER_WG : 0;
            if (ok[j]) {
                const int s = slot[j];
                const int e = s < k ? ids[(size_t)t * k + s] : E;
                if (s < k && (e < 0 || e >= E)) {
                    ok[j] = false;  // invalid expert id: this y row is zero
                } else {
                    const int n = n0 + q % DN_ROWS_PER_WG;
                    const uint8_t* base = packed + (size_t)e * L.stride;
                    ld[j] = load_chunk(base + L.down_q + n * qstride,
                                       reinterpret_cast<const uint32_t*>(base + L.down_sb) + n * sbstride, lr);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < DN_BATCH; ++j) {
            const int it = wave + 4 * (j0 + j);
            if (it >= n_it) break;  // wave-uniform
            const int q = it * rpw + rsub;
            float v = 0.f;
            if (ok[j]) {
                XSlice<1> hs;
                load_xslice(hbuf + ((size_t)t * S + slot[j]) * I, lr, lpr, hs);
                v = chunk_dot(ld[j], hs.p[0], hs.s[0]);
            }
            for (int off = lpr >> 1; off >= 1; off >>= 1) v += __shfl_xor(v, off);
            if (lr == 0 && q < n_dots) ysh[q / DN_ROWS_PER_WG][q % DN_ROWS_PER_WG] = v;
        }
    }
    __syncthreads();
    const int tid = threadIdx.x;
    if (y) {
        for (int i = tid; i < n_dots; i += 256)
            y[((size_t)t * S + i / DN_ROWS_PER_WG) * H + n0 + i % DN_ROWS_PER_WG] =
                ysh[i / DN_ROWS_PER_WG][i % DN_ROWS_PER_WG];
    }
    if (out && tid < DN_ROWS_PER_WG) {
        float a = 0.f;
        for (int s = 0; s < k; ++s) a = fmaf(bf16_to_f32(w[(size_t)t * k + s]), ysh[s][tid], a);
        if (has_shared) a = fmaf(bf16_to_f32(wsh[t]), ysh[k][tid], a);
        uint32_t b = f32_to_bf16(a);
        const size_t o = (size_t)t * H + n0 + tid;
        if (residual) b = f32_to_bf16(bf16_to_f32(residual[o]) + bf16_to_f32(b));
        out[o] = (uint16_t)b;
    }
}

static int cpl_for(int K) { return K / 32 <= 64 ? 1 : (K / 32) / 64; }

static void launch_gateup(const moe_shape& sh, const ExpertLayout& L, const uint8_t* p, const uint16_t* x, int T,
                          const int32_t* ids, uint16_t* hbuf, hipStream_t hs) {
    const int S = n_slots(sh), H = sh.hidden, I = sh.inter;
    dim3 g1(I / GU_ROWS_PER_WG, S, T);
    switch (cpl_for(H)) {
        case 1: hipLaunchKernelGGL(decode_gateup_kernel<1>, g1, dim3(256), 0, hs, p, L, H, I, sh.n_experts, sh.top_k,
                                   sh.has_shared, x, ids, hbuf); break;
        case 2: hipLaunchKernelGGL(decode_gateup_kernel<2>, g1, dim3(256), 0, hs, p, L, H, I, sh.n_experts, sh.top_k,
                                   sh.has_shared, x, ids, hbuf); break;
        default: hipLaunchKernelGGL(decode_gateup_kernel<4>, g1, dim3(256), 0, hs, p, L, H, I, sh.n_experts, sh.top_k,
                                    sh.has_shared, x, ids, hbuf); break;
    }
}

}  // namespace moe

using namespace moe;

static size_t hbuf_bytes(const moe_shape& sh, int T) {
    return align_up((size_t)T * n_slots(sh) * sh.inter * 2, 256);
}

extern "C" size_t moe_decode_workspace_bytes(const moe_shape* shape, int32_t T) {
    if (validate_shape(shape) != MOE_OK || T < 1) return 0;
    return hbuf_bytes(*shape, T) + 256;  // h rows, then the fused-routing counter word
}

static moe_status check_decode_args(const moe_shape* shape, const void* experts_packed, const uint16_t* x, int T,
                                    const void* ws, size_t ws_bytes) {
    moe_status st = validate_shape(shape);
    if (st != MOE_OK) return st;
    if (T < 1 || T > 16) return fail(MOE_ERR_INVALID_ARG, "decode path takes 1..16 rows, got T = %d", T);
    if (!experts_packed || !x || !ws || !aligned16(experts_packed) || !aligned16(x) || !aligned16(ws))
        return fail(MOE_ERR_INVALID_ARG, "NULL or unaligned pointer");
    if (ws_bytes < moe_decode_workspace_bytes(shape, T)) return fail(MOE_ERR_WORKSPACE, "decode workspace too small");
    return MOE_OK;
}

extern "C" moe_status moe_experts_decode(const moe_shape* shape, const void* experts_packed, const uint16_t* x,
                                         int32_t T, const int32_t* ids, void* ws, size_t ws_bytes, float* y,
                                         void* stream) {
    clear_error();
    moe_status st = check_decode_args(shape, experts_packed, x, T, ws, ws_bytes);
    if (st != MOE_OK) return st;
    if (!ids || !y || !aligned16(y)) return fail(MOE_ERR_INVALID_ARG, "ids or y NULL / unaligned");
    const moe_shape& sh = *shape;
    const ExpertLayout L = expert_layout(sh);
    hipStream_t hs = (hipStream_t)stream;
    const uint8_t* p = (const uint8_t*)experts_packed;
    uint16_t* hbuf = (uint16_t*)ws;
    launch_gateup(sh, L, p, x, T, ids, hbuf, hs);
    if ((st = check_launch("decode_gateup_kernel")) != MOE_OK) return st;
    hipLaunchKernelGGL(decode_down_kernel, dim3(sh.hidden / DN_ROWS_PER_WG, T), dim3(256), 0, hs, p, L, sh.hidden,
                       sh.inter, sh.n_experts, sh.top_k, sh.has_shared, hbuf, ids, y, (const uint16_t*)nullptr,
                       (const uint16_t*)nullptr, (const uint16_t*)nullptr, (uint16_t*)nullptr);
    return check_launch("decode_down_kernel");
}

extern "C" moe_status moe_decode_layer(const moe_shape* shape, const void* router_packed, const float* logit_bias,
                                       const void* experts_packed, const uint16_t* x, int32_t T, void* ws,
                                       size_t ws_bytes, float* logits, int32_t* ids, uint16_t* w, uint16_t* w_shared,
                                       float* y, const uint16_t* residual, uint16_t* out, void* stream) {
    clear_error();
    moe_status st = check_decode_args(shape, experts_packed, x, T, ws, ws_bytes);
    if (st != MOE_OK) return st;
    const moe_shape& sh = *shape;
    if ((st = check_route_outputs(sh, T, ids, w, w_shared)) != MOE_OK) return st;
    if (!router_packed || !logits || !out || !aligned16(router_packed))
        return fail(MOE_ERR_INVALID_ARG, "router, logits or out NULL / unaligned");
    if (y && !aligned16(y)) return fail(MOE_ERR_INVALID_ARG, "y unaligned");
    const ExpertLayout L = expert_layout(sh);
    hipStream_t hs = (hipStream_t)stream;
    const uint8_t* p = (const uint8_t*)experts_packed;
    uint16_t* hbuf = (uint16_t*)ws;
    unsigned int* counter = (unsigned int*)((char*)ws + hbuf_bytes(sh, T));
    if ((st = launch_route_fused(sh, router_packed, logit_bias, x, T, logits, counter, ids, w, w_shared, hs)) !=
        MOE_OK)
        return st;
    launch_gateup(sh, L, p, x, T, ids, hbuf, hs);
    if ((st = check_launch("decode_gateup_kernel")) != MOE_OK) return st;
    hipLaunchKernelGGL(decode_down_kernel, dim3(sh.hidden / DN_ROWS_PER_WG, T), dim3(256), 0, hs, p, L, sh.hidden,
                       sh.inter, sh.n_experts, sh.top_k, sh.has_shared, hbuf, ids, y, w, w_shared, residual, out);
    return check_launch("decode_down_kernel (combine)");
}

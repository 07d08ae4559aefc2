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

// This lane's share of the dot product of one int4 row with the activation slice.
template <int CPL>
__device__ __forceinline__ float row_dot(const uint8_t* __restrict__ qrow, const uint32_t* __restrict__ sbrow, int lr,
                                         int lpr, const XSlice<CPL>& xs) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int chunk = lr + lpr * c;
        const uint4 q = *reinterpret_cast<const uint4*>(qrow + 16 * chunk);
        const uint32_t sb = sbrow[chunk >> 1];
        const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t wp[4];
            int4x8_to_bf16_pairs(qw[j], wp);
            d0 = dot2_bf16(wp[0], xs.p[c][4 * j + 0], d0);
            d1 = dot2_bf16(wp[1], xs.p[c][4 * j + 1], d1);
            d0 = dot2_bf16(wp[2], xs.p[c][4 * j + 2], d0);
            d1 = dot2_bf16(wp[3], xs.p[c][4 * j + 3], d1);
        }
        const float s16 = 16.f * bf16_to_f32(sb & 0xFFFFu);
        const float b = bf16_to_f32(sb >> 16);
        acc = fmaf(s16, d0 + d1, acc);
        acc = fmaf(b - s16, xs.s[c], acc);
    }
    return acc;
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.f + expf(-g)); }

// Grid: (I / rows_per_wg, S, T); block 256 = 4 wavefronts, each owning
// rows_per_wg / 4 consecutive intermediate rows. Writes h[t][s][i] (bf16).
template <int CPL>
__global__ __launch_bounds__(256) void decode_gateup_kernel(const uint8_t* __restrict__ packed, ExpertLayout L, int H,
                                                            int I, int E, int k, int has_shared,
                                                            const uint16_t* __restrict__ x,
                                                            const int32_t* __restrict__ ids, int rows_per_wg,
                                                            uint16_t* __restrict__ hbuf) {
    const int t = blockIdx.z, s = blockIdx.y, S = k + has_shared;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int e = s < k ? ids[(size_t)t * k + s] : E;
    const bool valid = s < k ? (e >= 0 && e < E) : true;
    uint16_t* hrow = hbuf + ((size_t)t * S + s) * I;
    const int C = H / 32, lpr = C < 64 ? C : 64, rpw = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    const int per_wave = rows_per_wg / 4;
    const int r0 = blockIdx.x * rows_per_wg + wave * per_wave;
    if (!valid) {
        for (int r = r0 + lane; r < r0 + per_wave; r += 64) hrow[r] = 0;
        return;
    }
    XSlice<CPL> xs;
    load_xslice(x + (size_t)t * H, lr, lpr, xs);
    const uint8_t* base = packed + (size_t)e * L.stride;
    const uint8_t* gq = base + L.gate_q;
    const uint8_t* uq = base + L.up_q;
    const uint32_t* gsb = reinterpret_cast<const uint32_t*>(base + L.gate_sb);
    const uint32_t* usb = reinterpret_cast<const uint32_t*>(base + L.up_sb);
    const size_t qstride = H / 2, sbstride = H / 64;
    for (int it = 0; it < per_wave; it += rpw) {
        const int r = r0 + it + rsub;
        const bool act = it + rsub < per_wave;
        float g = 0.f, u = 0.f;
        if (act) {
            g = row_dot(gq + r * qstride, gsb + r * sbstride, lr, lpr, xs);
            u = row_dot(uq + r * qstride, usb + r * sbstride, lr, lpr, xs);
        }
        for (int off = lpr >> 1; off >= 1; off >>= 1) {
            g += __shfl_xor(g, off);
            u += __shfl_xor(u, off);
        }
        if (act && lr == 0) hrow[r] = (uint16_t)f32_to_bf16(silu_f32(g) * u);
    }
}

// Grid: (H / rows_per_wg, S, T). y[t][s][n] = sum_i Wd[n][i] * h[t][s][i] in fp32.
template <int CPL>
__global__ __launch_bounds__(256) void decode_down_kernel(const uint8_t* __restrict__ packed, ExpertLayout L, int H,
                                                          int I, int E, int k, int has_shared,
                                                          const uint16_t* __restrict__ hbuf,
                                                          const int32_t* __restrict__ ids, int rows_per_wg,
                                                          float* __restrict__ y) {
    const int t = blockIdx.z, s = blockIdx.y, S = k + has_shared;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int e = s < k ? ids[(size_t)t * k + s] : E;
    const bool valid = s < k ? (e >= 0 && e < E) : true;
    float* yrow = y + ((size_t)t * S + s) * H;
    const int C = I / 32, lpr = C < 64 ? C : 64, rpw = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    const int per_wave = rows_per_wg / 4;
    const int r0 = blockIdx.x * rows_per_wg + wave * per_wave;
    if (!valid) {
        for (int r = r0 + lane; r < r0 + per_wave; r += 64) yrow[r] = 0.f;
        return;
    }
    XSlice<CPL> xs;
    load_xslice(hbuf + ((size_t)t * S + s) * I, lr, lpr, xs);
    const uint8_t* base = packed + (size_t)e * L.stride;
    const uint8_t* dq = base + L.down_q;
    const uint32_t* dsb = reinterpret_cast<const uint32_t*>(base + L.down_sb);
    const size_t qstride = I / 2, sbstride = I / 64;
    for (int it = 0; it < per_wave; it += rpw) {
        const int r = r0 + it + rsub;
        const bool act = it + rsub < per_wave;
        float v = act ? row_dot(dq + r * qstride, dsb + r * sbstride, lr, lpr, xs) : 0.f;
        for (int off = lpr >> 1; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if (act && lr == 0) yrow[r] = v;
    }
}

static int cpl_for(int K) { return K / 32 <= 64 ? 1 : (K / 32) / 64; }

}  // namespace moe

using namespace moe;

extern "C" size_t moe_decode_workspace_bytes(const moe_shape* shape, int32_t T) {
    if (validate_shape(shape) != MOE_OK || T < 1) return 0;
    return align_up((size_t)T * n_slots(*shape) * shape->inter * 2, 256);
}

extern "C" moe_status moe_experts_decode(const moe_shape* shape, const void* experts_packed, const uint16_t* x,
                                         int32_t T, const int32_t* ids, void* ws, size_t ws_bytes, float* y,
                                         void* stream) {
    clear_error();
    moe_status st = validate_shape(shape);
    if (st != MOE_OK) return st;
    if (T < 1 || T > 16) return fail(MOE_ERR_INVALID_ARG, "decode path takes 1..16 rows, got T = %d", T);
    if (!experts_packed || !x || !ids || !ws || !y || !aligned16(experts_packed) || !aligned16(x) ||
        !aligned16(ws) || !aligned16(y))
        return fail(MOE_ERR_INVALID_ARG, "NULL or unaligned pointer");
    if (ws_bytes < moe_decode_workspace_bytes(shape, T)) return fail(MOE_ERR_WORKSPACE, "decode workspace too small");
    const moe_shape& sh = *shape;
    const ExpertLayout L = expert_layout(sh);
    const int S = n_slots(sh), H = sh.hidden, I = sh.inter;
    hipStream_t hs = (hipStream_t)stream;
    const uint8_t* p = (const uint8_t*)experts_packed;
    uint16_t* hbuf = (uint16_t*)ws;

    const int gu_rows = 16;
    dim3 g1(I / gu_rows, S, T);
    switch (cpl_for(H)) {
        case 1: hipLaunchKernelGGL(decode_gateup_kernel<1>, g1, dim3(256), 0, hs, p, L, H, I, sh.n_experts, sh.top_k,
                                   sh.has_shared, x, ids, gu_rows, hbuf); break;
        case 2: hipLaunchKernelGGL(decode_gateup_kernel<2>, g1, dim3(256), 0, hs, p, L, H, I, sh.n_experts, sh.top_k,
                                   sh.has_shared, x, ids, gu_rows, hbuf); break;
        default: hipLaunchKernelGGL(decode_gateup_kernel<4>, g1, dim3(256), 0, hs, p, L, H, I, sh.n_experts, sh.top_k,
                                    sh.has_shared, x, ids, gu_rows, hbuf); break;
    }
    if ((st = check_launch("decode_gateup_kernel")) != MOE_OK) return st;

    const int dn_rows = 64;
    dim3 g2(H / dn_rows, S, T);
    hipLaunchKernelGGL(decode_down_kernel<1>, g2, dim3(256), 0, hs, p, L, H, I, sh.n_experts, sh.top_k, sh.has_shared,
                       hbuf, ids, dn_rows, y);
    return check_launch("decode_down_kernel");
}

// Device-side routing pieces: one router row's fp32 logits and one token's
// selection (routing contract of TensorFold issue #931, "What I'd build").
#pragma once

#include "moe_internal.h"

namespace moe {

// Wave-wide maximum of an unsigned value with DPP row operations (quad
// permutations, half-row and row mirrors, then the row broadcasts 15 and 31);
// every lane must be active. Returns the maximum in all lanes.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast15
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Selection for one token by one full wavefront (see LogitSrc for where the
// logits come from). Logit e lives in lane e % 64,
// slot e / 64 as a 32-bit key: 0 once picked (or beyond E), else
// max(ordered_logit, 1) so NaN (ordered 0) still ranks above a removed entry but
// below every number. Each of the k rounds takes the wave maximum of the keys
// (DPP), then the lowest expert id holding it (ballots: lowest slot, then lowest
// lane), which realises the order (logit desc, id asc).
// Outputs: sel_id[i] and sel_w[i] (bf16 bits) for i < k in lane i's registers are
// written through the given pointers by lanes 0..k-1; *sel_wsh by lane 0.
template <int VPL>
__device__ __forceinline__ void select_token(const LogitSrc& lr, int E, int k, int has_shared, int lane,
                                             int32_t* sel_id, uint16_t* sel_w, uint16_t* sel_wsh) {
    uint32_t key[VPL], raw[VPL];
    if (lr.tagged) {
        const int n = lane < E ? (E - 1 - lane) / 64 + 1 : 0;  // this lane's logits: lane + 64 j < E
        load_tagged_many<VPL>(lr.tagged + lane, 64, n, lr.tag, lr.err, raw);
    } else {
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const int e = lane + 64 * j;
            raw[j] = e < E ? lr.get(e) : 0u;
        }
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        const int e = lane + 64 * j;
        const uint32_t o = e < E ? ordered_logit(__uint_as_float(raw[j])) : 0u;
        key[j] = e < E ? (o > 1u ? o : 1u) : 0u;
    }
    uint32_t my_id = 0, my_raw = 0;
    for (int i = 0; i < k; ++i) {
        uint32_t m = key[0];
#pragma unroll
        for (int j = 1; j < VPL; ++j) m = key[j] > m ? key[j] : m;
        m = wave_max_u32(m);
        int wj = 0;
        uint64_t mask = 0;
#pragma unroll
        for (int j = VPL - 1; j >= 0; --j) {
            const uint64_t b = __ballot(key[j] == m);
            if (b) {
                wj = j;
                mask = b;
            }
        }
        const int wl = __builtin_ctzll(mask);
        uint32_t rv = raw[0];
#pragma unroll
        for (int j = 1; j < VPL; ++j)
            if (j == wj) rv = raw[j];
        rv = (uint32_t)__builtin_amdgcn_readlane((int)rv, wl);  // the picked logit, from registers
#pragma unroll
        for (int j = 0; j < VPL; ++j)
            if (j == wj && lane == wl) key[j] = 0;
        if (lane == i) {
            my_id = (uint32_t)(64 * wj + wl);
            my_raw = rv;
        }
    }
    my_id = my_id < (uint32_t)E ? my_id : (uint32_t)(E - 1);
    const double li = lane < k ? (double)__uint_as_float(my_raw) : 0.0;
    const double l0 = readlane_f64(li, 0);
    const double ex = lane < k ? exp(li - l0) : 0.0;
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += readlane_f64(ex, j);
    if (lane < k) {
        sel_id[lane] = (int32_t)my_id;
        sel_w[lane] = (uint16_t)f64_to_bf16(ex / sum);
    }
    if (has_shared && lane == 0) {
        const double g = (double)bf16_to_f32(f32_to_bf16(__uint_as_float(lr.get(E))));
        *sel_wsh = (uint16_t)f64_to_bf16(1.0 / (1.0 + exp(-g)));
    }
}

// Dispatch on the number of keys per lane.
__device__ __forceinline__ void select_token_any(const LogitSrc& lr, int E, int k, int has_shared, int lane,
                                                 int32_t* sel_id, uint16_t* sel_w, uint16_t* sel_wsh) {
    const int vpl = (E + 63) / 64;
    if (vpl <= 1) select_token<1>(lr, E, k, has_shared, lane, sel_id, sel_w, sel_wsh);
    else if (vpl <= 2) select_token<2>(lr, E, k, has_shared, lane, sel_id, sel_w, sel_wsh);
    else if (vpl <= 4) select_token<4>(lr, E, k, has_shared, lane, sel_id, sel_w, sel_wsh);
    else if (vpl <= 8) select_token<8>(lr, E, k, has_shared, lane, sel_id, sel_w, sel_wsh);
    else select_token<16>(lr, E, k, has_shared, lane, sel_id, sel_w, sel_wsh);
}

// N consecutive dwords (N = 2 or 8) with 8- or 16-byte loads.
template <int N>
__device__ __forceinline__ void load_words(const uint16_t* p, uint32_t* out) {
    if constexpr (N == 8) {
        const uint4 a = *reinterpret_cast<const uint4*>(p);
        const uint4 b = *reinterpret_cast<const uint4*>(p + 8);
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
        out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    } else {
        const uint2 a = *reinterpret_cast<const uint2*>(p);
        out[0] = a.x;
        out[1] = a.y;
    }
}

// fp32 logits of router row r for TT tokens by one wavefront. A lane reads
// 16-byte chunks of the row (16 int8 or 4 fp32 weights) at chunk index
// lane + 64 i, so each load instruction covers 1 KiB of the row. Products are
// exact in fp64 and accumulate in fp64 in a fixed order (lane-sequential, then a
// butterfly), so a token's logits do not depend on T or on the other tokens.
// The logit of token t is written to logits[t][r] (coherently when `coherent`)
// and, when `tagged` is given, published to tagged[t][r] with tag `tag`.
template <int TT, bool AFF8>
__device__ __forceinline__ void router_row(const uint8_t* __restrict__ router, const float* __restrict__ logit_bias,
                                           const uint16_t* __restrict__ x, int t0, int nt, int H, int R, int E, int r,
                                           int lane, float* logits, bool coherent, uint64_t* tagged, uint32_t tag) {
    double acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.0;
    constexpr int EPC = AFF8 ? 16 : 4;  // elements per 16-byte chunk
    constexpr int NCH = 4;                // chunks per lane whose loads are issued together
    constexpr int XW = AFF8 ? 8 : 2;      // activation dwords per chunk and token
    constexpr int TH = TT <= 4 ? TT : 0;  // tokens whose activations are loaded with the weights
    const int C = H / EPC;
    const uint32_t* sb = reinterpret_cast<const uint32_t*>(router + (size_t)R * H);
    for (int j0 = lane; j0 < C; j0 += 64 * NCH) {
        uint4 wq[NCH];
        uint32_t wg[NCH];
        uint32_t xh[NCH][TH > 0 ? TH : 1][XW];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int j = j0 + 64 * c;
            if (j < C) {
                const int c0 = j * EPC;
                if constexpr (AFF8) {
                    wq[c] = *reinterpret_cast<const uint4*>(router + (size_t)r * H + c0);
                    wg[c] = sb[(size_t)r * (H / 64) + (c0 >> 6)];
                } else {
                    wq[c] = *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(router) + (size_t)r * H +
                                                            c0);
                }
#pragma unroll
                for (int t = 0; t < TH; ++t) {
                    if (t < nt) {
                        load_words<XW>(x + (size_t)(t0 + t) * H + c0, xh[c][t]);
                    }
                }
            }
        }
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int j = j0 + 64 * c;
            if (j >= C) break;
            const int c0 = j * EPC;
            double wv[EPC];
            const uint32_t qw[4] = {wq[c].x, wq[c].y, wq[c].z, wq[c].w};
            if constexpr (AFF8) {
                const double s = (double)bf16_to_f32(wg[c] & 0xFFFFu), b = (double)bf16_to_f32(wg[c] >> 16);
#pragma unroll
                for (int i = 0; i < EPC; ++i) wv[i] = s * (double)((qw[i >> 2] >> (8 * (i & 3))) & 0xFFu) + b;  // exact
            } else {
#pragma unroll
                for (int i = 0; i < EPC; ++i) wv[i] = (double)__uint_as_float(qw[i]);
            }
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                if (t < nt) {
                    uint32_t xw[XW];
                    if constexpr (TH > 0) {
#pragma unroll
                        for (int i = 0; i < XW; ++i) xw[i] = xh[c][t < TH ? t : 0][i];
                    } else {
                        load_words<XW>(x + (size_t)(t0 + t) * H + c0, xw);
                    }
#pragma unroll
                    for (int i = 0; i < EPC; ++i) {
                        const uint32_t bits = (i & 1) ? (xw[i >> 1] >> 16) : (xw[i >> 1] & 0xFFFFu);
                        acc[t] = fma((double)bf16_to_f32(bits), wv[i], acc[t]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = wave_sum_f64(acc[t]);
    if (lane == 63) {
        const double bias = (r < E && logit_bias) ? (double)logit_bias[r] : 0.0;
#pragma unroll
        for (int t = 0; t < TT; ++t)
            if (t < nt) {
                const size_t o = (size_t)(t0 + t) * R + r;
                const uint32_t v = __float_as_uint((float)(acc[t] + bias));
                if (coherent)
                    store_coherent(reinterpret_cast<uint32_t*>(logits) + o, v);
                else
                    reinterpret_cast<uint32_t*>(logits)[o] = v;
                if (tagged) store_tagged(tagged + o, tag, v);
            }
    }
}

}  // namespace moe

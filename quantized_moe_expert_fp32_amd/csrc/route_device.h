// Device-side routing pieces: one router row's fp32 logits and one token's
// selection (routing contract of TensorFold issue #931, "What I'd build").
#pragma once

#include "moe_internal.h"

namespace moe {

// Wave-wide maximum (or minimum) of an unsigned value with DPP row operations
// (quad permutations, half-row and row mirrors, then the row broadcasts 15 and
// 31); every lane must be active. Returns the result in all lanes.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_ext_u32(uint32_t v) {
    auto f = [](uint32_t a, uint32_t b) { return MAX ? max(a, b) : min(a, b); };
    const int fill = MAX ? 0 : -1;
    v = f(v, (uint32_t)__builtin_amdgcn_update_dpp(fill, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = f(v, (uint32_t)__builtin_amdgcn_update_dpp(fill, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = f(v, (uint32_t)__builtin_amdgcn_update_dpp(fill, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = f(v, (uint32_t)__builtin_amdgcn_update_dpp(fill, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
    v = f(v, (uint32_t)__builtin_amdgcn_update_dpp(fill, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast15
    v = f(v, (uint32_t)__builtin_amdgcn_update_dpp(fill, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return wave_ext_u32<true>(v); }

__device__ __forceinline__ double readlane_f64(double v, int l) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Selection for one token by one full wavefront (see LogitSrc for where the
// logits come from). Expert e's logit lives in lane e % 64, slot e / 64, as a
// 32-bit key: max(ordered_logit, 1) for e < E (so NaN, ordered 0, still ranks
// above an absent entry but below every number), 0 beyond E. Each lane first
// orders its own keys (descending; equal keys keep ascending slot, i.e. ascending
// id). A round then takes the wave maximum of the lanes' leading keys (DPP); the
// single lane holding it is the winner, and if several lanes hold it, the one
// whose leading key has the lowest expert id (a second DPP reduction). The winner
// drops its leading key. This realises the order (logit desc, id asc).
// select_ids writes sel_id[i] for i < k (lanes 0..k-1) and returns what the
// weights need; select_weights then gives lane i < k the bf16 bits of pick i's
// weight and lane k the shared weight's (its exp and division run beside the
// picks'). The weights are needed only by the combine, so a caller may compute
// them later than the ids. select_token does both and stores sel_w[i] (i < k)
// and *sel_wsh.
struct SelState {
    uint32_t id;     // lane i < k: pick i's expert id
    uint32_t raw;    // lane i < k: pick i's fp32 logit bits
    uint32_t gbits;  // every lane: the shared gate's fp32 logit bits
    bool won;        // false: another wavefront of a polling race selects this token (nothing written)
    bool timeout;    // a bounded wait for tagged logits timed out: the picks come from stale words
};

template <int VPL>
__device__ __forceinline__ SelState select_ids(const LogitSrc& lr, int E, int k, int has_shared, int lane,
                                               int32_t* sel_id) {
    uint32_t raw[VPL + 1];
    bool tmo = false;
    if (lr.tagged) {
        // this lane's logits lane + 64 j < E, and the shared gate (index E) in the same batch
        const int R = E + (has_shared ? 1 : 0);
        const int n = lane < R ? (R - 1 - lane) / 64 + 1 : 0;
        if (lr.race) {
            if (!load_tagged_race<VPL + 1>(lr.tagged + (lane < R ? lane : 0), 64, n, lr.tag, lr.err, lr.race, lr.me,
                                           raw, tmo))
                return SelState{0u, 0u, 0u, false, false};
        } else if (lr.batch)
            tmo = load_tagged_batch<VPL + 1>(lr.tagged + (lane < R ? lane : 0), 64, n, lr.tag, lr.err, raw);
        else
            tmo = load_tagged_many<VPL + 1>(lr.tagged + lane, 64, n, lr.tag, lr.err, raw);
        tmo = __ballot(tmo) != 0;
    } else {
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const int e = lane + 64 * j;
            raw[j] = e < E ? lr.get(e) : 0u;
        }
        raw[VPL] = 0u;
    }
    uint32_t gbits = 0u;  // the shared gate's logit, in every lane
    if (has_shared) {
        if (lr.tagged) {  // index E sits in lane E % 64, slot E / 64
            uint32_t v = raw[0];
#pragma unroll
            for (int j = 1; j <= VPL; ++j)
                if (j == E / 64) v = raw[j];
            gbits = (uint32_t)__builtin_amdgcn_readlane((int)v, E % 64);
        } else {
            gbits = (uint32_t)__builtin_amdgcn_readfirstlane((int)(lane == 0 ? lr.get(E) : 0u));
        }
    }
    uint32_t key[VPL], rv[VPL], id[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        const int e = lane + 64 * j;
        const uint32_t o = e < E ? ordered_logit(__uint_as_float(raw[j])) : 0u;
        key[j] = e < E ? (o > 1u ? o : 1u) : 0u;
        rv[j] = raw[j];
        id[j] = (uint32_t)e;
    }
    // stable odd-even transposition sort of this lane's keys, descending
#pragma unroll
    for (int pass = 0; pass < VPL; ++pass) {
#pragma unroll
        for (int j = pass & 1; j + 1 < VPL; j += 2) {
            const bool sw = key[j + 1] > key[j];
            const uint32_t k0 = key[j], r0 = rv[j], i0 = id[j];
            key[j] = sw ? key[j + 1] : k0;
            rv[j] = sw ? rv[j + 1] : r0;
            id[j] = sw ? id[j + 1] : i0;
            key[j + 1] = sw ? k0 : key[j + 1];
            rv[j + 1] = sw ? r0 : rv[j + 1];
            id[j + 1] = sw ? i0 : id[j + 1];
        }
    }
    uint32_t my_id = 0, my_raw = 0;
    for (int i = 0; i < k; ++i) {
        const uint32_t m = wave_max_u32(key[0]);
        const uint64_t b = __ballot(key[0] == m);
        int wl;
        if (__popcll(b) == 1) {
            wl = __builtin_ctzll(b);
        } else {  // equal leading keys in several lanes: the lowest expert id wins
            const uint32_t mid = wave_ext_u32<false>(key[0] == m ? id[0] : 0xFFFFFFFFu);
            wl = (int)(mid & 63u);
        }
        const uint32_t wid = (uint32_t)__builtin_amdgcn_readlane((int)id[0], wl);
        const uint32_t wraw = (uint32_t)__builtin_amdgcn_readlane((int)rv[0], wl);
        if (lane == wl) {
#pragma unroll
            for (int j = 0; j + 1 < VPL; ++j) {
                key[j] = key[j + 1];
                rv[j] = rv[j + 1];
                id[j] = id[j + 1];
            }
            key[VPL - 1] = 0u;
        }
        if (lane == i) {
            my_id = wid;
            my_raw = wraw;
        }
    }
    my_id = my_id < (uint32_t)E ? my_id : (uint32_t)(E - 1);
    if (lane < k) sel_id[lane] = (int32_t)my_id;
    return SelState{my_id, my_raw, gbits, true, tmo};
}

__device__ __forceinline__ uint16_t select_weights(const SelState& st, int k, int lane) {
    const double li = lane < k ? (double)__uint_as_float(st.raw) : 0.0;
    const double l0 = readlane_f64(li, 0);
    // lanes < k: exp(l_i - l_top); lane k: the shared gate's exp(-g), g = bf16(gate)
    const double g = (double)bf16_to_f32(f32_to_bf16(__uint_as_float(st.gbits)));
    const double ex = exp(lane < k ? li - l0 : -g);
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += readlane_f64(ex, j);
    const double num = lane < k ? ex : 1.0, den = lane < k ? sum : 1.0 + ex;
    return (uint16_t)f64_to_bf16(num / den);
}

template <int VPL>
__device__ __forceinline__ void select_token(const LogitSrc& lr, int E, int k, int has_shared, int lane,
                                             int32_t* sel_id, uint16_t* sel_w, uint16_t* sel_wsh) {
    const SelState st = select_ids<VPL>(lr, E, k, has_shared, lane, sel_id);
    const uint16_t wb = select_weights(st, k, lane);
    if (lane < k) sel_w[lane] = wb;
    if (has_shared && lane == k) *sel_wsh = wb;
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
// and, when `tagged` is given, published with tag `tag` to the two copies
// tagged[t * tstride + r] and tagged[t * tstride + tcopy + r].
// norm_eps >= 0 (one token, TT == 1): the row's input is bf16(RMSNorm(x)) of that
// token, with the scale of rms_scale(row_sumsq); with the 8-bit router and at
// most 4096 activations the squares come from the activations the products load
// (in row_sumsq's order), else from a pass of row_sumsq; xr_out (optional)
// receives that scale.
template <int TT, bool AFF8>
__device__ __forceinline__ void router_row(const uint8_t* __restrict__ router, const float* __restrict__ logit_bias,
                                           const uint16_t* __restrict__ x, int t0, int nt, int H, int R, int E, int r,
                                           int lane, float* logits, bool coherent, uint64_t* tagged, uint32_t tag,
                                           size_t tstride = 0, size_t tcopy = 0, float norm_eps = -1.f,
                                           float* xr_out = nullptr) {
    double acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.0;
    constexpr int EPC = AFF8 ? 16 : 4;  // elements per 16-byte chunk
    constexpr int NCH = 4;                // chunks per lane whose loads are issued together
    constexpr int XW = AFF8 ? 8 : 2;      // activation dwords per chunk and token
    constexpr int TH = TT <= 4 ? TT : 0;  // tokens whose activations are loaded with the weights
    const int C = H / EPC;
    const uint32_t* sb = reinterpret_cast<const uint32_t*>(router + (size_t)R * H);
    const bool norm = TT == 1 && norm_eps >= 0.f;
    const bool norm_regs = AFF8 && H <= 64 * NCH * EPC;  // one pass of the loop holds the whole row
    float xr = 1.f;  // the token's RMSNorm scale
    if (norm && !norm_regs) xr = rms_scale(row_sumsq(x + (size_t)t0 * H, H, lane), H, norm_eps);
    auto xin = [&](uint32_t bits) -> uint32_t { return norm ? norm_bf16(bits, xr) : bits; };
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
        if constexpr (AFF8 && TT == 1) {
            if (norm && norm_regs) {  // lane l holds the 16-element pieces l + 64 c of the token
                float ss = 0.f;
#pragma unroll
                for (int c = 0; c < NCH; ++c)
                    if (j0 + 64 * c < C)
                        ss = sumsq_piece16(make_uint4(xh[c][0][0], xh[c][0][1], xh[c][0][2], xh[c][0][3]),
                                           make_uint4(xh[c][0][4], xh[c][0][5], xh[c][0][6], xh[c][0][7]), ss);
                xr = rms_scale(sumsq_total(ss), H, norm_eps);
            }
        }
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int j = j0 + 64 * c;
            if (j >= C) break;
            const int c0 = j * EPC;
            const uint32_t qw[4] = {wq[c].x, wq[c].y, wq[c].z, wq[c].w};
            double s = 0.0, b = 0.0;
            if constexpr (AFF8) {
                s = (double)bf16_to_f32(wg[c] & 0xFFFFu);
                b = (double)bf16_to_f32(wg[c] >> 16);
            }
            // weight i of the chunk, exact in fp64
            auto wt = [&](int i) -> double {
                if constexpr (AFF8) return s * (double)((qw[i >> 2] >> (8 * (i & 3))) & 0xFFu) + b;
                else return (double)__uint_as_float(qw[i]);
            };
            if constexpr (TH > 0) {
                double wv[EPC];
#pragma unroll
                for (int i = 0; i < EPC; ++i) wv[i] = wt(i);
#pragma unroll
                for (int t = 0; t < TT; ++t) {
                    if (t < nt) {
#pragma unroll
                        for (int i = 0; i < EPC; ++i) {
                            const uint32_t w = xh[c][t < TH ? t : 0][i >> 1];
                            const uint32_t bits = xin((i & 1) ? (w >> 16) : (w & 0xFFFFu));
                            acc[t] = fma((double)bf16_to_f32(bits), wv[i], acc[t]);
                        }
                    }
                }
            } else {
                // many tokens: four weights at a time, each applied to every token
                // (per token the products still accumulate in element order); the
                // scheduling barrier keeps the compiler from hoisting the activation
                // reads of every group at once
#pragma unroll
                for (int g = 0; g < EPC / 4; ++g) {
                    double w4[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) w4[i] = wt(4 * g + i);
#pragma unroll
                    for (int t = 0; t < TT; ++t) {
                        if (t < nt) {
                            const uint2 xv = *reinterpret_cast<const uint2*>(x + (size_t)(t0 + t) * H + c0 + 4 * g);
                            acc[t] = fma((double)bf16_to_f32(xin(xv.x & 0xFFFFu)), w4[0], acc[t]);
                            acc[t] = fma((double)bf16_to_f32(xin(xv.x >> 16)), w4[1], acc[t]);
                            acc[t] = fma((double)bf16_to_f32(xin(xv.y & 0xFFFFu)), w4[2], acc[t]);
                            acc[t] = fma((double)bf16_to_f32(xin(xv.y >> 16)), w4[3], acc[t]);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);  // one group's activation reads in flight at a time
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = wave_sum_f64(acc[t]);
    if (norm && xr_out && lane == 0) *xr_out = xr;
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
                if (tagged) {
                    uint64_t* p = tagged + (size_t)(t0 + t) * tstride + r;
                    store_tagged(p, tag, v);
                    store_tagged(p + tcopy, tag, v);
                }
            }
    }
}

}  // namespace moe

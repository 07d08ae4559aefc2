// Decode path: int4 expert GEMVs for 1..16 token rows (the GEMV MoE path at
// batch 1 of the AGX Orin port, "Phase 1-4"; row windows of 1 to 16 of TensorFold
// issue #931, "What I'd build"). Expert gate/up pair with SwiGLU, then down.
//
// Data movement: every weight row is streamed once with 16-byte loads; a
// wavefront covers a 2048-wide int4 row with one 1 KiB load; every weight load of
// a work item is issued before the first is consumed. Each lane keeps its slice
// of the activation row in registers, so the HBM traffic is the weights.
//
// Arithmetic (exact weights): a group's weights are scale*q + bias. A lane's 32
// activations x meet the 32 nibbles q of the same group through
//   sum x*(scale*q + bias) = 16*scale * sum x*(1 + q/16) + (bias - 16*scale) * sum x,
// where 1 + q/16 is exactly a bf16 whose mantissa is q (one shift and one
// and-or per two weights; the packed nibble order makes the pairs line up with
// the activations as stored) and sum x*(1 + q/16) is a chain of bf16 dot2
// instructions accumulating in fp32.
#include <algorithm>

#include "moe_internal.h"
#include "route_device.h"
#include "route_internal.h"

namespace moe {

template <int CPL>
struct XSlice {
    uint32_t p[CPL][16];  // 32 bf16 per chunk as 16 natural-order pairs
    float s[CPL];         // plain sum of the chunk's 32 values, in element order
};

// Chunk c of this lane covers elements [32 * (lr + lpr * c), +32) of the row. The
// chunk sum is a chain of bf16 dot2 against (1, 1), in element order.
template <int CPL>
__device__ __forceinline__ void load_xslice(const uint16_t* __restrict__ row, int lr, int lpr, XSlice<CPL>& xs) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const uint4* src = reinterpret_cast<const uint4*>(row + 32 * (lr + lpr * c));
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const uint4 v = src[q4];
            xs.p[c][4 * q4 + 0] = v.x;
            xs.p[c][4 * q4 + 1] = v.y;
            xs.p[c][4 * q4 + 2] = v.z;
            xs.p[c][4 * q4 + 3] = v.w;
        }
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) sum = dot2_bf16(xs.p[c][j], 0x3F803F80u, sum);
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
// activation chunk xp (natural-order pairs) whose plain sum is xsum.
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

// ---------------------------------------------------------------- gate/up work item
// 16 intermediate rows (gate row and up row each) of expert e for one token, by
// one workgroup: wavefront w owns rows rb*16 + 4w .. +4.
constexpr int GU_ROWS = 16;
constexpr int GU_IT = 4;  // row iterations per wavefront (rows per iteration = 64 / lanes per row)

// A gate/up item's weight loads (issued by gu_load, consumed by gu_finish).
template <int CPL>
struct GuLoads {
    ChunkLoad g[GU_IT][CPL], u[GU_IT][CPL];
};

template <int CPL>
__device__ __forceinline__ void gu_load(const uint8_t* __restrict__ packed, const ExpertLayout& L, int H, int e,
                                        bool valid, int rb, int wave, int lane, GuLoads<CPL>& ld) {
    if (!valid) return;
    const int C = H / 32, lpr = C < 64 ? C : 64, rpw = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    constexpr int per_wave = GU_ROWS / 4;
    const int r0 = rb * GU_ROWS + wave * per_wave;
    const uint8_t* base = packed + (size_t)e * L.stride;
    const uint8_t* gq = base + L.gate_q;
    const uint8_t* uq = base + L.up_q;
    const uint32_t* gsb = reinterpret_cast<const uint32_t*>(base + L.gate_sb);
    const uint32_t* usb = reinterpret_cast<const uint32_t*>(base + L.up_sb);
    const size_t qstride = H / 2, sbstride = H / 64;
#pragma unroll
    for (int it = 0; it < GU_IT; ++it) {
        const int rr = it * rpw + rsub;
        const int r = r0 + (rr < per_wave ? rr : 0);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            if (rr < per_wave) {
                ld.g[it][c] = load_chunk(gq + r * qstride, gsb + r * sbstride, lr + lpr * c);
                ld.u[it][c] = load_chunk(uq + r * qstride, usb + r * sbstride, lr + lpr * c);
            }
        }
    }
}

// Rows rb*16 + 4*wave .. +4 of h = bf16(silu(gate . x) * (up . x)), written to hrow
// or, with htag (the tagged copy of the same h row, one 64-bit word per bf16
// pair), published there with tag `tag`.
template <int CPL>
__device__ __forceinline__ void gu_finish(const GuLoads<CPL>& ld, int H, bool valid,
                                          const uint16_t* __restrict__ xrow, uint16_t* __restrict__ hrow,
                                          uint64_t* htag, uint32_t tag, int rb, int wave, int lane) {
    const int C = H / 32, lpr = C < 64 ? C : 64, rpw = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    constexpr int per_wave = GU_ROWS / 4;
    const int r0 = rb * GU_ROWS + wave * per_wave;
    uint32_t* hrow32 = reinterpret_cast<uint32_t*>(hrow + r0);  // r0 is even: 4 rows = 2 dwords
    if (!valid) {
        if (lane < 2) {
            if (htag)
                store_tagged(htag + r0 / 2 + lane, tag, 0u);
            else
                hrow32[lane] = 0u;
        }
        return;
    }
    XSlice<CPL> xs;
    load_xslice(xrow, lr, lpr, xs);
    uint32_t hb[GU_IT] = {0u, 0u, 0u, 0u};  // bf16 of row it*rpw + rsub, in lanes with lr == 0
#pragma unroll
    for (int it = 0; it < GU_IT; ++it) {
        const int rr = it * rpw + rsub;
        if (it * rpw >= per_wave) break;  // wave-uniform
        const bool act = rr < per_wave;
        float g = 0.f, u = 0.f;
        if (act) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                g += chunk_dot(ld.g[it][c], xs.p[c], xs.s[c]);
                u += chunk_dot(ld.u[it][c], xs.p[c], xs.s[c]);
            }
        }
        g = group_sum(g, lpr);
        u = group_sum(u, lpr);
        hb[it] = f32_to_bf16(silu_f32(g) * u);
    }
    // gather the wavefront's 4 rows (row q sits in the last lane of group q % rpw,
    // iteration q / rpw)
    uint32_t r4[per_wave];
#pragma unroll
    for (int q = 0; q < per_wave; ++q) {
        const int it = q / rpw;
        const uint32_t v = it == 0 ? hb[0] : it == 1 ? hb[1] : it == 2 ? hb[2] : hb[3];
        r4[q] = (uint32_t)__builtin_amdgcn_readlane((int)v, (q % rpw) * lpr + lpr - 1);
    }
    if (lane < 2) {
        const uint32_t v = lane == 0 ? (r4[0] | (r4[1] << 16)) : (r4[2] | (r4[3] << 16));
        if (htag)
            store_tagged(htag + r0 / 2 + lane, tag, v);
        else
            hrow32[lane] = v;
    }
}

// 16 intermediate rows of expert e for one token (gate and up rows each).
template <int CPL>
__device__ __forceinline__ void gateup_item(const uint8_t* __restrict__ packed, const ExpertLayout& L, int H, int e,
                                            bool valid, const uint16_t* __restrict__ xrow,
                                            uint16_t* __restrict__ hrow, uint64_t* htag, uint32_t tag, int rb,
                                            int wave, int lane) {
    GuLoads<CPL> ld;
    gu_load<CPL>(packed, L, H, e, valid, rb, wave, lane, ld);
    gu_finish<CPL>(ld, H, valid, xrow, hrow, htag, tag, rb, wave, lane);
}

// ---------------------------------------------------------------- down (+ combine) work item
// Output rows n0 .. n0+7 of token t for every slot s (S*8 row dot products of
// length I, I/32 lanes each) by one workgroup. Results go to LDS (ysh), then to
// y[t][s][n] when y is given, and
//   out[t][n] = bf16(sum_{s<k} w[s] * y[s][n] + wsh * y[k][n])
// (then bf16(residual + out)) when out is given, with the same fp32 slot-order
// arithmetic as moe_combine. The weight loads depend only on the expert ids, so
// they are issued first; with WAIT the workgroup then waits until *ready >= target
// (the h rows of token t are complete) before it reads h.
constexpr int DN_ROWS = 8;
constexpr int DN_BATCH = 5;  // 9 slots x 8 rows at I = 512: 18 iterations, 4.5 per wavefront

// A down item's weight loads for one batch of DN_BATCH row iterations per
// wavefront; they depend only on the expert ids, so a workgroup can issue the
// first batch early (before its last gate/up item is computed).
struct DnLoads {
    ChunkLoad ld[DN_BATCH];
    int slot[DN_BATCH];
    bool ok[DN_BATCH];
};

__device__ __forceinline__ void dn_load(const uint8_t* __restrict__ packed, const ExpertLayout& L, int I, int E,
                                        int k, int has_shared, int n0, const int32_t* ids_t, int j0, DnLoads& d) {
    const int S = k + has_shared;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lpr = I / 32, rpw = 64 / lpr;  // I <= 2048: one chunk per lane
    const int lr = lane % lpr, rsub = lane / lpr;
    const int n_dots = S * DN_ROWS;
    const int n_it = (n_dots + rpw - 1) / rpw;
    const size_t qstride = I / 2, sbstride = I / 64;
#pragma unroll
    for (int j = 0; j < DN_BATCH; ++j) {
        const int it = wave + 4 * (j0 + j);
        const int q = it * rpw + rsub;
        d.ok[j] = it < n_it && q < n_dots;
        d.slot[j] = d.ok[j] ? q / DN_ROWS : 0;
        if (d.ok[j]) {
            const int s = d.slot[j];
            const int e = s < k ? ids_t[s] : E;
            if (s < k && (e < 0 || e >= E)) {
                d.ok[j] = false;  // invalid expert id: this y row is zero
            } else {
                const int n = n0 + q % DN_ROWS;
                const uint8_t* base = packed + (size_t)e * L.stride;
                d.ld[j] = load_chunk(base + L.down_q + n * qstride,
                                     reinterpret_cast<const uint32_t*>(base + L.down_sb) + n * sbstride, lr);
            }
        }
    }
}

// hsh: LDS of S * I bf16, the token's h rows of every slot, staged with one round
// of parallel loads before the dot products. With TAGGED the rows are read from
// their tagged copy (published in this launch), each word polled until it carries
// `tag`. d holds the first batch's weight loads (dn_load with j0 = 0).
template <bool TAGGED>
__device__ __forceinline__ void dn_finish(DnLoads& d, const uint8_t* __restrict__ packed, const ExpertLayout& L,
                                          int H, int I, int E, int k, int has_shared, int t, int n0,
                                          const uint16_t* __restrict__ hbuf, const int32_t* ids_t,
                                          const uint16_t* w_t, const uint16_t* wsh_t, float* __restrict__ y,
                                          const uint16_t* residual, uint16_t* out, float (*ysh)[DN_ROWS],
                                          uint32_t* hsh, const uint64_t* htag_t, uint32_t tag, unsigned* err) {
    const int S = k + has_shared;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lpr = I / 32, rpw = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    const int n_dots = S * DN_ROWS;
    const int n_it = (n_dots + rpw - 1) / rpw;
    for (int j0 = 0; 4 * j0 < n_it; j0 += DN_BATCH) {
        if (j0 > 0) dn_load(packed, L, I, E, k, has_shared, n0, ids_t, j0, d);
        if (j0 == 0) {
            const int nw = S * I / 2;
            if (TAGGED) {
                for (int i0 = threadIdx.x; i0 < nw; i0 += 256 * 16) {
                    uint32_t v[16];
                    const int n = min(16, (nw - 1 - i0) / 256 + 1);
                    load_tagged_many<16>(htag_t + i0, 256, n, tag, err, v);
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        if (j < n) hsh[i0 + 256 * j] = v[j];
                }
            } else {
                const uint32_t* src = reinterpret_cast<const uint32_t*>(hbuf + (size_t)t * S * I);
                for (int i = threadIdx.x; i < nw; i += 256) hsh[i] = src[i];
            }
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < DN_BATCH; ++j) {
            const int it = wave + 4 * (j0 + j);
            if (it >= n_it) break;  // wave-uniform
            const int q = it * rpw + rsub;
            float v = 0.f;
            if (d.ok[j]) {
                XSlice<1> hs;
                load_xslice(reinterpret_cast<const uint16_t*>(hsh) + (size_t)d.slot[j] * I, lr, lpr, hs);
                v = chunk_dot(d.ld[j], hs.p[0], hs.s[0]);
            }
            v = group_sum(v, lpr);
            if (lr == lpr - 1 && q < n_dots) ysh[q / DN_ROWS][q % DN_ROWS] = v;
        }
    }
    __syncthreads();
    const int tid = threadIdx.x;
    if (y) {
        for (int i = tid; i < n_dots; i += 256)
            y[((size_t)t * S + i / DN_ROWS) * H + n0 + i % DN_ROWS] = ysh[i / DN_ROWS][i % DN_ROWS];
    }
    if (out && tid < DN_ROWS) {
        float a = 0.f;
        for (int s = 0; s < k; ++s) a = fmaf(bf16_to_f32(w_t[s]), ysh[s][tid], a);
        if (has_shared) a = fmaf(bf16_to_f32(*wsh_t), ysh[k][tid], a);
        uint32_t b = f32_to_bf16(a);
        const size_t o = (size_t)t * H + n0 + tid;
        if (residual) b = f32_to_bf16(bf16_to_f32(residual[o]) + bf16_to_f32(b));
        out[o] = (uint16_t)b;
    }
    __syncthreads();  // ysh is reused by the next item
}

// ---------------------------------------------------------------- two-launch expert stage
// Grid (I / 16, S, T): one gate/up item per workgroup.
template <int CPL>
__global__ __launch_bounds__(256) void decode_gateup_kernel(const uint8_t* __restrict__ packed, ExpertLayout L, int H,
                                                            int I, int E, int k, int has_shared,
                                                            const uint16_t* __restrict__ x,
                                                            const int32_t* __restrict__ ids,
                                                            uint16_t* __restrict__ hbuf) {
    const int t = blockIdx.z, s = blockIdx.y, S = k + has_shared;
    const int e = s < k ? ids[(size_t)t * k + s] : E;
    const bool valid = s < k ? (e >= 0 && e < E) : true;
    gateup_item<CPL>(packed, L, H, e, valid, x + (size_t)t * H, hbuf + ((size_t)t * S + s) * I, nullptr, 0u,
                     blockIdx.x, threadIdx.x >> 6, threadIdx.x & 63);
}

// Grid (H / 8, T): one down item per workgroup; combine when out is given.
__global__ __launch_bounds__(256) void decode_down_kernel(const uint8_t* __restrict__ packed, ExpertLayout L, int H,
                                                          int I, int E, int k, int has_shared,
                                                          const uint16_t* __restrict__ hbuf,
                                                          const int32_t* __restrict__ ids, float* __restrict__ y,
                                                          const uint16_t* __restrict__ w,
                                                          const uint16_t* __restrict__ wsh, const uint16_t* residual,
                                                          uint16_t* out) {
    __shared__ float ysh[17][DN_ROWS];
    extern __shared__ __attribute__((aligned(16))) uint32_t hsh_dyn[];
    const int t = blockIdx.y;
    DnLoads d;
    dn_load(packed, L, I, E, k, has_shared, blockIdx.x * DN_ROWS, ids + (size_t)t * k, 0, d);
    dn_finish<false>(d, packed, L, H, I, E, k, has_shared, t, blockIdx.x * DN_ROWS, hbuf, ids + (size_t)t * k,
                     w ? w + (size_t)t * k : nullptr, wsh ? wsh + t : nullptr, y, residual, out, ysh, hsh_dyn,
                     nullptr, 0u, nullptr);
}

// ---------------------------------------------------------------- single-launch decode layer
// Control words in the workspace. A launch publishes with tag epoch + 1; the last
// workgroup to leave stores the new epoch, so stale words of earlier launches never
// carry the current tag and nothing has to be cleared between launches.
struct DecodeCtl {
    unsigned epoch;       // tag of the last completed launch
    unsigned exit_count;  // workgroups finished (back to zero after each launch)
    unsigned error;       // a bounded poll timed out (sticky)
    unsigned pad;
};

struct LayerArgs {
    const uint8_t* router;
    const float* logit_bias;
    const uint8_t* experts;
    const uint16_t* x;
    float* logits;
    int32_t* ids;
    uint16_t* w;
    uint16_t* wsh;
    float* y;
    const uint16_t* residual;
    uint16_t* out;
    DecodeCtl* ctl;
    uint64_t* tlogits;  // tagged logits [T][R]
    uint64_t* th;       // tagged h [T][S][I/2] (bf16 pairs)
    ExpertLayout L;
    int T, H, I, E, k, has_shared, R;
};

// Persistent kernel, at most one workgroup per CU, every workgroup resident.
// Work items (token-minor numbering; item i of a phase goes to workgroup i mod G):
//   A: router rows (4 per item) and the shared expert's gate/up items, which do
//      not depend on routing;
//   B: the routed gate/up items (16 rows of one token, one slot);
//   C: down items (8 output rows of one token, all slots) with the combine.
// Every workgroup computes the selection of the tokens it needs (DPP top-k, reading
// the tagged logits as they arrive) into LDS before its B items. The first C
// item's down-weight loads go out with the last B item's gate/up loads; a C item
// then stages its token's tagged h rows (polling each word).
template <int CPL, int TT, bool AFF8>
__global__ __launch_bounds__(256) void decode_layer_kernel(LayerArgs a) {
    __shared__ int32_t s_ids[16][16];
    __shared__ uint16_t s_w[16][16];
    __shared__ uint16_t s_wsh[16];
    __shared__ float ysh[17][DN_ROWS];
    extern __shared__ __attribute__((aligned(16))) uint32_t hsh_dyn[];
    const int G = gridDim.x, wg = blockIdx.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int T = a.T, H = a.H, I = a.I, E = a.E, k = a.k, R = a.R;
    const int S = k + a.has_shared;
    DecodeCtl* ctl = a.ctl;
    const uint32_t tag = load_coherent(&ctl->epoch) + 1u;
    const int n_router = (R + 3) / 4;
    const int gu_per_tok = I / GU_ROWS;
    const int n_shared = a.has_shared ? T * gu_per_tok : 0;
    const int n_A = n_router + n_shared;
    const int n_B = T * k * gu_per_tok;
    const int n_C = T * (H / DN_ROWS);

    // ---- phase A
    for (int item = wg; item < n_A; item += G) {
        if (item < n_router) {
            const int r = item * 4 + wave;
            if (r < R)
                router_row<TT, AFF8>(a.router, a.logit_bias, a.x, 0, T, H, R, E, r, lane, a.logits, false, a.tlogits,
                                     tag);
        } else {
            const int j = item - n_router, t = j % T, rb = j / T;
            const size_t row = (size_t)t * S + k;
            gateup_item<CPL>(a.experts, a.L, H, E, true, a.x + (size_t)t * H, nullptr, a.th + row * (I / 2), tag,
                             rb, wave, lane);
        }
    }

    // ---- selection of the tokens this workgroup needs
    uint32_t need = 0;
    for (int item = wg; item < n_B; item += G) need |= 1u << (item % T);
    for (int item = wg; item < n_C; item += G) need |= 1u << (item % T);
    if (wg < T) need |= 1u << wg;
    for (int t = 0, c = 0; t < T; ++t) {
        if (need >> t & 1u) {
            if ((c & 3) == wave) {
                const LogitSrc src{nullptr, a.tlogits + (size_t)t * R, tag, &ctl->error, false};
                select_token_any(src, E, k, a.has_shared, lane, s_ids[t], s_w[t], &s_wsh[t]);
            }
            ++c;
        }
    }
    __syncthreads();
    if (wg < T) {
        if (tid < k) {
            a.ids[(size_t)wg * k + tid] = s_ids[wg][tid];
            a.w[(size_t)wg * k + tid] = s_w[wg][tid];
        }
        if (a.has_shared && tid == 0) a.wsh[wg] = s_wsh[wg];
    }

    // ---- phase B (the first down item's weight loads are issued with the last
    // gate/up item's, so they overlap its arithmetic and the wait for h)
    DnLoads dl;
    bool dl_ready = false;
    for (int item = wg; item < n_B; item += G) {
        const int t = item % T, j = item / T, s = j / gu_per_tok, rb = j % gu_per_tok;
        const size_t row = (size_t)t * S + s;
        GuLoads<CPL> gl;
        gu_load<CPL>(a.experts, a.L, H, s_ids[t][s], true, rb, wave, lane, gl);
        if (item + G >= n_B && wg < n_C) {
            const int tc = wg % T;
            dn_load(a.experts, a.L, I, E, k, a.has_shared, (wg / T) * DN_ROWS, s_ids[tc], 0, dl);
            dl_ready = true;
        }
        gu_finish<CPL>(gl, H, true, a.x + (size_t)t * H, nullptr, a.th + row * (I / 2), tag, rb, wave, lane);
    }

    // ---- phase C
    for (int item = wg; item < n_C; item += G) {
        const int t = item % T, ng = item / T;
        if (!dl_ready) dn_load(a.experts, a.L, I, E, k, a.has_shared, ng * DN_ROWS, s_ids[t], 0, dl);
        dl_ready = false;
        dn_finish<true>(dl, a.experts, a.L, H, I, E, k, a.has_shared, t, ng * DN_ROWS, nullptr, s_ids[t], s_w[t],
                        &s_wsh[t], a.y, a.residual, a.out, ysh, hsh_dyn, a.th + (size_t)t * S * (I / 2), tag,
                        &ctl->error);
    }

    // ---- exit: the last workgroup out publishes the new epoch
    __syncthreads();
    if (tid == 0) {
        if (atomicAdd(&ctl->exit_count, 1u) == (unsigned)G - 1) {
            atomicExch(&ctl->exit_count, 0u);
            atomicExch(&ctl->epoch, tag);
        }
    }
}

static int cpl_for(int K) { return K / 32 <= 64 ? 1 : (K / 32) / 64; }

static void launch_gateup(const moe_shape& sh, const ExpertLayout& L, const uint8_t* p, const uint16_t* x, int T,
                          const int32_t* ids, uint16_t* hbuf, hipStream_t hs) {
    const int S = n_slots(sh), H = sh.hidden, I = sh.inter;
    dim3 g1(I / GU_ROWS, S, T);
    switch (cpl_for(H)) {
        case 1: hipLaunchKernelGGL(decode_gateup_kernel<1>, g1, dim3(256), 0, hs, p, L, H, I, sh.n_experts, sh.top_k,
                                   sh.has_shared, x, ids, hbuf); break;
        case 2: hipLaunchKernelGGL(decode_gateup_kernel<2>, g1, dim3(256), 0, hs, p, L, H, I, sh.n_experts, sh.top_k,
                                   sh.has_shared, x, ids, hbuf); break;
        default: hipLaunchKernelGGL(decode_gateup_kernel<4>, g1, dim3(256), 0, hs, p, L, H, I, sh.n_experts, sh.top_k,
                                    sh.has_shared, x, ids, hbuf); break;
    }
}

static int device_cus() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (!cache[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev] = n;
    }
    return cache[dev];
}

// LDS for one token's h rows of every slot.
static size_t hsh_bytes(const moe_shape& sh) { return (size_t)n_slots(sh) * sh.inter * 2; }

template <int CPL, int TT>
static void launch_layer_tt(const LayerArgs& a, bool aff8, int G, size_t lds, hipStream_t hs) {
    if (aff8)
        hipLaunchKernelGGL((decode_layer_kernel<CPL, TT, true>), dim3(G), dim3(256), lds, hs, a);
    else
        hipLaunchKernelGGL((decode_layer_kernel<CPL, TT, false>), dim3(G), dim3(256), lds, hs, a);
}

template <int CPL>
static void launch_layer(const LayerArgs& a, bool aff8, int G, size_t lds, hipStream_t hs) {
    if (a.T <= 1) launch_layer_tt<CPL, 1>(a, aff8, G, lds, hs);
    else if (a.T <= 4) launch_layer_tt<CPL, 4>(a, aff8, G, lds, hs);
    else launch_layer_tt<CPL, 16>(a, aff8, G, lds, hs);
}

}  // namespace moe

using namespace moe;

static size_t hbuf_bytes(const moe_shape& sh, int T) { return align_up((size_t)T * n_slots(sh) * sh.inter * 2, 256); }

// Workspace: h rows (bf16) | control words (256 B) | tagged logits | tagged h.
struct DecodeWs {
    size_t ctl, tlogits, th, total;
};

static DecodeWs decode_ws_layout(const moe_shape& sh, int T) {
    DecodeWs w;
    w.ctl = hbuf_bytes(sh, T);
    w.tlogits = w.ctl + 256;
    w.th = w.tlogits + align_up((size_t)T * router_rows(sh) * 8, 256);
    w.total = w.th + align_up((size_t)T * n_slots(sh) * (sh.inter / 2) * 8, 256);
    return w;
}

extern "C" size_t moe_decode_workspace_bytes(const moe_shape* shape, int32_t T) {
    if (validate_shape(shape) != MOE_OK || T < 1) return 0;
    return decode_ws_layout(*shape, T).total;
}

static moe_status check_decode_args(const moe_shape* shape, const void* experts_packed, const uint16_t* x, int T,
                                    const void* ws, size_t ws_bytes) {
    moe_status st = validate_shape(shape);
    if (st != MOE_OK) return st;
    if (T < 1 || T > 16) return fail(MOE_ERR_INVALID_ARG, "decode path takes 1..16 rows, got T = %d", T);
    if (!experts_packed || !x || !ws || !aligned16(experts_packed) || !aligned16(x) || !aligned16(ws))
        return fail(MOE_ERR_INVALID_ARG, "NULL or unaligned pointer");
    if (ws_bytes < moe_decode_workspace_bytes(shape, T)) return fail(MOE_ERR_WORKSPACE, "decode workspace too small");
    if (hsh_bytes(*shape) > 65536)
        return fail(MOE_ERR_UNSUPPORTED, "decode path: (top_k + shared) * inter * 2 bytes must fit 64 KiB of LDS");
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
    hipLaunchKernelGGL(decode_down_kernel, dim3(sh.hidden / DN_ROWS, T), dim3(256), hsh_bytes(sh), hs, p, L, sh.hidden,
                       sh.inter,
                       sh.n_experts, sh.top_k, sh.has_shared, hbuf, ids, y, (const uint16_t*)nullptr,
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
    if (cpl_for(sh.hidden) > 2) return fail(MOE_ERR_UNSUPPORTED, "single-launch decode layer serves hidden <= 4096");
    const int cus = device_cus();
    if (cus <= 0) return fail(MOE_ERR_HIP, "could not query the compute-unit count");
    hipStream_t hs = (hipStream_t)stream;
    LayerArgs a;
    a.router = (const uint8_t*)router_packed;
    a.logit_bias = logit_bias;
    a.experts = (const uint8_t*)experts_packed;
    a.x = x;
    a.logits = logits;
    a.ids = ids;
    a.w = w;
    a.wsh = w_shared;
    a.y = y;
    a.residual = residual;
    a.out = out;
    const DecodeWs W = decode_ws_layout(sh, T);
    a.ctl = (DecodeCtl*)((char*)ws + W.ctl);
    a.tlogits = (uint64_t*)((char*)ws + W.tlogits);
    a.th = (uint64_t*)((char*)ws + W.th);
    a.L = expert_layout(sh);
    a.T = T;
    a.H = sh.hidden;
    a.I = sh.inter;
    a.E = sh.n_experts;
    a.k = sh.top_k;
    a.has_shared = sh.has_shared;
    a.R = router_rows(sh);
    const int n_router = (a.R + 3) / 4;
    const int n_A = n_router + (sh.has_shared ? T * (a.I / GU_ROWS) : 0);
    const int items = std::max(std::max(n_A, T * sh.top_k * (a.I / GU_ROWS)), T * (a.H / DN_ROWS));
    const int G = std::min(cus, items);
    const bool aff8 = sh.router_fmt == MOE_ROUTER_AFFINE8;
    if (cpl_for(sh.hidden) == 1) launch_layer<1>(a, aff8, G, hsh_bytes(sh), hs);
    else launch_layer<2>(a, aff8, G, hsh_bytes(sh), hs);
    return check_launch("decode_layer_kernel");
}

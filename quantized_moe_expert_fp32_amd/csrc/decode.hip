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
#include <map>
#include <mutex>

#include "moe_internal.h"
#include "route_device.h"
#include "route_internal.h"

namespace moe {

template <int CPL>
struct XSlice {
    uint32_t p[CPL][16];  // 32 bf16 per chunk as 16 natural-order pairs
    float s[CPL];         // plain sum of the chunk's 32 values, in element order
};

// Chunk c of this lane covers weights [32 * (lr + lpr * c), +32) of a weight row,
// whose activations are elements [32 * ch, +32) of the activation row, ch = (lr +
// lpr * c) mod xc (xc: chunks of the activation row; a weight row of 8-bit codes
// is twice as long as its activations). The chunk sum is a chain of bf16 dot2
// against (1, 1), in element order.
template <int CPL>
__device__ __forceinline__ void load_xslice(const uint16_t* __restrict__ row, int lr, int lpr, int xc,
                                            XSlice<CPL>& xs) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        int ch = lr + lpr * c;
        if (ch >= xc) ch -= xc;
        const uint4* src = reinterpret_cast<const uint4*>(row + 32 * ch);
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

// qrow, sbrow: a row's bases in the blocked packed layout (gu_row_q / gu_row_sb,
// dn_row_q / dn_row_sb); chunk = 16-byte piece of 32 weights.
__device__ __forceinline__ ChunkLoad load_chunk(const uint8_t* __restrict__ qrow, const uint32_t* __restrict__ sbrow,
                                                int chunk) {
    ChunkLoad c;
    c.q = *reinterpret_cast<const uint4*>(qrow + piece_off(chunk));
    c.sb = sbrow[4 * (chunk >> 1)];
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
#pragma unroll
    for (int it = 0; it < GU_IT; ++it) {
        const int rr = it * rpw + rsub;
        const int r = r0 + (rr < per_wave ? rr : 0);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            if (rr < per_wave) {
                ld.g[it][c] = load_chunk(base + gu_row_q(L, H, 0, r),
                                         reinterpret_cast<const uint32_t*>(base + gu_row_sb(L, H, 0, r)), lr + lpr * c);
                ld.u[it][c] = load_chunk(base + gu_row_q(L, H, 1, r),
                                         reinterpret_cast<const uint32_t*>(base + gu_row_sb(L, H, 1, r)), lr + lpr * c);
            }
        }
    }
}

// Rows rb*16 + 4*wave .. +4 of h = bf16(silu(gate . x) * (up . x)), written to hrow
// or, with htag (the tagged copy of the same h row, one 64-bit word per bf16
// pair), published there with tag `tag`.
template <int CPL>
__device__ __forceinline__ void gu_finish(const GuLoads<CPL>& ld, int H, int xc, bool valid,
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
    load_xslice(xrow, lr, lpr, xc, xs);
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

// 16 intermediate rows of expert e for one token (gate and up rows each); H is the
// weight row length, xc the activation row's chunks of 32.
template <int CPL>
__device__ __forceinline__ void gateup_item(const uint8_t* __restrict__ packed, const ExpertLayout& L, int H, int xc,
                                            int e, bool valid, const uint16_t* __restrict__ xrow,
                                            uint16_t* __restrict__ hrow, uint64_t* htag, uint32_t tag, int rb,
                                            int wave, int lane) {
    GuLoads<CPL> ld;
    gu_load<CPL>(packed, L, H, e, valid, rb, wave, lane, ld);
    gu_finish<CPL>(ld, H, xc, valid, xrow, hrow, htag, tag, rb, wave, lane);
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
                d.ld[j] = load_chunk(base + dn_row_q(L, I, n),
                                     reinterpret_cast<const uint32_t*>(base + dn_row_sb(L, I, n)), lr);
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
                                          int H, int I, int Iw, int E, int k, int has_shared, int t, int n0,
                                          const uint16_t* __restrict__ hbuf, const int32_t* ids_t,
                                          const uint16_t* w_t, const uint16_t* wsh_t, float* __restrict__ y,
                                          const uint16_t* residual, uint16_t* out, float (*ysh)[DN_ROWS],
                                          uint32_t* hsh, const uint64_t* htag_t, uint32_t tag, unsigned* err) {
    const int S = k + has_shared;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lpr = Iw / 32, rpw = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    const int n_dots = S * DN_ROWS;
    const int n_it = (n_dots + rpw - 1) / rpw;
    for (int j0 = 0; 4 * j0 < n_it; j0 += DN_BATCH) {
        if (j0 > 0) dn_load(packed, L, Iw, E, k, has_shared, n0, ids_t, j0, d);
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
                load_xslice(reinterpret_cast<const uint16_t*>(hsh) + (size_t)d.slot[j] * I, lr, lpr, I / 32, hs);
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
// km: weight row length / activation length (1 for 4-bit experts, 2 for 8-bit).
template <int CPL>
__global__ __launch_bounds__(256) void decode_gateup_kernel(const uint8_t* __restrict__ packed, ExpertLayout L, int H,
                                                            int I, int km, int E, int k, int has_shared,
                                                            const uint16_t* __restrict__ x,
                                                            const int32_t* __restrict__ ids,
                                                            uint16_t* __restrict__ hbuf) {
    const int t = blockIdx.z, s = blockIdx.y, S = k + has_shared;
    const int e = s < k ? ids[(size_t)t * k + s] : E;
    const bool valid = s < k ? (e >= 0 && e < E) : true;
    gateup_item<CPL>(packed, L, H * km, H / 32, e, valid, x + (size_t)t * H, hbuf + ((size_t)t * S + s) * I, nullptr,
                     0u, blockIdx.x, threadIdx.x >> 6, threadIdx.x & 63);
}

// Grid (H / 8, T): one down item per workgroup; combine when out is given.
__global__ __launch_bounds__(256) void decode_down_kernel(const uint8_t* __restrict__ packed, ExpertLayout L, int H,
                                                          int I, int km, int E, int k, int has_shared,
                                                          const uint16_t* __restrict__ hbuf,
                                                          const int32_t* __restrict__ ids, float* __restrict__ y,
                                                          const uint16_t* __restrict__ w,
                                                          const uint16_t* __restrict__ wsh, const uint16_t* residual,
                                                          uint16_t* out) {
    __shared__ float ysh[17][DN_ROWS];
    extern __shared__ __attribute__((aligned(16))) uint32_t hsh_dyn[];
    const int t = blockIdx.y;
    DnLoads d;
    dn_load(packed, L, I * km, E, k, has_shared, blockIdx.x * DN_ROWS, ids + (size_t)t * k, 0, d);
    dn_finish<false>(d, packed, L, H, I, I * km, E, k, has_shared, t, blockIdx.x * DN_ROWS, hbuf, ids + (size_t)t * k,
                     w ? w + (size_t)t * k : nullptr, wsh ? wsh + t : nullptr, y, residual, out, ysh, hsh_dyn,
                     nullptr, 0u, nullptr);
}

// ---------------------------------------------------------------- single-launch decode layer
// Control words in the workspace. A launch publishes with tag epoch + 1. Each
// workgroup counts itself in once all of its wavefronts have read the epoch; the
// one that counts last stores the new epoch as it leaves, so stale words of earlier
// launches never carry the current tag and nothing has to be cleared between
// launches.
struct DecodeCtl {
    unsigned epoch;       // tag of the last completed launch
    unsigned exit_count;  // groups of workgroups that have all read the epoch (back to zero after each launch)
    unsigned error;       // a bounded poll timed out (sticky)
    unsigned pad[29];
    struct {
        unsigned count;  // workgroups wg with wg % 8 == g that have read the epoch
        unsigned pad[31];
    } group[8];
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
    uint64_t* tlogits;  // tagged logits: token t's copy c at tlogits + t * tl_stride + c * tl_copy
    size_t tl_stride, tl_copy;  // in words
    uint64_t* th;       // tagged h [T][S][I/2] (bf16 pairs); one token: two copies, th_word
    ExpertLayout L;
    int T, H, I, E, k, has_shared, R;
    int kmul;     // weight row length / activation length: 1 (4-bit experts) or 2 (8-bit)
    int stage_x;  // x and its chunk sums are staged in LDS (else read from global memory)
    float norm_eps;  // >= 0: the layer's input is bf16(RMSNorm(x)) (needs stage_x); < 0: x as given
};

// Tagged h of one token: word w in copy c (0, 1) sits at th_word(w, c). Blocks of
// 1024 words (8 KiB) alternate between the copies, so with a 16 KiB-aligned base
// the two copies of a word are 8 KiB apart, on the chip's two halves.
__device__ __forceinline__ size_t th_word(size_t w, int c) { return (w >> 10) * 2048 + (size_t)c * 1024 + (w & 1023); }

// ---- single-launch building blocks (16 wavefronts per workgroup)
constexpr int LW = 16;        // wavefronts per workgroup
constexpr int LTH = 64 * LW;  // threads per workgroup
constexpr int DNB = 3;        // down row iterations per wavefront whose loads are issued together
constexpr int MAXD = 272;     // distinct experts of one launch: at most 16 * 16 routed, plus the shared one

// Gate/up row-pair task: rows 2ip and 2ip+1 of the gate and up matrices of one
// expert. Row slot rs: 0, 1 = gate rows 2ip, 2ip+1; 2, 3 = up rows. The lane
// layout of a row (lpr lanes, CPL chunks of 32 each) and the arithmetic are those
// of gateup_item, so h is bit-identical between the decode entry points.
template <int CPL>
struct PairLoads {
    ChunkLoad c[4][CPL];
};

template <int CPL>
__device__ __forceinline__ void pair_load(const uint8_t* __restrict__ packed, const ExpertLayout& L, int H, int e,
                                          int ip, int lane, PairLoads<CPL>& ld) {
    const int C = H / 32, lpr = C < 64 ? C : 64, rpw = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    const uint8_t* base = packed + (size_t)e * L.stride;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        if (it * rpw >= 4) break;  // wave-uniform
        const int rs = it * rpw + rsub;
        if (rs < 4) {
            const int r = 2 * ip + (rs & 1);
            const uint8_t* q = base + gu_row_q(L, H, rs >= 2, r);
            const uint32_t* sb = reinterpret_cast<const uint32_t*>(base + gu_row_sb(L, H, rs >= 2, r));
#pragma unroll
            for (int c = 0; c < CPL; ++c) ld.c[it][c] = load_chunk(q, sb, lr + lpr * c);
        }
    }
}

// bf16 h of rows 2ip and 2ip+1 (low, high half) for one token's x slice.
template <int CPL>
__device__ __forceinline__ uint32_t pair_finish(const PairLoads<CPL>& ld, int H, const XSlice<CPL>& xs, int lane) {
    const int C = H / 32, lpr = C < 64 ? C : 64, rpw = 64 / lpr;
    const int rsub = lane / lpr;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        if (it * rpw >= 4) break;  // wave-uniform
        const int rs = it * rpw + rsub;
        float d = 0.f;
        if (rs < 4) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) d += chunk_dot(ld.c[it][c], xs.p[c], xs.s[c]);
        }
        v[it] = group_sum(d, lpr);
    }
    float r[4];
#pragma unroll
    for (int rs = 0; rs < 4; ++rs) {  // row slot rs: iteration rs / rpw, last lane of group rs % rpw
        const int it = rs / rpw;
        const float src = it == 0 ? v[0] : it == 1 ? v[1] : it == 2 ? v[2] : v[3];
        r[rs] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(src), (rs % rpw) * lpr + lpr - 1));
    }
    const uint32_t h0 = f32_to_bf16(silu_f32(r[0]) * r[2]);
    const uint32_t h1 = f32_to_bf16(silu_f32(r[1]) * r[3]);
    return h0 | (h1 << 16);
}

// This lane's slice of token t's activations for a weight row of Hw codes (H or
// 2H): from the workgroup's LDS copy (values and chunk sums, staged by stage_x) or
// from global memory; both give the values and sums of load_xslice.
template <int CPL>
__device__ __forceinline__ void token_xslice(bool lds, const uint16_t* s_x, const float* s_xs,
                                             const uint16_t* __restrict__ gx, int t, int H, int Hw, int lane,
                                             XSlice<CPL>& xs) {
    const int C = H / 32, Cw = Hw / 32, lpr = Cw < 64 ? Cw : 64;
    const int lr = lane % lpr;
    if (!lds) {
        load_xslice(gx + (size_t)t * H, lr, lpr, C, xs);
        return;
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        int ch = lr + lpr * c;
        if (ch >= C) ch -= C;
        const uint4* src = reinterpret_cast<const uint4*>(s_x + (size_t)t * H + 32 * ch);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const uint4 v = src[q4];
            xs.p[c][4 * q4 + 0] = v.x;
            xs.p[c][4 * q4 + 1] = v.y;
            xs.p[c][4 * q4 + 2] = v.z;
            xs.p[c][4 * q4 + 3] = v.w;
        }
        xs.s[c] = s_xs[t * C + ch];
    }
}

// Copies x [T][H] into LDS with the chunk sums of load_xslice (one chunk of 32 per
// thread and step); with xr (per-token RMSNorm scales) it stores bf16(x * r_t).
__device__ __forceinline__ void stage_x(const uint16_t* __restrict__ gx, int T, int H, uint16_t* s_x, float* s_xs,
                                        const float* xr) {
    const int C = H / 32;
    for (int i = threadIdx.x; i < T * C; i += blockDim.x) {
        const uint4* src = reinterpret_cast<const uint4*>(gx + (size_t)i * 32);
        uint4* dst = reinterpret_cast<uint4*>(s_x + (size_t)i * 32);
        uint32_t w[16];
        const float r = xr ? xr[i / C] : 1.f;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            uint4 v = src[q4];
            if (xr) {
                v.x = norm_bf16(v.x & 0xFFFFu, r) | (norm_bf16(v.x >> 16, r) << 16);
                v.y = norm_bf16(v.y & 0xFFFFu, r) | (norm_bf16(v.y >> 16, r) << 16);
                v.z = norm_bf16(v.z & 0xFFFFu, r) | (norm_bf16(v.z >> 16, r) << 16);
                v.w = norm_bf16(v.w & 0xFFFFu, r) | (norm_bf16(v.w >> 16, r) << 16);
            }
            dst[q4] = v;
            w[4 * q4 + 0] = v.x;
            w[4 * q4 + 1] = v.y;
            w[4 * q4 + 2] = v.z;
            w[4 * q4 + 3] = v.w;
        }
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) sum = dot2_bf16(w[j], 0x3F803F80u, sum);
        s_xs[i] = sum;
    }
}

// Down loads of one wavefront for one item (DR output rows, every slot): row
// iterations wave + LW * (b0 + j), j < DNB, with the lane layout of dn_load.
struct DnLoadsL {
    ChunkLoad ld[DNB];
    int slot[DNB];
    bool ok[DNB];
};

template <int DR>
__device__ __forceinline__ void dnl_load(const uint8_t* __restrict__ packed, const ExpertLayout& L, int I, int E,
                                         int k, int has_shared, int n0, const int32_t* ids_t, int b0, int wave,
                                         int lane, DnLoadsL& d) {
    const int S = k + has_shared;
    const int lpr = I / 32, rpw = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    const int n_dots = S * DR;
    const int n_it = (n_dots + rpw - 1) / rpw;
#pragma unroll
    for (int j = 0; j < DNB; ++j) {
        const int it = wave + LW * (b0 + j);
        const int q = it * rpw + rsub;
        d.ok[j] = it < n_it && q < n_dots;
        d.slot[j] = d.ok[j] ? q / DR : 0;
        if (d.ok[j]) {
            const int s = d.slot[j];
            const int e = s < k ? ids_t[s] : E;
            const int n = n0 + q % DR;
            const uint8_t* base = packed + (size_t)e * L.stride;
            d.ld[j] = load_chunk(base + dn_row_q(L, I, n), reinterpret_cast<const uint32_t*>(base + dn_row_sb(L, I, n)),
                                 lr);
        }
    }
}

// Persistent kernel: one workgroup of 16 wavefronts per CU (every workgroup
// resident); data moves between workgroups through epoch-tagged words.
//   A: router rows, one wavefront per (row, token), published tagged (twice, on
//      the chip's two halves); x is staged into LDS meanwhile.
//   S: token t is selected by wavefront t, or with up to four tokens by the
//      winner of a race between wavefronts t and T + t on the two logit copies
//      (DPP top-k). The workgroup then forms the distinct experts of the launch
//      (the shared expert first) and, per distinct expert, the (token, slot)
//      pairs that use it; the pick weights follow once the gate/up loads are out.
//   B: gate/up row-pair tasks (distinct expert, row pair), one per wavefront:
//      the four weight rows are loaded once and applied to every token of the
//      expert; h pairs are published tagged. Sixteen wavefronts per CU keep
//      enough loads in flight; the shared expert's tasks are loaded before the
//      selection.
//   C: down items (8 output rows with one token, 16 with more, every slot) with
//      the combine; a workgroup enters C when its own gate/up tasks are done and
//      stages a token's h once (polling the tagged words) for all of its items of
//      that token; an item's weight loads go out before that wait, and the next
//      item's before the arithmetic.
//
// HC, IC, KC, KMC (when HC is nonzero) fix hidden, inter, top_k and the weight
// row multiple at compile time; the shape of the served model gets its own
// instances (4-bit and 8-bit experts), with every lane layout and reduction width
// folded.
template <int CPL, int TT, bool AFF8, int VPL, int HC, int IC, int KC, int KMC>
__global__ __launch_bounds__(LTH) void decode_layer_kernel(LayerArgs a) {
    __shared__ int32_t s_ids[16][16];
    __shared__ uint16_t s_w[16][16];
    __shared__ uint16_t s_wsh[16];
    __shared__ uint32_t s_raw[16][16];  // the picks' fp32 logit bits, per token
    __shared__ uint32_t s_gbits[16];    // the shared gate's fp32 logit bits, per token
    __shared__ int s_race[16];          // per token: the wavefront that won its polling race
    __shared__ uint32_t s_used[32];
    __shared__ int32_t s_upre[32];
    __shared__ int32_t s_dexp[MAXD];
    __shared__ int32_t s_dcnt[MAXD];
    __shared__ uint16_t s_dtok[MAXD][16];
    __shared__ int32_t s_nd;
    __shared__ int s_bad;  // a bounded wait of this workgroup timed out: its h and outputs become NaN
    __shared__ float s_xr[16];  // per-token RMSNorm scales (norm_eps >= 0)
    // rows per down item: one token has one item per workgroup; more tokens run
    // items one after another, and items of 16 rows keep more loads in flight per
    // wavefront (T=16 69.4 -> 60.3 us, T=8 39.8 -> 35.6; 32 rows measured no better
    // at 8 and 16 tokens and worse at 2)
    constexpr int DR = TT == 1 ? DN_ROWS : 2 * DN_ROWS;
    __shared__ float ysh2[2][17][DR];  // down results, alternating between items
    extern __shared__ __attribute__((aligned(16))) uint32_t lds_dyn[];
    const int G = gridDim.x, wg = blockIdx.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int T = TT == 1 ? 1 : a.T, H = HC ? HC : a.H, I = IC ? IC : a.I, k = KC ? KC : a.k;
    const int KM = HC ? KMC : a.kmul;
    const int Hw = H * KM, Iw = I * KM, IXC = I / 32;  // weight row lengths; h chunks of 32
    const int E = a.E, R = a.R, hs_ = a.has_shared;
    const int S = k + hs_;
    const int npair = I / 2;
    DecodeCtl* ctl = a.ctl;
    const uint32_t tag = load_coherent(&ctl->epoch) + 1u;
    uint32_t* hsh = lds_dyn;                                                        // [S][I] bf16
    float* s_hs = reinterpret_cast<float*>(lds_dyn + (size_t)S * I / 2);           // [S][I/32] h chunk sums
    uint16_t* s_x = reinterpret_cast<uint16_t*>(s_hs + (size_t)S * (I / 32));      // [T][H] bf16
    float* s_xs = reinterpret_cast<float*>(s_x + (a.stage_x ? (size_t)T * H : 0));  // [T][H/32]
    if (tid < 32) s_used[tid] = 0u;
    if (tid < 16) s_race[tid] = -1;
    if (tid == 0) s_bad = 0;
    for (int i = tid; i < MAXD; i += LTH) s_dcnt[i] = 0;

    // Wavefronts that poll must have no loads or stores of their own outstanding:
    // the vector memory counter retires in order, so a poll's result would wait
    // for them. Router rows and gate/up tasks are therefore numbered from the top
    // wavefront down, and selection polls on wavefronts 0 .. npoll-1.
    const int wtop = LW - 1 - wave;
    // Up to four tokens, two wavefronts poll each token's logits, one per copy
    // (the tagged logits are published twice, 8 KiB apart, and device memory
    // alternates between the chip's two halves in 8 KiB blocks, by physical
    // address): the first to see them all selects, which is in effect the copy on
    // this XCD's half. More tokens: one wavefront per token, on copy 0.
    const bool race = T <= 4;
    const int npoll = race ? 2 * T : T;

    // ---- A: router rows, one wavefront per (row, token); the per-lane order of the
    // products and the reduction tree are those of router_row for any token count,
    // so the logits equal the staged router's bit for bit
    // One token: the router rows go to the workgroups with wg % 8 < 4, up to three
    // rows each on separate wavefronts. Workgroups are dealt to the XCDs in turn,
    // and XCDs 4-7 start about 0.6 us after XCDs 0-3; every selection waits for the
    // last logit, so the rows are best computed where the launch starts first (if
    // the dealing differs, only the speed changes). More tokens: rows beyond the
    // first G (the shared gate's at 256 experts) go to further wavefronts when
    // they fit above the selecting ones, so that no wavefront computes two rows
    // one after the other.
    // With the norm, a router row also gives its token's scale (xr_out): when every
    // workgroup computes row wg for each of its tokens (the multi-token instance,
    // G <= R), those rows leave the scales in s_xr and the pass below is not needed
    // (T=16 stack 69.9 -> 69.3 us per layer; in the one-token instance the same
    // change measured 0.5 us slower, so it keeps the pass).
    const int nrw = (R + G - 1) / G;
    const int GE = G / 2;                  // workgroups with wg % 8 < 4
    const int mE = (R * T + GE - 1) / GE;  // router rows per such workgroup
    const bool one_split = TT == 1 && G % 8 == 0 && mE + npoll <= LW;
    const bool xr_rows = TT != 1 && !one_split && G <= R && a.norm_eps >= 0.f;  // (the one-token instance keeps the pass)
    if (one_split) {
        if ((wg & 7) < 4 && wtop < mE) {
            const int r = (wg >> 3) * 4 + (wg & 7) + GE * wtop;
            if (r < R)
                router_row<1, AFF8>(a.router, a.logit_bias, a.x, 0, 1, H, R, E, r, lane, a.logits, false, a.tlogits,
                                    tag, a.tl_stride, a.tl_copy, a.norm_eps);
        }
    } else if (nrw * T + npoll <= LW) {
        if (wtop < nrw * T) {
            const int r = wg + G * (wtop / T);
            if (r < R)
                router_row<1, AFF8>(a.router, a.logit_bias, a.x, wtop % T, 1, H, R, E, r, lane, a.logits, false,
                                    a.tlogits, tag, a.tl_stride, a.tl_copy, a.norm_eps,
                                    xr_rows && wtop < T ? &s_xr[wtop] : nullptr);
        }
    } else if (wtop < T) {
        for (int r = wg; r < R; r += G)
            router_row<1, AFF8>(a.router, a.logit_bias, a.x, wtop, 1, H, R, E, r, lane, a.logits, false, a.tlogits,
                                tag, a.tl_stride, a.tl_copy, a.norm_eps, xr_rows && r == wg ? &s_xr[wtop] : nullptr);
    }
    // with the norm, the layer's input is bf16(x r_t): waves t < T compute the scales
    // (in row_sumsq's order, as the router rows do) before the staging
    const bool norm = a.norm_eps >= 0.f;
    if (norm) {
        if (!xr_rows && wave < T) {
            const float xr = rms_scale(row_sumsq(a.x + (size_t)wave * H, H, lane), H, a.norm_eps);
            if (lane == 0) s_xr[wave] = xr;
        }
        __syncthreads();
    }
    if (a.stage_x) stage_x(a.x, T, H, s_x, s_xs, norm ? s_xr : nullptr);
    __syncthreads();
    // the shared expert's row pairs are tasks 0 .. npair-1 of phase B
    PairLoads<CPL> cur;
    bool have = false;
    const int j0 = wg + G * wtop;
    if (hs_ && j0 < npair && wave >= npoll) {
        pair_load<CPL>(a.experts, a.L, Hw, E, j0, lane, cur);
        have = true;
    }
    // Every wavefront of this workgroup has read the epoch (the barrier above waited
    // for its loads), so the workgroup may count itself in now. With fewer tokens
    // than wavefronts the top wavefront selects nothing and does it here, after its
    // first task's loads: the count's round trip then overlaps the work rather than
    // a wavefront's next wait (the memory counter retires in order). Otherwise the
    // count waits for the exit. The workgroup that counted last resets the count and
    // publishes the next epoch: every workgroup has read the epoch by then, and the
    // next launch starts only after this one ends. An early count is settled after
    // phase B, when its round trip is long over.
    // The early count has two levels: one counter per group of workgroups
    // (wg % 8), each on its own 128-byte line, and the last of a group counts the
    // group in at the top. Atomics on one word are performed one after another, and
    // with a single counter the workgroups at the back of 256 waited so long for
    // the return that the logit polls queued behind it in the CU were late
    // (T=1 13.8 -> 12.3 us). At the exit a second level is one more round trip at
    // the very end, so the count there stays single.
    const bool count_early = T < LW;
    const int grp = wg & 7;
    const unsigned gsize = (unsigned)((G - grp + 7) / 8), ngrp = (unsigned)min(G, 8);
    unsigned counted = 0u;
    if (count_early && tid == LTH - 64) counted = atomicAdd(&ctl->group[grp].count, 1u);

    // ---- S: selection (the ids; the weights follow the first gate/up loads),
    // distinct experts, token lists
    if (wave < npoll) {
        // up to four tokens: all of a lane's logit words reloaded together in each
        // polling round (few wavefronts poll); more: only the stale ones
        const int t = wave < T ? wave : wave - T;
        const LogitSrc src{nullptr, a.tlogits + (size_t)t * a.tl_stride + (wave >= T ? a.tl_copy : 0), tag,
                           &ctl->error, false, race, race ? &s_race[t] : nullptr, wave};
        const SelState sel = select_ids<VPL>(src, E, k, hs_, lane, s_ids[t]);
        if (sel.won) {
            if (sel.timeout && lane == 0) s_bad = 1;
            if (lane < k) s_raw[t][lane] = sel.raw;
            if (lane == 0) s_gbits[t] = sel.gbits;
            if (wg == 0 && lane < k) a.ids[t * k + lane] = (int32_t)sel.id;
            if constexpr (TT == 1) {
                // one token: its k picks are k distinct experts (k <= E), listed in
                // pick order after the shared expert
                if (lane < k) {
                    s_dexp[hs_ + lane] = (int32_t)sel.id;
                    s_dcnt[hs_ + lane] = 1;
                    s_dtok[hs_ + lane][0] = (uint16_t)(lane << 5);
                }
                if (lane == 0) {
                    if (hs_) {
                        s_dexp[0] = E;
                        s_dcnt[0] = 1;
                        s_dtok[0][0] = (uint16_t)(k << 5);
                    }
                    s_nd = hs_ + k;
                }
            }
        }
    }
    __syncthreads();
    if constexpr (TT != 1) {
        // the shared expert serves every token: it is listed as ns entries of up to
        // two tokens each, so that its SwiGLU work spreads over several wavefronts
        // and SIMDs instead of one wavefront per workgroup doing all T tokens (each
        // entry reloads the shared gate/up rows; T=16 78.1 -> 70.6 us, T=8 42.5 ->
        // 40.1, four tokens per entry 71.4 / 40.9)
        const int ns = hs_ ? (T + 1) / 2 : 0;
        if (tid < T * k) {
            const int e = s_ids[tid / k][tid % k];
            atomicOr(&s_used[e >> 5], 1u << (e & 31));
        }
        __syncthreads();
        if (wave == 0) {
            const int nword = (E + 31) / 32;
            const uint32_t m = lane < nword ? s_used[lane] : 0u;
            const int c = __popc(m);
            int incl = c;
            for (int dd = 1; dd < 32; dd <<= 1) {
                const int o = __shfl_up(incl, dd);
                if (lane >= dd) incl += o;
            }
            int pos = ns + incl - c;
            if (lane < nword) s_upre[lane] = pos;
            for (uint32_t mm = m; mm; mm &= mm - 1) s_dexp[pos++] = 32 * lane + __builtin_ctz(mm);
            if (lane == 31) s_nd = ns + incl;
            if (lane < ns) s_dexp[lane] = E;
        }
        __syncthreads();
        if (tid < T * k) {
            const int t = tid / k, sl = tid % k, e = s_ids[t][sl];
            const int dd = s_upre[e >> 5] + __popc(s_used[e >> 5] & ((1u << (e & 31)) - 1u));
            const int p = atomicAdd(&s_dcnt[dd], 1);
            s_dtok[dd][p] = (uint16_t)(t | (sl << 5));
        }
        if (hs_ && tid < T) {
            s_dtok[tid / 2][tid % 2] = (uint16_t)(tid | (k << 5));
            if (tid < ns) s_dcnt[tid] = min(2, T - 2 * tid);
        }
        __syncthreads();
    }

    // ---- B: gate/up row pairs of the distinct experts
    const int nB = s_nd * npair;
    const int NBLK = H / DR, nC = T * NBLK;
    const int per = (nC + G - 1) / G, c0 = wg * per, c1 = min(nC, c0 + per);
    DnLoadsL dcur;
    bool dhave = false;
    // Every wavefront with a task issues its first task's loads here. With one token
    // there are fewer tasks than wavefronts (9 * 256 of 16 * 256 at hidden 2048,
    // inter 512, top-8 plus shared), and a barrier on the issue (not on the data)
    // lets every task's loads out before the selecting wavefront's fp64 weight
    // arithmetic and the idle wavefronts go on. It was first measured against idle
    // wavefronts' down loads and h polls (T=1 20.1 -> 18.0 us); with the barrier
    // before phase C in place it still saves 0.25 us. With more tokens every
    // wavefront has a task and the barrier measured slower.
    if (!have && j0 < nB) {
        pair_load<CPL>(a.experts, a.L, Hw, s_dexp[j0 / npair], j0 % npair, lane, cur);
        have = true;
    }
    if constexpr (TT == 1) __builtin_amdgcn_s_barrier();
    // The pick weights are read only by the combine, after phase C's first barrier;
    // the selecting wavefronts compute them while their first task's loads are out
    // (their inputs wait in LDS, not in registers, across the issue).
    if (wave < T) {
        const SelState sel{0u, lane < k ? s_raw[wave][lane] : 0u, s_gbits[wave]};
        const uint16_t wb = select_weights(sel, k, lane);
        if (lane < k) {
            s_w[wave][lane] = wb;
            if (wg == 0) a.w[wave * k + lane] = wb;
        }
        if (hs_ && lane == k) {
            s_wsh[wave] = wb;
            if (wg == 0) a.wsh[wave] = wb;
        }
    }
    for (int j = j0; j < nB; j += G * LW) {
        const int dd = j / npair, ip = j % npair;
        if (!have) pair_load<CPL>(a.experts, a.L, Hw, s_dexp[dd], ip, lane, cur);
        have = false;
        const int cnt = s_dcnt[dd];
        for (int u = 0; u < cnt; ++u) {
            const int ent = s_dtok[dd][u], t = ent & 31, sl = ent >> 5;
            XSlice<CPL> xs;
            token_xslice<CPL>(a.stage_x, s_x, s_xs, a.x, t, H, Hw, lane, xs);
            uint32_t hp = pair_finish<CPL>(cur, Hw, xs, lane);
            // after a timed-out wait in this workgroup its h pairs are NaN, so the
            // outputs of every token they reach are NaN rather than silently stale
            if (s_bad) hp = 0x7FC07FC0u;
            if (lane == 0) {
                const size_t w = ((size_t)t * S + sl) * npair + ip;
                if constexpr (TT == 1) {
                    store_tagged(a.th + th_word(w, 0), tag, hp);
                    store_tagged(a.th + th_word(w, 1), tag, hp);
                } else {
                    store_tagged(a.th + w, tag, hp);
                }
            }
        }
    }

    // Phase C starts with every wavefront polling for h. A workgroup goes on only when
    // all its own gate/up tasks are done: polls from the wavefronts that finished
    // first would otherwise share the memory system with the task loads still out
    // across the chip and slow them (T=1 17.5 -> 14.5 us, T=2 23.0 -> 19.5 us).
    __syncthreads();
    if (count_early && tid == LTH - 64 && counted == gsize - 1) {
        atomicExch(&ctl->group[grp].count, 0u);
        if (atomicAdd(&ctl->exit_count, 1u) == ngrp - 1) {
            atomicExch(&ctl->exit_count, 0u);
            atomicExch(&ctl->epoch, tag);
        }
    }

    // ---- C: down items with the combine
    const int lpr = Iw / 32, rpw = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    const int lrx = lr < IXC ? lr : lr - IXC;  // this lane's chunk of h
    const int n_dots = S * DR, n_it = (n_dots + rpw - 1) / rpw;
    int staged = -1;
    for (int c = c0; c < c1; ++c) {
        const int t = c / NBLK, n0 = (c % NBLK) * DR;
        float(*ysh)[DR] = ysh2[TT == 1 ? 0 : (c - c0) & 1];
        if (!dhave) dnl_load<DR>(a.experts, a.L, Iw, E, k, hs_, n0, s_ids[t], 0, wave, lane, dcur);
        DnLoadsL dnxt;
        const bool nhave = c + 1 < c1;
        if (nhave)
            dnl_load<DR>(a.experts, a.L, Iw, E, k, hs_, ((c + 1) % NBLK) * DR, s_ids[(c + 1) / NBLK], 0, wave, lane,
                         dnxt);
        if (t != staged) {
            const int nw = S * npair;
            // one token: h from the copy that won this workgroup's logit race (the
            // copy on its half of the chip when both regions sit in one 2 MiB page)
            static_assert(LTH == 1024, "staging steps one 1024-word block at a time");
            // (i0 = tid + 4 LTH m, so words i0 + LTH j, j < 4, sit at th_word(i0) + 2 LTH j)
            const int hc = s_race[0] >= T ? 1 : 0;
            bool tmo = false;
            for (int i0 = tid; i0 < nw; i0 += LTH * 4) {
                uint32_t v[4];
                const int n = min(4, (nw - 1 - i0) / LTH + 1);
                if constexpr (TT == 1)
                    tmo |= load_tagged_many<4>(a.th + th_word(i0, hc), 2 * LTH, n, tag, &ctl->error, v);
                else
                    tmo |= load_tagged_many<4>(a.th + (size_t)t * S * npair + i0, LTH, n, tag, &ctl->error, v);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (j < n) hsh[i0 + LTH * j] = v[j];
            }
            if (tmo) s_bad = 1;
            __syncthreads();
            if constexpr (TT != 1) {
                // the chunk sums of h, once per token (load_xslice's arithmetic, so
                // bit-identical to computing them per row)
                if (tid < S * IXC) {
                    XSlice<1> hx;
                    load_xslice(reinterpret_cast<const uint16_t*>(hsh) + (size_t)(tid / IXC) * I, tid % IXC, IXC, IXC,
                                hx);
                    s_hs[tid] = hx.s[0];
                }
                __syncthreads();
            }
            staged = t;
        }
        for (int b0 = 0; LW * b0 < n_it; b0 += DNB) {
            if (b0 > 0) dnl_load<DR>(a.experts, a.L, Iw, E, k, hs_, n0, s_ids[t], b0, wave, lane, dcur);
#pragma unroll
            for (int j = 0; j < DNB; ++j) {
                const int it = wave + LW * (b0 + j);
                if (it >= n_it) break;  // wave-uniform
                const int q = it * rpw + rsub;
                float v = 0.f;
                if (dcur.ok[j]) {
                    XSlice<1> hx;
                    if constexpr (TT != 1) {
                        const uint4* src = reinterpret_cast<const uint4*>(
                            reinterpret_cast<const uint16_t*>(hsh) + (size_t)dcur.slot[j] * I + 32 * lrx);
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            const uint4 hv = src[q4];
                            hx.p[0][4 * q4 + 0] = hv.x;
                            hx.p[0][4 * q4 + 1] = hv.y;
                            hx.p[0][4 * q4 + 2] = hv.z;
                            hx.p[0][4 * q4 + 3] = hv.w;
                        }
                        hx.s[0] = s_hs[dcur.slot[j] * IXC + lrx];
                    } else {
                        load_xslice(reinterpret_cast<const uint16_t*>(hsh) + (size_t)dcur.slot[j] * I, lr, lpr, IXC,
                                    hx);
                    }
                    v = chunk_dot(dcur.ld[j], hx.p[0], hx.s[0]);
                }
                v = group_sum(v, lpr);
                if (lr == lpr - 1 && q < n_dots) ysh[q / DR][q % DR] = v;
            }
        }
        __syncthreads();
        const bool bad = s_bad != 0;  // a timed-out wait here: y and out are NaN
        if (a.y) {
            for (int i = tid; i < n_dots; i += LTH)
                a.y[((size_t)t * S + i / DR) * H + n0 + i % DR] = bad ? __uint_as_float(0x7FC00000u)
                                                                      : ysh[i / DR][i % DR];
        }
        if (tid < DR) {
            float acc = 0.f;
            for (int sl = 0; sl < k; ++sl) acc = fmaf(bf16_to_f32(s_w[t][sl]), ysh[sl][tid], acc);
            if (hs_) acc = fmaf(bf16_to_f32(s_wsh[t]), ysh[k][tid], acc);
            uint32_t bb = f32_to_bf16(acc);
            const size_t o = (size_t)t * H + n0 + tid;
            if (a.residual) bb = f32_to_bf16(bf16_to_f32(a.residual[o]) + bf16_to_f32(bb));
            a.out[o] = bad ? (uint16_t)0x7FC0u : (uint16_t)bb;
        }
        // More tokens: no barrier here. The next item writes the other ysh buffer, hsh
        // is not read after the barrier above, and this buffer is written again only
        // after the next item's barrier, which every wavefront reaches after its reads
        // here. One token reuses the single buffer, so it waits here when another item
        // of its workgroup follows.
        if constexpr (TT == 1) {
            if (c + 1 < c1) __syncthreads();
        }
        dcur = dnxt;
        dhave = nhave;
    }

    // ---- exit: a workgroup that did not count itself in early does it now; the one
    // that counted last publishes the new epoch
    if (!count_early) {
        __syncthreads();
        if (tid == LTH - 64 && atomicAdd(&ctl->exit_count, 1u) == (unsigned)G - 1) {
            atomicExch(&ctl->exit_count, 0u);
            atomicExch(&ctl->epoch, tag);
        }
    }
}

static int cpl_for(int K) { return K / 32 <= 64 ? 1 : (K / 32) / 64; }

static void launch_gateup(const moe_shape& sh, const ExpertLayout& L, const uint8_t* p, const uint16_t* x, int T,
                          const int32_t* ids, uint16_t* hbuf, hipStream_t hs) {
    const int S = n_slots(sh), H = sh.hidden, I = sh.inter, km = kmul(sh);
    dim3 g1(I / GU_ROWS, S, T);
    switch (cpl_for(H * km)) {
        case 1: hipLaunchKernelGGL(decode_gateup_kernel<1>, g1, dim3(256), 0, hs, p, L, H, I, km, sh.n_experts,
                                   sh.top_k, sh.has_shared, x, ids, hbuf); break;
        case 2: hipLaunchKernelGGL(decode_gateup_kernel<2>, g1, dim3(256), 0, hs, p, L, H, I, km, sh.n_experts,
                                   sh.top_k, sh.has_shared, x, ids, hbuf); break;
        default: hipLaunchKernelGGL(decode_gateup_kernel<4>, g1, dim3(256), 0, hs, p, L, H, I, km, sh.n_experts,
                                    sh.top_k, sh.has_shared, x, ids, hbuf); break;
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

// LDS copy of x [T][H] with its chunk sums.
static size_t xsh_bytes(const moe_shape& sh, int T) { return (size_t)T * sh.hidden * 2 + (size_t)T * (sh.hidden / 32) * 4; }

typedef void (*LayerKernel)(LayerArgs);

template <int CPL, int TT, int VPL>
static LayerKernel pick_layer_v(const LayerArgs& a, bool aff8) {
    if constexpr (VPL == 4 && (CPL == 1 || CPL == 2)) {
        // the served model's shape: 4-bit experts (rows of 2048 codes, one chunk per
        // lane) and 8-bit experts (rows of 4096 codes, two)
        if (aff8 && a.H == 2048 && a.I == 512 && a.k == 8 && a.kmul == CPL)
            return decode_layer_kernel<CPL, TT, true, VPL, 2048, 512, 8, CPL>;
    }
    return aff8 ? decode_layer_kernel<CPL, TT, true, VPL, 0, 0, 0, 1>
                : decode_layer_kernel<CPL, TT, false, VPL, 0, 0, 0, 1>;
}

template <int CPL, int TT>
static LayerKernel pick_layer_tt(const LayerArgs& a, bool aff8) {
    const int vpl = (a.E + 63) / 64;
    if (vpl <= 1) return pick_layer_v<CPL, TT, 1>(a, aff8);
    if (vpl <= 4) return pick_layer_v<CPL, TT, 4>(a, aff8);
    return pick_layer_v<CPL, TT, 16>(a, aff8);
}

// The kernel instance for a launch: hidden (chunks per lane), one token or more,
// keys per lane of the selection, router format, and the served shape.
static LayerKernel pick_layer(const LayerArgs& a, bool aff8) {
    if (cpl_for(a.H * a.kmul) == 1) return a.T <= 1 ? pick_layer_tt<1, 1>(a, aff8) : pick_layer_tt<1, 16>(a, aff8);
    return a.T <= 1 ? pick_layer_tt<2, 1>(a, aff8) : pick_layer_tt<2, 16>(a, aff8);
}

// Workgroups of kernel f (LTH threads, lds bytes of dynamic LDS) that one compute
// unit can hold at once, cached per (instance, LDS size); 0 if the query fails.
static int layer_blocks_per_cu(LayerKernel f, size_t lds) {
    static std::mutex mu;
    static std::map<std::pair<const void*, size_t>, int> cache;
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_pair(reinterpret_cast<const void*>(f), lds);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, f, LTH, lds) != hipSuccess) return 0;
    cache[key] = nb;
    return nb;
}

static int device_max_lds() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (!cache[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return 0;
        cache[dev] = n;
    }
    return cache[dev];
}

}  // namespace moe

using namespace moe;

static size_t hbuf_bytes(const moe_shape& sh, int T) { return align_up((size_t)T * n_slots(sh) * sh.inter * 2, 256); }

// Workspace: h rows (bf16) | control words (256 B) | tagged logits | tagged h.
//
// Tagged logits: every selecting wavefront polls all of its token's logits, from
// every XCD. Device memory alternates between the two halves of the chip in
// 8 KiB blocks (measured on MI355X: a coherent load from an XCD of the other half
// takes the longer path; which half a block is on depends on address bit 13 and
// on bits of the physical page), so a small buffer sits on one half. The router
// therefore publishes every logit twice, in two copies 8 KiB apart, one on each
// half, and with up to four tokens two wavefronts race, one per copy. The region
// starts on a 16 KiB boundary of the device address; a token takes 2 * tl_half
// bytes.
static size_t tl_half(const moe_shape& sh) { return align_up((size_t)router_rows(sh) * 8, 8192); }

struct DecodeWs {
    size_t ctl, tlogits, th, total;
};

static DecodeWs decode_ws_layout(const moe_shape& sh, int T) {
    DecodeWs w;
    w.ctl = hbuf_bytes(sh, T);
    w.tlogits = w.ctl + align_up(sizeof(DecodeCtl), 256);
    w.th = w.tlogits + 16384 + (size_t)T * 2 * tl_half(sh);
    // tagged h; one token: 16 KiB of alignment slack, then blocks of 16 KiB (8 KiB
    // per copy)
    const size_t nh = (size_t)T * n_slots(sh) * (sh.inter / 2);
    w.total = w.th + (T == 1 ? 16384 + (nh + 1023) / 1024 * 16384 : align_up(nh * 8, 256));
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

// The two launches of the staged expert stage (gate/up with SwiGLU into hbuf,
// then down into y); hbuf holds T * S * I bf16 values.
static moe_status launch_decode_experts(const moe_shape& sh, const uint8_t* p, const uint16_t* x, int T,
                                        const int32_t* ids, uint16_t* hbuf, float* y, hipStream_t hs) {
    const ExpertLayout L = expert_layout(sh);
    launch_gateup(sh, L, p, x, T, ids, hbuf, hs);
    moe_status st = check_launch("decode_gateup_kernel");
    if (st != MOE_OK) return st;
    hipLaunchKernelGGL(decode_down_kernel, dim3(sh.hidden / DN_ROWS, T), dim3(256), hsh_bytes(sh), hs, p, L, sh.hidden,
                       sh.inter, kmul(sh), sh.n_experts, sh.top_k, sh.has_shared, hbuf, ids, y, (const uint16_t*)nullptr,
                       (const uint16_t*)nullptr, (const uint16_t*)nullptr, (uint16_t*)nullptr);
    return check_launch("decode_down_kernel");
}

extern "C" moe_status moe_experts_decode(const moe_shape* shape, const void* experts_packed, const uint16_t* x,
                                         int32_t T, const int32_t* ids, void* ws, size_t ws_bytes, float* y,
                                         void* stream) {
    clear_error();
    moe_status st = check_decode_args(shape, experts_packed, x, T, ws, ws_bytes);
    if (st != MOE_OK) return st;
    if (!ids || !y || !aligned16(y)) return fail(MOE_ERR_INVALID_ARG, "ids or y NULL / unaligned");
    return launch_decode_experts(*shape, (const uint8_t*)experts_packed, x, T, ids, (uint16_t*)ws, y,
                                 (hipStream_t)stream);
}

// ---------------------------------------------------------------- allocation-free staged decode
// moe_experts_decode_noalloc keeps the bf16 h rows in this file-scope array instead
// of a caller workspace: at most 16 tokens x 17 slots x 2048 intermediate values.
// Each GPU holds its own copy until the process ends. In host code `scratch` names
// a host-side stand-in, never the device memory: kernels and copies get the
// address from scratch_device_ptr().
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)16 * 17 * 2048 * 2;
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device: looked up with
// hipGetSymbolAddress on the first call on each device (with that device current)
// and kept per device. NULL if the lookup fails.
static void* scratch_device_ptr() {
    static std::mutex mu;
    static void* ptr[64] = {nullptr};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        ptr[dev] = p;
    }
    return ptr[dev];
}

extern "C" moe_status moe_experts_decode_noalloc(const moe_shape* shape, const void* experts_packed,
                                                 const uint16_t* x, int32_t T, const int32_t* ids, float* y,
                                                 void* stream) {
    clear_error();
    moe_status st = validate_shape(shape);
    if (st != MOE_OK) return st;
    if (T < 1 || T > 16) return fail(MOE_ERR_INVALID_ARG, "decode path takes 1..16 rows, got T = %d", T);
    if (!experts_packed || !x || !ids || !y || !aligned16(experts_packed) || !aligned16(x) || !aligned16(y))
        return fail(MOE_ERR_INVALID_ARG, "NULL or unaligned pointer");
    if (hsh_bytes(*shape) > 65536)
        return fail(MOE_ERR_UNSUPPORTED, "decode path: (top_k + shared) * inter * 2 bytes must fit 64 KiB of LDS");
    const size_t need = (size_t)T * n_slots(*shape) * shape->inter * 2;
    if (need > NOALLOC_SCRATCH_BYTES)
        return fail(MOE_ERR_UNSUPPORTED, "h rows of %zu bytes exceed the %zu-byte device scratch", need,
                    NOALLOC_SCRATCH_BYTES);
    void* hbuf = scratch_device_ptr();
    if (!hbuf) return fail(MOE_ERR_HIP, "could not look up the device address of the decode scratch");
    return launch_decode_experts(*shape, (const uint8_t*)experts_packed, x, T, ids, (uint16_t*)hbuf, y,
                                 (hipStream_t)stream);
}

// One launch of decode_layer_kernel (moe_decode_layer, moe_decode_block).
static moe_status decode_layer_launch(const moe_shape* shape, const void* router_packed, const float* logit_bias,
                                      const void* experts_packed, const uint16_t* x, int32_t T, void* ws,
                                      size_t ws_bytes, float* logits, int32_t* ids, uint16_t* w, uint16_t* w_shared,
                                      float* y, const uint16_t* residual, uint16_t* out, float norm_eps,
                                      void* stream) {
    moe_status st = check_decode_args(shape, experts_packed, x, T, ws, ws_bytes);
    if (st != MOE_OK) return st;
    const moe_shape& sh = *shape;
    if ((st = check_route_outputs(sh, T, ids, w, w_shared)) != MOE_OK) return st;
    if (!router_packed || !logits || !out || !aligned16(router_packed) || !aligned16(out))
        return fail(MOE_ERR_INVALID_ARG, "router, logits or out NULL / unaligned");
    if ((y && !aligned16(y)) || (residual && !aligned16(residual)))
        return fail(MOE_ERR_INVALID_ARG, "y or residual unaligned");
    if (cpl_for(sh.hidden * kmul(sh)) > 2)
        return fail(MOE_ERR_UNSUPPORTED, "single-launch decode layer serves rows of at most 4096 int4 codes (hidden "
                    "<= 4096 with 4-bit experts, <= 2048 with 8-bit)");
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
    a.tlogits = (uint64_t*)align_up((size_t)((char*)ws + W.tlogits), 16384);
    a.tl_stride = 2 * tl_half(sh) / 8;
    a.tl_copy = tl_half(sh) / 8;
    a.th = (uint64_t*)(T == 1 ? align_up((size_t)((char*)ws + W.th), 16384) : (size_t)((char*)ws + W.th));
    a.L = expert_layout(sh);
    a.T = T;
    a.H = sh.hidden;
    a.I = sh.inter;
    a.E = sh.n_experts;
    a.k = sh.top_k;
    a.has_shared = sh.has_shared;
    a.R = router_rows(sh);
    a.kmul = kmul(sh);
    a.norm_eps = norm_eps;
    // 16 KiB covers the kernel's static LDS (selection results, distinct-expert lists)
    // h rows and their chunk sums, then (when staged) x and its chunk sums
    const size_t lds_h = hsh_bytes(sh) + (size_t)n_slots(sh) * (sh.inter / 32) * 4, lds_x = xsh_bytes(sh, T);
    const int max_lds = device_max_lds();
    if (max_lds <= 0) return fail(MOE_ERR_HIP, "could not query the LDS size");
    a.stage_x = lds_h + lds_x + 16384 <= (size_t)max_lds ? 1 : 0;
    if (norm_eps >= 0.f && !a.stage_x)
        return fail(MOE_ERR_UNSUPPORTED, "decode block: the normalised activations of %d tokens do not fit in LDS", T);
    const size_t lds = lds_h + (a.stage_x ? lds_x : 0);
    const int G = std::min(cus, std::max(a.R, T * (a.H / DN_ROWS)));
    const LayerKernel f = pick_layer(a, sh.router_fmt == MOE_ROUTER_AFFINE8);
    // the workgroups wait for each other, so all G must be resident at once
    const int nb = layer_blocks_per_cu(f, lds);
    if (nb <= 0 || (long long)nb * cus < G)
        return fail(MOE_ERR_UNSUPPORTED, "decode layer: %d workgroups of %d threads with %zu bytes of LDS cannot all be "
                    "resident (%d per compute unit, %d compute units)", G, LTH, lds, nb, cus);
    void* args[] = {&a};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(f), dim3(G), dim3(LTH), args, lds, hs);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "decode_layer_kernel: %s", hipGetErrorString(e));
    return check_launch("decode_layer_kernel");
}

extern "C" moe_status moe_decode_layer(const moe_shape* shape, const void* router_packed, const float* logit_bias,
                                       const void* experts_packed, const uint16_t* x, int32_t T, void* ws,
                                       size_t ws_bytes, float* logits, int32_t* ids, uint16_t* w, uint16_t* w_shared,
                                       float* y, const uint16_t* residual, uint16_t* out, void* stream) {
    clear_error();
    return decode_layer_launch(shape, router_packed, logit_bias, experts_packed, x, T, ws, ws_bytes, logits, ids, w,
                               w_shared, y, residual, out, -1.f, stream);
}

extern "C" moe_status moe_decode_block(const moe_shape* shape, const void* router_packed, const float* logit_bias,
                                       const void* experts_packed, const uint16_t* x, int32_t T, float eps, void* ws,
                                       size_t ws_bytes, float* logits, int32_t* ids, uint16_t* w,
                                       uint16_t* w_shared, float* y, uint16_t* x_out, void* stream) {
    clear_error();
    if (!(eps >= 0.f)) return fail(MOE_ERR_INVALID_ARG, "eps must be >= 0");
    if (x && x_out && (const void*)x == (const void*)x_out)
        return fail(MOE_ERR_INVALID_ARG, "x_out may not alias x (other workgroups still read x)");
    return decode_layer_launch(shape, router_packed, logit_bias, experts_packed, x, T, ws, ws_bytes, logits, ids, w,
                               w_shared, y, x, x_out, eps, stream);
}

extern "C" moe_status moe_decode_layer_check(const moe_shape* shape, int32_t T, void* ws, size_t ws_bytes,
                                             void* stream) {
    clear_error();
    moe_status st = validate_shape(shape);
    if (st != MOE_OK) return st;
    if (T < 1 || T > 16) return fail(MOE_ERR_INVALID_ARG, "decode path takes 1..16 rows, got T = %d", T);
    if (!ws || !aligned16(ws)) return fail(MOE_ERR_INVALID_ARG, "NULL or unaligned workspace");
    if (ws_bytes < moe_decode_workspace_bytes(shape, T)) return fail(MOE_ERR_WORKSPACE, "decode workspace too small");
    unsigned* err = &reinterpret_cast<DecodeCtl*>((char*)ws + decode_ws_layout(*shape, T).ctl)->error;
    unsigned v = 0;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess ||
        hipMemcpy(&v, err, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess)
        return fail(MOE_ERR_HIP, "could not read the decode error word");
    if (v == 0) return MOE_OK;
    if (hipMemset(err, 0, sizeof(v)) != hipSuccess) return fail(MOE_ERR_HIP, "could not clear the decode error word");
    return fail(MOE_ERR_TIMEOUT, "a bounded wait of moe_decode_layer timed out; outputs since the last check are "
                                 "undefined");
}

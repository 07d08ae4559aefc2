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

// ---------------------------------------------------------------- XCD-aware item mapping
// The GEMM grids are one-dimensional over (tile, column block) items, numbered
// tile-major so that neighbouring items share an activation tile or an expert's
// weights. Workgroups are handed to the 8 XCDs round-robin by linear id, and each
// XCD has its own L2, so block b takes item (b % 8) * per + b / 8: each XCD walks
// one contiguous range of items and the sharing stays inside one L2. The grid is
// 8 * ceil(max_tiles * nb / 8) blocks; blocks beyond the live items return.
constexpr int N_XCD = 8;

__device__ __forceinline__ bool xcd_item(int ntiles, int nb, int& tile, int& cb) {
    const int n = ntiles * nb, per = (n + N_XCD - 1) / N_XCD;
    const int j = (int)blockIdx.x / N_XCD, item = ((int)blockIdx.x % N_XCD) * per + j;
    if (j >= per || item >= n) return false;
    tile = item / nb;
    cb = item - tile * nb;
    return true;
}

static unsigned xcd_grid(int max_tiles, int nb) {
    return (unsigned)((((long long)max_tiles * nb + N_XCD - 1) / N_XCD) * N_XCD);
}

// ---------------------------------------------------------------- staged GEMM core
// Both expert GEMMs walk K in chunks of KC = 128 (two quantisation groups). Per
// chunk a workgroup stages, with coalesced 16-byte loads:
//   A: 64 activation rows x 128 bf16 (256 contiguous bytes per row; 16 lanes per
//      row), stored in LDS as they are, with the per-group row sums X;
//   B: NB int4 weight rows x 64 bytes (4 lanes per row) and their two (scale, bias)
//      words.
// The next chunk's loads are issued into registers before the current chunk is
// multiplied, so they are in flight during the MFMAs; two barriers per chunk.
constexpr int KC = 128;
constexpr int AS = KC + 8;       // A row stride in LDS (bf16)
constexpr int BS = KC / 2 + 16;  // B row stride in LDS (bytes)

// Sum over aligned groups of 8 lanes (DPP); the result is in every lane of the group.
__device__ __forceinline__ float sum8_lanes(float v) {
    v += __uint_as_float(dpp_u32<0xB1, 0xF>(__float_as_uint(v)));
    v += __uint_as_float(dpp_u32<0x4E, 0xF>(__float_as_uint(v)));
    v += __uint_as_float(dpp_u32<0x141, 0xF>(__float_as_uint(v)));
    return v;
}

// A chunk: thread tid holds 16-byte piece c16 = tid % 16 of rows tid/16 + 16 j.
struct AChunk {
    uint4 v[4];
};

__device__ __forceinline__ void load_a(const uint16_t* const rowp[4], int c, int kc_valid, int tid, AChunk& a) {
    const int c16 = tid & 15;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        a.v[j] = (rowp[j] && 8 * c16 < kc_valid) ? *reinterpret_cast<const uint4*>(rowp[j] + c * KC + 8 * c16)
                                                 : make_uint4(0, 0, 0, 0);
}

__device__ __forceinline__ void store_a(uint16_t* __restrict__ a_lds, float (*x_lds)[64], const AChunk& a, int tid) {
    const int c16 = tid & 15;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = (tid >> 4) + 16 * j;
        const uint32_t in[4] = {a.v[j].x, a.v[j].y, a.v[j].z, a.v[j].w};
        *reinterpret_cast<uint4*>(a_lds + row * AS + 8 * c16) = a.v[j];
        float sm = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sm += bf16_to_f32(in[i] & 0xFFFFu);
            sm += bf16_to_f32(in[i] >> 16);
        }
        sm = sum8_lanes(sm);
        if ((c16 & 7) == 0) x_lds[c16 >> 3][row] = sm;
    }
}

// B chunk of NB rows: thread tid holds 16-byte piece tid % 4 of rows tid/4 + 64 j,
// and (tid < NB) the two (scale, bias) words of row tid.
template <int NB>
struct BChunk {
    uint4 v[NB / 64];
    uint2 sb;
};

template <int NB, typename RowQ, typename RowSB>
__device__ __forceinline__ void load_b(RowQ rowq, RowSB rowsb, int c, int kc_valid, int tid, BChunk<NB>& b) {
    const int c4 = tid & 3;
#pragma unroll
    for (int j = 0; j < NB / 64; ++j) {
        const int row = (tid >> 2) + 64 * j;
        b.v[j] = 16 * c4 < kc_valid / 2 ? *reinterpret_cast<const uint4*>(rowq(row) + c * (KC / 2) + 16 * c4)
                                        : make_uint4(0, 0, 0, 0);
    }
    if (tid < NB) {
        const uint32_t* sp = rowsb(tid) + c * (KC / 64);
        b.sb.x = sp[0];
        b.sb.y = kc_valid > 64 ? sp[1] : 0u;
    }
}

template <int NB>
__device__ __forceinline__ void store_b(uint8_t* __restrict__ b_lds, uint2* __restrict__ sb_lds, const BChunk<NB>& b,
                                        int tid) {
    const int c4 = tid & 3;
#pragma unroll
    for (int j = 0; j < NB / 64; ++j) {
        const int row = (tid >> 2) + 64 * j;
        *reinterpret_cast<uint4*>(b_lds + row * BS + 16 * c4) = b.v[j];
    }
    if (tid < NB) sb_lds[tid] = b.sb;
}

// One 64-wide group gi of the staged chunk for weight row br: accumulates
// 16*s*P + (b - 16*s)*X into acc for the m-subtiles below n_ms.
__device__ __forceinline__ void mma_group(const uint16_t* __restrict__ a_lds, const float (*x_lds)[64],
                                          const uint8_t* __restrict__ b_lds, const uint2* __restrict__ sb_lds, int br,
                                          int gi, int n_ms, int lc, int lg, f32x4_t acc[4]) {
    const uint8_t* bp = b_lds + br * BS + 32 * gi + 4 * lg;
    const uint4 b0 = bfrag(*reinterpret_cast<const uint32_t*>(bp));
    const uint4 b1 = bfrag(*reinterpret_cast<const uint32_t*>(bp + 16));
    const uint2 sbw = sb_lds[br];
    const uint32_t sb = gi ? sbw.y : sbw.x;
    const float s16 = 16.f * bf16_to_f32(sb & 0xFFFFu), cc = bf16_to_f32(sb >> 16) - s16;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        if (m < n_ms) {
            const uint16_t* ar = a_lds + (16 * m + lc) * AS + 64 * gi + 8 * lg;
            const uint4 a0 = *reinterpret_cast<const uint4*>(ar);
            const uint4 a1 = *reinterpret_cast<const uint4*>(ar + 32);
            const float4 xs = *reinterpret_cast<const float4*>(&x_lds[gi][16 * m + 4 * lg]);
            f32x4_t p = mfma16x16x32(a0, b0, f32x4_t{0.f, 0.f, 0.f, 0.f});
            p = mfma16x16x32(a1, b1, p);
            acc[m][0] = fmaf(cc, xs.x, fmaf(s16, p[0], acc[m][0]));
            acc[m][1] = fmaf(cc, xs.y, fmaf(s16, p[1], acc[m][1]));
            acc[m][2] = fmaf(cc, xs.z, fmaf(s16, p[2], acc[m][2]));
            acc[m][3] = fmaf(cc, xs.w, fmaf(s16, p[3], acc[m][3]));
        }
    }
}

// ---------------------------------------------------------------- gate/up + SwiGLU
// Items: (tile, ib) for ib < I / 64. B rows 0..63 are gate rows ib*64 .., rows
// 64..127 the matching up rows. Wavefront w computes gate and up for intermediate columns
// ib*64 + 16w .. +16 over the tile's rows and writes h[row][i] = bf16(silu(gate) * up)
// in expert-sorted row order.
__global__ __launch_bounds__(256) void gateup_gemm_kernel(const uint8_t* __restrict__ packed, ExpertLayout L, int H,
                                                          int I, int S, const uint16_t* __restrict__ x,
                                                          const int32_t* __restrict__ ntiles,
                                                          const Tile* __restrict__ tiles,
                                                          const int32_t* __restrict__ order,
                                                          uint16_t* __restrict__ hbuf) {
    __shared__ __attribute__((aligned(16))) uint16_t a_lds[BM * AS];
    __shared__ __attribute__((aligned(16))) float x_lds[2][64];
    __shared__ __attribute__((aligned(16))) uint8_t b_lds[128 * BS];
    __shared__ __attribute__((aligned(16))) uint2 sb_lds[128];
    int ti, ib;
    if (!xcd_item(*ntiles, I / BN, ti, ib)) return;
    const Tile tl = tiles[ti];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lg = lane >> 4, lc = lane & 15;
    const int i0 = ib * BN;
    const int n_ms = (tl.nrows + 15) >> 4;

    const uint16_t* rowp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = (tid >> 4) + 16 * j;
        rowp[j] = row < tl.nrows ? x + (size_t)(order[tl.row0 + row] / S) * H : nullptr;
    }
    const uint8_t* base = packed + (size_t)tl.expert * L.stride;
    const uint8_t* gq = base + L.gate_q + (size_t)i0 * (H / 2);
    const uint8_t* uq = base + L.up_q + (size_t)i0 * (H / 2);
    const uint32_t* gsb = reinterpret_cast<const uint32_t*>(base + L.gate_sb) + (size_t)i0 * (H / 64);
    const uint32_t* usb = reinterpret_cast<const uint32_t*>(base + L.up_sb) + (size_t)i0 * (H / 64);
    auto rowq = [&](int r) { return r < 64 ? gq + (size_t)r * (H / 2) : uq + (size_t)(r - 64) * (H / 2); };
    auto rowsb = [&](int r) { return r < 64 ? gsb + (size_t)r * (H / 64) : usb + (size_t)(r - 64) * (H / 64); };

    f32x4_t accg[4], accu[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        accg[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        accu[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const int NC = (H + KC - 1) / KC;
    AChunk ac;
    BChunk<128> bc;
    load_a(rowp, 0, min(KC, H), tid, ac);
    load_b<128>(rowq, rowsb, 0, min(KC, H), tid, bc);
    for (int c = 0; c < NC; ++c) {
        const int kcv = min(KC, H - c * KC);
        store_a(a_lds, x_lds, ac, tid);
        store_b<128>(b_lds, sb_lds, bc, tid);
        __syncthreads();
        if (c + 1 < NC) {
            const int kn = min(KC, H - (c + 1) * KC);
            load_a(rowp, c + 1, kn, tid, ac);
            load_b<128>(rowq, rowsb, c + 1, kn, tid, bc);
        }
        for (int gi = 0; gi < kcv / 64; ++gi) {
            mma_group(a_lds, x_lds, b_lds, sb_lds, wave * 16 + lc, gi, n_ms, lc, lg, accg);
            mma_group(a_lds, x_lds, b_lds, sb_lds, 64 + wave * 16 + lc, gi, n_ms, lc, lg, accu);
        }
        __syncthreads();
    }
    const int i_col = i0 + wave * 16 + lc;
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
// Items: (tile, nb) for nb < H / 64. B rows are down rows nb*64 .. +64; A = h rows,
// contiguous in expert-sorted order. Wavefront w computes output columns
// nb*64 + 16w .. +16 and writes y[p][n] for the row's pick p = order[row].
__global__ __launch_bounds__(256) void down_gemm_kernel(const uint8_t* __restrict__ packed, ExpertLayout L, int H,
                                                        int I, const int32_t* __restrict__ ntiles,
                                                        const Tile* __restrict__ tiles,
                                                        const int32_t* __restrict__ order,
                                                        const uint16_t* __restrict__ hbuf, float* __restrict__ y) {
    __shared__ __attribute__((aligned(16))) uint16_t a_lds[BM * AS];
    __shared__ __attribute__((aligned(16))) float x_lds[2][64];
    __shared__ __attribute__((aligned(16))) uint8_t b_lds[64 * BS];
    __shared__ __attribute__((aligned(16))) uint2 sb_lds[64];
    int ti, nbk;
    if (!xcd_item(*ntiles, H / BN, ti, nbk)) return;
    const Tile tl = tiles[ti];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lg = lane >> 4, lc = lane & 15;
    const int n0 = nbk * BN;
    const int n_ms = (tl.nrows + 15) >> 4;

    const uint16_t* rowp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = (tid >> 4) + 16 * j;
        rowp[j] = row < tl.nrows ? hbuf + (size_t)(tl.row0 + row) * I : nullptr;
    }
    const uint8_t* base = packed + (size_t)tl.expert * L.stride;
    const uint8_t* dq = base + L.down_q + (size_t)n0 * (I / 2);
    const uint32_t* dsb = reinterpret_cast<const uint32_t*>(base + L.down_sb) + (size_t)n0 * (I / 64);
    auto rowq = [&](int r) { return dq + (size_t)r * (I / 2); };
    auto rowsb = [&](int r) { return dsb + (size_t)r * (I / 64); };

    f32x4_t acc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int NC = (I + KC - 1) / KC;
    AChunk ac;
    BChunk<64> bc;
    load_a(rowp, 0, min(KC, I), tid, ac);
    load_b<64>(rowq, rowsb, 0, min(KC, I), tid, bc);
    for (int c = 0; c < NC; ++c) {
        const int kcv = min(KC, I - c * KC);
        store_a(a_lds, x_lds, ac, tid);
        store_b<64>(b_lds, sb_lds, bc, tid);
        __syncthreads();
        if (c + 1 < NC) {
            const int kn = min(KC, I - (c + 1) * KC);
            load_a(rowp, c + 1, kn, tid, ac);
            load_b<64>(rowq, rowsb, c + 1, kn, tid, bc);
        }
        for (int gi = 0; gi < kcv / 64; ++gi)
            mma_group(a_lds, x_lds, b_lds, sb_lds, wave * 16 + lc, gi, n_ms, lc, lg, acc);
        __syncthreads();
    }
    const int n_col = n0 + wave * 16 + lc;
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
    hipLaunchKernelGGL(gateup_gemm_kernel, dim3(xcd_grid(W.max_tiles, I / BN)), dim3(256), 0, hs, p, L, H, I, S, x, ntiles,
                       tiles, order, hbuf);
    if ((st = check_launch("gateup_gemm_kernel")) != MOE_OK) return st;
    hipLaunchKernelGGL(down_gemm_kernel, dim3(xcd_grid(W.max_tiles, H / BN)), dim3(256), 0, hs, p, L, H, I, ntiles, tiles, order,
                       hbuf, y);
    return check_launch("down_gemm_kernel");
}

// Prefill path: dispatch of the T*S picks into expert-sorted rows, then two
// grouped GEMMs on the matrix cores (the tensor-core MoE GEMM with int4 dequant
// and dispatch table of the AGX Orin port, "Phase 9b", re-designed for CDNA4).
//
// GEMM operands (exact): activations enter as bf16; each int4 weight q enters the
// MFMA as the bf16 value 1 + q/16 (exact), so one 64-wide group's MFMA partial is
// P = sum x*(1 + q/16). With X = sum x over the same group the group's
// contribution is 16*scale*P + (bias - 16*scale)*X. The first term is applied per
// group on the accumulator (one fp32 FMA per output); the second, summed over the
// groups, is itself a small product of row sums X[row][g] and column terms
// c[col][g] = bias - 16*scale, done at the end of the tile on the matrix cores
// with X and c each split into three bf16 parts (products exact, the neglected
// parts below 2^-24 relative). X of the activations comes from a pre-pass, X of h
// from the gate/up epilogue. No weight is rounded.
//
// Tiles: 128 expert-sorted rows x 64*NCS weight rows per workgroup of four
// wavefronts (gate/up, NCS = 2: 64 gate + 64 up rows of the same 64 intermediate
// columns; down, NCS = 4: 256 output columns); wavefront w owns weight rows
// cs*64 + 16w .. (cs < NCS) over all 128 rows, with v_mfma_f32_16x16x32_bf16 in the
// main loop, so every activation fragment read from LDS feeds NCS products.
#include <type_traits>

#include "mfma_common.h"
#include "moe_internal.h"

namespace moe {

constexpr int BM = 128;  // rows per tile

struct Tile {
    int32_t expert, row0, nrows, pad;
};

// Workspace layout for moe_experts_prefill.
struct PrefillWs {
    size_t counts, offsets, cursor, ntiles, tiles, order, h, xs_x, xs_h, total;
    int max_tiles, gs_x, gs_h;  // group strides of the row-sum planes (multiples of 16)
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
    w.gs_x = ((s.hidden / 64 + 15) / 16) * 16;
    w.gs_h = ((s.inter / 64 + 15) / 16) * 16;
    w.xs_x = o;    o = align_up(o + 3 * 2 * (size_t)T * w.gs_x, 256);      // [3][T][gs_x] bf16
    w.xs_h = o;    o = align_up(o + 3 * 2 * (size_t)T * S * w.gs_h, 256);  // [3][T*S][gs_h] bf16
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

// ---------------------------------------------------------------- row sums in three bf16 parts
// v = hi + mid + lo: hi and mid are v and the remainder truncated to bf16 (both
// remainders exact in fp32), lo the last remainder rounded to bf16.
__device__ __forceinline__ void split3_bf16(float v, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
    const uint32_t h = __float_as_uint(v) & 0xFFFF0000u;
    const float r1 = v - __uint_as_float(h);
    const uint32_t m = __float_as_uint(r1) & 0xFFFF0000u;
    const float r2 = r1 - __uint_as_float(m);
    hi = h >> 16;
    mid = m >> 16;
    lo = f32_to_bf16(r2);
}

// X[t][g] = sum of x[t][64g .. 64g+63] (a chain of bf16 dot2 against (1, 1)) for
// g < H/64, zero for the padding groups up to gs; stored as three bf16 planes.
__global__ __launch_bounds__(256) void xsum_kernel(const uint16_t* __restrict__ x, int T, int H, int gs,
                                                   uint16_t* __restrict__ planes) {
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long long)T * gs) return;
    const int t = (int)(idx / gs), g = (int)(idx % gs);
    float sum = 0.f;
    if (g < H / 64) {
        const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)t * H + 64 * g);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint4 v = src[q];
            sum = dot2_bf16(v.x, 0x3F803F80u, sum);
            sum = dot2_bf16(v.y, 0x3F803F80u, sum);
            sum = dot2_bf16(v.z, 0x3F803F80u, sum);
            sum = dot2_bf16(v.w, 0x3F803F80u, sum);
        }
    }
    uint32_t hi, mid, lo;
    split3_bf16(sum, hi, mid, lo);
    const size_t plane = (size_t)T * gs;
    planes[idx] = (uint16_t)hi;
    planes[plane + idx] = (uint16_t)mid;
    planes[2 * plane + idx] = (uint16_t)lo;
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

// ---------------------------------------------------------------- grouped GEMM
// K walks in chunks of KC = 128 (two groups). Per chunk a workgroup stages, with
// coalesced 16-byte loads:
//   A: 128 activation rows x 128 bf16 (256 contiguous bytes per row, 16 lanes per
//      row; rows beyond the tile are not loaded);
//   B: 128 int4 weight rows x 64 bytes (4 lanes per row) and their (scale, bias)
//      words for the two groups.
// The next chunk's loads are issued into registers before the current chunk is
// multiplied; two barriers per chunk.
constexpr int KC = 128;
constexpr int AS = KC + 8;       // A row stride in LDS (bf16): 16-lane groups read distinct banks
constexpr int BS = KC / 2 + 16;  // B row stride in LDS (bytes): the 64 fragment lanes read distinct banks
// weight rows per workgroup: 64 * NCS, NCS = 16-column sets per wavefront (2 for
// gate/up, 4 for down; measured)

struct GemmArgs {
    const uint8_t* packed;
    ExpertLayout L;
    int H, I, S;
    const uint16_t* x;          // gate/up: activations [T][H]
    const int32_t* ntiles;
    const Tile* tiles;
    const int32_t* order;
    uint16_t* hbuf;             // h [T*S][I] bf16, expert-sorted rows (written by gate/up, read by down)
    float* y;                   // down: [T][S][H]
    const uint16_t* xs_a;       // row-sum planes of this GEMM's A rows
    uint16_t* xs_h;             // gate/up: row-sum planes of h (written)
    int T, gs_a, gs_h;
};

typedef short short4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16x16x16(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, a), __builtin_bit_cast(short4_t, b),
                                                     c, 0, 0, 0);
}

// GATEUP: B rows 0..127 are gate rows cb*128 .., rows 128..255 the matching up
// rows; the epilogue writes h = bf16(silu(gate) * up) and the row sums of that h
// block (two groups of the down GEMM's K). Else (down): B rows are down rows
// cb*256 ..; the epilogue writes y[t][s][n] for the row's pick p = order[row].
// Wavefront w owns B rows cs*64 + 16w .. +16 for cs < 4.
template <bool GATEUP, int NCS>
__global__ __launch_bounds__(256, 2) void expert_gemm_kernel(GemmArgs a) {
    constexpr int NBR = 64 * NCS;  // weight rows per workgroup
    constexpr int HALF = NBR / 2;  // gate/up: gate rows 0 .. HALF-1, up rows HALF .. NBR-1
    __shared__ __attribute__((aligned(16))) uint16_t a_lds[BM * AS];
    __shared__ __attribute__((aligned(16))) uint8_t b_lds[NBR * BS];
    __shared__ __attribute__((aligned(16))) uint2 sb_lds[NBR];
    __shared__ float xpart[NCS / 2][4][BM];
    __shared__ uint32_t arow_lds[BM];  // element offset of each tile row in its source, ~0 beyond the tile
    const int H = a.H, I = a.I, S = a.S;
    const int K = GATEUP ? H : I;
    const int nblk = GATEUP ? (I + HALF - 1) / HALF : (H + NBR - 1) / NBR;
    int ti, cb;
    if (!xcd_item(*a.ntiles, nblk, ti, cb)) return;
    const Tile tl = a.tiles[ti];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lg = lane >> 4, lc = lane & 15;
    const int n_ms = (tl.nrows + 15) >> 4;
    const int col0 = GATEUP ? cb * HALF : cb * NBR;

    // A rows: this thread stages 16-byte piece c16 of rows tid/16 + 16 j
    const int c16 = tid & 15;
    if (tid < BM) {
        uint32_t off = 0xFFFFFFFFu;
        if (tid < tl.nrows) {
            if constexpr (GATEUP) off = (uint32_t)((a.order[tl.row0 + tid] / S) * H);
            else off = (uint32_t)((tl.row0 + tid) * I);
        }
        arow_lds[tid] = off;
    }
    __syncthreads();
    const uint16_t* asrc = GATEUP ? a.x : a.hbuf;
    // B rows: this thread stages 16-byte piece c4 of rows tid/4 + 64 j
    const uint8_t* ebase = a.packed + (size_t)tl.expert * a.L.stride;
    auto brow_q = [&](int r) -> const uint8_t* {
        if constexpr (GATEUP) return ebase + (r < HALF ? a.L.gate_q : a.L.up_q) + (size_t)(col0 + r % HALF) * (K / 2);
        else return ebase + a.L.down_q + (size_t)(col0 + r) * (K / 2);
    };
    auto brow_sb = [&](int r) -> const uint32_t* {
        if constexpr (GATEUP)
            return reinterpret_cast<const uint32_t*>(ebase + (r < HALF ? a.L.gate_sb : a.L.up_sb)) +
                   (size_t)(col0 + r % HALF) * (K / 64);
        else return reinterpret_cast<const uint32_t*>(ebase + a.L.down_sb) + (size_t)(col0 + r) * (K / 64);
    };
    auto brow_ok = [&](int r) -> bool { return GATEUP ? col0 + r % HALF < I : col0 + r < H; };
    const int c4 = tid & 3;

    // a chunk's staged loads (chunk c+1 loads while chunk c is multiplied)
    struct ChunkRegs {
        uint4 av[8], bv[NBR / 64];
        uint2 sbv;
    };
    auto load_chunk_regs = [&](ChunkRegs& R, int c) {
        const int kcv = min(KC, K - c * KC);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t off = arow_lds[(tid >> 4) + 16 * j];
            R.av[j] = (off != 0xFFFFFFFFu && 8 * c16 < kcv)
                          ? *reinterpret_cast<const uint4*>(asrc + off + c * KC + 8 * c16)
                          : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int j = 0; j < NBR / 64; ++j) {
            const int r = (tid >> 2) + 64 * j;
            R.bv[j] = (brow_ok(r) && 16 * c4 < kcv / 2)
                          ? *reinterpret_cast<const uint4*>(brow_q(r) + c * (KC / 2) + 16 * c4)
                          : make_uint4(0u, 0u, 0u, 0u);
        }
        R.sbv = make_uint2(0u, 0u);
        if (tid < NBR) {
            const uint32_t* sp = brow_sb(tid) + c * (KC / 64);
            R.sbv.x = brow_ok(tid) ? sp[0] : 0u;
            R.sbv.y = (brow_ok(tid) && kcv > 64) ? sp[1] : 0u;
        }
    };
    auto store_chunk = [&](const ChunkRegs& R) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            *reinterpret_cast<uint4*>(a_lds + ((tid >> 4) + 16 * j) * AS + 8 * c16) = R.av[j];
#pragma unroll
        for (int j = 0; j < NBR / 64; ++j)
            *reinterpret_cast<uint4*>(b_lds + ((tid >> 2) + 64 * j) * BS + 16 * c4) = R.bv[j];
        if (tid < NBR) sb_lds[tid] = R.sbv;
    };

    f32x4_t acc[8][NCS];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int cs = 0; cs < NCS; ++cs) acc[m][cs] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // The K loop is instantiated for 1, 2, 4 and 8 row blocks of 16 (the tile's count
    // rounded up), so its body is straight-line code the compiler can interleave;
    // the rows beyond the tile are zeros in LDS.
    auto kloop = [&](auto nm_tag) {
        constexpr int NM = decltype(nm_tag)::value;
        const int NC = (K + KC - 1) / KC;
        auto compute = [&](int c) {
            const int kcv = min(KC, K - c * KC);
            for (int gi = 0; gi < kcv / 64; ++gi) {
                uint4 b0[NCS], b1[NCS];
                float s16[NCS];
#pragma unroll
                for (int cs = 0; cs < NCS; ++cs) {
                    const int br = cs * 64 + 16 * wave + lc;
                    const uint8_t* bp = b_lds + br * BS + 32 * gi + 4 * lg;
                    b0[cs] = bfrag(*reinterpret_cast<const uint32_t*>(bp));
                    b1[cs] = bfrag(*reinterpret_cast<const uint32_t*>(bp + 16));
                    const uint2 w = sb_lds[br];
                    s16[cs] = 16.f * bf16_to_f32((gi ? w.y : w.x) & 0xFFFFu);
                }
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    const uint16_t* ar = a_lds + (16 * m + lc) * AS + 64 * gi + 8 * lg;
                    const uint4 a0 = *reinterpret_cast<const uint4*>(ar);
                    const uint4 a1 = *reinterpret_cast<const uint4*>(ar + 32);
#pragma unroll
                    for (int cs = 0; cs < NCS; ++cs) {
                        f32x4_t p = mfma16x16x32(a0, b0[cs], f32x4_t{0.f, 0.f, 0.f, 0.f});
                        p = mfma16x16x32(a1, b1[cs], p);
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[m][cs][r] = fmaf(s16[cs], p[r], acc[m][cs][r]);
                    }
                }
            }
        };
        ChunkRegs r0;
        load_chunk_regs(r0, 0);
        for (int c = 0; c < NC; ++c) {
            store_chunk(r0);
            __syncthreads();
            if (c + 1 < NC) load_chunk_regs(r0, c + 1);
            compute(c);
            __syncthreads();
        }
    };
    if (n_ms <= 1) kloop(std::integral_constant<int, 1>{});
    else if (n_ms <= 2) kloop(std::integral_constant<int, 2>{});
    else if (n_ms <= 4) kloop(std::integral_constant<int, 4>{});
    else kloop(std::integral_constant<int, 8>{});

    // ---- bias term: sum over groups of X[row][g] * (bias - 16 scale)[col][g], 16 groups per MFMA
    const int G = K / 64;
    for (int kb = 0; kb < (G + 15) / 16; ++kb) {
        uint2 ch[NCS], cm[NCS], cl[NCS];
#pragma unroll
        for (int cs = 0; cs < NCS; ++cs) {
            const int br = cs * 64 + 16 * wave + lc;
            uint32_t h4[4], m4[4], l4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int g = 16 * kb + 4 * lg + i;
                float cc = 0.f;
                if (g < G && brow_ok(br)) {
                    const uint32_t w = brow_sb(br)[g];
                    cc = bf16_to_f32(w >> 16) - 16.f * bf16_to_f32(w & 0xFFFFu);
                }
                split3_bf16(cc, h4[i], m4[i], l4[i]);
            }
            ch[cs] = make_uint2(h4[0] | (h4[1] << 16), h4[2] | (h4[3] << 16));
            cm[cs] = make_uint2(m4[0] | (m4[1] << 16), m4[2] | (m4[3] << 16));
            cl[cs] = make_uint2(l4[0] | (l4[1] << 16), l4[2] | (l4[3] << 16));
        }
        const size_t plane = (size_t)(GATEUP ? a.T : a.T * S) * a.gs_a;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            if (m < n_ms) {
                const int row = 16 * m + lc;
                uint2 xh = make_uint2(0u, 0u), xm = xh, xl = xh;
                if (row < tl.nrows) {
                    const int src = GATEUP ? a.order[tl.row0 + row] / S : tl.row0 + row;
                    const uint16_t* xp = a.xs_a + (size_t)src * a.gs_a + 16 * kb + 4 * lg;
                    xh = *reinterpret_cast<const uint2*>(xp);
                    xm = *reinterpret_cast<const uint2*>(xp + plane);
                    xl = *reinterpret_cast<const uint2*>(xp + 2 * plane);
                }
#pragma unroll
                for (int cs = 0; cs < NCS; ++cs) {
                    f32x4_t v = acc[m][cs];
                    v = mfma16x16x16(xh, ch[cs], v);
                    v = mfma16x16x16(xh, cm[cs], v);
                    v = mfma16x16x16(xm, ch[cs], v);
                    v = mfma16x16x16(xh, cl[cs], v);
                    v = mfma16x16x16(xl, ch[cs], v);
                    v = mfma16x16x16(xm, cm[cs], v);
                    acc[m][cs] = v;
                }
            }
        }
    }

    // ---- epilogue
    if constexpr (GATEUP) {
        // h[row][i] = bf16(silu(gate) * up), i = col0 + 64 hs + 16 wave + lc (gate set
        // hs, up set NCS/2 + hs); row sums of each 64-column part hs of this block of
        // h (fp32, fixed order: 16 lanes by DPP, then the four wavefronts in order)
        // into the down GEMM's X planes, group col0/64 + hs
#pragma unroll
        for (int hs = 0; hs < NCS / 2; ++hs) {
            const int i_col = col0 + 64 * hs + 16 * wave + lc;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * m + 4 * lg + r;
                    const float gv = acc[m][hs][r], uv = acc[m][NCS / 2 + hs][r];
                    const uint32_t hb = f32_to_bf16(gv / (1.f + expf(-gv)) * uv);
                    if (row < tl.nrows && i_col < I) a.hbuf[(size_t)(tl.row0 + row) * I + i_col] = (uint16_t)hb;
                    const float part = group_sum(row < tl.nrows ? bf16_to_f32(hb) : 0.f, 16);
                    if (lc == 0) xpart[hs][wave][row] = part;
                }
            }
        }
        __syncthreads();
        if (tid < (NCS / 2) * BM && (tid & (BM - 1)) < tl.nrows && col0 + 64 * (tid / BM) < I) {
            const int row = tid & (BM - 1), hs = tid / BM, g = col0 / 64 + hs;
            const float xs = ((xpart[hs][0][row] + xpart[hs][1][row]) + xpart[hs][2][row]) + xpart[hs][3][row];
            uint32_t hi, mid, lo;
            split3_bf16(xs, hi, mid, lo);
            const size_t plane = (size_t)a.T * S * a.gs_h;
            uint16_t* xp = a.xs_h + (size_t)(tl.row0 + row) * a.gs_h;
            xp[g] = (uint16_t)hi;
            xp[plane + g] = (uint16_t)mid;
            xp[2 * plane + g] = (uint16_t)lo;
            if (col0 == 0 && hs == 0) {  // padding groups of the planes
                for (int gp = I / 64; gp < a.gs_h; ++gp) {
                    xp[gp] = 0;
                    xp[plane + gp] = 0;
                    xp[2 * plane + gp] = 0;
                }
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * m + 4 * lg + r;
                if (row < tl.nrows) {
                    float* yr = a.y + (size_t)a.order[tl.row0 + row] * H;
#pragma unroll
                    for (int cs = 0; cs < NCS; ++cs) {
                        const int n = col0 + cs * 64 + 16 * wave + lc;
                        if (n < H) yr[n] = acc[m][cs][r];
                    }
                }
            }
        }
    }
}

static_assert(BM == 128, "tile rows");

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
    GemmArgs ga;
    ga.packed = (const uint8_t*)experts_packed;
    ga.L = L;
    ga.H = H;
    ga.I = I;
    ga.S = S;
    ga.x = x;
    ga.ntiles = ntiles;
    ga.tiles = tiles;
    ga.order = order;
    ga.hbuf = hbuf;
    ga.y = y;
    ga.T = T;
    ga.gs_h = W.gs_h;
    uint16_t* xs_x = (uint16_t*)(w + W.xs_x);
    uint16_t* xs_h = (uint16_t*)(w + W.xs_h);
    const long long nsum = (long long)T * W.gs_x;
    hipLaunchKernelGGL(xsum_kernel, dim3((unsigned)((nsum + 255) / 256)), dim3(256), 0, hs, x, T, H, W.gs_x, xs_x);
    if ((st = check_launch("xsum_kernel")) != MOE_OK) return st;
    ga.xs_a = xs_x;
    ga.xs_h = xs_h;
    ga.gs_a = W.gs_x;
    hipLaunchKernelGGL((expert_gemm_kernel<true, 2>), dim3(xcd_grid(W.max_tiles, (I + 63) / 64)), dim3(256), 0, hs, ga);
    if ((st = check_launch("expert_gemm_kernel<gate/up>")) != MOE_OK) return st;
    ga.xs_a = xs_h;
    ga.xs_h = nullptr;
    ga.gs_a = W.gs_h;
    hipLaunchKernelGGL((expert_gemm_kernel<false, 4>), dim3(xcd_grid(W.max_tiles, (H + 255) / 256)), dim3(256), 0, hs, ga);
    return check_launch("expert_gemm_kernel<down>");
}

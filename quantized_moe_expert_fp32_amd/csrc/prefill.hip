// Prefill path: dispatch of the T*S picks into expert-sorted rows, then two
// grouped GEMMs on the matrix cores (the tensor-core MoE GEMM with int4 dequant
// and dispatch table of the AGX Orin port, "Phase 9b", re-designed for CDNA4).
//
// GEMM operands (exact): activations enter as bf16; each int4 weight q enters the
// MFMA as the bf16 value 1 + q/16 (exact), so one 64-wide group's MFMA partial is
// P = sum x*(1 + q/16). With X = sum x over the same group (two more MFMAs against
// ones) the group's contribution is 16*scale*P + (bias - 16*scale)*X, added to the
// accumulator group by group with two fp32 FMAs per output. No weight is rounded,
// and every output's arithmetic depends only on its own activation row and weight
// row: a row's result is the same in any tile, at any token count, run to run.
//
// Tiles: 128 expert-sorted rows x 256 weight rows per workgroup of four
// wavefronts (gate/up: 128 gate + 128 up rows of the same 128 intermediate
// columns; down: 256 output columns); wavefront w owns weight rows cs*64 + 16w ..
// (cs < 4) over all 128 rows, with v_mfma_f32_16x16x32_bf16 in the main loop, so
// every activation fragment read from LDS feeds four products.
#include "mfma_common.h"
#include "moe_internal.h"
#include "prefill_internal.h"

namespace moe {

constexpr int BM = 128;  // rows per tile
// Up to 1024 tokens the tiles are 64 rows (the three-workgroups-per-CU GEMM takes 64
// rows per pass): a 128-row tile there ran as one item of two passes, and the shared
// expert's 128-row items, started first, ran 85 us of the 87 us gate/up launch at
// 512 tokens while the rest of the chip was done at about 60 us.
constexpr int BM3 = 64;
static int prefill_tile_rows(int T) { return T <= 1024 ? BM3 : BM; }

constexpr int SLICE = 1024;  // picks per slice (one workgroup of the dispatch each)

// ---------------------------------------------------------------- prefill layout of the experts
// A grouped-GEMM workgroup takes 256 weight rows, 64 four-row blocks of the packed
// layout, and one 64-code group of them per chunk. In the packed layout a block
// holds all its groups (4 KiB at hidden 2048), so one chunk's 64 lines sat on 64
// different 4 KiB pages; a workgroup pays for every page it touches, and small
// tiles, bound by their load latency, paid most (both GEMMs at 512 tokens read in
// this order in a timing-only build: 129.8 -> 117.8 us). The prefill layout keeps
// each set of PF_SET consecutive blocks (the last set of a matrix may be shorter) in
// the bytes it has in the packed layout, but group-major: line (block j, group g) of
// a set of n blocks sits at set + 128 (g n + j), and its (scale, bias) unit at
// sb set + 16 (g n + j). Decode keeps the packed layout, whose row-pair tasks read
// one block (one page) each.
constexpr int PF_SET = 64;

// One thread per 16-byte unit of one expert (blockIdx.y): q lines are eight units,
// sb units one. Regions in order: gate/up q, down q, gate/up sb, down sb.
__device__ __forceinline__ void pf_unit(long long u, int nblk, int G, int ub, size_t& so, size_t& dof) {
    const int per = G * (ub / 16);  // units per block
    const int b = (int)(u / per), r = (int)(u % per), g = r / (ub / 16), p = r % (ub / 16);
    const int s0 = b / PF_SET * PF_SET, n = min(PF_SET, nblk - s0);
    so = (size_t)b * G * ub + (size_t)g * ub + (size_t)p * 16;
    dof = (size_t)s0 * G * ub + ((size_t)g * n + (b - s0)) * ub + (size_t)p * 16;
}

__global__ __launch_bounds__(256) void relayout_prefill_kernel(const uint8_t* __restrict__ src,
                                                               uint8_t* __restrict__ dst, ExpertLayout L,
                                                               int nblk_gu, int G_gu, int nblk_dn, int G_dn) {
    const long long u = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long n0 = (long long)nblk_gu * G_gu * 8, n1 = (long long)nblk_dn * G_dn * 8;
    const long long n2 = (long long)nblk_gu * G_gu, n3 = (long long)nblk_dn * G_dn;
    size_t so, dof, base;
    if (u < n0) {
        base = L.gu_q;
        pf_unit(u, nblk_gu, G_gu, 128, so, dof);
    } else if (u < n0 + n1) {
        base = L.down_q;
        pf_unit(u - n0, nblk_dn, G_dn, 128, so, dof);
    } else if (u < n0 + n1 + n2) {
        base = L.gu_sb;
        pf_unit(u - n0 - n1, nblk_gu, G_gu, 16, so, dof);
    } else if (u < n0 + n1 + n2 + n3) {
        base = L.down_sb;
        pf_unit(u - n0 - n1 - n2, nblk_dn, G_dn, 16, so, dof);
    } else {
        return;
    }
    const size_t e = (size_t)blockIdx.y * L.stride + base;
    *reinterpret_cast<uint4*>(dst + e + dof) = *reinterpret_cast<const uint4*>(src + e + so);
}

DispatchWs dispatch_ws_layout(const moe_shape& s, int T, int bm, size_t& o) {
    DispatchWs w;
    const int M = n_mats(s);
    const long long picks = (long long)T * s.top_k;
    const long long routed_tiles = picks / bm + (picks < s.n_experts ? picks : s.n_experts) + 1;
    const long long shared_tiles = s.has_shared ? (T + bm - 1) / bm : 0;
    w.bm = bm;
    w.max_tiles = (int)(routed_tiles + shared_tiles);
    w.counts = o;  o = align_up(o + 4 * (size_t)M, 256);
    w.offsets = o; o = align_up(o + 4 * (size_t)(M + 1), 256);
    w.cursor = o;  o = align_up(o + 4 * (size_t)M, 256);
    w.ntiles = o;  o = align_up(o + 4, 256);
    w.tiles = o;   o = align_up(o + sizeof(Tile) * (size_t)w.max_tiles, 256);
    w.order = o;   o = align_up(o + 4 * (size_t)T * n_slots(s), 256);
    w.n_slices = (int)((picks + SLICE - 1) / SLICE);
    w.slices = o;  o = align_up(o + 4 * (size_t)w.n_slices * s.n_experts, 256);  // [n_slices][E] counts
    return w;
}

// Workspace layout for moe_experts_prefill: the dispatch (tiles of BM rows), then h.
struct PrefillWs {
    DispatchWs D;
    size_t h, total;
};

static PrefillWs prefill_ws_layout(const moe_shape& s, int T) {
    PrefillWs w;
    size_t o = 0;
    w.D = dispatch_ws_layout(s, T, prefill_tile_rows(T), o);
    w.h = o;
    o = align_up(o + 2 * (size_t)T * n_slots(s) * s.inter, 256);
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

// ---------------------------------------------------------------- set-up: dispatch
// One or two launches before the GEMMs. The picks p = t*k + s are cut into slices of
// SLICE consecutive picks, one workgroup each.
//   count (more than SELF_COUNT picks): each slice's per-expert counts (an LDS
//     histogram) go to slices[b][e].
//   scatter: every slice's workgroup reads the whole count matrix (n_slices x E), or
//     with at most SELF_COUNT picks counts them all itself, and derives the experts'
//     totals, their offsets in the expert-sorted order and its own base within each
//     expert (the picks of the earlier slices), then places its
//     picks in ascending pick order: wavefront w takes the slice's picks SLICE/4 w ..
//     SLICE/4 (w+1) - 1, 64 at a time, and ranks each among the lower lanes holding
//     the same id (one ballot per id bit) plus the wavefront's earlier picks of that
//     id (a per-wavefront count in LDS); after one barrier the counts of the lower
//     wavefronts are added. One more workgroup, after the slices', writes the
//     counts, the offsets, the shared expert's rows (it takes every token) and the
//     tile list: every full tile first (expert order), then the partial tiles with
//     the most row blocks first (expert order within a size), so the items that
//     start last are the cheapest.
// Everything the dispatch writes is a function of the ids alone. Picks with an
// id outside [0, E) are skipped and their y rows zeroed. A slice's picks are loaded
// before any is counted or placed.
constexpr int DT = 256, DPT = SLICE / DT;  // threads per workgroup, picks per thread
// Up to this many picks (1024 tokens at top-8) the scatter workgroups count the picks
// themselves and the count launch is skipped (one launch and its gap fewer).
constexpr int SELF_COUNT = 8192;

__global__ __launch_bounds__(DT) void prefill_count_kernel(const int32_t* __restrict__ ids, long long P, int E,
                                                           int32_t* __restrict__ slices) {
    __shared__ int cnt[1024];
    const int tid = threadIdx.x;
    for (int i = tid; i < E; i += DT) cnt[i] = 0;
    __syncthreads();
    const long long p0 = (long long)blockIdx.x * SLICE;
    int ev[DPT];
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
        const long long p = p0 + j * DT + tid;
        ev[j] = p < P ? ids[p] : -1;
    }
#pragma unroll
    for (int j = 0; j < DPT; ++j)
        if (ev[j] >= 0 && ev[j] < E) atomicAdd(&cnt[ev[j]], 1);
    __syncthreads();
    for (int i = tid; i < E; i += DT) slices[(size_t)blockIdx.x * E + i] = cnt[i];
}

// Lanes of this wavefront whose key equals this lane's (keys below 2^11), from one
// ballot per key bit; every lane must be active.
__device__ __forceinline__ uint64_t equal_key_lanes(uint32_t key) {
    uint64_t m = ~0ull;
#pragma unroll
    for (int b = 0; b < 11; ++b) {
        const uint64_t v = __ballot((key >> b) & 1u);
        m &= ((key >> b) & 1u) ? v : ~v;
    }
    return m;
}

template <int TBM>
__global__ __launch_bounds__(DT) void prefill_scatter_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, int has_shared, int H, int n_slices,
    const int32_t* __restrict__ slices, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ ntiles, Tile* __restrict__ tiles, int32_t* __restrict__ order, float* __restrict__ y) {
    __shared__ int cnt[1025];             // the experts' totals
    __shared__ int off[1026];             // their offsets in the order
    __shared__ int foff[1026];            // their full tiles' offsets in the tile list
    __shared__ int cur[1024];             // this slice's next position per expert
    __shared__ int wcnt[DT / 64][1024];   // picks per (wavefront, expert) among the current 256
    const int M = E + has_shared, S = k + has_shared;
    const int tid = threadIdx.x, b = blockIdx.x, wave = tid >> 6, lane = tid & 63;
    for (int i = tid; i < (DT / 64) * 1024; i += DT) (&wcnt[0][0])[i] = 0;
    const long long P = (long long)T * k, p0 = (long long)b * SLICE;
    // pick j of this thread: p0 + DPT * 64 * wave + 64 j + lane (a wavefront's picks
    // are consecutive)
    int ev[DPT];
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
        const long long p = p0 + DPT * 64 * wave + 64 * j + lane;
        ev[j] = p < P ? ids[p] : -1;
    }
    if (slices) {
        for (int e = tid; e < E; e += DT) {
            int tot = 0, base = 0;
#pragma unroll 8
            for (int s2 = 0; s2 < n_slices; ++s2) {
                const int c = slices[(size_t)s2 * E + e];
                base += s2 < b ? c : 0;
                tot += c;
            }
            cnt[e] = tot;
            cur[e] = base;
        }
    } else {
        // at most SELF_COUNT picks: the workgroup counts them all itself (the totals,
        // and the picks before its slice for its base), all loads issued first
        for (int e = tid; e < E; e += DT) {
            cnt[e] = 0;
            cur[e] = 0;
        }
        int ea[SELF_COUNT / DT];
#pragma unroll
        for (int j = 0; j < SELF_COUNT / DT; ++j) {
            const long long p = (long long)j * DT + tid;
            ea[j] = p < P ? ids[p] : -1;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < SELF_COUNT / DT; ++j) {
            const long long p = (long long)j * DT + tid;
            if (ea[j] >= 0 && ea[j] < E) {
                atomicAdd(&cnt[ea[j]], 1);
                if (p < p0) atomicAdd(&cur[ea[j]], 1);
            }
        }
    }
    __syncthreads();
    if (has_shared && tid == 0) cnt[E] = T;
    __syncthreads();
    if (tid < 64) {  // exclusive scans of the rows and the full tiles over the experts
        const int per = (M + 63) / 64;
        const int beg = tid * per, end = min(M, beg + per);
        int lc = 0, lt = 0;
        for (int i2 = beg; i2 < end; ++i2) {
            lc += cnt[i2];
            lt += cnt[i2] / TBM;
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
        for (int i2 = beg; i2 < end; ++i2) {
            off[i2] = rc;
            foff[i2] = rt;
            rc += cnt[i2];
            rt += cnt[i2] / TBM;
        }
        if (tid == 63) {
            off[M] = ic;
            foff[M] = it;
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += DT) cur[e] += off[e];
    if (b == n_slices) {  // the extra workgroup: counts, offsets, shared rows, tile list
        for (int e = tid; e < M; e += DT) {
            counts[e] = cnt[e];
            offsets[e] = off[e];
            const int nfull = cnt[e] / TBM;
            for (int q = 0; q < nfull; ++q) {
                Tile tl;
                tl.expert = e;
                tl.row0 = off[e] + q * TBM;
                tl.nrows = TBM;
                tl.pad = 0;
                tiles[foff[e] + q] = tl;
            }
        }
        if (has_shared)
            for (int t = tid; t < T; t += DT) order[off[E] + t] = t * S + k;
        if (tid < 64) {
            // partial tiles by size class q = TBM/16 - (row blocks), in expert order within a
            // class: count the classes, then place each tile at its class base plus its
            // rank among the lower experts of the class
            constexpr int NCL = TBM / 16;
            int tot[NCL], run[NCL];
#pragma unroll
            for (int q = 0; q < NCL; ++q) tot[q] = 0;
            for (int e0 = 0; e0 < M; e0 += 64) {
                const int e = e0 + tid, rem = e < M ? cnt[e] % TBM : 0;
                const int cls = rem ? NCL - (rem + 15) / 16 : -1;
#pragma unroll
                for (int q = 0; q < NCL; ++q) tot[q] += __popcll(__ballot(cls == q));
            }
            int acc = foff[M];
#pragma unroll
            for (int q = 0; q < NCL; ++q) {
                run[q] = acc;
                acc += tot[q];
            }
            if (tid == 0) {
                *ntiles = acc;
                offsets[M] = off[M];
            }
            const uint64_t below = (1ull << tid) - 1ull;
            for (int e0 = 0; e0 < M; e0 += 64) {
                const int e = e0 + tid, rem = e < M ? cnt[e] % TBM : 0;
                const int cls = rem ? NCL - (rem + 15) / 16 : -1;
#pragma unroll
                for (int q = 0; q < NCL; ++q) {
                    const uint64_t m = __ballot(cls == q);
                    if (cls == q) {
                        Tile tl;
                        tl.expert = e;
                        tl.row0 = off[e] + (cnt[e] / TBM) * TBM;
                        tl.nrows = rem;
                        tl.pad = 0;
                        tiles[run[q] + __popcll(m & below)] = tl;
                    }
                    run[q] += __popcll(m);
                }
            }
        }
        return;
    }
    __syncthreads();
    // pass 1, per wavefront (LDS accesses of one wavefront take effect in order): the
    // rank of each pick among the wavefront's earlier picks of the same expert
    const uint64_t below = (1ull << lane) - 1ull;
    int lpos[DPT];
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
        const long long p = p0 + DPT * 64 * wave + 64 * j + lane;
        const int e = ev[j];
        const bool ok = p < P && e >= 0 && e < E;
        const uint64_t peers = equal_key_lanes(ok ? (uint32_t)e : 2047u);
        const int rank = __popcll(peers & below);
        lpos[j] = ok ? wcnt[wave][e] + rank : 0;
        if (ok && rank == 0) wcnt[wave][e] += __popcll(peers);
    }
    __syncthreads();
    // pass 2: add the slice's base and the lower wavefronts' counts
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
        const long long p = p0 + DPT * 64 * wave + 64 * j + lane;
        const int e = ev[j];
        if (p >= P) continue;
        if (e >= 0 && e < E) {
            int pos = cur[e] + lpos[j];
            for (int w2 = 0; w2 < wave; ++w2) pos += wcnt[w2][e];
            order[pos] = (int)(p / k) * S + (int)(p % k);
        } else {
            float* yr = y + ((size_t)(p / k) * S + (size_t)(p % k)) * H;
            for (int n = 0; n < H; ++n) yr[n] = 0.f;
        }
    }
}


// ---------------------------------------------------------------- grouped GEMM
// A workgroup multiplies one tile (up to 128 expert-sorted rows) by a block of
// NBR = 256 weight rows of the tile's expert over the whole K: gate/up takes 128
// gate rows and the matching 128 up rows, down takes 256 rows. Wavefront w owns
// the weight rows cs*64 + 16w .. +16 (cs < 4) for every tile row. K walks in
// chunks of one quantisation group (KC = 64); per chunk, direct global-to-LDS
// loads stage
//   A: the tile's rows x 64 bf16 (128 B per row),
//   B: the 256 int4 weight rows x 32 B,
//   sb: the 256 rows' (scale, bias) words of the group,
// into a ring of LDS stages that runs one chunk fewer than it has stages ahead of
// the one being multiplied. A stage holds only the A rows the tile loads, so
// tiles of up to 32 rows get five stages, 64 rows four, 128 rows three. Two
// workgroups share a CU, so one's prologue and epilogue overlap the other's main
// loop.
constexpr int KC = 64;
constexpr int NBR = 256;
constexpr int B_BYTES = NBR * KC / 2, SB_BYTES = NBR * 4;
constexpr int RING = 3 * (BM * KC * 2 + B_BYTES + SB_BYTES);  // 75 KiB: three stages of a full tile
// Up to 1024 tokens most tiles hold a few row blocks and a workgroup's time goes to
// streaming its weight rows, bound by the loads in flight: the kernel's second
// instance takes at most 64 rows per pass (the dispatch cuts tiles of 64 rows there,
// so it makes one pass; a tile of more rows would take two passes over the
// weights), with at most 168 VGPRs and a 51 KiB ring, so three workgroups share a
// CU (at 512 tokens 141.6 -> 132.4 us for both GEMMs on 128-row tiles). A row's
// arithmetic is the same in both instances and in every tile, and so are its
// results, bit for bit.
constexpr int RING3 = 3 * (64 * KC * 2 + B_BYTES + SB_BYTES);  // 51 KiB

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
    int T;
    int km;                     // weight row length / activation length: 1 (4-bit experts) or 2 (8-bit)
};



// GATEUP: weight rows 0..127 are gate rows cb*128 .., rows 128..255 the matching up
// rows; the epilogue writes h = bf16(silu(gate) * up). Else (down): weight rows are
// down rows cb*256 ..; the epilogue writes y[t][s][n] for the row's pick p = order[row].
// WPC: workgroups per CU (2: one pass of up to 128 rows; 3: passes of 64 rows).
template <bool GATEUP, int WPC>
__global__ __launch_bounds__(256, WPC) void expert_gemm_kernel(GemmArgs a) {
    constexpr int NCS = NBR / 64;  // 16-column sets per wavefront
    constexpr int HALF = NBR / 2;  // gate/up: gate rows 0 .. HALF-1, up rows HALF .. NBR-1
    static_assert(WPC == 2 || WPC == 3, "instances");
    constexpr int MAXNM = WPC == 3 ? 4 : 8;          // row blocks of 16 per pass
    constexpr int PR = 16 * MAXNM;                   // rows per pass
    constexpr int RINGW = WPC == 3 ? RING3 : RING;   // the launch's dynamic LDS
    extern __shared__ __attribute__((aligned(16))) uint8_t ring[];  // ring of stages, each (A | B | sb)
    __shared__ uint32_t arow_lds[BM];  // byte offset of each tile row in its source, ~0 beyond the tile
    __shared__ int32_t pick_lds[BM];   // down: pick p = order[row] of each tile row (its y row)
    const int H = a.H, I = a.I, S = a.S;
    // K: activations per row; the weight rows hold K * km int4 codes (8-bit rows as
    // two planes), whose chunk c meets activation chunk c mod K/64
    const int K = GATEUP ? H : I, Kw = K * a.km, GX = K / 64;
    const int nblk = GATEUP ? (I + HALF - 1) / HALF : (H + NBR - 1) / NBR;
    int ti, cb;
    if (!xcd_item(*a.ntiles, nblk, ti, cb)) return;
    const Tile tl = a.tiles[ti];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lg = lane >> 4, lc = lane & 15;
    const int col0 = GATEUP ? cb * HALF : cb * NBR;

    // down: the tile row's pick is needed only by the epilogue, so its load stays in
    // flight through the K loop and the value reaches pick_lds after it (the set-up
    // barrier then waits for no global load: 1 us less per down item)
    int pick_v = 0;
    if (tid < BM) {
        uint32_t off = 0xFFFFFFFFu;
        int src = 0;
        if (tid < tl.nrows) {
            if constexpr (GATEUP) src = a.order[tl.row0 + tid] / S;
            else src = tl.row0 + tid;
            off = (uint32_t)src * (uint32_t)(2 * K);
        }
        arow_lds[tid] = off;
        if constexpr (!GATEUP) pick_v = tid < tl.nrows ? a.order[tl.row0 + tid] : 0;
    }
    __syncthreads();
    const uint8_t* asrc = reinterpret_cast<const uint8_t*>(GATEUP ? a.x : a.hbuf);
    const uint8_t* ebase = a.packed + (size_t)tl.expert * a.L.stride;
    auto brow_ok = [&](int r) -> bool { return GATEUP ? col0 + r % HALF < I : col0 + r < H; };
    // The workgroup's 256 weight rows are 64 four-row blocks of the packed layout
    // (gate/up: block col0/2 + jb holds gate and up rows col0 + 2jb, col0 + 2jb + 1;
    // down: block col0/4 + jb holds rows col0 + 4jb .. +3). Weight row br (gate
    // column br, up column br - 128, or down row br) sits in block jb at slot:
    auto brow_block = [&](int br, int& jb, int& slot) {
        if constexpr (GATEUP) {
            const int i = br % HALF;
            jb = i >> 1;
            slot = (br >= HALF ? 2 : 0) + (i & 1);
        } else {
            jb = br >> 2;
            slot = br & 3;
        }
    };
    // The workgroup's blocks blk0 .. blk0 + nbs - 1 are one set of the prefill layout
    // (moe_pack_experts_prefill): group c of the set's blocks is nbs consecutive
    // 128-byte lines (block jb at 128 jb) and nbs consecutive 16-byte sb units, so a
    // chunk reads two contiguous runs. Blocks beyond the matrix read the set's first.
    const int nblk_mat = GATEUP ? I / 2 : H / 4;
    const int blk0 = GATEUP ? col0 / 2 : col0 / 4;
    const int nbs = min(PF_SET, nblk_mat - blk0);
    auto lblock = [&](int jb) -> int { return jb < nbs ? jb : 0; };
    const size_t q_region = GATEUP ? a.L.gu_q : a.L.down_q, sb_region = GATEUP ? a.L.gu_sb : a.L.down_sb;
    const int G = Kw / 64;

    // ---- ring layout within a stage:
    //   A: the loaded rows x 128 B, the 16-byte piece p of row r at position p ^ (r & 7);
    //   B: 64 blocks x 128 B (the group's line of each block: slot s, 16-byte half h
    //      is piece 2s + h), piece p of block jb at position p ^ bsw(jb);
    //   sb: 64 blocks x 4 words.
    // The XOR positions spread the fragment reads of neighbouring lanes over the
    // banks. Rows beyond the tile or the matrix load a valid row instead, so every
    // lane issues every load, each wavefront has exactly LPC loads per chunk in
    // flight, and the wait for a chunk is an exact vector-memory count. Per-lane
    // offsets are fixed for the tile; the chunk advances the uniform base by one
    // group of the set: nbs lines (q) or nbs 16-byte units (sb).
    auto bsw = [](int jb) -> int { return ((jb >> 1) & 3) << 1; };  // even: keeps a slot's two halves adjacent
    const uint32_t ring_lds = lds_addr(ring);
    uint32_t b_off[2];  // B: instruction j = 2 wave + i covers blocks 8j .. 8j+7
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int jb = 8 * (2 * wave + i) + (lane >> 3);
        const int piece = (lane & 7) ^ bsw(jb);
        b_off[i] = (uint32_t)(q_region + (size_t)blk0 * G * 128 + lblock(jb) * 128 + 16 * piece);
    }
    // sb: one instruction per wavefront, blocks 16 wave .. +16, four words each
    const uint32_t sb_off =
        (uint32_t)(sb_region + (size_t)blk0 * G * 16 + lblock(16 * wave + (lane >> 2)) * 16 + 4 * (lane & 3));

    f32x4_t acc[MAXNM][NCS];
    // passes over the tile's rows; a tile fits one pass of the two-per-CU instance
    const int pass_end = WPC == 2 ? 1 : tl.nrows;
    for (int r0 = 0; r0 < pass_end; r0 += PR) {
    const int n_ms = min(MAXNM, (tl.nrows - r0 + 15) >> 4);
    if (r0 > 0) __syncthreads();  // the previous pass's epilogue has read the ring
#pragma unroll
    for (int m = 0; m < MAXNM; ++m)
#pragma unroll
        for (int cs = 0; cs < NCS; ++cs) acc[m][cs] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // The K loop is instantiated for 1, 2, 4 and 8 row blocks of 16 (the tile's count
    // rounded up), so its body is straight-line code the compiler can interleave.
    auto kloop = [&](auto nm_tag) __attribute__((always_inline)) {
        constexpr int NM = decltype(nm_tag)::value;
        constexpr int NA = NM >= 2 ? NM / 2 : 1;  // A instructions (8 rows each) per wavefront
        constexpr int LPC = NA + 3;               // loads per wavefront and chunk
        constexpr int SA = 4 * NA * 1024;         // A bytes per stage (32 NA rows)
        constexpr int STAGE = SA + B_BYTES + SB_BYTES;
        constexpr int NS = RINGW / STAGE;         // stages: 5, 4 or 3 (three-per-CU instance: 3)
        static_assert(NS >= 3 && NS * STAGE <= RINGW && LPC * (NS - 2) < 64, "ring");
        const uint32_t arow0 = arow_lds[0];       // row 0 is always inside the tile
        uint32_t a_off[NA];
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int row = 8 * (NA * wave + i) + (lane >> 3);
            const uint32_t off = arow_lds[r0 + row];
            a_off[i] = (off == 0xFFFFFFFFu ? arow0 : off) + 16 * ((lane & 7) ^ (row & 7));
        }
        auto issue = [&](int c) __attribute__((always_inline)) {
            const uint32_t st = ring_lds + (uint32_t)((c % NS) * STAGE);
            const uint8_t* ab = asrc + (size_t)(c < GX ? c : c - GX) * (KC * 2);
#pragma unroll
            for (int i = 0; i < NA; ++i) lds_dma16(ab, a_off[i], st + (NA * wave + i) * 1024);
            const uint8_t* bb = ebase + (size_t)c * nbs * 128;
#pragma unroll
            for (int i = 0; i < 2; ++i) lds_dma16(bb, b_off[i], st + SA + (2 * wave + i) * 1024);
            lds_dma4(ebase + (size_t)c * nbs * 16, sb_off, st + SA + B_BYTES + wave * 256);
        };
        auto compute = [&](int c) __attribute__((always_inline)) {
            const uint8_t* st = ring + (size_t)(c % NS) * STAGE;
            const uint32_t* sb_st = reinterpret_cast<const uint32_t*>(st + SA + B_BYTES);
            uint4 b0[NCS], b1[NCS];
            float s16[NCS], cb16[NCS];
#pragma unroll
            for (int cs = 0; cs < NCS; ++cs) {
                int jb, slot;
                brow_block(cs * 64 + 16 * wave + lc, jb, slot);
                const uint8_t* bp = st + SA + jb * 128 + 16 * ((2 * slot) ^ bsw(jb)) + 4 * lg;
                b0[cs] = bfrag(*reinterpret_cast<const uint32_t*>(bp));
                b1[cs] = bfrag(*reinterpret_cast<const uint32_t*>(bp + 16));
                const uint32_t w = sb_st[4 * jb + slot];
                s16[cs] = 16.f * bf16_to_f32(w & 0xFFFFu);
                cb16[cs] = brow_ok(cs * 64 + 16 * wave + lc) ? bf16_to_f32(w >> 16) - s16[cs] : 0.f;
            }
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const uint8_t* ar = st + (16 * m + lc) * 128;
                const uint4 a0 = *reinterpret_cast<const uint4*>(ar + 16 * (lg ^ (lc & 7)));
                const uint4 a1 = *reinterpret_cast<const uint4*>(ar + 16 * ((4 + lg) ^ (lc & 7)));
                // the chunk's row sums X (every column alike)
                const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
                f32x4_t xs = mfma16x16x32(a0, ones, f32x4_t{0.f, 0.f, 0.f, 0.f});
                xs = mfma16x16x32(a1, ones, xs);
#pragma unroll
                for (int cs = 0; cs < NCS; ++cs) {
                    f32x4_t p = mfma16x16x32(a0, b0[cs], f32x4_t{0.f, 0.f, 0.f, 0.f});
                    p = mfma16x16x32(a1, b1[cs], p);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[m][cs][r] = fmaf(xs[r], cb16[cs], fmaf(s16[cs], p[r], acc[m][cs][r]));
                }
            }
        };
        const int NC = Kw / KC;
        for (int c = 0; c < NS - 1 && c < NC; ++c) issue(c);
        for (int c = 0; c < NC; ++c) {
            // this wavefront's loads of chunk c are done once only the later chunks'
            // (at most NS - 2 of them) are left
            wait_chunks<LPC, NS - 2>(NC - 1 - c);
            // every wavefront's loads of chunk c are in LDS, and every wavefront has
            // finished chunk c-1, whose stage the next loads refill
            lds_barrier();
            if (c + NS - 1 < NC) issue(c + NS - 1);
            compute(c);
        }
    };
    if (n_ms <= 1) kloop(std::integral_constant<int, 1>{});
    else if (n_ms <= 2) kloop(std::integral_constant<int, 2>{});
    else if (MAXNM == 4 || n_ms <= 4) kloop(std::integral_constant<int, 4>{});
    else kloop(std::integral_constant<int, MAXNM>{});

    // ---- epilogue: the ring's memory is free once every wavefront is past its last chunk
    if constexpr (!GATEUP) {
        if (tid < BM) pick_lds[tid] = pick_v;
    }
    __syncthreads();
    if constexpr (GATEUP) {
        // h = bf16(silu(gate) * up) for this block's 128 intermediate columns i =
        // col0 + c, c = 64 hs + 16 wave + lc (gate set hs, up set 2 + hs), staged as a
        // bf16 tile in LDS (rows beyond the tile hold zeros), then stored with 16-byte
        // row pieces.
        constexpr int HS = 128 + 8;  // tile row stride (bf16)
        uint16_t* hl = reinterpret_cast<uint16_t*>(ring);
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            const int c = 64 * hs + 16 * wave + lc;
#pragma unroll
            for (int m = 0; m < MAXNM; ++m) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * m + 4 * lg + r;  // within the pass
                    const float gv = acc[m][hs][r], uv = acc[m][2 + hs][r];
                    // silu(g) = g / (1 + e^-g), e^-g = 2^(-g log2 e)
                    const float sg = gv * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-gv * 1.44269504088896341f));
                    const __bf16 hb = (__bf16)(sg * uv);
                    hl[row * HS + c] = r0 + row < tl.nrows ? __builtin_bit_cast(uint16_t, hb) : (uint16_t)0;
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < MAXNM; ++it) {
            const int row = 16 * it + (tid >> 4), pc = tid & 15;
            if (r0 + row < tl.nrows && col0 + 8 * pc < I)
                *reinterpret_cast<uint4*>(a.hbuf + (size_t)(tl.row0 + r0 + row) * I + col0 + 8 * pc) =
                    *reinterpret_cast<const uint4*>(hl + row * HS + 8 * pc);
        }
    } else {
        // y[order[row]][col0 + n], n < 256, staged SR rows at a time as an fp32 tile in
        // LDS and stored with 16-byte row pieces. The stores are non-temporal: y is read
        // once, by the combine, and would otherwise evict weight lines and activation
        // tiles that later workgroups read again.
        constexpr int YS = NBR + 4;  // tile row stride (floats)
        constexpr int SR = WPC == 3 ? 32 : 64;  // rows per staging step (the ring holds SR * YS floats)
        static_assert(SR * YS * 4 <= RINGW && PR * (128 + 8) * 2 <= RINGW, "epilogue staging fits the ring");
        float* yl = reinterpret_cast<float*>(ring);
#pragma unroll
        for (int q = 0; q < PR / SR; ++q) {
            if (r0 + SR * q < tl.nrows) {
                if (q) __syncthreads();
#pragma unroll
                for (int mm = 0; mm < SR / 16; ++mm) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int rl = 16 * mm + 4 * lg + r;
#pragma unroll
                        for (int cs = 0; cs < NCS; ++cs)
                            yl[rl * YS + cs * 64 + 16 * wave + lc] = acc[(SR / 16) * q + mm][cs][r];
                    }
                }
                __syncthreads();
#pragma unroll 4
                for (int it = 0; it < SR / 4; ++it) {
                    const int rl = 4 * it + (tid >> 6), row = r0 + SR * q + rl, pc = tid & 63;
                    if (row < tl.nrows && col0 + 4 * pc < H)
                        __builtin_nontemporal_store(*reinterpret_cast<const f32x4_t*>(yl + rl * YS + 4 * pc),
                                                    reinterpret_cast<f32x4_t*>(a.y + (size_t)pick_lds[row] * H + col0 + 4 * pc));
                }
            }
        }
    }
    }  // passes
}

static_assert(BM == 128, "tile rows");

moe_status launch_prefill_dispatch(const moe_shape& sh, int T, const int32_t* ids, const DispatchWs& D, char* w,
                                   float* y, hipStream_t hs) {
    const long long P = (long long)T * sh.top_k;
    int32_t* slices = nullptr;
    if (P > SELF_COUNT) {
        slices = (int32_t*)(w + D.slices);
        hipLaunchKernelGGL(prefill_count_kernel, dim3((unsigned)D.n_slices), dim3(DT), 0, hs, ids, P, sh.n_experts,
                           slices);
        moe_status st = check_launch("prefill_count_kernel");
        if (st != MOE_OK) return st;
    }
    auto scatter = D.bm == 256 ? prefill_scatter_kernel<256>
                   : D.bm == 64 ? prefill_scatter_kernel<64> : prefill_scatter_kernel<128>;
    hipLaunchKernelGGL(scatter, dim3((unsigned)D.n_slices + 1), dim3(DT), 0, hs, ids, T, sh.top_k, sh.n_experts,
                       sh.has_shared, sh.hidden, D.n_slices, slices, (int32_t*)(w + D.counts),
                       (int32_t*)(w + D.offsets), (int32_t*)(w + D.ntiles), (Tile*)(w + D.tiles),
                       (int32_t*)(w + D.order), y);
    return check_launch("prefill_scatter_kernel");
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_pack_experts_prefill(const moe_shape* shape, const void* experts_packed,
                                               void* experts_prefill, size_t bytes, void* stream) {
    clear_error();
    moe_status st = validate_shape(shape);
    if (st != MOE_OK) return st;
    if (!experts_packed || !experts_prefill || !aligned16(experts_packed) || !aligned16(experts_prefill))
        return fail(MOE_ERR_INVALID_ARG, "NULL or unaligned pointer");
    const ExpertLayout L = expert_layout(*shape);
    const int M = n_mats(*shape);
    const size_t total = L.stride * (size_t)M;
    if (bytes < total) return fail(MOE_ERR_WORKSPACE, "prefill expert buffer too small (%zu < %zu)", bytes, total);
    const char* a0 = (const char*)experts_packed;
    const char* b0 = (const char*)experts_prefill;
    if (a0 < b0 + total && b0 < a0 + total) return fail(MOE_ERR_INVALID_ARG, "the two expert buffers overlap");
    const int Hw = shape->hidden * kmul(*shape), Iw = shape->inter * kmul(*shape);
    const int nblk_gu = shape->inter / 2, G_gu = Hw / 64, nblk_dn = shape->hidden / 4, G_dn = Iw / 64;
    const long long units = (long long)nblk_gu * G_gu * 9 + (long long)nblk_dn * G_dn * 9;
    hipLaunchKernelGGL(relayout_prefill_kernel, dim3((unsigned)((units + 255) / 256), (unsigned)M), dim3(256), 0,
                       (hipStream_t)stream, (const uint8_t*)experts_packed, (uint8_t*)experts_prefill, L, nblk_gu,
                       G_gu, nblk_dn, G_dn);
    return check_launch("relayout_prefill_kernel");
}

extern "C" size_t moe_prefill_workspace_bytes(const moe_shape* shape, int32_t T) {
    if (validate_shape(shape) != MOE_OK || T < 1) return 0;
    return prefill_ws_layout(*shape, T).total;
}

extern "C" moe_status moe_prefill_dispatch_layout(const moe_shape* shape, int32_t T, moe_prefill_dispatch_view* v) {
    clear_error();
    moe_status st = validate_shape(shape);
    if (st != MOE_OK) return st;
    if (T < 1 || !v) return fail(MOE_ERR_INVALID_ARG, "T = %d or NULL view", T);
    const DispatchWs D = prefill_ws_layout(*shape, T).D;
    v->counts = D.counts;
    v->offsets = D.offsets;
    v->ntiles = D.ntiles;
    v->tiles = D.tiles;
    v->order = D.order;
    v->max_tiles = D.max_tiles;
    v->tile_rows = D.bm;
    return MOE_OK;
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

extern "C" moe_status moe_experts_prefill(const moe_shape* shape, const void* experts_prefill, const uint16_t* x,
                                          int32_t T, const int32_t* ids, void* ws, size_t ws_bytes, float* y,
                                          void* stream) {
    clear_error();
    moe_status st = validate_shape(shape);
    if (st != MOE_OK) return st;
    if (T < 1) return fail(MOE_ERR_INVALID_ARG, "T = %d, need T >= 1", T);
    if (!experts_prefill || !x || !ids || !ws || !y || !aligned16(experts_prefill) || !aligned16(x) ||
        !aligned16(ws) || !aligned16(y))
        return fail(MOE_ERR_INVALID_ARG, "NULL or unaligned pointer");
    const moe_shape& sh = *shape;
    const PrefillWs W = prefill_ws_layout(sh, T);
    if (ws_bytes < W.total) return fail(MOE_ERR_WORKSPACE, "prefill workspace too small (%zu < %zu)", ws_bytes, W.total);
    const ExpertLayout L = expert_layout(sh);
    const int S = n_slots(sh), H = sh.hidden, I = sh.inter;
    // the GEMMs address activation rows and expert segments with 32-bit byte offsets
    if ((size_t)T * H * 2 > 0xFFFF0000u || (size_t)T * S * I * 2 > 0xFFFF0000u || L.stride > 0xFFFF0000u)
        return fail(MOE_ERR_UNSUPPORTED, "T = %d too large for this shape (32-bit row offsets)", T);
    int max_lds = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
        return fail(MOE_ERR_HIP, "cannot query the device's LDS size");
    // up to 1024 tokens: the three-workgroups-per-CU instance on 64-row tiles
    const bool three = W.D.bm == BM3;
    const int ring = three ? RING3 : RING;
    if (max_lds < ring + 2048)
        return fail(MOE_ERR_UNSUPPORTED, "the grouped GEMM needs %d bytes of LDS per workgroup, the device has %d",
                    ring + 2048, max_lds);
    hipStream_t hs = (hipStream_t)stream;
    char* w = (char*)ws;
    int32_t* ntiles = (int32_t*)(w + W.D.ntiles);
    Tile* tiles = (Tile*)(w + W.D.tiles);
    int32_t* order = (int32_t*)(w + W.D.order);
    uint16_t* hbuf = (uint16_t*)(w + W.h);
    if ((st = launch_prefill_dispatch(sh, T, ids, W.D, w, y, hs)) != MOE_OK) return st;
    GemmArgs ga;
    ga.packed = (const uint8_t*)experts_prefill;
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
    ga.km = kmul(sh);
    const dim3 gu_grid(xcd_grid(W.D.max_tiles, (I + NBR / 2 - 1) / (NBR / 2))), dn_grid(xcd_grid(W.D.max_tiles, (H + NBR - 1) / NBR));
    if (three) hipLaunchKernelGGL((expert_gemm_kernel<true, 3>), gu_grid, dim3(256), ring, hs, ga);
    else hipLaunchKernelGGL((expert_gemm_kernel<true, 2>), gu_grid, dim3(256), ring, hs, ga);
    if ((st = check_launch("expert_gemm_kernel<gate/up>")) != MOE_OK) return st;
    if (three) hipLaunchKernelGGL((expert_gemm_kernel<false, 3>), dn_grid, dim3(256), ring, hs, ga);
    else hipLaunchKernelGGL((expert_gemm_kernel<false, 2>), dn_grid, dim3(256), ring, hs, ga);
    return check_launch("expert_gemm_kernel<down>");
}

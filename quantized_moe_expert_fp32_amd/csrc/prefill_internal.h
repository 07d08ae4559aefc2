// Shared by the grouped expert GEMMs of the prefill path (bf16 MFMA on exact int4
// operands, prefill.hip) and of the FP8 route (prefill_fp8.hip): the tile list,
// the dispatch that builds it, direct global-to-LDS loads and the XCD-aware
// mapping of (tile, column block) items to workgroups.
#pragma once

#include "moe_internal.h"

namespace moe {

// A tile: rows row0 .. row0 + nrows - 1 of the expert-sorted order, all of one expert.
struct Tile {
    int32_t expert, row0, nrows, pad;
};

// Dispatch arrays inside a workspace (byte offsets), for tiles of at most bm rows.
struct DispatchWs {
    size_t counts, offsets, cursor, ntiles, tiles, order, slices;
    int max_tiles;
    int n_slices;  // pick slices of the dispatch
    int bm;        // rows per tile: 128 or 256
};

// Lays the dispatch arrays out from byte offset o (advanced past them).
DispatchWs dispatch_ws_layout(const moe_shape& s, int T, int bm, size_t& o);

// The two dispatch launches (count, scatter) into the arrays of D inside ws: the
// counts, offsets, expert-sorted order and tile list of the ids [T][k]; y rows of
// picks with an id outside [0, E) are zeroed. Every array is a function of the ids.
moe_status launch_prefill_dispatch(const moe_shape& s, int T, const int32_t* ids, const DispatchWs& D, char* ws,
                                   float* y, hipStream_t st);

// Direct global-to-LDS loads from base + off (base wavefront-uniform, off per lane):
// lane l's 16 (or 4) bytes land at LDS byte address lds + 16 l (4 l); lds is
// wavefront-uniform and goes in M0, written at least one wait state before the
// load (the s_nop). Written as inline asm so the compiler does not treat them as
// LDS stores (it would otherwise wait for every outstanding one before the first
// LDS read); completion is awaited explicitly with wait_vmcnt, and the memory
// clobber keeps LDS reads behind the barrier that follows that wait.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void lds_dma4(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Workgroup barrier that also keeps the compiler from moving memory accesses
// across it. This wavefront's LDS reads are complete before it (lgkmcnt 0), so a
// stage every wavefront has passed the barrier after reading may be refilled; the
// waits for outstanding global loads are explicit at the call sites.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited for
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt with only the vector-memory count (expcnt and lgkmcnt left at their
// maximum, i.e. not waited for); N < 64.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most min(later, L) chunks of LPC loads each are outstanding.
template <int LPC, int L>
__device__ __forceinline__ void wait_chunks(int later) {
    if constexpr (L == 0) {
        wait_vmcnt<0>();
    } else {
        if (later >= L) wait_vmcnt<L * LPC>();
        else wait_chunks<LPC, L - 1>(later);
    }
}

// ---------------------------------------------------------------- XCD-aware item mapping
// The GEMM grids are one-dimensional over (tile, column block) items. Workgroups
// are handed to the 8 XCDs round-robin by linear id, and each XCD has its own L2.
// Block b runs on XCD x = b % 8 as that XCD's j-th block, j = b / 8. Tiles are
// dealt to the XCDs in runs of XCD_RUN consecutive tiles, and an XCD takes its
// tiles in order, all column blocks of a tile in a row: the workgroups that share
// a tile's activations share one L2, and a tile list sorted by cost stays balanced
// across the XCDs. Runs of one tile measured best on the 512-token and skewed
// 4096-token workloads: longer runs keep an expert's consecutive tiles in one L2
// but put the few heavy tiles at the head of the list on one XCD. Blocks beyond
// the live tiles return.
constexpr int N_XCD = 8, XCD_RUN = 1;

__device__ __forceinline__ bool xcd_item(int ntiles, int nb, int& tile, int& cb) {
    const int x = (int)blockIdx.x % N_XCD, j = (int)blockIdx.x / N_XCD;
    const int lt = j / nb;  // this XCD's lt-th tile
    tile = (lt / XCD_RUN) * (N_XCD * XCD_RUN) + x * XCD_RUN + lt % XCD_RUN;
    cb = j % nb;
    return tile < ntiles;
}

inline unsigned xcd_grid(int max_tiles, int nb) {
    const int runs = (max_tiles + N_XCD * XCD_RUN - 1) / (N_XCD * XCD_RUN);
    return (unsigned)(runs * XCD_RUN * N_XCD * nb);
}

}  // namespace moe

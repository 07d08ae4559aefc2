// C-ABI plumbing: status strings, per-thread last error, shape validation, packing.
#include <stdarg.h>
#include <stdio.h>

#include "moe_internal.h"

namespace moe {

static thread_local char g_last_error[512] = "";

moe_status fail(moe_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

void clear_error() { g_last_error[0] = 0; }

moe_status check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return MOE_OK;
}

static bool pow2_in(int32_t v, int32_t lo, int32_t hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

moe_status validate_shape(const moe_shape* sh) {
    if (!sh) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
    if (sh->bits != 4 && sh->bits != 8)
        return fail(MOE_ERR_UNSUPPORTED, "expert bit width %d is not served (4-bit or 8-bit only)", sh->bits);
    if (sh->group != 64) return fail(MOE_ERR_UNSUPPORTED, "group %d is not served (64 only)", sh->group);
    if (sh->router_fmt != MOE_ROUTER_F32 && sh->router_fmt != MOE_ROUTER_AFFINE8)
        return fail(MOE_ERR_UNSUPPORTED, "router format %d is not served", sh->router_fmt);
    if (!pow2_in(sh->hidden, 64, 8192))
        return fail(MOE_ERR_UNSUPPORTED, "hidden %d: need a power of two in [64, 8192]", sh->hidden);
    if (!pow2_in(sh->inter, 64, 2048))
        return fail(MOE_ERR_UNSUPPORTED, "inter %d: need a power of two in [64, 2048]", sh->inter);
    if (sh->n_experts < 1 || sh->n_experts > 1024)
        return fail(MOE_ERR_INVALID_ARG, "n_experts %d out of [1, 1024]", sh->n_experts);
    if (sh->has_shared != 0 && sh->has_shared != 1)
        return fail(MOE_ERR_INVALID_ARG, "has_shared must be 0 or 1");
    if (sh->top_k < 1 || sh->top_k > 16 || sh->top_k > sh->n_experts)
        return fail(MOE_ERR_INVALID_ARG, "top_k %d out of [1, min(n_experts, 16)]", sh->top_k);
    if (sh->bits == 8 && (sh->hidden > 4096 || sh->inter > 1024))
        return fail(MOE_ERR_UNSUPPORTED, "8-bit experts: hidden <= 4096 and inter <= 1024 (rows of at most 8192 "
                    "and 2048 int4 codes)");
    return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" int32_t moe_abi_version(void) { return 1; }

extern "C" const char* moe_status_str(int32_t st) {
    switch (st) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape or format";
        case MOE_ERR_WORKSPACE: return "buffer too small";
        case MOE_ERR_HIP: return "HIP runtime error";
        case MOE_ERR_TIMEOUT: return "a bounded in-kernel wait timed out";
        default: return "unknown status";
    }
}

extern "C" const char* moe_last_error(void) { return g_last_error; }

extern "C" moe_status moe_shape_check(const moe_shape* shape) { return validate_shape(shape); }

// ------------------------------------------------------------------ packing

extern "C" size_t moe_experts_packed_bytes(const moe_shape* sh) {
    if (validate_shape(sh) != MOE_OK) return 0;
    return expert_layout(*sh).stride * (size_t)n_mats(*sh);
}

extern "C" size_t moe_router_packed_bytes(const moe_shape* sh) {
    if (validate_shape(sh) != MOE_OK) return 0;
    const size_t R = (size_t)router_rows(*sh), H = (size_t)sh->hidden;
    if (sh->router_fmt == MOE_ROUTER_F32) return R * H * 4;
    return R * H + R * (H / 64) * 4;
}

// Copies n16 16-byte units per expert from src (stride src_stride bytes) to dst.
// Four low (or high) nibbles of a dword's bytes -> one 16-bit value, byte b's
// nibble at bits 4b.
__device__ __forceinline__ uint32_t gather_nibbles(uint32_t v) {
    v &= 0x0F0F0F0Fu;
    v = (v | (v >> 4)) & 0x00FF00FFu;
    return (v | (v >> 8)) & 0x0000FFFFu;
}

// Canonical int4 dword (byte b = k_{2b} | k_{2b+1} << 4) -> packed order: k0, k2, k4,
// k6 in the low and k1, k3, k5, k7 in the high 16 bits.
__device__ __forceinline__ uint32_t pack_q_dword(uint32_t c) {
    return gather_nibbles(c) | (gather_nibbles(c >> 4) << 16);
}

// The high (hi = true) or low nibbles of the 4 bytes of two dwords as one dword of
// canonical int4 codes: byte b of a gives codes 2b' ... (a's four nibbles in the low
// 16 bits, b's in the high 16 bits, element order kept).
__device__ __forceinline__ uint32_t nibbles_of_bytes(uint32_t a, uint32_t b, bool hi) {
    if (hi) {
        a >>= 4;
        b >>= 4;
    }
    auto half = [](uint32_t d) -> uint32_t {
        return (d & 0xFu) | ((d >> 4) & 0xF0u) | ((d >> 8) & 0xF00u) | ((d >> 12) & 0xF000u);
    };
    return half(a) | (half(b) << 16);
}

// One canonical int4 matrix [N][K/2] per expert into the blocked layout (see
// ExpertLayout): row r goes to block r / spb, slot slot0 + r % spb, and its 16-byte
// piece c (weights 32c .. 32c+31) to ((block * K/64 + c/2) * 4 + slot) * 2 + c % 2
// in 16-byte units; nibbles reordered within each dword. SPLIT8: the source is an
// 8-bit matrix [N][K/2] (one code per byte, K/2 codes a row) read as the int4 row
// of K codes that holds its high nibbles and then its low nibbles.
template <bool SPLIT8>
__global__ void pack_q_kernel(const uint4* __restrict__ src, size_t n16, int K, int spb, int slot0,
                              uint4* __restrict__ dst, size_t dst_stride16) {
    const size_t m = blockIdx.y;
    const size_t cpr = (size_t)K / 32, gpr = (size_t)K / 64;  // pieces and groups per row
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x) {
        uint4 v;
        if constexpr (SPLIT8) {
            // piece c of the int4 row: codes 32c .. 32c+31 = nibbles of source bytes
            // 32 (c mod cpr/2) .. +31 (high nibbles for c < cpr/2), two 16-byte units
            const size_t r = i / cpr, c = i % cpr, h = cpr / 2;
            const bool hi = c < h;
            const uint4* s = src + m * n16 + r * cpr + 2 * (hi ? c : c - h);
            const uint4 a = s[0], b = s[1];
            v = make_uint4(nibbles_of_bytes(a.x, a.y, hi), nibbles_of_bytes(a.z, a.w, hi),
                           nibbles_of_bytes(b.x, b.y, hi), nibbles_of_bytes(b.z, b.w, hi));
        } else {
            v = src[m * n16 + i];
        }
        const size_t r = i / cpr, c = i % cpr;
        const size_t blk = r / spb, slot = slot0 + r % spb;
        const size_t o = ((blk * gpr + c / 2) * 4 + slot) * 2 + c % 2;
        dst[m * dst_stride16 + o] = make_uint4(pack_q_dword(v.x), pack_q_dword(v.y), pack_q_dword(v.z),
                                               pack_q_dword(v.w));
    }
}

// Plain 16-byte copy (router codes).
__global__ void pack_copy_kernel(const uint4* __restrict__ src, size_t src_stride16, uint4* __restrict__ dst,
                                 size_t dst_stride16, size_t n16) {
    const size_t m = blockIdx.y;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        dst[m * dst_stride16 + i] = src[m * src_stride16 + i];
}

// sb = scale | bias << 16 for n entries per expert. gpr > 0: the entries are
// [N][gpr] (row, group) of an expert matrix, placed like the q rows of
// pack_q_kernel at (block * gpr + g) * 4 + slot; gpr == 0: copied in order.
// SPLIT8: the source holds [N][gpr / 2] groups of an 8-bit matrix; int4 group g
// of a row is (16 scale, bias) of source group g for g < gpr / 2 (high nibbles)
// and (scale, 0) of source group g - gpr / 2 (low nibbles).
template <bool SPLIT8>
__global__ void pack_sb_kernel(const uint16_t* __restrict__ s, const uint16_t* __restrict__ b, size_t n, int gpr,
                               int spb, int slot0, uint32_t* __restrict__ dst, size_t dst_stride4) {
    const size_t m = blockIdx.y;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        size_t o = i;
        if (gpr > 0) {
            const size_t r = i / gpr, g = i % gpr;
            o = ((r / spb) * gpr + g) * 4 + slot0 + r % spb;
        }
        uint32_t w;
        if constexpr (SPLIT8) {
            const size_t h = (size_t)gpr / 2, r = i / gpr, g = i % gpr;
            const size_t si = m * (n / 2) + r * h + (g < h ? g : g - h);
            if (g < h)  // 16 scale is exact in bf16: the exponent moves by 4
                w = f32_to_bf16(16.f * bf16_to_f32(s[si])) | ((uint32_t)b[si] << 16);
            else
                w = (uint32_t)s[si];
        } else {
            w = (uint32_t)s[m * n + i] | ((uint32_t)b[m * n + i] << 16);
        }
        dst[m * dst_stride4 + o] = w;
    }
}

static dim3 pack_grid(size_t n, int M) {
    return dim3((unsigned)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024), (unsigned)M);
}

// Expert matrix [N][K/2] per expert (canonical int4), or [N][K/2] bytes of 8-bit
// codes when split8 (K is then the int4 row length, twice the codes), into the
// blocked layout with spb rows per block from slot slot0 (gate 2, 0; up 2, 2;
// down 4, 0).
static moe_status copy_q(const void* src, size_t N, int K, int spb, int slot0, char* dst, size_t stride, int M,
                         bool split8, hipStream_t st) {
    if (!src || !aligned16(src)) return fail(MOE_ERR_INVALID_ARG, "q source NULL or not 16-byte aligned");
    const size_t n16 = N * (size_t)K / 32;
    if (split8)
        hipLaunchKernelGGL(pack_q_kernel<true>, pack_grid(n16, M), dim3(256), 0, st, (const uint4*)src, n16, K, spb,
                           slot0, (uint4*)dst, stride / 16);
    else
        hipLaunchKernelGGL(pack_q_kernel<false>, pack_grid(n16, M), dim3(256), 0, st, (const uint4*)src, n16, K, spb,
                           slot0, (uint4*)dst, stride / 16);
    return check_launch("pack_q_kernel");
}

// Router codes or fp32 router rows, unchanged.
static moe_status copy_raw(const void* src, size_t bytes, char* dst, hipStream_t st) {
    if (!src || !aligned16(src)) return fail(MOE_ERR_INVALID_ARG, "source NULL or not 16-byte aligned");
    const size_t n16 = bytes / 16;
    hipLaunchKernelGGL(pack_copy_kernel, pack_grid(n16, 1), dim3(256), 0, st, (const uint4*)src, n16, (uint4*)dst,
                       (size_t)0, n16);
    return check_launch("pack_copy_kernel");
}

// (scale, bias) words: n entries per expert, blocked like copy_q when gpr > 0
// (split8: n and gpr count the int4 groups, twice the source's).
static moe_status copy_sb(const uint16_t* s, const uint16_t* b, size_t n, int gpr, int spb, int slot0, char* dst,
                          size_t stride, int M, bool split8, hipStream_t st) {
    if (!s || !b) return fail(MOE_ERR_INVALID_ARG, "scale/bias source NULL");
    if (split8)
        hipLaunchKernelGGL(pack_sb_kernel<true>, pack_grid(n, M), dim3(256), 0, st, s, b, n, gpr, spb, slot0,
                           (uint32_t*)dst, stride / 4);
    else
        hipLaunchKernelGGL(pack_sb_kernel<false>, pack_grid(n, M), dim3(256), 0, st, s, b, n, gpr, spb, slot0,
                           (uint32_t*)dst, stride / 4);
    return check_launch("pack_sb_kernel");
}

extern "C" moe_status moe_pack_experts(const moe_shape* sh, const moe_expert_canon* src, void* packed,
                                       size_t packed_bytes, void* stream) {
    clear_error();
    moe_status st = validate_shape(sh);
    if (st != MOE_OK) return st;
    if (!src || !packed || !aligned16(packed)) return fail(MOE_ERR_INVALID_ARG, "NULL or unaligned pointer");
    const ExpertLayout L = expert_layout(*sh);
    const int M = n_mats(*sh);
    if (packed_bytes < L.stride * (size_t)M) return fail(MOE_ERR_WORKSPACE, "packed buffer too small");
    // H, I: row lengths in int4 codes (8-bit rows are packed as int4 rows twice as long)
    const size_t H = (size_t)sh->hidden * kmul(*sh), I = (size_t)sh->inter * kmul(*sh);
    const size_t Ho = sh->hidden, Io = sh->inter;  // rows of the down and gate/up matrices
    const bool sp = sh->bits == 8;
    hipStream_t s = (hipStream_t)stream;
    char* d = (char*)packed;
    const int Hi = (int)H, Ii = (int)I;
    if ((st = copy_q(src->q_gate, Io, Hi, 2, 0, d + L.gu_q, L.stride, M, sp, s)) != MOE_OK) return st;
    if ((st = copy_q(src->q_up, Io, Hi, 2, 2, d + L.gu_q, L.stride, M, sp, s)) != MOE_OK) return st;
    if ((st = copy_q(src->q_down, Ho, Ii, 4, 0, d + L.down_q, L.stride, M, sp, s)) != MOE_OK) return st;
    if ((st = copy_sb(src->s_gate, src->b_gate, Io * (H / 64), Hi / 64, 2, 0, d + L.gu_sb, L.stride, M, sp, s)) !=
        MOE_OK)
        return st;
    if ((st = copy_sb(src->s_up, src->b_up, Io * (H / 64), Hi / 64, 2, 2, d + L.gu_sb, L.stride, M, sp, s)) != MOE_OK)
        return st;
    if ((st = copy_sb(src->s_down, src->b_down, Ho * (I / 64), Ii / 64, 4, 0, d + L.down_sb, L.stride, M, sp, s)) !=
        MOE_OK)
        return st;
    return MOE_OK;
}

extern "C" moe_status moe_pack_router(const moe_shape* sh, const void* w, const uint16_t* s, const uint16_t* b,
                                      void* packed, size_t packed_bytes, void* stream) {
    clear_error();
    moe_status st = validate_shape(sh);
    if (st != MOE_OK) return st;
    if (!w || !packed || !aligned16(packed) || !aligned16(w))
        return fail(MOE_ERR_INVALID_ARG, "NULL or unaligned pointer");
    const size_t need = moe_router_packed_bytes(sh);
    if (packed_bytes < need) return fail(MOE_ERR_WORKSPACE, "router buffer too small");
    const size_t R = router_rows(*sh), H = sh->hidden;
    hipStream_t hs = (hipStream_t)stream;
    if (sh->router_fmt == MOE_ROUTER_F32) {
        if (s || b) return fail(MOE_ERR_INVALID_ARG, "fp32 router takes no scale/bias");
        return copy_raw(w, R * H * 4, (char*)packed, hs);
    }
    if ((st = copy_raw(w, R * H, (char*)packed, hs)) != MOE_OK) return st;
    return copy_sb(s, b, R * (H / 64), 0, 1, 0, (char*)packed + R * H, 0, 1, false, hs);
}

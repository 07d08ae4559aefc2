// Internal helpers shared by the HIP kernels and the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ------------------------------------------------------------------ host side

moe_status fail(moe_status st, const char* fmt, ...);
moe_status check_launch(const char* what);
void clear_error();

// Validates the shape for every entry point (formats served, size limits).
moe_status validate_shape(const moe_shape* sh);

// Expert weight rows as the kernels read them. A 4-bit row of K weights is a row of
// K int4 codes. An 8-bit row is packed as an int4 row of 2K codes: the high nibbles
// of its K codes (groups 0 .. K/64-1, with scale 16 * scale and the bias) and then
// the low nibbles (groups K/64 .. 2K/64-1, with scale and bias 0), so that
//   sum_k x_k (s q_k + b) = sum_k x_k (16 s hi_k + b) + sum_k x_k (s lo_k + 0)
// exactly; the activation of code j is x[j mod K]. kmul = row length / K.
inline int32_t kmul(const moe_shape& s) { return s.bits / 4; }

inline int32_t n_mats(const moe_shape& s) { return s.n_experts + (s.has_shared ? 1 : 0); }
inline int32_t n_slots(const moe_shape& s) { return s.top_k + (s.has_shared ? 1 : 0); }
inline int32_t router_rows(const moe_shape& s) { return s.n_experts + (s.has_shared ? 1 : 0); }

// Byte offsets of one expert's segments inside the packed buffer. Weight rows are
// stored in blocks of four rows per quantisation group: each 128-byte line holds
// the 32 bytes (64 int4 weights) of one group for four rows, so a grouped GEMM
// that walks K one group at a time reads whole lines, and a wavefront that
// streams the four rows of a block back to back reads the same lines.
//   gu_q    [I/2][H/64][4][32 B]: block b holds gate rows 2b, 2b+1 and up rows 2b, 2b+1
//   down_q  [H/4][I/64][4][32 B]: block b holds down rows 4b .. 4b+3
//   gu_sb   [I/2][H/64][4] and down_sb [H/4][I/64][4]: the (scale | bias << 16) words
//           of the same rows and groups, in the same order
struct ExpertLayout {
    size_t gu_q, down_q, gu_sb, down_sb, stride;
};

inline ExpertLayout expert_layout(const moe_shape& s) {
    // 2 I gate/up rows of Hw int4 codes and H down rows of Iw codes (Hw = H kmul,
    // Iw = I kmul); half a byte per code, one (scale, bias) word per 64 codes
    const size_t H = (size_t)s.hidden, I = (size_t)s.inter, G = 64;
    const size_t Hw = H * kmul(s), Iw = I * kmul(s);
    ExpertLayout L;
    L.gu_q = 0;
    L.down_q = L.gu_q + 2 * I * Hw / 2;
    L.gu_sb = L.down_q + H * Iw / 2;
    L.down_sb = L.gu_sb + 2 * I * (Hw / G) * 4;
    L.stride = L.down_sb + H * (Iw / G) * 4;
    return L;
}

// Row bases inside one expert (byte offsets); H and I are the weight row lengths
// (hidden and inter times kmul). The 16-byte piece ch (weights 32 ch .. 32 ch + 31)
// of a row is at base + (ch / 2) * 128 + (ch % 2) * 16; the word of group g of a
// row's sb is at sb base + 16 g.
__host__ __device__ inline size_t gu_row_q(const ExpertLayout& L, int H, int up, int i) {
    return L.gu_q + (size_t)(i >> 1) * (size_t)(H / 64) * 128 + (size_t)((up ? 2 : 0) + (i & 1)) * 32;
}
__host__ __device__ inline size_t gu_row_sb(const ExpertLayout& L, int H, int up, int i) {
    return L.gu_sb + (size_t)(i >> 1) * (size_t)(H / 64) * 16 + (size_t)((up ? 2 : 0) + (i & 1)) * 4;
}
__host__ __device__ inline size_t dn_row_q(const ExpertLayout& L, int I, int n) {
    return L.down_q + (size_t)(n >> 2) * (size_t)(I / 64) * 128 + (size_t)(n & 3) * 32;
}
__host__ __device__ inline size_t dn_row_sb(const ExpertLayout& L, int I, int n) {
    return L.down_sb + (size_t)(n >> 2) * (size_t)(I / 64) * 16 + (size_t)(n & 3) * 4;
}
__host__ __device__ inline size_t piece_off(int ch) { return (size_t)(ch >> 1) * 128 + (size_t)(ch & 1) * 16; }

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// ------------------------------------------------------------------ device side

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN -> 0x7FC0 (keeps the sign bit clear).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// fp64 -> bf16 bits with one round-to-nearest-even step (no fp32 intermediate).
// The value is sig * 2^(e-52) with a 53-bit significand; the bf16 quantum is
// 2^max(e-7, -133). The encoding ((qe + 134) << 7) + n - 128 covers normal
// results, subnormal results (qe = -133, n < 128) and the carry into the next
// binade (n = 256); an exponent field of 255 is infinity.
__device__ __forceinline__ uint32_t f64_to_bf16(double d) {
    const uint64_t u = (uint64_t)__double_as_longlong(d);
    const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
    const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
    if (a > 0x7FF0000000000000ull) return 0x7FC0u;
    if (a == 0x7FF0000000000000ull) return sign | 0x7F80u;
    const int bexp = (int)(a >> 52);
    if (bexp == 0) return sign;  // fp64 subnormal: far below half the least bf16 subnormal
    const int e = bexp - 1023;
    if (e >= 128) return sign | 0x7F80u;
    if (e < -135) return sign;
    const uint64_t sig = (a & 0x000FFFFFFFFFFFFFull) | 0x0010000000000000ull;
    const int qe = e - 7 > -133 ? e - 7 : -133;
    const int sh = 52 + qe - e;  // 45 for normal results, up to 54 here
    uint64_t n = sig >> sh;
    const uint64_t rem = sig & ((1ull << sh) - 1);
    const uint64_t half = 1ull << (sh - 1);
    if (rem > half || (rem == half && (n & 1))) ++n;
    uint32_t bits = (uint32_t)(((int64_t)(qe + 134) << 7) + (int64_t)n - 128);
    if (bits >= 0x7F80u) bits = 0x7F80u;
    return sign | bits;
}

// (v & m) | c in one v_and_or_b32. The VOP3 encoding takes no literal and (on this
// chip) at most one scalar operand, so the mask goes in an SGPR and the constant in
// a VGPR.
__device__ __forceinline__ uint32_t and_or_b32(uint32_t v, uint32_t m, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "s"(m), "v"(c));
    return r;
}

// Eight int4 weights of one packed dword (nibble j = k_{2j}, nibble 4+j = k_{2j+1})
// as four bf16 pairs (k0,k1), (k2,k3), (k4,k5), (k6,k7), each value 1 + q/16
// exactly: q lands in mantissa bits 3..6 under the exponent of 1.0. A dot product
// with activations in their natural order gives sum x * (1 + q/16).
__device__ __forceinline__ void int4x8_to_bf16_pairs(uint32_t v, uint32_t out[4]) {
    const uint32_t one = 0x3F803F80u;
    out[0] = and_or_b32(v << 3, 0x00780078u, one);
    out[1] = and_or_b32(v >> 1, 0x00780078u, one);
    out[2] = and_or_b32(v >> 5, 0x00780078u, one);
    out[3] = and_or_b32(v >> 9, 0x00780078u, one);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Coherent (agent-scope) 32-bit accesses for data that one workgroup publishes to
// others inside a kernel: they go to the device coherence point, so publishing
// needs no cache-wide write-back or invalidate, only store completion
// (publish_fence) before the counter that announces them.
__device__ __forceinline__ void store_coherent(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_coherent(const uint32_t* p) {
    return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until every memory operation this wavefront issued has completed.
__device__ __forceinline__ void publish_fence() { __builtin_amdgcn_s_waitcnt(0); }

// Tagged publishing inside one launch: a 64-bit coherent store of (tag, value);
// a reader polls the word until its tag is the launch's tag, so the data itself
// announces that it is ready (no separate counter round trip). Polls are bounded:
// after SPIN_LIMIT polls the error word is set and the stale value is returned.
constexpr unsigned SPIN_LIMIT = 1u << 20;

__device__ __forceinline__ void store_tagged(uint64_t* p, uint32_t tag, uint32_t v) {
    __hip_atomic_store(p, ((uint64_t)tag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_tagged_wait(const uint64_t* p, uint32_t tag, unsigned* err) {
    uint64_t v = __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned it = 0;
    while ((uint32_t)(v >> 32) != tag) {
        if (++it >= SPIN_LIMIT) {
            atomicOr(err, 1u);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
        v = __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return (uint32_t)v;
}

// N tagged words at p[0], p[stride], ...: all loads issued at once, then only the
// stale ones are polled again (bounded). Returns true if the wait timed out (the
// error word is then set and out[] may hold stale values).
template <int N>
__device__ __forceinline__ bool load_tagged_many(const uint64_t* p, int stride, int n, uint32_t tag, unsigned* err,
                                                 uint32_t* out) {
    uint64_t v[N];
#pragma unroll
    for (int j = 0; j < N; ++j)
        v[j] = j < n ? __hip_atomic_load(const_cast<uint64_t*>(p + (size_t)j * stride), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT)
                     : ((uint64_t)tag << 32);
    bool timed_out = false;
    for (unsigned it = 0;; ++it) {
        bool ok = true;
#pragma unroll
        for (int j = 0; j < N; ++j) ok = ok && (uint32_t)(v[j] >> 32) == tag;
        if (ok) break;
        if (it >= SPIN_LIMIT) {
            atomicOr(err, 1u);
            timed_out = true;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int j = 0; j < N; ++j)
            if ((uint32_t)(v[j] >> 32) != tag)
                v[j] = __hip_atomic_load(const_cast<uint64_t*>(p + (size_t)j * stride), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int j = 0; j < N; ++j) out[j] = (uint32_t)v[j];
    return timed_out;
}

// As load_tagged_many, but every round reloads all n words together (0 <= n <= N;
// p[0] must be readable even when n = 0; out[j] = 0 for j >= n). A word that
// carries the launch's tag never changes again within the launch, so reloading it
// is harmless. The loads are unconditional and the empty asm statements keep them
// together; with a per-word test the compiler gives each reload a branch and a
// wait of its own, one round trip per stale word. For short lists of words that
// few wavefronts wait on: the decode layer's selection with few tokens. With many
// polling wavefronts the extra loads in flight slow the producers more than the
// serial re-polls cost (measured at 16 tokens per launch). Returns true if the
// wait timed out.
template <int N>
__device__ __forceinline__ bool load_tagged_batch(const uint64_t* p, int stride, int n, uint32_t tag, unsigned* err,
                                                  uint32_t* out) {
    uint64_t v[N];
    bool timed_out = false;
    for (unsigned it = 0;; ++it) {
#pragma unroll
        for (int j = 0; j < N; ++j)
            v[j] = __hip_atomic_load(const_cast<uint64_t*>(p + (size_t)(j < n ? j : 0) * stride), __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int j = 0; j < N; ++j) asm volatile("" : "+v"(v[j]));
        bool ok = true;
#pragma unroll
        for (int j = 0; j < N; ++j) ok = ok && (j >= n || (uint32_t)(v[j] >> 32) == tag);
        if (ok) break;
        if (it >= SPIN_LIMIT) {
            atomicOr(err, 1u);
            timed_out = true;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int j = 0; j < N; ++j) out[j] = j < n ? (uint32_t)v[j] : 0u;
    return timed_out;
}

// As load_tagged_batch, for a race between wavefronts that poll copies of the
// same words: *owner (LDS, -1 before the race) takes the id `me` of the first
// wavefront whose words all carry the tag, or that gives up after SPIN_LIMIT
// rounds (the error word is then set); the others stop at their next round.
// Returns whether this wavefront won; only the winner's out[] is meaningful, and
// gave_up tells the winner that its words may be stale (it timed out).
template <int N>
__device__ __forceinline__ bool load_tagged_race(const uint64_t* p, int stride, int n, uint32_t tag, unsigned* err,
                                                 int* owner, int me, uint32_t* out, bool& gave_up) {
    uint64_t v[N];
    gave_up = false;
    for (unsigned it = 0;; ++it) {
#pragma unroll
        for (int j = 0; j < N; ++j)
            v[j] = __hip_atomic_load(const_cast<uint64_t*>(p + (size_t)(j < n ? j : 0) * stride), __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int j = 0; j < N; ++j) asm volatile("" : "+v"(v[j]));
        bool ok = true;
#pragma unroll
        for (int j = 0; j < N; ++j) ok = ok && (j >= n || (uint32_t)(v[j] >> 32) == tag);
        const bool give_up = it >= SPIN_LIMIT;
        if (__ballot(ok) == __ballot(true) || give_up) {
            if (give_up) atomicOr(err, 1u);
            gave_up = give_up;
            int prev = 0;
            if ((threadIdx.x & 63) == 0) prev = atomicCAS(owner, -1, me);
            prev = __shfl(prev, 0);
#pragma unroll
            for (int j = 0; j < N; ++j) out[j] = j < n ? (uint32_t)v[j] : 0u;
            return prev == -1;
        }
        if (*reinterpret_cast<volatile int*>(owner) != -1) return false;
        __builtin_amdgcn_s_sleep(1);
    }
}

// DPP move of a 32-bit value (every lane must be active).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// Sum over aligned groups of `lpr` lanes (a power of two up to 64) with DPP: quad
// permutations, half-row and row mirrors, then the row broadcasts 15 and 31. The
// sum is valid in the last lane of each group (and, for lpr <= 16, in every lane).
__device__ __forceinline__ float group_sum(float v, int lpr) {
    if (lpr >= 2) v += __uint_as_float(dpp_u32<0xB1, 0xF>(__float_as_uint(v)));
    if (lpr >= 4) v += __uint_as_float(dpp_u32<0x4E, 0xF>(__float_as_uint(v)));
    if (lpr >= 8) v += __uint_as_float(dpp_u32<0x141, 0xF>(__float_as_uint(v)));
    if (lpr >= 16) v += __uint_as_float(dpp_u32<0x140, 0xF>(__float_as_uint(v)));
    if (lpr >= 32) v += __uint_as_float(dpp_u32<0x142, 0xA>(__float_as_uint(v)));
    if (lpr >= 64) v += __uint_as_float(dpp_u32<0x143, 0xC>(__float_as_uint(v)));
    return v;
}

// ---- unit-weight RMSNorm (the stack's pre-norm reading): every kernel that
// normalises a row computes the sum of squares in this one order, so the staged
// norm and the norm inside the decode layer give the same bf16 values.
// Lane l adds the squares of the 16-element pieces starting at 16 (l + 64 c),
// c = 0, 1, ... (in element order, fp32 fused multiply-adds); group_sum's tree
// adds the 64 lane sums. row_sumsq returns the total in every lane.
__device__ __forceinline__ float sumsq_piece16(uint4 a, uint4 b, float ss) {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xFFFF0000u);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
    }
    return ss;
}
__device__ __forceinline__ float sumsq_total(float lane_sum) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(group_sum(lane_sum, 64)), 63));
}
__device__ __forceinline__ float row_sumsq(const uint16_t* __restrict__ row, int H, int lane) {
    float ss = 0.f;
    for (int c = 0; 16 * (lane + 64 * c) < H; ++c) {
        const uint4* p = reinterpret_cast<const uint4*>(row + 16 * (lane + 64 * c));
        ss = sumsq_piece16(p[0], p[1], ss);
    }
    return sumsq_total(ss);
}
// 1 / sqrt(mean(x^2) + eps) in fp32 (correctly rounded division and square root).
__device__ __forceinline__ float rms_scale(float sumsq, int H, float eps) {
    return 1.f / sqrtf(sumsq / (float)H + eps);
}
// bf16(x * r) of one bf16 value.
__device__ __forceinline__ uint32_t norm_bf16(uint32_t xbits, float r) {
    return f32_to_bf16(bf16_to_f32(xbits) * r);
}

__device__ __forceinline__ double dpp_f64_step(double v, int step) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
    switch (step) {
        case 0: lo = dpp_u32<0xB1, 0xF>(lo); hi = dpp_u32<0xB1, 0xF>(hi); break;
        case 1: lo = dpp_u32<0x4E, 0xF>(lo); hi = dpp_u32<0x4E, 0xF>(hi); break;
        case 2: lo = dpp_u32<0x141, 0xF>(lo); hi = dpp_u32<0x141, 0xF>(hi); break;
        case 3: lo = dpp_u32<0x140, 0xF>(lo); hi = dpp_u32<0x140, 0xF>(hi); break;
        case 4: lo = dpp_u32<0x142, 0xA>(lo); hi = dpp_u32<0x142, 0xA>(hi); break;
        default: lo = dpp_u32<0x143, 0xC>(lo); hi = dpp_u32<0x143, 0xC>(hi); break;
    }
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// fp64 sum over the whole wavefront with DPP; valid in lane 63.
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int step = 0; step < 6; ++step) v += dpp_f64_step(v, step);
    return v;
}

// Where a selection reads its fp32 logits: a plain array (written by an earlier
// launch), a coherently written array (same launch, completion announced by a
// counter), or a tagged array (same launch, tag-polled).
struct LogitSrc {
    const float* plain;
    const uint64_t* tagged;
    uint32_t tag;
    unsigned* err;
    bool coherent;
    bool batch;  // tagged: reload every word in each polling round (load_tagged_batch)
    int* race = nullptr;  // tagged, batch: LDS word of a polling race (load_tagged_race)
    int me = 0;           // this wavefront's entry in that race
    __device__ __forceinline__ uint32_t get(int i) const {
        if (tagged) return load_tagged_wait(tagged + i, tag, err);
        if (coherent) return load_coherent(reinterpret_cast<const uint32_t*>(plain) + i);
        return __float_as_uint(plain[i]);
    }
};

// Unsigned key ordering fp32 logits: larger logit -> larger key; -0 equals +0;
// NaN gets key 0, below every number.
__device__ __forceinline__ uint32_t ordered_logit(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace moe

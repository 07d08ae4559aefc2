// Weighted combine (one bf16 rounding of the weighted slot sum: TensorFold issue
// #931, "What I'd build") with the optional residual add of a stacked block, and
// the unit-weight RMSNorm used between stacked blocks.
#include "moe_internal.h"

namespace moe {
typedef float f4_t __attribute__((ext_vector_type(4)));

// One thread per four consecutive outputs of a token; slots are summed in slot
// order (0..k-1, then the shared slot) with fp32 fused multiply-adds. y is read
// once, with non-temporal loads, so it does not displace other data in the caches.
// Every load of a thread (its k + 1 weights and slot values) is issued before the
// first sum: a loop that loaded and summed one slot at a time waited for nine round
// trips in turn (512 tokens: 9 us). KM >= k bounds the unrolled slots.
template <int KM>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const uint16_t* __restrict__ w,
                                                      const uint16_t* __restrict__ wsh, int T, int H, int k, int S,
                                                      const uint16_t* residual, uint16_t* out) {
    const size_t n4 = H / 4;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)T * n4) return;
    const size_t t = idx / n4, c = (idx % n4) * 4;
    const float* yt = y + t * S * H + c;
    uint32_t wr[KM + 1];  // raw bf16 weights, one per register: converted only when summed, so no load waits for another
    f4_t v[KM + 1];
#pragma unroll
    for (int s = 0; s < KM; ++s) {
        if (s < k) {
            wr[s] = w[t * k + s];
            v[s] = __builtin_nontemporal_load(reinterpret_cast<const f4_t*>(yt + (size_t)s * H));
        }
    }
    if (wsh) {
        wr[KM] = wsh[t];
        v[KM] = __builtin_nontemporal_load(reinterpret_cast<const f4_t*>(yt + (size_t)k * H));
    }
    uint2 r = make_uint2(0u, 0u);
    if (residual) r = *reinterpret_cast<const uint2*>(residual + t * H + c);
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int s = 0; s < KM; ++s) {
        if (s < k) {
            const float ws = bf16_to_f32(wr[s]);
            a0 = fmaf(ws, v[s].x, a0);
            a1 = fmaf(ws, v[s].y, a1);
            a2 = fmaf(ws, v[s].z, a2);
            a3 = fmaf(ws, v[s].w, a3);
        }
    }
    if (wsh) {
        const float ws = bf16_to_f32(wr[KM]);
        a0 = fmaf(ws, v[KM].x, a0);
        a1 = fmaf(ws, v[KM].y, a1);
        a2 = fmaf(ws, v[KM].z, a2);
        a3 = fmaf(ws, v[KM].w, a3);
    }
    uint32_t b0 = f32_to_bf16(a0), b1 = f32_to_bf16(a1), b2 = f32_to_bf16(a2), b3 = f32_to_bf16(a3);
    if (residual) {
        b0 = f32_to_bf16(bf16_to_f32(r.x & 0xFFFFu) + bf16_to_f32(b0));
        b1 = f32_to_bf16(bf16_to_f32(r.x >> 16) + bf16_to_f32(b1));
        b2 = f32_to_bf16(bf16_to_f32(r.y & 0xFFFFu) + bf16_to_f32(b2));
        b3 = f32_to_bf16(bf16_to_f32(r.y >> 16) + bf16_to_f32(b3));
    }
    uint2 o;
    o.x = b0 | (b1 << 16);
    o.y = b2 | (b3 << 16);
    *reinterpret_cast<uint2*>(out + t * H + c) = o;
}

// One wavefront per row (four rows per workgroup): the sum of squares in the
// order of row_sumsq, r = 1 / sqrt(mean + eps), out = bf16(x * r).
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ x, int T, int H, float eps,
                                                      uint16_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const uint16_t* row = x + (size_t)t * H;
    const float r = rms_scale(row_sumsq(row, H, lane), H, eps);
    for (int i = 8 * lane; i < H; i += 512) {
        const uint4 v = *reinterpret_cast<const uint4*>(row + i);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = norm_bf16(w[j] & 0xFFFFu, r) | (norm_bf16(w[j] >> 16, r) << 16);
        *reinterpret_cast<uint4*>(out + (size_t)t * H + i) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_combine(const moe_shape* shape, const float* y, const uint16_t* w, const uint16_t* w_shared,
                                  int32_t T, const uint16_t* residual, uint16_t* out, void* stream) {
    clear_error();
    moe_status st = validate_shape(shape);
    if (st != MOE_OK) return st;
    if (T < 1) return fail(MOE_ERR_INVALID_ARG, "T = %d, need T >= 1", T);
    if (!y || !w || !out || !aligned16(y) || !aligned16(out) || (residual && !aligned16(residual)))
        return fail(MOE_ERR_INVALID_ARG, "NULL or unaligned pointer");
    if (shape->has_shared != (w_shared != nullptr))
        return fail(MOE_ERR_INVALID_ARG, "w_shared must be given iff the layer has a shared expert");
    const int H = shape->hidden;
    const size_t n = (size_t)T * (H / 4);
    auto kern = shape->top_k <= 8 ? combine_kernel<8> : combine_kernel<16>;
    hipLaunchKernelGGL(kern, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream, y, w, w_shared, T,
                       H, shape->top_k, n_slots(*shape), residual, out);
    return check_launch("combine_kernel");
}

extern "C" moe_status moe_rmsnorm(int32_t hidden, const uint16_t* x, int32_t T, float eps, uint16_t* out,
                                  void* stream) {
    clear_error();
    if (hidden < 64 || hidden % 64 != 0) return fail(MOE_ERR_INVALID_ARG, "hidden %d must be a multiple of 64", hidden);
    if (T < 1 || !x || !out || x == out || !aligned16(x) || !aligned16(out))
        return fail(MOE_ERR_INVALID_ARG, "bad T or pointers (NULL, unaligned or aliased)");
    hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, (hipStream_t)stream, x, T, hidden,
                       eps, out);
    return check_launch("rmsnorm_kernel");
}

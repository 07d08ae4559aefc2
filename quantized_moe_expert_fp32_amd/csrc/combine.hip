// Weighted combine (one bf16 rounding of the weighted slot sum: TensorFold issue
// #931, "What I'd build") with the optional residual add of a stacked block, and
// the unit-weight RMSNorm used between stacked blocks.
#include "moe_internal.h"

namespace moe {
typedef float f4_t __attribute__((ext_vector_type(4)));

// One thread per four consecutive outputs of a token; slots are summed in slot
// order (0..k-1, then the shared slot) with fp32 fused multiply-adds. y is read
// once, with non-temporal loads, so it does not displace other data in the caches.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const uint16_t* __restrict__ w,
                                                      const uint16_t* __restrict__ wsh, int T, int H, int k, int S,
                                                      const uint16_t* residual, uint16_t* out) {
    const size_t n4 = H / 4;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)T * n4) return;
    const size_t t = idx / n4, c = (idx % n4) * 4;
    const float* yt = y + t * S * H + c;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int s = 0; s < k; ++s) {
        const float ws = bf16_to_f32(w[t * k + s]);
        const f4_t v = __builtin_nontemporal_load(reinterpret_cast<const f4_t*>(yt + (size_t)s * H));
        a0 = fmaf(ws, v.x, a0);
        a1 = fmaf(ws, v.y, a1);
        a2 = fmaf(ws, v.z, a2);
        a3 = fmaf(ws, v.w, a3);
    }
    if (wsh) {
        const float ws = bf16_to_f32(wsh[t]);
        const f4_t v = __builtin_nontemporal_load(reinterpret_cast<const f4_t*>(yt + (size_t)k * H));
        a0 = fmaf(ws, v.x, a0);
        a1 = fmaf(ws, v.y, a1);
        a2 = fmaf(ws, v.z, a2);
        a3 = fmaf(ws, v.w, a3);
    }
    uint32_t b0 = f32_to_bf16(a0), b1 = f32_to_bf16(a1), b2 = f32_to_bf16(a2), b3 = f32_to_bf16(a3);
    if (residual) {
        const uint2 r = *reinterpret_cast<const uint2*>(residual + t * H + c);
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

// One block per row: sum of squares in a fixed order (per-thread strided partial
// sums, then a tree over the block), r = 1 / sqrt(mean + eps), out = bf16(x * r).
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ x, int H, float eps,
                                                      uint16_t* __restrict__ out) {
    __shared__ float red[256];
    const uint16_t* row = x + (size_t)blockIdx.x * H;
    float ss = 0.f;
    for (int i = threadIdx.x; i < H; i += 256) {
        const float v = bf16_to_f32(row[i]);
        ss = fmaf(v, v, ss);
    }
    red[threadIdx.x] = ss;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    const float r = 1.f / sqrtf(red[0] / (float)H + eps);
    for (int i = threadIdx.x; i < H; i += 256)
        out[(size_t)blockIdx.x * H + i] = (uint16_t)f32_to_bf16(bf16_to_f32(row[i]) * r);
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
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream, y, w,
                       w_shared, T, H, shape->top_k, n_slots(*shape), residual, out);
    return check_launch("combine_kernel");
}

extern "C" moe_status moe_rmsnorm(int32_t hidden, const uint16_t* x, int32_t T, float eps, uint16_t* out,
                                  void* stream) {
    clear_error();
    if (hidden < 64 || hidden % 64 != 0) return fail(MOE_ERR_INVALID_ARG, "hidden %d must be a multiple of 64", hidden);
    if (T < 1 || !x || !out || x == out) return fail(MOE_ERR_INVALID_ARG, "bad T or pointers");
    hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)T), dim3(256), 0, (hipStream_t)stream, x, hidden, eps, out);
    return check_launch("rmsnorm_kernel");
}

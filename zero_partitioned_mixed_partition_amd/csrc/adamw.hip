// Fused mixed-precision AdamW update of one rank's shard (gfx950).
//
// "Zero Redundancy Optimizer (ZeRO) and Fully Sharded Data Parallelism (FSDP):
// Mathematical Foundations ...": section "Static Memory Allocation" fixes the
// state (fp32 master, m_t, v_t; 16-bit parameters), "Execution Flow for
// ZeRO-1" steps 3-4 the work (update the own slice, emit 16-bit parameters),
// and "ZeRO-Offload Mechanics" its cost (O(1) per parameter). The update
// formula follows decoupled-weight-decay AdamW with bias correction; the
// per-element order of fp32 operations is fixed (see the ABI header) and the
// library is compiled without floating-point contraction, so results do not
// depend on the launch shape.
//
// Memory: 28 bytes per element (read 12 fp32 + 2 bf16, write 12 fp32 + 2
// bf16), about 15 flops: HBM-bound by a factor of ~40 against the fp32
// vector ridge point, so no matrix cores. Each thread moves groups of 8
// elements with 16-byte non-temporal loads and stores: two dwordx4 per fp32
// array, one for the bf16 gradient and one for the bf16 parameters. The grid
// is persistent (a few workgroups per compute unit, sized from the device's
// CU count) and grid-strides over the groups with 64-bit indices.
#include <hip/hip_runtime.h>

#include <cmath>
#include <string>

#include "device_common.hpp"
#include "internal.hpp"

#pragma clang fp contract(off)

namespace {

using zero::dev::f32x4;
using zero::dev::u32x4;

constexpr int kThreads = 256;
#ifndef ZERO_ADAMW_OVERSUB
#define ZERO_ADAMW_OVERSUB 1
#endif
#ifndef ZERO_ADAMW_UNROLL
#define ZERO_ADAMW_UNROLL 2
#endif

struct AdamScalars {
    float beta1, one_minus_beta1, beta2, one_minus_beta2, eps, step_size, sqrt_bc2, decay;
};

// One element, in the documented order; every line is one IEEE fp32 operation.
__device__ __forceinline__ void adam_elem(float& p, float& m, float& v, float g,
                                          const AdamScalars& c) {
    const float bm = c.beta1 * m;
    const float gm = c.one_minus_beta1 * g;
    m = bm + gm;
    const float bv = c.beta2 * v;
    const float gg = g * g;
    const float gv = c.one_minus_beta2 * gg;
    v = bv + gv;
    p = p * c.decay;
    const float root = sqrtf(v);
    const float denom = root / c.sqrt_bc2 + c.eps;
    const float ratio = m / denom;
    p = p - c.step_size * ratio;
}

__device__ __forceinline__ float read_clip(const float* clip_scale) {
    return clip_scale != nullptr ? *clip_scale : 1.0f;
}

struct Group {   // 8 consecutive elements of every stream
    f32x4 p[2], m[2], v[2];
    u32x4 g;
};

__device__ __forceinline__ void load_group(Group& x, const f32x4* master, const f32x4* m,
                                           const f32x4* v, const u32x4* grad, int64_t i) {
    x.p[0] = zero::dev::ld_stream(master + 2 * i);
    x.p[1] = zero::dev::ld_stream(master + 2 * i + 1);
    x.m[0] = zero::dev::ld_stream(m + 2 * i);
    x.m[1] = zero::dev::ld_stream(m + 2 * i + 1);
    x.v[0] = zero::dev::ld_stream(v + 2 * i);
    x.v[1] = zero::dev::ld_stream(v + 2 * i + 1);
    x.g = zero::dev::ld_stream(grad + i);
}

__device__ __forceinline__ void update_group(Group& x, float clip, const AdamScalars& c,
                                             u32x4& out) {
    float pv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t w = x.g[j / 2];
        const float gj = (j & 1) ? zero::dev::hi_bf16(w) : zero::dev::lo_bf16(w);
        float p = x.p[j / 4][j % 4], m = x.m[j / 4][j % 4], v = x.v[j / 4][j % 4];
        adam_elem(p, m, v, gj * clip, c);
        x.p[j / 4][j % 4] = p;
        x.m[j / 4][j % 4] = m;
        x.v[j / 4][j % 4] = v;
        pv[j] = p;
    }
    out.x = zero::dev::pack_bf16(pv[0], pv[1]);
    out.y = zero::dev::pack_bf16(pv[2], pv[3]);
    out.z = zero::dev::pack_bf16(pv[4], pv[5]);
    out.w = zero::dev::pack_bf16(pv[6], pv[7]);
}

__device__ __forceinline__ void store_group(const Group& x, const u32x4& out, f32x4* master,
                                            f32x4* m, f32x4* v, u32x4* param, int64_t i) {
    zero::dev::st_stream(master + 2 * i, x.p[0]);
    zero::dev::st_stream(master + 2 * i + 1, x.p[1]);
    zero::dev::st_stream(m + 2 * i, x.m[0]);
    zero::dev::st_stream(m + 2 * i + 1, x.m[1]);
    zero::dev::st_stream(v + 2 * i, x.v[0]);
    zero::dev::st_stream(v + 2 * i + 1, x.v[1]);
    zero::dev::st_stream(param + i, out);
}

__device__ __forceinline__ void scalar_elem(float* __restrict__ master, float* __restrict__ m,
                                            float* __restrict__ v,
                                            const uint16_t* __restrict__ grad,
                                            uint16_t* __restrict__ param, int64_t i, float clip,
                                            const AdamScalars& c) {
    float p = master[i], mm = m[i], vv = v[i];
    adam_elem(p, mm, vv, zero::dev::bf16_to_f32(grad[i]) * clip, c);
    master[i] = p;
    m[i] = mm;
    v[i] = vv;
    param[i] = static_cast<uint16_t>(zero::dev::f32_to_bf16(p));
}

// Vector path: groups [0, n_groups) of 8 elements, then elements
// [8*n_groups, n) one per thread. All five pointers are 16-byte aligned.
template <int kUnroll>
__global__ __launch_bounds__(kThreads) void adamw_vec(float* __restrict__ master,
                                                      float* __restrict__ m,
                                                      float* __restrict__ v,
                                                      const uint16_t* __restrict__ grad,
                                                      uint16_t* __restrict__ param, int64_t n,
                                                      AdamScalars c,
                                                      const float* __restrict__ clip_scale) {
    const float clip = read_clip(clip_scale);
    if (!isfinite(clip)) return;
    f32x4* m4 = reinterpret_cast<f32x4*>(m);
    f32x4* v4 = reinterpret_cast<f32x4*>(v);
    f32x4* p4 = reinterpret_cast<f32x4*>(master);
    const u32x4* g8 = reinterpret_cast<const u32x4*>(grad);
    u32x4* o8 = reinterpret_cast<u32x4*>(param);
    const int64_t n_groups = n / 8;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;

    int64_t i = tid;
    // Main loop: kUnroll groups per thread in flight, all loads issued first.
    for (; i + (kUnroll - 1) * stride < n_groups; i += kUnroll * stride) {
        Group x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) load_group(x[u], p4, m4, v4, g8, i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            u32x4 out;
            update_group(x[u], clip, c, out);
            store_group(x[u], out, p4, m4, v4, o8, i + u * stride);
        }
    }
    for (; i < n_groups; i += stride) {
        Group x;
        load_group(x, p4, m4, v4, g8, i);
        u32x4 out;
        update_group(x, clip, c, out);
        store_group(x, out, p4, m4, v4, o8, i);
    }
    const int64_t tail = n - n_groups * 8;
    if (tid < tail) scalar_elem(master, m, v, grad, param, n_groups * 8 + tid, clip, c);
}

// Fallback for pointers that are not 16-byte aligned: one element per thread.
__global__ __launch_bounds__(kThreads) void adamw_scalar(float* __restrict__ master,
                                                         float* __restrict__ m,
                                                         float* __restrict__ v,
                                                         const uint16_t* __restrict__ grad,
                                                         uint16_t* __restrict__ param, int64_t n,
                                                         AdamScalars c,
                                                         const float* __restrict__ clip_scale) {
    const float clip = read_clip(clip_scale);
    if (!isfinite(clip)) return;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n; i += stride)
        scalar_elem(master, m, v, grad, param, i, clip, c);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool ranges_overlap(const void* a, size_t a_bytes, const void* b, size_t b_bytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + b_bytes && y < x + a_bytes;
}

}  // namespace

extern "C" zero_status zero_shard_adamw_step(float* master, float* exp_avg, float* exp_avg_sq,
                                             const uint16_t* grad, uint16_t* param_out, int64_t n,
                                             int64_t step, double lr, double beta1, double beta2,
                                             double eps, double weight_decay,
                                             const float* clip_scale, hipStream_t stream) {
    using zero::fail;
    zero::clear_error();
    if (n < 0) return fail(ZERO_EINVAL, "zero_shard_adamw_step: n < 0");
    if (step < 1) return fail(ZERO_EINVAL, "zero_shard_adamw_step: step must be >= 1");
    if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0))
        return fail(ZERO_EINVAL, "zero_shard_adamw_step: betas must lie in [0, 1)");
    if (!(eps > 0.0) || !std::isfinite(eps))
        return fail(ZERO_EINVAL, "zero_shard_adamw_step: eps must be finite and > 0");
    if (!(lr >= 0.0) || !std::isfinite(lr) || !std::isfinite(weight_decay))
        return fail(ZERO_EINVAL, "zero_shard_adamw_step: lr and weight_decay must be finite, lr >= 0");
    if (n == 0) return ZERO_OK;
    if (!master || !exp_avg || !exp_avg_sq || !grad || !param_out)
        return fail(ZERO_EINVAL, "zero_shard_adamw_step: NULL array");
    const size_t fbytes = static_cast<size_t>(n) * 4, hbytes = static_cast<size_t>(n) * 2;
    if (ranges_overlap(param_out, hbytes, master, fbytes) ||
        ranges_overlap(param_out, hbytes, exp_avg, fbytes) ||
        ranges_overlap(param_out, hbytes, exp_avg_sq, fbytes))
        return fail(ZERO_EINVAL, "zero_shard_adamw_step: param_out overlaps the fp32 state");

    // Scalars in fp64, each rounded once to fp32.
    const double bc1 = 1.0 - std::pow(beta1, static_cast<double>(step));
    const double bc2 = 1.0 - std::pow(beta2, static_cast<double>(step));
    if (!(bc1 > 0.0) || !(bc2 > 0.0))
        return fail(ZERO_EINVAL, "zero_shard_adamw_step: bias correction is zero");
    AdamScalars c;
    c.beta1 = static_cast<float>(beta1);
    c.one_minus_beta1 = static_cast<float>(1.0 - beta1);
    c.beta2 = static_cast<float>(beta2);
    c.one_minus_beta2 = static_cast<float>(1.0 - beta2);
    c.eps = static_cast<float>(eps);
    c.step_size = static_cast<float>(lr / bc1);
    c.sqrt_bc2 = static_cast<float>(std::sqrt(bc2));
    c.decay = static_cast<float>(1.0 - lr * weight_decay);

    const bool vec = aligned16(master) && aligned16(exp_avg) && aligned16(exp_avg_sq) &&
                     aligned16(grad) && aligned16(param_out);
    // Persistent grid: every workgroup resident at once (occupancy x CUs, times
    // ZERO_ADAMW_OVERSUB), none idle when the work is small.
    if (vec) {
        const void* kern = reinterpret_cast<const void*>(&adamw_vec<ZERO_ADAMW_UNROLL>);
        static thread_local int cached_dev = -1, cached_blocks = 0;
        int dev = 0;
        (void)hipGetDevice(&dev);
        if (dev != cached_dev) {
            cached_blocks = zero::device_resident_blocks(kern, kThreads) * ZERO_ADAMW_OVERSUB;
            cached_dev = dev;
        }
        const int64_t groups = n / 8;
        int64_t blocks = (groups + kThreads - 1) / kThreads;
        if (blocks > cached_blocks) blocks = cached_blocks;
        if (blocks < 1) blocks = 1;
        hipLaunchKernelGGL(adamw_vec<ZERO_ADAMW_UNROLL>, dim3(static_cast<unsigned>(blocks)),
                           dim3(kThreads), 0, stream, master, exp_avg, exp_avg_sq, grad, param_out,
                           n, c, clip_scale);
    } else {
        int64_t blocks = (n + kThreads - 1) / kThreads;
        const int64_t cap = static_cast<int64_t>(zero::device_cu_count()) * 8;
        if (blocks > cap) blocks = cap;
        hipLaunchKernelGGL(adamw_scalar, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                           stream, master, exp_avg, exp_avg_sq, grad, param_out, n, c, clip_scale);
    }
    return zero::check_hip(hipGetLastError(), "zero_shard_adamw_step launch");
}

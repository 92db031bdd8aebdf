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
// vector ridge point, so no matrix cores. Each thread updates four
// consecutive elements with non-temporal accesses: one dwordx4 per fp32
// array, one dwordx2 for the bf16 gradient and one for the bf16 parameters.
// The grid covers the shard with one group per thread (up to 2^20
// workgroups, then threads stride): measured on MI355X, short-lived waves
// that the dispatcher keeps refilling sustain more HBM bandwidth than a
// persistent few-workgroups-per-CU loop. Indices are 64-bit.
#include <hip/hip_runtime.h>

#include <cmath>
#include <string>

#include "device_common.hpp"
#include "internal.hpp"

#pragma clang fp contract(off)

namespace {

using zero::dev::f32x4;
using zero::dev::u32x2;

#ifndef ZERO_ADAMW_THREADS
#define ZERO_ADAMW_THREADS 256
#endif
// Upper bound on the grid; below it every thread updates exactly one group of
// four elements (no loop), above it threads stride over the groups.
#ifndef ZERO_ADAMW_MAX_BLOCKS
#define ZERO_ADAMW_MAX_BLOCKS (1 << 20)
#endif
constexpr int kThreads = ZERO_ADAMW_THREADS;

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

// Four consecutive elements: 16-byte accesses for each fp32 array, 8-byte
// accesses for the bf16 gradient and parameters.
__device__ __forceinline__ void update4(f32x4* __restrict__ p4, f32x4* __restrict__ m4,
                                        f32x4* __restrict__ v4, const u32x2* __restrict__ g4,
                                        u32x2* __restrict__ o4, int64_t i, float clip,
                                        const AdamScalars& c) {
    f32x4 p = zero::dev::ld_stream(p4 + i);
    f32x4 m = zero::dev::ld_stream(m4 + i);
    f32x4 v = zero::dev::ld_stream(v4 + i);
    const u32x2 g = zero::dev::ld_stream(g4 + i);
    const float gs[4] = {zero::dev::lo_bf16(g.x), zero::dev::hi_bf16(g.x), zero::dev::lo_bf16(g.y),
                         zero::dev::hi_bf16(g.y)};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float pj = p[j], mj = m[j], vj = v[j];
        adam_elem(pj, mj, vj, gs[j] * clip, c);
        p[j] = pj;
        m[j] = mj;
        v[j] = vj;
    }
    zero::dev::st_stream(p4 + i, p);
    zero::dev::st_stream(m4 + i, m);
    zero::dev::st_stream(v4 + i, v);
    const u32x2 out = {zero::dev::pack_bf16(p[0], p[1]), zero::dev::pack_bf16(p[2], p[3])};
    zero::dev::st_stream(o4 + i, out);
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

// Vector path: groups [0, n/4) of four elements, then the n % 4 tail elements
// one per thread. master/m/v are 16-byte aligned, grad and param 8-byte.
__global__ __launch_bounds__(kThreads) void adamw_vec(float* __restrict__ master,
                                                      float* __restrict__ m,
                                                      float* __restrict__ v,
                                                      const uint16_t* __restrict__ grad,
                                                      uint16_t* __restrict__ param, int64_t n,
                                                      AdamScalars c,
                                                      const float* __restrict__ clip_scale) {
    const float clip = read_clip(clip_scale);
    if (!isfinite(clip)) return;
    const int64_t groups = n / 4;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    for (int64_t i = tid; i < groups; i += stride)
        update4(reinterpret_cast<f32x4*>(master), reinterpret_cast<f32x4*>(m),
                reinterpret_cast<f32x4*>(v), reinterpret_cast<const u32x2*>(grad),
                reinterpret_cast<u32x2*>(param), i, clip, c);
    const int64_t tail = n - groups * 4;
    if (tid < tail) scalar_elem(master, m, v, grad, param, groups * 4 + tid, clip, c);
}

// Fallback for pointers without that alignment: one element per thread.
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

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool ranges_overlap(const void* a, size_t a_bytes, const void* b, size_t b_bytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + b_bytes && y < x + a_bytes;
}

int64_t blocks_for(int64_t items) {
    int64_t blocks = (items + kThreads - 1) / kThreads;
    if (blocks > ZERO_ADAMW_MAX_BLOCKS) blocks = ZERO_ADAMW_MAX_BLOCKS;
    return blocks < 1 ? 1 : blocks;
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

    const bool vec = aligned(master, 16) && aligned(exp_avg, 16) && aligned(exp_avg_sq, 16) &&
                     aligned(grad, 8) && aligned(param_out, 8);
    if (vec) {
        hipLaunchKernelGGL(adamw_vec, dim3(static_cast<unsigned>(blocks_for(n / 4))), dim3(kThreads),
                           0, stream, master, exp_avg, exp_avg_sq, grad, param_out, n, c, clip_scale);
    } else {
        hipLaunchKernelGGL(adamw_scalar, dim3(static_cast<unsigned>(blocks_for(n))), dim3(kThreads),
                           0, stream, master, exp_avg, exp_avg_sq, grad, param_out, n, c, clip_scale);
    }
    return zero::check_hip(hipGetLastError(), "zero_shard_adamw_step launch");
}

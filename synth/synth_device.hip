// Seeded synthetic inputs, device side (gfx950). Bit-identical twin of
// synth_host.c: the same counter-based SplitMix64 definition, evaluated one
// element per lane. Holds none of the optimizer step's arithmetic; the product
// library never links it. Only the test harness and the benchmark call it, to
// fill multi-gigabyte input buffers without a host round trip.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ULL;

__host__ __device__ inline uint64_t mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

__host__ __device__ inline uint64_t h(uint64_t x) { return mix(x + kGamma); }

__device__ inline float value_at(uint64_t key, int64_t g, int64_t phi, double sigma) {
    if (g >= phi) return 0.0f;
    const uint64_t n = 3ULL * static_cast<uint64_t>(g);
    int64_t s = 0;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const uint64_t w = mix(key + (n + static_cast<uint64_t>(j) + 1ULL) * kGamma);
        s += static_cast<int64_t>(w & 0xFFFFu) + static_cast<int64_t>((w >> 16) & 0xFFFFu) +
             static_cast<int64_t>((w >> 32) & 0xFFFFu) + static_cast<int64_t>((w >> 48) & 0xFFFFu);
    }
    const double z = static_cast<double>(s - 393210) / 65536.0;
    return static_cast<float>(z * sigma);
}

__device__ inline uint16_t to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__global__ void fill_f32(float* __restrict__ out, int64_t n, uint64_t key, int64_t g0, int64_t phi,
                         double sigma) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        out[i] = value_at(key, g0 + i, phi, sigma);
}

__global__ void fill_bf16(uint16_t* __restrict__ out, int64_t n, uint64_t key, int64_t g0,
                          int64_t phi, double sigma) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        out[i] = to_bf16(value_at(key, g0 + i, phi, sigma));
}

uint64_t make_key(uint64_t seed, uint64_t kind, uint64_t step, uint64_t replica) {
    uint64_t k = h(seed);
    k = h(k ^ kind);
    k = h(k ^ step);
    k = h(k ^ replica);
    return k;
}

unsigned grid_for(int64_t n) {
    const int64_t blocks = (n + 255) / 256;
    return static_cast<unsigned>(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536);
}

}  // namespace

extern "C" {

// Returns 0 on success, otherwise the hipError_t of the failed launch.
int synth_device_normal_f32(float* out, int64_t n, uint64_t seed, uint64_t kind, uint64_t step,
                            uint64_t replica, int64_t g0, int64_t phi, double sigma,
                            hipStream_t stream) {
    if (n <= 0) return 0;
    if (out == nullptr) return static_cast<int>(hipErrorInvalidValue);
    hipLaunchKernelGGL(fill_f32, dim3(grid_for(n)), dim3(256), 0, stream, out, n,
                       make_key(seed, kind, step, replica), g0, phi, sigma);
    return static_cast<int>(hipGetLastError());
}

int synth_device_normal_bf16(uint16_t* out, int64_t n, uint64_t seed, uint64_t kind, uint64_t step,
                             uint64_t replica, int64_t g0, int64_t phi, double sigma,
                             hipStream_t stream) {
    if (n <= 0) return 0;
    if (out == nullptr) return static_cast<int>(hipErrorInvalidValue);
    hipLaunchKernelGGL(fill_bf16, dim3(grid_for(n)), dim3(256), 0, stream, out, n,
                       make_key(seed, kind, step, replica), g0, phi, sigma);
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"

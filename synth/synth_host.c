/*
 * Seeded synthetic inputs, host side (plain C, OpenMP over elements).
 *
 * This file holds the input generator only: it contains none of the optimizer
 * step's arithmetic. Both the CPU oracle and the GPU path receive inputs made
 * by this generator or by its device twin (synth_device.hip), which computes
 * bit-identical values; a test checks the two against each other and against
 * a pure-Python transcription of the definition below.
 *
 * Definition (counter-based, one value per global flat index g):
 *   H(x)        = splitmix64_mix(x + GAMMA)            one SplitMix64 step
 *                 (Steele, Lea, Flood, "Fast splittable pseudorandom number
 *                  generators", OOPSLA 2014: GAMMA = 0x9E3779B97F4A7C15 and the
 *                  variant-13 output mix with shifts 30/27/31)
 *   key         = H(H(H(H(seed) ^ kind) ^ step) ^ replica)
 *   word n      = H(key + n * GAMMA)                    (the n-th SplitMix64 output
 *                                                       of a generator seeded with key)
 *   element g   uses words 3g, 3g+1, 3g+2; each word gives four 16-bit fields,
 *                 s = sum of the twelve fields (an integer in [0, 786420])
 *   z           = (s - 393210) / 65536                  exact in binary64; this is the
 *                 Irwin-Hall sum of twelve midpoint uniforms minus 6 (mean 0, var ~1)
 *   x           = fp32(z * sigma)                       binary64 product, one RNE to fp32
 *   bf16 form   = RNE(x) to bfloat16, NaN never occurs here
 *   g >= phi    gives exactly 0 (padding of the flat buffer)
 */
#include <stdint.h>
#include <string.h>

#define SYN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t syn_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t syn_h(uint64_t x) { return syn_mix(x + SYN_GAMMA); }

uint64_t synth_key(uint64_t seed, uint64_t kind, uint64_t step, uint64_t replica) {
    uint64_t k = syn_h(seed);
    k = syn_h(k ^ kind);
    k = syn_h(k ^ step);
    k = syn_h(k ^ replica);
    return k;
}

static inline float syn_value(uint64_t key, int64_t g, int64_t phi, double sigma) {
    if (g >= phi) return 0.0f;
    uint64_t n = 3ULL * (uint64_t)g;
    int64_t s = 0;
    for (int j = 0; j < 3; ++j) {
        uint64_t w = syn_mix(key + (n + (uint64_t)j + 1ULL) * SYN_GAMMA);
        s += (int64_t)(w & 0xFFFFu) + (int64_t)((w >> 16) & 0xFFFFu) +
             (int64_t)((w >> 32) & 0xFFFFu) + (int64_t)((w >> 48) & 0xFFFFu);
    }
    double z = (double)(s - 393210) / 65536.0;
    return (float)(z * sigma);
}

static inline uint16_t syn_bf16(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* out[i] = value at global index g0 + i, for i in [0, n). */
void synth_normal_f32(float* out, int64_t n, uint64_t seed, uint64_t kind, uint64_t step,
                      uint64_t replica, int64_t g0, int64_t phi, double sigma) {
    uint64_t key = synth_key(seed, kind, step, replica);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = syn_value(key, g0 + i, phi, sigma);
}

void synth_normal_bf16(uint16_t* out, int64_t n, uint64_t seed, uint64_t kind, uint64_t step,
                       uint64_t replica, int64_t g0, int64_t phi, double sigma) {
    uint64_t key = synth_key(seed, kind, step, replica);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = syn_bf16(syn_value(key, g0 + i, phi, sigma));
}

/*
 * Seeded, counter-based synthetic input generator.
 *
 * This module produces the input tensors (tokens, router and expert weights,
 * per-expert logit offsets) that both the HIP path and the CPU oracle consume.
 * It holds none of the MoE layer's arithmetic: it only draws numbers.
 *
 * Definition (every element is a pure function of (seed, tensor_id, index)):
 *   mix64(z)      : the SplitMix64 output finaliser (Steele, Lea & Flood 2014),
 *                   z ^= z>>30; z *= 0xBF58476D1CE4E5B9;
 *                   z ^= z>>27; z *= 0x94D049BB133111EB; z ^= z>>31.
 *   key           = mix64(seed ^ (tensor_id * GAMMA)),  GAMMA = 0x9E3779B97F4A7C15
 *   word(i)       = mix64(key + (i + 1) * GAMMA)       (the i-th SplitMix64 output)
 *   normal pair j : u1 = ((word(2j) >> 11) + 1) * 2^-53  in (0, 1]
 *                   u2 =  (word(2j+1) >> 11)    * 2^-53  in [0, 1)
 *                   r  = sqrt(-2 ln u1)
 *                   element 2j = r cos(2 pi u2), element 2j+1 = r sin(2 pi u2)
 *                   (Box & Muller 1958), computed in double.
 *   uniform i     : u = (word(i) >> 11) * 2^-53, value = lo + (hi - lo) u.
 *   The double is scaled by sigma and rounded to float (round to nearest even);
 *   bf16 outputs then round that float to bf16 (round to nearest even).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z ^= z >> 30; z *= 0xBF58476D1CE4E5B9ULL;
    z ^= z >> 27; z *= 0x94D049BB133111EBULL;
    z ^= z >> 31;
    return z;
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tensor_id) {
    return mix64(seed ^ (tensor_id * GAMMA));
}

static inline uint64_t word_at(uint64_t key, uint64_t i) {
    return mix64(key + (i + 1) * GAMMA);
}

static inline double normal_at(uint64_t key, uint64_t idx) {
    const double two_pi = 6.283185307179586476925286766559;
    uint64_t j = idx >> 1;
    double u1 = (double)((word_at(key, 2 * j) >> 11) + 1) * 0x1.0p-53;
    double u2 = (double)(word_at(key, 2 * j + 1) >> 11) * 0x1.0p-53;
    double r = sqrt(-2.0 * log(u1));
    return (idx & 1) ? r * sin(two_pi * u2) : r * cos(two_pi * u2);
}

/* float -> bf16 bits, round to nearest even (inputs are finite here). */
static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

void gen_normal_f32(uint64_t seed, uint64_t tensor_id, uint64_t offset,
                    int64_t count, double sigma, float* out) {
    uint64_t key = stream_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        out[i] = (float)(sigma * normal_at(key, offset + (uint64_t)i));
}

void gen_normal_bf16(uint64_t seed, uint64_t tensor_id, uint64_t offset,
                     int64_t count, double sigma, uint16_t* out) {
    uint64_t key = stream_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        out[i] = f32_to_bf16_rne((float)(sigma * normal_at(key, offset + (uint64_t)i)));
}

void gen_uniform_f32(uint64_t seed, uint64_t tensor_id, uint64_t offset,
                     int64_t count, double lo, double hi, float* out) {
    uint64_t key = stream_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        double u = (double)(word_at(key, offset + (uint64_t)i) >> 11) * 0x1.0p-53;
        out[i] = (float)(lo + (hi - lo) * u);
    }
}

/* Raw 64-bit words, exposed so tests can check the generator itself. */
void gen_words(uint64_t seed, uint64_t tensor_id, uint64_t offset, int64_t count,
               uint64_t* out) {
    uint64_t key = stream_key(seed, tensor_id);
    for (int64_t i = 0; i < count; ++i) out[i] = word_at(key, offset + (uint64_t)i);
}

/* Plain SplitMix64 sequence from a given state (outputs 1..count). */
void gen_splitmix64(uint64_t state, int64_t count, uint64_t* out) {
    for (int64_t i = 0; i < count; ++i) out[i] = word_at(state, (uint64_t)i);
}

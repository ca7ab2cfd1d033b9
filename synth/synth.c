/*
 * Seeded synthetic inputs, shared by the CPU oracle tests and the GPU path.
 *
 * This module holds none of the method's arithmetic (no quantization, no
 * norm, no attention): it only draws numbers.  Every draw is counter based,
 * so any slice of any tensor can be produced on its own and the result does
 * not depend on the number of threads.
 *
 *  - splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 *    generators", OOPSLA 2014): the n-th output (n = 0, 1, ...) of the stream
 *    with key s is mix(s + (n + 1) * 0x9E3779B97F4A7C15).
 *  - uniform in (0, 1): ((z >> 11) + 0.5) * 2^-53 (the top 53 bits).
 *  - normal: Box and Muller (1958).  Element e of a tensor belongs to the
 *    pair j = e / 2, which uses outputs 2j and 2j + 1 as (u1, u2):
 *    r = sqrt(-2 ln u1), even e -> r cos(2 pi u2), odd e -> r sin(2 pi u2).
 *    The result mean + std * z is formed in double and rounded to fp32.
 *  - integers in [0, bound): z % bound.
 *
 * The stream key of a tensor is seed * 1000003 + tensor_id.
 */
#include <math.h>
#include <stdint.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t sm64_at(uint64_t key, uint64_t n) {
    return sm64_mix(key + (n + 1) * SM64_GAMMA);
}

static inline double unit_open(uint64_t z) {
    return ((double)(z >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

uint64_t synth_stream_key(uint64_t seed, uint64_t tensor_id) {
    return seed * 1000003ULL + tensor_id;
}

uint64_t synth_u64(uint64_t seed, uint64_t tensor_id, uint64_t n) {
    return sm64_at(synth_stream_key(seed, tensor_id), n);
}

/* out[i] = element (offset + i) of the N(mean, std^2) tensor (seed, tensor_id). */
void synth_normal_f32(uint64_t seed, uint64_t tensor_id, uint64_t offset, int64_t n,
                      double mean, double std, float* out) {
    if (n <= 0) return;
    const uint64_t key = synth_stream_key(seed, tensor_id);
    const double two_pi = 6.283185307179586476925286766559;
    const uint64_t first = offset, last = offset + (uint64_t)n - 1;
    const int64_t npairs = (int64_t)((last >> 1) - (first >> 1) + 1);
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npairs; ++p) {
        const uint64_t j = (first >> 1) + (uint64_t)p;
        const double u1 = unit_open(sm64_at(key, 2 * j));
        const double u2 = unit_open(sm64_at(key, 2 * j + 1));
        const double r = sqrt(-2.0 * log(u1));
        const uint64_t e0 = 2 * j, e1 = 2 * j + 1;
        if (e0 >= first && e0 <= last) out[e0 - first] = (float)(mean + std * (r * cos(two_pi * u2)));
        if (e1 >= first && e1 <= last) out[e1 - first] = (float)(mean + std * (r * sin(two_pi * u2)));
    }
}

/* out[i] = element (offset + i) of the uniform-integer tensor in [0, bound). */
void synth_uniform_i32(uint64_t seed, uint64_t tensor_id, uint64_t offset, int64_t n,
                       uint32_t bound, int32_t* out) {
    const uint64_t key = synth_stream_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = (int32_t)(sm64_at(key, offset + (uint64_t)i) % bound);
}

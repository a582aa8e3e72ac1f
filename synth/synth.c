/*
 * Seeded, counter-based synthetic input generator.
 *
 * This file holds no arithmetic of the attention method.  It only turns
 * (seed, stream id, flat element index) into a normally distributed number,
 * scaled and rounded to the requested storage type.  Both the GPU tests and
 * the oracle take their inputs from here, so the two sides see the same
 * bytes; nothing else is shared between them.
 *
 * Generator, per element i of stream (seed, id):
 *   key   = mix64(seed * 0xD1342543DE82EF95 + id * 0x9E3779B97F4A7C15 + 0x5851F42D4C957F2D)
 *   x(c)  = mix64(key + (c + 1) * 0x9E3779B97F4A7C15)
 * where mix64 is the SplitMix64 output function (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014; constants
 * as in Vigna's public-domain splitmix64.c).  Element pairs (2p, 2p+1) use
 * Box-Muller on u1 = ((x(2p) >> 11) + 1) * 2^-53 in (0, 1] and
 * u2 = (x(2p+1) >> 11) * 2^-53 in [0, 1):
 *   z(2p) = sqrt(-2 ln u1) cos(2 pi u2),  z(2p+1) = sqrt(-2 ln u1) sin(2 pi u2).
 * The stored value is scale * z computed in double, rounded to float
 * (round-to-nearest-even), and for bf16 rounded again from that float to
 * bf16 (round-to-nearest-even).
 *
 * Since each element depends only on its flat index, any contiguous slice
 * (for example one (batch, head) sequence) can be regenerated on its own.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t id) {
    return mix64(seed * 0xD1342543DE82EF95ULL + id * GOLDEN + 0x5851F42D4C957F2DULL);
}

static inline uint64_t draw(uint64_t key, uint64_t c) { return mix64(key + (c + 1) * GOLDEN); }

/* The plain SplitMix64 sequence from a seed, exposed so that a test can
 * compare mix64 with published outputs of the reference generator. */
void synth_splitmix64_sequence(uint64_t seed, int64_t count, uint64_t* out) {
    uint64_t x = seed;
    for (int64_t i = 0; i < count; ++i) {
        x += GOLDEN;
        out[i] = mix64(x);
    }
}

void synth_raw_u64(uint64_t seed, uint64_t id, int64_t start, int64_t count, uint64_t* out) {
    uint64_t key = stream_key(seed, id);
    for (int64_t i = 0; i < count; ++i) out[i] = draw(key, (uint64_t)(start + i));
}

static inline double normal_at(uint64_t key, uint64_t idx) {
    uint64_t p = idx >> 1;
    uint64_t a = draw(key, 2 * p), b = draw(key, 2 * p + 1);
    double u1 = ((double)(a >> 11) + 1.0) * 0x1.0p-53;
    double u2 = (double)(b >> 11) * 0x1.0p-53;
    double r = sqrt(-2.0 * log(u1));
    double ang = 2.0 * M_PI * u2;
    return (idx & 1) ? r * sin(ang) : r * cos(ang);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* Normal draws for flat indices [start, start + count) of stream (seed, id),
 * times scale.  dtype 0 writes float, 1 writes bf16 (uint16 bit patterns),
 * 2 writes double (the unrounded scaled value).  Threaded with OpenMP. */
void synth_normal(uint64_t seed, uint64_t id, int64_t start, int64_t count, double scale, int dtype,
                  void* out) {
    uint64_t key = stream_key(seed, id);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        double z = scale * normal_at(key, (uint64_t)(start + i));
        if (dtype == 2) {
            ((double*)out)[i] = z;
        } else {
            float f = (float)z;
            if (dtype == 0)
                ((float*)out)[i] = f;
            else
                ((uint16_t*)out)[i] = f32_to_bf16_rne(f);
        }
    }
}

/* Round float values to bf16 bit patterns (round-to-nearest-even). */
void synth_f32_to_bf16(const float* in, int64_t count, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) out[i] = f32_to_bf16_rne(in[i]);
}

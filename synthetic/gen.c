/*
 * gen.c -- seeded synthetic bfloat16 inputs (the bulk path of the synthetic module).
 *
 * Draws numbers only; holds none of the FP8 method's arithmetic.  The definition is the one
 * stated in synthetic/__init__.py: SplitMix64 words (Steele, Lea, Flood, OOPSLA 2014) as a
 * counter-based stream, uniforms from the top 53 bits, Box-Muller in float64 on word pairs
 * (2j, 2j+1), float64 -> float32 -> bfloat16 with round-to-nearest-even at both steps.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static uint64_t sm64(uint64_t seed, uint64_t i)
{
    uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ULL;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static double unif(uint64_t seed, uint64_t i) { return (double)(sm64(seed, i) >> 11) * (1.0 / 9007199254740992.0); }

static uint16_t f64_to_bf16(double v)
{
    float f = (float)v;
    uint32_t b;
    memcpy(&b, &f, 4);
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

/* The float64 normal sample at element index e of stream seed (standard deviation 1). */
double synth_normal_at(uint64_t seed, int64_t e)
{
    uint64_t p = (uint64_t)e >> 1;
    double u0 = unif(seed, 2 * p), u1 = unif(seed, 2 * p + 1);
    double r = sqrt(-2.0 * log1p(-u0)), t = 6.283185307179586 * u1;
    return (e & 1) ? r * sin(t) : r * cos(t);
}

/* out[i] = bf16(std * z_(start+i)) for i in [0, n); start must be even. */
void synth_normal_bf16(uint64_t seed, int64_t start, int64_t n, double std, uint16_t *out)
{
    int64_t p0 = start >> 1;
    for (int64_t p = 0; 2 * p < n; ++p) {
        double u0 = unif(seed, 2 * (p0 + p)), u1 = unif(seed, 2 * (p0 + p) + 1);
        double r = sqrt(-2.0 * log1p(-u0)), t = 6.283185307179586 * u1;
        out[2 * p] = f64_to_bf16(std * r * cos(t));
        if (2 * p + 1 < n) out[2 * p + 1] = f64_to_bf16(std * r * sin(t));
    }
}

/* out[pos[j]] = bf16(std * factor * z_pos[j]) for the k given element indices. */
void synth_scale_at(uint64_t seed, const int64_t *pos, int64_t k, double std, double factor, uint16_t *out)
{
    for (int64_t j = 0; j < k; ++j) out[pos[j]] = f64_to_bf16(std * synth_normal_at(seed, pos[j]) * factor);
}

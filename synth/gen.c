/*
 * Seeded synthetic inputs for the shard-step workloads (host side).
 *
 * This module holds no arithmetic of the optimizer step.  It produces the
 * inputs that both the CPU oracle and the GPU library consume: per-rank
 * gradient partials (bf16 or fp32), fp32 master weights, and the index map
 * used to spread a warm-started optimizer-state prefix over a whole shard.
 * Its device twin (fill.hip in this directory) must give the same bits for
 * the same (seed, stream, index); a GPU test checks that.
 *
 * Definition (every value is a pure function of seed, stream and index):
 *   mix64(z)       : the splitmix64 finaliser (Steele, Lea, Flood, "Fast
 *                    splittable pseudorandom number generators", OOPSLA 2014;
 *                    constants as published by S. Vigna).
 *   key(seed, st)  = mix64(seed ^ mix64(st + GOLDEN))
 *   bits(key, c)   = mix64(key + c * GOLDEN)            (counter c)
 *   unif(key, c)   = (bits >> 40) * 2^-24                (exact in fp32)
 *   normal(i)      = ((u0 + u1) + (u2 + u3) - 2) * scale (fp32 ops, this order)
 *                    with uj = unif(key, 4 i + j): Irwin-Hall(4), variance 1/3,
 *                    so scale = (float)(sqrt(3) * sigma) gives std sigma.
 *   outlier        : if unif(mask_key, i) < frac then value *= mult (fp32).
 *   bf16           : round-to-nearest-even of the fp32 value (no NaN occurs).
 *
 * Built with gcc -O2 -ffp-contract=off; float arithmetic on x86-64 is SSE
 * single precision with round-to-nearest-even, so each op is IEEE-exact.
 */
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z)
{
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z;
}

uint64_t synth_key(uint64_t seed, uint64_t stream)
{
    return mix64(seed ^ mix64(stream + GOLDEN));
}

static inline float unif(uint64_t key, uint64_t c)
{
    uint64_t b = mix64(key + c * GOLDEN);
    return (float)(b >> 40) * 0x1p-24f;
}

static inline float normal_at(uint64_t key, uint64_t i, float scale)
{
    float u0 = unif(key, 4 * i + 0);
    float u1 = unif(key, 4 * i + 1);
    float u2 = unif(key, 4 * i + 2);
    float u3 = unif(key, 4 * i + 3);
    float s = (u0 + u1) + (u2 + u3);
    return (s - 2.0f) * scale;
}

static inline float value_at(uint64_t key, uint64_t mkey, uint64_t i, float scale,
                             float frac, float mult)
{
    float x = normal_at(key, i, scale);
    if (frac > 0.0f && unif(mkey, i) < frac)
        x = x * mult;
    return x;
}

static inline uint16_t to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* out[j] = value at index start + j, fp32. */
void synth_fill_f32(float *out, uint64_t seed, uint64_t stream, int64_t start,
                    int64_t count, float scale, uint64_t mask_stream, float frac,
                    float mult)
{
    uint64_t key = synth_key(seed, stream), mkey = synth_key(seed, mask_stream);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < count; ++j)
        out[j] = value_at(key, mkey, (uint64_t)(start + j), scale, frac, mult);
}

/* out[j] = bf16 bits of the value at index start + j. */
void synth_fill_bf16(uint16_t *out, uint64_t seed, uint64_t stream, int64_t start,
                     int64_t count, float scale, uint64_t mask_stream, float frac,
                     float mult)
{
    uint64_t key = synth_key(seed, stream), mkey = synth_key(seed, mask_stream);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < count; ++j)
        out[j] = to_bf16(value_at(key, mkey, (uint64_t)(start + j), scale, frac, mult));
}

/* Same values at an arbitrary list of indices (sampled parity checks). */
void synth_gather_f32(float *out, uint64_t seed, uint64_t stream, const int64_t *idx,
                      int64_t count, float scale, uint64_t mask_stream, float frac,
                      float mult)
{
    uint64_t key = synth_key(seed, stream), mkey = synth_key(seed, mask_stream);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < count; ++j)
        out[j] = value_at(key, mkey, (uint64_t)idx[j], scale, frac, mult);
}

void synth_gather_bf16(uint16_t *out, uint64_t seed, uint64_t stream, const int64_t *idx,
                       int64_t count, float scale, uint64_t mask_stream, float frac,
                       float mult)
{
    uint64_t key = synth_key(seed, stream), mkey = synth_key(seed, mask_stream);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < count; ++j)
        out[j] = to_bf16(value_at(key, mkey, (uint64_t)idx[j], scale, frac, mult));
}

/*
 * Warm-start spreading: element i >= plen of a shard takes its optimizer
 * state from prefix element src(i) = bits(key, i) mod plen; elements below
 * plen keep their own.  out[j] = src(idx[j]).
 */
void synth_prefix_src(int64_t *out, uint64_t seed, uint64_t stream, const int64_t *idx,
                      int64_t count, int64_t plen)
{
    uint64_t key = synth_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < count; ++j) {
        uint64_t i = (uint64_t)idx[j];
        out[j] = (i < (uint64_t)plen) ? (int64_t)i
                                      : (int64_t)(mix64(key + i * GOLDEN) % (uint64_t)plen);
    }
}

/* out[j] = unif(key(seed, stream), idx[j]): plain uniforms for shape recipes. */
void synth_uniform(float *out, uint64_t seed, uint64_t stream, const int64_t *idx,
                   int64_t count)
{
    uint64_t key = synth_key(seed, stream);
    for (int64_t j = 0; j < count; ++j)
        out[j] = unif(key, (uint64_t)idx[j]);
}

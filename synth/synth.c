/*
 * synth.c - seeded synthetic inputs for the routed-expert layer step.
 *
 * This module only draws numbers. It holds none of the layer's arithmetic
 * (no routing, no dequantisation, no matmul) and is the one piece of code that
 * both the CPU oracle and the GPU library's callers use: the oracle reads the
 * arrays it writes, and the same arrays are packed and copied to the GPU.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014), used as a counter-based generator. A
 * stream is named by a 64-bit key; draw i of the stream is the SplitMix64
 * output after i+1 increments of the state, starting from the key, so any
 * element can be computed without the ones before it.
 *
 *   uniform u in [0,1)  : top 24 bits of a draw times 2^-24
 *   normal              : Box-Muller in double from draws 2i and 2i+1
 *   int4 / int8 weights : the raw little-endian bytes of consecutive draws.
 *                         Every nibble (byte) is uniform over its 16 (256)
 *                         two's-complement codes, i.e. uniform on [-8,7]
 *                         ([-128,127]).
 *
 * The canonical expert block (one contiguous block per expert, the three
 * matrices stored next to each other as the Colibri pages describe):
 *   gate_q [f][d] , up_q [f][d] , down_q [d][f]   packed codes
 *        int4: two's-complement nibbles, element 2i in the low nibble of byte i
 *        int8: one two's-complement byte per element
 *   gate_s [f][d/G], up_s [f][d/G], down_s [d][f/G]  float32 scales
 *        group G along the input dimension; G == 0 means one scale per row.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* draw i of the stream keyed by `key` */
static inline uint64_t draw(uint64_t key, uint64_t i)
{
    return mix64(key + (i + 1) * GOLDEN);
}

uint64_t synth_key(uint64_t seed, uint64_t cfg, uint64_t layer, uint64_t tensor,
                   uint64_t index, uint64_t attempt)
{
    uint64_t fields[5] = {cfg, layer, tensor, index, attempt};
    uint64_t k = mix64(seed + GOLDEN);
    for (int i = 0; i < 5; ++i)
        k = mix64(k ^ (fields[i] + (uint64_t)(i + 1) * GOLDEN));
    return k;
}

uint64_t synth_draw(uint64_t key, uint64_t i) { return draw(key, i); }

void synth_fill_bytes(uint64_t key, uint8_t *out, size_t n)
{
    size_t nw = n / 8;
#pragma omp parallel for schedule(static)
    for (size_t w = 0; w < nw; ++w) {
        uint64_t z = draw(key, w);
        memcpy(out + 8 * w, &z, 8); /* little-endian hosts only (x86-64) */
    }
    if (n % 8) {
        uint64_t z = draw(key, nw);
        memcpy(out + 8 * nw, &z, n % 8);
    }
}

static inline double unit24(uint64_t z) { return (double)(z >> 40) * (1.0 / 16777216.0); }

void synth_fill_uniform(uint64_t key, float *out, size_t n, double lo, double hi)
{
#pragma omp parallel for schedule(static)
    for (size_t i = 0; i < n; ++i)
        out[i] = (float)(lo + (hi - lo) * unit24(draw(key, i)));
}

void synth_fill_normal(uint64_t key, float *out, size_t n, double mean, double stdev)
{
    const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
    for (size_t i = 0; i < n; ++i) {
        double u1 = ((double)(draw(key, 2 * i) >> 11) + 1.0) * (1.0 / 9007199254740992.0);
        double u2 = (double)(draw(key, 2 * i + 1) >> 11) * (1.0 / 9007199254740992.0);
        double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
        out[i] = (float)(mean + stdev * z);
    }
}

/* Fisher-Yates shuffle of 0..n-1 driven by the stream */
void synth_permutation(uint64_t key, int32_t *perm, int n)
{
    for (int i = 0; i < n; ++i) perm[i] = i;
    for (int i = n - 1; i > 0; --i) {
        uint64_t j = ((draw(key, (uint64_t)i) >> 32) * (uint64_t)(i + 1)) >> 32;
        int32_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
    }
}

/* tensor tags of the stream keys */
enum { T_X = 1, T_WR = 2, T_BIAS = 3, T_GATE_Q = 4, T_UP_Q = 5, T_DOWN_Q = 6,
       T_GATE_S = 7, T_UP_S = 8, T_DOWN_S = 9 };

size_t synth_block_bytes(int d, int f, int wbits, int group)
{
    size_t q = (size_t)d * f * wbits / 8;
    size_t ns_gu = group ? (size_t)f * (d / group) : (size_t)f;
    size_t ns_dn = group ? (size_t)d * (f / group) : (size_t)d;
    return 3 * q + 4 * (2 * ns_gu + ns_dn);
}

/* Writes the canonical block of expert `expert` of layer `layer` (the shared
 * expert uses expert = n_experts). Scales are uniform on [slo, shi). */
void synth_expert_block(uint64_t seed, uint64_t cfg, uint64_t layer, uint64_t expert,
                        int d, int f, int wbits, int group, double slo, double shi,
                        uint8_t *block)
{
    size_t q = (size_t)d * f * wbits / 8;
    size_t ns_gu = group ? (size_t)f * (d / group) : (size_t)f;
    size_t ns_dn = group ? (size_t)d * (f / group) : (size_t)d;
    uint8_t *gq = block, *uq = block + q, *dq = block + 2 * q;
    float *gs = (float *)(block + 3 * q);
    float *us = gs + ns_gu;
    float *ds = us + ns_gu;
    synth_fill_bytes(synth_key(seed, cfg, layer, T_GATE_Q, expert, 0), gq, q);
    synth_fill_bytes(synth_key(seed, cfg, layer, T_UP_Q, expert, 0), uq, q);
    synth_fill_bytes(synth_key(seed, cfg, layer, T_DOWN_Q, expert, 0), dq, q);
    synth_fill_uniform(synth_key(seed, cfg, layer, T_GATE_S, expert, 0), gs, ns_gu, slo, shi);
    synth_fill_uniform(synth_key(seed, cfg, layer, T_UP_S, expert, 0), us, ns_gu, slo, shi);
    synth_fill_uniform(synth_key(seed, cfg, layer, T_DOWN_S, expert, 0), ds, ns_dn, slo, shi);
}

/* n_blocks consecutive experts first..first+n_blocks-1, `stride` bytes apart */
void synth_expert_pool(uint64_t seed, uint64_t cfg, uint64_t layer, uint64_t first, int n_blocks,
                       int d, int f, int wbits, int group, double slo, double shi,
                       uint8_t *out, size_t stride)
{
    for (int e = 0; e < n_blocks; ++e)
        synth_expert_block(seed, cfg, layer, first + (uint64_t)e, d, f, wbits, group, slo, shi,
                           out + (size_t)e * stride);
}

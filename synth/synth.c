/*
 * synth.c -- seeded synthetic inputs for the balanced expert-parallel path.
 *
 * This module only draws inputs: router choices (top-K expert ids), gate
 * weights, bf16 activations and fp32 gradients.  It holds none of the
 * arithmetic of the method itself (no counts, no maxvio, no plan), so that
 * the CPU oracle and the GPU library can both consume its bytes without
 * sharing any of their own code.
 *
 * Random numbers: every stream is a SplitMix64 counter generator (Steele,
 * Lea, Flood, "Fast splittable pseudorandom number generators", OOPSLA
 * 2014).  Element i of a stream with key k is mix64(k + (i + 1) * GAMMA), so
 * any element can be drawn on its own and threads never change the result.
 * Uniforms take the top 53 bits; normals use the Box-Muller transform on the
 * pair (2p, 2p + 1).
 *
 * Routing: expert popularity follows a Zipf law over a seeded permutation of
 * the experts; each token draws K distinct experts one after another,
 * without replacement, from the remaining popularity mass.  A balanced
 * routing and a fixed adversarial routing are also provided.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Stream key: the first SplitMix64 output for `seed`, xor a stream tag. */
uint64_t synth_key(uint64_t seed, uint64_t tag)
{
    return mix64(seed + GAMMA) ^ tag;
}

static inline uint64_t draw_u64(uint64_t key, uint64_t i)
{
    return mix64(key + (i + 1ULL) * GAMMA);
}

static inline double draw_unit(uint64_t key, uint64_t i)
{
    return (double)(draw_u64(key, i) >> 11) * (1.0 / 9007199254740992.0);
}

static inline double draw_normal(uint64_t key, uint64_t i)
{
    const uint64_t p = i >> 1;
    const double u1 = draw_unit(key, 2 * p);
    const double u2 = draw_unit(key, 2 * p + 1);
    const double r = sqrt(-2.0 * log(1.0 - u1)); /* 1 - u1 lies in (0, 1] */
    const double t = 6.283185307179586 * u2;
    return (i & 1) ? r * sin(t) : r * cos(t);
}

/* float -> bf16 bits, round to nearest even (inputs are finite). */
static inline uint16_t f32_to_bf16(float f)
{
    uint32_t b;
    memcpy(&b, &f, 4);
    if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu))
        return (uint16_t)((b >> 16) | 0x0040u);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

void synth_u64(uint64_t key, uint64_t start, int64_t n, uint64_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = draw_u64(key, start + (uint64_t)i);
}

void synth_uniform(uint64_t key, uint64_t start, int64_t n, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = draw_unit(key, start + (uint64_t)i);
}

void synth_normal_f64(uint64_t key, uint64_t start, int64_t n, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = draw_normal(key, start + (uint64_t)i);
}

/* N(0, std^2) rounded to fp32. */
void synth_normal_f32(uint64_t key, uint64_t start, int64_t n, double std, float *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)(std * draw_normal(key, start + (uint64_t)i));
}

/* N(0, 1) rounded to fp32, then to bf16. */
void synth_normal_bf16(uint64_t key, uint64_t start, int64_t n, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_bf16((float)draw_normal(key, start + (uint64_t)i));
}

/* Fisher-Yates shuffle of 0..E-1; rank_of[e] is expert e's popularity rank. */
void synth_permutation(uint64_t key, int32_t E, int32_t *rank_of)
{
    for (int32_t e = 0; e < E; ++e)
        rank_of[e] = e;
    for (int32_t i = E - 1; i >= 1; --i) {
        const double u = draw_unit(key, (uint64_t)(E - 1 - i));
        int32_t j = (int32_t)floor(u * (double)(i + 1));
        if (j > i)
            j = i;
        const int32_t t = rank_of[i];
        rank_of[i] = rank_of[j];
        rank_of[j] = t;
    }
}

/*
 * Zipf routing.  Token n (0 <= n < N) draws K distinct experts for k = 0..K-1
 * with u = U(route, n*K + k): scanning the not-yet-chosen popularity ranks q
 * ascending with weights (q+1)^-alpha, it takes the first q whose running
 * weight exceeds u times the remaining weight (the last remaining rank if
 * rounding leaves none).  topk[n*K + k] = the expert whose rank is q.
 * Returns 0, or -1 if K > E or E > 65536.
 */
int synth_zipf_topk(uint64_t seed, int64_t N, int32_t E, int32_t K, double alpha, int32_t *topk)
{
    if (K > E || E > 65536 || K < 1)
        return -1;
    int32_t *rank_of = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    int32_t *expert_of = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    double *w = (double *)malloc(sizeof(double) * (size_t)E);
    synth_permutation(synth_key(seed, 1), E, rank_of);
    for (int32_t e = 0; e < E; ++e)
        expert_of[rank_of[e]] = e;
    for (int32_t q = 0; q < E; ++q)
        w[q] = pow((double)(q + 1), -alpha);
    const uint64_t rkey = synth_key(seed, 2);
#pragma omp parallel
    {
        unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
        int32_t *picked = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            for (int32_t k = 0; k < K; ++k) {
                const double u = draw_unit(rkey, (uint64_t)(n * K + k));
                double wrem = 0.0;
                int32_t last = -1;
                for (int32_t q = 0; q < E; ++q)
                    if (!taken[q]) {
                        wrem += w[q];
                        last = q;
                    }
                const double target = u * wrem;
                double cum = 0.0;
                int32_t pick = last;
                for (int32_t q = 0; q < E; ++q) {
                    if (taken[q])
                        continue;
                    cum += w[q];
                    if (cum > target) {
                        pick = q;
                        break;
                    }
                }
                taken[pick] = 1;
                picked[k] = pick;
                topk[n * K + k] = expert_of[pick];
            }
            for (int32_t k = 0; k < K; ++k)
                taken[picked[k]] = 0;
        }
        free(taken);
        free(picked);
    }
    free(rank_of);
    free(expert_of);
    free(w);
    return 0;
}

/* Balanced routing: topk[n*K + k] = (n + k*(E/K)) mod E.  Needs E % K == 0. */
int synth_balanced_topk(int64_t N, int32_t E, int32_t K, int32_t *topk)
{
    if (K < 1 || K > E || E % K != 0)
        return -1;
    const int64_t stride = E / K;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int32_t k = 0; k < K; ++k)
            topk[n * K + k] = (int32_t)((n + (int64_t)k * stride) % E);
    return 0;
}

/* Every token routes to experts 0..K-1 in order: topk[n*K + k] = k. */
void synth_fixed_topk(int64_t N, int32_t K, int32_t *topk)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int32_t k = 0; k < K; ++k)
            topk[n * K + k] = k;
}

/*
 * Router gate weights: logits l = N(0,1) from stream `logit` at element
 * n*K + k, rounded to fp32; gates are their softmax over k, in double,
 * rounded to fp32.
 */
void synth_softmax_gates(uint64_t seed, int64_t N, int32_t K, float *gates)
{
    const uint64_t key = synth_key(seed, 3);
#pragma omp parallel
    {
        double *l = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            double m = -INFINITY;
            for (int32_t k = 0; k < K; ++k) {
                l[k] = (double)(float)draw_normal(key, (uint64_t)(n * K + k));
                if (l[k] > m)
                    m = l[k];
            }
            double s = 0.0;
            for (int32_t k = 0; k < K; ++k) {
                l[k] = exp(l[k] - m);
                s += l[k];
            }
            for (int32_t k = 0; k < K; ++k)
                gates[n * K + k] = (float)(l[k] / s);
        }
        free(l);
    }
}

void synth_fill_f32(int64_t n, float v, float *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = v;
}

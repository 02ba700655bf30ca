/*
 * Seeded synthetic input generator.
 *
 * This module produces the random inputs (weights, hidden states, router
 * logits, routing traces) that both the CPU oracle and the GPU library are
 * fed. It holds none of the MoE layer's arithmetic: no quantisation, no
 * routing, no packing. Both sides receive the very same host arrays.
 *
 * Generator: SplitMix64 (G. L. Steele, D. Lea, C. H. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: the n-th output of a stream with key K is mix(K + (n+1)*GAMMA),
 * which is exactly SplitMix64's output sequence started from state K. Every
 * element is therefore a pure function of (seed, stream, index) and any range
 * of a stream can be generated independently and in parallel.
 *
 * Normals: Box-Muller transform (G. E. P. Box, M. E. Muller, 1958) in double
 * precision, element 2i from the cosine branch and 2i+1 from the sine branch
 * of pair i, rounded to float at the end.
 * Gumbel(0,1): -ln(-ln U) with U in (0,1).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SM_GAMMA 0x9e3779b97f4a7c15ULL

static inline uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

/* Key of stream `stream` under `seed`. */
uint64_t synth_stream_key(uint64_t seed, uint64_t stream) {
  return sm_mix(sm_mix(seed + SM_GAMMA) ^ sm_mix(stream * 0xd1b54a32d192ed03ULL + SM_GAMMA));
}

/* n-th raw 64-bit output of the stream with key `key`. */
static inline uint64_t sm_at(uint64_t key, uint64_t n) { return sm_mix(key + (n + 1) * SM_GAMMA); }

/* uniform in (0, 1]: 53 random bits, +1 so that log() never sees 0 */
static inline double u_open0(uint64_t r) { return ((double)(r >> 11) + 1.0) * 0x1.0p-53; }
/* uniform in [0, 1) */
static inline double u_closed0(uint64_t r) { return (double)(r >> 11) * 0x1.0p-53; }

uint64_t synth_u64_at(uint64_t seed, uint64_t stream, uint64_t n) {
  return sm_at(synth_stream_key(seed, stream), n);
}

/* out[i] = mean + std * N_i for i in [0, n); N_i standard normal. */
void synth_normal_f32(uint64_t seed, uint64_t stream, int64_t n, double mean, double std, float *out) {
  const uint64_t key = synth_stream_key(seed, stream);
  const int64_t npairs = (n + 1) / 2;
  const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < npairs; ++p) {
    double u1 = u_open0(sm_at(key, 2 * (uint64_t)p));
    double u2 = u_closed0(sm_at(key, 2 * (uint64_t)p + 1));
    double rad = sqrt(-2.0 * log(u1));
    double ang = two_pi * u2;
    int64_t i = 2 * p;
    out[i] = (float)(mean + std * rad * cos(ang));
    if (i + 1 < n) out[i + 1] = (float)(mean + std * rad * sin(ang));
  }
}

/* out[i] uniform in (0, 1], double */
void synth_uniform_f64(uint64_t seed, uint64_t stream, int64_t n, double *out) {
  const uint64_t key = synth_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = u_open0(sm_at(key, (uint64_t)i));
}

/* out[i] ~ Gumbel(0, 1) */
void synth_gumbel_f64(uint64_t seed, uint64_t stream, int64_t n, double *out) {
  const uint64_t key = synth_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double u = u_open0(sm_at(key, (uint64_t)i));
    if (u >= 1.0) u = 1.0 - 0x1.0p-53; /* keep -ln(u) > 0 */
    out[i] = -log(-log(u));
  }
}

/* Seeded permutation of [0, n) (Fisher-Yates, Durstenfeld's variant). */
void synth_permutation(uint64_t seed, uint64_t stream, int32_t n, int32_t *perm) {
  const uint64_t key = synth_stream_key(seed, stream);
  for (int32_t i = 0; i < n; ++i) perm[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    /* unbiased enough for n << 2^32: 64-bit multiply-shift range reduction */
    uint64_t r = sm_at(key, (uint64_t)(n - 1 - i));
    int32_t j = (int32_t)(((unsigned __int128)r * (uint64_t)(i + 1)) >> 64);
    int32_t t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
}

/*
 * Router logits with Zipf-distributed expert popularity.
 * Expert e has popularity rank rank_of[e] in 1..E and probability
 * p_r = r^-s / sum_q q^-s. z[t][e] = ln p_{rank_of[e]} + Gumbel. Taking the
 * top-k of z per token samples k experts without replacement from p
 * (the Gumbel-top-k construction), so expert popularity follows Zipf(s).
 */
void synth_zipf_logits(uint64_t seed, uint64_t stream, int32_t T, int32_t E, double s, const int32_t *rank_of,
                       float *z) {
  double *lp = (double *)malloc(sizeof(double) * (size_t)E);
  double norm = 0.0;
  for (int32_t r = 1; r <= E; ++r) norm += pow((double)r, -s);
  for (int32_t e = 0; e < E; ++e) lp[e] = -s * log((double)rank_of[e]) - log(norm);
  const uint64_t key = synth_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)T * E; ++i) {
    double u = u_open0(sm_at(key, (uint64_t)i));
    if (u >= 1.0) u = 1.0 - 0x1.0p-53;
    z[i] = (float)(lp[i % E] - log(-log(u)));
  }
  free(lp);
}

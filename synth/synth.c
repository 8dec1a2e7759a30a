/*
 * Seeded synthetic inputs for the MoE layout / dispatch / combine path.
 *
 * This library only draws random numbers. It holds none of the arithmetic of
 * the method under test (no counting, no offsets, no permutation, no weighted
 * sum); both the CPU oracle and the GPU path receive the arrays it writes.
 *
 * Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014). Its i-th output for a start state `key` is
 * mix64(key + (i + 1) * gamma), so every draw is addressed by a counter and
 * any element range can be produced independently, in any order, on any
 * number of threads, with identical bits.
 *
 * Derived draws:
 *   uniform double in [0,1)  : (z >> 11) * 2^-53
 *   uniform double in (0,1)  : ((z >> 11) + 0.5) * 2^-53
 *   integer in [0,n)         : Lemire, "Fast random integer generation in an
 *                              interval", ACM TOMACS 2019 (multiply-shift with
 *                              rejection, unbiased)
 *   standard normal          : Box & Muller 1958; pair j uses draws 2j, 2j+1
 *   bf16 input values        : fp32 normal rounded to nearest-even bf16
 *   distinct top-k (uniform) : partial Fisher-Yates over [0,E), kept in draw order
 *   top-k Zipf(s) w/o repl.  : Efraimidis & Spirakis 2006 keys log(u)/p, K largest,
 *                              in descending key order
 *   routing weights          : softmax (in double) of standard-normal logits
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* i-th output of SplitMix64 started at state `key`. */
static inline uint64_t sm64(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * SM64_GAMMA); }

static inline double u01(uint64_t z) { return (double)(z >> 11) * 0x1.0p-53; }
static inline double u01_open(uint64_t z) { return ((double)(z >> 11) + 0.5) * 0x1.0p-53; }

uint64_t synth_splitmix64(uint64_t key, uint64_t i) { return sm64(key, i); }

/* Key of one independent stream: (seed, salt, stream id) -> start state. */
uint64_t synth_stream_key(uint64_t seed, uint64_t salt, uint64_t stream) {
    return sm64(sm64(seed, salt), stream);
}

/* Element i of the standard-normal sequence of stream `key`. */
static inline double normal_at(uint64_t key, uint64_t i) {
    uint64_t j = i >> 1;
    double u1 = u01_open(sm64(key, 2 * j));
    double u2 = u01(sm64(key, 2 * j + 1));
    double r = sqrt(-2.0 * log(u1));
    double a = 6.283185307179586476925286766559 * u2;
    return (i & 1) ? r * sin(a) : r * cos(a);
}

/* Nearest-even bf16 of a finite fp32 value (input synthesis only). */
static inline uint16_t f32_to_bf16_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

void synth_normal_f64(uint64_t key, int64_t offset, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = normal_at(key, (uint64_t)(offset + i));
}

void synth_normal_bf16(uint64_t key, int64_t offset, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_bits((float)normal_at(key, (uint64_t)(offset + i)));
}

/* Lemire's unbiased bounded integer; *ctr walks the token's own draw sequence. */
static inline uint32_t bounded(uint64_t key, uint64_t* ctr, uint32_t n) {
    uint64_t z = sm64(key, (*ctr)++);
    unsigned __int128 m = (unsigned __int128)z * n;
    uint64_t l = (uint64_t)m;
    if (l < n) {
        uint64_t t = (0 - (uint64_t)n) % n;
        while (l < t) {
            z = sm64(key, (*ctr)++);
            m = (unsigned __int128)z * n;
            l = (uint64_t)m;
        }
    }
    return (uint32_t)(m >> 64);
}

/* Uniform distinct top-k: per token, a partial Fisher-Yates shuffle of
 * [0,E); the first K positions, in draw order, are the token's experts. */
int synth_topk_uniform(uint64_t key, int64_t T, int K, int E, int64_t* out) {
    if (T < 0 || K < 1 || E < 1 || K > E) return -1;
#pragma omp parallel
    {
        int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            uint64_t tk = sm64(key, (uint64_t)t);
            uint64_t ctr = 0;
            for (int e = 0; e < E; ++e) perm[e] = e;
            for (int k = 0; k < K; ++k) {
                int j = k + (int)bounded(tk, &ctr, (uint32_t)(E - k));
                int32_t tmp = perm[k];
                perm[k] = perm[j];
                perm[j] = tmp;
                out[t * K + k] = perm[k];
            }
        }
        free(perm);
    }
    return 0;
}

/* Seeded permutation of [0,E) (Fisher-Yates, Durstenfeld form). */
int synth_permutation(uint64_t key, int E, int32_t* out) {
    if (E < 1) return -1;
    uint64_t ctr = 0;
    for (int e = 0; e < E; ++e) out[e] = e;
    for (int i = E - 1; i > 0; --i) {
        int j = (int)bounded(key, &ctr, (uint32_t)(i + 1));
        int32_t tmp = out[i];
        out[i] = out[j];
        out[j] = tmp;
    }
    return 0;
}

/* Zipf(s) popularity over a seeded permutation, K draws without replacement
 * per token. Popularity rank i (1-based) has p_i = i^-s / sum_j j^-s and maps
 * to expert perm[i-1]. Each token draws u_i in (0,1) per rank and keeps the K
 * largest keys log(u_i)/p_i (Efraimidis-Spirakis), which is successive
 * sampling without replacement; ties go to the smaller expert id. Slots are
 * written in descending key order. */
int synth_topk_zipf(uint64_t key_perm, uint64_t key_draw, int64_t T, int K, int E, double s, int64_t* out) {
    if (T < 0 || K < 1 || E < 1 || K > E) return -1;
    int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
    synth_permutation(key_perm, E, perm);
    double z = 0.0;
    for (int i = 1; i <= E; ++i) z += pow((double)i, -s);
    for (int i = 1; i <= E; ++i) p[i - 1] = pow((double)i, -s) / z;
#pragma omp parallel
    {
        double* kv = (double*)malloc(sizeof(double) * (size_t)K);
        int32_t* ke = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            uint64_t tk = sm64(key_draw, (uint64_t)t);
            int n = 0; /* kept entries, sorted by (key desc, expert asc) */
            for (int i = 0; i < E; ++i) {
                double key = log(u01_open(sm64(tk, (uint64_t)i))) / p[i];
                int32_t e = perm[i];
                /* does (key, e) rank above the current last kept entry? */
                int pos = n;
                while (pos > 0 && (key > kv[pos - 1] || (key == kv[pos - 1] && e < ke[pos - 1]))) --pos;
                if (pos >= K) continue;
                int last = (n < K) ? n : K - 1;
                for (int q = last; q > pos; --q) { kv[q] = kv[q - 1]; ke[q] = ke[q - 1]; }
                kv[pos] = key;
                ke[pos] = e;
                if (n < K) ++n;
            }
            for (int k = 0; k < K; ++k) out[t * K + k] = ke[k];
        }
        free(kv);
        free(ke);
    }
    free(perm);
    free(p);
    return 0;
}

/* Routing weights: softmax over the K slots of standard-normal logits
 * (logit of slot (t,k) is element t*K+k of the stream), in double, stored fp32. */
void synth_softmax_weights(uint64_t key, int64_t T, int K, float* out) {
#pragma omp parallel
    {
        double* l = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            double m = -INFINITY, s = 0.0;
            for (int k = 0; k < K; ++k) {
                l[k] = normal_at(key, (uint64_t)(t * K + k));
                if (l[k] > m) m = l[k];
            }
            for (int k = 0; k < K; ++k) {
                l[k] = exp(l[k] - m);
                s += l[k];
            }
            for (int k = 0; k < K; ++k) out[t * K + k] = (float)(l[k] / s);
        }
        free(l);
    }
}

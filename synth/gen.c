/*
 * gen.c -- seeded, counter-based synthetic input generator.
 *
 * This module holds no arithmetic of the attention method. It only draws
 * numbers: the tensors it writes are handed unchanged to both the GPU
 * library and the CPU oracle, so the two always see identical inputs.
 *
 * Definition (one normal deviate per element, independent of threading):
 *   key(seed, stream) = splitmix64(splitmix64(seed) ^ (stream * 0xD1B54A32D192ED03))
 *   elements 2i and 2i+1 form one Box-Muller pair:
 *                   a = splitmix64(key + 2i), b = splitmix64(key + 2i + 1)
 *                   u1 = ((a >> 11) + 1) * 2^-53        in (0, 1]
 *                   u2 =  (b >> 11)      * 2^-53        in [0, 1)
 *                   z[2i]   = sqrt(-2 ln u1) * cos(2 pi u2)
 *                   z[2i+1] = sqrt(-2 ln u1) * sin(2 pi u2)
 *                   value = mean + std * z, rounded to float32, then to
 *                   bfloat16 (nearest, ties to even)
 * splitmix64 is the finaliser of Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators" (OOPSLA 2014).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t splitmix64(uint64_t x) {
    x += 0x9E3779B97F4A7C15ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
    return splitmix64(splitmix64(seed) ^ (stream * 0xD1B54A32D192ED03ull));
}

/* float -> bfloat16 bits, round to nearest, ties to even (finite inputs). */
static inline uint16_t f32_to_bf16_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

static inline double normal_at(uint64_t key, uint64_t e) {
    uint64_t i = e >> 1;
    uint64_t a = splitmix64(key + 2 * i);
    uint64_t b = splitmix64(key + 2 * i + 1);
    double u1 = (double)((a >> 11) + 1) * 0x1p-53;
    double u2 = (double)(b >> 11) * 0x1p-53;
    double r = sqrt(-2.0 * log(u1));
    double t = 6.283185307179586476925286766559 * u2;
    return (e & 1) ? r * sin(t) : r * cos(t);
}

static inline void normal_pair(uint64_t key, uint64_t i, double* z0, double* z1) {
    uint64_t a = splitmix64(key + 2 * i);
    uint64_t b = splitmix64(key + 2 * i + 1);
    double u1 = (double)((a >> 11) + 1) * 0x1p-53;
    double u2 = (double)(b >> 11) * 0x1p-53;
    double r = sqrt(-2.0 * log(u1));
    double t = 6.283185307179586476925286766559 * u2;
    *z0 = r * cos(t);
    *z1 = r * sin(t);
}

typedef struct {
    uint64_t key, offset, begin, end;
    double mean, stdv;
    uint16_t* out_bf16;
    double* out_f64;
} job_t;

static void emit(job_t* j, uint64_t i, double z) {
    z = j->mean + j->stdv * z;
    if (j->out_bf16) j->out_bf16[i] = f32_to_bf16_bits((float)z);
    if (j->out_f64) j->out_f64[i] = z;
}

static void* run_job(void* p) {
    job_t* j = (job_t*)p;
    uint64_t i = j->begin;
    if (i < j->end && ((j->offset + i) & 1)) {  /* odd start: second half of a pair */
        emit(j, i, normal_at(j->key, j->offset + i));
        ++i;
    }
    for (; i + 1 < j->end; i += 2) {
        double z0, z1;
        normal_pair(j->key, (j->offset + i) >> 1, &z0, &z1);
        emit(j, i, z0);
        emit(j, i + 1, z1);
    }
    if (i < j->end) emit(j, i, normal_at(j->key, j->offset + i));
    return NULL;
}

static void run_parallel(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n,
                         double mean, double stdv, uint16_t* ob, double* od, int threads) {
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    if ((uint64_t)threads > n / 4096 + 1) threads = (int)(n / 4096 + 1);
    pthread_t tid[256];
    job_t jobs[256];
    uint64_t key = stream_key(seed, stream);
    for (int t = 0; t < threads; ++t) {
        jobs[t].key = key;
        jobs[t].offset = offset;
        jobs[t].begin = n * (uint64_t)t / (uint64_t)threads;
        jobs[t].end = n * (uint64_t)(t + 1) / (uint64_t)threads;
        jobs[t].mean = mean;
        jobs[t].stdv = stdv;
        jobs[t].out_bf16 = ob;
        jobs[t].out_f64 = od;
    }
    for (int t = 1; t < threads; ++t) pthread_create(&tid[t], NULL, run_job, &jobs[t]);
    run_job(&jobs[0]);
    for (int t = 1; t < threads; ++t) pthread_join(tid[t], NULL);
}

/* Elements offset .. offset+n-1 of stream `stream`, as bfloat16 bit patterns. */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n,
                       double mean, double stdv, uint16_t* out, int threads) {
    run_parallel(seed, stream, offset, n, mean, stdv, out, NULL, threads);
}

/* Same deviates, unrounded (float64). */
void synth_normal_f64(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n,
                      double mean, double stdv, double* out, int threads) {
    run_parallel(seed, stream, offset, n, mean, stdv, NULL, out, threads);
}

/* Raw 64-bit counter output, for tests of the generator itself. */
uint64_t synth_splitmix64(uint64_t x) { return splitmix64(x); }

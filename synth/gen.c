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
#include <stdlib.h>
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

/*
 * Smooth video field (the full-layer workload's video rows): for every
 * channel c of a T x Hh x Ww latent grid,
 *   white noise   z[t][h][w] = normal deviate of element ((t*Hh + h)*Ww + w)*C + c
 *                 of stream `stream` (same definition as above);
 *   blur          a separable Gaussian filter, standard deviations (st, sh, sw)
 *                 grid cells, weights exp(-i^2 / (2 s^2)) for |i| <= ceil(3 s),
 *                 normalised to sum 1, half-sample symmetric boundary
 *                 (x[-1] = x[0], x[-2] = x[1], ...), applied along t, then h, then w;
 *   normalise     divided by the root mean square of the channel over the grid;
 * rounded to bfloat16 and written in tile-packed token order: tiles of
 * pt x ph x pw grid points in raster order over the tile grid, points in
 * raster order inside a tile.  Grid point (t, h, w) goes to row
 *   ((t/pt * (Hh/ph) + h/ph) * (Ww/pw) + w/pw) * (pt*ph*pw) + ((t%pt)*ph + h%ph)*pw + w%pw
 * of `out` (row stride ld elements).  Hh, Ww, T must be multiples of ph, pw, pt.
 */
typedef struct {
    uint64_t key;
    int T, Hh, Ww, C, pt, ph, pw, c_begin, c_end;
    double st, sh, sw;
    uint16_t* out;
    int64_t ld;
} field_job_t;

static int gauss_weights(double s, double* w) {
    int R = (int)ceil(3.0 * s);
    double sum = 0.0;
    for (int i = -R; i <= R; ++i) sum += (w[i + R] = exp(-(double)(i * i) / (2.0 * s * s)));
    for (int i = 0; i <= 2 * R; ++i) w[i] /= sum;
    return R;
}

static inline int reflect_index(int i, int n) {
    /* half-sample symmetric: ... 1 0 | 0 1 ... n-1 | n-1 n-2 ... */
    int period = 2 * n;
    i %= period;
    if (i < 0) i += period;
    return i < n ? i : period - 1 - i;
}

/* blur one channel block along one axis: n points, stride between points,
   `lines` lines starting at line_start(k) */
static void* run_field(void* p) {
    field_job_t* j = (field_job_t*)p;
    const int T = j->T, Hh = j->Hh, Ww = j->Ww, C = j->C;
    const int64_t G = (int64_t)T * Hh * Ww;
    double wt[64], wh[64], ww[64];
    const int Rt = gauss_weights(j->st, wt), Rh = gauss_weights(j->sh, wh), Rw = gauss_weights(j->sw, ww);
    double* a = (double*)malloc(sizeof(double) * G);
    double* b = (double*)malloc(sizeof(double) * G);
    for (int c = j->c_begin; c < j->c_end; ++c) {
        for (int64_t g = 0; g < G; ++g) a[g] = normal_at(j->key, (uint64_t)(g * C + c));
        /* along t */
        for (int t = 0; t < T; ++t)
            for (int hw = 0; hw < Hh * Ww; ++hw) {
                double s = 0.0;
                for (int i = -Rt; i <= Rt; ++i) s += wt[i + Rt] * a[(int64_t)reflect_index(t + i, T) * Hh * Ww + hw];
                b[(int64_t)t * Hh * Ww + hw] = s;
            }
        /* along h */
        for (int t = 0; t < T; ++t)
            for (int h = 0; h < Hh; ++h)
                for (int w = 0; w < Ww; ++w) {
                    double s = 0.0;
                    for (int i = -Rh; i <= Rh; ++i) s += wh[i + Rh] * b[((int64_t)t * Hh + reflect_index(h + i, Hh)) * Ww + w];
                    a[((int64_t)t * Hh + h) * Ww + w] = s;
                }
        /* along w */
        double ss = 0.0;
        for (int64_t r = 0; r < (int64_t)T * Hh; ++r)
            for (int w = 0; w < Ww; ++w) {
                double s = 0.0;
                for (int i = -Rw; i <= Rw; ++i) s += ww[i + Rw] * a[r * Ww + reflect_index(w + i, Ww)];
                b[r * Ww + w] = s;
                ss += s * s;
            }
        const double inv = 1.0 / sqrt(ss / (double)G);
        const int nth = Hh / j->ph, ntw = Ww / j->pw, pts = j->pt * j->ph * j->pw;
        for (int t = 0; t < T; ++t)
            for (int h = 0; h < Hh; ++h)
                for (int w = 0; w < Ww; ++w) {
                    const int64_t tile = ((int64_t)(t / j->pt) * nth + h / j->ph) * ntw + w / j->pw;
                    const int64_t row = tile * pts + ((t % j->pt) * j->ph + h % j->ph) * j->pw + w % j->pw;
                    j->out[row * j->ld + c] = f32_to_bf16_bits((float)(b[((int64_t)t * Hh + h) * Ww + w] * inv));
                }
    }
    free(a);
    free(b);
    return NULL;
}

void synth_smooth_field_bf16(uint64_t seed, uint64_t stream, int T, int Hh, int Ww, int C,
                             double st, double sh, double sw, int pt, int ph, int pw,
                             uint16_t* out, int64_t ld, int threads) {
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    if (threads > C) threads = C;
    pthread_t tid[256];
    field_job_t jobs[256];
    const uint64_t key = stream_key(seed, stream);
    for (int t = 0; t < threads; ++t) {
        field_job_t* j = &jobs[t];
        j->key = key; j->T = T; j->Hh = Hh; j->Ww = Ww; j->C = C;
        j->pt = pt; j->ph = ph; j->pw = pw;
        j->st = st; j->sh = sh; j->sw = sw;
        j->c_begin = (int)((int64_t)C * t / threads);
        j->c_end = (int)((int64_t)C * (t + 1) / threads);
        j->out = out; j->ld = ld;
    }
    for (int t = 1; t < threads; ++t) pthread_create(&tid[t], NULL, run_field, &jobs[t]);
    run_field(&jobs[0]);
    for (int t = 1; t < threads; ++t) pthread_join(tid[t], NULL);
}

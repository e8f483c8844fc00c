/*
 * vsa_oracle.c -- CPU oracle for the video sparse attention (VSA) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain, float64 statement
 * of what the GPU library must compute.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load it; the GPU library never
 * calls, links or includes it, and it shares no code with the library.
 *
 * Source of the method: the page "UniServe: serving FastH3 at its fastest",
 * section "The FastH3 workload" (VSA definition), section "Fused attention
 * preprocessing" (FP32 pooled tile statistics; top-k, fine and coarse are
 * separate steps), section "Fused output combination" (the combination
 * equation) and section "Setup" (the top-k video tiles are selected exactly).
 * Where those passages leave a step open, the reading taken is stated at the
 * function that implements the step.
 *
 * Notation: H heads, head dimension D = 128, tiles of T = 64 tokens.  The
 * sequence is [text | video | audio] with token counts S_t, S_v, S_a (each a
 * multiple of 64); n_t, n_v, n_a are the tile counts and N their sum.
 * Tensors are bfloat16 bit patterns, token-major [S][H][128].  Video tile u
 * (0 <= u < n_v) holds tokens S_t + 64u .. S_t + 64u + 63.
 *
 * Every value below is computed in float64 unless stated otherwise.  A
 * bfloat16 input widens to float64 exactly.  The one stated exception: a
 * tile mean (and a SubBlock piece mean) is rounded once to float32 after its
 * float64 sum is divided by the row count, because the page fixes the pooled
 * statistics as FP32; the scores are then float64 dot products of those
 * float32 means.
 *
 * Parity pins (tests under tests/, marked "not gpu"): brute-force masked
 * dense attention on tiny inputs, topk_frac = 1 against the textbook dense
 * softmax attention of torch on CPU, closed forms (constant V, Q = 0, a
 * single video tile, a two-tile coarse softmax, gate extremes), designed
 * rankings and ties, exact k counts, permutation and head-slice invariances,
 * and float64 -> bfloat16 rounding cases.
 */
#include <math.h>
#include <pthread.h>
#include <stdatomic.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define D 128
#define T 64

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

static double bf16_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* float64 -> bfloat16, one rounding, to nearest with ties to even.
 * bfloat16 has 8 significant bits and the exponent range of float32
 * (smallest subnormal 2^-133).  Exported for the rounding pins. */
uint16_t vsa_oracle_bf16_from_f64(double x) {
    if (isnan(x)) return 0x7FC0;
    if (isinf(x)) return x > 0 ? 0x7F80 : 0xFF80;
    if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
    int e;
    frexp(x, &e);                 /* |x| = m * 2^e, 0.5 <= m < 1 */
    int lead = e - 1;             /* exponent of the leading bit  */
    if (lead < -126) lead = -126; /* subnormal range: fixed quantum */
    int qexp = lead - 7;          /* value of the last kept bit   */
    double r = nearbyint(ldexp(x, -qexp)); /* default mode: nearest, ties even */
    double y = ldexp(r, qexp);
    if (fabs(y) >= 0x1p128) return x > 0 ? 0x7F80 : 0xFF80;
    float f = (float)y; /* exact: y has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------ */
/* Step 1: number of selected video tiles                                    */
/* ------------------------------------------------------------------------ */

/* "The FastH3 workload": video queries keep the highest-scoring 20% of the
 * video key tiles, rounded to a whole number of tiles.  Reading: k is
 * frac * n_v rounded half up, computed in float64, and at least one tile
 * when there is any video (the pages never select zero tiles); k = 0 when
 * there are no video tiles.  Returns -1 for a fraction outside (0, 1]. */
int32_t vsa_oracle_topk_count(int64_t n_v, double frac) {
    if (!(frac > 0.0 && frac <= 1.0) || n_v < 0) return -1;
    if (n_v == 0) return 0;
    double k = floor(frac * (double)n_v + 0.5);
    if (k < 1.0) k = 1.0;
    if (k > (double)n_v) k = (double)n_v;
    return (int32_t)k;
}

/* ------------------------------------------------------------------------ */
/* Step 2: tile mean-pooling                                                 */
/* ------------------------------------------------------------------------ */

/* "The FastH3 workload" (coarse branch over mean-pooled tiles) and "Fused
 * attention preprocessing" (the pooled statistics are FP32, pooled over valid
 * tokens).  For head h and tile u (tiles counted from token row0), the mean
 * of the tile's valid rows -- the first `valid` rows from row0 are valid, so
 * tile u has n = min(64, valid - 64u) of them -- summed in row order in
 * float64, divided by n in float64 and rounded once to float32.  out is
 * [H][n_tiles][128]. */
static void pool_one(const uint16_t* x, int32_t H, int64_t row0, int64_t n_tiles, int64_t valid,
                     int32_t h, int64_t u, float* out) {
    int64_t n = valid - u * T;
    if (n > T) n = T;
    for (int d = 0; d < D; ++d) {
        double s = 0.0;
        for (int64_t r = 0; r < n; ++r) {
            int64_t row = row0 + u * T + r;
            s += bf16_to_f64(x[(row * H + h) * D + d]);
        }
        out[((int64_t)h * n_tiles + u) * D + d] = (float)(s / (double)n);
    }
}

/* ------------------------------------------------------------------------ */
/* Step 3: ranking scores                                                    */
/* ------------------------------------------------------------------------ */

/* Score of video query tile u against video key tile w in one head: the dot
 * product of the two FP32 pooled vectors, each product formed exactly in
 * float64 and summed in dimension order (d = 0..127) in float64.  The scale
 * 1/sqrt(128) is left out of the ranking (it is positive, so the order is
 * the same). */
static double pooled_score(const float* qb, const float* kb) {
    double s = 0.0;
    for (int d = 0; d < D; ++d) s += (double)qb[d] * (double)kb[d];
    return s;
}

/* All scores of one row: s[w] for w < n_v, given the pooled [H][n_v][128]. */
void vsa_oracle_row_scores(const float* qbar, const float* kbar, int32_t h, int64_t n_v,
                           int64_t u, double* s) {
    const float* qb = qbar + ((int64_t)h * n_v + u) * D;
    for (int64_t w = 0; w < n_v; ++w) s[w] = pooled_score(qb, kbar + ((int64_t)h * n_v + w) * D);
}

/* ------------------------------------------------------------------------ */
/* Step 4: exact top-k selection                                             */
/* ------------------------------------------------------------------------ */

typedef struct {
    double score;
    int64_t idx;
} scored_t;

/* Total order: higher score first, equal scores by lower tile index. */
static int by_score_then_index(const void* a, const void* b) {
    const scored_t* x = (const scored_t*)a;
    const scored_t* y = (const scored_t*)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->idx > y->idx) - (x->idx < y->idx);
}

static int ascending_i32(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/* "The FastH3 workload" and "Setup": the k highest-scoring video key tiles,
 * selected exactly.  Ties go to the lower tile index.  Output: k video-local
 * tile indices in ascending order.  kth (optional) receives the k-th largest
 * score. */
static void select_row(const double* s, int64_t n_v, int32_t k, scored_t* scratch, int32_t* sel,
                       double* kth) {
    for (int64_t w = 0; w < n_v; ++w) {
        scratch[w].score = s[w];
        scratch[w].idx = w;
    }
    qsort(scratch, (size_t)n_v, sizeof(scored_t), by_score_then_index);
    for (int32_t i = 0; i < k; ++i) sel[i] = (int32_t)scratch[i].idx;
    if (kth) *kth = k > 0 ? scratch[k - 1].score : 0.0;
    qsort(sel, (size_t)k, sizeof(int32_t), ascending_i32);
}

/* ------------------------------------------------------------------------ */
/* Step 5: coarse branch                                                     */
/* ------------------------------------------------------------------------ */

/* "The FastH3 workload": a coarse branch attends over the mean-pooled tiles;
 * "Fused output combination": its per-tile output is added to every row of
 * the tile.  Reading: the pooled query of video tile u attends over the
 * pooled keys/values of the video tiles only, with scale 1/sqrt(128):
 *   a_w = s[w] / sqrt(128),  c_u = sum_w exp(a_w - max a) vbar_w / sum_w exp(a_w - max a). */
static void coarse_row(const double* s, int64_t n_v, const float* vbar_h, double* c) {
    const double alpha = 1.0 / sqrt((double)D);
    double m = -INFINITY;
    for (int64_t w = 0; w < n_v; ++w)
        if (alpha * s[w] > m) m = alpha * s[w];
    double den = 0.0;
    double num[D];
    for (int d = 0; d < D; ++d) num[d] = 0.0;
    for (int64_t w = 0; w < n_v; ++w) {
        double e = exp(alpha * s[w] - m);
        den += e;
        for (int d = 0; d < D; ++d) num[d] += e * (double)vbar_h[w * D + d];
    }
    for (int d = 0; d < D; ++d) c[d] = num[d] / den;
}

/* ------------------------------------------------------------------------ */
/* Thread pool over independent work items                                    */
/* ------------------------------------------------------------------------ */

typedef struct {
    void (*fn)(void* ctx, int64_t item, void* scratch);
    void* ctx;
    int64_t n_items;
    size_t scratch_bytes;
    atomic_llong next;
} pool_t;

static void* pool_worker(void* p) {
    pool_t* pl = (pool_t*)p;
    void* scratch = pl->scratch_bytes ? malloc(pl->scratch_bytes) : NULL;
    for (;;) {
        long long i = atomic_fetch_add(&pl->next, 1);
        if (i >= pl->n_items) break;
        pl->fn(pl->ctx, (int64_t)i, scratch);
    }
    free(scratch);
    return NULL;
}

static int resolve_threads(int threads) {
    if (threads <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        threads = n > 0 ? (int)n : 1;
    }
    return threads > 512 ? 512 : threads;
}

static void run_pool(void (*fn)(void*, int64_t, void*), void* ctx, int64_t n_items,
                     size_t scratch_bytes, int threads) {
    pool_t pl;
    pl.fn = fn;
    pl.ctx = ctx;
    pl.n_items = n_items;
    pl.scratch_bytes = scratch_bytes;
    atomic_init(&pl.next, 0);
    threads = resolve_threads(threads);
    if (threads > n_items) threads = n_items > 0 ? (int)n_items : 1;
    pthread_t* tid = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)threads);
    for (int t = 1; t < threads; ++t) pthread_create(&tid[t], NULL, pool_worker, &pl);
    pool_worker(&pl);
    for (int t = 1; t < threads; ++t) pthread_join(tid[t], NULL);
    free(tid);
}

typedef struct {
    const uint16_t* x;
    int32_t H;
    int64_t row0, n_tiles, valid;
    float* out;
} pool_ctx_t;

static void pool_item(void* p, int64_t item, void* scratch) {
    (void)scratch;
    pool_ctx_t* c = (pool_ctx_t*)p;
    pool_one(c->x, c->H, c->row0, c->n_tiles, c->valid, (int32_t)(item / c->n_tiles),
             item % c->n_tiles, c->out);
}

/* Pooled FP32 means of n_tiles tiles starting at token row0, every head, over
 * the first `valid` rows (every tile must hold at least one). */
void vsa_oracle_pool_valid(const uint16_t* x, int32_t H, int64_t row0, int64_t n_tiles,
                           int64_t valid, float* out, int threads) {
    pool_ctx_t c = {x, H, row0, n_tiles, valid, out};
    run_pool(pool_item, &c, (int64_t)H * n_tiles, 0, threads);
}

/* Pooled FP32 means of n_tiles full tiles starting at token row0, every head. */
void vsa_oracle_pool_threads(const uint16_t* x, int32_t H, int64_t row0, int64_t n_tiles, float* out,
                             int threads) {
    vsa_oracle_pool_valid(x, H, row0, n_tiles, n_tiles * T, out, threads);
}

void vsa_oracle_pool(const uint16_t* x, int32_t H, int64_t row0, int64_t n_tiles, float* out) {
    vsa_oracle_pool_threads(x, H, row0, n_tiles, out, 1);
}

/* ------------------------------------------------------------------------ */
/* Steps 2-5 for every (head, video query tile)                              */
/* ------------------------------------------------------------------------ */

typedef struct {
    const float *qbar, *kbar, *vbar;
    int64_t n_v;
    int32_t k;
    int32_t* sel;    /* [H][n_v][k]          */
    double* coarse;  /* [H][n_v][128]        */
    double* kth;     /* [H][n_v] or NULL     */
    double* scores;  /* [H][n_v][n_v] or NULL */
} select_ctx_t;

static void select_item(void* p, int64_t item, void* scratch) {
    select_ctx_t* c = (select_ctx_t*)p;
    int64_t n_v = c->n_v;
    int32_t h = (int32_t)(item / n_v);
    int64_t u = item % n_v;
    double* s = (double*)scratch;
    scored_t* tmp = (scored_t*)(s + n_v);
    vsa_oracle_row_scores(c->qbar, c->kbar, h, n_v, u, s);
    if (c->scores) memcpy(c->scores + item * n_v, s, sizeof(double) * (size_t)n_v);
    select_row(s, n_v, c->k, tmp, c->sel + item * c->k, c->kth ? c->kth + item : NULL);
    coarse_row(s, n_v, c->vbar + (int64_t)h * n_v * D, c->coarse + item * D);
}

/* Pools Q, K, V over the video tiles, then selects and computes the coarse
 * branch for every (head, video query tile).  Outputs (caller-allocated):
 *   qbar, kbar, vbar : float32 [H][n_v][128]  (pooled statistics)
 *   sel              : int32   [H][n_v][k]    (ascending video-local indices)
 *   coarse           : float64 [H][n_v][128]
 *   kth              : float64 [H][n_v]       (k-th largest score; may be NULL)
 *   scores           : float64 [H][n_v][n_v]  (all scores; may be NULL)
 * Returns k, or -1 on bad arguments. */
/* As vsa_oracle_select_coarse, for a video segment whose first V_v of S_v
 * rows are valid (S_v - 64 < V_v <= S_v: only the last tile may be partial):
 * the pooled statistics average each tile's valid rows only. */
int32_t vsa_oracle_select_coarse_valid(const uint16_t* q, const uint16_t* kk, const uint16_t* v,
                                       int32_t H, int64_t S_t, int64_t S_v, int64_t S_a,
                                       int64_t V_v, double frac, float* qbar, float* kbar,
                                       float* vbar, int32_t* sel, double* coarse, double* kth,
                                       double* scores, int threads) {
    (void)S_a;
    if (H < 1 || S_t % T || S_v % T || S_a % T || S_t < 0 || S_v < 0 || S_a < 0) return -1;
    if (V_v > S_v || (S_v > 0 && V_v <= S_v - T)) return -1;
    int64_t n_v = S_v / T;
    int32_t k = vsa_oracle_topk_count(n_v, frac);
    if (k < 0) return -1;
    if (n_v == 0) return 0;
    vsa_oracle_pool_valid(q, H, S_t, n_v, V_v, qbar, threads);
    vsa_oracle_pool_valid(kk, H, S_t, n_v, V_v, kbar, threads);
    vsa_oracle_pool_valid(v, H, S_t, n_v, V_v, vbar, threads);
    select_ctx_t c = {qbar, kbar, vbar, n_v, k, sel, coarse, kth, scores};
    size_t scratch = sizeof(double) * (size_t)n_v + sizeof(scored_t) * (size_t)n_v;
    run_pool(select_item, &c, (int64_t)H * n_v, scratch, threads);
    return k;
}

int32_t vsa_oracle_select_coarse(const uint16_t* q, const uint16_t* kk, const uint16_t* v,
                                 int32_t H, int64_t S_t, int64_t S_v, int64_t S_a, double frac,
                                 float* qbar, float* kbar, float* vbar, int32_t* sel,
                                 double* coarse, double* kth, double* scores, int threads) {
    return vsa_oracle_select_coarse_valid(q, kk, v, H, S_t, S_v, S_a, S_v, frac, qbar, kbar, vbar,
                                          sel, coarse, kth, scores, threads);
}

/* ------------------------------------------------------------------------ */
/* Steps 6-7: fine attention and gated combination for chosen rows            */
/* ------------------------------------------------------------------------ */

typedef struct {
    const uint16_t *q, *k, *v, *g;
    int32_t H;
    int64_t S_t, S_v, S_a;
    int64_t V_t, V_v, V_a; /* valid rows at the start of each segment */
    const int32_t* sel; /* [H][n_v][kk] */
    int32_t kk;
    const double* coarse; /* [H][n_v][128] */
    const int64_t* rows;
    int64_t n_rows;
    uint16_t* out_bf16; /* [n_rows][H][128] */
    double* out_f64;    /* [n_rows][H][128] or NULL */
} fine_ctx_t;

/* One output row i of one head h.
 * "The FastH3 workload": text and audio queries attend to every key; a video
 * query attends to all text and audio keys and to the keys of the selected
 * video tiles of its own tile.  Reading: one softmax over the union of those
 * keys, with logits q.k / sqrt(128).
 * "Fused output combination": a video row adds the gated coarse output of its
 * tile; the gate is sigmoid(G) per channel.  Text and audio rows have no
 * coarse term.  The result is rounded once to bfloat16.
 * "Fused attention preprocessing" (padding handled inside the kernel, never
 * an input to later computation).  Reading: each segment's first V rows are
 * its tokens and the rest padding; padding rows are never keys, and a
 * padding query row outputs zeros. */
static int is_valid_row(const fine_ctx_t* c, int64_t j) {
    if (j < c->S_t) return j < c->V_t;
    if (j < c->S_t + c->S_v) return j - c->S_t < c->V_v;
    return j - c->S_t - c->S_v < c->V_a;
}

static void fine_item(void* p, int64_t item, void* scratch) {
    fine_ctx_t* c = (fine_ctx_t*)p;
    const int32_t H = c->H;
    const int64_t ri = item / H;
    const int32_t h = (int32_t)(item % H);
    const int64_t i = c->rows[ri];
    const int64_t S = c->S_t + c->S_v + c->S_a;
    const int64_t n_v = c->S_v / T;
    const double alpha = 1.0 / sqrt((double)D);
    const int is_video = (i >= c->S_t && i < c->S_t + c->S_v);
    const int64_t u = is_video ? (i - c->S_t) / T : -1;

    int64_t* keys = (int64_t*)scratch;
    double* logit = (double*)(keys + S);
    int64_t base = (ri * H + h) * D;
    if (!is_valid_row(c, i)) {
        for (int d = 0; d < D; ++d) {
            if (c->out_f64) c->out_f64[base + d] = 0.0;
            c->out_bf16[base + d] = 0;
        }
        return;
    }
    int64_t nk = 0;
    if (!is_video) {
        for (int64_t j = 0; j < S; ++j)
            if (is_valid_row(c, j)) keys[nk++] = j;
    } else {
        for (int64_t j = 0; j < c->S_t; ++j)
            if (is_valid_row(c, j)) keys[nk++] = j;
        const int32_t* srow = c->sel + ((int64_t)h * n_v + u) * c->kk;
        for (int32_t t = 0; t < c->kk; ++t)
            for (int r = 0; r < T; ++r) {
                const int64_t j = c->S_t + (int64_t)srow[t] * T + r;
                if (is_valid_row(c, j)) keys[nk++] = j;
            }
        for (int64_t j = c->S_t + c->S_v; j < S; ++j)
            if (is_valid_row(c, j)) keys[nk++] = j;
    }

    double qi[D];
    for (int d = 0; d < D; ++d) qi[d] = bf16_to_f64(c->q[(i * H + h) * D + d]);
    double m = -INFINITY;
    for (int64_t t = 0; t < nk; ++t) {
        const uint16_t* kj = c->k + (keys[t] * H + h) * D;
        double s = 0.0;
        for (int d = 0; d < D; ++d) s += qi[d] * bf16_to_f64(kj[d]);
        logit[t] = alpha * s;
        if (logit[t] > m) m = logit[t];
    }
    double den = 0.0, o[D];
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t t = 0; t < nk; ++t) {
        double e = exp(logit[t] - m);
        den += e;
        const uint16_t* vj = c->v + (keys[t] * H + h) * D;
        for (int d = 0; d < D; ++d) o[d] += e * bf16_to_f64(vj[d]);
    }
    for (int d = 0; d < D; ++d) {
        double y = o[d] / den;
        if (is_video) {
            double g = bf16_to_f64(c->g[(i * H + h) * D + d]);
            double sig = 1.0 / (1.0 + exp(-g));
            y += sig * c->coarse[((int64_t)h * n_v + u) * D + d];
        }
        if (c->out_f64) c->out_f64[base + d] = y;
        c->out_bf16[base + d] = vsa_oracle_bf16_from_f64(y);
    }
}

/* Output rows `rows` (absolute token indices) of every head, given ANY
 * selection `sel` ([H][n_v][kk], video-local tile indices) and coarse output
 * `coarse` ([H][n_v][128], float64).  Taking the selection as an argument
 * lets a test evaluate the fine branch on exactly the index sets another
 * implementation chose.  Returns 0, or -1 on bad arguments. */
int32_t vsa_oracle_fine_valid(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const uint16_t* g, int32_t H, int64_t S_t, int64_t S_v, int64_t S_a,
                              int64_t V_t, int64_t V_v, int64_t V_a, const int32_t* sel,
                              int32_t kk, const double* coarse, const int64_t* rows,
                              int64_t n_rows, uint16_t* out_bf16, double* out_f64, int threads) {
    if (H < 1 || S_t % T || S_v % T || S_a % T || S_t < 0 || S_v < 0 || S_a < 0) return -1;
    if (V_t < 0 || V_t > S_t || V_v < 0 || V_v > S_v || V_a < 0 || V_a > S_a) return -1;
    int64_t S = S_t + S_v + S_a;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= S) return -1;
    if (S_v > 0) {
        int64_t n_v = S_v / T;
        if (kk < 0 || kk > n_v) return -1;
        for (int64_t e = 0; e < (int64_t)H * n_v * kk; ++e)
            if (sel[e] < 0 || sel[e] >= n_v) return -1;
    }
    fine_ctx_t c = {q, k, v, g, H, S_t, S_v, S_a, V_t, V_v, V_a, sel, kk, coarse, rows, n_rows,
                    out_bf16, out_f64};
    size_t scratch = (sizeof(int64_t) + sizeof(double)) * (size_t)S;
    run_pool(fine_item, &c, n_rows * H, scratch, threads);
    return 0;
}

int32_t vsa_oracle_fine(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
                        int32_t H, int64_t S_t, int64_t S_v, int64_t S_a, const int32_t* sel,
                        int32_t kk, const double* coarse, const int64_t* rows, int64_t n_rows,
                        uint16_t* out_bf16, double* out_f64, int threads) {
    return vsa_oracle_fine_valid(q, k, v, g, H, S_t, S_v, S_a, S_t, S_v, S_a, sel, kk, coarse,
                                 rows, n_rows, out_bf16, out_f64, threads);
}

/* Threads a call with threads <= 0 would use. */
int32_t vsa_oracle_default_threads(void) { return resolve_threads(0); }

/* ------------------------------------------------------------------------ */
/* SubBlock router (a second selection rule feeding the same fine branch)    */
/* ------------------------------------------------------------------------ */

/* The SGLang Diffusion benchmark page, section "How SubBlock Sparse
 * Attention Works", describes this router.  Restated: on both the query and
 * the key side a 64-token tile is cut into four 16-token pieces; for one
 * head, the pull of key tile w on query tile u is summarised by a single
 * number, the log of the summed exponentials of the 16 scaled dot products
 * between piece means, which stands in for the unnormalised softmax weight
 * the key tile would receive.  Each query tile keeps the key tiles with the
 * largest such numbers; `sparsity` is the share of candidate tiles dropped
 * and the number kept is a whole multiple of 8.
 * Readings: the piece statistics are FP32 means of 16 rows (as the tile
 * means above); the score of key tile w for query tile u is
 *   score(u, w) = log sum_{a, b < 4} exp(alpha * qsub[u][a] . ksub[w][b]),
 * alpha = 1/sqrt(128), dots as in pooled_score; the kept count is
 *   k = 8 * floor((1 - sparsity) * n / 8 + 1/2), clamped to [min(8, n), n]
 * for n candidate tiles; ties go to the lower tile index (as the main rule).
 * Two candidate sets are offered.  Video mode: the router ranks the video
 * key tiles of each video query tile (n = n_v); text and audio keys stay
 * dense and text/audio queries attend to everything, so the main path's
 * fine branch is reused as it is.  Whole-sequence mode, the page's own
 * reading: every query tile of the joint sequence (text, video and audio)
 * ranks every key tile of the sequence (n = N) and attends to its kept
 * tiles only.  Neither mode has a coarse term. */
int32_t vsa_oracle_subblock_count(int64_t n_v, double sparsity) {
    if (!(sparsity >= 0.0 && sparsity < 1.0) || n_v < 0) return -1;
    if (n_v == 0) return 0;
    double k = 8.0 * floor((1.0 - sparsity) * (double)n_v / 8.0 + 0.5);
    const double lo = n_v < 8 ? (double)n_v : 8.0;
    if (k < lo) k = lo;
    if (k > (double)n_v) k = (double)n_v;
    return (int32_t)k;
}

/* FP32 means of the 16-row sub-blocks of the video tiles: out [H][n_v][4][128]. */
static void subpool_one(const uint16_t* x, int32_t H, int64_t row0, int64_t n_v, int32_t h,
                        int64_t u, float* out) {
    for (int a = 0; a < 4; ++a)
        for (int d = 0; d < D; ++d) {
            double s = 0.0;
            for (int r = 0; r < 16; ++r) {
                int64_t row = row0 + u * T + 16 * a + r;
                s += bf16_to_f64(x[(row * H + h) * D + d]);
            }
            out[(((int64_t)h * n_v + u) * 4 + a) * D + d] = (float)(s / 16.0);
        }
}

typedef struct {
    const uint16_t *q, *k;
    int32_t H;
    int64_t S_t, n_v;
    int32_t kk;
    float *qsub, *ksub;
    int32_t* sel;
    double* kth;
    double* scores;
    const int64_t* rows;  /* NULL: every (head, tile) in order; else rows[i] = h * n_v + u */
} sub_ctx_t;

static void subpool_item(void* p, int64_t item, void* scratch) {
    (void)scratch;
    sub_ctx_t* c = (sub_ctx_t*)p;
    const int32_t h = (int32_t)(item / c->n_v);
    const int64_t u = item % c->n_v;
    subpool_one(c->q, c->H, c->S_t, c->n_v, h, u, c->qsub);
    subpool_one(c->k, c->H, c->S_t, c->n_v, h, u, c->ksub);
}

static void subscore_item(void* p, int64_t item, void* scratch) {
    sub_ctx_t* c = (sub_ctx_t*)p;
    const int64_t n_v = c->n_v;
    const int64_t hu = c->rows ? c->rows[item] : item;
    const int32_t h = (int32_t)(hu / n_v);
    const int64_t u = hu % n_v;
    const double alpha = 1.0 / sqrt((double)D);
    double* s = (double*)scratch;
    scored_t* tmp = (scored_t*)(s + n_v);
    for (int64_t w = 0; w < n_v; ++w) {
        double x[16], m = -INFINITY;
        for (int a = 0; a < 4; ++a)
            for (int b = 0; b < 4; ++b) {
                const float* qa = c->qsub + (((int64_t)h * n_v + u) * 4 + a) * D;
                const float* kb = c->ksub + (((int64_t)h * n_v + w) * 4 + b) * D;
                x[4 * a + b] = alpha * pooled_score(qa, kb);
                if (x[4 * a + b] > m) m = x[4 * a + b];
            }
        double e = 0.0;
        for (int i = 0; i < 16; ++i) e += exp(x[i] - m);
        s[w] = m + log(e);
    }
    if (c->scores) memcpy(c->scores + item * n_v, s, sizeof(double) * (size_t)n_v);
    select_row(s, n_v, c->kk, tmp, c->sel + item * c->kk, c->kth ? c->kth + item : NULL);
}

/* Sub-block statistics, scores and selection for every (head, video query
 * tile).  Outputs (caller-allocated): qsub, ksub float32 [H][n_v][4][128];
 * sel int32 [H][n_v][k] (ascending); kth float64 [H][n_v] (k-th largest
 * score; may be NULL); scores float64 [H][n_v][n_v] (may be NULL).
 * Returns k, or -1 on bad arguments. */
int32_t vsa_oracle_subblock_select(const uint16_t* q, const uint16_t* k, int32_t H, int64_t S_t,
                                   int64_t S_v, int64_t S_a, double sparsity, float* qsub,
                                   float* ksub, int32_t* sel, double* kth, double* scores,
                                   int threads) {
    if (H < 1 || S_t % T || S_v % T || S_a % T || S_t < 0 || S_v < 0 || S_a < 0) return -1;
    const int64_t n_v = S_v / T;
    const int32_t kk = vsa_oracle_subblock_count(n_v, sparsity);
    if (kk < 0) return -1;
    if (n_v == 0) return 0;
    sub_ctx_t c = {q, k, H, S_t, n_v, kk, qsub, ksub, sel, kth, scores, NULL};
    run_pool(subpool_item, &c, (int64_t)H * n_v, 0, threads);
    size_t scratch = sizeof(double) * (size_t)n_v + sizeof(scored_t) * (size_t)n_v;
    run_pool(subscore_item, &c, (int64_t)H * n_v, scratch, threads);
    return kk;
}

/* As vsa_oracle_subblock_select, for the listed rows only (rows[i] = h * n_v
 * + u): sub-block means of every tile (qsub, ksub as above), then scores and
 * selection of n_rows rows: sel [n_rows][k], kth [n_rows], scores [n_rows][n_v]
 * (may be NULL).  Returns k, or -1 on bad arguments. */
int32_t vsa_oracle_subblock_select_rows(const uint16_t* q, const uint16_t* k, int32_t H,
                                        int64_t S_t, int64_t S_v, int64_t S_a, double sparsity,
                                        const int64_t* rows, int64_t n_rows, float* qsub,
                                        float* ksub, int32_t* sel, double* kth, double* scores,
                                        int threads) {
    if (H < 1 || S_t % T || S_v % T || S_a % T || S_t < 0 || S_v < 0 || S_a < 0 || n_rows < 0)
        return -1;
    const int64_t n_v = S_v / T;
    const int32_t kk = vsa_oracle_subblock_count(n_v, sparsity);
    if (kk < 0) return -1;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= (int64_t)H * n_v) return -1;
    if (n_v == 0) return 0;
    sub_ctx_t c = {q, k, H, S_t, n_v, kk, qsub, ksub, sel, kth, scores, rows};
    run_pool(subpool_item, &c, (int64_t)H * n_v, 0, threads);
    size_t scratch = sizeof(double) * (size_t)n_v + sizeof(scored_t) * (size_t)n_v;
    run_pool(subscore_item, &c, n_rows, scratch, threads);
    return kk;
}

/* ------------------------------------------------------------------------ */
/* SubBlock router, whole-sequence mode (the page's own reading)             */
/* ------------------------------------------------------------------------ */

/* Every 64-token tile of the joint [text | video | audio] sequence is both a
 * query tile and a candidate key tile: N = S / 64 tiles, tile j holding
 * tokens 64j .. 64j + 63.  Piece means, scores and the ranking are exactly
 * those of the video mode above, taken over all N tiles instead of the n_v
 * video tiles: the ranking of each (head, query tile) row runs over every
 * key tile of the sequence, and the kept count is
 * vsa_oracle_subblock_count(N, sparsity).  Selected indices are global tile
 * indices 0..N-1, ascending.  Outputs as vsa_oracle_subblock_select with n_v
 * replaced by N. */
int32_t vsa_oracle_subblock_select_whole(const uint16_t* q, const uint16_t* k, int32_t H,
                                         int64_t S_t, int64_t S_v, int64_t S_a, double sparsity,
                                         float* qsub, float* ksub, int32_t* sel, double* kth,
                                         double* scores, int threads) {
    if (H < 1 || S_t % T || S_v % T || S_a % T || S_t < 0 || S_v < 0 || S_a < 0) return -1;
    const int64_t N = (S_t + S_v + S_a) / T;
    const int32_t kk = vsa_oracle_subblock_count(N, sparsity);
    if (kk < 0) return -1;
    if (N == 0) return 0;
    /* the video mode's machinery over rows 0 .. S - 1: tile j starts at row 64j */
    sub_ctx_t c = {q, k, H, 0, N, kk, qsub, ksub, sel, kth, scores, NULL};
    run_pool(subpool_item, &c, (int64_t)H * N, 0, threads);
    size_t scratch = sizeof(double) * (size_t)N + sizeof(scored_t) * (size_t)N;
    run_pool(subscore_item, &c, (int64_t)H * N, scratch, threads);
    return kk;
}

/* As vsa_oracle_subblock_select_whole for the listed rows only (rows[i] =
 * h * N + j): piece means of every tile, then sel [n_rows][k], kth [n_rows],
 * scores [n_rows][N] (may be NULL). */
int32_t vsa_oracle_subblock_select_whole_rows(const uint16_t* q, const uint16_t* k, int32_t H,
                                              int64_t S_t, int64_t S_v, int64_t S_a,
                                              double sparsity, const int64_t* rows,
                                              int64_t n_rows, float* qsub, float* ksub,
                                              int32_t* sel, double* kth, double* scores,
                                              int threads) {
    if (H < 1 || S_t % T || S_v % T || S_a % T || S_t < 0 || S_v < 0 || S_a < 0 || n_rows < 0)
        return -1;
    const int64_t N = (S_t + S_v + S_a) / T;
    const int32_t kk = vsa_oracle_subblock_count(N, sparsity);
    if (kk < 0) return -1;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= (int64_t)H * N) return -1;
    if (N == 0) return 0;
    sub_ctx_t c = {q, k, H, 0, N, kk, qsub, ksub, sel, kth, scores, rows};
    run_pool(subpool_item, &c, (int64_t)H * N, 0, threads);
    size_t scratch = sizeof(double) * (size_t)N + sizeof(scored_t) * (size_t)N;
    run_pool(subscore_item, &c, n_rows, scratch, threads);
    return kk;
}

/* ------------------------------------------------------------------------ */
/* Fine attention over per-tile key lists                                     */
/* ------------------------------------------------------------------------ */

typedef struct {
    const uint16_t *q, *k, *v;
    int32_t H;
    int64_t S;
    const int32_t* lists; /* [H][N][kk] global key-tile indices */
    int32_t kk;
    const int64_t* rows;
    uint16_t* out_bf16; /* [n_rows][H][128] */
    double* out_f64;    /* [n_rows][H][128] or NULL */
} lists_ctx_t;

/* Query row i (tile j = i / 64) of head h attends to the keys of the tiles
 * lists[h][j][0 .. kk): one softmax over those keys with logits
 * q.k / sqrt(128), no coarse term and no gate; the result is rounded once to
 * bfloat16.  This is the fine step of the whole-sequence router (section
 * "How SubBlock Sparse Attention Works": the kept key blocks of each query
 * block go to the block-sparse attention kernel). */
static void lists_item(void* p, int64_t item, void* scratch) {
    lists_ctx_t* c = (lists_ctx_t*)p;
    const int32_t H = c->H;
    const int64_t ri = item / H;
    const int32_t h = (int32_t)(item % H);
    const int64_t i = c->rows[ri];
    const int64_t N = c->S / T;
    const double alpha = 1.0 / sqrt((double)D);
    double* logit = (double*)scratch;
    const int32_t* lst = c->lists + ((int64_t)h * N + i / T) * c->kk;
    double qi[D];
    for (int d = 0; d < D; ++d) qi[d] = bf16_to_f64(c->q[(i * H + h) * D + d]);
    double m = -INFINITY;
    int64_t nk = 0;
    for (int32_t t = 0; t < c->kk; ++t)
        for (int r = 0; r < T; ++r) {
            const int64_t j = (int64_t)lst[t] * T + r;
            const uint16_t* kj = c->k + (j * H + h) * D;
            double s = 0.0;
            for (int d = 0; d < D; ++d) s += qi[d] * bf16_to_f64(kj[d]);
            logit[nk] = alpha * s;
            if (logit[nk] > m) m = logit[nk];
            ++nk;
        }
    double den = 0.0, o[D];
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    nk = 0;
    for (int32_t t = 0; t < c->kk; ++t)
        for (int r = 0; r < T; ++r) {
            const int64_t j = (int64_t)lst[t] * T + r;
            const double e = exp(logit[nk++] - m);
            den += e;
            const uint16_t* vj = c->v + (j * H + h) * D;
            for (int d = 0; d < D; ++d) o[d] += e * bf16_to_f64(vj[d]);
        }
    const int64_t base = (ri * H + h) * D;
    for (int d = 0; d < D; ++d) {
        const double y = o[d] / den;
        if (c->out_f64) c->out_f64[base + d] = y;
        c->out_bf16[base + d] = vsa_oracle_bf16_from_f64(y);
    }
}

/* Output rows `rows` of every head, each query tile attending to its own list
 * of kk key tiles (lists [H][N][kk], global indices in [0, N), distinct).
 * Returns 0, or -1 on bad arguments. */
int32_t vsa_oracle_fine_lists(const uint16_t* q, const uint16_t* k, const uint16_t* v, int32_t H,
                              int64_t S, const int32_t* lists, int32_t kk, const int64_t* rows,
                              int64_t n_rows, uint16_t* out_bf16, double* out_f64, int threads) {
    if (H < 1 || S <= 0 || S % T || kk < 1 || n_rows < 0) return -1;
    const int64_t N = S / T;
    if (kk > N) return -1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= S) return -1;
    for (int64_t e = 0; e < (int64_t)H * N * kk; ++e)
        if (lists[e] < 0 || lists[e] >= N) return -1;
    lists_ctx_t c = {q, k, v, H, S, lists, kk, rows, out_bf16, out_f64};
    run_pool(lists_item, &c, n_rows * H, sizeof(double) * (size_t)kk * T, threads);
    return 0;
}

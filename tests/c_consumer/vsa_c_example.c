/* vsa_c_example.c -- a consumer of the VSA library written in plain C, with
 * no Python and no torch: the C ABI of include/vsa.h used the way a serving
 * runtime in C or C++ would use it.  Test program only.
 *
 * For each case it draws Q, K, V and G (bfloat16, iid N(0, 1), token-major
 * [S][H][128]) with the seeded generator, copies them to the device with the
 * HIP runtime, sizes and allocates the workspace with vsa_workspace_bytes,
 * runs vsa_forward on a stream of its own, and compares the result with the
 * CPU oracle (test infrastructure, linked here only because this is a test):
 *   - every selection row equal to the oracle's (page "UniServe: serving
 *     FastH3 at its fastest", section "The FastH3 workload": the top
 *     round(0.2 n) video tiles by pooled-query . pooled-key score);
 *   - every output row within max-abs 2e-2, mean-abs 2e-3 and relative
 *     RMS 5e-3 of the oracle's float64 output on the same selection.
 * It also checks that a malformed call (topk_frac = 0) is refused with
 * VSA_ERR_BAD_TOPK before any device work.
 *
 * Exit status 0 when every case passes, 1 on a mismatch, 2 on a HIP or
 * library error.  Usage: vsa_c_example [threads] */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "vsa.h"

/* the seeded generator (synth/gen.c) */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n, double mean,
                       double stdv, uint16_t* out, int threads);
/* the CPU oracle (oracle/vsa_oracle.c) */
int32_t vsa_oracle_select_coarse(const uint16_t* q, const uint16_t* kk, const uint16_t* v,
                                 int32_t H, int64_t S_t, int64_t S_v, int64_t S_a, double frac,
                                 float* qbar, float* kbar, float* vbar, int32_t* sel,
                                 double* coarse, double* kth, double* scores, int threads);
int32_t vsa_oracle_fine(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
                        int32_t H, int64_t S_t, int64_t S_v, int64_t S_a, const int32_t* sel,
                        int32_t kk, const double* coarse, const int64_t* rows, int64_t n_rows,
                        uint16_t* out_bf16, double* out_f64, int threads);

#define D 128
#define T 64

#define HIP_OK(call)                                                                   \
    do {                                                                               \
        hipError_t e_ = (call);                                                        \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #call,               \
                    hipGetErrorString(e_));                                            \
            exit(2);                                                                   \
        }                                                                              \
    } while (0)

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of host memory (%zu bytes)\n", n);
        exit(2);
    }
    return p;
}

static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

typedef struct {
    const char* name;
    int32_t heads;
    int64_t text_tiles, video_tiles, audio_tiles;
    uint64_t seed;
} vsa_case;

static int run_case(const vsa_case* c, int threads) {
    const int32_t H = c->heads;
    const int64_t s_t = c->text_tiles * T, s_v = c->video_tiles * T, s_a = c->audio_tiles * T;
    const int64_t S = s_t + s_v + s_a, n_v = c->video_tiles;
    const float frac = 0.2f;
    const size_t elems = (size_t)S * H * D, bytes = elems * sizeof(uint16_t);
    const int32_t k = vsa_topk_count(s_v, frac);
    const size_t ws_bytes = vsa_workspace_bytes(H, s_t, s_v, s_a, frac);
    printf("[%s] heads %d, tiles (%lld, %lld, %lld), k %d, workspace %zu bytes\n", c->name, H,
           (long long)c->text_tiles, (long long)n_v, (long long)c->audio_tiles, k, ws_bytes);
    fflush(stdout);
    if (k < 1 || ws_bytes == 0) {
        fprintf(stderr, "[%s] shape rejected by the library\n", c->name);
        return 2;
    }

    /* inputs: streams 0..3 of the generator are Q, K, V, G */
    uint16_t* host[4];
    for (int t = 0; t < 4; ++t) {
        host[t] = (uint16_t*)xmalloc(bytes);
        synth_normal_bf16(c->seed, (uint64_t)t, 0, elems, 0.0, 1.0, host[t], threads);
    }
    void* dev[4];
    for (int t = 0; t < 4; ++t) {
        HIP_OK(hipMalloc(&dev[t], bytes));
        HIP_OK(hipMemcpy(dev[t], host[t], bytes, hipMemcpyHostToDevice));
    }
    void *d_out, *d_ws;
    int32_t* d_sel;
    const size_t sel_elems = (size_t)H * n_v * k;
    HIP_OK(hipMalloc(&d_out, bytes));
    HIP_OK(hipMalloc((void**)&d_sel, sel_elems * sizeof(int32_t)));
    HIP_OK(hipMalloc(&d_ws, ws_bytes));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    /* a malformed call is refused before any device work */
    vsa_status st = vsa_forward(dev[0], dev[1], dev[2], dev[3], H, s_t, s_v, s_a, 0.0f, d_out,
                                d_sel, d_ws, ws_bytes, (void*)stream);
    if (st != VSA_ERR_BAD_TOPK) {
        fprintf(stderr, "[%s] topk_frac 0 returned %s\n", c->name, vsa_status_string(st));
        return 1;
    }
    st = vsa_forward(dev[0], dev[1], dev[2], dev[3], H, s_t, s_v, s_a, frac, d_out, d_sel, d_ws,
                     ws_bytes, (void*)stream);
    if (st != VSA_OK) {
        fprintf(stderr, "[%s] vsa_forward: %s\n", c->name, vsa_status_string(st));
        return 2;
    }
    HIP_OK(hipStreamSynchronize(stream));

    uint16_t* out = (uint16_t*)xmalloc(bytes);
    int32_t* sel = (int32_t*)xmalloc(sel_elems * sizeof(int32_t));
    HIP_OK(hipMemcpy(out, d_out, bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(sel, d_sel, sel_elems * sizeof(int32_t), hipMemcpyDeviceToHost));

    /* oracle selection and coarse vectors */
    const size_t pooled = (size_t)H * n_v * D;
    float* qbar = (float*)xmalloc(pooled * sizeof(float));
    float* kbar = (float*)xmalloc(pooled * sizeof(float));
    float* vbar = (float*)xmalloc(pooled * sizeof(float));
    int32_t* ref_sel = (int32_t*)xmalloc(sel_elems * sizeof(int32_t));
    double* coarse = (double*)xmalloc(pooled * sizeof(double));
    double* kth = (double*)xmalloc((size_t)H * n_v * sizeof(double));
    double* scores = (double*)xmalloc((size_t)H * n_v * n_v * sizeof(double));
    const int32_t ref_k = vsa_oracle_select_coarse(host[0], host[1], host[2], H, s_t, s_v, s_a,
                                                   frac, qbar, kbar, vbar, ref_sel, coarse, kth,
                                                   scores, threads);
    int bad = 0;
    if (ref_k != k) {
        fprintf(stderr, "[%s] k %d, oracle %d\n", c->name, k, ref_k);
        bad = 1;
    }
    int64_t sel_mismatch = 0;
    for (size_t i = 0; !bad && i < sel_elems; ++i) sel_mismatch += sel[i] != ref_sel[i];
    if (sel_mismatch) {
        fprintf(stderr, "[%s] %lld selection entries differ from the oracle\n", c->name,
                (long long)sel_mismatch);
        bad = 1;
    }

    /* oracle output on every row, with the (equal) selection */
    double max_abs = 0.0, sum_abs = 0.0, sum_sq_err = 0.0, sum_sq_ref = 0.0;
    if (!bad) {
        int64_t* rows = (int64_t*)xmalloc((size_t)S * sizeof(int64_t));
        for (int64_t i = 0; i < S; ++i) rows[i] = i;
        uint16_t* ref_bf16 = (uint16_t*)xmalloc(bytes);
        double* ref = (double*)xmalloc(elems * sizeof(double));
        vsa_oracle_fine(host[0], host[1], host[2], host[3], H, s_t, s_v, s_a, ref_sel, k, coarse,
                        rows, S, ref_bf16, ref, threads);
        for (size_t i = 0; i < elems; ++i) {
            const double got = bf16_to_double(out[i]);
            const double err = fabs(got - ref[i]);
            if (!(err <= max_abs)) max_abs = err; /* NaN propagates */
            sum_abs += err;
            sum_sq_err += err * err;
            sum_sq_ref += ref[i] * ref[i];
        }
        free(rows);
        free(ref_bf16);
        free(ref);
        const double mean_abs = sum_abs / (double)elems;
        const double rel_rms = sqrt(sum_sq_err / (sum_sq_ref > 0 ? sum_sq_ref : 1.0));
        printf("[%s] every row: max-abs %.3e, mean-abs %.3e, rel-RMS %.3e\n", c->name, max_abs,
               mean_abs, rel_rms);
        if (!(max_abs <= 2e-2 && mean_abs <= 2e-3 && rel_rms <= 5e-3)) bad = 1;
    }

    HIP_OK(hipStreamDestroy(stream));
    for (int t = 0; t < 4; ++t) {
        HIP_OK(hipFree(dev[t]));
        free(host[t]);
    }
    HIP_OK(hipFree(d_out));
    HIP_OK(hipFree(d_sel));
    HIP_OK(hipFree(d_ws));
    free(out);
    free(sel);
    free(qbar);
    free(kbar);
    free(vbar);
    free(ref_sel);
    free(coarse);
    free(kth);
    free(scores);
    printf("[%s] %s\n", c->name, bad ? "FAIL" : "ok");
    fflush(stdout);
    return bad;
}

int main(int argc, char** argv) {
    const int threads = argc > 1 ? atoi(argv[1]) : 8;
    static const vsa_case cases[] = {
        /* the tiny workload: 1 head, 64 text + 1,024 video + 64 audio tokens, k = 3 */
        {"tiny", 1, 1, 16, 1, 0},
        /* three heads, a ragged video tile count, more than one text and audio tile */
        {"ragged", 3, 2, 37, 3, 11},
    };
    int worst = 0;
    for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i) {
        const int r = run_case(&cases[i], threads);
        if (r > worst) worst = r;
    }
    return worst;
}

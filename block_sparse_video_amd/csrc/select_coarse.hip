// select_coarse.hip -- stage 2 of the VSA forward on gfx950: tile ranking
// scores, exact top-k selection and the coarse branch, one kernel.
//
// Page "UniServe: serving FastH3 at its fastest":
//   section "The FastH3 workload": a video query tile keeps the highest-
//     scoring 20% of the video key tiles (rounded), and a coarse branch
//     attends over mean-pooled tiles;
//   section "Setup": the top-k tiles are selected exactly;
//   section "Fused attention preprocessing": pooled statistics are FP32.
// Definitions used (per head h, video query tile u, video key tile w):
//   score s(u,w) = sum over d = 0..127, in order, in float64, of
//                  Qbar[u][d] * Kbar[w][d]   (FP32 statistics; each product
//                  is exact in float64, so fma and multiply-then-add agree)
//   selection    = the k tiles that come first in the order (score desc,
//                  index asc), written in ascending index order
//   coarse c[u]  = sum_w softmax_w(s(u,w)/sqrt(128)) * Vbar[w]  (float64
//                  accumulation of float32 weights, stored as float32)
//
// One workgroup owns R consecutive query tiles of one head; the R rows of
// float64 scores live in LDS for the whole kernel, so scores never touch HBM.
// Selection is a wavefront-level radix select on 64-bit order-preserving keys
// (8 passes of 8 bits), then a ballot compaction that emits indices in
// ascending order and takes tied keys by lowest index.
#include "topk_wave.h"
#include "vsa_internal.h"

#include <atomic>

namespace vsa {
namespace {

template <int R, int NS>
__global__ __launch_bounds__(256) void select_coarse_kernel(const double* __restrict__ qbar64,
                                                            const float* __restrict__ kbar,
                                                            const float* __restrict__ vbar, int n_v,
                                                            int k, int ldw, float alpha,
                                                            int32_t* __restrict__ sel,
                                                            float* __restrict__ coarse) {
    extern __shared__ __align__(16) unsigned char smem[];
    double* sc = (double*)smem;                       // [R][ldw] scores, later softmax weights
    uint32_t* hist_all = (uint32_t*)(sc + R * ldw);   // [4 waves][256]
    double* rowsum = (double*)(hist_all + 4 * 256);   // [R]

    const int h = blockIdx.y;
    const int u0 = blockIdx.x * R;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;

    // ---- scores: thread = key tile w, R query rows in registers ----------
    {
        const double* qb[R];
#pragma unroll
        for (int r = 0; r < R; ++r) qb[r] = qbar64 + ((int64_t)h * n_v + min(u0 + r, n_v - 1)) * kD;
        const float* kb = kbar + (int64_t)h * n_v * kD;
        for (int w0 = 0; w0 < n_v; w0 += 256) {
            const int w = w0 + tid;
            const int wc = min(w, n_v - 1);
            const float* kw = kb + (int64_t)wc * kD;
            double acc[R];
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = 0.0;
#pragma unroll 8
            for (int d = 0; d < kD; ++d) {
                const int pd = pooled_dim_pos(d);
                const double kd = (double)kw[pd];
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] = __fma_rn(qb[r][pd], kd, acc[r]);
            }
            if (w < n_v) {
#pragma unroll
                for (int r = 0; r < R; ++r) sc[r * ldw + w] = acc[r] + 0.0;
            }
        }
    }
    __syncthreads();

    // ---- exact top-k per row: one wavefront per row -----------------------
    uint32_t* hist = hist_all + wv * 256;
    constexpr int RW = (R + 3) / 4;  // rows per wave (every wave runs the same passes)
    for (int t = 0; t < RW; ++t) {
        const int r = wv + 4 * t;
        const bool active = (r < R) && (u0 + r < n_v);
        const double* row = sc + min(r, R - 1) * ldw;
        uint64_t prefix = 0;
        uint32_t remaining = (uint32_t)k;
        if constexpr (NS > 0) {
            if (active) prefix = kth_key_bisect<NS>(row, n_v, k, lane, remaining);
        } else {
            uint64_t mask = 0;
            for (int shift = 56; shift >= 0; shift -= 8) {
                if (active)
                    for (int i = lane; i < 256; i += 64) hist[i] = 0u;
                __syncthreads();
                if (active) {
                    for (int w = lane; w < n_v; w += 64) {
                        const uint64_t key = order_key(row[w]);
                        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
                    }
                }
                __syncthreads();
                if (active) {
                    // lane i owns bins 255-4i .. 252-4i (descending)
                    const uint32_t c0 = hist[255 - 4 * lane], c1 = hist[254 - 4 * lane];
                    const uint32_t c2 = hist[253 - 4 * lane], c3 = hist[252 - 4 * lane];
                    const uint32_t tot = c0 + c1 + c2 + c3;
                    uint32_t incl = tot;
    #pragma unroll
                    for (int off = 1; off < 64; off <<= 1) {
                        const uint32_t y = __shfl_up(incl, off);
                        if (lane >= off) incl += y;
                    }
                    const uint32_t excl = incl - tot;
                    const bool hit = excl < remaining && remaining <= incl;
                    const uint64_t hb = __ballot(hit);
                    const int src = __ffsll((long long)hb) - 1;
                    int digit = 0;
                    uint32_t above = 0;
                    if (hit) {
                        uint32_t cum = excl;
                        if (cum + c0 >= remaining) {
                            digit = 255 - 4 * lane;
                        } else {
                            cum += c0;
                            if (cum + c1 >= remaining) {
                                digit = 254 - 4 * lane;
                            } else {
                                cum += c1;
                                if (cum + c2 >= remaining) {
                                    digit = 253 - 4 * lane;
                                } else {
                                    cum += c2;
                                    digit = 252 - 4 * lane;
                                }
                            }
                        }
                        above = cum;
                    }
                    digit = __shfl(digit, src);
                    above = __shfl(above, src);
                    prefix |= (uint64_t)digit << shift;
                    mask |= 255ull << shift;
                    remaining -= above;
                }
                __syncthreads();
            }

        }
        if (active) {
            emit_topk(row, n_v, k, prefix, remaining, lane,
                      sel + ((int64_t)blockIdx.y * n_v + u0 + r) * k);
            // coarse softmax weights, in place: p_w = exp((s_w - max s) * alpha)
            double* wrow = sc + r * ldw;
            double m = -INFINITY;
            for (int w = lane; w < n_v; w += 64) m = fmax(m, wrow[w]);
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off));
            double lsum = 0.0;
            for (int w = lane; w < n_v; w += 64) {
                const float p = __expf((float)((wrow[w] - m) * (double)alpha));
                wrow[w] = (double)p;
                lsum += (double)p;
            }
            for (int w = n_v + lane; w < ldw; w += 64) wrow[w] = 0.0;  // pad: weight 0
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off);
            if (lane == 0) rowsum[r] = lsum;
        }
    }
    __syncthreads();

    // ---- coarse output: c[u][d] = sum_w p_w Vbar[w][d] / sum_w p_w --------
    // thread (d, half) accumulates rows half*RH .. half*RH + RH - 1; pooled V
    // values are requested 32 columns at a time and the weights of two
    // columns come in one LDS read (rows are padded with zero weights to a
    // multiple of 32 columns)
    constexpr int RH = (R + 1) / 2;
    const int d = tid & 127;
    const int half = tid >> 7;
    double acc[RH];
#pragma unroll
    for (int i = 0; i < RH; ++i) acc[i] = 0.0;
    const float* vb = vbar + ((int64_t)h * kD + d) * vbar_pitch(n_v);  // transposed pooled V
    const double* prow[RH];
#pragma unroll
    for (int i = 0; i < RH; ++i) prow[i] = sc + min(half * RH + i, R - 1) * ldw;
    // pooled V values of the next group of 32 columns are requested while
    // the current group is multiplied
    float vn[32];
    auto load_group = [&](int w0) {
        if (w0 + 32 <= n_v) {
#pragma unroll
            for (int i = 0; i < 32; ++i) vn[i] = vb[w0 + i];
        } else {
#pragma unroll
            for (int i = 0; i < 32; ++i) vn[i] = vb[min(w0 + i, n_v - 1)];
        }
    };
    load_group(0);
    for (int w0 = 0; w0 < n_v; w0 += 32) {
        float vr[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) vr[i] = vn[i];
        if (w0 + 32 < n_v) load_group(w0 + 32);
#pragma unroll
        for (int i = 0; i < 32; i += 2) {
#pragma unroll
            for (int r = 0; r < RH; ++r) {
                const double2 p2 = *(const double2*)(prow[r] + w0 + i);
                acc[r] = __fma_rn(p2.x, (double)vr[i], acc[r]);
                acc[r] = __fma_rn(p2.y, (double)vr[i + 1], acc[r]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < RH; ++i) {
        const int r = half * RH + i;
        if (r < R && u0 + r < n_v)
            coarse[((int64_t)h * n_v + u0 + r) * kD + d] = (float)(acc[i] / rowsum[r]);
    }
}

// ---- matrix-core version: 16 query rows per workgroup ----------------------
//
// Both products run on the float32 matrix instruction v_mfma_f32_16x16x4f32
// (twice the float64 one's rate on gfx950).  Each score is eight chains of
// four instructions (16 products of dims 16c .. 16c + 15, from a zero
// accumulator), whose float32 results are added in float64 and rounded once
// to float32.  The stored score a differs from the exact float64 score e by
//   |a - e| <= eps = 2.1e-6 * |Qbar[u]| * max_w |Kbar[w]|  (+ a denormal term)
// (Euclidean norms): a 16-term float32 dot product of any summation order
// and any rounding mode is within gamma_16 = 16u / (1 - 16u), u = 2^-23, of
// the sum of |products|, which Cauchy-Schwarz bounds by the norms; the
// float64 sum adds ~1e-15 and the final rounding 2^-24 of that bound.
// Selection stays exact: with T the k-th largest stored score of a row,
// every key above T + 2 eps is in the exact top k and every key below
// T - 2 eps is not (at least k keys have e >= T - eps, at most k - 1 have
// e > T + eps), so only the band [T - 2 eps, T + 2 eps] can need more.  When
// the band holds more keys than are still to be taken, their float64 scores
// are recomputed (the d-order chain of exact products, the oracle's
// definition) and ranked among themselves, ties to the lower index.  The
// band is ~1e-4 of the score spread: almost every row takes it whole.
// The coarse product runs on the same float32 instruction, in chains of four
// (16 keys) whose results are added in float64.
// Operand layout (lane l): A[row l % 16][k l / 16], B[k l / 16][col l % 16];
// result D[row 4 (l / 16) + v][col l % 16] in element v.
//
// The 16 score rows are kept in LDS as float32 (74 KiB at 1,134 tiles, so two
// workgroups share a CU and one's top-k overlaps the other's matrix work).
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowsM = 16;   // query rows per workgroup: the instruction's M
constexpr int kWavesM = 8;   // 512 threads
constexpr int kSlotsM = 20;  // keys per lane in the top-k (n_v <= 64 * 20)

// LDS row pitch in floats: at least n_v rounded up to 16 (whole 16-key
// blocks), 8 modulo 64, so that the 16 rows of one operand read fall on 8
// different groups of banks.
__host__ __device__ inline int mfma_pitch(int n_v) { return ((((n_v + 15) & ~15) + 55) / 64) * 64 + 8; }

__device__ __forceinline__ f32x4 mfma32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Bound on |stored score - float64 score| per unit of |Qbar[u]| max|Kbar[w]|:
// gamma_16 (u = 2^-23) + 2^-24 + the float64 sum, ~1.967e-6, with ~7% to
// spare (which also covers the float32 sum of squares behind max|Kbar[w]|).
constexpr double kScoreErr = 2.1e-6;
// Flushed denormal operands or partial results: at most 2^-126 per product
// or addition, times the larger operand; 256 of them per score.
constexpr double kScoreDenorm = 0x1p-117;

// Selection of one row whose band (stored scores with keys in [lo, hi])
// holds more entries than the `need` still to take: the band's float64
// scores are recomputed as the d-order chain of exact products (the oracle's
// scores), and the row's selection is every key above hi plus the band's
// `need` best by (float64 score desc, index asc), written in ascending index
// order.  Rows whose band is exactly what is needed (nearly all) never run it.
__device__ __forceinline__ void emit_band_resolved(const float* row, const double* qrow,
                                                const float* kb_h, int n_v, int k, uint32_t lo,
                                                uint32_t hi, uint32_t need, int lane,
                                                int32_t* out) {
    uint64_t kb64[kSlotsM];
#pragma unroll
    for (int i = 0; i < kSlotsM; ++i) {
        const int w = lane + 64 * i;
        kb64[i] = 0ull;
        if (w < n_v) {
            const uint32_t key = order_key32(row[w]);
            if (key >= lo && key <= hi) {
                double s = 0.0;
                for (int d = 0; d < kD; ++d) {
                    const int pd = pooled_dim_pos(d);
                    s = __builtin_fma(qrow[pd], (double)kb_h[(int64_t)w * kD + pd], s);
                }
                kb64[i] = order_key(s + 0.0);
            }
        }
    }
    uint32_t gt64;
    const uint64_t t64 = kth_largest(kb64, need, gt64);
    const uint32_t need64 = need - gt64;  // band entries equal to t64 to take, lowest index first
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    uint32_t outc = 0, eqseen = 0;
#pragma unroll
    for (int i = 0; i < kSlotsM; ++i) {
        const int w = lane + 64 * i;
        const bool valid = w < n_v;
        const uint32_t key = valid ? order_key32(row[w]) : 0u;
        const bool eq64 = kb64[i] != 0ull && kb64[i] == t64;
        const uint64_t em = __ballot(eq64);
        const uint32_t erank = eqseen + (uint32_t)__popcll(em & lt_mask);
        const bool take = key > hi || kb64[i] > t64 || (eq64 && erank < need64);
        const uint64_t tm = __ballot(take);
        const uint32_t pos = outc + (uint32_t)__popcll(tm & lt_mask);
        if (take && valid && pos < (uint32_t)k) out[pos] = w;
        outc += (uint32_t)__popcll(tm);
        eqseen += (uint32_t)__popcll(em);
    }
}

__global__ __launch_bounds__(512, 4) void select_coarse_mfma_kernel(
    const double* __restrict__ qbar64, const float* __restrict__ kbar,
    const float* __restrict__ vbar, int n_v, int k, int pitch, float alpha,
    int32_t* __restrict__ sel, float* __restrict__ coarse) {
    extern __shared__ __align__(16) unsigned char smem[];
    float* sc = (float*)smem;                          // [16][pitch] scores, later weights
    double* rowsum = (double*)(sc + kRowsM * pitch);   // [16]
    double* qnorm2 = rowsum + kRowsM;                  // [16] |Qbar[u0 + r]|^2
    float* knorm2 = (float*)(qnorm2 + kRowsM);         // [8] per wave: max |Kbar[w]|^2

    const int h = blockIdx.y;
    const int u0 = blockIdx.x * kRowsM;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int lr = lane & 15, lk = lane >> 4;
    const float* kb_h = kbar + (int64_t)h * n_v * kD;

    // ---- scores S[r][w] ~ sum_d Qbar[u0 + r][d] Kbar[w][d] ------------------
    // wave wv computes the 16-key blocks wv, wv + 8, ...; the A operands (this
    // workgroup's query rows, all 32 dimension groups) are loaded once.  Lane
    // group lk feeds dims 4 ds + lk, stored contiguously (pooled_dim_pos), so
    // a lane's 32 operands of a row are one 256-byte (Q) or 128-byte (K) run.
    // Each chain of four instructions (dims 16c .. 16c + 15) starts from zero
    // and its result is added in float64.  The squared norms of the rows and the
    // largest squared norm of the keys go to LDS for the selection's bound.
    {
        float qa[32];
        const double* qrow = qbar64 + ((int64_t)h * n_v + min(u0 + lr, n_v - 1)) * kD + 32 * lk;
        double qq = 0.0;
#pragma unroll
        for (int ds = 0; ds < 32; ds += 2) {
            const double2 q2 = *(const double2*)(qrow + ds);
            qa[ds] = (float)q2.x;  // float32 means: exact
            qa[ds + 1] = (float)q2.y;
            qq = __builtin_fma(q2.x, q2.x, qq);
            qq = __builtin_fma(q2.y, q2.y, qq);
        }
        if (wv == 0) {
            qq += __shfl_xor(qq, 16);
            qq += __shfl_xor(qq, 32);
            if (lk == 0) qnorm2[lr] = qq;
        }
        float kmax2 = 0.0f;
        const int nblk = (n_v + 15) / 16;
#pragma unroll 1
        for (int b = wv; b < nblk; b += kWavesM) {
            const int w = min(16 * b + lr, n_v - 1);
            const float* kw = kb_h + (int64_t)w * kD + 32 * lk;
            float kc[32];
#pragma unroll
            for (int ds = 0; ds < 32; ds += 4) {
                const float4 k4 = *(const float4*)(kw + ds);
                kc[ds] = k4.x;
                kc[ds + 1] = k4.y;
                kc[ds + 2] = k4.z;
                kc[ds + 3] = k4.w;
            }
            f64x4 acc = {0.0, 0.0, 0.0, 0.0};
            float kk = 0.0f;
#pragma unroll
            for (int ds = 0; ds < 32; ds += 4) {
                f32x4 p = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int j = 0; j < 4; ++j) p = mfma32(qa[ds + j], kc[ds + j], p);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[v] += (double)p[v];
#pragma unroll
                for (int j = 0; j < 4; ++j) kk = fmaf(kc[ds + j], kc[ds + j], kk);
            }
            kk += __shfl_xor(kk, 16);
            kk += __shfl_xor(kk, 32);
            if (16 * b + lr < n_v) {
                kmax2 = fmaxf(kmax2, kk);
                // x + 0.0 turns -0.0 into +0.0, so equal scores have equal keys
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    sc[(4 * lk + v) * pitch + 16 * b + lr] = (float)(acc[v] + 0.0);
            }
        }
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) kmax2 = fmaxf(kmax2, __shfl_xor(kmax2, off));
        if (lane == 0) knorm2[wv] = kmax2;
    }
    __syncthreads();

    // ---- exact top-k and softmax weights: rows wv and wv + 8 --------------
    float km2 = 0.0f;
#pragma unroll
    for (int i = 0; i < kWavesM; ++i) km2 = fmaxf(km2, knorm2[i]);
    const double kmax = sqrt((double)km2);
#pragma unroll 1
    for (int t = 0; t < 2; ++t) {
        const int r = wv + kWavesM * t;
        const int u = u0 + r;
        if (u >= n_v) continue;
        float* row = sc + r * pitch;
        uint32_t kv[kSlotsM];
#pragma unroll
        for (int i = 0; i < kSlotsM; ++i) {
            const int w = lane + 64 * i;
            kv[i] = w < n_v ? order_key32(row[w]) : 0u;
        }
        uint32_t gt32;
        const uint32_t t32 = kth_largest(kv, (uint32_t)k, gt32);
        // the band [lo, hi] around the k-th stored score that the bound on
        // |stored - float64 score| leaves undecided; all keys when the bound
        // is not finite or the products could leave the float32 range
        const double qn = sqrt(qnorm2[r]);
        uint32_t lo = 1u, hi = 0xFFFFFFFFu;
        if (qn * kmax < 0x1p100) {
            const double eps = kScoreErr * qn * kmax + kScoreDenorm * (qn + kmax + 1.0);
            const double tv = (double)key32_value(t32);
            lo = key32_at_or_below(tv - 2.0 * eps);
            hi = key32_at_or_above(tv + 2.0 * eps);
        }
        uint32_t above = 0, band = 0;
#pragma unroll
        for (int i = 0; i < kSlotsM; ++i) {
            above += (uint32_t)__popcll(__ballot(kv[i] > hi));
            band += (uint32_t)__popcll(__ballot(kv[i] >= lo && kv[i] <= hi));
        }
        uint32_t need = (uint32_t)k - above;  // entries still to take from the band
        if (band < need) {
            // cannot happen while the bound holds; rank the whole row instead
            lo = 1u;
            hi = 0xFFFFFFFFu;
            need = (uint32_t)k;
            band = (uint32_t)n_v;
        }
        int32_t* out = sel + ((int64_t)h * n_v + u) * k;
        if (band > need) {
            // band wider than what is left to take: rank it by float64 score
            emit_band_resolved(row, qbar64 + ((int64_t)h * n_v + u) * kD, kb_h, n_v, k, lo, hi,
                               need, lane, out);
        } else {
            // keys above the band and the whole band, in ascending index order
            const uint64_t lt_mask = (1ull << lane) - 1ull;
            uint32_t outc = 0;
#pragma unroll
            for (int i = 0; i < kSlotsM; ++i) {
                const int w = lane + 64 * i;
                const bool take = kv[i] >= lo;
                const uint64_t tm = __ballot(take);
                const uint32_t pos = outc + (uint32_t)__popcll(tm & lt_mask);
                if (take && w < n_v && pos < (uint32_t)k) out[pos] = w;
                outc += (uint32_t)__popcll(tm);
            }
        }
        float m = -INFINITY;
        for (int w = lane; w < n_v; w += 64) m = fmaxf(m, row[w]);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        double lsum = 0.0;
        for (int w = lane; w < n_v; w += 64) {
            const float p = __expf((float)(((double)row[w] - (double)m) * (double)alpha));
            row[w] = p;
            lsum += (double)p;
        }
        for (int w = n_v + lane; w < pitch; w += 64) row[w] = 0.0f;  // padding: weight 0
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off);
        if (lane == 0) rowsum[r] = lsum;
    }
    __syncthreads();

    // ---- coarse C[r][d] = sum_w P[r][w] Vbar[w][d] / sum_w P[r][w] --------
    // wave wv: dims 16 wv .. 16 wv + 15, one 16-key block per step: MFMA t of
    // block j takes key 16 j + 4 (lane / 16) + t in lane group lane / 16, so a
    // lane reads its four weights (one LDS read) and its four pooled V values
    // (one load from the transposed, padded rows) at once; padding keys have
    // weight 0 and value 0.  Each block's four float32 instructions start
    // from zero and their sum is added in float64, so float32 rounding acts
    // on 16-term partial sums only (no long float32 accumulation, whose
    // cancellation over a thousand terms would cost the coarse vector its
    // relative accuracy).  Rows past n_v (ragged last workgroup) compute
    // garbage that is never stored.
    {
        const float* vb = vbar + ((int64_t)h * kD + 16 * wv + lr) * vbar_pitch(n_v) + 4 * lk;
        const float* prow = sc + lr * pitch + 4 * lk;
        const int nb16 = (n_v + 15) / 16;
        f64x4 c = {0.0, 0.0, 0.0, 0.0};
        float4 pn = *(const float4*)prow, vn = *(const float4*)vb;
#pragma unroll 2
        for (int j = 0; j < nb16; ++j) {
            const float4 pw = pn, vv = vn;
            if (j + 1 < nb16) {
                pn = *(const float4*)(prow + 16 * (j + 1));
                vn = *(const float4*)(vb + 16 * (j + 1));
            }
            f32x4 p = {0.0f, 0.0f, 0.0f, 0.0f};
            p = mfma32(pw.x, vv.x, p);
            p = mfma32(pw.y, vv.y, p);
            p = mfma32(pw.z, vv.z, p);
            p = mfma32(pw.w, vv.w, p);
#pragma unroll
            for (int v = 0; v < 4; ++v) c[v] += (double)p[v];
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 4 * lk + v;
            if (u0 + r < n_v)
                coarse[((int64_t)h * n_v + u0 + r) * kD + 16 * wv + lr] = (float)(c[v] / rowsum[r]);
        }
    }
}

template <int R, int NS>
hipError_t launch_r(const Shape& s, int32_t* sel, uint8_t* ws, const Layout& L, hipStream_t stream,
                    int ldw, size_t lds) {
    // Raise the kernel's dynamic-LDS limit when a larger row pitch needs it.
    static std::atomic<size_t> lds_allowed[kMaxDevices];
    hipError_t e = ensure_dynamic_lds((const void*)select_coarse_kernel<R, NS>, lds_allowed, lds);
    if (e != hipSuccess) return e;
    dim3 grid((s.n_v + R - 1) / R, s.H);
    const float alpha = (float)(1.0 / 11.313708498984761);  // 1/sqrt(128)
    hipLaunchKernelGGL((select_coarse_kernel<R, NS>), grid, dim3(256), lds, stream,
                       (const double*)(ws + L.qbar64), (const float*)(ws + L.kbar),
                       (const float*)(ws + L.vbar), s.n_v, s.k, ldw, alpha, sel,
                       (float*)(ws + L.coarse));
    return hipGetLastError();
}

}  // namespace

// LDS budget of one workgroup (bytes): gfx950 allows 160 KiB per workgroup.
constexpr size_t kSelectLdsMax = 160 * 1024;

size_t select_lds_bytes(int R, int ldw) { return (size_t)R * ldw * 8 + 4 * 256 * 4 + (size_t)R * 8; }

size_t select_mfma_lds_bytes(int n_v) {
    return (size_t)kRowsM * mfma_pitch(n_v) * 4 + 2 * kRowsM * 8 + kWavesM * 4;
}

hipError_t launch_select_coarse(const Shape& s, int32_t* sel, uint8_t* ws, const Layout& L,
                                hipStream_t stream) {
    // rows of up to 64 * 20 keys whose 16 float64 rows fit the LDS: the
    // matrix-core kernel
    if (s.n_v <= 64 * kSlotsM && select_mfma_lds_bytes(s.n_v) <= kSelectLdsMax) {
        static std::atomic<size_t> lds_allowed[kMaxDevices];
        const size_t lds = select_mfma_lds_bytes(s.n_v);
        hipError_t e = ensure_dynamic_lds((const void*)select_coarse_mfma_kernel, lds_allowed, lds);
        if (e != hipSuccess) return e;
        dim3 grid((s.n_v + kRowsM - 1) / kRowsM, s.H);
        const float alpha = (float)(1.0 / 11.313708498984761);  // 1/sqrt(128)
        hipLaunchKernelGGL(select_coarse_mfma_kernel, grid, dim3(64 * kWavesM), lds, stream,
                           (const double*)(ws + L.qbar64), (const float*)(ws + L.kbar),
                           (const float*)(ws + L.vbar), s.n_v, s.k, mfma_pitch(s.n_v), alpha, sel,
                           (float*)(ws + L.coarse));
        return hipGetLastError();
    }
    const int ldw = (s.n_v + 31) & ~31;  // row pitch: whole groups of 32 columns
    // rows of up to 64 * 20 keys are selected from registers, longer rows by
    // the LDS radix select
    if (s.n_v <= 64 * 20 && select_lds_bytes(8, ldw) <= kSelectLdsMax / 2)
        return launch_r<8, 20>(s, sel, ws, L, stream, ldw, select_lds_bytes(8, ldw));
    if (select_lds_bytes(8, ldw) <= kSelectLdsMax / 2)
        return launch_r<8, 0>(s, sel, ws, L, stream, ldw, select_lds_bytes(8, ldw));
    if (select_lds_bytes(4, ldw) <= kSelectLdsMax / 2)
        return launch_r<4, 0>(s, sel, ws, L, stream, ldw, select_lds_bytes(4, ldw));
    if (select_lds_bytes(2, ldw) <= kSelectLdsMax)
        return launch_r<2, 0>(s, sel, ws, L, stream, ldw, select_lds_bytes(2, ldw));
    return launch_r<1, 0>(s, sel, ws, L, stream, ldw, select_lds_bytes(1, ldw));
}

}  // namespace vsa

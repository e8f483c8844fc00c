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
                                                            const float* __restrict__ kbar_t,
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
        const float* kb = kbar_t + (int64_t)h * kD * n_v;
        for (int w0 = 0; w0 < n_v; w0 += 256) {
            const int w = w0 + tid;
            const int wc = min(w, n_v - 1);
            double acc[R];
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = 0.0;
#pragma unroll 8
            for (int d = 0; d < kD; ++d) {
                const double kd = (double)kb[(int64_t)d * n_v + wc];
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] = __fma_rn(qb[r][d], kd, acc[r]);
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
    const float* vb = vbar + (int64_t)h * n_v * kD + d;
    const double* prow[RH];
#pragma unroll
    for (int i = 0; i < RH; ++i) prow[i] = sc + min(half * RH + i, R - 1) * ldw;
    // pooled V values of the next group of 32 columns are requested while
    // the current group is multiplied
    float vn[32];
    auto load_group = [&](int w0) {
        if (w0 + 32 <= n_v) {
            const float* p = vb + (int64_t)w0 * kD;
#pragma unroll
            for (int i = 0; i < 32; ++i) vn[i] = p[i * kD];
        } else {
#pragma unroll
            for (int i = 0; i < 32; ++i) vn[i] = vb[(int64_t)min(w0 + i, n_v - 1) * kD];
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
                       (const double*)(ws + L.qbar64), (const float*)(ws + L.kbar_t),
                       (const float*)(ws + L.vbar), s.n_v, s.k, ldw, alpha, sel,
                       (float*)(ws + L.coarse));
    return hipGetLastError();
}

}  // namespace

// LDS budget of one workgroup (bytes): gfx950 allows 160 KiB per workgroup.
constexpr size_t kSelectLdsMax = 160 * 1024;

size_t select_lds_bytes(int R, int ldw) { return (size_t)R * ldw * 8 + 4 * 256 * 4 + (size_t)R * 8; }

hipError_t launch_select_coarse(const Shape& s, int32_t* sel, uint8_t* ws, const Layout& L,
                                hipStream_t stream) {
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

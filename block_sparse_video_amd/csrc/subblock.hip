// subblock.hip -- the SubBlock router on gfx950: a second tile-selection rule
// whose selection feeds the same fine attention kernel.
//
// Router of the SGLang Diffusion benchmark page, section "How SubBlock Sparse
// Attention Works", restated: query and key tiles of 64 tokens are each cut
// into four 16-token pieces; one number per (head, query tile, key tile),
// built from the means of the pieces with a log-sum-exp, estimates the key
// tile's unnormalised softmax weight for that query tile, and each query tile
// keeps its highest-scoring key tiles, the count a whole multiple of 8.
// Definitions used (head h, video query tile u, video key tile w):
//   Qs[u][a], Ks[w][b] = float32 means of the 16 rows of sub-block a (b),
//                        summed in float64 (exact for bfloat16 inputs)
//   x_ab(u,w)          = (1/sqrt(128)) * sum_d Qs[u][a][d] * Ks[w][b][d], float64
//   score(u,w)         = log sum_{a,b} exp(x_ab(u,w)), float64
//   kept count k       = 8 * floor((1 - sparsity) * n_v / 8 + 1/2), clamped to
//                        [min(8, n_v), n_v]
//   selection          = the k tiles first in the order (score desc, index asc),
//                        written in ascending index order.
// Text and audio keys stay dense and there is no coarse term.
//
// Stage 1 (subpool_kernel) writes the sub-block means of Q and K in the exact
// per-lane order of the float64 MFMA operands of stage 2, so each operand
// load there is a contiguous 1 KiB wavefront read.  Packed layout per head
// and group c of four video tiles (16 sub-block rows j = 4 * (u % 4) + a):
//   [c][i = 0..7][lane = 16 g + j][e = 0..3] = mean of row j, dim 32 g + 4 i + e.
// Stage 2 (subblock_route_kernel) is a float64 MFMA product Qs Ks^T per head
// (16 x 16 x 4 tiles: four query tiles x four key tiles per output tile, the
// 16 sub-block pairs of one tile pair in 4 lanes x 4 registers),
// the log-sum-exp of each tile pair in registers, one row of scores per
// query tile in LDS, and the wavefront top-k of topk_wave.h.  The score
// arithmetic is float64 throughout, so selections agree with a float64
// statement of the rule except where scores tie to rounding.
#include "topk_wave.h"
#include "vsa_internal.h"

#include <atomic>

namespace vsa {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// grid (4 * n_c, ceil(H / 8)), 128 threads = 8 heads x 16 chunks of 8 dims.
// Block x = video tile u (tiles u >= n_v of the last group are written as
// zeros).  Each thread sums its 8 dims over each sub-block's 16 rows of Q and
// of K in float64 and writes the float32 means into the packed layout.
__global__ __launch_bounds__(128) void subpool_kernel(const uint16_t* __restrict__ q,
                                                      const uint16_t* __restrict__ k, int H,
                                                      int ldh, int64_t S_t, int n_v, int n_c,
                                                      float* __restrict__ qsub,
                                                      float* __restrict__ ksub) {
    const int u = blockIdx.x;
    const int h = blockIdx.y * 8 + (threadIdx.x >> 4);
    const int cc = threadIdx.x & 15;  // dims 8 cc .. 8 cc + 7
    if (h >= H) return;
    const int64_t rs = (int64_t)ldh * kD;
    const int grp = u >> 2;
    const int g = cc >> 2, i0 = 2 * (cc & 3);
    const int64_t gbase = ((int64_t)h * n_c + grp) * 8;  // in units of [64][4] floats
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const uint16_t* p = (t ? k : q) + (S_t + (int64_t)u * kT) * rs + (int64_t)h * kD + cc * 8;
        float4* out = (float4*)(t ? ksub : qsub);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            double acc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = 0.0;
            if (u < n_v) {
#pragma unroll 4
                for (int r = 16 * a; r < 16 * a + 16; ++r) {
                    const uint4 w = *(const uint4*)(p + (int64_t)r * rs);
                    acc[0] += (double)bf16_lo(w.x);
                    acc[1] += (double)bf16_hi(w.x);
                    acc[2] += (double)bf16_lo(w.y);
                    acc[3] += (double)bf16_hi(w.y);
                    acc[4] += (double)bf16_lo(w.z);
                    acc[5] += (double)bf16_hi(w.z);
                    acc[6] += (double)bf16_lo(w.w);
                    acc[7] += (double)bf16_hi(w.w);
                }
            }
            float m[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) m[e] = (float)(acc[e] * (1.0 / 16.0));
            const int lane = 16 * g + 4 * (u & 3) + a;
            out[(gbase + i0) * 64 + lane] = make_float4(m[0], m[1], m[2], m[3]);
            out[(gbase + i0 + 1) * 64 + lane] = make_float4(m[4], m[5], m[6], m[7]);
        }
    }
}

// One 16-row group of packed sub-block means (Qs or Ks) as this lane's 32
// float MFMA operands: element s is dim 32 (lane / 16) + s of row `row`
// (lane % 16 for the B operand; a permuted row for the A operand).
__device__ __forceinline__ void load_group(const float* __restrict__ base, int lane, int row,
                                           float (&x)[32]) {
    const float4* p = (const float4*)base + ((lane & 48) | row);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 t = p[64 * i];
        x[4 * i + 0] = t.x;
        x[4 * i + 1] = t.y;
        x[4 * i + 2] = t.z;
        x[4 * i + 3] = t.w;
    }
}

// Log-sum-exp of the 16 sub-block logits of each tile pair in one 16 x 16
// MFMA output tile.  The float64 16x16x4 MFMA leaves output row
// l / 16 + 4 v of column l % 16 in register v of lane l; lane l of the A
// operand therefore loads query sub-row sigma(l % 16), sigma(i) = 4 (i % 4) +
// i / 4, so that register v of lane l holds query sub-block a = v of query
// tile l / 16 against key sub-block l % 4 of key tile (l % 16) / 4.  The
// pair's 16 values sit in 4 adjacent lanes; every lane returns its pair's
// score.
__device__ __forceinline__ double pair_lse(const f64x4& acc) {
    constexpr double alpha = 0.088388347648318440550;  // 1/sqrt(128)
    const double x0 = alpha * acc[0], x1 = alpha * acc[1];
    const double x2 = alpha * acc[2], x3 = alpha * acc[3];
    double m = fmax(fmax(x0, x1), fmax(x2, x3));
    m = fmax(m, __shfl_xor(m, 1));
    m = fmax(m, __shfl_xor(m, 2));
    double e = exp(x0 - m) + exp(x1 - m) + exp(x2 - m) + exp(x3 - m);
    e += __shfl_xor(e, 1);
    e += __shfl_xor(e, 2);
    return m + log(e);
}

// grid (H * ceil(n_c / RT)), 512 threads = 8 wavefronts.  A workgroup owns
// RT groups of four query tiles of one head (4 RT rows of scores in LDS).
// Wavefront wv multiplies query group wv % RT against the key groups c with
// c % (8 / RT) == wv / RT, four key groups per step (four independent MFMA
// chains; two, then one, for the remainder), and stores the scores; then
// each wavefront selects rows wv, wv + 8.
// Blocks are mapped so that each XCD walks a contiguous, head-major range of
// (head, query block) items: the key means of one head (n_c * 8 KiB) stay in
// that XCD's L2 while its CUs share them.
template <int RT, int NS>
__global__ __launch_bounds__(512) void subblock_route_kernel(const float* __restrict__ qsub,
                                                             const float* __restrict__ ksub,
                                                             int H, int n_v, int n_c, int k,
                                                             int ldw, int32_t* __restrict__ sel) {
    extern __shared__ __align__(16) unsigned char smem[];
    double* sc = (double*)smem;  // [4 RT][ldw]
    constexpr int PH = 8 / RT;
    const int nub = (n_c + RT - 1) / RT;
    const int64_t items = (int64_t)H * nub;
    const int64_t b = blockIdx.x;
    const int64_t x8 = b & 7, q8 = items >> 3, r8 = items & 7;
    const int64_t item = x8 * q8 + (x8 < r8 ? x8 : r8) + (b >> 3);
    const int h = (int)(item / nub);
    const int ub = (int)(item % nub);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rt = wv % RT, ph = wv / RT;
    const int cq = ub * RT + rt;

    if (cq < n_c) {
        float a[32];
        const int arow = ((lane & 3) << 2) | ((lane >> 2) & 3);  // sigma(lane % 16)
        load_group(qsub + ((int64_t)h * n_c + cq) * 2048, lane, arow, a);
        // rows of query tiles past n_v (last group) are zero
        if (4 * cq + (arow >> 2) >= n_v) {
#pragma unroll
            for (int s = 0; s < 32; ++s) a[s] = 0.0f;
        }
        const float* kh = ksub + (int64_t)h * n_c * 2048;
        const int uq = 4 * cq + (lane >> 4);  // this lane's query tile
        const int lrow = 4 * rt + (lane >> 4);
        const bool store_lane = (lane & 3) == 0 && uq < n_v;
        auto finish = [&](const f64x4& acc, int c) {
            const double s = pair_lse(acc);
            const int w = 4 * c + ((lane & 15) >> 2);
            if (store_lane && w < n_v) sc[lrow * ldw + w] = s + 0.0;
        };
        int c = ph;
        for (; c + 3 * PH < n_c; c += 4 * PH) {
            float bq[4][32];
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                load_group(kh + (int64_t)(c + gq * PH) * 2048, lane, lane & 15, bq[gq]);
                if (4 * (c + gq * PH) + ((lane & 15) >> 2) >= n_v) {
#pragma unroll
                    for (int s = 0; s < 32; ++s) bq[gq][s] = 0.0f;
                }
            }
            f64x4 accq[4];
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) accq[gq] = (f64x4){0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int s = 0; s < 32; ++s) {
                const double as = (double)a[s];
#pragma unroll
                for (int gq = 0; gq < 4; ++gq)
                    accq[gq] = __builtin_amdgcn_mfma_f64_16x16x4f64(as, (double)bq[gq][s], accq[gq], 0, 0, 0);
            }
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) finish(accq[gq], c + gq * PH);
        }
        for (; c + PH < n_c; c += 2 * PH) {
            float b0[32], b1[32];
            load_group(kh + (int64_t)c * 2048, lane, lane & 15, b0);
            load_group(kh + (int64_t)(c + PH) * 2048, lane, lane & 15, b1);
            if (4 * (c + PH) + ((lane & 15) >> 2) >= n_v) {
#pragma unroll
                for (int s = 0; s < 32; ++s) b1[s] = 0.0f;
            }
            f64x4 acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = acc0;
#pragma unroll
            for (int s = 0; s < 32; ++s) {
                const double as = (double)a[s];
                acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(as, (double)b0[s], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(as, (double)b1[s], acc1, 0, 0, 0);
            }
            finish(acc0, c);
            finish(acc1, c + PH);
        }
        if (c < n_c) {
            float b0[32];
            load_group(kh + (int64_t)c * 2048, lane, lane & 15, b0);
            if (4 * c + ((lane & 15) >> 2) >= n_v) {
#pragma unroll
                for (int s = 0; s < 32; ++s) b0[s] = 0.0f;
            }
            f64x4 acc0 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int s = 0; s < 32; ++s)
                acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a[s], (double)b0[s], acc0, 0, 0, 0);
            finish(acc0, c);
        }
    }
    __syncthreads();

    // ---- exact top-k of each score row: one wavefront per row ------------
    for (int r = wv; r < 4 * RT; r += 8) {
        const int u = 4 * ub * RT + r;
        if (u >= n_v) break;
        const double* row = sc + r * ldw;
        uint32_t need = 0;
        const uint64_t kth = kth_key_bisect<NS>(row, n_v, k, lane, need);
        emit_topk(row, n_v, k, kth, need, lane, sel + ((int64_t)h * n_v + u) * k);
    }
}

template <int RT, int NS>
hipError_t launch_route(const Shape& s, int32_t* sel, const uint8_t* ws, const Layout& L,
                        hipStream_t stream) {
    const int n_c = (s.n_v + 3) / 4;
    const int ldw = (s.n_v + 3) & ~3;
    const size_t lds = (size_t)4 * RT * ldw * sizeof(double);
    static std::atomic<size_t> lds_allowed[kMaxDevices];
    hipError_t e = ensure_dynamic_lds((const void*)subblock_route_kernel<RT, NS>, lds_allowed, lds);
    if (e != hipSuccess) return e;
    const int64_t blocks = (int64_t)s.H * ((n_c + RT - 1) / RT);
    hipLaunchKernelGGL((subblock_route_kernel<RT, NS>), dim3((unsigned)blocks), dim3(512), lds,
                       stream, (const float*)(ws + L.qsub), (const float*)(ws + L.ksub), s.H,
                       s.n_v, n_c, s.k, ldw, sel);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_subblock_route(const uint16_t* q, const uint16_t* k, const Shape& s,
                                 int32_t* sel, uint8_t* ws, const Layout& L, hipStream_t stream) {
    if (s.n_v == 0) return hipSuccess;
    const int n_c = (s.n_v + 3) / 4;
    hipLaunchKernelGGL(subpool_kernel, dim3(4 * n_c, (s.H + 7) / 8), dim3(128), 0, stream, q, k,
                       s.H, s.ldh, s.S_t, s.n_v, n_c, (float*)(ws + L.qsub), (float*)(ws + L.ksub));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // rows of 4 RT query tiles x ldw float64 scores must fit the 160 KiB of LDS
    if (s.n_v <= 1280) return launch_route<4, 20>(s, sel, ws, L, stream);
    if (s.n_v <= 2560) return launch_route<2, 40>(s, sel, ws, L, stream);
    return launch_route<1, 80>(s, sel, ws, L, stream);
}

}  // namespace vsa

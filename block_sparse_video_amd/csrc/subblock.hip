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
// per-lane order of the MFMA operands of stage 2, so each operand load there
// is a contiguous 1 KiB wavefront read.  Packed layout per head and group c
// of four video tiles (16 sub-block rows j = 4 * (u % 4) + a):
//   [c][i = 0..7][lane = 16 g + j][e = 0..3] = mean of row j, dim 32 g + 4 i + e.
// Stage 2 (subblock_route_kernel) is a float32 MFMA product Qs Ks^T per head
// (16 x 16 x 4 tiles: four query tiles x four key tiles per output tile, the
// 16 sub-block pairs of one tile pair in 4 lanes x 4 registers), the float32
// log-sum-exp of each tile pair in registers, one row of score slots per
// query tile in LDS (each score with a proven bound on its distance from the
// float64 score of the definition), and a wavefront top-k that takes every
// key the bounds decide and ranks the undecided band by recomputed float64
// scores.  Selections therefore agree with the float64 statement of the rule
// except where float64 scores tie to rounding.
#include "topk_wave.h"
#include "vsa_internal.h"

#include <atomic>

namespace vsa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

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
// (lane % 16 for both operands).  Returns the sum of their squares.
__device__ __forceinline__ float load_group(const float* __restrict__ base, int lane, int row,
                                            float (&x)[32]) {
    const float4* p = (const float4*)base + ((lane & 48) | row);
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 t = p[64 * i];
        x[4 * i + 0] = t.x;
        x[4 * i + 1] = t.y;
        x[4 * i + 2] = t.z;
        x[4 * i + 3] = t.w;
        ss = fmaf(t.x, t.x, fmaf(t.y, t.y, fmaf(t.z, t.z, fmaf(t.w, t.w, ss))));
    }
    return ss;
}

// Largest |row| of the four sub-block rows of each tile of a 16-row group:
// the four lane groups' partial sums of squares added (lanes 16 g + j hold
// row j), then the maximum over the tile's rows j = 4 t .. 4 t + 3.  Every
// lane returns the value of tile (lane % 16) / 4.
__device__ __forceinline__ float tile_max_norm2(float ss) {
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    ss = fmaxf(ss, __shfl_xor(ss, 1));
    return fmaxf(ss, __shfl_xor(ss, 2));
}

constexpr double kAlphaR = 0.088388347648318440550;  // 1/sqrt(128)

// Log-sum-exp of the 16 sub-block logits of each tile pair in one 16 x 16
// output tile.  The float32 16x16x4 MFMA leaves output row 4 (l / 16) + v of
// column l % 16 in register v of lane l; with the operand rows in their
// natural order (row 4 t + a = sub-block a of tile t of the group), register
// v of lane l holds query sub-block a = v of query tile l / 16 against key
// sub-block l % 4 of key tile (l % 16) / 4.  The pair's 16 values sit in 4
// adjacent lanes; every lane returns its pair's score.  Float32 throughout:
// the logits rounded once, expf and logf within 3 ulp as OpenCL requires of
// them; kLse32 bounds the result's error.
__device__ __forceinline__ float pair_lse(const f32x4& acc) {
    // no multiply-add contraction: x - m must subtract the rounded logits the
    // maximum was taken over (fused, the maximum's own term would be its
    // product's rounding error, which overflows exp at large magnitudes)
#pragma clang fp contract(off)
    constexpr float alpha = (float)kAlphaR;
    const float x0 = alpha * acc[0], x1 = alpha * acc[1];
    const float x2 = alpha * acc[2], x3 = alpha * acc[3];
    float m = fmaxf(fmaxf(x0, x1), fmaxf(x2, x3));
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    float e = expf(x0 - m) + expf(x1 - m) + expf(x2 - m) + expf(x3 - m);
    e += __shfl_xor(e, 1);
    e += __shfl_xor(e, 2);
    return m + logf(e);
}

// Logits: each is one chain of 32 float32 MFMAs (128 products).  A 128-term
// float32 dot product in any order and rounding mode is within gamma_128 =
// 128u / (1 - 128u), u = 2^-23, of the sum of |products|, which
// Cauchy-Schwarz bounds by |Qs[u][a]| |Ks[w][b]|; so every computed logit of
// a tile pair is within
//   alpha * kLogitErr * max_a |Qs[u][a]| * max_b |Ks[w][b]|
// (+ a term for flushed denormals) of the float64 logit, and the log-sum-exp,
// 1-Lipschitz in the max norm, moves by no more.  (Shorter chains added in
// float64 narrow the bound but cost more than the recomputes they save.)
constexpr double kLogitErr = 1.6e-5;  // gamma_128 = 1.526e-5; float32 norms
constexpr double kLogitDenorm = 0x1p-117;
// Error of the float32 log-sum-exp given its float64 logits, beside the
// 2^-22 |score| of rounding the logits, the maximum and the final sum: the
// differences x - m rounded (their relative 2^-24 |t| moves each term e^t by
// at most 2^-24 / e of the sum, which is >= 1), expf and logf within 3 ulp,
// 15 float32 additions of terms in (0, 1]; about 3.5e-6 in all, so 1e-5.  The
// float64 recompute of a band key is within ~1e-15 of the definition.
constexpr double kLse32 = 1e-5;

template <int NG>
__device__ __forceinline__ void logit_chains(const float (&a)[32], const float (&bq)[NG][32],
                                             f32x4 (&acc)[NG]) {
#pragma unroll
    for (int g = 0; g < NG; ++g) acc[g] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 32; ++s)
#pragma unroll
        for (int g = 0; g < NG; ++g)
            acc[g] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], bq[g][s], acc[g], 0, 0, 0);
}

// A score slot of the LDS rows: the stored float32 score (low word) and a
// bound on its distance from the float64 score (high word, rounded up).
__device__ __forceinline__ uint64_t pack_slot(float s, double bound) {
    const float sf = s + 0.0f;
    const double e = bound;
    float ef = (float)e;
    if ((double)ef < e) ef = __uint_as_float(__float_as_uint(ef) + 1u);  // round up (e >= 0)
    if (!(e < 0x1p100)) ef = INFINITY;
    return ((uint64_t)__float_as_uint(ef) << 32) | __float_as_uint(sf);
}

// The float64 score of (query tile u, key tile w) of one head, computed by
// the whole wavefront: lane l forms logit p = l % 16 (query sub-block p / 4,
// key sub-block p % 4) over dims 32 (l / 16) .. + 31, the four partial dot
// products are added, and the 16 logits' max + log of summed exponentials
// follows in float64.  Every lane returns the score.  q_h, k_h: the head's
// packed sub-block means.
__device__ double score_f64(const float* __restrict__ q_h, const float* __restrict__ k_h, int u,
                            int w, int lane) {
#pragma clang fp contract(off)  // as in pair_lse: x - m on the rounded logits
    const int p = lane & 15, c4 = lane >> 4;
    const float* qr = q_h + (int64_t)(u >> 2) * 2048 + 64 * c4 + 4 * (4 * (u & 3) + (p >> 2));
    const float* kr = k_h + (int64_t)(w >> 2) * 2048 + 64 * c4 + 4 * (4 * (w & 3) + (p & 3));
    double dot = 0.0;
#pragma unroll 2
    for (int i = 0; i < 8; ++i) {
        const float4 q4 = *(const float4*)(qr + 256 * i);
        const float4 k4 = *(const float4*)(kr + 256 * i);
        dot = __builtin_fma((double)q4.x, (double)k4.x, dot);
        dot = __builtin_fma((double)q4.y, (double)k4.y, dot);
        dot = __builtin_fma((double)q4.z, (double)k4.z, dot);
        dot = __builtin_fma((double)q4.w, (double)k4.w, dot);
    }
    dot += __shfl_xor(dot, 16);
    dot += __shfl_xor(dot, 32);
    const double x = kAlphaR * dot;
    double m = x;
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off));
    double e = exp(x - m);
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) e += __shfl_xor(e, off);
    return m + log(e);
}

// Selection of one row (query tile u) from its score slots.  With E the
// row's largest bound and T the k-th largest stored score, every key stored
// above T + 2E is in the exact top k by float64 score and every key below
// T - 2E is not (at least k keys have a float64 score >= T - E, at most
// k - 1 one > T + E); the keys in between (the band) are ranked by their
// recomputed float64 scores when they outnumber the places left, ties to the
// lower index.  zero_q: every logit of the row is exactly 0, so every stored
// score is the same value and the lowest k indices are the selection.
template <int NS>
__device__ void select_row_band(uint64_t* row, int n_v, int k, bool zero_q, int lane,
                                const float* __restrict__ q_h, const float* __restrict__ k_h,
                                int u, int32_t* __restrict__ out) {
    static_assert(NS <= 128, "band masks hold 128 slots");
    if (zero_q) {
        for (int i = lane; i < k; i += 64) out[i] = i;
        return;
    }
    uint32_t kv[NS];
    float emax = 0.0f;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int w = lane + 64 * i;
        kv[i] = 0u;
        if (w < n_v) {
            const uint64_t sl = row[w];
            kv[i] = order_key32(__uint_as_float((uint32_t)sl));
            emax = fmaxf(emax, __uint_as_float((uint32_t)(sl >> 32)));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) emax = fmaxf(emax, __shfl_xor(emax, off));
    uint32_t gt;
    const uint32_t t = kth_largest(kv, (uint32_t)k, gt);
    uint32_t lo = 1u, hi = 0xFFFFFFFFu;
    if (emax < 0x1p100f) {
        const double T = (double)key32_value(t);
        lo = key32_at_or_below(T - 2.0 * (double)emax);
        hi = key32_at_or_above(T + 2.0 * (double)emax);
    }
    uint64_t above_m[2] = {0ull, 0ull}, band_m[2] = {0ull, 0ull};
    uint32_t above = 0, band = 0;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const bool ab = kv[i] > hi, bd = kv[i] != 0u && kv[i] >= lo && kv[i] <= hi;
        above_m[i >> 6] |= (uint64_t)ab << (i & 63);
        band_m[i >> 6] |= (uint64_t)bd << (i & 63);
        above += (uint32_t)__popcll(__ballot(ab));
        band += (uint32_t)__popcll(__ballot(bd));
    }
    uint32_t need = (uint32_t)k - above;
    if (band < need) {
        // cannot happen while the bounds hold: rank the whole row instead
        above_m[0] = above_m[1] = band_m[0] = band_m[1] = 0ull;
#pragma unroll
        for (int i = 0; i < NS; ++i)
            if (kv[i] != 0u) band_m[i >> 6] |= 1ull << (i & 63);
        need = (uint32_t)k;
        band = (uint32_t)n_v;
    }
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    if (band == need) {
        uint32_t outc = 0;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const bool take = ((above_m[i >> 6] | band_m[i >> 6]) >> (i & 63)) & 1ull;
            const uint64_t tm = __ballot(take);
            const uint32_t pos = outc + (uint32_t)__popcll(tm & lt_mask);
            if (take && pos < (uint32_t)k) out[pos] = lane + 64 * i;
            outc += (uint32_t)__popcll(tm);
        }
        return;
    }
    // the band's float64 scores are recomputed, member j's (order key, index)
    // kept in lane j, and member j is taken if fewer than `need` members come
    // before it in the order (score desc, index asc); its slot then holds 1,
    // else 0 (this wavefront owns the row).  A band of more than 64 keys
    // (rows of nearly equal scores) is ranked by bisection on the recomputed
    // keys held in the slots.
    auto in_band = [&](int i) -> bool { return ((i < 64 ? band_m[0] : band_m[1]) >> (i & 63)) & 1ull; };
    uint64_t mkey = 0ull;
    int mw = 0x7FFFFFFF;
    uint32_t nb = 0;
#pragma unroll 1
    for (int i = 0; i < NS; ++i) {
        uint64_t todo = __ballot(in_band(i));
        while (todo) {
            const int ln = __builtin_ctzll(todo);  // wave-uniform
            todo &= todo - 1ull;
            const int w = ln + 64 * i;
            const uint64_t key = order_key(score_f64(q_h, k_h, u, w, lane) + 0.0);
            if (band <= 64) {
                if (lane == (int)nb) {
                    mkey = key;
                    mw = w;
                }
            } else if (lane == ln) {
                row[w] = key;
            }
            ++nb;
        }
    }
    if (band <= 64) {
        uint32_t before = 0;
        for (uint32_t j = 0; j < nb; ++j) {
            const uint64_t kj = __shfl(mkey, (int)j);
            const int wj = __shfl(mw, (int)j);
            before += (kj > mkey || (kj == mkey && wj < mw)) ? 1u : 0u;
        }
        if ((uint32_t)lane < nb) row[mw] = before < need ? 1ull : 0ull;
    } else {
        uint64_t bmin = ~0ull, bmax = 0ull;
#pragma unroll 1
        for (int i = 0; i < NS; ++i)
            if (in_band(i)) {
                const uint64_t key = row[lane + 64 * i];
                bmin = key < bmin ? key : bmin;
                bmax = key > bmax ? key : bmax;
            }
#pragma unroll 1
        for (int off = 32; off >= 1; off >>= 1) {
            const uint64_t x = __shfl_xor(bmin, off), y = __shfl_xor(bmax, off);
            bmin = x < bmin ? x : bmin;
            bmax = y > bmax ? y : bmax;
        }
        bmin = uniform_key(bmin);
        bmax = uniform_key(bmax);
        auto count_ge = [&](uint64_t th) -> uint32_t {
            uint32_t c = 0;
#pragma unroll 1
            for (int i = 0; i < NS; ++i)
                c += (uint32_t)__popcll(__ballot(in_band(i) && row[lane + 64 * i] >= th));
            return c;
        };
        // the need-th largest band key: the largest th with count_ge(th) >= need
        uint64_t blo = bmin, bhi = bmax;
        while (blo < bhi) {
            const uint64_t mid = blo + ((bhi - blo + 1) >> 1);
            if (count_ge(mid) >= need) blo = mid;
            else bhi = mid - 1;
        }
        uint32_t bgt = 0;
#pragma unroll 1
        for (int i = 0; i < NS; ++i)
            bgt += (uint32_t)__popcll(__ballot(in_band(i) && row[lane + 64 * i] > blo));
        const uint32_t take_eq = need - bgt;  // band keys equal to blo to take, lowest index first
        uint32_t eqseen = 0;
#pragma unroll 1
        for (int i = 0; i < NS; ++i) {
            const int w = lane + 64 * i;
            const bool bd = in_band(i);
            const uint64_t key = bd ? row[w] : 0ull;
            const bool eq = bd && key == blo;
            const uint64_t em = __ballot(eq);
            const uint32_t erank = eqseen + (uint32_t)__popcll(em & lt_mask);
            if (bd) row[w] = (key > blo || (eq && erank < take_eq)) ? 1ull : 0ull;
            eqseen += (uint32_t)__popcll(em);
        }
    }
    uint32_t outc = 0;
#pragma unroll 1
    for (int i = 0; i < NS; ++i) {
        const int w = lane + 64 * i;
        const bool ab = ((i < 64 ? above_m[0] : above_m[1]) >> (i & 63)) & 1ull;
        const bool take = ab || (in_band(i) && row[w] == 1ull);
        const uint64_t tm = __ballot(take);
        const uint32_t pos = outc + (uint32_t)__popcll(tm & lt_mask);
        if (take && pos < (uint32_t)k) out[pos] = w;
        outc += (uint32_t)__popcll(tm);
    }
}

// grid (H * ceil(n_c / RT)), 512 threads = 8 wavefronts.  A workgroup owns
// RT groups of four query tiles of one head (4 RT rows of score slots in
// LDS).  Wavefront wv multiplies query group wv % RT against the key groups
// c with c % (8 / RT) == wv / RT, one key group per step with the next
// step's group loaded while this step's log-sum-exps run, and stores the
// slots; then each wavefront selects rows wv, wv + 8.  MINB workgroups share
// a CU (the registers are capped for it): with two, one workgroup's top-k
// runs beside the other's matrix work.
// Blocks are mapped so that each XCD walks a contiguous, head-major range of
// (head, query block) items: the key means of one head (n_c * 8 KiB) stay in
// that XCD's L2 while its CUs share them.
template <int RT, int NS, int MINB>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2 * MINB))) void
subblock_route_kernel(const float* __restrict__ qsub, const float* __restrict__ ksub, int H,
                      int n_v, int n_c, int k, int ldw, int32_t* __restrict__ sel) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint64_t* sc = (uint64_t*)smem;  // [4 RT][ldw] score slots
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
    const float* qh = qsub + (int64_t)h * n_c * 2048;
    const float* kh = ksub + (int64_t)h * n_c * 2048;

    if (cq < n_c) {
        float a[32];
        const int arow = lane & 15;
        float qq = load_group(qh + (int64_t)cq * 2048, lane, arow, a);
        // rows of query tiles past n_v (last group) are zero
        if (4 * cq + (arow >> 2) >= n_v) {
#pragma unroll
            for (int s = 0; s < 32; ++s) a[s] = 0.0f;
            qq = 0.0f;
        }
        // max_a |Qs[u][a]| of this lane's output query tile, lane / 16
        const double qmax = sqrt((double)__shfl(tile_max_norm2(qq), 4 * (lane >> 4)));
        const int uq = 4 * cq + (lane >> 4);
        const int lrow = 4 * rt + (lane >> 4);
        const bool store_lane = (lane & 3) == 0 && uq < n_v;
        // kn: max_b |Ks[w][b]| of this lane's output key tile, (lane % 16) / 4
        auto finish = [&](const f32x4& acc, int c, double kn) {
            const float s = pair_lse(acc);
            const int w = 4 * c + ((lane & 15) >> 2);
            if (store_lane && w < n_v) {
                const double qk = qmax * kn;
                const double bound = kAlphaR * (kLogitErr * qk + kLogitDenorm * (qmax + kn + 1.0)) +
                                     kLse32 + 0x1p-22 * fabs((double)s);
                sc[lrow * ldw + w] = pack_slot(s, qk < 0x1p100 ? bound : INFINITY);
            }
        };
        // key groups: the packed means of tiles past n_v are zero (subpool)
        auto issue_keys = [&](int c, float (&bq)[32]) {
            const float4* p = (const float4*)(kh + (int64_t)c * 2048) + lane;  // row lane % 16, dims 32 (lane / 16) + ...
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 t = p[64 * i];
                bq[4 * i + 0] = t.x;
                bq[4 * i + 1] = t.y;
                bq[4 * i + 2] = t.z;
                bq[4 * i + 3] = t.w;
            }
        };
        auto key_norm = [&](const float (&bq)[32]) -> double {
            float ss = 0.0f;
#pragma unroll
            for (int s = 0; s < 32; ++s) ss = fmaf(bq[s], bq[s], ss);
            return sqrt((double)tile_max_norm2(ss));
        };
        // one key group per step; the next step's group is loaded while this
        // step's log-sum-exps run
        float bq[1][32];
        if (ph < n_c) issue_keys(ph, bq[0]);
        for (int c = ph; c < n_c; c += PH) {
            const double kn = key_norm(bq[0]);
            f32x4 acc[1];
            logit_chains<1>(a, bq, acc);
            __builtin_amdgcn_sched_barrier(0);
            if (c + PH < n_c) issue_keys(c + PH, bq[0]);
            __builtin_amdgcn_sched_barrier(0);
            finish(acc[0], c, kn);
        }
    }
    __syncthreads();

    // ---- exact top-k of each score row: one wavefront per row ------------
    for (int r = wv; r < 4 * RT; r += 8) {
        const int u = 4 * ub * RT + r;
        if (u >= n_v) break;
        // is the whole query tile zero (every logit of the row exactly 0)?
        // (lane 4 g + a < 16 reads dims 32 g + 4 i .. + 3 of sub-block a)
        const float* qg = qh + (int64_t)(u >> 2) * 2048 + 16 * (u & 3);
        bool nz = false;
        if (lane < 16)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 t = *(const float4*)(qg + i * 256 + 64 * (lane >> 2) + 4 * (lane & 3));
                nz |= t.x != 0.0f || t.y != 0.0f || t.z != 0.0f || t.w != 0.0f;
            }
        const bool zero_q = __ballot(nz) == 0ull;
        select_row_band<NS>(sc + r * ldw, n_v, k, zero_q, lane, qh, kh, u,
                            sel + ((int64_t)h * n_v + u) * k);
    }
}

template <int RT, int NS, int MINB>
hipError_t launch_route(const Shape& s, int32_t* sel, const uint8_t* ws, const Layout& L,
                        hipStream_t stream) {
    const int n_c = (s.n_v + 3) / 4;
    const int ldw = (s.n_v + 3) & ~3;
    const size_t lds = (size_t)4 * RT * ldw * sizeof(uint64_t);
    static std::atomic<size_t> lds_allowed[kMaxDevices];
    hipError_t e = ensure_dynamic_lds((const void*)subblock_route_kernel<RT, NS, MINB>, lds_allowed, lds);
    if (e != hipSuccess) return e;
    const int64_t blocks = (int64_t)s.H * ((n_c + RT - 1) / RT);
    hipLaunchKernelGGL((subblock_route_kernel<RT, NS, MINB>), dim3((unsigned)blocks), dim3(512), lds,
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
    // rows of 4 RT query tiles x ldw 8-byte score slots must fit the LDS:
    // two workgroups per CU (80 KiB each) up to 1,280 tiles, then one
    if (s.n_v <= 1280) return launch_route<2, 20, 2>(s, sel, ws, L, stream);
    if (s.n_v <= 2560) return launch_route<2, 40, 1>(s, sel, ws, L, stream);
    return launch_route<1, 80, 1>(s, sel, ws, L, stream);
}

}  // namespace vsa

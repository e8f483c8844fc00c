// pool_pack.hip -- stage 1 of the VSA forward on gfx950: FP32 tile pooling of
// Q, K, V over the video tiles, and packing of K and V tiles for the attention stage.
//
// Page "UniServe: serving FastH3 at its fastest", section "Fused attention
// preprocessing": the preprocessing pass pools tiles into FP32 statistics and
// packs tiles into the layout the attention kernels read.  Here:
//   pooled X[h][u][d] = float32( (sum over the 64 rows r, in row order, in
//                                 float64, of X[S_t + 64u + r][h][d]) / 64 )
// The float64 sum of 64 bfloat16 values is exact for any inputs whose
// magnitudes within one tile span less than 2^45, so the statistic is the
// correctly rounded mean; the row order makes it reproducible regardless.
//
// HBM-bound: Q video rows are read once for pooling, K and V of every tile are
// read once and written once more in the attention stage's operand order
// (coalesced 16-byte accesses).
#include "vsa_internal.h"

namespace vsa {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// grid (n_v, ceil(H/8)): pools Q over the video tiles.  128 threads = 8
// heads x 16 column chunks of 8 dims; each thread walks the tile's valid rows
// (64, or fewer in the segment's last tile) and divides by their count.
__global__ __launch_bounds__(128) void pool_q_kernel(const uint16_t* __restrict__ q, int H,
                                                     int ldh, int64_t S_t, int n_v, int64_t V_v,
                                                     double* __restrict__ qbar64) {
    const int u = blockIdx.x;
    const int h = blockIdx.y * 8 + (threadIdx.x >> 4);
    const int c = threadIdx.x & 15;
    if (h >= H) return;
    const int64_t rem = V_v - (int64_t)u * kT;
    const int n = rem >= kT ? kT : (int)rem;
    const int64_t rs = (int64_t)ldh * kD;
    const uint16_t* p = q + (S_t + (int64_t)u * kT) * rs + (int64_t)h * kD + c * 8;
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll 16
    for (int r = 0; r < n; ++r) {
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
    double* o = qbar64 + ((int64_t)h * n_v + u) * kD;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[pooled_dim_pos(c * 8 + e)] = (double)(float)(acc[e] / (double)n);
}

// ---- attention preprocessing: learned RMSNorm and partial 3D RoPE ---------
// Page "UniServe: serving FastH3 at its fastest", section "Fused attention
// preprocessing" (learned Q/K RMSNorm and partial RoPE before tile pooling,
// padding handled inside the kernel); the SGLang Diffusion benchmark page
// gives RoPE dimension 96 and the rounding order (normalised value rounded to
// bf16 before RoPE).  Per head and token: y = bf16(x / sqrt(mean(x^2) + 1e-6)
// * gamma); video tokens then turn dims 0..95 -- axis a in (t, h, w) owns dims
// 32a .. 32a+31 as 16 interleaved pairs (2i, 2i+1) -- by pos_a * 10000^(-i/16)
// and round to bf16 again.  Text and audio tokens are not rotated; padding
// rows become zeros.  Arithmetic in fp32.
constexpr float kRmsEps = 1e-6f;

struct PrepArgs {
    const uint16_t* gamma;  // [H][128]
    int gt, gh, gw;         // latent grid of the valid video tokens
    int pt, ph, pw;         // tile-packing shape
};

// Latent-grid position of video token i (tile-packed order: tiles of
// pt x ph x pw points in raster order, raster order inside a tile).
__device__ __forceinline__ void video_pos(const PrepArgs& a, int64_t i, int& t, int& h, int& w) {
    const int pts = a.pt * a.ph * a.pw;
    const int64_t tile = i / pts;
    const int off = (int)(i - tile * pts);
    const int nth = a.gh / a.ph, ntw = a.gw / a.pw;
    const int tt = (int)(tile / ((int64_t)nth * ntw));
    const int th = (int)((tile / ntw) % nth), tw = (int)(tile % ntw);
    t = tt * a.pt + off / (a.ph * a.pw);
    h = th * a.ph + (off / a.pw) % a.ph;
    w = tw * a.pw + off % a.pw;
}

// Rotate dims d0 .. d0+7 (d0 a multiple of 8, < 96) of one token in place:
// 4 pairs of axis d0 / 32, frequency index (d0 % 32) / 2 + p.
__device__ __forceinline__ void rope8(float (&y)[8], int d0, int pos) {
    const int i0 = (d0 & 31) >> 1;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        // 10000^(-i/16) = 2^(-i * log2(10000) / 16)
        const float theta = exp2f(-(float)(i0 + p) * 0.83048202372184058696f);
        float sn, cs;
        sincosf((float)pos * theta, &sn, &cs);
        const float a = y[2 * p], b = y[2 * p + 1];
        y[2 * p] = a * cs - b * sn;
        y[2 * p + 1] = a * sn + b * cs;
    }
}

__device__ __forceinline__ float bf16_round_f(float x) {
    return (float)(__bf16)x;  // round to nearest even
}

// grid (N, ceil(H/8)), 128 threads = 8 heads x 16 chunks of 8 dims.  For every
// row of the tile: RMSNorm (+ RoPE for video tokens) of Q into q_out, and for
// video tiles the FP32 mean of the preprocessed rows over the valid ones.
__global__ __launch_bounds__(128) void prep_q_kernel(const uint16_t* __restrict__ q,
                                                     PrepArgs pa, int H, int ldh, int n_t, int n_v,
                                                     int64_t S_t, int64_t V_t, int64_t V_v,
                                                     int64_t V_a, int64_t S_v,
                                                     uint16_t* __restrict__ q_out,
                                                     double* __restrict__ qbar64) {
    const int j = blockIdx.x;
    const int h = blockIdx.y * 8 + (threadIdx.x >> 4);
    const int c = threadIdx.x & 15;
    const bool active = h < H;
    const int hh = active ? h : H - 1;
    const int64_t rs = (int64_t)ldh * kD;
    const bool video = j >= n_t && j < n_t + n_v;
    // first token row of the tile and its valid rows
    int64_t row0, valid;
    if (j < n_t) { row0 = (int64_t)j * kT; valid = V_t - row0; }
    else if (video) { row0 = S_t + (int64_t)(j - n_t) * kT; valid = V_v - (row0 - S_t); }
    else { const int64_t a0 = (int64_t)(j - n_t - n_v) * kT; row0 = S_t + S_v + a0; valid = V_a - a0; }
    const int n = valid >= kT ? kT : (valid > 0 ? (int)valid : 0);
    float g[8];
    {
        const uint4 gw = *(const uint4*)(pa.gamma + (int64_t)hh * kD + c * 8);
        g[0] = bf16_lo(gw.x); g[1] = bf16_hi(gw.x); g[2] = bf16_lo(gw.y); g[3] = bf16_hi(gw.y);
        g[4] = bf16_lo(gw.z); g[5] = bf16_hi(gw.z); g[6] = bf16_lo(gw.w); g[7] = bf16_hi(gw.w);
    }
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    for (int r = 0; r < kT; ++r) {
        const int64_t off = (row0 + r) * rs + (int64_t)hh * kD + c * 8;
        float y[8];
        if (r < n) {
            const uint4 w = *(const uint4*)(q + off);
            float x[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                          bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
            // sum over the 16 lanes of this head (consecutive lanes of one wave)
            ss += __shfl_xor(ss, 1);
            ss += __shfl_xor(ss, 2);
            ss += __shfl_xor(ss, 4);
            ss += __shfl_xor(ss, 8);
            const float inv = 1.0f / sqrtf(ss * (1.0f / kD) + kRmsEps);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = bf16_round_f(x[e] * inv * g[e]);
            if (video && c < 12) {
                int pt, ph, pw;
                video_pos(pa, row0 - S_t + r, pt, ph, pw);
                const int axis = c >> 2;
                rope8(y, c * 8, axis == 0 ? pt : (axis == 1 ? ph : pw));
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = bf16_round_f(y[e]);
            }
            if (video) {
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += (double)y[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = 0.0f;
        }
        if (active) {
            typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
            typedef float f32x8_t __attribute__((ext_vector_type(8)));
            const f32x8_t v = {y[0], y[1], y[2], y[3], y[4], y[5], y[6], y[7]};
            *(bf16x8_t*)(q_out + off) = __builtin_convertvector(v, bf16x8_t);
        }
    }
    if (video && active) {
        double* o = qbar64 + ((int64_t)h * n_v + (j - n_t)) * kD;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[pooled_dim_pos(c * 8 + e)] = (double)(float)(acc[e] / (double)n);
    }
}

// Key order inside a packed half-tile: operand row r holds key kappa(r), r
// with bits 2 and 3 swapped (see fine_attn.hip for why).
__device__ __forceinline__ int kappa(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// grid (N, H), 256 threads.  Loads one 64-token K tile and V tile of one head
// into LDS, writes the pooled K and V means (video tiles), and writes both
// tiles in the exact per-lane order of the attention stage's MFMA operands,
// so that every operand load there is one contiguous 1 KiB wavefront read:
//   K: [half][s = 0..7][lane][8]: lane (r = lane%32, g = lane/32) holds
//      K[key 32*half + kappa(r)][dims 16s + 8g .. 16s + 8g + 7];
//   V: [half][db = 0..3][m = 0..1][lane][8]: lane (c = lane%32, g) holds
//      V[keys 32*half + 16m + 8g .. +7][dim 32*db + c].
constexpr int kPitch = kD + 8;  // LDS row pitch in bf16 elements (272 bytes)

__global__ __launch_bounds__(256) void pack_kv_kernel(const uint16_t* __restrict__ k,
                                                      const uint16_t* __restrict__ v, int H,
                                                      int ldh, int n_t, int n_v, int N, int64_t S_t,
                                                      int64_t S_v, int64_t V_t, int64_t V_v,
                                                      int64_t V_a, PrepArgs pa, int pool,
                                                      float* __restrict__ kbar,
                                                      float* __restrict__ vbar,
                                                      uint16_t* __restrict__ kpack,
                                                      uint16_t* __restrict__ vpack) {
    __shared__ __align__(16) uint16_t ktile[kT * kPitch];
    __shared__ __align__(16) uint16_t vtile[kT * kPitch];
    const int t = blockIdx.x;
    const int h = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t rs = (int64_t)ldh * kD;
    const int64_t src = (int64_t)t * kT * rs + (int64_t)h * kD;
    // valid rows of this tile; padding rows are stored as zeros
    int64_t valid;
    if (t < n_t) valid = V_t - (int64_t)t * kT;
    else if (t < n_t + n_v) valid = V_v - (int64_t)(t - n_t) * kT;
    else valid = V_a - (int64_t)(t - n_t - n_v) * kT;
    const int n = valid >= kT ? kT : (valid > 0 ? (int)valid : 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int id = tid + 256 * i;
        const int r = id >> 4, c = id & 15;
        uint4 kw = make_uint4(0, 0, 0, 0), vw = kw;
        if (r < n) {
            kw = *(const uint4*)(k + src + (int64_t)r * rs + c * 8);
            vw = *(const uint4*)(v + src + (int64_t)r * rs + c * 8);
        }
        *(uint4*)(ktile + r * kPitch + c * 8) = kw;
        *(uint4*)(vtile + r * kPitch + c * 8) = vw;
    }
    __syncthreads();
    if (pa.gamma) {
        // RMSNorm (+ RoPE for video tokens) of the K rows in place: thread =
        // (row tid / 4, dims 32 (tid % 4) .. +31); quarter q < 3 is RoPE axis q.
        const int r = tid >> 2, qd = tid & 3;
        uint16_t* kr = ktile + r * kPitch + 32 * qd;
        float x[32];
#pragma unroll
        for (int e = 0; e < 32; ++e) x[e] = __uint_as_float((uint32_t)kr[e] << 16);
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < 32; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
        ss += __shfl_xor(ss, 1);
        ss += __shfl_xor(ss, 2);
        const float inv = 1.0f / sqrtf(ss * (1.0f / kD) + kRmsEps);
        const uint16_t* gp = pa.gamma + (int64_t)h * kD + 32 * qd;
#pragma unroll
        for (int e = 0; e < 32; ++e)
            x[e] = bf16_round_f(x[e] * inv * __uint_as_float((uint32_t)gp[e] << 16));
        const bool video = t >= n_t && t < n_t + n_v;
        if (video && qd < 3 && r < n) {
            int pt, ph, pw;
            video_pos(pa, (int64_t)(t - n_t) * kT + r, pt, ph, pw);
            const int pos = qd == 0 ? pt : (qd == 1 ? ph : pw);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                float y8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) y8[e] = x[8 * b + e];
                rope8(y8, 32 * qd + 8 * b, pos);
#pragma unroll
                for (int e = 0; e < 8; ++e) x[8 * b + e] = bf16_round_f(y8[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < 32; ++e)
            kr[e] = r < n ? (uint16_t)(__float_as_uint(x[e]) >> 16) : (uint16_t)0;
        __syncthreads();
    }
    const int u = t - n_t;
    if (pool && u >= 0 && u < n_v) {
        const uint16_t* tl = tid < kD ? ktile : vtile;
        const int d = tid & (kD - 1);
        double s = 0.0;
        for (int r = 0; r < n; ++r) s += (double)__uint_as_float((uint32_t)tl[r * kPitch + d] << 16);
        const float mean = (float)(s / (double)n);
        if (tid < kD) {
            kbar[((int64_t)h * n_v + u) * kD + pooled_dim_pos(d)] = mean;
        } else {
            // transposed, rows padded to vbar_pitch(n_v); the last tile zeroes the padding
            const int ldv = vbar_pitch(n_v);
            float* vrow = vbar + ((int64_t)h * kD + d) * ldv;
            vrow[u] = mean;
            if (u == n_v - 1)
                for (int w = n_v; w < ldv; ++w) vrow[w] = 0.0f;
        }
    }
    const int64_t base = ((int64_t)h * N + t) * (kT * kD);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int id = tid + 256 * i;  // 16-byte piece: half | s (3 bits) | lane (6 bits)
        const int half = id >> 9, s8 = (id >> 6) & 7, lane = id & 63;
        const int key = 32 * half + kappa(lane & 31);
        const int d0 = 16 * s8 + 8 * (lane >> 5);
        *(uint4*)(kpack + base + id * 8) = *(const uint4*)(ktile + key * kPitch + d0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int id = tid + 256 * i;  // 16-byte piece: half | db (2 bits) | m | lane (6 bits)
        const int half = id >> 9, db = (id >> 7) & 3, m = (id >> 6) & 1, lane = id & 63;
        const int d = 32 * db + (lane & 31);
        const int key0 = 32 * half + 16 * m + 8 * (lane >> 5);
        uint32_t wds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            wds[e] = (uint32_t)vtile[(key0 + 2 * e) * kPitch + d] |
                     ((uint32_t)vtile[(key0 + 2 * e + 1) * kPitch + d] << 16);
        *(uint4*)(vpack + base + id * 8) = make_uint4(wds[0], wds[1], wds[2], wds[3]);
    }
}

}  // namespace

hipError_t launch_pool_pack(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const Shape& s, uint8_t* ws, const Layout& L, hipStream_t stream,
                            const Prep* prep, uint16_t* q_out, bool pooled) {
    PrepArgs qa{nullptr, 1, 1, 1, 1, 1, 1}, ka = qa;
    if (prep && prep->gamma_q) {
        qa = PrepArgs{prep->gamma_q, prep->grid[0], prep->grid[1], prep->grid[2],
                      prep->tile[0], prep->tile[1], prep->tile[2]};
        ka = qa;
        ka.gamma = prep->gamma_k;
        hipLaunchKernelGGL(prep_q_kernel, dim3(s.N, (s.H + 7) / 8), dim3(128), 0, stream, q, qa, s.H,
                           s.ldh, s.n_t, s.n_v, s.S_t, s.V_t, s.V_v, s.V_a, s.S_v, q_out,
                           (double*)(ws + L.qbar64));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    } else if (s.n_v > 0 && pooled) {
        hipLaunchKernelGGL(pool_q_kernel, dim3(s.n_v, (s.H + 7) / 8), dim3(128), 0, stream, q, s.H,
                           s.ldh, s.S_t, s.n_v, s.V_v, (double*)(ws + L.qbar64));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(pack_kv_kernel, dim3(s.N, s.H), dim3(256), 0, stream, k, v, s.H, s.ldh, s.n_t, s.n_v,
                       s.N, s.S_t, s.S_v, s.V_t, s.V_v, s.V_a, ka, pooled ? 1 : 0, (float*)(ws + L.kbar),
                       (float*)(ws + L.vbar), (uint16_t*)(ws + L.kpack), (uint16_t*)(ws + L.vpack));
    return hipGetLastError();
}

}  // namespace vsa

// pool_pack.hip -- stage 1 of the VSA forward on gfx950: FP32 tile pooling of
// Q, K, V over the video tiles, and packing of V tiles for the attention stage.
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
// heads x 16 column chunks of 8 dims; each thread walks the tile's 64 rows.
__global__ __launch_bounds__(128) void pool_q_kernel(const uint16_t* __restrict__ q, int H,
                                                     int64_t S_t, int n_v,
                                                     double* __restrict__ qbar64) {
    const int u = blockIdx.x;
    const int h = blockIdx.y * 8 + (threadIdx.x >> 4);
    const int c = threadIdx.x & 15;
    if (h >= H) return;
    const int64_t rs = (int64_t)H * kD;
    const uint16_t* p = q + (S_t + (int64_t)u * kT) * rs + (int64_t)h * kD + c * 8;
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll 16
    for (int r = 0; r < kT; ++r) {
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
    double* o = qbar64 + ((int64_t)h * n_v + u) * kD + c * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (double)(float)(acc[e] * (1.0 / kT));
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
                                                      int n_t, int n_v, int N,
                                                      float* __restrict__ kbar_t,
                                                      float* __restrict__ vbar,
                                                      uint16_t* __restrict__ kpack,
                                                      uint16_t* __restrict__ vpack) {
    __shared__ __align__(16) uint16_t ktile[kT * kPitch];
    __shared__ __align__(16) uint16_t vtile[kT * kPitch];
    const int t = blockIdx.x;
    const int h = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t rs = (int64_t)H * kD;
    const int64_t src = (int64_t)t * kT * rs + (int64_t)h * kD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int id = tid + 256 * i;
        const int r = id >> 4, c = id & 15;
        *(uint4*)(ktile + r * kPitch + c * 8) = *(const uint4*)(k + src + (int64_t)r * rs + c * 8);
        *(uint4*)(vtile + r * kPitch + c * 8) = *(const uint4*)(v + src + (int64_t)r * rs + c * 8);
    }
    __syncthreads();
    const int u = t - n_t;
    if (u >= 0 && u < n_v) {
        const uint16_t* tl = tid < kD ? ktile : vtile;
        const int d = tid & (kD - 1);
        double s = 0.0;
        for (int r = 0; r < kT; ++r) s += (double)__uint_as_float((uint32_t)tl[r * kPitch + d] << 16);
        const float mean = (float)(s * (1.0 / kT));
        if (tid < kD) kbar_t[((int64_t)h * kD + d) * n_v + u] = mean;
        else vbar[((int64_t)h * n_v + u) * kD + d] = mean;
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
                            const Shape& s, uint8_t* ws, const Layout& L, hipStream_t stream) {
    if (s.n_v > 0) {
        hipLaunchKernelGGL(pool_q_kernel, dim3(s.n_v, (s.H + 7) / 8), dim3(128), 0, stream, q, s.H,
                           s.S_t, s.n_v, (double*)(ws + L.qbar64));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(pack_kv_kernel, dim3(s.N, s.H), dim3(256), 0, stream, k, v, s.H, s.n_t, s.n_v,
                       s.N, (float*)(ws + L.kbar_t), (float*)(ws + L.vbar), (uint16_t*)(ws + L.kpack),
                       (uint16_t*)(ws + L.vpack));
    return hipGetLastError();
}

}  // namespace vsa

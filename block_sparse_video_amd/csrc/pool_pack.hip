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
// HBM-bound: every byte of Q, K, V video rows is read once (coalesced 16-byte
// loads, 1 KiB contiguous per wave instruction), V of all tiles once more.
#include "vsa_internal.h"

namespace vsa {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// grid (n_v, ceil(H/8), 2): z = 0 pools Q, z = 1 pools K.  128 threads = 8
// heads x 16 column chunks of 8 dims; each thread walks the tile's 64 rows.
__global__ __launch_bounds__(128) void pool_qk_kernel(const uint16_t* __restrict__ q,
                                                      const uint16_t* __restrict__ k, int H,
                                                      int64_t S_t, int n_v,
                                                      double* __restrict__ qbar64,
                                                      float* __restrict__ kbar_t) {
    const int u = blockIdx.x;
    const int h = blockIdx.y * 8 + (threadIdx.x >> 4);
    const int c = threadIdx.x & 15;
    if (h >= H) return;
    const uint16_t* src = blockIdx.z == 0 ? q : k;
    const int64_t rs = (int64_t)H * kD;
    const uint16_t* p = src + (S_t + (int64_t)u * kT) * rs + (int64_t)h * kD + c * 8;
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
    if (blockIdx.z == 0) {
        double* o = qbar64 + ((int64_t)h * n_v + u) * kD + c * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (double)(float)(acc[e] * (1.0 / kT));
    } else {
        float* o = kbar_t + ((int64_t)h * kD + c * 8) * n_v + u;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[(int64_t)e * n_v] = (float)(acc[e] * (1.0 / kT));
    }
}

// grid (N, H), 256 threads.  Loads one 64 x 128 V tile of one head into LDS,
// writes its pooled mean (video tiles) and its transpose, split by key
// halves: [2 halves][128 d][32 keys] bf16 (16 KiB), so that each half-tile
// of V^T is one contiguous 8 KiB block for the attention stage.
constexpr int kPitch = kD + 8;  // LDS row pitch in bf16 elements (272 bytes)

__global__ __launch_bounds__(256) void pack_v_kernel(const uint16_t* __restrict__ v, int H,
                                                     int n_t, int n_v, int N,
                                                     float* __restrict__ vbar,
                                                     uint16_t* __restrict__ vpack) {
    __shared__ __align__(16) uint16_t tile[kT * kPitch];
    const int t = blockIdx.x;
    const int h = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t rs = (int64_t)H * kD;
    const uint16_t* src = v + (int64_t)t * kT * rs + (int64_t)h * kD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int id = tid + 256 * i;
        const int r = id >> 4, c = id & 15;
        const uint4 w = *(const uint4*)(src + (int64_t)r * rs + c * 8);
        *(uint4*)(tile + r * kPitch + c * 8) = w;
    }
    __syncthreads();
    const int u = t - n_t;
    if (u >= 0 && u < n_v && tid < kD) {
        double s = 0.0;
        for (int r = 0; r < kT; ++r) s += (double)__uint_as_float((uint32_t)tile[r * kPitch + tid] << 16);
        vbar[((int64_t)h * n_v + u) * kD + tid] = (float)(s * (1.0 / kT));
    }
    uint16_t* dst = vpack + ((int64_t)h * N + t) * (kT * kD);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // 16-byte piece id: half (1 bit) | d (7 bits) | piece of 8 keys (2 bits)
        const int id = tid + 256 * i;
        const int half = id >> 9, d = (id >> 2) & 127, piece = id & 3;
        const int key0 = 32 * half + 8 * piece;
        uint32_t wds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            wds[e] = (uint32_t)tile[(key0 + 2 * e) * kPitch + d] |
                     ((uint32_t)tile[(key0 + 2 * e + 1) * kPitch + d] << 16);
        *(uint4*)(dst + id * 8) = make_uint4(wds[0], wds[1], wds[2], wds[3]);
    }
}

}  // namespace

hipError_t launch_pool_pack(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const Shape& s, uint8_t* ws, const Layout& L, hipStream_t stream) {
    if (s.n_v > 0) {
        dim3 grid(s.n_v, (s.H + 7) / 8, 2);
        hipLaunchKernelGGL(pool_qk_kernel, grid, dim3(128), 0, stream, q, k, s.H, s.S_t, s.n_v,
                           (double*)(ws + L.qbar64), (float*)(ws + L.kbar_t));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(pack_v_kernel, dim3(s.N, s.H), dim3(256), 0, stream, v, s.H, s.n_t, s.n_v,
                       s.N, (float*)(ws + L.vbar), (uint16_t*)(ws + L.vpack));
    return hipGetLastError();
}

}  // namespace vsa

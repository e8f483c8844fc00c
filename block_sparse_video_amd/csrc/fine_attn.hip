// fine_attn.hip -- stage 3 of the VSA forward on gfx950: block-sparse flash
// attention over 64x64 tiles with bf16 MFMA, online softmax in fp32, and the
// gated coarse combination fused into the epilogue.
//
// Page "UniServe: serving FastH3 at its fastest":
//   section "The FastH3 workload": text and audio query tiles attend to every
//     key tile; a video query tile attends to the text and audio key tiles and
//     to its selected video key tiles (one softmax over the union);
//   section "Fused output combination": out = O_fine + gate * O_coarse, with
//     the gate taken as sigmoid(G) per channel (video rows only).
//
// Work unit = (head h, query tile j): 64 query rows, 2 wavefronts x 32 rows.
// Each wavefront computes S^T = K Q^T for a 64-key tile as two 32x32 blocks
// with v_mfma_f32_32x32x16_bf16, so every lane owns ONE query column and 32
// of its scores: the row max needs one cross-half exchange and the running
// max / sum are per lane.  P stays in registers and feeds O^T += V^T P^T
// (again 32x32x16 MFMAs) through a fixed permutation of the key index that
// matches the accumulator layout; V^T comes from the packed, swizzled tile
// image written by stage 1.  K is read straight from the token-major input and
// swizzled on its way into LDS.
//
// Accumulator layout of a 32x32 MFMA (lane l, element i of the 16 floats):
//   row = 8*(i/4) + 4*(l/32) + (i%4), column = l%32.
#include "vsa_internal.h"

namespace vsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 2;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileBytes = kT * kD * 2;       // 16 KiB per K or V tile
constexpr int kStagePitch = kD + 4;           // fp32 epilogue staging pitch (floats)
constexpr int kSmemBytes = kT * kStagePitch * 4;  // 33,792 B >= 2 tiles (32 KiB)
static_assert(kSmemBytes >= 2 * kTileBytes, "LDS must hold a K and a V tile");

struct FineArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* gate;
    const uint16_t* vpack;
    const int32_t* sel;
    const float* coarse;
    uint16_t* out;
    int H, n_t, n_v, n_a, N, kk;
    float scale_log2;  // log2(e) / sqrt(128)
};

// blockIdx -> (head, query tile).  Workgroups are dealt round-robin to the 8
// XCDs, so XCD x runs blocks x, x+8, x+16, ...  Each XCD is given one
// contiguous range of the head-major unit order (a few heads, so its L2 sees
// one head's K/V at a time), and inside its range the dense text/audio
// units (N key tiles each) are issued before the video units (n_t+k+n_a).
__device__ __forceinline__ void unit_of(int b, int H, int N, int n_t, int n_v, int n_a, int& h,
                                        int& j) {
    const int n_h = n_t + n_a;
    const int64_t G = (int64_t)H * N;
    const int x = b & 7;
    const int64_t i = b >> 3;
    const int64_t G8 = G >> 3, rem = G & 7;
    const int64_t a = (int64_t)x * G8 + (x < rem ? x : rem);
    const int64_t cnt = G8 + (x < rem ? 1 : 0);
    const int hA = (int)(a / N), hB = (int)((a + cnt - 1) / N);
    int64_t heavy_total = 0;
    for (int hh = hA; hh <= hB; ++hh) {
        const int64_t base = (int64_t)hh * N;
        const int64_t lo = a > base ? a : base;
        const int64_t hi0 = a + cnt, hi1 = base + n_h;
        const int64_t hi = hi0 < hi1 ? hi0 : hi1;
        if (hi > lo) heavy_total += hi - lo;
    }
    const bool want_heavy = i < heavy_total;
    int64_t rank = want_heavy ? i : i - heavy_total;
    int64_t pos = a;
    for (int hh = hA; hh <= hB; ++hh) {
        const int64_t base = (int64_t)hh * N;
        const int64_t lo_all = a > base ? a : base;
        const int64_t hi_all = (a + cnt) < (base + N) ? (a + cnt) : (base + N);
        const int64_t hv_lo = lo_all, hv_hi = hi_all < base + n_h ? hi_all : base + n_h;
        const int64_t nh = hv_hi > hv_lo ? hv_hi - hv_lo : 0;
        const int64_t vd_lo = lo_all > base + n_h ? lo_all : base + n_h;
        const int64_t nv = hi_all > vd_lo ? hi_all - vd_lo : 0;
        if (want_heavy) {
            if (rank < nh) { pos = hv_lo + rank; break; }
            rank -= nh;
        } else {
            if (rank < nv) { pos = vd_lo + rank; break; }
            rank -= nv;
        }
    }
    h = (int)(pos / N);
    const int p = (int)(pos - (int64_t)h * N);
    j = p < n_h ? (p < n_t ? p : n_v + p) : n_t + (p - n_h);
}

__device__ __forceinline__ int vswz(int d) { return (d & 15) ^ ((d >> 4) & 1); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float sigmoidf(float g) { return 1.0f / (1.0f + __expf(-g)); }

__global__ __launch_bounds__(kThreads) void fine_attn_kernel(FineArgs a) {
    __shared__ __align__(16) unsigned char smem[kSmemBytes];
    unsigned char* ks = smem;               // K tile, [64 keys][128 d], 16-byte chunks swizzled
    unsigned char* vs = smem + kTileBytes;  // V^T tile, [128 d][64 keys], 8-byte chunks swizzled

    int h, j;
    unit_of(blockIdx.x, a.H, a.N, a.n_t, a.n_v, a.n_a, h, j);
    if (h >= a.H || j >= a.N) return;  // not reached: the map is a bijection onto the units
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
    const int64_t rs = (int64_t)a.H * kD;
    const bool video = j >= a.n_t && j < a.n_t + a.n_v;
    const int u = j - a.n_t;
    const int n_iter = video ? a.n_t + a.kk + a.n_a : a.N;
    const int32_t* selrow = a.sel + ((int64_t)h * a.n_v + (video ? u : 0)) * a.kk;

    // Q^T fragments (B operand of S^T = K Q^T): query column l32, dims 16s + 8g .. +7
    const int64_t qrow = (int64_t)j * kT + wave * 32 + l32;
    bf16x8 qf[8];
    {
        const uint16_t* qp = a.q + qrow * rs + (int64_t)h * kD + 8 * g;
#pragma unroll
        for (int s = 0; s < 8; ++s) qf[s] = *(const bf16x8*)(qp + 16 * s);
    }

    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    const uint16_t* kbase = a.k + (int64_t)h * kD;
    const uint16_t* vbase = a.vpack + (int64_t)h * a.N * (kT * kD);
    uint4 kreg[8], vreg[8];
    auto tile_at = [&](int it) -> int {
        if (!video || it < a.n_t) return it;
        if (it < a.n_t + a.kk) {
            // caller-supplied index sets are clamped into range, never followed out of bounds
            const int w = selrow[it - a.n_t];
            return a.n_t + (w < 0 ? 0 : (w >= a.n_v ? a.n_v - 1 : w));
        }
        return a.n_v + it - a.kk;
    };
    auto load_tile = [&](int tile) {
        const uint16_t* kt = kbase + (int64_t)tile * kT * rs;
        const uint16_t* vt = vbase + (int64_t)tile * (kT * kD);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int id = tid + kThreads * i;
            const int row = id >> 4, c = id & 15;
            kreg[i] = *(const uint4*)(kt + (int64_t)row * rs + c * 8);
            vreg[i] = *(const uint4*)(vt + id * 8);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int id = tid + kThreads * i;
            const int row = id >> 4, c = id & 15;
            *(uint4*)(ks + row * 256 + ((c ^ (row & 15)) << 4)) = kreg[i];
            *(uint4*)(vs + id * 16) = vreg[i];
        }
    };

    const int vsw = vswz(l32);  // d = 32*db + l32 has the same swizzle for every db
    load_tile(tile_at(0));
    for (int it = 0; it < n_iter; ++it) {
        __syncthreads();  // every wave is done with the previous tile
        store_tile();
        __syncthreads();
        if (it + 1 < n_iter) load_tile(tile_at(it + 1));

        // S^T blocks: keys 0..31 and 32..63 of the tile (rows) x 32 queries (cols)
        f32x16 s0, s1;
#pragma unroll
        for (int i = 0; i < 16; ++i) { s0[i] = 0.0f; s1[i] = 0.0f; }
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int chunk = 2 * s + g;
            const bf16x8 a0 = *(const bf16x8*)(ks + l32 * 256 + ((chunk ^ (l32 & 15)) << 4));
            const bf16x8 a1 = *(const bf16x8*)(ks + (32 + l32) * 256 + ((chunk ^ (l32 & 15)) << 4));
            s0 = mfma32(a0, qf[s], s0);
            s1 = mfma32(a1, qf[s], s1);
        }

        // online softmax for query column l32 (this lane holds 32 of its 64 scores)
        float mx = s0[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s0[i]);
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s1[i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float corr = __builtin_amdgcn_exp2f((m_run - m_new) * a.scale_log2);
        m_run = m_new;
        l_run *= corr;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] *= corr;
        const float mb = m_new * a.scale_log2;
        f32x8 pf[2][2];
        float lsum = 0.0f;
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[8 * m2 + e], a.scale_log2, -mb));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[8 * m2 + e], a.scale_log2, -mb));
                pf[0][m2][e] = p0;
                pf[1][m2][e] = p1;
                lsum += p0 + p1;
            }
        l_run += lsum;
        bf16x8 pb[2][2];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2) pb[b][m2] = __builtin_convertvector(pf[b][m2], bf16x8);

        // O^T[db] (32 dims x 32 queries) += V^T (32 dims x 16 keys) P^T (16 keys x 32 queries).
        // MFMA (b, m2) covers keys 32b + 16m2 + {0..15}; lane half g supplies
        // keys +4g..+4g+3 and +8+4g..+8+4g+3 (the accumulator rows it holds).
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const unsigned char* vrow = vs + (32 * db + l32) * (kT * 2);
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2) {
                    const int c_lo = 8 * b + 4 * m2 + g;
                    const bf16x4 lo = *(const bf16x4*)(vrow + ((c_lo ^ vsw) << 3));
                    const bf16x4 hi = *(const bf16x4*)(vrow + (((c_lo + 2) ^ vsw) << 3));
                    const bf16x8 av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    o[db] = mfma32(av, pb[b][m2], o[db]);
                }
        }
    }

    // ---- epilogue: normalise, stage through LDS, add sigmoid(G) * coarse ----
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.0f / l_tot;
    __syncthreads();
    float* ost = (float*)smem;  // [64 queries][kStagePitch]
    {
        float* orow = ost + (wave * 32 + l32) * kStagePitch;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int d0 = 32 * db + 8 * a4 + 4 * g;
                *(float4*)(orow + d0) = make_float4(o[db][4 * a4 + 0] * inv, o[db][4 * a4 + 1] * inv,
                                                    o[db][4 * a4 + 2] * inv, o[db][4 * a4 + 3] * inv);
            }
    }
    __syncthreads();
    const float* cp = a.coarse + ((int64_t)h * a.n_v + (video ? u : 0)) * kD;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int id = tid + kThreads * i;
        const int row = id >> 4, c = id & 15;
        const float4 x0 = *(const float4*)(ost + row * kStagePitch + 8 * c);
        const float4 x1 = *(const float4*)(ost + row * kStagePitch + 8 * c + 4);
        f32x8 y = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        const int64_t grow = (int64_t)j * kT + row;
        if (video) {
            const uint4 gw = *(const uint4*)(a.gate + grow * rs + (int64_t)h * kD + 8 * c);
            const float4 c0 = *(const float4*)(cp + 8 * c);
            const float4 c1 = *(const float4*)(cp + 8 * c + 4);
            const uint32_t gwv[4] = {gw.x, gw.y, gw.z, gw.w};
            const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float g0 = __uint_as_float(gwv[e] << 16);
                const float g1 = __uint_as_float(gwv[e] & 0xFFFF0000u);
                y[2 * e] += sigmoidf(g0) * cv[2 * e];
                y[2 * e + 1] += sigmoidf(g1) * cv[2 * e + 1];
            }
        }
        const bf16x8 yb = __builtin_convertvector(y, bf16x8);
        *(bf16x8*)(a.out + grow * rs + (int64_t)h * kD + 8 * c) = yb;
    }
}

}  // namespace

hipError_t launch_fine_attention(const uint16_t* q, const uint16_t* k, const uint16_t* gate,
                                 const int32_t* sel, uint16_t* out, const Shape& s,
                                 const uint8_t* ws, const Layout& L, hipStream_t stream) {
    FineArgs a;
    a.q = q;
    a.k = k;
    a.gate = gate;
    a.vpack = (const uint16_t*)(ws + L.vpack);
    a.sel = sel;
    a.coarse = (const float*)(ws + L.coarse);
    a.out = out;
    a.H = s.H;
    a.n_t = s.n_t;
    a.n_v = s.n_v;
    a.n_a = s.n_a;
    a.N = s.N;
    a.kk = s.k;
    a.scale_log2 = (float)(1.4426950408889634 / 11.313708498984761);
    const int64_t units = (int64_t)s.H * s.N;
    hipLaunchKernelGGL(fine_attn_kernel, dim3((unsigned)units), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace vsa

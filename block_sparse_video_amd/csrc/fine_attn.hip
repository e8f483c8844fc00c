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
// Key tiles are consumed as half-tiles of 32 keys.  Per half-tile a wavefront
// computes S^T = K Q^T (32 keys x 32 queries) with eight
// v_mfma_f32_32x32x16_bf16, so each lane owns ONE query column and 16 of its
// scores; the running max and sum are per lane and one cross-half exchange
// completes a column.  P stays in registers and feeds O^T += V^T P^T (eight
// more MFMAs).
//
// Data movement: half-tiles (K 8 KiB + V^T 8 KiB) stream from global memory
// straight into an LDS ring of STAGES slots with global_load_lds_dwordx4
// (no register staging).  Each lane chooses the global address whose 16 bytes
// belong at its LDS position, which applies the bank swizzles and a fixed key
// permutation on the way in.  The ring is synchronised by explicit vmcnt
// waits and workgroup barriers.
//
// Accumulator layout of a 32x32 MFMA (lane l, element i of the 16 floats):
//   row = 8*(i/4) + 4*(l/32) + (i%4), column = l%32.
// Key permutation: LDS K row r of a half-tile holds key kappa(r) = r with
// bits 2 and 3 swapped.  Then in the PV MFMA m (keys 16m..16m+15), lane half
// g holds P for the 8 consecutive keys 16m + 8g .. 16m + 8g + 7, which makes
// its V^T operand one contiguous 16-byte LDS read.
#include "vsa_internal.h"

namespace vsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kWaves = 2;
constexpr int kThreads = 64 * kWaves;
constexpr int kHalfK = 32 * kD * 2;          // 8 KiB: 32 keys x 128 dims
constexpr int kSlot = 2 * kHalfK;            // 16 KiB: K half + V^T half
constexpr int kStageBytes = kT * kD * 4;     // 32 KiB: fp32 epilogue staging

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

// LDS swizzles.  K: 16-byte chunk c of row r at chunk position c ^ (r & 15).
// V^T: 16-byte piece p (8 keys) of 64-byte row d at position p ^ vswz(d);
// conflict-free for 16 consecutive rows read at one logical piece whether the
// LDS serves 16 lanes over 64 banks or 8 lanes over 32 banks per cycle.
__device__ __forceinline__ int vswz(int d) { return ((d >> 1) ^ (d >> 3)) & 3; }
__device__ __forceinline__ int kappa(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float sigmoidf(float g) {
    return __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// max(x[l], x[l ^ 32]) and x[l] + x[l ^ 32] through v_permlane32_swap
__device__ __forceinline__ float xhalf_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wait until at most n of this wave's vector-memory loads are outstanding
// (s_waitcnt encoding: vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt at
// their "no wait" maxima).  The compiler does not track the LDS writes of
// global_load_lds, so these waits are what makes a ring slot readable.
__device__ __forceinline__ void wait_vmcnt(int n) {
    switch (n) {
        case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
        case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
        case 16: __builtin_amdgcn_s_waitcnt(0x4F70); break;
        case 24: __builtin_amdgcn_s_waitcnt(0x4F78); break;
        case 32: __builtin_amdgcn_s_waitcnt(0x8F70); break;
        default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
}

// Scalar (wave-uniform) load of one selected-tile index.
__device__ __forceinline__ int load_uniform(const int32_t* p) {
    int v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
    return v;
}

__device__ __forceinline__ void block_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Depth of the half-tile ring (16 KiB per slot).
constexpr int kFineStages = 3;

template <int STAGES>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void fine_attn_kernel(FineArgs a) {
    static_assert(STAGES >= 2 && STAGES <= 6, "ring depth");
    constexpr int kSmem = STAGES * kSlot > kStageBytes ? STAGES * kSlot : kStageBytes;
    __shared__ __align__(1024) unsigned char smem[kSmem];

    int h, j;
    unit_of(blockIdx.x, a.H, a.N, a.n_t, a.n_v, a.n_a, h, j);
    if (h >= a.H || j >= a.N) return;  // not reached: the map is a bijection onto the units
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
    const int64_t rs = (int64_t)a.H * kD;  // elements between consecutive tokens
    const bool video = j >= a.n_t && j < a.n_t + a.n_v;
    const int u = j - a.n_t;
    const int n_half = 2 * (video ? a.n_t + a.kk + a.n_a : a.N);
    const int32_t* selrow = a.sel + ((int64_t)h * a.n_v + (video ? u : 0)) * a.kk;

    // Q^T fragments (B operand of S^T = K Q^T): query column l32, dims 16s + 8g .. +7
    bf16x8 qf[8];
    {
        const uint16_t* qp = a.q + ((int64_t)j * kT + wave * 32 + l32) * rs + (int64_t)h * kD + 8 * g;
#pragma unroll
        for (int s = 0; s < 8; ++s) qf[s] = *(const bf16x8*)(qp + 16 * s);
        wait_vmcnt(0);  // Q is resident before the ring starts counting loads
    }

    // Per-lane source offsets of this wave's 4 K and 4 V^T load instructions
    // per half-tile (each instruction fills 1 KiB of LDS, 16 bytes per lane).
    uint32_t koff[4], voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (wave * 4 + i) * 4 + (lane >> 4);   // LDS K row 0..31
        const int c = (lane & 15) ^ (r & 15);              // logical 16-byte chunk
        koff[i] = (uint32_t)(kappa(r) * rs * 2 + c * 16);
        const int d = (wave * 4 + i) * 16 + (lane >> 2);   // LDS V^T row 0..127
        const int p = (lane & 3) ^ vswz(d);                // logical piece (8 keys)
        voff[i] = (uint32_t)(d * 64 + p * 16);
    }

    auto tile_at = [&](int it) -> int {
        if (!video || it < a.n_t) return it;
        if (it < a.n_t + a.kk) {
            // caller-supplied index sets are clamped into range, never followed out of bounds
            const int w = load_uniform(selrow + (it - a.n_t));
            return a.n_t + (w < 0 ? 0 : (w >= a.n_v ? a.n_v - 1 : w));
        }
        return a.n_v + it - a.kk;
    };
    const char* kbase = (const char*)(a.k + (int64_t)h * kD);
    const char* vbase = (const char*)(a.vpack + (int64_t)h * a.N * (kT * kD));
    auto issue = [&](int hx, int slot) {
        const int tile = tile_at(hx >> 1), half = hx & 1;
        const char* ksrc = kbase + ((int64_t)tile * kT + 32 * half) * rs * 2;
        const char* vsrc = vbase + ((int64_t)tile * 2 + half) * kHalfK;
        unsigned char* kdst = smem + slot * kSlot + wave * 4096;
        unsigned char* vdst = smem + slot * kSlot + kHalfK + wave * 4096;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(ksrc + koff[i]), (lds_ptr_t)(kdst + i * 1024),
                                             16, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(vsrc + voff[i]), (lds_ptr_t)(vdst + i * 1024),
                                             16, 0, 0);
    };

    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.0f;
    float mc_run = -INFINITY;  // running max of this query's scores, times scale_log2
    float l_run = 0.0f;        // this lane's share of the running softmax denominator
    const float c2 = a.scale_log2;
    const int kvsw = (l32 & 15) << 4;

#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < n_half) issue(s, s);

    for (int hx = 0; hx < n_half; ++hx) {
        const int ahead = n_half - 1 - hx;
        wait_vmcnt(8 * (ahead < STAGES - 2 ? ahead : STAGES - 2));
        block_sync();
        if (hx + STAGES - 1 < n_half) issue(hx + STAGES - 1, (hx + STAGES - 1) % STAGES);

        const unsigned char* ks = smem + (hx % STAGES) * kSlot;
        const unsigned char* vs = ks + kHalfK;
        f32x16 sacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = 0.0f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const bf16x8 ka = *(const bf16x8*)(ks + l32 * 256 + (((2 * s + g) << 4) ^ kvsw));
            sacc = mfma32(ka, qf[s], sacc);
        }

        // online softmax of this query column over 32 keys (16 here, 16 in lane ^ 32)
        float mx = fmaxf(fmaxf(sacc[0], sacc[1]), sacc[2]);
#pragma unroll
        for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, sacc[i]), sacc[i + 1]);
        mx = fmaxf(mx, sacc[15]);
        mx = xhalf_max(mx) * c2;
        // Lazy rescaling: the reference max only moves when some column's max
        // has grown by more than 2^8; until then P may exceed 1 (by at most
        // 2^8), which changes nothing mathematically.
        if (__builtin_amdgcn_read_exec() & __ballot(mx > mc_run + 8.0f)) {
            const float mc_new = fmaxf(mc_run, mx);
            const float corr = __builtin_amdgcn_exp2f(mc_run - mc_new);
            mc_run = mc_new;
            l_run *= corr;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][i] *= corr;
        }
        f32x8 pf0, pf1;
        float lsum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pf0[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[e], c2, -mc_run));
            pf1[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[8 + e], c2, -mc_run));
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) lsum += pf0[e] + pf1[e];
        l_run += lsum;
        const bf16x8 pb0 = __builtin_convertvector(pf0, bf16x8);
        const bf16x8 pb1 = __builtin_convertvector(pf1, bf16x8);

        // O^T[db] (32 dims x 32 queries) += V^T (32 dims x 16 keys) P^T (16 keys x 32 queries)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const int d = 32 * db + l32;
            const unsigned char* vrow = vs + d * 64;
            const int sw = vswz(d);
            const bf16x8 v0 = *(const bf16x8*)(vrow + (((0 + g) ^ sw) << 4));
            const bf16x8 v1 = *(const bf16x8*)(vrow + (((2 + g) ^ sw) << 4));
            o[db] = mfma32(v0, pb0, o[db]);
            o[db] = mfma32(v1, pb1, o[db]);
        }
    }

    // ---- epilogue: normalise, stage through LDS, add sigmoid(G) * coarse ----
    const float inv = __builtin_amdgcn_rcpf(xhalf_sum(l_run));
    wait_vmcnt(0);
    block_sync();
    float* ost = (float*)smem;  // [64 queries][128 dims], 16-byte chunks swizzled by row
    {
        const int q = wave * 32 + l32;
        float* orow = ost + q * kD;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int chunk = 8 * db + 2 * a4 + g;  // dims 4*chunk .. 4*chunk+3
                *(float4*)(orow + 4 * (chunk ^ (q & 15))) =
                    make_float4(o[db][4 * a4 + 0] * inv, o[db][4 * a4 + 1] * inv,
                                o[db][4 * a4 + 2] * inv, o[db][4 * a4 + 3] * inv);
            }
    }
    block_sync();
    const float* cp = a.coarse + ((int64_t)h * a.n_v + (video ? u : 0)) * kD;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int id = tid + kThreads * i;
        const int row = id >> 4, c = id & 15;
        const float4 x0 = *(const float4*)(ost + row * kD + 4 * ((2 * c) ^ (row & 15)));
        const float4 x1 = *(const float4*)(ost + row * kD + 4 * ((2 * c + 1) ^ (row & 15)));
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
                y[2 * e] += sigmoidf(__uint_as_float(gwv[e] << 16)) * cv[2 * e];
                y[2 * e + 1] += sigmoidf(__uint_as_float(gwv[e] & 0xFFFF0000u)) * cv[2 * e + 1];
            }
        }
        *(bf16x8*)(a.out + grow * rs + (int64_t)h * kD + 8 * c) = __builtin_convertvector(y, bf16x8);
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
    hipLaunchKernelGGL(fine_attn_kernel<kFineStages>, dim3((unsigned)units), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace vsa

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
// One wavefront computes one work unit (head h, query tile j): 64 query rows
// against every key tile of the unit's list, walked as half-tiles of 32 keys.
// Every K/V element a unit needs is used by that wavefront only, so the
// wavefront streams its operands into a private 32 KiB LDS ring (two K slots,
// two V slots) with global_load_lds_dwordx4 and needs no barriers.  Stage 1
// stored the K and V tiles in the exact per-lane operand order, so every load
// and every LDS operand read is one contiguous 1 KiB wavefront access.
//
// Per half-tile, for each of the two 32-query blocks qb:
//   S^T[qb] (32 keys x 32 queries) = K Q^T  -- eight v_mfma_f32_32x32x16_bf16
//   softmax numerators per query column against a fixed per-column reference
//   (each lane owns one column and 16 of its 32 scores; lane ^ 32 owns the
//   other 16)
//   O^T[qb] (128 dims x 32 queries) += V^T P^T  -- eight more MFMAs
// Software pipeline: the S^T MFMAs of the next half-tile are issued in the
// same step as the softmax numerators of the current one, so matrix and
// vector units overlap within the wavefront; K is fetched two half-tiles
// ahead of its use, V one.
//
// Accumulator layout of a 32x32 MFMA (lane l, element i of the 16 floats):
//   row = 8*(i/4) + 4*(l/32) + (i%4), column = l%32.
// Key order: row r of a packed K half-tile is key kappa(r) (r with bits 2 and
// 3 swapped).  Element e of the P^T operand of PV MFMA m in lane half g is
// then the score of key 16m + 8g + e: eight consecutive keys, matching the
// packed V operand.
#include "vsa_internal.h"

namespace vsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 64;
constexpr int kHalfElems = 32 * kD;  // bf16 elements per packed half-tile (8 KiB)
constexpr int kTileElems = 2 * kHalfElems;

struct FineArgs {
    const uint16_t* q;
    const uint16_t* gate;
    const uint16_t* kpack;
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

// Scalar (wave-uniform) load of one selected-tile index: a scalar load keeps
// it out of the vector-memory counter that the operand prefetches occupy.
__device__ __forceinline__ int load_uniform(const int32_t* p) {
    int v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
    return v;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Start the copy of one packed half-tile operand block (8 KiB, 8 x 1 KiB) from
// global memory into an LDS slot: `src` is the block's (wave-uniform) byte
// address, `lane_off` = 16 * lane.  Completion is tracked by vmcnt only.
__device__ __forceinline__ void fetch_half(unsigned char* slot, const char* src, uint32_t lane_off) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(src + (lane_off + i * 1024u)),
                                         (lds_ptr_t)(slot + i * 1024), 16, 0, 0);
}

// Wait until at most n of this wave's vector-memory loads are outstanding
// (s_waitcnt encoding: vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt at
// their "no wait" maxima).  The compiler does not track the LDS writes of
// global_load_lds, so these waits are what makes a ring slot readable.
__device__ __forceinline__ void wait_vmcnt(int n) {
    if (n >= 16) __builtin_amdgcn_s_waitcnt(0x4F70);       // vmcnt(16)
    else if (n >= 8) __builtin_amdgcn_s_waitcnt(0x0F78);   // vmcnt(8)
    else __builtin_amdgcn_s_waitcnt(0x0F70);               // vmcnt(0)
    asm volatile("" ::: "memory");
}

// S^T (32 keys x 32 queries) of one query block: eight MFMAs over the 128
// dims, K operands read from an LDS slot (lane-contiguous, conflict-free).
__device__ __forceinline__ f32x16 qk_block(const bf16x8* kslot, const bf16x8 (&q)[8]) {
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = mfma32(kslot[s * 64], q[s], acc);
    return acc;
}

// Reference-scaled softmax numerators of one 32-query block over one
// half-tile: P = 2^(s * scale_log2 - m_ref) with a per-column reference
// m_ref that stays fixed for the whole key list (see the kernel), so O never
// needs rescaling inside the loop.  Returns P as two bf16 operands (keys
// 0..15 and 16..31 of the half-tile, in operand order) and adds this lane's
// share of the denominator to l_run.
__device__ __forceinline__ void numerators(const f32x16& s, float c2, float m_ref, float& l_run,
                                           bf16x8& p0, bf16x8& p1) {
    f32x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], c2, -m_ref));
        b[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 + e], c2, -m_ref));
    }
    float lsum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) lsum += a[e] + b[e];
    l_run += lsum;
    p0 = __builtin_convertvector(a, bf16x8);
    p1 = __builtin_convertvector(b, bf16x8);
}

// Column max of one S^T block (16 values here, 16 in lane ^ 32), times scale_log2.
__device__ __forceinline__ float column_max(const f32x16& s, float c2) {
    float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, s[i]), s[i + 1]);
    mx = fmaxf(mx, s[15]);
    return xhalf_max(mx) * c2;
}

// O^T[qb] += V^T P^T for both query blocks; each V operand is read from the
// LDS slot once and used by both blocks.
__device__ __forceinline__ void pv(f32x16 (&o)[2][4], const bf16x8* vslot, const bf16x8 (&p)[2][2]) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const bf16x8 v = vslot[(2 * db + m) * 64];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) o[qb][db] = mfma32(v, p[qb][m], o[qb][db]);
        }
}

__global__ __launch_bounds__(kThreads) void fine_attn_kernel(FineArgs a) {
    // Ring: K slots at 0 and 8 KiB, V slots at 16 and 24 KiB.  After the loop
    // the same 32 KiB stage the fp32 output.
    __shared__ __align__(1024) unsigned char lds[4 * 8192];
    unsigned char* const kslot[2] = {lds, lds + 8192};
    unsigned char* const vslot[2] = {lds + 16384, lds + 24576};

    int h, j;
    unit_of(blockIdx.x, a.H, a.N, a.n_t, a.n_v, a.n_a, h, j);
    if (h >= a.H || j >= a.N) return;  // not reached: the map is a bijection onto the units
    const int lane = threadIdx.x, g = lane >> 5, l32 = lane & 31;
    const int64_t rs = (int64_t)a.H * kD;  // elements between consecutive tokens
    const bool video = j >= a.n_t && j < a.n_t + a.n_v;
    const int u = j - a.n_t;
    const int n_half = 2 * (video ? a.n_t + a.kk + a.n_a : a.N);
    const int32_t* selrow = a.sel + ((int64_t)h * a.n_v + (video ? u : 0)) * a.kk;
    const float c2 = a.scale_log2;

    // position `it` of this unit's ascending key-tile list -> tile index
    auto tile_at = [&](int it) -> int {
        if (!video || it < a.n_t) return it;
        if (it < a.n_t + a.kk) {
            // caller-supplied index sets are clamped into range, never followed out of bounds
            const int w = load_uniform(selrow + (it - a.n_t));
            return a.n_t + (w < 0 ? 0 : (w >= a.n_v ? a.n_v - 1 : w));
        }
        return a.n_v + it - a.kk;
    };
    // per-head bases of the packed operands (bytes): 16 KiB per tile and
    // tensor, two 8 KiB half-tiles each
    const char* kbase = (const char*)(a.kpack + (int64_t)h * a.N * (kT * kD));
    const char* vbase = (const char*)(a.vpack + (int64_t)h * a.N * (kT * kD));
    const uint32_t lane_off = 16u * lane;
    constexpr int64_t kTileBytes = 2 * kTileElems;
    constexpr int64_t kHalfBytes = 2 * kHalfElems;

    // Q^T fragments (B operand of S^T = K Q^T): query l32 of block qb, dims 16s + 8g .. +7
    bf16x8 qf[2][8];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const uint16_t* qp = a.q + ((int64_t)j * kT + 32 * qb + l32) * rs + (int64_t)h * kD + 8 * g;
#pragma unroll
        for (int s = 0; s < 8; ++s) qf[qb][s] = *(const bf16x8*)(qp + 16 * s);
    }
    wait_vmcnt(0);  // Q is resident before the ring starts counting loads

    const int n_tiles = n_half / 2;
    const int first = tile_at(0);
    const int second = n_tiles > 1 ? tile_at(1) : first;

    // Softmax reference.  Each column uses one fixed reference m_ref (in units
    // of scale_log2 * score) for its whole key list: P = 2^(x - m_ref) and
    // O, l accumulate without any rescaling.  m_ref starts at the column max
    // of the first half-tile, so the largest P of that half-tile is 1.  If a
    // later score exceeds it by so much that the denominator passes 2^100 (or
    // overflows), the unit is recomputed with m_ref raised by log2 of the
    // denominator (by 126 if it overflowed); the result is the same softmax,
    // and for ordinary inputs the first pass is the only pass.
    float m_ref[2];
    f32x16 o[2][4];
    float l_run[2];
    for (int pass = 0;; ++pass) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            l_run[qb] = 0.0f;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[qb][db][i] = 0.0f;
        }
        // cur / nxt: tile of the current half-tiles and the next list entry
        // (past the end of the list both name the last tile, whose data is
        // then fetched again and left unused: the loop body has no branches)
        int cur = first, nxt = second;
        // prologue: K(0), V(0), K(1) in that order, then S^T of half-tile 0
        fetch_half(kslot[0], kbase + cur * kTileBytes, lane_off);
        fetch_half(vslot[0], vbase + cur * kTileBytes, lane_off);
        fetch_half(kslot[1], kbase + cur * kTileBytes + kHalfBytes, lane_off);
        wait_vmcnt(16);
        f32x16 sacc[2][2];  // [parity of the half-tile][query block]
        sacc[0][0] = qk_block((const bf16x8*)kslot[0] + lane, qf[0]);
        sacc[0][1] = qk_block((const bf16x8*)kslot[0] + lane, qf[1]);
        if (pass == 0) {
            m_ref[0] = column_max(sacc[0][0], c2);
            m_ref[1] = column_max(sacc[0][1], c2);
        }

        // Step h (half-tile h, parity pp): fetch V(h+1) and K(h+2); wait for
        // K(h+1) and V(h) (issued one step earlier); then, without branches:
        //   S^T(h+1) (16 MFMAs)      alongside  numerators(h, block 0)
        //   O[0] += V(h) P(h, 0)     alongside  numerators(h, block 1)
        //   O[1] += V(h) P(h, 1)
        // Issue order keeps "everything up to K(h+1)" = "all but this step's
        // 16 fetches", so one vmcnt(16) wait serves every step.
        for (int t = 0; t < n_tiles; ++t) {
            const int nn = t + 2 < n_tiles ? tile_at(t + 2) : nxt;
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                asm volatile("" ::: "memory");
                const int tile_v = pp == 0 ? cur : nxt;  // V(h+1): (t, half 1) or (t+1, half 0)
                fetch_half(vslot[pp ^ 1], vbase + tile_v * kTileBytes + (pp ^ 1) * kHalfBytes, lane_off);
                fetch_half(kslot[pp], kbase + nxt * kTileBytes + pp * kHalfBytes, lane_off);  // K(h+2)
                wait_vmcnt(16);
                const bf16x8* ks = (const bf16x8*)kslot[pp ^ 1] + lane;
                const bf16x8* vs = (const bf16x8*)vslot[pp] + lane;
                bf16x8 kop[8];
#pragma unroll
                for (int s8 = 0; s8 < 8; ++s8) kop[s8] = ks[s8 * 64];
                f32x16 n0, n1;
#pragma unroll
                for (int i = 0; i < 16; ++i) { n0[i] = 0.0f; n1[i] = 0.0f; }
                bf16x8 p0[2], p1[2];
#pragma unroll
                for (int s8 = 0; s8 < 8; ++s8) {
                    n0 = mfma32(kop[s8], qf[0][s8], n0);
                    n1 = mfma32(kop[s8], qf[1][s8], n1);
                }
                numerators(sacc[pp][0], c2, m_ref[0], l_run[0], p0[0], p0[1]);
                bf16x8 vop[8];
#pragma unroll
                for (int m8 = 0; m8 < 8; ++m8) vop[m8] = vs[m8 * 64];
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int m = 0; m < 2; ++m) o[0][db] = mfma32(vop[2 * db + m], p0[m], o[0][db]);
                numerators(sacc[pp][1], c2, m_ref[1], l_run[1], p1[0], p1[1]);
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int m = 0; m < 2; ++m) o[1][db] = mfma32(vop[2 * db + m], p1[m], o[1][db]);
                sacc[pp ^ 1][0] = n0;
                sacc[pp ^ 1][1] = n1;
            }
            cur = nxt;
            nxt = nn;
        }
        wait_vmcnt(0);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        l_run[0] = xhalf_sum(l_run[0]);
        l_run[1] = xhalf_sum(l_run[1]);
        const bool big0 = !(l_run[0] <= 0x1p100f), big1 = !(l_run[1] <= 0x1p100f);
        if (!__ballot(big0 || big1) || pass >= 3) break;
        if (big0) m_ref[0] += l_run[0] <= 0x1p126f ? __log2f(l_run[0]) : 126.0f;
        if (big1) m_ref[1] += l_run[1] <= 0x1p126f ? __log2f(l_run[1]) : 126.0f;
    }

    // ---- epilogue: normalise, stage through LDS, add sigmoid(G) * coarse ----
    float* ost = (float*)lds;  // [64 queries][128 dims], 16-byte chunks swizzled by row
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float inv = __builtin_amdgcn_rcpf(l_run[qb]);
        const int q = 32 * qb + l32;
        float* orow = ost + q * kD;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int chunk = 8 * db + 2 * a4 + g;  // dims 4*chunk .. 4*chunk+3
                *(float4*)(orow + 4 * (chunk ^ (q & 15))) =
                    make_float4(o[qb][db][4 * a4 + 0] * inv, o[qb][db][4 * a4 + 1] * inv,
                                o[qb][db][4 * a4 + 2] * inv, o[qb][db][4 * a4 + 3] * inv);
            }
    }
    __syncthreads();
    const float* cp = a.coarse + ((int64_t)h * a.n_v + (video ? u : 0)) * kD;
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
        const int id = lane + kThreads * i;
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

hipError_t launch_fine_attention(const uint16_t* q, const uint16_t* gate, const int32_t* sel,
                                 uint16_t* out, const Shape& s, const uint8_t* ws, const Layout& L,
                                 hipStream_t stream) {
    FineArgs a;
    a.q = q;
    a.gate = gate;
    a.kpack = (const uint16_t*)(ws + L.kpack);
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

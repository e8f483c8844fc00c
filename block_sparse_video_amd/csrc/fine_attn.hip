// fine_attn.hip -- stage 3 of the VSA forward on gfx950: block-sparse flash
// attention over 64x64 tiles with bf16 MFMA, online softmax in fp32, and the
// gated coarse combination fused into the epilogue (none when gate is NULL:
// selections of the SubBlock router carry no coarse term).
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
// The kernel is persistent: each single-wavefront workgroup takes units from
// shared work queues (one per head group of XCDs for video units, one per XCD
// for text/audio units; counters in the workspace) until every queue is empty.
// Every K/V element a unit needs is used by that wavefront only, so the
// wavefront streams its operands into a private 40 KiB LDS ring (three K
// slots, two V slots) with global_load_lds_dwordx4 and needs no barriers.
// Stage 1 stored the K and V tiles in the exact per-lane operand order, so
// every load and every LDS operand read is one contiguous 1 KiB wavefront
// access.
//
// Per half-tile, for each of the two 32-query blocks qb:
//   S^T[qb] (32 keys x 32 queries) = K Q^T  -- eight v_mfma_f32_32x32x16_bf16
//   softmax numerators per query column against a fixed per-column reference
//   (each lane owns one column and 16 of its 32 scores; lane ^ 32 owns the
//   other 16)
//   O^T[qb] (128 dims x 32 queries) += V^T P^T  -- eight more MFMAs
// Software pipeline: step x issues the S^T MFMAs of half-tile x+1 and the PV
// MFMAs of half-tile x-1 while the vector unit computes the numerators of
// half-tile x, so no MFMA of a step depends on that step's vector work.  The
// instruction order inside a step is fixed by hand: each MFMA is followed by
// its share of the vector work (one element pair of the numerators) and each
// MFMA pair by one 1 KiB operand copy, so the vector unit works while the
// matrix unit is busy.
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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 64;
// s_getreg_b32 operand for HW_REG_XCC_ID (register 20, bits 0..31): the XCD
// the wavefront runs on, in bits 0..3
constexpr int kHwRegXccId = (31 << 11) | 20;
constexpr int kHalfElems = 32 * kD;  // bf16 elements per packed half-tile (8 KiB)
constexpr int kTileElems = 2 * kHalfElems;
constexpr int kPartFloats = kT * kD + 2 * kT;  // one dense part's record (33,280 bytes)

struct FineArgs {
    const uint16_t* q;
    const uint16_t* gate;
    const uint16_t* kpack;
    const uint16_t* vpack;
    const int32_t* sel;
    const float* coarse;
    uint16_t* out;
    uint32_t* sched;    // kQueues + 4 work-queue counters, 32 words apart, zero at launch
    float* partial;     // dense parts: [dense unit][part][64 x 128 O, 64 l, 64 reference]
    int parts;          // key-list parts per dense unit (1: no split)
    int check_sel;      // nonzero: validate each selection row before use (caller-supplied rows)
    int H, ldh, n_t, n_v, n_a, N, kk;  // ldh: heads per token row (row stride / 128)
    int last_valid[3];  // token rows in the last text / video / audio tile (64 when full)
    float scale_log2;   // log2(e) / sqrt(128)
};

// Work queues.  The kernel is persistent: one workgroup per wavefront slot,
// each taking units (head h, query tile j) from shared counters until every
// queue is empty.  Two kinds of queue:
//  - video queues, one per head group: with NG groups (4 when the head count
//    is a multiple of 4, 2 when it is even, else 1), XCDs 8G/NG .. take the
//    video units of heads h = G mod NG from one counter per group, in
//    head-major order, query tiles ascending.  NG heads are then in flight at
//    a time, each pulled into 8/NG L2s, all of them within the last-level
//    cache, and the XCDs of a group always work on the same head: an XCD that
//    runs slower simply takes fewer units.  (With one queue per XCD the XCDs
//    of a group drift apart on inputs whose selections cluster around each
//    query tile: a lagging XCD's units slow down further and the group ends
//    up spread over several heads.  On such inputs two XCDs per head also
//    keep neighbouring query tiles, which share key tiles, in fewer L2s than
//    four do.);
//  - dense queues, one per XCD: a contiguous 1/8 share of the dense
//    (text/audio query) items, ordered by head, then key-list part, then
//    query tile.  A dense unit's list is every tile (~4.5x a video unit's),
//    so it is walked as P parts of about half a video unit's length and the
//    parts are combined afterwards; the parts of one head share one L2 and
//    sweep their key ranges in step.  They follow the video units (dense items
//    first measured 15-20% slower: the video units then start unevenly).
// Counters: dense queue x at word 32x, video queue G at word 32 (8 + G).
constexpr int kVideoQueue = kQueues;  // queue index of head group 0's video queue
constexpr int kVideoQueues = 4;       // at most four head groups

__device__ __forceinline__ int video_groups(int H) { return (H & 3) == 0 ? 4 : ((H & 1) == 0 ? 2 : 1); }

__device__ __forceinline__ int dense_begin(int D, int x) { return (int)(((int64_t)D * x) / kQueues); }

// Units in queue q (dense: q < 8; video: q = kVideoQueue + G).
__device__ __forceinline__ int queue_count(int H, int n_v, int D, int q) {
    if (q < kQueues) return dense_begin(D, q + 1) - dense_begin(D, q);
    const int G = q - kVideoQueue, NG = video_groups(H);
    return G < NG ? (H / NG) * n_v : 0;
}

// Unit i of queue q -> (h, j) and, for a dense unit, its key-list part p.
__device__ __forceinline__ void queue_unit(int H, int n_t, int n_v, int n_a, int P, int q, int i,
                                           int& h, int& j, int& p) {
    const int n_h = n_t + n_a;
    p = 0;
    if (q < kQueues) {
        const int item = dense_begin(H * P * n_h, q) + i;
        const int hp = item / n_h;  // head-major, then part, then query tile
        const int t = item - hp * n_h;
        h = hp / P;
        p = hp - h * P;
        j = t < n_t ? t : n_v + t;
    } else {
        const int hh = i / n_v;
        h = video_groups(H) * hh + (q - kVideoQueue);
        j = n_t + (i - hh * n_v);
    }
}

// Queue s of the order a workgroup on XCD xcc tries: its group's video
// queue, its own dense queue, the other XCDs' dense queues, then the other
// groups' video queues (empty ones are skipped), so that faster XCDs take
// units from slower ones and no slot idles while work remains.
__device__ __forceinline__ int queue_order(int H, int xcc, int s) {
    const int NG = video_groups(H);
    const int G = xcc / (kQueues / NG);
    if (s == 0) return kVideoQueue + G;
    if (s <= kQueues) return (xcc + s - 1) & (kQueues - 1);
    return kVideoQueue + (G + s - kQueues) % NG;
}

// Returns the index of the next unit in queue `q`, or -1 when every queue is
// empty.  `empty` collects the queues this workgroup has seen exhausted.
__device__ __forceinline__ int next_unit(uint32_t* sched, int H, int n_t, int n_v, int n_a, int P,
                                         int xcc, uint32_t& empty, int& q) {
    const int D = H * P * (n_t + n_a);
#pragma unroll 1
    for (int s = 0; s < kQueues + kVideoQueues; ++s) {
        q = queue_order(H, xcc, s);
        if ((empty >> q) & 1u) continue;
        const int count = queue_count(H, n_v, D, q);
        uint32_t i = 0;
        if (count > 0) {
            if (threadIdx.x == 0) i = atomicAdd(sched + 32 * q, 1u);
            i = __builtin_amdgcn_readfirstlane(i);
            if ((int)i < count) return (int)i;
        }
        empty |= 1u << q;
    }
    return -1;
}

__global__ void clear_sched_kernel(uint32_t* sched) {
    for (int i = threadIdx.x; i < 32 * (kQueues + kVideoQueues); i += blockDim.x) sched[i] = 0u;
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Token (non-padding) rows of global tile t: 64 except in a segment's last
// tile when the segment is padded.  Padding rows are never keys and output
// zeros (page "UniServe: serving FastH3 at its fastest", section "Fused
// attention preprocessing": padding never becomes an input of later steps).
__device__ __forceinline__ int tile_rows(const FineArgs& a, int t) {
    if (t == a.n_t - 1) return a.last_valid[0];
    if (t == a.n_t + a.n_v - 1) return a.last_valid[1];
    if (t == a.N - 1) return a.last_valid[2];
    return kT;
}

// Drop the keys at or past `nvh` (keys of a half-tile, in packed order) from
// one S^T block: lane l, element e holds key kappa(8(e/4) + 4(l/32) + e%4).
__device__ __forceinline__ void mask_keys(f32x16& s, int nvh, int g) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int r = 8 * (e >> 2) + 4 * g + (e & 3);
        const int key = (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
        if (key >= nvh) s[e] = -__builtin_inff();
    }
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

// A selection row is usable when it holds kk distinct video tiles in
// ascending order, each in [0, n_v).  Checked by the whole wavefront, 64
// entries at a time; ordinary vector loads, issued before the unit starts
// its own copies.
__device__ __forceinline__ bool selection_row_ok(const int32_t* row, int kk, int n_v, int lane) {
    bool bad = false;
#pragma unroll 1
    for (int i0 = 0; i0 < kk; i0 += 64) {
        const int i = i0 + lane;
        if (i < kk) {
            const int w = row[i];
            const int prev = i > 0 ? row[i - 1] : -1;
            bad = bad || w < 0 || w >= n_v || w <= prev;
        }
    }
    return __ballot(bad) == 0;
}

// Scalar (wave-uniform) load of one selected-tile index: a scalar load keeps
// it out of the vector-memory counter that the operand prefetches occupy.
__device__ __forceinline__ int load_uniform(const int32_t* p) {
    int v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
    return v;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Start the copy of one packed half-tile operand block (8 KiB = 8 x 1 KiB)
// from global memory straight into an LDS slot: eight global_load_lds_dwordx4
// with a wave-uniform 64-bit base in SGPRs and the per-lane offsets
// voff[i] = 16 * lane + 1024 * i, so issuing them costs no vector ALU work.
// M0 holds the LDS destination of each 1 KiB piece (lane l writes bytes
// 16l .. 16l+15 of it).  Nothing else in the kernel uses M0.  Completion is
// tracked by vmcnt only; the compiler does not see these loads, so every
// consumer waits with an explicit vmcnt value.
__device__ __forceinline__ void fetch_half(uint32_t slot, const char* base, const uint32_t (&voff)[8]) {
    asm volatile(
        "s_mov_b32 m0, %[s]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[v0], %[b]\n\t"
        "s_add_u32 m0, %[s], 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[v1], %[b]\n\t"
        "s_add_u32 m0, %[s], 0x800\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[v2], %[b]\n\t"
        "s_add_u32 m0, %[s], 0xc00\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[v3], %[b]\n\t"
        "s_add_u32 m0, %[s], 0x1000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[v4], %[b]\n\t"
        "s_add_u32 m0, %[s], 0x1400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[v5], %[b]\n\t"
        "s_add_u32 m0, %[s], 0x1800\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[v6], %[b]\n\t"
        "s_add_u32 m0, %[s], 0x1c00\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[v7], %[b]"
        :
        : [s] "s"(slot), [b] "s"(base), [v0] "v"(voff[0]), [v1] "v"(voff[1]), [v2] "v"(voff[2]),
          [v3] "v"(voff[3]), [v4] "v"(voff[4]), [v5] "v"(voff[5]), [v6] "v"(voff[6]),
          [v7] "v"(voff[7])
        : "memory", "m0", "scc");
}

// One 1 KiB piece of a half-tile copy: LDS bytes ldsaddr + 16 lane .. +15
// from global base + voff (voff = 16 lane + 1024 i for piece i).
__device__ __forceinline__ void fetch_piece(uint32_t ldsaddr, const char* base, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %[s]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[v], %[b]"
                 :
                 : [s] "s"(ldsaddr), [b] "s"(base), [v] "v"(voff)
                 : "memory", "m0");
}

// Wait until at most n of this wave's vector-memory loads are outstanding
// (s_waitcnt encoding: vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt at
// their "no wait" maxima).  The compiler does not track the LDS writes of
// global_load_lds, so these waits are what makes a ring slot readable.
__device__ __forceinline__ void wait_vmcnt(int n) {
    if (n >= 32) __builtin_amdgcn_s_waitcnt(0x8F70);       // vmcnt(32)
    else if (n >= 24) __builtin_amdgcn_s_waitcnt(0x4F78);  // vmcnt(24)
    else if (n >= 16) __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16)
    else if (n >= 8) __builtin_amdgcn_s_waitcnt(0x0F78);   // vmcnt(8)
    else __builtin_amdgcn_s_waitcnt(0x0F70);               // vmcnt(0)
    asm volatile("" ::: "memory");
}

// Wait for every outstanding LDS read (and scalar load) of this wave.  Issued
// through the builtin, so the compiler knows that everything it tracks on
// this counter is complete afterwards and inserts no further waits for it.
__device__ __forceinline__ void wait_lgkm() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("" ::: "memory");
}

// Column max of one S^T block (16 values here, 16 in lane ^ 32), times scale_log2.
__device__ __forceinline__ float column_max(const f32x16& s, float c2) {
    float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, s[i]), s[i + 1]);
    mx = fmaxf(mx, s[15]);
    return xhalf_max(mx) * c2;
}

// The four packed operand blocks (8 K or V operands of one half-tile) this
// lane reads from a ring slot: operand i is at byte 1024 i + 16 lane.
typedef __attribute__((address_space(3))) const bf16x8* lds_bf16x8_ptr;
__device__ __forceinline__ void read_ops(bf16x8 (&op)[8], uint32_t slot, int lane) {
    const lds_bf16x8_ptr p = (lds_bf16x8_ptr)(uintptr_t)slot + lane;
#pragma unroll
    for (int i = 0; i < 8; ++i) op[i] = p[i * 64];
}

__global__ __launch_bounds__(kThreads) void fine_attn_kernel(FineArgs a) {
    // Ring: K slots at 0, 8 and 16 KiB, V slots at 24 and 32 KiB.  After the
    // loop the first 32 KiB stage the fp32 output.
    __shared__ __align__(1024) unsigned char lds[5 * 8192];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)lds;
    const uint32_t vslot[2] = {lds0 + 24576u, lds0 + 32768u};
    auto kslot = [&](int i) -> uint32_t { return lds0 + 8192u * (uint32_t)i; };

    const int xcc = (int)(__builtin_amdgcn_s_getreg(kHwRegXccId) & (kQueues - 1));
    uint32_t empty = 0;
#pragma unroll 1
    for (;;) {
        int qx;
        const int qi = next_unit(a.sched, a.H, a.n_t, a.n_v, a.n_a, a.parts, xcc, empty, qx);
        if (qi < 0) break;
        // the lane index passes through an opaque move in every iteration, so the
        // compiler keeps no lane-dependent address of the unit body live across
        // units (hoisting them out of this loop would spill)
        int lane;
        asm volatile("v_mov_b32 %0, %1" : "=v"(lane) : "v"((int)threadIdx.x));
        const int g = lane >> 5, l32 = lane & 31;
        int h, j, part;
        queue_unit(a.H, a.n_t, a.n_v, a.n_a, a.parts, qx, qi, h, j, part);
        if (h >= a.H || j >= a.N) break;  // not reached: the queues partition the units
        const int64_t rs = (int64_t)a.ldh * kD;  // elements between consecutive tokens
        const bool video = j >= a.n_t && j < a.n_t + a.n_v;
        const int u = j - a.n_t;
        // a dense unit's list (every tile) is walked as `parts` contiguous
        // ranges by separate units whose unnormalised results are combined
        // afterwards; part p covers tiles it0 .. it0 + n_tiles - 1
        const bool split = !video && a.parts > 1;
        const int it0 = video ? 0 : (int)((int64_t)part * a.N / a.parts);
        const int n_tiles =
            video ? a.n_t + a.kk + a.n_a : (int)((int64_t)(part + 1) * a.N / a.parts) - it0;
        const int32_t* selrow = a.sel + ((int64_t)h * a.n_v + (video ? u : 0)) * a.kk;
        const float c2 = a.scale_log2;
        if (a.check_sel && video && !selection_row_ok(selrow, a.kk, a.n_v, lane)) {
            // a malformed row is not attended: the unit's 64 output rows are
            // written as NaN, so the error cannot pass for a result
            const uint4 nan8 = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = (lane >> 4) + 4 * i;
                *(uint4*)(a.out + ((int64_t)j * kT + row) * rs + (int64_t)h * kD + 8 * (lane & 15)) = nan8;
            }
            continue;
        }

        // position `it` of this unit's ascending key-tile list -> tile index;
        // positions past the end name the last tile
        auto tile_at = [&](int it) -> int {
            if (it >= n_tiles) it = n_tiles - 1;
            if (!video) return it0 + it;
            if (it < a.n_t) return it;
            if (it < a.n_t + a.kk) {
                // rows are validated (caller-supplied) or valid by construction;
                // the clamp only keeps every address inside the packed tiles
                const int w = load_uniform(selrow + (it - a.n_t));
                return a.n_t + (w < 0 ? 0 : (w >= a.n_v ? a.n_v - 1 : w));
            }
            return a.n_v + it - a.kk;
        };
        // request the raw selection word for list position `it` (clamped to
        // the list) with an ordinary scalar load from a uniform address in the
        // constant address space; decode it later (tile_dec), so the load's own
        // wait is paid where nothing else is pending.  Positions that need no
        // word load a harmless one (the work-queue counters).
        auto tile_req = [&](int it) -> int {
            if (it >= n_tiles) it = n_tiles - 1;
            const bool need = video && it >= a.n_t && it < a.n_t + a.kk;
            const int32_t* src = need ? selrow + (it - a.n_t) : (const int32_t*)a.sched;
            const uint64_t pa = (uint64_t)(uintptr_t)src;
            const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)pa);
            const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(pa >> 32));
            typedef __attribute__((address_space(4))) const int32_t* const_i32_ptr;
            return *(const_i32_ptr)(((uint64_t)hi << 32) | lo);
        };
        auto tile_dec = [&](int it, int word) -> int {
            if (it >= n_tiles) it = n_tiles - 1;
            if (!video) return it0 + it;
            if (it < a.n_t) return it;
            if (it < a.n_t + a.kk) return a.n_t + (word < 0 ? 0 : (word >= a.n_v ? a.n_v - 1 : word));
            return a.n_v + it - a.kk;
        };
        // per-head bases of the packed operands (bytes): 16 KiB per tile and
        // tensor, two 8 KiB half-tiles each
        const char* kbase = (const char*)(a.kpack + (int64_t)h * a.N * (kT * kD));
        const char* vbase = (const char*)(a.vpack + (int64_t)h * a.N * (kT * kD));
        constexpr int64_t kTileBytes = 2 * kTileElems;
        constexpr int64_t kHalfBytes = 2 * kHalfElems;
        uint32_t voff[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) voff[i] = 16u * lane + 1024u * i;
        auto fetch_k = [&](uint32_t slot, int tile, int half) {
            fetch_half(slot, kbase + tile * kTileBytes + half * kHalfBytes, voff);
        };
        auto fetch_v = [&](uint32_t slot, int tile, int half) {
            fetch_half(slot, vbase + tile * kTileBytes + half * kHalfBytes, voff);
        };

        // Q^T fragments (B operand of S^T = K Q^T): query l32 of block qb, dims 16s + 8g .. +7
        bf16x8 qf[2][8];
#pragma unroll
        // Q, the gate and the output rows are each touched once: non-temporal
        // accesses keep them from displacing K/V lines in the L2
        for (int qb = 0; qb < 2; ++qb) {
            const uint16_t* qp = a.q + ((int64_t)j * kT + 32 * qb + l32) * rs + (int64_t)h * kD + 8 * g;
#pragma unroll
            for (int s8 = 0; s8 < 8; ++s8)
                qf[qb][s8] = __builtin_nontemporal_load((const bf16x8*)(qp + 16 * s8));
        }
        wait_vmcnt(0);  // Q is resident before the ring starts counting loads
        // padding query rows (past the tile's token rows) attend with zeros and
        // are written as zeros
        const int nq = tile_rows(a, j);
        if (nq < kT) {
            bf16x8 z8;
#pragma unroll
            for (int i = 0; i < 8; ++i) z8[i] = (__bf16)0.0f;
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
                if (32 * qb + l32 >= nq)
#pragma unroll
                    for (int s8 = 0; s8 < 8; ++s8) qf[qb][s8] = z8;
        }

        // Q fragments live in AGPRs (the MFMA reads its B operand from either
        // register file), which leaves the vector registers to the values that
        // change every step
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int s8 = 0; s8 < 8; ++s8) asm volatile("" : "=a"(qf[qb][s8]) : "0"(qf[qb][s8]));
        const int t0 = tile_at(0), t1 = tile_at(1);

        // Softmax reference.  Each column uses one fixed reference m_ref (in units
        // of scale_log2 * score) for its whole key list: P = 2^(x - m_ref), and O
        // and l accumulate without any rescaling.  m_ref starts at the column max
        // of the first half-tile, so the largest P of that half-tile is 1.  If a
        // later score exceeds it by so much that the denominator passes 2^100 (or
        // overflows), the unit is recomputed with m_ref raised by log2 of the
        // denominator (by 126 if it overflowed); the result is the same softmax,
        // and for ordinary inputs the first pass is the only pass.
        float m_ref[2];
        f32x16 o[2][4];
        float l_run[2];
        f32x16 zero16;
#pragma unroll
        for (int i = 0; i < 16; ++i) zero16[i] = 0.0f;
        bf16x8 zero8;
#pragma unroll
        for (int i = 0; i < 8; ++i) zero8[i] = (__bf16)0.0f;
        for (int pass = 0;; ++pass) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                l_run[qb] = 0.0f;
#pragma unroll
                for (int db = 0; db < 4; ++db) o[qb][db] = zero16;
            }
            // Half-tile x of the list: K(x) and V(x) are half (x & 1) of tile
            // (x >> 1), staged in K slot x mod 3 and V slot x mod 2.  Step x
            // computes
            //   S^T(x+1) = K(x+1) Q^T              (16 MFMAs)
            //   P(x)     = 2^(S^T(x) scale_log2 - m_ref), rounded to bf16, and
            //              its sum added to the denominators (vector ALU)
            //   O       += V(x-1) P(x-1)            (16 MFMAs)
            // so none of its matrix work waits for its own vector work.  Operands
            // enter registers one step ahead (K(x+2) in the middle of step x,
            // V(x) at its end).  Step x fetches V(x+1), one 1 KiB piece after
            // each pair of S^T MFMAs, and then K(x+4), one piece after each pair
            // of PV MFMAs, so the copies issue while the matrix unit is busy; a
            // K half-tile has about two steps to arrive and a V half-tile two.
            // In issue order, K(x+2) is complete once at most 24 fetches are
            // outstanding at the middle of the step (V(x), K(x+3) of step x-1 and
            // V(x+1)), and V(x) once at most 24 are at its end (K(x+3), V(x+1),
            // K(x+4)).
            bf16x8 kop[8], vop[8];
            bf16x8 pprev[2][2];
            f32x16 sc[2];
            // prologue: K(0), K(1), K(2); S^T(0); then V(0), K(3) as the fetches
            // of step -1; PV(-1) multiplies zeros
            fetch_k(kslot(0), t0, 0);
            fetch_k(kslot(1), t0, 1);
            fetch_k(kslot(2), t1, 0);
            wait_vmcnt(16);
            read_ops(kop, kslot(0), lane);
            sc[0] = zero16;
            sc[1] = zero16;
#pragma unroll
            for (int s8 = 0; s8 < 8; ++s8) {
                sc[0] = mfma32(kop[s8], qf[0][s8], sc[0]);
                sc[1] = mfma32(kop[s8], qf[1][s8], sc[1]);
            }
            wait_vmcnt(8);
            wait_lgkm();
            read_ops(kop, kslot(1), lane);
            fetch_v(vslot[0], t0, 0);
            fetch_k(kslot(0), t1, 1);
#pragma unroll
            for (int i = 0; i < 8; ++i) vop[i] = zero8;
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) pprev[qb][0] = pprev[qb][1] = zero8;
            {
                const int nv0 = tile_rows(a, t0);  // S^T(0) is half 0 of the first tile
                if (nv0 < 32) {
                    mask_keys(sc[0], nv0, g);
                    mask_keys(sc[1], nv0, g);
                }
            }
            if (pass == 0) {
                m_ref[0] = column_max(sc[0], c2);
                m_ref[1] = column_max(sc[1], c2);
            }

            // tiles of list positions t, t+1 (cur, nxt) carried across iterations;
            // xm3 = x mod 3 for the current step x
            int cur = t0, nxt = t1;
            int xm3 = 0;
            for (int t = 0; t < n_tiles; ++t) {
                int nn = 0, nn_word = 0;
                const int rows_cur = tile_rows(a, cur);  // token rows of the tile in use
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    // step x = 2t + pp
                    const int k_wr = xm3 == 2 ? 0 : xm3 + 1;  // (x + 4) mod 3
                    const int k_rd = xm3 == 0 ? 2 : xm3 - 1;  // (x + 2) mod 3
                    // V(x+1): (t, half 1) or (t+1, half 0); K(x+4): (t+2, half pp),
                    // issued one 1 KiB piece at a time between MFMAs below
                    const char* vsrc = vbase + (pp == 0 ? cur : nxt) * kTileBytes + (pp ^ 1) * kHalfBytes;
                    const char* ksrc = kbase + pp * kHalfBytes;  // + nn * kTileBytes below
                    const uint32_t vdst = vslot[pp ^ 1], kdst = kslot(k_wr);
                    f32x16 n0 = zero16, n1 = zero16;
                    bf16x8 pc[2][2];
                    {
                        // keys of half pp of the current tile that are tokens
                        const int nvh = rows_cur - 32 * pp;
                        if (nvh < 32) {
                            mask_keys(sc[0], nvh, g);
                            mask_keys(sc[1], nvh, g);
                        }
                    }
                    // The step in issue order.  Every MFMA is followed by one element
                    // pair (e, 8 + e) of the numerators of S^T(x) (first half: block 0
                    // with the S^T MFMAs; second half: block 1 with the PV MFMAs) and
                    // every MFMA pair by one operand copy.  MFMAs and numerators have no
                    // side effects, so instruction selection would otherwise gather
                    // them next to their uses (16 MFMAs in a row, the exponentials of
                    // two steps in a row): each result passes through an empty asm
                    // statement right where it is made, which fixes its place in the
                    // program order, and sched_barrier(0) keeps the machine scheduler
                    // from merging the groups.  The denominators add the pairs in the
                    // order e = 0..7, as a plain loop would.
                    f32x8 na0, nb0, na1, nb1;
                    float ls0 = 0.0f, ls1 = 0.0f;
                    const float mr0 = m_ref[0], mr1 = m_ref[1];
#pragma unroll
                    for (int s8 = 0; s8 < 8; ++s8) {
                        n0 = mfma32(kop[s8], qf[0][s8], n0);
                        asm volatile("" : "+a"(n0));
                        __builtin_amdgcn_sched_barrier(0);
                        na0[s8] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[0][s8], c2, -mr0));
                        nb0[s8] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[0][8 + s8], c2, -mr0));
                        __builtin_amdgcn_sched_barrier(0);
                        n1 = mfma32(kop[s8], qf[1][s8], n1);
                        asm volatile("" : "+a"(n1));
                        __builtin_amdgcn_sched_barrier(0);
                        // exp2 results are >= +0, so starting from the first pair's sum
                        // equals adding it to 0
                        ls0 = s8 == 0 ? na0[s8] + nb0[s8] : ls0 + (na0[s8] + nb0[s8]);
                        asm volatile("" ::"v"(na0[s8]), "v"(nb0[s8]), "v"(ls0));
                        if (s8 == 0) {
                            // the V slot written next was read at the end of the last
                            // step: those reads must be complete first.  Waiting here,
                            // one MFMA pair into the step, lets their latency pass
                            // under matrix work.  In the first step of a tile the next
                            // tile index is requested right after the wait and used at
                            // the end of this half, so no scalar load is ever pending
                            // where the compiler waits for LDS reads.
                            wait_lgkm();
                            if (pp == 0) nn_word = tile_req(t + 2);
                        }
                        fetch_piece(vdst + 1024u * s8, vsrc, voff[s8]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    l_run[0] += ls0;
                    pc[0][0] = __builtin_convertvector(na0, bf16x8);
                    pc[0][1] = __builtin_convertvector(nb0, bf16x8);
                    asm volatile("" ::"v"(pc[0][0]), "v"(pc[0][1]));
                    if (pp == 0) {
                        asm volatile("" : "+s"(nn_word));
                        nn = tile_dec(t + 2, nn_word);
                    }
                    wait_vmcnt(24);  // K(x+2)
                    read_ops(kop, kslot(k_rd), lane);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int db = 0; db < 4; ++db)
#pragma unroll
                        for (int m = 0; m < 2; ++m) {
                            const int e = 2 * db + m;
                            o[0][db] = mfma32(vop[e], pprev[0][m], o[0][db]);
                            asm volatile("" : "+a"(o[0][db]));
                            __builtin_amdgcn_sched_barrier(0);
                            na1[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[1][e], c2, -mr1));
                            nb1[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[1][8 + e], c2, -mr1));
                            __builtin_amdgcn_sched_barrier(0);
                            o[1][db] = mfma32(vop[e], pprev[1][m], o[1][db]);
                            asm volatile("" : "+a"(o[1][db]));
                            __builtin_amdgcn_sched_barrier(0);
                            ls1 = e == 0 ? na1[e] + nb1[e] : ls1 + (na1[e] + nb1[e]);
                            asm volatile("" ::"v"(na1[e]), "v"(nb1[e]), "v"(ls1));
                            fetch_piece(kdst + 1024u * e, ksrc + nn * kTileBytes, voff[e]);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    l_run[1] += ls1;
                    pc[1][0] = __builtin_convertvector(na1, bf16x8);
                    pc[1][1] = __builtin_convertvector(nb1, bf16x8);
                    asm volatile("" ::"v"(pc[1][0]), "v"(pc[1][1]));
                    wait_vmcnt(24);  // V(x)
                    read_ops(vop, vslot[pp], lane);
                    sc[0] = n0;
                    sc[1] = n1;
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) {
                        pprev[qb][0] = pc[qb][0];
                        pprev[qb][1] = pc[qb][1];
                    }
                    xm3 = k_wr;  // (x + 1) mod 3
                }
                cur = nxt;
                nxt = nn;
            }
            // the last PV
            wait_lgkm();
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    o[0][db] = mfma32(vop[2 * db + m], pprev[0][m], o[0][db]);
                    o[1][db] = mfma32(vop[2 * db + m], pprev[1][m], o[1][db]);
                }
            wait_vmcnt(0);
            l_run[0] = xhalf_sum(l_run[0]);
            l_run[1] = xhalf_sum(l_run[1]);
            const bool big0 = !(l_run[0] <= 0x1p100f), big1 = !(l_run[1] <= 0x1p100f);
            if (!__ballot(big0 || big1) || pass >= 3) break;
            if (big0) m_ref[0] += l_run[0] <= 0x1p126f ? __log2f(l_run[0]) : 126.0f;
            if (big1) m_ref[1] += l_run[1] <= 0x1p126f ? __log2f(l_run[1]) : 126.0f;
        }

        // ---- epilogue: normalise, stage through LDS, add sigmoid(G) * coarse ----
        // Lane l writes dims 8(l%16) .. +7 of rows l/16 + 4i, i < 16.  The gate
        // rows (never read before, so they come from HBM) and the lane's eight
        // coarse values are all requested here, before the staging, so their
        // latency is paid once per unit rather than once per group of rows.
        const bool gated = video && a.gate;
        const int c16 = lane & 15;
        uint4 gw[16];
        float4 cv0, cv1;
        if (gated) {
            const uint16_t* gp = a.gate + ((int64_t)j * kT + (lane >> 4)) * rs + (int64_t)h * kD + 8 * c16;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const u32x4 t4 = __builtin_nontemporal_load((const u32x4*)(gp + 4 * i * rs));
                gw[i] = make_uint4(t4[0], t4[1], t4[2], t4[3]);
            }
            const float* cp = a.coarse + ((int64_t)h * a.n_v + u) * kD + 8 * c16;
            cv0 = *(const float4*)cp;
            cv1 = *(const float4*)(cp + 4);
        }
        float* ost = (float*)lds;  // [64 queries][128 dims], 16-byte chunks swizzled by row
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float inv = split ? 1.0f : __builtin_amdgcn_rcpf(l_run[qb]);
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
        if (split) {
            // unnormalised O, the denominators and the references of this part
            float* pp = a.partial + (((int64_t)h * (a.n_t + a.n_a) + (j < a.n_t ? j : j - a.n_v)) *
                                         a.parts + part) * kPartFloats;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = (lane >> 4) + 4 * i, c = c16;
                *(float4*)(pp + row * kD + 8 * c) =
                    *(const float4*)(ost + row * kD + 4 * ((2 * c) ^ (row & 15)));
                *(float4*)(pp + row * kD + 8 * c + 4) =
                    *(const float4*)(ost + row * kD + 4 * ((2 * c + 1) ^ (row & 15)));
            }
            if (g == 0) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    pp[kT * kD + 32 * qb + l32] = l_run[qb];
                    pp[kT * kD + kT + 32 * qb + l32] = m_ref[qb];
                }
            }
            wait_lgkm();
            __syncthreads();
            continue;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = (lane >> 4) + 4 * i, c = c16;
            const float4 x0 = *(const float4*)(ost + row * kD + 4 * ((2 * c) ^ (row & 15)));
            const float4 x1 = *(const float4*)(ost + row * kD + 4 * ((2 * c + 1) ^ (row & 15)));
            f32x8 y = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            const int64_t grow = (int64_t)j * kT + row;
            if (row >= nq) {
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = 0.0f;
            } else if (gated) {
                const uint32_t gwv[4] = {gw[i].x, gw[i].y, gw[i].z, gw[i].w};
                const float cv[8] = {cv0.x, cv0.y, cv0.z, cv0.w, cv1.x, cv1.y, cv1.z, cv1.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    y[2 * e] += sigmoidf(__uint_as_float(gwv[e] << 16)) * cv[2 * e];
                    y[2 * e + 1] += sigmoidf(__uint_as_float(gwv[e] & 0xFFFF0000u)) * cv[2 * e + 1];
                }
            }
            __builtin_nontemporal_store(__builtin_convertvector(y, bf16x8),
                                        (bf16x8*)(a.out + grow * rs + (int64_t)h * kD + 8 * c));
        }
        // the next unit's copies overwrite the staging area
        wait_lgkm();
        __syncthreads();
    }
}

// Combination of a split dense unit's parts: with references m_p and
// denominators l_p (per query row), O = sum_p O_p 2^(m_p - M) and
// l = sum_p l_p 2^(m_p - M), M = max_p m_p; out = O / l, in part order.
// One workgroup per dense unit; thread t covers rows t/16 + 16i, dims
// 8(t%16) .. +7.
__global__ __launch_bounds__(256) void combine_parts_kernel(FineArgs a) {
    const int n_h = a.n_t + a.n_a;
    const int du = blockIdx.x;  // h * n_h + dense tile
    const int h = du / n_h, t = du - h * n_h;
    const int j = t < a.n_t ? t : a.n_v + t;
    const int nq = tile_rows(a, j);
    const int64_t rs = (int64_t)a.ldh * kD;
    const float* base = a.partial + (int64_t)du * a.parts * kPartFloats;
    const int c = threadIdx.x & 15;
#pragma unroll 1
    for (int i = 0; i < 4; ++i) {
        const int row = (threadIdx.x >> 4) + 16 * i;
        f32x8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = 0.0f;
        if (row < nq) {
            float mx = -__builtin_inff();
            for (int p = 0; p < a.parts; ++p) mx = fmaxf(mx, base[p * kPartFloats + kT * kD + kT + row]);
            float l = 0.0f;
            for (int p = 0; p < a.parts; ++p) {
                const float* pp = base + p * kPartFloats;
                const float w = __builtin_amdgcn_exp2f(pp[kT * kD + kT + row] - mx);
                l += w * pp[kT * kD + row];
                const float4 x0 = *(const float4*)(pp + row * kD + 8 * c);
                const float4 x1 = *(const float4*)(pp + row * kD + 8 * c + 4);
                y[0] += w * x0.x; y[1] += w * x0.y; y[2] += w * x0.z; y[3] += w * x0.w;
                y[4] += w * x1.x; y[5] += w * x1.y; y[6] += w * x1.z; y[7] += w * x1.w;
            }
            const float inv = __builtin_amdgcn_rcpf(l);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] *= inv;
        }
        *(bf16x8*)(a.out + ((int64_t)j * kT + row) * rs + (int64_t)h * kD + 8 * c) =
            __builtin_convertvector(y, bf16x8);
    }
}

}  // namespace

// Wavefront slots of the device: 4 per CU (40 KiB of LDS each), cached per device.
int fine_slots() {
    static std::atomic<int> slots[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 1024;
    int n = slots[dev].load();
    if (n == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        n = 4 * cus;
        slots[dev].store(n);
    }
    return n;
}

hipError_t launch_fine_attention(const uint16_t* q, const uint16_t* gate, const int32_t* sel,
                                 uint16_t* out, const Shape& s, uint8_t* ws, const Layout& L,
                                 hipStream_t stream, bool check_sel) {
    FineArgs a;
    a.q = q;
    a.gate = gate;
    a.kpack = (const uint16_t*)(ws + L.kpack);
    a.vpack = (const uint16_t*)(ws + L.vpack);
    a.sel = sel;
    a.coarse = (const float*)(ws + L.coarse);
    a.out = out;
    a.sched = (uint32_t*)(ws + L.sched);
    a.partial = (float*)(ws + L.partial);
    a.parts = dense_parts(s);
    a.check_sel = check_sel ? 1 : 0;
    a.H = s.H;
    a.ldh = s.ldh;
    a.n_t = s.n_t;
    a.n_v = s.n_v;
    a.n_a = s.n_a;
    a.N = s.N;
    a.kk = s.k;
    a.last_valid[0] = s.n_t ? (int)(s.V_t - 64 * (int64_t)(s.n_t - 1)) : kT;
    a.last_valid[1] = s.n_v ? (int)(s.V_v - 64 * (int64_t)(s.n_v - 1)) : kT;
    a.last_valid[2] = s.n_a ? (int)(s.V_a - 64 * (int64_t)(s.n_a - 1)) : kT;
    a.scale_log2 = (float)(1.4426950408889634 / 11.313708498984761);
    const int64_t units = (int64_t)s.H * s.N;
    // counters start at zero (a kernel, not a memset node, so that the call
    // can be recorded into a HIP graph)
    hipLaunchKernelGGL(clear_sched_kernel, dim3(1), dim3(64), 0, stream, a.sched);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t grid = units < fine_slots() ? units : fine_slots();
    hipLaunchKernelGGL(fine_attn_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess || a.parts == 1) return e;
    hipLaunchKernelGGL(combine_parts_kernel, dim3((unsigned)(s.H * (s.n_t + s.n_a))), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace vsa

// vsa_internal.h -- shapes, workspace layout and kernel launchers shared by
// the host dispatcher and the gfx950 kernels of the VSA forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <atomic>

namespace vsa {

constexpr int kD = 128;   // head dimension
constexpr int kT = 64;    // tokens per tile
constexpr size_t kAlign = 256;

struct Shape {
    int32_t H;                 // heads this call computes
    // heads per token row of the caller's q/k/v/gate/out (the row stride is
    // ldh * 128 elements): H, unless a call works on a slice of the heads
    int32_t ldh;
    int64_t S_t, S_v, S_a, S;
    int32_t n_t, n_v, n_a, N;  // tile counts
    int32_t k;                 // selected tiles per video query tile
    // valid (token) rows at the start of each segment; the rest of the
    // segment's last tile is padding (S_x - 64 < V_x <= S_x when S_x > 0)
    int64_t V_t, V_v, V_a;
};

// Valid rows of global tile j (64 for every tile but a segment's last).
__host__ __device__ inline int tile_valid_rows(const Shape& s, int j) {
    int64_t v;
    if (j < s.n_t) v = s.V_t - 64 * (int64_t)j;
    else if (j < s.n_t + s.n_v) v = s.V_v - 64 * (int64_t)(j - s.n_t);
    else v = s.V_a - 64 * (int64_t)(j - s.n_t - s.n_v);
    return v >= 64 ? 64 : (v > 0 ? (int)v : 0);
}

// Attention preprocessing (learned Q/K RMSNorm, partial 3D RoPE of video
// tokens at their latent-grid positions).  gamma_q == nullptr: none.
struct Prep {
    const uint16_t* gamma_q;  // bf16 [H][128]
    const uint16_t* gamma_k;  // bf16 [H][128]
    int32_t grid[3];          // latent grid T x H x W of the valid video tokens
    int32_t tile[3];          // tile-packing shape
};

// Workspace regions (byte offsets from the workspace base).
struct Layout {
    size_t qbar64;  // double [H][n_v][128], dims in pooled_dim_pos order
    size_t kbar;    // float  [H][n_v][128], dims in pooled_dim_pos order
    size_t vbar;    // float  [H][128][vbar_pitch(n_v)] (transposed; columns past n_v are zero)
    size_t coarse;  // float  [H][n_v][128]
    size_t kpack;   // bf16   [H][N][2][8][64][8]      K tiles in MFMA A-operand order
    size_t vpack;   // bf16   [H][N][2][4][2][64][8]   V^T tiles in MFMA A-operand order
    size_t partial; // float  [H][n_t+n_a][kMaxParts][64*128 + 128]  split dense units' partial results
    size_t sched;   // uint32 [12][32] fine-attention work-queue counters (one 128-byte line each)
    size_t qsub;    // float  [H][n_c][8][64][4]  SubBlock router: Q sub-block means (0 bytes
    size_t ksub;    // float  [H][n_c][8][64][4]  without the router), n_c = ceil(n_v / 4)
    size_t total;
};

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Largest n_v the SubBlock router takes: 4 rows of n_v float64 scores fill
// the 160 KiB of LDS, and the wavefront top-k holds 80 keys per lane.
constexpr int kSubblockMaxTiles = 5120;

// Fine-attention work queues: kQueues dense (text/audio unit) queues, one per
// XCD, then up to four video-unit queues, one per head group of XCDs; each
// counter on its own 128-byte line.
constexpr int kQueues = 8;
constexpr size_t kSchedBytes = (kQueues + 4) * 128;
// A dense (text/audio query) unit's key list is split into at most this many
// parts; one part's record is 64 x 128 unnormalised outputs, 64 denominators
// and 64 softmax references, float32.
constexpr int kMaxParts = 8;
constexpr size_t kPartBytes = (64 * 128 + 128) * sizeof(float);

// Key-list parts of a dense unit: about half the length of a video unit's
// list, at most kMaxParts; 1 without video tiles.  No unit is then much
// longer than the rest, and the dense parts that close the queues are short,
// so the launch ends with little idle time.  The count depends on the
// per-head shape only, so a call split into groups of heads splits its
// dense units exactly as the whole call does.
inline int dense_parts(const Shape& s) {
    if (s.n_v == 0 || s.n_t + s.n_a == 0) return 1;
    const int lv = s.n_t + s.k + s.n_a;
    int p = (int)(2.0 * (double)s.N / (double)lv + 0.5);
    return p < 1 ? 1 : (p > kMaxParts ? kMaxParts : p);
}

// Storage order of the 128 dims of a pooled Q or K row: dim d = 4 s + g sits
// at position 32 g + s, so that the score MFMAs' lane group g (which feeds
// dims 4 s + g, s = 0..31) reads 32 consecutive values.
__host__ __device__ inline int pooled_dim_pos(int d) { return (d & 3) * 32 + (d >> 2); }

// Row pitch (floats) of the transposed pooled V: n_v rounded up to 16, so
// that every 16-key block of a row is 64-byte aligned and lies inside it.
__host__ __device__ inline int vbar_pitch(int n_v) { return (n_v + 15) & ~15; }

// pooled = false: no pooled statistics or coarse regions (a caller that only
// packs tiles and routes with the SubBlock piece means).
inline Layout make_layout(const Shape& s, bool subblock = false, bool pooled = true) {
    Layout L;
    size_t off = 0;
    const size_t hv = pooled ? (size_t)s.H * (size_t)s.n_v * kD : 0;
    L.qbar64 = off; off = align_up(off + hv * sizeof(double));
    L.kbar = off;   off = align_up(off + hv * sizeof(float));
    L.vbar = off;   off = align_up(off + (pooled ? (size_t)s.H * kD * vbar_pitch(s.n_v) : 0) * sizeof(float));
    L.coarse = off; off = align_up(off + hv * sizeof(float));
    L.kpack = off;  off = align_up(off + (size_t)s.H * (size_t)s.N * kT * kD * 2);
    L.vpack = off;  off = align_up(off + (size_t)s.H * (size_t)s.N * kT * kD * 2);
    const size_t sub = subblock ? (size_t)s.H * (size_t)((s.n_v + 3) / 4) * 2048 * sizeof(float) : 0;
    const size_t dense_units = (size_t)s.H * (size_t)(s.n_t + s.n_a);
    // sized for kMaxParts, so that the layout does not depend on k (which the
    // layout query does not take)
    L.partial = off; off = align_up(off + (s.n_v > 0 ? dense_units * kMaxParts * kPartBytes : 0));
    L.sched = off;  off = align_up(off + kSchedBytes);
    L.qsub = off;   off = align_up(off + sub);
    L.ksub = off;   off = align_up(off + sub);
    L.total = off;
    return L;
}

// Devices a process may use with this library (the host entry points
// reject device ordinals at or past it).
constexpr int kMaxDevices = 64;

// Raise `kernel`'s dynamic-LDS limit to `bytes` on the current device the
// first time a launch there needs it; `allowed` keeps the limit set so far per
// device (concurrent first calls only repeat the same attribute call).
inline hipError_t ensure_dynamic_lds(const void* kernel, std::atomic<size_t>* allowed,
                                     size_t bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (bytes > allowed[dev].load()) {
        e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
        if (e != hipSuccess) return e;
        allowed[dev].store(bytes);
    }
    return hipSuccess;
}

// ---- launchers (each enqueues on `stream`, returns the launch status) ----
hipError_t launch_pool_pack(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const Shape& s, uint8_t* ws, const Layout& L, hipStream_t stream,
                            const Prep* prep = nullptr, uint16_t* q_out = nullptr,
                            bool pooled = true);
hipError_t launch_select_coarse(const Shape& s, int32_t* sel, uint8_t* ws, const Layout& L,
                                hipStream_t stream);
// check_sel: validate every selection row on the device first (rows given by
// the caller); a malformed row's 64 output rows are written as NaN.
hipError_t launch_fine_attention(const uint16_t* q, const uint16_t* gate,
                                 const int32_t* sel, uint16_t* out, const Shape& s,
                                 uint8_t* ws, const Layout& L, hipStream_t stream,
                                 bool check_sel = false);

// SubBlock router: sub-block means of Q and K, scores and top-k (s.k tiles).
hipError_t launch_subblock_route(const uint16_t* q, const uint16_t* k, const Shape& s,
                                 int32_t* sel, uint8_t* ws, const Layout& L, hipStream_t stream);

// Device address and size of the fixed scratch array of vsa_forward_noalloc
// on the current device (looked up once per device, then cached).
hipError_t noalloc_scratch(void** out, size_t* bytes);

hipError_t launch_project_qkvg(const uint16_t* x, const uint16_t* w, uint16_t* const out[4],
                               int64_t tokens, int hidden, int n_out, hipStream_t stream);

}  // namespace vsa

// vsa_api.cpp -- host side of the C ABI declared in include/vsa.h: argument
// validation (before any HIP call), shape bookkeeping, workspace carving and
// kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "vsa.h"
#include "vsa_internal.h"

using vsa::Layout;
using vsa::Shape;

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Shape validation shared by every entry point.  No HIP call.
vsa_status make_shape(int32_t H, int64_t S_t, int64_t S_v, int64_t S_a, Shape* s) {
    if (H < 1 || S_t < 0 || S_v < 0 || S_a < 0) return VSA_ERR_BAD_SHAPE;
    if (H > VSA_MAX_HEADS || S_t > VSA_MAX_TOKENS || S_v > VSA_MAX_TOKENS || S_a > VSA_MAX_TOKENS)
        return VSA_ERR_TOO_LARGE;
    const int64_t S = S_t + S_v + S_a;
    if (S == 0) return VSA_ERR_BAD_SHAPE;
    if (S_t % VSA_TILE || S_v % VSA_TILE || S_a % VSA_TILE) return VSA_ERR_UNALIGNED_LENGTH;
    if (S > VSA_MAX_TOKENS) return VSA_ERR_TOO_LARGE;
    if (S_v / VSA_TILE > VSA_MAX_VIDEO_TILES) return VSA_ERR_TOO_LARGE;
    s->H = H;
    s->ldh = H;
    s->S_t = S_t;
    s->S_v = S_v;
    s->S_a = S_a;
    s->S = S;
    s->n_t = (int32_t)(S_t / VSA_TILE);
    s->n_v = (int32_t)(S_v / VSA_TILE);
    s->n_a = (int32_t)(S_a / VSA_TILE);
    s->N = s->n_t + s->n_v + s->n_a;
    s->k = 0;
    s->V_t = S_t;
    s->V_v = S_v;
    s->V_a = S_a;
    return VSA_OK;
}

int32_t topk_count(int64_t n_v, float frac) {
    const double f = (double)frac;
    if (!(f > 0.0 && f <= 1.0) || n_v < 0) return -1;
    if (n_v == 0) return 0;
    double k = std::floor(f * (double)n_v + 0.5);
    if (k < 1.0) k = 1.0;
    if (k > (double)n_v) k = (double)n_v;
    return (int32_t)k;
}

// SubBlock router kept count: whole groups of 8 tiles, at least one group
// (or every tile when there are fewer than 8), at most n_v.
int32_t subblock_count(int64_t n_v, float sparsity) {
    const double f = (double)sparsity;
    if (!(f >= 0.0 && f < 1.0) || n_v < 0) return -1;
    if (n_v == 0) return 0;
    double k = 8.0 * std::floor((1.0 - f) * (double)n_v / 8.0 + 0.5);
    const double lo = n_v < 8 ? (double)n_v : 8.0;
    if (k < lo) k = lo;
    if (k > (double)n_v) k = (double)n_v;
    return (int32_t)k;
}

// The whole-sequence SubBlock mode on a relabelled shape: every tile counts
// as a "video" tile (no text or audio segment, n_v = N), so the router ranks
// all N tiles for every query tile and the fine kernel walks exactly each
// query tile's kept list.  No pooled statistics and no coarse term.
vsa_status whole_shape(int32_t H, int64_t S_t, int64_t S_v, int64_t S_a, float sparsity,
                       Shape* w) {
    Shape s;
    vsa_status st = make_shape(H, S_t, S_v, S_a, &s);
    if (st != VSA_OK) return st;
    if (s.N > vsa::kSubblockMaxTiles) return VSA_ERR_TOO_LARGE;
    const int32_t kk = subblock_count(s.N, sparsity);
    if (kk < 0) return VSA_ERR_BAD_TOPK;
    *w = s;
    w->S_t = 0;
    w->S_v = s.S;
    w->S_a = 0;
    w->n_t = 0;
    w->n_v = s.N;
    w->n_a = 0;
    w->V_t = 0;
    w->V_v = s.S;
    w->V_a = 0;
    w->k = kk;
    return VSA_OK;
}

vsa_status check_topk(float frac, Shape* s) {
    const int32_t k = topk_count(s->n_v, frac);
    if (k < 0) return VSA_ERR_BAD_TOPK;
    s->k = k;
    return VSA_OK;
}

vsa_status check_workspace(const void* ws, size_t bytes, const Layout& L) {
    if (!ws) return VSA_ERR_WORKSPACE;
    if (!aligned(ws, vsa::kAlign)) return VSA_ERR_MISALIGNED;
    if (bytes < L.total) return VSA_ERR_WORKSPACE;
    return VSA_OK;
}

// The kernels are written for gfx950 only.  Checked once per device.
vsa_status check_device() {
    static std::mutex mu;
    static int known[64] = {0};  // 0 unknown, 1 ok, 2 wrong arch
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return VSA_ERR_HIP;
    if (dev < 0 || dev >= 64) return VSA_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(mu);
    if (known[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return VSA_ERR_HIP;
        known[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    }
    return known[dev] == 1 ? VSA_OK : VSA_ERR_DEVICE;
}

// Library-owned workspace for vsa_forward(workspace = NULL): grow-only, one per device.
struct OwnedWorkspace {
    void* ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_ws_mu;
OwnedWorkspace g_ws[64];

vsa_status owned_workspace(size_t need, void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return VSA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_ws_mu);
    OwnedWorkspace& w = g_ws[dev];
    if (w.bytes < need) {
        if (w.ptr) {
            if (hipDeviceSynchronize() != hipSuccess) return VSA_ERR_HIP;
            if (hipFree(w.ptr) != hipSuccess) return VSA_ERR_HIP;
            w.ptr = nullptr;
            w.bytes = 0;
        }
        if (hipMalloc(&w.ptr, need) != hipSuccess) return VSA_ERR_HIP;
        w.bytes = need;
    }
    *out = w.ptr;
    return VSA_OK;
}

vsa_status from_hip(hipError_t e) { return e == hipSuccess ? VSA_OK : VSA_ERR_HIP; }

}  // namespace

extern "C" {

const char* vsa_status_string(vsa_status s) {
    switch (s) {
        case VSA_OK: return "VSA_OK";
        case VSA_ERR_NULL_POINTER: return "VSA_ERR_NULL_POINTER";
        case VSA_ERR_BAD_SHAPE: return "VSA_ERR_BAD_SHAPE";
        case VSA_ERR_UNALIGNED_LENGTH: return "VSA_ERR_UNALIGNED_LENGTH";
        case VSA_ERR_BAD_TOPK: return "VSA_ERR_BAD_TOPK";
        case VSA_ERR_MISALIGNED: return "VSA_ERR_MISALIGNED";
        case VSA_ERR_WORKSPACE: return "VSA_ERR_WORKSPACE";
        case VSA_ERR_DEVICE: return "VSA_ERR_DEVICE";
        case VSA_ERR_HIP: return "VSA_ERR_HIP";
        case VSA_ERR_TOO_LARGE: return "VSA_ERR_TOO_LARGE";
    }
    return "VSA_ERR_UNKNOWN";
}

int32_t vsa_topk_count(int64_t video_len, float topk_frac) {
    if (video_len < 0 || video_len % VSA_TILE) return -1;
    return topk_count(video_len / VSA_TILE, topk_frac);
}

size_t vsa_workspace_bytes(int32_t num_heads, int64_t text_len, int64_t video_len, int64_t audio_len,
                           float topk_frac) {
    Shape s;
    if (make_shape(num_heads, text_len, video_len, audio_len, &s) != VSA_OK) return 0;
    if (check_topk(topk_frac, &s) != VSA_OK) return 0;
    return vsa::make_layout(s).total;
}

vsa_status vsa_workspace_layout(int32_t num_heads, int64_t text_len, int64_t video_len,
                                int64_t audio_len, size_t offsets[7]) {
    if (!offsets) return VSA_ERR_NULL_POINTER;
    Shape s;
    vsa_status st = make_shape(num_heads, text_len, video_len, audio_len, &s);
    if (st != VSA_OK) return st;
    const Layout L = vsa::make_layout(s);
    offsets[0] = L.qbar64;
    offsets[1] = L.kbar;
    offsets[2] = L.vbar;
    offsets[3] = L.coarse;
    offsets[4] = L.kpack;
    offsets[5] = L.vpack;
    offsets[6] = L.total;
    return VSA_OK;
}

vsa_status vsa_pool_pack(const void* q, const void* k, const void* v, int32_t num_heads,
                         int64_t text_len, int64_t video_len, int64_t audio_len, void* workspace,
                         size_t workspace_bytes, void* stream) {
    if (!q || !k || !v) return VSA_ERR_NULL_POINTER;
    Shape s;
    vsa_status st = make_shape(num_heads, text_len, video_len, audio_len, &s);
    if (st != VSA_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16)) return VSA_ERR_MISALIGNED;
    const Layout L = vsa::make_layout(s);
    if ((st = check_workspace(workspace, workspace_bytes, L)) != VSA_OK) return st;
    if ((st = check_device()) != VSA_OK) return st;
    return from_hip(vsa::launch_pool_pack((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                                          s, (uint8_t*)workspace, L, (hipStream_t)stream));
}

vsa_status vsa_select_coarse(int32_t num_heads, int64_t text_len, int64_t video_len,
                             int64_t audio_len, float topk_frac, int32_t* selected_tiles,
                             void* workspace, size_t workspace_bytes, void* stream) {
    if (!selected_tiles) return VSA_ERR_NULL_POINTER;
    Shape s;
    vsa_status st = make_shape(num_heads, text_len, video_len, audio_len, &s);
    if (st != VSA_OK) return st;
    if (s.n_v == 0) return VSA_ERR_BAD_SHAPE;
    if ((st = check_topk(topk_frac, &s)) != VSA_OK) return st;
    if (!aligned(selected_tiles, 16)) return VSA_ERR_MISALIGNED;
    const Layout L = vsa::make_layout(s);
    if ((st = check_workspace(workspace, workspace_bytes, L)) != VSA_OK) return st;
    if ((st = check_device()) != VSA_OK) return st;
    return from_hip(vsa::launch_select_coarse(s, selected_tiles, (uint8_t*)workspace, L,
                                              (hipStream_t)stream));
}

vsa_status vsa_fine_attention(const void* q, const void* gate, int32_t num_heads,
                              int64_t text_len, int64_t video_len, int64_t audio_len,
                              float topk_frac, const int32_t* selected_tiles, void* out,
                              void* workspace, size_t workspace_bytes, void* stream) {
    if (!q || !out) return VSA_ERR_NULL_POINTER;
    if (video_len != 0 && (!gate || !selected_tiles)) return VSA_ERR_NULL_POINTER;
    Shape s;
    vsa_status st = make_shape(num_heads, text_len, video_len, audio_len, &s);
    if (st != VSA_OK) return st;
    if ((st = check_topk(topk_frac, &s)) != VSA_OK) return st;
    if (!aligned(q, 16) || !aligned(out, 16) || (gate && !aligned(gate, 16)) ||
        (selected_tiles && !aligned(selected_tiles, 4)))
        return VSA_ERR_MISALIGNED;
    const Layout L = vsa::make_layout(s);
    if ((st = check_workspace(workspace, workspace_bytes, L)) != VSA_OK) return st;
    if ((st = check_device()) != VSA_OK) return st;
    return from_hip(vsa::launch_fine_attention((const uint16_t*)q, (const uint16_t*)gate,
                                               selected_tiles, (uint16_t*)out, s,
                                               (uint8_t*)workspace, L, (hipStream_t)stream,
                                               /*check_sel=*/true));
}

vsa_status vsa_forward(const void* q, const void* k, const void* v, const void* gate,
                       int32_t num_heads, int64_t text_len, int64_t video_len, int64_t audio_len,
                       float topk_frac, void* out, int32_t* selected_tiles, void* workspace,
                       size_t workspace_bytes, void* stream) {
    if (!q || !k || !v || !out) return VSA_ERR_NULL_POINTER;
    if (video_len != 0 && (!gate || !selected_tiles)) return VSA_ERR_NULL_POINTER;
    Shape s;
    vsa_status st = make_shape(num_heads, text_len, video_len, audio_len, &s);
    if (st != VSA_OK) return st;
    if ((st = check_topk(topk_frac, &s)) != VSA_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        (gate && !aligned(gate, 16)) || (selected_tiles && !aligned(selected_tiles, 16)))
        return VSA_ERR_MISALIGNED;
    const Layout L = vsa::make_layout(s);
    if (workspace) {
        if ((st = check_workspace(workspace, workspace_bytes, L)) != VSA_OK) return st;
    }
    if ((st = check_device()) != VSA_OK) return st;
    if (!workspace) {
        if ((st = owned_workspace(L.total, &workspace)) != VSA_OK) return st;
    }
    hipStream_t strm = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)workspace;
    hipError_t e = vsa::launch_pool_pack((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                                         s, ws, L, strm);
    if (e == hipSuccess && s.n_v > 0) e = vsa::launch_select_coarse(s, selected_tiles, ws, L, strm);
    if (e == hipSuccess)
        e = vsa::launch_fine_attention((const uint16_t*)q, (const uint16_t*)gate,
                                       selected_tiles, (uint16_t*)out, s, ws, L, strm);
    return from_hip(e);
}

vsa_status vsa_forward_noalloc(const void* q, const void* k, const void* v, const void* gate,
                               int32_t num_heads, int64_t text_len, int64_t video_len,
                               int64_t audio_len, float topk_frac, void* out,
                               int32_t* selected_tiles, void* stream) {
    if (!q || !k || !v || !out) return VSA_ERR_NULL_POINTER;
    if (video_len != 0 && (!gate || !selected_tiles)) return VSA_ERR_NULL_POINTER;
    Shape s;
    vsa_status st = make_shape(num_heads, text_len, video_len, audio_len, &s);
    if (st != VSA_OK) return st;
    if ((st = check_topk(topk_frac, &s)) != VSA_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        (gate && !aligned(gate, 16)) || (selected_tiles && !aligned(selected_tiles, 16)))
        return VSA_ERR_MISALIGNED;
    // the largest group of heads whose workspace fits the array (the layout
    // grows with the head count)
    const size_t cap = VSA_NOALLOC_SCRATCH_BYTES;
    Shape g = s;
    g.H = 1;
    if (vsa::make_layout(g).total > cap) return VSA_ERR_TOO_LARGE;
    int32_t lo = 1, hi = s.H;
    while (lo < hi) {
        const int32_t mid = lo + (hi - lo + 1) / 2;
        g.H = mid;
        if (vsa::make_layout(g).total <= cap) lo = mid;
        else hi = mid - 1;
    }
    const int32_t per_group = lo;
    if ((st = check_device()) != VSA_OK) return st;
    void* scratch = nullptr;
    size_t scratch_bytes = 0;
    if (vsa::noalloc_scratch(&scratch, &scratch_bytes) != hipSuccess) return VSA_ERR_HIP;
    if (scratch_bytes < cap) return VSA_ERR_HIP;
    hipStream_t strm = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)scratch;
    hipError_t e = hipSuccess;
    for (int32_t h0 = 0; h0 < s.H && e == hipSuccess; h0 += per_group) {
        // heads h0 .. h0 + c.H - 1, reading and writing the caller's tensors in
        // place: row stride stays the caller's head count
        Shape c = s;
        c.H = s.H - h0 < per_group ? s.H - h0 : per_group;
        c.ldh = s.H;
        const Layout L = vsa::make_layout(c);
        const int64_t hoff = (int64_t)h0 * VSA_HEAD_DIM;
        const uint16_t* qh = (const uint16_t*)q + hoff;
        const uint16_t* kh = (const uint16_t*)k + hoff;
        const uint16_t* vh = (const uint16_t*)v + hoff;
        const uint16_t* gh = gate ? (const uint16_t*)gate + hoff : nullptr;
        uint16_t* oh = (uint16_t*)out + hoff;
        int32_t* selh = selected_tiles ? selected_tiles + (int64_t)h0 * s.n_v * s.k : nullptr;
        e = vsa::launch_pool_pack(qh, kh, vh, c, ws, L, strm);
        if (e == hipSuccess && c.n_v > 0) e = vsa::launch_select_coarse(c, selh, ws, L, strm);
        if (e == hipSuccess) e = vsa::launch_fine_attention(qh, gh, selh, oh, c, ws, L, strm);
    }
    return from_hip(e);
}

vsa_status vsa_forward_padded(const void* q, const void* k, const void* v, const void* gate,
                              const void* gamma_q, const void* gamma_k, const int32_t grid[6],
                              int32_t num_heads, int64_t text_len, int64_t video_len,
                              int64_t audio_len, int64_t text_valid, int64_t video_valid,
                              int64_t audio_valid, float topk_frac, void* q_out, void* out,
                              int32_t* selected_tiles, void* workspace, size_t workspace_bytes,
                              void* stream) {
    if (!q || !k || !v || !out) return VSA_ERR_NULL_POINTER;
    if (video_len != 0 && (!gate || !selected_tiles)) return VSA_ERR_NULL_POINTER;
    const bool prep = gamma_q || gamma_k;
    if (prep && (!gamma_q || !gamma_k || !q_out || !grid)) return VSA_ERR_NULL_POINTER;
    Shape s;
    vsa_status st = make_shape(num_heads, text_len, video_len, audio_len, &s);
    if (st != VSA_OK) return st;
    // each segment: its first `valid` rows are tokens, and only its last tile
    // may hold padding
    const int64_t lens[3] = {text_len, video_len, audio_len};
    const int64_t vals[3] = {text_valid, video_valid, audio_valid};
    for (int i = 0; i < 3; ++i) {
        if (lens[i] == 0 ? vals[i] != 0 : (vals[i] > lens[i] || vals[i] <= lens[i] - VSA_TILE))
            return VSA_ERR_BAD_SHAPE;
    }
    s.V_t = text_valid;
    s.V_v = video_valid;
    s.V_a = audio_valid;
    vsa::Prep pp{};
    if (prep) {
        for (int i = 0; i < 6; ++i)
            if (grid[i] < 1) return VSA_ERR_BAD_SHAPE;
        for (int i = 0; i < 3; ++i)
            if (grid[i] % grid[3 + i]) return VSA_ERR_BAD_SHAPE;
        if ((int64_t)grid[0] * grid[1] * grid[2] != video_valid) return VSA_ERR_BAD_SHAPE;
        pp.gamma_q = (const uint16_t*)gamma_q;
        pp.gamma_k = (const uint16_t*)gamma_k;
        for (int i = 0; i < 3; ++i) {
            pp.grid[i] = grid[i];
            pp.tile[i] = grid[3 + i];
        }
    }
    if ((st = check_topk(topk_frac, &s)) != VSA_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        (gate && !aligned(gate, 16)) || (selected_tiles && !aligned(selected_tiles, 16)) ||
        (prep && (!aligned(q_out, 16) || !aligned(gamma_q, 16) || !aligned(gamma_k, 16))))
        return VSA_ERR_MISALIGNED;
    const Layout L = vsa::make_layout(s);
    if (workspace) {
        if ((st = check_workspace(workspace, workspace_bytes, L)) != VSA_OK) return st;
    }
    if ((st = check_device()) != VSA_OK) return st;
    if (!workspace) {
        if ((st = owned_workspace(L.total, &workspace)) != VSA_OK) return st;
    }
    hipStream_t strm = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)workspace;
    hipError_t e = vsa::launch_pool_pack((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                                         s, ws, L, strm, prep ? &pp : nullptr, (uint16_t*)q_out);
    if (e == hipSuccess && s.n_v > 0) e = vsa::launch_select_coarse(s, selected_tiles, ws, L, strm);
    if (e == hipSuccess)
        e = vsa::launch_fine_attention(prep ? (const uint16_t*)q_out : (const uint16_t*)q,
                                       (const uint16_t*)gate, selected_tiles, (uint16_t*)out, s, ws,
                                       L, strm);
    return from_hip(e);
}

int32_t vsa_subblock_count(int64_t video_len, float sparsity) {
    if (video_len < 0 || video_len % VSA_TILE) return -1;
    return subblock_count(video_len / VSA_TILE, sparsity);
}

size_t vsa_subblock_workspace_bytes(int32_t num_heads, int64_t text_len, int64_t video_len,
                                    int64_t audio_len) {
    Shape s;
    if (make_shape(num_heads, text_len, video_len, audio_len, &s) != VSA_OK) return 0;
    if (s.n_v > vsa::kSubblockMaxTiles) return 0;
    return vsa::make_layout(s, true).total;
}

vsa_status vsa_forward_subblock(const void* q, const void* k, const void* v, int32_t num_heads,
                                int64_t text_len, int64_t video_len, int64_t audio_len,
                                float sparsity, void* out, int32_t* selected_tiles,
                                void* workspace, size_t workspace_bytes, void* stream) {
    if (!q || !k || !v || !out) return VSA_ERR_NULL_POINTER;
    if (video_len != 0 && !selected_tiles) return VSA_ERR_NULL_POINTER;
    Shape s;
    vsa_status st = make_shape(num_heads, text_len, video_len, audio_len, &s);
    if (st != VSA_OK) return st;
    if (s.n_v > vsa::kSubblockMaxTiles) return VSA_ERR_TOO_LARGE;
    const int32_t kk = subblock_count(s.n_v, sparsity);
    if (kk < 0) return VSA_ERR_BAD_TOPK;
    s.k = kk;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        (selected_tiles && !aligned(selected_tiles, 16)))
        return VSA_ERR_MISALIGNED;
    const Layout L = vsa::make_layout(s, true);
    if (workspace) {
        if ((st = check_workspace(workspace, workspace_bytes, L)) != VSA_OK) return st;
    }
    if ((st = check_device()) != VSA_OK) return st;
    if (!workspace) {
        if ((st = owned_workspace(L.total, &workspace)) != VSA_OK) return st;
    }
    hipStream_t strm = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)workspace;
    hipError_t e = vsa::launch_pool_pack((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                                         s, ws, L, strm);
    if (e == hipSuccess)
        e = vsa::launch_subblock_route((const uint16_t*)q, (const uint16_t*)k, s, selected_tiles,
                                       ws, L, strm);
    if (e == hipSuccess)
        e = vsa::launch_fine_attention((const uint16_t*)q, nullptr, selected_tiles,
                                       (uint16_t*)out, s, ws, L, strm);
    return from_hip(e);
}

vsa_status vsa_subblock_select(const void* q, const void* k, int32_t num_heads, int64_t text_len,
                               int64_t video_len, int64_t audio_len, float sparsity,
                               int32_t* selected_tiles, void* workspace, size_t workspace_bytes,
                               void* stream) {
    if (!q || !k || !selected_tiles) return VSA_ERR_NULL_POINTER;
    Shape s;
    vsa_status st = make_shape(num_heads, text_len, video_len, audio_len, &s);
    if (st != VSA_OK) return st;
    if (s.n_v == 0) return VSA_ERR_BAD_SHAPE;
    if (s.n_v > vsa::kSubblockMaxTiles) return VSA_ERR_TOO_LARGE;
    const int32_t kk = subblock_count(s.n_v, sparsity);
    if (kk < 0) return VSA_ERR_BAD_TOPK;
    s.k = kk;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(selected_tiles, 16))
        return VSA_ERR_MISALIGNED;
    const Layout L = vsa::make_layout(s, true);
    if ((st = check_workspace(workspace, workspace_bytes, L)) != VSA_OK) return st;
    if ((st = check_device()) != VSA_OK) return st;
    return from_hip(vsa::launch_subblock_route((const uint16_t*)q, (const uint16_t*)k, s,
                                               selected_tiles, (uint8_t*)workspace, L,
                                               (hipStream_t)stream));
}

size_t vsa_subblock_whole_workspace_bytes(int32_t num_heads, int64_t text_len, int64_t video_len,
                                          int64_t audio_len) {
    Shape w;
    if (whole_shape(num_heads, text_len, video_len, audio_len, 0.5f, &w) != VSA_OK) return 0;
    return vsa::make_layout(w, true, false).total;
}

vsa_status vsa_forward_subblock_whole(const void* q, const void* k, const void* v,
                                      int32_t num_heads, int64_t text_len, int64_t video_len,
                                      int64_t audio_len, float sparsity, void* out,
                                      int32_t* selected_tiles, void* workspace,
                                      size_t workspace_bytes, void* stream) {
    if (!q || !k || !v || !out || !selected_tiles) return VSA_ERR_NULL_POINTER;
    Shape w;
    vsa_status st = whole_shape(num_heads, text_len, video_len, audio_len, sparsity, &w);
    if (st != VSA_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(selected_tiles, 16))
        return VSA_ERR_MISALIGNED;
    const Layout L = vsa::make_layout(w, true, false);
    if (workspace) {
        if ((st = check_workspace(workspace, workspace_bytes, L)) != VSA_OK) return st;
    }
    if ((st = check_device()) != VSA_OK) return st;
    if (!workspace) {
        if ((st = owned_workspace(L.total, &workspace)) != VSA_OK) return st;
    }
    hipStream_t strm = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)workspace;
    hipError_t e = vsa::launch_pool_pack((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                                         w, ws, L, strm, nullptr, nullptr, /*pooled=*/false);
    if (e == hipSuccess)
        e = vsa::launch_subblock_route((const uint16_t*)q, (const uint16_t*)k, w, selected_tiles,
                                       ws, L, strm);
    if (e == hipSuccess)
        e = vsa::launch_fine_attention((const uint16_t*)q, nullptr, selected_tiles,
                                       (uint16_t*)out, w, ws, L, strm);
    return from_hip(e);
}

vsa_status vsa_subblock_select_whole(const void* q, const void* k, int32_t num_heads,
                                     int64_t text_len, int64_t video_len, int64_t audio_len,
                                     float sparsity, int32_t* selected_tiles, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    if (!q || !k || !selected_tiles) return VSA_ERR_NULL_POINTER;
    Shape w;
    vsa_status st = whole_shape(num_heads, text_len, video_len, audio_len, sparsity, &w);
    if (st != VSA_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(selected_tiles, 16))
        return VSA_ERR_MISALIGNED;
    const Layout L = vsa::make_layout(w, true, false);
    if ((st = check_workspace(workspace, workspace_bytes, L)) != VSA_OK) return st;
    if ((st = check_device()) != VSA_OK) return st;
    return from_hip(vsa::launch_subblock_route((const uint16_t*)q, (const uint16_t*)k, w,
                                               selected_tiles, (uint8_t*)workspace, L,
                                               (hipStream_t)stream));
}

vsa_status vsa_project_qkvg(const void* x, const void* w, int64_t tokens, int32_t hidden,
                            int32_t num_heads, void* q, void* k, void* v, void* gate,
                            void* stream) {
    if (!x || !w || !q || !k || !v || !gate) return VSA_ERR_NULL_POINTER;
    if (tokens < 1 || hidden < 64 || num_heads < 2) return VSA_ERR_BAD_SHAPE;
    if (hidden % 64 || num_heads % 2) return VSA_ERR_UNALIGNED_LENGTH;
    if (hidden > 16384 || num_heads > VSA_MAX_HEADS || tokens > VSA_MAX_TOKENS)
        return VSA_ERR_TOO_LARGE;
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(q, 16) || !aligned(k, 16) ||
        !aligned(v, 16) || !aligned(gate, 16))
        return VSA_ERR_MISALIGNED;
    vsa_status st = check_device();
    if (st != VSA_OK) return st;
    uint16_t* const outs[4] = {(uint16_t*)q, (uint16_t*)k, (uint16_t*)v, (uint16_t*)gate};
    return from_hip(vsa::launch_project_qkvg((const uint16_t*)x, (const uint16_t*)w, outs, tokens,
                                             hidden, num_heads * VSA_HEAD_DIM,
                                             (hipStream_t)stream));
}

}  // extern "C"

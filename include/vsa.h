/*
 * vsa.h -- C ABI of the MI355X (gfx950) video sparse attention (VSA) forward.
 *
 * The operation: the page "UniServe: serving FastH3 at its fastest", section
 * "The FastH3 workload", defines VSA over a joint [text | video | audio]
 * token sequence cut into tiles of 64 tokens, with 128-dimensional heads:
 *   - text and audio queries attend to every key;
 *   - a video query attends to every text and audio key and to the keys of
 *     the video tiles its own tile selected: the top 20% (rounded to whole
 *     tiles) by a tile score, chosen exactly (section "Setup");
 *   - a coarse branch attends over mean-pooled tiles and is added to the
 *     fine output through a learned gate (section "Fused output combination",
 *     the combination equation).
 * Section "Fused attention preprocessing" fixes the pooled statistics as
 * FP32 and keeps top-k selection, fine attention and coarse attention as
 * separate steps.  The algebra the page leaves open is fixed as follows:
 *   - tile score s(u,w) = dot(pooled Q of video tile u, pooled K of video
 *     tile w), per head, from the FP32 pooled vectors, accumulated in float64;
 *   - k = floor(topk_frac * n_v + 0.5), clamped to [1, n_v] (0 when n_v = 0);
 *   - ties in the ranking go to the lower tile index;
 *   - the coarse branch: softmax over the video tiles w of s(u,w)/sqrt(128)
 *     applied to the pooled V, one vector per video tile, added to each of
 *     the tile's 64 rows;
 *   - out = O_fine + sigmoid(G) * O_coarse on video rows, out = O_fine on
 *     text and audio rows; softmax scale 1/sqrt(128); fp32 accumulation.
 * The device forms the tile scores on the float32 matrix unit with a proven
 * bound on their error and recomputes the float64 score wherever that bound
 * leaves the ranking open, so the selection is exactly that of the float64
 * scores above; the coarse softmax uses the float32 scores.
 *
 * Layout.  q, k, v, gate and out are bfloat16, token-major [S][H][128]
 * (element (s,h,d) at index (s*H + h)*128 + d), S = text_len + video_len +
 * audio_len, in the order text, video, audio.  Video tile u (0 <= u < n_v)
 * is tokens text_len + 64u .. text_len + 64u + 63.  selected_tiles is int32
 * [H][n_v][k]: for head h and video query tile u, the k selected video tiles
 * as video-local indices (0..n_v-1), ascending.
 *
 * Memory and ownership.  Every tensor pointer is device memory owned by the
 * caller, 16-byte aligned.  The library keeps no pointer after a call
 * returns and frees nothing it was given.  The workspace is caller-owned
 * device memory of at least vsa_workspace_bytes(...) bytes, 256-byte aligned;
 * vsa_forward also accepts workspace == NULL, in which case it uses a
 * grow-only buffer the library owns per device (allocated with hipMalloc on
 * first use and on growth, after a device synchronisation; kept until the
 * process ends).
 *
 * Execution.  Calls are asynchronous: on return the kernels are enqueued on
 * `stream` (a hipStream_t, NULL = the null stream).  Argument errors are
 * returned before any HIP call and leave every output untouched.  A launch
 * failure returns VSA_ERR_HIP; a fault inside a kernel surfaces at the
 * caller's next synchronisation of the stream.  Two calls that run at the
 * same time must use different workspaces (the library-owned workspace is
 * shared by every NULL-workspace call on a device).
 *
 * Limits: num_heads <= VSA_MAX_HEADS, S <= VSA_MAX_TOKENS,
 * n_v <= VSA_MAX_VIDEO_TILES.  Head dimension is fixed at 128.
 */
#ifndef VSA_H
#define VSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VSA_HEAD_DIM 128
#define VSA_TILE 64
#define VSA_MAX_HEADS 1024
#define VSA_MAX_TOKENS (1LL << 24)
#define VSA_MAX_VIDEO_TILES 16384

typedef enum vsa_status {
    VSA_OK = 0,
    VSA_ERR_NULL_POINTER = 1,     /* a required pointer is NULL                         */
    VSA_ERR_BAD_SHAPE = 2,        /* num_heads < 1, a negative length, or S == 0         */
    VSA_ERR_UNALIGNED_LENGTH = 3, /* a length is not a multiple of 64                    */
    VSA_ERR_BAD_TOPK = 4,         /* topk_frac is NaN, <= 0 or > 1                       */
    VSA_ERR_MISALIGNED = 5,       /* a tensor is not 16-byte / workspace not 256-byte aligned */
    VSA_ERR_WORKSPACE = 6,        /* workspace too small (or NULL where one is required) */
    VSA_ERR_DEVICE = 7,           /* the current device is not gfx950                    */
    VSA_ERR_HIP = 8,              /* a HIP runtime call or kernel launch failed          */
    VSA_ERR_TOO_LARGE = 9         /* beyond VSA_MAX_HEADS / _TOKENS / _VIDEO_TILES       */
} vsa_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* vsa_status_string(vsa_status s);

/* Number of selected video tiles per video query tile (section "The FastH3
 * workload": 20% of the video tiles, rounded to whole tiles):
 * k = floor(topk_frac * n_v + 0.5) in double, clamped to [1, n_v];
 * 0 when video_len == 0.  Returns -1 if video_len is negative or not a
 * multiple of 64, or topk_frac is outside (0, 1].  Host only. */
int32_t vsa_topk_count(int64_t video_len, float topk_frac);

/* Workspace bytes needed by vsa_forward and the stage calls below for this
 * shape and top-k fraction; 0 if the shape or topk_frac is invalid (the
 * same checks as vsa_forward).  Host only. */
size_t vsa_workspace_bytes(int32_t num_heads, int64_t text_len, int64_t video_len, int64_t audio_len,
                           float topk_frac);

/* Byte offsets of the workspace regions, for inspection by tests:
 *   offsets[0] pooled Q   float64 [H][n_v][128] (the FP32 statistic, widened)
 *   offsets[1] pooled K   float32 [H][n_v][128]
 *              (in both, dim d = 4 s + g of a row is stored at 32 g + s)
 *   offsets[2] pooled V   float32 [H][128][n_v rounded up to 16] (transposed;
 *              the columns past n_v are zero)
 *   offsets[3] coarse     float32 [H][n_v][128]
 *   offsets[4] packed K   bfloat16, 16 KiB per (head, tile), in MFMA operand order
 *   offsets[5] packed V   bfloat16, 16 KiB per (head, tile), in MFMA operand order
 *   offsets[6] total bytes (= vsa_workspace_bytes).  Between packed V and
 *              the total lie the partial results of text/audio query tiles
 *              whose key list the fine stage splits into parts (float32,
 *              33,280 bytes per part, up to 8 parts per tile; none without
 *              video tiles) and, in the last 1,536 bytes, the fine
 *              stage's twelve work-queue counters, which every call clears
 *              before use
 * Returns VSA_OK or a shape error.  Host only. */
vsa_status vsa_workspace_layout(int32_t num_heads, int64_t text_len, int64_t video_len,
                                int64_t audio_len, size_t offsets[7]);

/* The whole forward pass: pooling and K/V packing, ranking + exact top-k +
 * coarse branch, then fine block-sparse attention with the gated
 * combination.  Writes out [S][H][128] bf16 and selected_tiles
 * [H][n_v][k].  gate and selected_tiles may be NULL only when video_len is
 * 0.  workspace may be NULL (library-owned buffer, see above). */
vsa_status vsa_forward(const void* q, const void* k, const void* v, const void* gate,
                       int32_t num_heads, int64_t text_len, int64_t video_len, int64_t audio_len,
                       float topk_frac, void* out, int32_t* selected_tiles,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Stage 1 (section "Fused attention preprocessing": FP32 tile pooling and
 * tile packing): pooled Q, K, V of every video tile into the workspace, and
 * K and V of every tile packed for the attention stage.  workspace is
 * required. */
vsa_status vsa_pool_pack(const void* q, const void* k, const void* v, int32_t num_heads,
                         int64_t text_len, int64_t video_len, int64_t audio_len,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Stage 2 (section "The FastH3 workload": ranking, exact top-k, coarse
 * branch): reads the pooled statistics of stage 1 from the workspace,
 * writes selected_tiles and the coarse output (workspace).  Requires
 * video_len > 0.  workspace is required. */
vsa_status vsa_select_coarse(int32_t num_heads, int64_t text_len, int64_t video_len,
                             int64_t audio_len, float topk_frac, int32_t* selected_tiles,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Stage 3 (sections "The FastH3 workload" and "Fused output combination"):
 * fine block-sparse attention of every query tile over its key tiles, with
 * the gated coarse term added in the epilogue.  selected_tiles is any
 * [H][n_v][k] array of video tile indices (k from topk_frac) whose rows each
 * hold k distinct indices in [0, n_v), ascending.  Every row is checked on
 * the device before it is used: a row that breaks this (an index out of
 * range, repeated or out of order) is not attended, and the 64 output rows
 * of that (head, video query tile) are written as NaN, so a malformed
 * selection shows as NaN rather than as a plausible result.  The call itself
 * still returns VSA_OK (the rows live on the device); other rows are
 * computed normally.
 * Reads the packed K and V tiles and the coarse output that stages 1 and 2
 * left in the workspace.  workspace is required. */
vsa_status vsa_fine_attention(const void* q, const void* gate, int32_t num_heads,
                              int64_t text_len, int64_t video_len, int64_t audio_len,
                              float topk_frac, const int32_t* selected_tiles, void* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/* The forward pass on padded segments, optionally with the attention
 * preprocessing fused into stage 1 (page "UniServe: serving FastH3 at its
 * fastest", section "Fused attention preprocessing": learned Q/K RMSNorm,
 * partial RoPE and tile pooling over valid tokens in one pass, padding
 * handled inside the kernel).
 *   text_valid, video_valid, audio_valid: the first `valid` rows of each
 *     segment are tokens, the rest padding; only a segment's last tile may be
 *     padded (len - 64 < valid <= len; valid == 0 when len == 0).  Padding
 *     rows are never keys, are left out of the tile means, and output zeros.
 *   gamma_q, gamma_k: bf16 [H][128] learned RMSNorm weights, or both NULL for
 *     no preprocessing (q and k are then used as given; q_out and grid are
 *     ignored).  With them, every token row of q and k becomes
 *       y = bf16(x / sqrt(mean over the head's 128 dims of x^2 + 1e-6) * gamma),
 *     and video tokens then rotate dims 0..95 -- axis a of (t, h, w) owns dims
 *     32a .. 32a+31 as 16 interleaved pairs (2i, 2i+1) -- by the angle
 *     pos_a * 10000^(-i/16), rounded to bf16 again (the RoPE dimension 96 and
 *     the rounding order follow the SGLang Diffusion benchmark page, section
 *     "How SubBlock Sparse Attention Works" and its kernel table).  Text and
 *     audio tokens are not rotated.
 *   grid: {T, H, W, pt, ph, pw}: the valid video tokens are the T x H x W
 *     latent grid points in tile-packed order (tiles of pt x ph x pw points
 *     in raster order, raster order inside a tile); T*H*W == video_valid.
 *   q_out: bf16 [S][H][128], receives the preprocessed q (padding rows zero);
 *     the attention reads it.  The preprocessed k lives only in the
 *     workspace (packed).
 * Everything else as vsa_forward; workspace may be NULL. */
vsa_status vsa_forward_padded(const void* q, const void* k, const void* v, const void* gate,
                              const void* gamma_q, const void* gamma_k, const int32_t grid[6],
                              int32_t num_heads, int64_t text_len, int64_t video_len,
                              int64_t audio_len, int64_t text_valid, int64_t video_valid,
                              int64_t audio_valid, float topk_frac, void* q_out, void* out,
                              int32_t* selected_tiles, void* workspace, size_t workspace_bytes,
                              void* stream);

/* SubBlock router (the SGLang Diffusion benchmark page, section "How
 * SubBlock Sparse Attention Works"): a second rule for choosing each video
 * query tile's video key tiles, fed to the same fine attention.  Every
 * 64-token tile is split into four 16-token sub-blocks; per head, video
 * query tile u and video key tile w,
 *   x_ab = dot(mean Q of sub-block a of u, mean K of sub-block b of w) / sqrt(128)
 *          (means of 16 rows as float32, dots and everything after in float64)
 *   score(u, w) = log sum over the 16 pairs (a, b) of exp(x_ab),
 * which estimates the unnormalised softmax mass of key tile w for query tile
 * u.  The kept count is vsa_subblock_count(video_len, sparsity); ties in the
 * ranking go to the lower tile index.  As for the tile scores, the device
 * computes in float32 with error bounds and recomputes in float64 where the
 * bounds leave the ranking open (float64 exp and log, so scores tied to
 * within their rounding may order differently from a host evaluation).  Text and audio queries attend to every
 * key, video queries to every text and audio key and to their kept video
 * tiles; there is no coarse branch and no gate (out = O_fine).
 *
 * vsa_subblock_count: sparsity is the fraction of video tiles dropped,
 * 0 <= sparsity < 1; the kept count is rounded to whole groups of 8 tiles:
 *   k = 8 * floor((1 - sparsity) * n_v / 8 + 1/2)   (double arithmetic),
 * clamped to [min(8, n_v), n_v]; 0 when video_len == 0.  Returns -1 if
 * video_len is negative or not a multiple of 64, or sparsity is out of range.
 * Host only. */
int32_t vsa_subblock_count(int64_t video_len, float sparsity);

/* Workspace bytes of vsa_forward_subblock; 0 if the shape is invalid or
 * n_v exceeds VSA_SUBBLOCK_MAX_VIDEO_TILES.  Its first vsa_workspace_bytes()
 * bytes are laid out as vsa_workspace_layout() states; the Q sub-block means
 * follow, then the K sub-block means, each float32, 8 KiB per (head, group of
 * 4 video tiles), at the next 256-byte boundaries.  Host only. */
#define VSA_SUBBLOCK_MAX_VIDEO_TILES 5120
size_t vsa_subblock_workspace_bytes(int32_t num_heads, int64_t text_len, int64_t video_len,
                                    int64_t audio_len);

/* The VSA forward with the SubBlock router in place of the tile score and the
 * coarse branch.  q, k, v, out: bf16 [S][H][128] as vsa_forward;
 * selected_tiles: int32 [H][n_v][k], k = vsa_subblock_count(video_len,
 * sparsity), ascending video-local indices (may be NULL only when video_len
 * is 0).  Padding rows are not supported here (every row is a token).
 * n_v <= VSA_SUBBLOCK_MAX_VIDEO_TILES (VSA_ERR_TOO_LARGE otherwise); a bad
 * sparsity returns VSA_ERR_BAD_TOPK.  workspace: NULL (library-owned) or at
 * least vsa_subblock_workspace_bytes(...) bytes, 256-byte aligned.
 * Everything else as vsa_forward. */
vsa_status vsa_forward_subblock(const void* q, const void* k, const void* v, int32_t num_heads,
                                int64_t text_len, int64_t video_len, int64_t audio_len,
                                float sparsity, void* out, int32_t* selected_tiles,
                                void* workspace, size_t workspace_bytes, void* stream);

/* The router stage of vsa_forward_subblock alone: sub-block means of Q and K
 * into the workspace, scores and selection into selected_tiles.  Requires
 * video_len > 0 (VSA_ERR_BAD_SHAPE otherwise) and a caller workspace of
 * vsa_subblock_workspace_bytes(...) bytes.  Other arguments and errors as
 * vsa_forward_subblock. */
vsa_status vsa_subblock_select(const void* q, const void* k, int32_t num_heads, int64_t text_len,
                               int64_t video_len, int64_t audio_len, float sparsity,
                               int32_t* selected_tiles, void* workspace, size_t workspace_bytes,
                               void* stream);

/* The SubBlock router over the whole sequence, the page's own reading
 * (section "How SubBlock Sparse Attention Works": the sequence is divided
 * into 64-token blocks and every query block ranks the key blocks of its row).
 * All N = (text_len + video_len + audio_len) / 64 tiles of [text | video |
 * audio] are query tiles and candidate key tiles alike: the score of the video
 * mode above (log-sum-exp over the 16 piece pairs, piece means FP32, float64
 * after them) ranks every key tile of the sequence for every (head, query
 * tile), the kept count is k = vsa_subblock_count(text_len + video_len +
 * audio_len, sparsity) (the same rounding to whole groups of 8, over N tiles),
 * ties go to the lower tile index, and each query tile attends to the keys of
 * its kept tiles only: nothing is dense, text and audio keys compete like
 * video keys, and there is no coarse term and no gate.
 *   selected_tiles: int32 [H][N][k], global tile indices 0..N-1, ascending.
 * N <= VSA_SUBBLOCK_MAX_VIDEO_TILES (VSA_ERR_TOO_LARGE otherwise).  q, k, v,
 * out: bf16 [S][H][128] as vsa_forward; every row is a token.  workspace:
 * NULL (library-owned) or at least vsa_subblock_whole_workspace_bytes(...)
 * bytes, 256-byte aligned.  Other arguments and errors as vsa_forward. */
size_t vsa_subblock_whole_workspace_bytes(int32_t num_heads, int64_t text_len, int64_t video_len,
                                          int64_t audio_len);
vsa_status vsa_forward_subblock_whole(const void* q, const void* k, const void* v,
                                      int32_t num_heads, int64_t text_len, int64_t video_len,
                                      int64_t audio_len, float sparsity, void* out,
                                      int32_t* selected_tiles, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* The router stage of vsa_forward_subblock_whole alone (piece means of Q and
 * K into the workspace, scores and selection into selected_tiles); a caller
 * workspace of vsa_subblock_whole_workspace_bytes(...) bytes is required. */
vsa_status vsa_subblock_select_whole(const void* q, const void* k, int32_t num_heads,
                                     int64_t text_len, int64_t video_len, int64_t audio_len,
                                     float sparsity, int32_t* selected_tiles, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* The Q, K, V and gate projections that produce this path's inputs (page
 * "UniServe: serving FastH3 at its fastest", section "The FastH3 workload":
 * hidden size 5,376, 56 heads of 128, so each projection maps 5,376 channels
 * to 7,168):
 *   out_p[s][n] = sum_c x[s][c] * w[p][n][c]    for p = 0 (q), 1 (k), 2 (v), 3 (gate)
 * with fp32 accumulation and each result rounded to bf16 (nearest even).
 *   x        bf16 [tokens][hidden], row-major
 *   w        bf16 [4][num_heads * 128][hidden]: the four weight matrices,
 *            each out x in (row n = output channel n)
 *   q, k, v, gate   bf16 [tokens][num_heads][128] outputs, the layout
 *            vsa_forward reads
 * Requirements: tokens >= 1; hidden a multiple of 64 and at most 16384;
 * num_heads even (num_heads * 128 a multiple of 256) and at most
 * VSA_MAX_HEADS; every pointer 16-byte aligned; tokens <= VSA_MAX_TOKENS.
 * No workspace.  Asynchronous on `stream`, like vsa_forward. */
vsa_status vsa_project_qkvg(const void* x, const void* w, int64_t tokens, int32_t hidden,
                            int32_t num_heads, void* q, void* k, void* v, void* gate,
                            void* stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * vsa_forward with the workspace taken from a fixed array inside the library
 * instead of from the caller or from hipMalloc: VSA_NOALLOC_SCRATCH_BYTES of
 * device memory per device, set up on the first call on that device (which
 * looks up its address with hipGetSymbolAddress) and held until the process
 * ends.  The call allocates nothing and issues no memset; the caller still
 * passes q, k, v, gate, out and selected_tiles as for vsa_forward, with the
 * same meaning, layout and checks.
 * Heads are processed in consecutive groups small enough for one group's
 * workspace to fit the array (results are bit-identical to vsa_forward's).
 * A shape whose single head needs more workspace than the array holds is
 * rejected with VSA_ERR_TOO_LARGE, before any HIP call (at the 10 s shape of
 * 1,166 tiles one head needs about 45 MB, so about 5 heads run per group).
 * Every call on a device shares that device's array, and the array keeps the
 * last call's contents (nothing in it needs to start at zero: work-queue
 * counters are cleared by a kernel at each launch).  Calls that overlap in
 * time on one device -- other streams or other host threads -- race on the
 * array and give wrong results: serialise them. */
#define VSA_NOALLOC_SCRATCH_BYTES (256u << 20)
vsa_status vsa_forward_noalloc(const void* q, const void* k, const void* v, const void* gate,
                               int32_t num_heads, int64_t text_len, int64_t video_len,
                               int64_t audio_len, float topk_frac, void* out,
                               int32_t* selected_tiles, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VSA_H */

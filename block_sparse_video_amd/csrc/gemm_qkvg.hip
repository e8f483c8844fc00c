// gemm_qkvg.hip -- the Q/K/V/gate projections of one DiT attention layer on
// gfx950: out_p[s][n] = sum_c X[s][c] * W_p[n][c] for p in {q, k, v, gate},
// bf16 inputs, fp32 accumulation, bf16 (round to nearest even) outputs.
//
// Page "UniServe: serving FastH3 at its fastest", section "The FastH3
// workload": hidden size 5,376 and 56 heads of 128, so each of the four
// projections maps 5,376 channels to 7,168.  W_p is stored out x in (row n
// holds the weights of output channel n), so both operands are read along
// the contracted dimension and out_p is token-major [S][H][128], the layout
// the attention stages read.
//
// Tiling.  One workgroup (8 wavefronts, two per SIMD) computes 256 output
// channels x 256 tokens; wavefront (wf, wt) owns channels 128 wf .. +127 and
// tokens 64 wt .. +63 as 4 x 2 blocks of v_mfma_f32_32x32x16_bf16 (channels
// are the MFMA rows, tokens its columns, so each lane ends with runs of four
// consecutive channels of one token).  The contracted dimension advances 64
// at a time through two 64 KiB LDS stages (double buffering), each holding
// the 256 x 64 slices of W and X; row r's 16-byte chunk c sits at chunk
// c ^ ((r >> 1) & 7) of its 128-byte row, so the 16 rows that one LDS cycle
// serves of an operand read (16 lanes x 16 bytes over 64 banks) fall on
// distinct banks.  Slices are copied with global_load_lds_dwordx4 (8 rows x
// 128 bytes per instruction; each wavefront copies 32 rows of W and 32 of X
// per stage) one stage ahead; one barrier per stage both publishes the next
// stage and frees the current buffer for the stage after it; operands are
// read from LDS one MFMA step ahead of their use, the reads spread between
// the MFMAs.
#include "vsa_internal.h"

namespace vsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) const bf16x8* lds_bf16x8_ptr;

constexpr int kBM = 256;       // channels per workgroup
constexpr int kBT = 256;       // tokens per workgroup
constexpr int kBK = 64;        // contracted slice per stage
constexpr int kStages = 2;     // LDS ring depth
constexpr int kStageBytes = (kBM + kBT) * kBK * 2;  // 32 KiB

struct GemmArgs {
    const uint16_t* x;   // [tokens][hidden]
    const uint16_t* w;   // [4][out][hidden]
    uint16_t* out[4];    // [tokens][out] each
    int64_t tokens;
    int hidden, n_out;   // n_out = heads * 128, a multiple of 256
    int tiles_n;         // n_out / 256 (the channel tiles of one projection)
    int proj;            // the projection this launch computes (0 q, 1 k, 2 v, 3 gate)
};

__device__ __forceinline__ void wait_vm(int n) {
    if (n >= 8) __builtin_amdgcn_s_waitcnt(0x0F78);       // vmcnt(8)
    else if (n >= 4) __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
    else __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0)
    asm volatile("" ::: "memory");
}

// Two 1 KiB direct-to-LDS copies (slot, slot + 1024) from base + voff[0], voff[1].
__device__ __forceinline__ void fetch4(uint32_t slot, const void* base, const uint32_t (&v)[4]) {
    asm volatile(
        "s_mov_b32 m0, %[s]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[v0], %[b]\n\t"
        "s_add_u32 m0, %[s], 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[v1], %[b]\n\t"
        "s_add_u32 m0, %[s], 0x800\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[v2], %[b]\n\t"
        "s_add_u32 m0, %[s], 0xc00\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[v3], %[b]"
        :
        : [s] "s"(slot), [b] "s"(base), [v0] "v"(v[0]), [v1] "v"(v[1]), [v2] "v"(v[2]),
          [v3] "v"(v[3])
        : "memory", "m0", "scc");
}

__device__ __forceinline__ void barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(512) void gemm_qkvg_kernel(GemmArgs a) {
    extern __shared__ __align__(1024) unsigned char smem[];  // 2 stages x 64 KiB
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)smem;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wf = wave & 1, wt = wave >> 1;  // 128 channels x 64 tokens per wave

    // Tile order: workgroups are dealt round-robin to the 8 XCDs; each XCD
    // walks its own share of the tiles channel-tile-major within a band of
    // 4 token tiles, so the tiles running together on one XCD share their
    // W and X slices in its L2.
    const int tiles_t = (int)((a.tokens + kBT - 1) / kBT);
    const int nb = gridDim.x;  // = tiles_t * tiles_n
    const int b = blockIdx.x;
    const int x8 = b & 7, q8 = nb >> 3, r8 = nb & 7;
    const int lin = x8 * q8 + (x8 < r8 ? x8 : r8) + (b >> 3);  // XCD x8: a contiguous range
    constexpr int kBand = 4;
    const int band = lin / (kBand * a.tiles_n);
    const int in_band = lin - band * kBand * a.tiles_n;
    const int band_t = min(kBand, tiles_t - band * kBand);
    const int tn = in_band / band_t;
    const int tt = band * kBand + (in_band - tn * band_t);

    const int proj = a.proj;
    const int n0 = tn * kBM;  // first channel
    const int64_t t0 = (int64_t)tt * kBT;                  // first token
    const int K = a.hidden;
    const uint16_t* wbase = a.w + ((int64_t)proj * a.n_out + n0) * K;
    const uint16_t* xbase = a.x + t0 * K;

    // Per-lane byte offsets of this wave's 4 W-row and 4 X-row copy
    // instructions (32 rows each, 8 per instruction): row 32 wave + 8 i +
    // lane / 8, global chunk (lane % 8) ^ ((row >> 1) & 7).  Token rows past
    // the end read the last token (valid memory; never stored).
    uint32_t wo[4], xo[4];
    {
        const int rl = lane >> 3;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 32 * wave + 8 * i + rl;
            const int ch = (lane & 7) ^ ((r >> 1) & 7);
            wo[i] = (uint32_t)((r * K + 8 * ch) * 2);
            const int64_t tr = t0 + r < a.tokens ? r : (int)(a.tokens - 1 - t0);
            xo[i] = (uint32_t)((tr * K + 8 * ch) * 2);
        }
    }
    // 4 W and 4 X copies of 1 KiB (8 rows of 128 bytes each) for stage buffer `buf`
    auto fetch_w = [&](int buf, int k0) {
        const uint32_t st = lds0 + (uint32_t)buf * kStageBytes;
        fetch4(st + 4096u * wave, wbase + k0, wo);  // W rows 32 wave .. +31
    };
    auto fetch_x = [&](int buf, int k0) {
        const uint32_t st = lds0 + (uint32_t)buf * kStageBytes;
        fetch4(st + 32768u + 4096u * wave, xbase + k0, xo);  // X rows 32 wave .. +31
    };
    auto fetch_stage = [&](int buf, int k0) {
        const uint32_t st = lds0 + (uint32_t)buf * kStageBytes;
        fetch4(st + 4096u * wave, wbase + k0, wo);           // W rows 32 wave .. +31
        fetch4(st + 32768u + 4096u * wave, xbase + k0, xo);  // X rows 32 wave .. +31
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // operand read offsets inside a stage for MFMA step s (0, 1): rows
    // 32 i + lane % 32 of the wave's half, chunk (lane / 32) + 2 s swizzled
    const int orow = lane & 31, ohalf = lane >> 5;
    uint32_t ow[4][4], ox[4][2];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
        const int c = ohalf + 2 * s2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rw = 128 * wf + 32 * i + orow;
            ow[s2][i] = (uint32_t)(rw * 128 + 16 * (c ^ ((rw >> 1) & 7)));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int rx = 64 * wt + 32 * j + orow;
            ox[s2][j] = 32768u + (uint32_t)(rx * 128 + 16 * (c ^ ((rx >> 1) & 7)));
        }
    }
    auto read_ops = [&](bf16x8 (&wa)[4], bf16x8 (&xb)[2], int buf, int s2) {
        const uint32_t st = lds0 + (uint32_t)buf * kStageBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i) wa[i] = *(lds_bf16x8_ptr)(uintptr_t)(st + ow[s2][i]);
#pragma unroll
        for (int j = 0; j < 2; ++j) xb[j] = *(lds_bf16x8_ptr)(uintptr_t)(st + ox[s2][j]);
    };
    // the next step's six operand reads, issued in source order before this
    // step's eight MFMAs, are spread one after each of the first six MFMAs
    // (issued as a burst they queue in the LDS behind the other waves' reads
    // and copies)
    auto interleave = [&]() {
#pragma unroll
        for (int g = 0; g < 6; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    };
    auto mfma_step = [&](const bf16x8 (&wa)[4], const bf16x8 (&xb)[2]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(wa[i], xb[j], acc[i][j]);
    };

    // Ring: stage kt lives in buffer kt % 2.  Each stage: MFMA steps 0..3,
    // each with the next step's operands read beside it; before the last
    // step, one barrier publishes stage kt+1 and frees buffer kt % 2, which
    // then takes stage kt+2.
    const int KT = K / kBK;
    fetch_stage(0, 0);
    if (KT > 1) fetch_stage(1, kBK);
    wait_vm(KT > 1 ? 8 : 0);
    barrier();
    bf16x8 wa0[4], xb0[2], wa1[4], xb1[2];
    read_ops(wa0, xb0, 0, 0);
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        read_ops(wa1, xb1, buf, 1);
        mfma_step(wa0, xb0);
        interleave();
        read_ops(wa0, xb0, buf, 2);
        mfma_step(wa1, xb1);
        interleave();
        read_ops(wa1, xb1, buf, 3);
        mfma_step(wa0, xb0);
        interleave();
        if (kt + 1 < KT) {
            wait_vm(0);
            barrier();
            if (kt + 2 < KT) fetch_w(buf, (kt + 2) * kBK);
        }
        // issued in every stage so that the reads interleave with this step's
        // MFMAs; after the last stage they read the other buffer's stale
        // values, which are never used
        read_ops(wa0, xb0, buf ^ 1, 0);
        mfma_step(wa1, xb1);
        interleave();
        // the X half of stage kt + 2 one step after its W half, so that the
        // copies do not all land in the LDS at once
        if (kt + 2 < KT) fetch_x(buf, (kt + 2) * kBK);
    }
    barrier();  // every wave is done with the ring before it becomes staging

    // ---- epilogue: bf16, staged through LDS as [token][channel], then
    // 16-byte stores along each token's row
    // lane l of block (i, j): token 32 j + l % 32, channels 32 i + 8 q + 4 (l / 32) + r
    unsigned char* stg = smem + wave * 16384;  // 64 tokens x 128 channels x 2 B
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                 acc[i][j][4 * q + 3]};
                const bf16x4 hv = __builtin_convertvector(v, bf16x4);
                const int tok = 32 * j + orow;
                const int ch = 32 * i + 8 * q + 4 * ohalf;          // 4 channels = 8 bytes
                const int chunk = ch >> 3, sub = (ch & 7) * 2;      // 16-byte chunk, byte in it
                *(bf16x4*)(stg + tok * 256 + 16 * (chunk ^ (tok & 15)) + sub) = hv;
            }
    __syncthreads();
    uint16_t* obase = a.out[proj];
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
        const int id = it * 64 + lane;       // 1024 chunks of 16 bytes
        const int tok = id >> 4, chunk = id & 15;
        const int64_t gt = t0 + 64 * wt + tok;
        const uint4 v = *(const uint4*)(stg + tok * 256 + 16 * (chunk ^ (tok & 15)));
        if (gt < a.tokens)
            *(uint4*)(obase + gt * a.n_out + n0 + 128 * wf + 8 * chunk) = v;
    }
}

}  // namespace

hipError_t launch_project_qkvg(const uint16_t* x, const uint16_t* w, uint16_t* const out[4],
                               int64_t tokens, int hidden, int n_out, hipStream_t stream) {
    static std::atomic<size_t> lds_allowed[kMaxDevices];
    hipError_t e = ensure_dynamic_lds((const void*)gemm_qkvg_kernel, lds_allowed,
                                      (size_t)kStages * kStageBytes);
    if (e != hipSuccess) return e;
    GemmArgs a;
    a.x = x;
    a.w = w;
    for (int p = 0; p < 4; ++p) a.out[p] = out[p];
    a.tokens = tokens;
    a.hidden = hidden;
    a.n_out = n_out;
    a.tiles_n = n_out / kBM;
    const int64_t tiles = ((tokens + kBT - 1) / kBT) * a.tiles_n;
    // one launch per projection: its 77 MB of weights (10 s shape) stay in
    // the 256 MB last-level cache while every token band streams past them,
    // where the four projections' 308 MB together did not fit
    for (int p = 0; p < 4; ++p) {
        a.proj = p;
        hipLaunchKernelGGL(gemm_qkvg_kernel, dim3((unsigned)tiles), dim3(512),
                           kStages * kStageBytes, stream, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace vsa

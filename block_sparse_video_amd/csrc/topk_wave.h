// topk_wave.h -- exact top-k of one row of scores by one wavefront:
// order-preserving 32- and 64-bit keys, the k-th largest key by bisection with
// the row held in registers, and the compaction that writes the selected
// indices in ascending order, tied keys taken by lowest index.  Used by both
// tile selection rules (the pooled tile score and the SubBlock router).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vsa {
namespace {

// Order-preserving map of a float64 to uint64 (larger double -> larger key).
// Scores are stored after x + 0.0, which turns -0.0 into +0.0, so equal
// doubles always give equal keys.
__device__ __forceinline__ uint64_t order_key(double x) {
    const uint64_t b = (uint64_t)__double_as_longlong(x);
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// Order-preserving map of a float32 to uint32 (key 0 is never a finite score).
// Consecutive keys are consecutive floats (-0 and +0 apart), so key + 1 is
// the next float up.
__device__ __forceinline__ uint32_t order_key32(float x) {
    const uint32_t b = __float_as_uint(x);
    return (b >> 31) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key32_value(uint32_t key) {
    return __uint_as_float((key >> 31) ? (key & 0x7FFFFFFFu) : ~key);
}
// Smallest key whose float is >= x, and largest whose float is <= x.
__device__ __forceinline__ uint32_t key32_at_or_above(double x) {
    const float f = (float)x + 0.0f;
    return order_key32(f) + ((double)f < x ? 1u : 0u);
}
__device__ __forceinline__ uint32_t key32_at_or_below(double x) {
    const float f = (float)x + 0.0f;
    return order_key32(f) - ((double)f > x ? 1u : 0u);
}

__device__ __forceinline__ uint32_t uniform_key(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}
__device__ __forceinline__ uint64_t uniform_key(uint64_t x) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(x >> 32)) << 32) |
           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
}

// The kk-th largest of the keys a wavefront holds (kk >= 1, at least kk keys
// nonzero; zero keys are absent), by bisection on the key value; `gt`
// returns the number of keys above it.  The search stops at the first probe
// that exactly kk keys reach (about log2 of the row length probes for
// spread-out keys instead of one per key bit); the kk-th largest key is then
// the smallest key at or above that probe.
template <typename Key, int NS>
__device__ __forceinline__ Key kth_largest(const Key (&kv)[NS], uint32_t kk, uint32_t& gt) {
    Key kmin = ~(Key)0, kmax = 0;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        kmax = kv[i] > kmax ? kv[i] : kmax;
        kmin = (kv[i] != 0 && kv[i] < kmin) ? kv[i] : kmin;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const Key a = __shfl_xor(kmin, off), b = __shfl_xor(kmax, off);
        kmin = a < kmin ? a : kmin;
        kmax = b > kmax ? b : kmax;
    }
    // every lane now holds the same range: make it wave-uniform, so that the
    // search below runs on the scalar unit
    kmin = uniform_key(kmin);
    kmax = uniform_key(kmax);
    auto count_ge = [&](Key th) -> uint32_t {
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < NS; ++i) c += (uint32_t)__popcll(__ballot(kv[i] >= th));
        return c;
    };
    // invariant: count_ge(lo) >= kk, and the answer (the largest T with
    // count_ge(T) >= kk, a key value) is in [lo, hi]
    Key lo = kmin, hi = kmax;
    while (lo < hi) {
        const Key mid = lo + (Key)((hi - lo + 1) >> 1);
        const uint32_t c = count_ge(mid);
        if (c >= kk) {
            lo = mid;
            if (c == kk) break;  // the keys >= mid are exactly the kk largest
        } else {
            hi = mid - 1;
        }
    }
    Key t = ~(Key)0;
#pragma unroll
    for (int i = 0; i < NS; ++i) t = (kv[i] >= lo && kv[i] < t) ? kv[i] : t;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const Key a = __shfl_xor(t, off);
        t = a < t ? a : t;
    }
    t = uniform_key(t);
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < NS; ++i) c += (uint32_t)__popcll(__ballot(kv[i] > t));
    gt = c;
    return t;
}

// Exact k-th largest of one row's keys by bisection on the 64-bit key value,
// one wavefront per row, the row's keys held in registers (lane l owns
// columns l, l + 64, ...; NS slots, n_v <= 64 * NS).  count(T) = number of
// keys >= T is taken with one ballot per slot.  Invariant: count(lo) >= k >
// count(hi).  A probe with count exactly k ends the search early (the keys >=
// it are the selection); otherwise lo ends at the k-th largest key.  Returns
// T and sets `need` = k - #(keys > T), the number of keys equal to T to take.
template <int NS>
__device__ __forceinline__ uint64_t kth_key_bisect(const double* row, int n_v, int k, int lane,
                                                   uint32_t& need) {
    uint64_t kv[NS];
    uint64_t kmin = ~0ull, kmax = 0ull;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int w = lane + 64 * i;
        kv[i] = w < n_v ? order_key(row[w]) : 0ull;  // finite scores never map to 0
        if (w < n_v) {
            kmin = kv[i] < kmin ? kv[i] : kmin;
            kmax = kv[i] > kmax ? kv[i] : kmax;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint64_t a = __shfl_xor(kmin, off), b = __shfl_xor(kmax, off);
        kmin = a < kmin ? a : kmin;
        kmax = b > kmax ? b : kmax;
    }
    // every lane now holds the row's min and max; make them wave-uniform
    kmin = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(kmin >> 32)) << 32) |
           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)kmin);
    kmax = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(kmax >> 32)) << 32) |
           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)kmax);
    auto count_ge = [&](uint64_t t) -> uint32_t {
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < NS; ++i) c += (uint32_t)__popcll(__ballot(kv[i] >= t));
        return c;
    };
    uint64_t lo = kmin, hi = kmax + 1;  // count(kmin) = n_v >= k; count(kmax + 1) = 0 < k
    while (hi - lo > 1) {
        const uint64_t mid = lo + ((hi - lo) >> 1);
        const uint32_t c = count_ge(mid);
        if (c >= (uint32_t)k) {
            lo = mid;
            if (c == (uint32_t)k) break;
        } else {
            hi = mid;
        }
    }
    uint32_t gt = 0;
#pragma unroll
    for (int i = 0; i < NS; ++i) gt += (uint32_t)__popcll(__ballot(kv[i] > lo));
    need = (uint32_t)k - gt;
    return lo;
}

// Writes the k selected indices of `row` in ascending order: every key above
// `kth`, and the `need` lowest-index keys equal to it.
__device__ __forceinline__ void emit_topk(const double* row, int n_v, int k, uint64_t kth,
                                          uint32_t need, int lane, int32_t* __restrict__ out) {
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    uint32_t outc = 0, eqseen = 0;
    for (int w0 = 0; w0 < n_v; w0 += 64) {
        const int w = w0 + lane;
        const bool valid = w < n_v;
        const uint64_t key = valid ? order_key(row[w]) : 0ull;
        const bool gt = valid && key > kth;
        const bool eq = valid && key == kth;
        const uint64_t em = __ballot(eq);
        const uint32_t erank = eqseen + (uint32_t)__popcll(em & lt_mask);
        const bool take = gt || (eq && erank < need);
        const uint64_t tm = __ballot(take);
        const uint32_t pos = outc + (uint32_t)__popcll(tm & lt_mask);
        if (take && pos < (uint32_t)k) out[pos] = w;
        outc += (uint32_t)__popcll(tm);
        eqseen += (uint32_t)__popcll(em);
    }
}

}  // namespace
}  // namespace vsa

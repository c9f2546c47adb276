// kd_topk_select.hpp -- producer of the offline teacher cache: per row of a
// [T, V] logit matrix, the K largest logits and their ids.
//
// Page cited: [TH] ai-thai.com/posts/846 (Thai translation of "Efficient
// Knowledge Distillation for LLMs: Offline Top-K Logits and a Fused Chunked KL
// Loss"), section "Offline distillation": the teacher runs once over the data
// and only its top-100 logits per position, with their token ids, are kept.
//
// Order: logits descending, equal logits by increasing id, over the total
// order of the IEEE patterns (-0 below +0, NaN below -inf).  Every element is
// mapped to a 64-bit key, (order-preserving 32-bit key of the value) << 32 |
// ~id, so that all keys of a row are distinct and "the K largest keys" is the
// answer.
//
// One workgroup per row; the row is streamed from HBM about once:
//   1. a 12-bit histogram of the keys of every 16th 128-byte line gives a
//      lower bound L expected to leave a few hundred candidates;
//   2. one pass over the row appends every key >= L to an LDS buffer (for a
//      non-negative bound, whole 16-byte vectors below it are skipped after
//      one integer max);
//   3. if the count is in [K, capacity] the buffer is sorted (bitonic) and the
//      first K are written; otherwise an exact radix select over the full row
//      (8-bit digits of the 64-bit key, one pass per digit) finds a bound
//      whose candidate count fits, and the row is collected again.
#pragma once

#include "kd_common.hpp"

namespace kd {

constexpr int kSelThreads = 256;
constexpr int kSelCap = 2048;    // candidate keys held in LDS
constexpr int kSelBins = 4096;   // sampled histogram over the top 12 key bits
constexpr int kSelMaxK = 1024;

__device__ __forceinline__ uint32_t sel_key(uint32_t u) {
    const bool nan = (u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u;
    const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return nan ? 0u : k;
}

__device__ __forceinline__ float sel_value(uint32_t key) {
    const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
    return __uint_as_float(u);
}

// fp32 bit patterns of the 16 bytes at element index 8 c (bf16) or 4 c (fp32)
template <typename E> struct SelVec;
template <> struct SelVec<bf16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void bits(const u32x4& v, uint32_t (&u)[8]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            u[2 * q] = v[q] << 16;
            u[2 * q + 1] = v[q] & 0xFFFF0000u;
        }
    }
    static __device__ __forceinline__ uint32_t bits1(const void* row, int i) {
        return (uint32_t)reinterpret_cast<const uint16_t*>(row)[i] << 16;
    }
};
template <> struct SelVec<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void bits(const u32x4& v, uint32_t (&u)[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) u[q] = v[q];
    }
    static __device__ __forceinline__ uint32_t bits1(const void* row, int i) {
        return reinterpret_cast<const uint32_t*>(row)[i];
    }
};

// Elements before the row's first 16-byte boundary (rows need only be
// element-aligned).
template <typename E>
__device__ __forceinline__ int sel_head(const void* row, int V) {
    const int h = (int)(((16u - (uint32_t)(reinterpret_cast<uintptr_t>(row) & 15u)) & 15u) / sizeof(E));
    return h < V ? h : V;
}

// Calls f(key32, id) for every element of the row: the unaligned head, 16-byte
// vectors strided over the workgroup, then the scalar tail.
template <typename E, class F>
__device__ __forceinline__ void sel_for_row(const void* row, int V, int tid, F&& f) {
    constexpr int N = SelVec<E>::N;
    const int head = sel_head<E>(row, V);
    for (int i = tid; i < head; i += kSelThreads) f(sel_key(SelVec<E>::bits1(row, i)), i);
    const u32x4* vec = reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(row) + head * (int)sizeof(E));
    const int nv = (V - head) / N;
    constexpr int U = 8;   // 16-byte loads in flight per thread
    int c = tid;
    for (; c + (U - 1) * kSelThreads < nv; c += U * kSelThreads) {
        u32x4 v[U];
#pragma unroll
        for (int w = 0; w < U; ++w) v[w] = vec[c + w * kSelThreads];
#pragma unroll
        for (int w = 0; w < U; ++w) {
            uint32_t u[N];
            SelVec<E>::bits(v[w], u);
#pragma unroll
            for (int e = 0; e < N; ++e) f(sel_key(u[e]), head + (c + w * kSelThreads) * N + e);
        }
    }
    for (; c < nv; c += kSelThreads) {
        uint32_t u[N];
        SelVec<E>::bits(vec[c], u);
#pragma unroll
        for (int e = 0; e < N; ++e) f(sel_key(u[e]), head + c * N + e);
    }
    for (int i = head + nv * N + tid; i < V; i += kSelThreads) f(sel_key(SelVec<E>::bits1(row, i)), i);
}

// Prefilter of the collection pass for bounds L >= 2^63 (a non-negative
// value): an element can have a key >= L only if it is non-negative and its
// bit pattern, read as a signed integer of the element's width, is at least
// the pattern of the bound's top 32 key bits -- for non-negative values the
// signed order of the patterns is the value order, negative values read as
// negative integers.  A 16-byte vector whose largest such integer is below
// that threshold holds no candidate; any other vector goes through the exact
// per-element key test (which also rejects a NaN that passed the filter).
template <typename E> struct SelFilter;
template <> struct SelFilter<bf16_t> {
    typedef __attribute__((ext_vector_type(2))) short s16x2;
    static __device__ __forceinline__ s16x2 halves(uint32_t w) { return __builtin_bit_cast(s16x2, w); }
    static __device__ __forceinline__ int vmax(const u32x4& v) {
        // scalar copies first: bit-casting the vector elements in place
        // compiles to one register read for all four
        const uint32_t w0 = v[0], w1 = v[1], w2 = v[2], w3 = v[3];
        const s16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(halves(w0), halves(w1)),
                                                  __builtin_elementwise_max(halves(w2), halves(w3)));
        return m[0] > m[1] ? (int)m[0] : (int)m[1];
    }
    static __device__ __forceinline__ int threshold(uint32_t key32) { return (int)((key32 & 0x7FFFFFFFu) >> 16); }
};
template <> struct SelFilter<float> {
    static __device__ __forceinline__ int vmax(const u32x4& v) {
        return max(max((int)v[0], (int)v[1]), max((int)v[2], (int)v[3]));
    }
    static __device__ __forceinline__ int threshold(uint32_t key32) { return (int)(key32 & 0x7FFFFFFFu); }
};

// sel_for_row restricted to the vectors that pass the prefilter (threshold
// thr); the head and tail elements are always visited.
template <typename E, class F>
__device__ __forceinline__ void sel_for_row_filtered(const void* row, int V, int tid, int thr, F&& f) {
    constexpr int N = SelVec<E>::N;
    const int head = sel_head<E>(row, V);
    for (int i = tid; i < head; i += kSelThreads) f(sel_key(SelVec<E>::bits1(row, i)), i);
    const u32x4* vec = reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(row) + head * (int)sizeof(E));
    const int nv = (V - head) / N;
    auto visit = [&](const u32x4& v, int c) {
        if (SelFilter<E>::vmax(v) < thr) return;
        uint32_t u[N];
        SelVec<E>::bits(v, u);
#pragma unroll
        for (int e = 0; e < N; ++e) f(sel_key(u[e]), head + c * N + e);
    };
    constexpr int U = 8;   // 16-byte loads in flight per thread
    int c = tid;
    for (; c + (U - 1) * kSelThreads < nv; c += U * kSelThreads) {
        u32x4 v[U];
#pragma unroll
        for (int w = 0; w < U; ++w) v[w] = vec[c + w * kSelThreads];
#pragma unroll
        for (int w = 0; w < U; ++w) visit(v[w], c + w * kSelThreads);
    }
    for (; c < nv; c += kSelThreads) visit(vec[c], c);
    for (int i = head + nv * N + tid; i < V; i += kSelThreads) f(sel_key(SelVec<E>::bits1(row, i)), i);
}

__device__ __forceinline__ uint64_t sel_full(uint32_t key, int id) {
    return ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)id);
}

// Steps 3'-4, shared by both select kernels: with n candidates collected (all
// keys >= some bound, capped at kSelCap), an exact radix select over the full
// row when n is outside [K, kSelCap], then the bitonic sort and the output.
template <typename E>
__device__ __forceinline__ void sel_finish(const char* row, int V, int K, int64_t t, int tid, uint32_t n, uint64_t* cand,
                           uint32_t* hist, uint32_t* part, uint32_t* count, int32_t* out_idx, float* out_val) {
    auto collect = [&](uint64_t L) {
        auto take = [&](uint32_t key, int id) {
            const uint64_t k = sel_full(key, id);
            if (k >= L) {
                const uint32_t pos = atomicAdd(count, 1u);
                if (pos < (uint32_t)kSelCap) cand[pos] = k;
            }
        };
        if (L >> 63) sel_for_row_filtered<E>(row, V, tid, SelFilter<E>::threshold((uint32_t)(L >> 32)), take);
        else         sel_for_row<E>(row, V, tid, take);
        __syncthreads();
    };
    if (n < (uint32_t)K || n > (uint32_t)kSelCap) {
        // exact: radix select over the 64-bit keys of the full row
        uint64_t P = 0;
        uint32_t above = 0;
        int nb = 0;
        __syncthreads();
        while (true) {
            for (int b = tid; b < 256; b += kSelThreads) hist[b] = 0u;
            __syncthreads();
            const int sh = 56 - nb;
            sel_for_row<E>(row, V, tid, [&](uint32_t key, int id) {
                const uint64_t k = sel_full(key, id);
                if (nb == 0 || (k >> (64 - nb)) == P) atomicAdd(&hist[(k >> sh) & 0xFFu], 1u);
            });
            __syncthreads();
            if (tid == 0) {
                uint32_t acc = above;
                int v = 0;
                for (int d = 255; d >= 0; --d) {
                    if (acc + hist[d] >= (uint32_t)K) { v = d; break; }
                    acc += hist[d];
                }
                part[0] = (uint32_t)v;
                part[1] = acc;
                part[2] = acc + hist[v];
            }
            __syncthreads();
            const uint32_t v = part[0];
            above = part[1];
            const uint32_t cnt = part[2];
            P = (P << 8) | v;
            nb += 8;
            __syncthreads();
            if (cnt <= (uint32_t)kSelCap || nb == 64) break;
        }
        if (tid == 0) *count = 0u;
        __syncthreads();
        collect(nb == 64 ? P : (P << (64 - nb)));
        n = *count;
    }

    // bitonic sort of the candidates, descending (padding keys 0 sort last)
    int n2 = 1;
    while (n2 < (int)n) n2 <<= 1;
    for (int i = (int)n + tid; i < n2; i += kSelThreads) cand[i] = 0ull;
    __syncthreads();
    for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < n2 / 2; i += kSelThreads) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const uint64_t a = cand[lo], b = cand[hi];
                if ((a < b) == desc) {
                    cand[lo] = b;
                    cand[hi] = a;
                }
            }
            __syncthreads();
        }
    }
    for (int k = tid; k < K; k += kSelThreads) {
        const uint64_t c = cand[k];
        out_idx[t * K + k] = (int32_t)(~(uint32_t)c);
        out_val[t * K + k] = sel_value((uint32_t)(c >> 32));
    }
}

template <typename E>
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(const void* logits, int64_t ld, int V, int K,
                                                                  int32_t* out_idx, float* out_val) {
    // the histogram is dead once a bound is known and the candidates are dead
    // while an exact pass histograms: one buffer serves both
    __shared__ uint64_t buf[kSelCap];
    static_assert(kSelBins * 4 <= kSelCap * 8, "histogram fits the candidate buffer");
    uint64_t* cand = buf;
    uint32_t* hist = reinterpret_cast<uint32_t*>(buf);
    __shared__ uint32_t part[kSelThreads];
    __shared__ uint32_t count;
    __shared__ uint64_t bound;
    const int t = (int)blockIdx.x;
    const int tid = (int)threadIdx.x;
    const char* row = reinterpret_cast<const char*>(logits) + (int64_t)t * ld * (int64_t)sizeof(E);
    constexpr int N = SelVec<E>::N;

    // 1. sampled histogram: every 16th 128-byte line (128 / 16 = 8 vectors per line)
    for (int b = tid; b < kSelBins; b += kSelThreads) hist[b] = 0u;
    __syncthreads();
    {
        const int head = sel_head<E>(row, V);
        const u32x4* vec = reinterpret_cast<const u32x4*>(row + head * (int)sizeof(E));
        const int nv = (V - head) / N;
        // sampled vector s is vector 128 (s / 8) + s % 8; four in flight per thread
        for (int s0 = tid;; s0 += 4 * kSelThreads) {
            if (128 * (s0 >> 3) + (s0 & 7) >= nv) break;
            u32x4 v[4];
            bool ok[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int s = s0 + w * kSelThreads;
                const int c = 128 * (s >> 3) + (s & 7);
                ok[w] = c < nv;
                v[w] = ok[w] ? vec[c] : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                if (!ok[w]) continue;
                uint32_t u[N];
                SelVec<E>::bits(v[w], u);
#pragma unroll
                for (int e = 0; e < N; ++e) atomicAdd(&hist[sel_key(u[e]) >> 20], 1u);
            }
        }
    }
    __syncthreads();
    // bin b*: the highest bin whose suffix count reaches m = ceil(K / 16) + 8
    {
        const uint32_t m = (uint32_t)((K + 15) / 16 + 8);
        constexpr int PER = kSelBins / kSelThreads;   // 16 bins per thread, thread 255 the highest
        uint32_t local = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) local += hist[tid * PER + i];
        part[tid] = local;
        if (tid == 0) bound = 0;
        __syncthreads();
        if (tid == 0) {
            uint32_t acc = 0;
            int b = -1;
            for (int w = kSelThreads - 1; w >= 0 && b < 0; --w) {
                if (acc + part[w] >= m) {
                    for (int i = PER - 1; i >= 0; --i) {
                        acc += hist[w * PER + i];
                        if (acc >= m) { b = w * PER + i; break; }
                    }
                } else {
                    acc += part[w];
                }
            }
            bound = b > 0 ? ((uint64_t)b << 52) : 0ull;
            count = 0u;
        }
        __syncthreads();
    }

    // 2. collect every key >= bound
    {
        const uint64_t L = bound;
        auto take = [&](uint32_t key, int id) {
            const uint64_t k = sel_full(key, id);
            if (k >= L) {
                const uint32_t pos = atomicAdd(&count, 1u);
                if (pos < (uint32_t)kSelCap) cand[pos] = k;
            }
        };
        if (L >> 63) sel_for_row_filtered<E>(row, V, tid, SelFilter<E>::threshold((uint32_t)(L >> 32)), take);
        else         sel_for_row<E>(row, V, tid, take);
        __syncthreads();
    }
    // 3, 4
    sel_finish<E>(row, V, K, t, tid, count, cand, hist, part, &count, out_idx, out_val);
}

// ---------------------------------------------------------------------------
// Select over fp32 rows that come with a record of every block of kSelBlock
// consecutive values: bmax[t][b] is never below the largest order key of the
// block (written by the producing logits contraction; blocks beyond V hold 0).
// Bound: the lowest key of the 12-bit key bin in which the records, counted
// from the top, reach K.  Every element with a key >= that bound sits in a
// block whose record is >= it, so only those blocks are read (for a row of
// Gaussian-like logits a few hundred of ceil(V / 128)), and every key >= the
// bound in them is collected.  When each such record is exactly its block's
// largest key (the usual case) there are at least K such keys; otherwise, or
// when ties push the count beyond the buffer, the shared finish runs the exact
// full-row select.  Requires nblk <= kSelMaxBlocks.
// ---------------------------------------------------------------------------
constexpr int kSelBlock = 128;
constexpr int kSelMaxBlocks = 2048;

__global__ __launch_bounds__(kSelThreads) void topk_select_blocks_kernel(const float* logits, int64_t ld, int V,
                                                                         int K, const uint32_t* bmax, int nblk,
                                                                         int32_t* out_idx, float* out_val) {
    __shared__ uint64_t cand[kSelCap];
    static_assert(kSelBins * 4 <= kSelCap * 8, "histogram fits the candidate buffer");
    __shared__ uint32_t bk[kSelMaxBlocks];     // block records
    __shared__ uint32_t part[kSelThreads];
    __shared__ uint32_t count, bin;
    uint32_t* hist = reinterpret_cast<uint32_t*>(cand);
    const int t = (int)blockIdx.x;
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const float* row = logits + (int64_t)t * ld;

    // 1. the records and their 12-bit histogram
    for (int b = tid; b < kSelBins; b += kSelThreads) hist[b] = 0u;
    __syncthreads();
    for (int b = tid; b < nblk; b += kSelThreads) {
        const uint32_t k = bmax[(int64_t)t * nblk + b];
        bk[b] = k;
        atomicAdd(&hist[k >> 20], 1u);
    }
    __syncthreads();
    // 2. the highest bin whose suffix count reaches K
    {
        constexpr int PER = kSelBins / kSelThreads;   // 16 bins per thread, thread 255 the highest
        uint32_t local = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) local += hist[tid * PER + i];
        part[tid] = local;
        __syncthreads();
        if (tid == 0) {
            uint32_t acc = 0;
            int bb = 0;
            bool found = false;
            for (int w = kSelThreads - 1; w >= 0 && !found; --w) {
                if (acc + part[w] >= (uint32_t)K) {
                    for (int i = PER - 1; i >= 0; --i) {
                        acc += hist[w * PER + i];
                        if (acc >= (uint32_t)K) { bb = w * PER + i; found = true; break; }
                    }
                } else {
                    acc += part[w];
                }
            }
            bin = (uint32_t)bb;
            count = 0u;
        }
        __syncthreads();
    }
    const uint32_t B = bin << 20;
    // 3. the blocks whose record is >= B, listed in bk (each thread first takes
    // its own records into registers, so the list can overwrite them)
    constexpr int RPT = kSelMaxBlocks / kSelThreads;
    uint32_t rec[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int b = tid + i * kSelThreads;
        rec[i] = b < nblk ? bk[b] : 0u;
    }
    if (tid == 0) part[0] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int b = tid + i * kSelThreads;
        if (b < nblk && rec[i] >= B) bk[atomicAdd(&part[0], 1u)] = (uint32_t)b;
    }
    __syncthreads();
    const int nq = (int)part[0];
    // every key >= B of the listed blocks: one half-wave per block, 16 bytes a
    // lane, four blocks in flight
    const uint64_t L = (uint64_t)B << 32;
    const int hw = 2 * wave + (lane >> 5), hl = lane & 31;
    constexpr int NHW = 2 * (kSelThreads / 64);
    constexpr int U = 4;
    for (int q0 = hw; q0 < nq; q0 += NHW * U) {
        u32x4 v[U];
        int id0[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = q0 + u * NHW;
            id0[u] = q < nq ? (int)bk[q] * kSelBlock + 4 * hl : V;
            if (id0[u] + 3 < V) {
                v[u] = *reinterpret_cast<const u32x4*>(row + id0[u]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[u][e] = id0[u] + e < V ? __float_as_uint(row[id0[u] + e]) : 0x7FC00000u;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint64_t k = sel_full(sel_key(v[u][e]), id0[u] + e);
                if (id0[u] + e < V && k >= L) {
                    const uint32_t pos = atomicAdd(&count, 1u);
                    if (pos < (uint32_t)kSelCap) cand[pos] = k;
                }
            }
    }
    __syncthreads();
    // 4. sort, or the exact full-row select
    sel_finish<float>(reinterpret_cast<const char*>(row), V, K, t, tid, count, cand, hist, part, &count, out_idx,
                      out_val);
}

}  // namespace kd

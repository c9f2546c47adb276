// kd_kernels.hpp -- epilogues of the three contractions and the per-row
// kernels of the fused chunked top-K KL loss.
//
// Pages cited: [TH] ai-thai.com/posts/846 (Thai translation of "Efficient
// Knowledge Distillation for LLMs: Offline Top-K Logits and a Fused Chunked KL
// Loss"), section "Fused Chunked KL Loss", items "Dense KL" and "Fused chunked
// KL"; [TA] scitechpulse.com/ta (Tamil report on the same post), closing
// paragraph (the backward recomputes each slice, doubling projection work).
//
// Notation: a = z / tau are the student logits of one chunk row over the full
// vocabulary; everything inside a chunk is carried in base 2, y = a * log2(e),
// so that the hardware exp2/log2 apply directly.  lse values handed across
// the boundary are natural-log.
#pragma once

#include "kd_gemm_dtl.hpp"
#include "kd_topk_select.hpp"

namespace kd {

enum LogitsMode { kStats = 0, kFused = 1, kBwd = 2 };

// Per-call scalars kept at the head of the workspace.
struct WsHeader {
    double loss_acc;   // running sum of row losses (fixed chunk order)
    int64_t N;         // number of kept positions
    float s;           // g / (tau N), 0 when N = 0
    int dirty;         // fused entry: rows of the current chunk that need rescaling
    float pad[10];
};
static_assert(sizeof(WsHeader) <= 256, "header slot");

// Layout of a chunk's G (and of the softmax numerators it is built from).
// bf16: blocked by 64 vocabulary ids -- element (r, v) at ((v / 64) C + r) 64 +
// v % 64 -- so that a gradient-GEMM K step (64 ids of 256 consecutive rows, or
// 64 rows of 256 ids) reads contiguous 128-byte rows instead of rows 400 KB
// apart.  fp32 (the small-problem engine): row-major [C][V_pad].
constexpr int kGBlock = 64;
template <typename E> struct GLayout {
    static constexpr bool kBlocked = Elem<E>::size == 2;
    static __device__ __forceinline__ int64_t index(int64_t r, int64_t v, int64_t C, int64_t V_pad) {
        if constexpr (kBlocked) return ((v >> 6) * C + r) * kGBlock + (v & (kGBlock - 1));
        else return r * V_pad + v;
    }
};

// ---------------------------------------------------------------------------
// Logit-tile epilogue: the tile is Z^T (rows = vocabulary ids v, columns =
// chunk rows t).  Each wave reduces its own 128 ids of a column to a partial
// (reference R, sum of 2^(y - R)) in base 2, so a 256-id tile leaves two
// partials per row and no wave waits for another -- the online logsumexp of
// [TH] "Fused chunked KL" is this blocked reduction plus a merge in the row
// kernel.  R is the row's R0 (from the row kernel's first pass) unless the
// block's max lies more than kRefSlack above it.
//   kStats: write the partials only (forward).
//   kFused: also write e = 2^(y - R) as the MFMA operand of the gradient GEMMs
//           (G = one factor per row times e; see the row kernel).
//   kBwd  : lse is known: write the dense part of G, s * exp(a - lse), directly.
constexpr int kStatIds = 128;   // vocabulary ids per partial
// ---------------------------------------------------------------------------
struct LogitsParams {
    f32x2* stats;          // [C][nst] (max2, sum) per (row, 128-id block)
    void* E;               // C x V_pad, GLayout<E>, element type of the operands
    int V, V_pad, nst, rows, C;
    float scale2;          // log2(e) / tau
    const float* lse;      // kBwd: natural-log lse of the chunk rows
    const uint8_t* ignore; // kBwd: ignore flags of the chunk rows (may be null)
    const WsHeader* hdr;   // kBwd: s
    const float* ref;      // kStats / kFused: per-row base-2 reference R0 (of the sums and stored exponentials)
};

// kFused: a block whose max exceeds the row's reference R0 by more than this
// (base 2) stores its exponentials relative to its own max instead, so every
// stored value is at most 2^kRefSlack and no row can overflow.
constexpr float kRefSlack = 64.f;

// bf16 logit tiles leave through LDS so that every global store writes whole
// 512-byte rows: the MFMA layout gives a lane four consecutive vocabulary ids
// of one chunk row, i.e. 8-byte pieces scattered over 32 rows per store.
// Staging layout: [t][256] bf16, 16-byte chunk c of row t at c ^ (t & 31).
__device__ __forceinline__ int stage_off(int t, int chunk) { return t * 512 + ((chunk ^ (t & 31)) << 4); }

template <class Mma>
__device__ __forceinline__ void stage_write4(lds_t* st, int wm, int wn, int i, int j, int q, int lane, float x0,
                                             float x1, float x2, float x3) {
    const int t = Mma::col(wn, j, lane);
    const int v = Mma::row(wm, i, q, lane);   // multiple of 4
    const u32x2 w = {pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
    *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(st + stage_off(t, v >> 3) + ((v & 4) << 1)) = w;
}

// Writes the staged 256 x 256 tile into the blocked bf16 G layout (C rows per
// 64-id block): rows t < rows, columns v0 .. v0 + 255; every 8 lanes write one
// whole 128-byte row segment of a block.
__device__ __forceinline__ void stage_flush(const lds_t* st, uint16_t* dst, int64_t C, int n0, int v0, int rows,
                                            int tid) {
    const int wave = tid >> 6, lane = tid & 63;
    const int c = lane & 31;
    const int64_t blk = (int64_t)(v0 / kGBlock + (c >> 3)) * C;
    constexpr int RW = 256 / kDtlWaves;   // staged rows per wave
#pragma unroll 4
    for (int k = 0; k < RW / 2; ++k) {
        const int tl = wave * RW + 2 * k + (lane >> 5);
        const u32x4 val = lds_read16(st, stage_off(tl, c));
        const int t = n0 + tl;
        if (t < rows) *reinterpret_cast<u32x4*>(dst + (blk + t) * kGBlock + (c & 7) * 8) = val;
    }
}

template <typename E, int BM, int BN, int MODE> struct LogitsEpi {
    using Params = LogitsParams;
    static constexpr bool kStaged = Elem<E>::size == 2;   // bf16 engine: 128 KiB of stage LDS to reuse
    static_assert(BM == 2 * kStatIds, "one partial per wave half of the tile");

    static __device__ __forceinline__ void store4(const Params& p, int t, int v0, float x0, float x1,
                                                  float x2, float x3) {
        if constexpr (Elem<E>::size == 2) {
            u32x2 w = {pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
            *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.E) + GLayout<E>::index(t, v0, p.C, p.V_pad)) = w;
        } else {
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.E) + GLayout<E>::index(t, v0, p.C, p.V_pad)) =
                f32x4{x0, x1, x2, x3};
        }
    }

    // The accumulators hold raw logits z; base-2 values are y = z * scale2
    // (scale2 = log2(e) / tau > 0), formed inside the exponent with one fma.
    // Ids at or beyond V (the padding of the last vocabulary tile only) are
    // excluded as -inf.  The values are computed in place in the accumulators;
    // the staged path synchronises the workgroup only before its first LDS
    // write (other waves may still be reading their last fragments).
    template <class Mma>
    static __device__ __forceinline__ void apply(Mma& mma, int m0, int n0, int /*split*/, int wm, int wn,
                                                 int lane, int tid, lds_t* smem, const Params& p) {
        constexpr int FM = Mma::FM, FN = Mma::FN;
        const float sc = p.scale2;
        // per-column inputs, all requested before any of them is needed
        float colv[FN];
        bool kept[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int t = n0 + Mma::col(wn, j, lane);
            const bool live = t < p.rows;
            if constexpr (MODE == kBwd) {
                colv[j] = live ? p.lse[t] : 0.f;
                kept[j] = live && ((p.ignore == nullptr) || (p.ignore[t] == 0));
            } else {
                colv[j] = live ? p.ref[t] : -INFINITY;
            }
        }
        if (m0 + BM > p.V) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int v0 = m0 + Mma::row(wm, i, q, lane);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bool ok = v0 + r < p.V;
#pragma unroll
                        for (int j = 0; j < FN; ++j)
                            mma.acc[i][j][4 * q + r] = ok ? mma.acc[i][j][4 * q + r] : -INFINITY;
                    }
                }
        }

        if constexpr (MODE == kBwd) {
            const float s = p.hdr->s;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                // ignored (and padding) rows: exactly 0, whatever their lse
                const float l2 = kept[j] ? colv[j] * kLog2e : INFINITY;
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        mma.acc[i][j][e] = s * fast_exp2(fmaf(mma.acc[i][j][e], sc, -l2));
            }
        } else {
            // this wave's 128 ids of each of its columns (lanes l and l + 32
            // hold the same column): max, then exp2 relative to a reference and
            // the sum.  scale2 > 0, so the max of y is the scaled max of z.
            // The reference is the row's R0 (the largest student logit at its
            // cached ids), unless the block max exceeds it by more than
            // kRefSlack -- then the block max; the forward and fused entries
            // thus produce identical statistics.
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                float mz = -INFINITY;
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int e = 0; e < 16; ++e) mz = fmaxf(mz, mma.acc[i][j][e]);
                mz = halves_max(mz);
                const int t = n0 + Mma::col(wn, j, lane);
                float my = mz * sc;
                my = my <= colv[j] + kRefSlack ? colv[j] : my;
                // every id of the block beyond V (kStats) or no reference: all
                // terms are exp2(-inf) = 0
                const float off = my == -INFINITY ? 0.f : my;
                float sum = 0.f;
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const float x = fast_exp2(fmaf(mma.acc[i][j][e], sc, -off));
                        mma.acc[i][j][e] = x;
                        sum += x;
                    }
                sum = halves_sum(sum);
                if (lane < 32 && t < p.rows)
                    p.stats[(int64_t)t * p.nst + (m0 / BM) * 2 + wm] = f32x2{my, sum};
            }
        }
        if constexpr (MODE != kStats) {
            if constexpr (kStaged) {
                __syncthreads();   // every wave is past its main loop: the stage LDS is free
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            stage_write4<Mma>(smem, wm, wn, i, j, q, lane, mma.acc[i][j][4 * q],
                                              mma.acc[i][j][4 * q + 1], mma.acc[i][j][4 * q + 2],
                                              mma.acc[i][j][4 * q + 3]);
                __syncthreads();
                stage_flush(smem, reinterpret_cast<uint16_t*>(p.E), p.C, n0, m0, p.rows, tid);
            } else {
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int t = n0 + Mma::col(wn, j, lane);
                    if (t >= p.rows) continue;
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            store4(p, t, m0 + Mma::row(wm, i, q, lane), mma.acc[i][j][4 * q],
                                   mma.acc[i][j][4 * q + 1], mma.acc[i][j][4 * q + 2], mma.acc[i][j][4 * q + 3]);
                }
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Raw logit epilogue (teacher cache producer): the tile Z^T (rows = vocabulary
// ids v, columns = chunk rows t) is stored as fp32 into out[t * ld + v] for
// v < V and t < rows; ld is a multiple of 4 and out 16-byte aligned.
// ---------------------------------------------------------------------------
struct RawLogitsParams {
    float* out;
    int64_t ld;
    int V, rows;
    uint32_t* bmax;   // optional (bf16 engine) [rows][nblk]: a record never below the largest select order key
                      // of each 128-id block (0 for blocks beyond V)
    int nblk;
};

// True when the wave half wm of the 256-id tile at m0 holds no id below V.
__device__ __forceinline__ bool v0_all_padding(int m0, int wm, int V) { return m0 + 128 * wm >= V; }

template <typename E, int BM, int BN> struct RawLogitsEpi {
    using Params = RawLogitsParams;
    static constexpr bool kStaged = Elem<E>::size == 2;   // bf16 engine: stage LDS free for the epilogue

    template <class Mma>
    static __device__ __forceinline__ void apply(Mma& mma, int m0, int n0, int, int wm, int wn, int lane, int tid,
                                                 lds_t* smem, const Params& p) {
        constexpr int FM = Mma::FM, FN = Mma::FN;
        static_assert(BM == 2 * kSelBlock, "one 128-id block per wave half of the tile");
        if (kStaged && p.bmax) {
            // this wave's 128 ids of each of its chunk rows: the select order
            // key of their largest value (a float max; a zero is recorded as
            // +0 and a block of NaNs as the lowest key, so the record is never
            // below the block's largest key; ids at or beyond V are left out)
            const int blk = (m0 / BM) * 2 + wm;
            const bool tail = m0 + BM > p.V;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                float mv = -INFINITY;
                if (!tail) {
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int e = 0; e < 16; ++e) mv = fmaxf(mv, mma.acc[i][j][e]);
                } else {
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int v0 = m0 + Mma::row(wm, i, q, lane);
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (v0 + r < p.V) mv = fmaxf(mv, mma.acc[i][j][4 * q + r]);
                        }
                }
                mv = halves_max(mv);
                const uint32_t key = mv == 0.f ? sel_key(0u) : sel_key(__float_as_uint(mv));
                const int t = n0 + Mma::col(wn, j, lane);
                if (lane < 32 && t < p.rows) p.bmax[(int64_t)t * p.nblk + blk] = (v0_all_padding(m0, wm, p.V) ? 0u : key);
            }
        }
        if constexpr (kStaged) {
            // Two passes over halves of 128 vocabulary ids (held by the waves
            // with wm = half): the half tile goes to LDS as [t][128] fp32
            // (16-byte chunk c of row t at slot c ^ (t & 31)), then every wave
            // writes whole 512-byte row segments of the output.
            const int wave = tid >> 6;
            const int c = lane & 31;
            constexpr int RW = 256 / kDtlWaves;   // staged rows per wave
            __syncthreads();   // every wave is past its main loop: the stage LDS is free
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                if (wm == half) {
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const int t = Mma::col(wn, j, lane);
#pragma unroll
                        for (int i = 0; i < FM; ++i)
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const int vv = Mma::row(0, i, q, lane);   // within the half, multiple of 4
                                *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(
                                    smem + t * 512 + (((vv >> 2) ^ (t & 31)) << 4)) =
                                    f32x4{mma.acc[i][j][4 * q], mma.acc[i][j][4 * q + 1], mma.acc[i][j][4 * q + 2],
                                          mma.acc[i][j][4 * q + 3]};
                            }
                    }
                }
                __syncthreads();
                const int v0 = m0 + 128 * half + 4 * c;
#pragma unroll
                for (int k = 0; k < RW / 2; ++k) {
                    const int tl = wave * RW + 2 * k + (lane >> 5);
                    const f32x4 val = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
                        smem + tl * 512 + ((c ^ (tl & 31)) << 4));
                    const int t = n0 + tl;
                    if (t >= p.rows) continue;
                    float* dst = p.out + (int64_t)t * p.ld + v0;
                    if (v0 + 3 < p.V) {
                        // streamed past the caches: the select reads a few
                        // blocks of each row much later, and the lines would
                        // only displace the contraction's operand slices
                        __builtin_nontemporal_store(val, reinterpret_cast<f32x4*>(dst));
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (v0 + r < p.V) dst[r] = val[r];
                    }
                }
                if (half == 0) __syncthreads();
            }
        } else {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int t = n0 + Mma::col(wn, j, lane);
                if (t >= p.rows) continue;
                float* row = p.out + (int64_t)t * p.ld;
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int v0 = m0 + Mma::row(wm, i, q, lane);   // multiple of 4
                        if (v0 + 3 < p.V) {
                            *reinterpret_cast<f32x4*>(row + v0) =
                                f32x4{mma.acc[i][j][4 * q], mma.acc[i][j][4 * q + 1], mma.acc[i][j][4 * q + 2],
                                      mma.acc[i][j][4 * q + 3]};
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (v0 + r < p.V) row[v0 + r] = mma.acc[i][j][4 * q + r];
                        }
                    }
            }
        }
    }
};

// ---------------------------------------------------------------------------
// grad_H epilogue: tile of dH^T (rows = hidden index j, columns = chunk rows t).
// One split writes grad_H directly; several splits write fp32 partials that a
// fixed-order reduction sums.
// ---------------------------------------------------------------------------
struct GradHParams {
    void* out;            // grad_H of the chunk's first row (element type)
    float* partial;       // [splits][C][d] fp32
    int d, rows, C, direct;
    const float* fscale;  // fused entry: per-row factor of G (G = fscale_t * stored values), else null
};

template <typename E, int BM, int BN> struct GradHEpi {
    using Params = GradHParams;
    template <class Mma>
    static __device__ __forceinline__ void apply(Mma& mma, int m0, int n0, int split, int wm, int wn, int lane,
                                                 int, lds_t*, const Params& p) {
        constexpr int FM = Mma::FM, FN = Mma::FN;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int t = n0 + Mma::col(wn, j, lane);
            if (t >= p.rows) continue;
            const float f = p.fscale ? p.fscale[t] : 1.f;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int h = m0 + Mma::row(wm, i, q, lane);
                    if (h >= p.d) continue;
                    const f32x4 v = {mma.acc[i][j][4 * q] * f, mma.acc[i][j][4 * q + 1] * f,
                                     mma.acc[i][j][4 * q + 2] * f, mma.acc[i][j][4 * q + 3] * f};
                    if (p.direct) {
                        if constexpr (Elem<E>::size == 2) {
                            u32x2 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                            *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + (int64_t)t * p.d + h) = w;
                        } else {
                            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + (int64_t)t * p.d + h) = v;
                        }
                    } else {
                        *reinterpret_cast<f32x4*>(p.partial + ((int64_t)split * p.C + t) * p.d + h) = v;
                    }
                }
        }
    }
};

// ---------------------------------------------------------------------------
// grad_W epilogue: tile of dW^T (rows = hidden index j, columns = vocab ids v),
// written to (first chunk) or added to (later chunks) the fp32 grad_W[V][d].
// Every element has one owner per chunk: no atomics, fixed chunk order.
// ---------------------------------------------------------------------------
struct GradWParams {
    float* gw;
    int d, V, accumulate;
};

template <typename E, int BM, int BN> struct GradWEpi {
    using Params = GradWParams;
    static constexpr bool kStaged = Elem<E>::size == 2;   // bf16 engine: stage LDS free for the epilogue

    template <class Mma>
    static __device__ __forceinline__ void apply(Mma& mma, int m0, int n0, int, int wm, int wn, int lane, int tid,
                                                 lds_t* smem, const Params& p) {
        constexpr int FM = Mma::FM, FN = Mma::FN;
        if constexpr (kStaged) {
            // Two passes over halves of 128 hidden indices (owned by the waves
            // with wm = half): the half tile goes to LDS as [v][128] fp32
            // (16-byte chunk c of row v at c ^ (v & 31)), then every wave
            // updates whole 512-byte row segments of grad_W.  The thread index
            // goes through an empty asm first, so that none of the addresses
            // below is computed ahead of the main loop (where they would hold
            // registers the whole time).
            int tid_o = tid;
            opaque(tid_o);
            const int wave = tid_o >> 6;
            const int lane_o = tid_o & 63;
            const int c = lane_o & 31;
            constexpr int RW = 256 / kDtlWaves;   // staged rows per wave
            constexpr int NK = RW / 2;            // 16-byte pieces per thread and half
            // this thread's pieces of grad_W: the first half's are read before
            // anything is staged, the second half's as the first half's stores
            // free their registers, so the latency overlaps staging and barriers.
            // The tile's rows n0.. go through one buffer resource (at most
            // 256 · 2^20 · 4 bytes, below kOOB): a piece past the hidden size
            // gets the out-of-range offset and a row past V lies beyond
            // num_records, so the hardware drops those stores and reads zeros
            // (also everywhere when not accumulating).  Without branches the
            // compiler counts the loads in flight exactly instead of waiting
            // for every earlier store before each one (vmcnt(0)).
            const int rows = min(256, p.V - n0);
            const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.gw + (int64_t)n0 * p.d, (uint32_t)rows * (uint32_t)p.d * 4u);
            const __amdgpu_buffer_rsrc_t rr = make_rsrc(p.gw + (int64_t)n0 * p.d,
                                                        p.accumulate ? (uint32_t)rows * (uint32_t)p.d * 4u : 0u);
            auto off_of = [&](int half, int k) -> uint32_t {
                const int vl = wave * RW + 2 * k + (lane_o >> 5);
                const int h = m0 + 128 * half + 4 * c;
                return h < p.d ? ((uint32_t)vl * (uint32_t)p.d + (uint32_t)h) * 4u : kOOB;
            };
            auto load_old = [&](int half, int k) {   // read once: non-temporal too
                return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, off_of(half, k), 0, 2));
            };
            f32x4 old[NK];
#pragma unroll
            for (int k = 0; k < NK; ++k) old[k] = load_old(0, k);
            __syncthreads();   // every wave is past its main loop: the stage LDS is free
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                if (wm == half) {
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const int v = Mma::col(wn, j, lane);
#pragma unroll
                        for (int i = 0; i < FM; ++i)
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const int hh = Mma::row(0, i, q, lane);   // within the half, multiple of 4
                                const f32x4 val = {mma.acc[i][j][4 * q], mma.acc[i][j][4 * q + 1],
                                                   mma.acc[i][j][4 * q + 2], mma.acc[i][j][4 * q + 3]};
                                *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(
                                    smem + v * 512 + (((hh >> 2) ^ (v & 31)) << 4)) = val;
                            }
                    }
                }
                __syncthreads();
#pragma unroll
                for (int k = 0; k < NK; ++k) {
                    const int vl = wave * RW + 2 * k + (lane_o >> 5);
                    const f32x4 val = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
                        smem + vl * 512 + ((c ^ (vl & 31)) << 4));
                    // non-temporal (cache policy 2), like the loads of the old
                    // values: grad_W is not touched again before the next
                    // chunk, and its lines would displace operand slices from
                    // L2 (together -0.8% on the GPT-OSS-like grad_W, -3% on
                    // the Llama-like one)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, val + old[k]), rw,
                                                           off_of(half, k), 0, 2);
                    if (half == 0) old[k] = load_old(1, k);
                }
                if (half == 0) __syncthreads();
            }
        } else {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int v = n0 + Mma::col(wn, j, lane);
                if (v >= p.V) continue;
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int h = m0 + Mma::row(wm, i, q, lane);
                        if (h >= p.d) continue;
                        f32x4* dst = reinterpret_cast<f32x4*>(p.gw + (int64_t)v * p.d + h);
                        f32x4 val = {mma.acc[i][j][4 * q], mma.acc[i][j][4 * q + 1], mma.acc[i][j][4 * q + 2],
                                     mma.acc[i][j][4 * q + 3]};
                        if (p.accumulate) val += *dst;
                        *dst = val;
                    }
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Block reductions (256 threads)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float block_max(float v, float* sh) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    return fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}

__device__ __forceinline__ float block_sum(float v, float* sh) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

// ---------------------------------------------------------------------------
// Prepass: N, s = g / (tau N), loss accumulator reset.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void prepass_kernel(WsHeader* hdr, const uint8_t* ignore, int64_t T,
                                                           const float* grad_loss, float tau) {
    __shared__ float sh[4];
    int64_t cnt = 0;
    for (int64_t t = threadIdx.x; t < T; t += kThreads) cnt += (ignore == nullptr || ignore[t] == 0);
    // counts are exact in fp32 up to 2^24 per thread; sum per wave in integers
    int64_t c = cnt;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o, kWave);
    __shared__ int64_t shc[4];
    if ((threadIdx.x & 63) == 0) shc[threadIdx.x >> 6] = c;
    __syncthreads();
    (void)sh;
    if (threadIdx.x == 0) {
        const int64_t N = shc[0] + shc[1] + shc[2] + shc[3];
        const float g = grad_loss ? *grad_loss : 1.0f;
        hdr->N = N;
        hdr->s = N > 0 ? g / (tau * (float)N) : 0.f;
        hdr->loss_acc = 0.0;
    }
}

// ---------------------------------------------------------------------------
// Row kernel: one workgroup per chunk row.
//   merge the logit tiles' partials into lse (kStats / kFused),
//   teacher softmax over the K cached logits ([TH] "Dense KL": the teacher
//   distribution comes from the cached top-K logits),
//   student logits at the cached ids as K dot products H_t . W_id,
//   row loss  L = sum_k p_k (log p_k - a_k + lse),
//   kBwd: replace the K cached entries of G by s (q - P).
// The forward and fused entries run it twice per chunk.  Before the logits
// GEMM (pre): the dot products, kept for later, and the row's reference
// R0 = max_k y_k (base 2), relative to which the GEMM sums (and, fused,
// stores) the exponentials.  After it: lse, loss and, fused, the factor that
// turns the stored exponentials into G.  The GEMM stores 2^(y - R0) wherever a block's max stays within
// kRefSlack of R0 (the usual case: some cached id is among the student's
// largest logits), so G = s 2^(R0 - lse) * stored value with one factor per
// row, which the gradient GEMMs apply (grad_H in its epilogue, grad_W through
// a scaled copy of the chunk's H).  A row with a block stored relative to its
// own max R_b is marked dirty: every block is brought to the row's largest
// reference by rescale_kernel.  The cached entries are stored as
// 2^(y_k - R) - P_k 2^(lse - R), i.e. s (q - P) divided by the row factor.
// ---------------------------------------------------------------------------
struct RowParams {
    int mode;
    int t0, rows;
    int d, V, V_pad, K, nst, C;
    float inv_tau;
    const void* H;          // [T][d]
    const void* W;          // [V][d]
    const int32_t* idx;     // [T][K]
    const void* logit;      // [T][K] fp32, or bf16 when logit_bf16
    int logit_bf16;
    const uint8_t* ignore;  // [T] or null
    const f32x2* stats;     // [C][nst]
    const float* lse_in;    // [T] (kBwd)
    float* lse_out;         // [T] or null
    float* row_loss;        // [T] or null
    float* chunk_loss;      // [C]
    void* G;                // C x V_pad, GLayout<E>
    int2* sparse;           // kFused: [C][K] (id or -1, stored value bits) of the cached entries
    WsHeader* hdr;
    // fused entry
    int pre;                // 1: the pass before the logits GEMM (dot products and references)
    float* zc;              // [C][K] student logits a = z / tau at the cached ids
    float* ref;             // [C] base-2 reference R0 of the stored exponentials
    float* fscale;          // [C] G = fscale_t * stored values
    uint8_t* dirty;         // [C] 1: some block of the row is stored relative to its own max
};

constexpr int kMaxK = 1024;

// Cached teacher logit i (fp32, or bf16 widened exactly).
__device__ __forceinline__ float teacher_logit(const void* logit, int bf16, int64_t i) {
    return bf16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(logit)[i])
                : reinterpret_cast<const float*>(logit)[i];
}

template <typename E>
__device__ __forceinline__ float dot_row(const E* h, const E* w, int d, int lane) {
    float acc = 0.f;
    if constexpr (Elem<E>::size == 2) {
        const u32x4* hv = reinterpret_cast<const u32x4*>(h);
        const u32x4* wv = reinterpret_cast<const u32x4*>(w);
        for (int c = lane; c < d / 8; c += kWave) {
            const u32x4 a = hv[c], b = wv[c];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc = fmaf(bf16_bits_to_f32(a[q] & 0xFFFFu), bf16_bits_to_f32(b[q] & 0xFFFFu), acc);
                acc = fmaf(bf16_bits_to_f32(a[q] >> 16), bf16_bits_to_f32(b[q] >> 16), acc);
            }
        }
    } else {
        const f32x4* hv = reinterpret_cast<const f32x4*>(h);
        const f32x4* wv = reinterpret_cast<const f32x4*>(w);
        for (int c = lane; c < d / 4; c += kWave) {
            const f32x4 a = hv[c], b = wv[c];
            acc = fmaf(a[0], b[0], acc);
            acc = fmaf(a[1], b[1], acc);
            acc = fmaf(a[2], b[2], acc);
            acc = fmaf(a[3], b[3], acc);
        }
    }
    return wave_sum(acc);
}

// The wave's share of the K dot products H_t . W_id (bf16 rows of nc 16-byte
// chunks, NR >= ceil(nc / 64) chunks per lane): the H row stays in registers,
// and NP W rows are loaded before any of them is multiplied (NP = 2 measured
// best: 3 and 4 lose more to occupancy than they gain).  Each packed pair of
// bf16 products is added to the fp32 sum by one v_dot2 (the products of bf16
// values are exact in fp32).  Writes z / tau.
template <int NR>
__device__ __forceinline__ void dots_bf16(const void* h, const void* W, const int* ids, int K, int d, int nc,
                                          int wave, int lane, float inv_tau, float* out) {
    constexpr int NW = kThreads / kWave;
    constexpr int NP = 2;
    const u32x4* hv = reinterpret_cast<const u32x4*>(h);
    u32x4 a[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int c = lane + kWave * r;
        a[r] = c < nc ? hv[c] : u32x4{0u, 0u, 0u, 0u};
    }
    for (int k = wave; k < K; k += NP * NW) {
        u32x4 b[NP][NR];
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int kk = k + j * NW;
            const u32x4* w = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(W) +
                                                            (int64_t)ids[kk < K ? kk : k] * d);
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int c = lane + kWave * r;
                b[j][r] = (c < nc && kk < K) ? w[c] : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    // scalar copies first: bit-casting the vector elements in
                    // place compiled to one register read for all four q
                    const uint32_t x = a[r][q], y = b[j][r][q];
                    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y),
                                                          acc, false);
                }
            const float z = wave_sum(acc);
            const int kk = k + j * NW;
            if (lane == 0 && kk < K) out[kk] = z * inv_tau;
        }
    }
}

template <typename E>
__global__ __launch_bounds__(kThreads) void row_kernel(RowParams p) {
    __shared__ float sh_p[kMaxK], sh_lp[kMaxK], sh_a[kMaxK];
    __shared__ int sh_id[kMaxK];
    __shared__ float red[4];
    const int r = (int)blockIdx.x;
    const int t = p.t0 + r;
    const int tid = (int)threadIdx.x;
    const bool kept = (p.ignore == nullptr) || (p.ignore[t] == 0);
    const int K = p.K;
    const int wave = tid >> 6, lane = tid & 63;
    const bool fused = p.mode == kFused;
    const bool two_pass = p.mode != kBwd;   // forward and fused entries: a pass before the logits GEMM

    // student logits at the cached ids (the split backward; the forward and
    // fused entries compute them in their first pass)
    auto dots = [&]() {
        const E* hrow = reinterpret_cast<const E*>(p.H) + (int64_t)t * p.d;
        const int nc8 = p.d / 8;   // 16-byte chunks of a bf16 row
        bool done = false;
        if constexpr (Elem<E>::size == 2) {
            done = true;
            if (nc8 <= 2 * kWave)      dots_bf16<2>(hrow, p.W, sh_id, K, p.d, nc8, wave, lane, p.inv_tau, sh_a);
            else if (nc8 <= 4 * kWave) dots_bf16<4>(hrow, p.W, sh_id, K, p.d, nc8, wave, lane, p.inv_tau, sh_a);
            else if (nc8 <= 6 * kWave) dots_bf16<6>(hrow, p.W, sh_id, K, p.d, nc8, wave, lane, p.inv_tau, sh_a);
            else                       done = false;
        }
        if (!done) {
            for (int k = wave; k < K; k += kThreads / kWave) {
                const E* wrow = reinterpret_cast<const E*>(p.W) + (int64_t)sh_id[k] * p.d;
                const float z = dot_row<E>(hrow, wrow, p.d, lane);
                if (lane == 0) sh_a[k] = z * p.inv_tau;
            }
        }
        __syncthreads();
    };

    if (two_pass && p.pre) {
        if (r == 0 && tid == 0) p.hdr->dirty = 0;
        if (!kept) {
            // no reference: every block sums relative to its own max, so the
            // row's lse stays finite however small its logits are (its G is 0)
            if (tid == 0) p.ref[r] = -INFINITY;
            return;
        }
        for (int k = tid; k < K; k += kThreads) sh_id[k] = clamp_id(p.idx[(int64_t)t * K + k], p.V);
        __syncthreads();
        dots();
        float ym = -INFINITY;
        for (int k = tid; k < K; k += kThreads) {
            p.zc[(int64_t)r * K + k] = sh_a[k];
            ym = fmaxf(ym, sh_a[k] * kLog2e);
        }
        ym = block_max(ym, red);
        if (tid == 0) p.ref[r] = ym;
        return;
    }

    // 1. lse of the row; Mall = the largest block reference
    float lse2, Mall = 0.f;
    if (p.mode != kBwd) {
        const f32x2* st = p.stats + (int64_t)r * p.nst;
        float M = -INFINITY, S = 0.f;
        for (int i = tid; i < p.nst; i += kThreads) {
            const f32x2 v = st[i];
            const float Mn = fmaxf(M, v[0]);
            if (Mn > -INFINITY) S = S * fast_exp2(M - Mn) + v[1] * fast_exp2(v[0] - Mn);
            M = Mn;
        }
        Mall = block_max(M, red);
        const float Sall = block_sum(M > -INFINITY ? S * fast_exp2(M - Mall) : 0.f, red);
        lse2 = Mall + fast_log2(Sall);
        if (tid == 0 && p.lse_out) p.lse_out[t] = lse2 * kLn2;
    } else {
        lse2 = p.lse_in[t] * kLog2e;
    }

    if (!kept) {
        if (p.mode != kBwd) {
            if (tid == 0) {
                p.chunk_loss[r] = 0.f;
                if (p.row_loss) p.row_loss[t] = 0.f;
            }
        }
        if (fused) {
            // factor 0: the row contributes nothing; no cached entries
            if (tid == 0) {
                p.fscale[r] = 0.f;
                p.dirty[r] = 0;
            }
            for (int k = tid; k < K; k += kThreads) p.sparse[(int64_t)r * K + k] = int2{-1, 0};
        }
        return;
    }

    // 2. teacher distribution over the cached entries
    float bmax = -INFINITY;
    for (int k = tid; k < K; k += kThreads) {
        const float b = teacher_logit(p.logit, p.logit_bf16, (int64_t)t * K + k) * p.inv_tau;
        sh_lp[k] = b;
        sh_id[k] = clamp_id(p.idx[(int64_t)t * K + k], p.V);
        if (two_pass) sh_a[k] = p.zc[(int64_t)r * K + k];
        bmax = fmaxf(bmax, b);
    }
    bmax = block_max(bmax, red);
    float esum = 0.f;
    for (int k = tid; k < K; k += kThreads) esum += fast_exp2((sh_lp[k] - bmax) * kLog2e);
    esum = block_sum(esum, red);
    const float logS = fast_log2(esum) * kLn2;
    for (int k = tid; k < K; k += kThreads) {
        const float lp = sh_lp[k] - bmax - logS;
        sh_lp[k] = lp;
        sh_p[k] = fast_exp2(lp * kLog2e);
    }

    // 3. student logits at the cached ids
    if (!two_pass) dots();
    else __syncthreads();
    const float lse = lse2 * kLn2;

    // 4. row loss (entries with p = 0 contribute 0)
    if (p.mode != kBwd) {
        float L = 0.f;
        for (int k = tid; k < K; k += kThreads)
            if (sh_p[k] > 0.f) L += sh_p[k] * (sh_lp[k] - sh_a[k] + lse);
        L = block_sum(L, red);
        if (tid == 0) {
            p.chunk_loss[r] = L;
            if (p.row_loss) p.row_loss[t] = L;
        }
        if (p.mode == kStats) return;
    }

    const float s = p.hdr->s;
    // 5. fused: the row factor and, for a dirty row, the per-block factors
    // 2^(R_b - Mall) (each <= 1) in place of the blocks' references
    if (fused) {
        const bool clean = Mall == p.ref[r];
        if (tid == 0) {
            p.fscale[r] = s * fast_exp2(Mall - lse2);
            p.dirty[r] = clean ? 0 : 1;
            if (!clean) atomicAdd(&p.hdr->dirty, 1);
        }
        if (!clean) {
            f32x2* st = const_cast<f32x2*>(p.stats + (int64_t)r * p.nst);
            float* fac = reinterpret_cast<float*>(st);
            for (int i = tid; i < p.nst; i += kThreads) fac[2 * i] = fast_exp2(st[i][0] - Mall);
        }
    }

    // 6. cached entries: G = s (q - P), P summing duplicate ids; first occurrence
    // writes (fused: into the sparse list as s (q - P) / row factor, written
    // into G after any rescale)
    const float up = fast_exp2(lse2 - Mall);
    for (int k = tid; k < K; k += kThreads) {
        const int id = sh_id[k];
        bool first = true;
        for (int k2 = 0; k2 < k; ++k2) first &= (sh_id[k2] != id);
        if (!first) {
            if (fused) p.sparse[(int64_t)r * K + k] = int2{-1, 0};
            continue;
        }
        float P = sh_p[k];
        for (int k2 = k + 1; k2 < K; ++k2) P += (sh_id[k2] == id) ? sh_p[k2] : 0.f;
        if (fused) {
            const float val = fast_exp2(sh_a[k] * kLog2e - Mall) - P * up;
            p.sparse[(int64_t)r * K + k] = int2{id, __float_as_int(val)};
            continue;
        }
        const float q = fast_exp2(sh_a[k] * kLog2e - lse2);
        const float gval = s * (q - P);
        if constexpr (Elem<E>::size == 2) {
            reinterpret_cast<uint16_t*>(p.G)[GLayout<E>::index(r, id, p.C, p.V_pad)] =
                (uint16_t)(pack_bf16x2(gval, 0.f) & 0xFFFFu);
        } else {
            reinterpret_cast<float*>(p.G)[GLayout<E>::index(r, id, p.C, p.V_pad)] = gval;
        }
    }
}

// Fused entry, dirty rows only: stored value *= 2^(R_b - Mall) per 128-id
// block (the factors the row kernel left in the block statistics), in place,
// over the chunk's G buffer in its physical order.  The buffer is cut into
// spans of kRescaleSpan contiguous 16-byte chunks: bf16 (blocked layout)
// span (sx, sy) = chunks sx * span .. of 64-id block sy, nx = C * 8 / span;
// fp32 (row-major) span (sx, sy) = row sx, chunks sy * span .., nx = C.  A
// grid of at most kRescaleGrid workgroups strides over the spans, so that a
// chunk with no dirty row (the usual case) costs one small launch whose
// workgroups all exit at once.
constexpr int kRescaleU = 8;                          // chunks in flight per thread
constexpr int kRescaleSpan = kThreads * kRescaleU;    // chunks per span
constexpr int kRescaleGrid = 1024;

template <typename E>
__global__ __launch_bounds__(kThreads) void rescale_kernel(void* G, const f32x2* fac, const uint8_t* dirty,
                                                           const WsHeader* hdr, int nst, int C, int V_pad, int rows,
                                                           int nx, int64_t nspans) {
    if (hdr->dirty == 0) return;
    constexpr int kEpc = 16 / Elem<E>::size;          // elements per 16-byte chunk
    auto scale = [&](u32x4& x, float f) {
        if constexpr (Elem<E>::size == 2) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                x[q] = pack_bf16x2(bf16_bits_to_f32(x[q] & 0xFFFFu) * f, bf16_bits_to_f32(x[q] >> 16) * f);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) x[q] = __float_as_uint(__uint_as_float(x[q]) * f);
        }
    };
    u32x4* g = reinterpret_cast<u32x4*>(G);
    for (int64_t sp = blockIdx.x; sp < nspans; sp += gridDim.x) {
        const int sx = (int)(sp % nx), sy = (int)(sp / nx);
        int64_t base;                                 // first chunk of this span
        int64_t end;                                  // end of its contiguous range
        int r0, v0;                                   // (row, id) of chunk `base`
        if constexpr (GLayout<E>::kBlocked) {
            const int per_blk = C * (kGBlock / kEpc); // chunks of one 64-id block
            const int w0 = sx * kRescaleSpan;
            base = (int64_t)sy * per_blk + w0;
            end = (int64_t)sy * per_blk + min(per_blk, w0 + kRescaleSpan);
            r0 = w0 / (kGBlock / kEpc);
            v0 = sy * kGBlock;
        } else {
            const int per_row = V_pad / kEpc;
            const int w0 = sy * kRescaleSpan;
            base = (int64_t)sx * per_row + w0;
            end = (int64_t)sx * per_row + min(per_row, w0 + kRescaleSpan);
            r0 = sx;
            v0 = w0 * kEpc;
        }
        // chunk base + w -> (row, id)
        auto where = [&](int w, int& r, int& v) {
            if constexpr (GLayout<E>::kBlocked) {
                r = r0 + w / (kGBlock / kEpc);
                v = v0 + (w % (kGBlock / kEpc)) * kEpc;
            } else {
                r = r0;
                v = v0 + w * kEpc;
            }
        };
        u32x4 x[kRescaleU];
        float f[kRescaleU];
        bool live[kRescaleU];
#pragma unroll
        for (int u = 0; u < kRescaleU; ++u) {
            const int w = u * kThreads + (int)threadIdx.x;
            int r, v;
            where(w, r, v);
            live[u] = base + w < end && r < rows && dirty[r] != 0;
            f[u] = live[u] ? fac[(int64_t)r * nst + v / kStatIds][0] : 0.f;
            x[u] = live[u] ? g[base + w] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kRescaleU; ++u) {
            if (!live[u]) continue;
            scale(x[u], f[u]);
            g[base + u * kThreads + (int)threadIdx.x] = x[u];
        }
    }
}

// kFused: the cached entries of the sparse list into G (after the rescale).
template <typename E>
__global__ __launch_bounds__(kThreads) void sparse_kernel(void* G, const int2* sparse, int64_t n, int K, int C,
                                                          int V_pad) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    const int2 e = sparse[i];
    if (e.x < 0) return;
    const int64_t at = GLayout<E>::index(i / K, e.x, C, V_pad);
    const float gval = __int_as_float(e.y);
    if constexpr (Elem<E>::size == 2)
        reinterpret_cast<uint16_t*>(G)[at] = (uint16_t)(pack_bf16x2(gval, 0.f) & 0xFFFFu);
    else
        reinterpret_cast<float*>(G)[at] = gval;
}

// Fused entry: Hs = fscale_t * H_t for the chunk's rows (rounded to the element
// type), the grad_W operand that carries G's per-row factor.  Grid: rows x
// ceil(d / 8 / 256) workgroups of 16-byte chunks (8 bf16 or 4 fp32 elements).
template <typename E>
__global__ __launch_bounds__(kThreads) void scale_rows_kernel(const void* H, void* Hs, const float* fscale, int d) {
    constexpr int kEpc = 16 / Elem<E>::size;
    const int r = (int)blockIdx.y;
    const int c = (int)blockIdx.x * kThreads + (int)threadIdx.x;
    if (c * kEpc >= d) return;
    const float f = fscale[r];
    u32x4 x = reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(H) + (int64_t)r * d * Elem<E>::size)[c];
    if constexpr (Elem<E>::size == 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            x[q] = pack_bf16x2(bf16_bits_to_f32(x[q] & 0xFFFFu) * f, bf16_bits_to_f32(x[q] >> 16) * f);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = __float_as_uint(__uint_as_float(x[q]) * f);
    }
    reinterpret_cast<u32x4*>(reinterpret_cast<char*>(Hs) + (int64_t)r * d * Elem<E>::size)[c] = x;
}

// Sum of the chunk's row losses in a fixed order, added to the running total.
__global__ __launch_bounds__(kThreads) void loss_chunk_kernel(WsHeader* hdr, const float* chunk_loss, int rows) {
    __shared__ double sh[kThreads];
    double acc = 0.0;
    for (int i = threadIdx.x; i < rows; i += kThreads) acc += (double)chunk_loss[i];
    sh[threadIdx.x] = acc;
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) hdr->loss_acc += sh[0];
}

__global__ void loss_final_kernel(const WsHeader* hdr, float* loss) {
    if (threadIdx.x == 0 && blockIdx.x == 0)
        *loss = hdr->N > 0 ? (float)(hdr->loss_acc / (double)hdr->N) : 0.f;
}

// grad_H rows of a chunk = fixed-order sum of the split partials.
template <typename E>
__global__ __launch_bounds__(kThreads) void gradh_reduce_kernel(void* out, const float* partial, int rows,
                                                                int d, int C, int splits) {
    const int64_t n4 = (int64_t)rows * d / 4;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kThreads) {
        const int64_t e = i * 4;
        f32x4 acc = *reinterpret_cast<const f32x4*>(partial + e);
        for (int s = 1; s < splits; ++s)
            acc += *reinterpret_cast<const f32x4*>(partial + (int64_t)s * C * d + e);
        if constexpr (Elem<E>::size == 2) {
            u32x2 w = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
            *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + e) = w;
        } else {
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + e) = acc;
        }
    }
}

__global__ __launch_bounds__(kThreads) void zero_kernel(u32x4* p, int64_t n16) {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += (int64_t)gridDim.x * kThreads)
        p[i] = u32x4{0u, 0u, 0u, 0u};
}

// Precondition check: ids outside [0, V) and kept rows without a finite teacher logit.
__global__ __launch_bounds__(kThreads) void validate_kernel(const int32_t* idx, const void* logit, int logit_bf16,
                                                            const uint8_t* ignore, int64_t T, int K, int V,
                                                            unsigned long long* bad) {
    const int64_t t = blockIdx.x;
    if (t >= T) return;
    if (ignore && ignore[t]) return;
    unsigned long long nbad = 0;
    int finite = 0, nan = 0;
    for (int k = threadIdx.x; k < K; k += kThreads) {
        const int id = idx[t * K + k];
        nbad += (id < 0 || id >= V);
        const float l = teacher_logit(logit, logit_bf16, t * K + k);
        nan |= (l != l);
        finite |= (l > -INFINITY && l == l);
    }
    __shared__ int shf[kThreads], shn[kThreads];
    __shared__ unsigned long long shb[kThreads];
    shf[threadIdx.x] = finite;
    shn[threadIdx.x] = nan;
    shb[threadIdx.x] = nbad;
    __syncthreads();
    if (threadIdx.x == 0) {
        int f = 0, n = 0;
        unsigned long long b = 0;
        for (int i = 0; i < kThreads; ++i) { f |= shf[i]; n |= shn[i]; b += shb[i]; }
        b += (!f || n) ? 1ull : 0ull;
        if (b) atomicAdd(bad, b);
    }
}

// out = g[0] * in over n elements (g = NULL: 1), element types EI -> EO (bf16
// results rounded to nearest even); n is a multiple of 8 (a whole 16-byte
// chunk of bf16 input or output).  out may be in itself when EI == EO.
template <typename EI, typename EO>
__global__ __launch_bounds__(kThreads) void scale_kernel(const void* in, void* out, int64_t n, const float* g) {
    const float s = g ? *g : 1.0f;
    const int64_t n8 = n / 8;   // groups of 8 elements
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n8; i += (int64_t)gridDim.x * kThreads) {
        float v[8];
        if constexpr (Elem<EI>::size == 2) {
            const u32x4 x = reinterpret_cast<const u32x4*>(in)[i];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v[2 * q] = bf16_bits_to_f32(x[q] & 0xFFFFu);
                v[2 * q + 1] = bf16_bits_to_f32(x[q] >> 16);
            }
        } else {
            const f32x4 a = reinterpret_cast<const f32x4*>(in)[2 * i];
            const f32x4 b = reinterpret_cast<const f32x4*>(in)[2 * i + 1];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v[q] = a[q];
                v[4 + q] = b[q];
            }
        }
        if constexpr (Elem<EO>::size == 2) {
            reinterpret_cast<u32x4*>(out)[i] = u32x4{pack_bf16x2(v[0] * s, v[1] * s), pack_bf16x2(v[2] * s, v[3] * s),
                                                     pack_bf16x2(v[4] * s, v[5] * s), pack_bf16x2(v[6] * s, v[7] * s)};
        } else {
            reinterpret_cast<f32x4*>(out)[2 * i] = f32x4{v[0] * s, v[1] * s, v[2] * s, v[3] * s};
            reinterpret_cast<f32x4*>(out)[2 * i + 1] = f32x4{v[4] * s, v[5] * s, v[6] * s, v[7] * s};
        }
    }
}

__global__ void set_zero_u64(unsigned long long* p) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *p = 0ull;
}

}  // namespace kd

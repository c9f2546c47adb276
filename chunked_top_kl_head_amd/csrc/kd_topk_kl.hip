// kd_topk_kl.hip -- C ABI and host-side chunk scheduler of the fused chunked
// top-K KL distillation loss on MI355X (gfx950).
//
// Pages cited: [TH] ai-thai.com/posts/846 (Thai translation of "Efficient
// Knowledge Distillation for LLMs: Offline Top-K Logits and a Fused Chunked KL
// Loss"), section "Fused Chunked KL Loss", item "Fused chunked KL": the
// sequence is processed slice by slice, each slice's logits are formed from
// the hidden states, folded into the loss and dropped, the backward pass
// recomputes them, and memory grows linearly with the sequence length.
//
// Per chunk of C rows the scheduler enqueues, on the caller's stream:
//   forward : row kernel (cached-id logits, row references) -> logits GEMM
//             (block partials) -> row kernel (lse, teacher, row loss) -> chunk
//             loss sum
//   backward: logits GEMM recomputed with the forward's lse (dense G) -> row
//             kernel (cached-id entries of G) -> grad_H GEMM -> grad_W GEMM
//   fused   : row kernel (cached-id logits, references) -> logits GEMM
//             (partials + softmax numerators relative to the references) ->
//             row kernel (lse, loss, row factors, cached entries) -> rescale of
//             rows whose references moved (usually none) -> cached entries
//             into G -> row-scaled H_c -> grad_H GEMM (row factors in its
//             epilogue) -> grad_W GEMM (on the row-scaled H_c)
// The workspace holds one chunk's G (C x V_pad) and partials, so its size is
// independent of T; the T-sized arrays are the caller's inputs and outputs.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <algorithm>
#include <cstring>
#include <mutex>

#include "kd_kernels.hpp"
#include "kd_topk_select.hpp"
#include "kd_topk_kl.h"
#include "kd_topk_select.h"

namespace kd {

constexpr int BM = 256, BN = 256;      // output tile of every contraction
constexpr int64_t kOperandLimit = (int64_t)1 << 31;

// fp32 operands: register-staged engine (4 waves, 32x32x2 fp32 MFMA)
template <typename E, bool AK, bool BK, class Epi>
__global__ __launch_bounds__(kThreads) void gemm_kernel(Operand A, Operand B, GemmGeom g, typename Epi::Params ep) {
    __shared__ __attribute__((aligned(16))) char smem[gemm_lds_bytes<BM, BN>()];
    gemm_body<E, BM, BN, AK, BK, Epi>(A, B, g, ep, (lds_t*)smem);
}

// bf16 operands: direct-to-LDS engine (8 waves, 32x32x16 bf16 MFMA); BB: B is
// the chunk's G in its blocked layout; RING: the operand-ring schedule (A tiles
// two steps ahead) instead of the two-stage one
template <bool AK, bool BK, bool BB, bool RING, class Epi>
__global__ __launch_bounds__(kDtlThreads) void gemm_kernel_dtl(Operand A, Operand B, GemmGeom g,
                                                               typename Epi::Params ep) {
    __shared__ __attribute__((aligned(1024))) char smem[dtl_lds_bytes<RING>()];
    gemm_body_dtl<BM, BN, AK, BK, BB, RING, Epi>(A, B, g, ep, (lds_t*)smem);
}

// Chunks of at most this many rows run their contractions on the operand ring
// (the bf16 engine's deeper prefetch): with few rows per chunk each W tile is
// shared by few output tiles and its slices come from HBM, and the two-stage
// schedule leaves the matrix cores waiting for them.  Measured on the
// GPT-OSS-like shapes (d = 2880, V = 201088): the ring is faster for the
// logits and grad_H contractions at 1,024-4,096 rows and for grad_W at
// 1,024-2,048, slower for all three at 8,192 rows, where the part runs at its
// power limit.
constexpr int64_t kRingRows = 4096;        // logits (loss and teacher) and grad_H
constexpr int64_t kRingRowsGradW = 2048;   // grad_W

// Launch of one contraction on the engine that matches the element type.
// BB: B is the chunk's G (blocked in the bf16 layout, row-major for fp32);
// ring: the bf16 engine's schedule (ignored by the fp32 engine).
template <typename E, bool AK, bool BK, bool BB, class Epi>
static void launch_gemm(dim3 grid, hipStream_t stream, const Operand& A, const Operand& B, const GemmGeom& g,
                        const typename Epi::Params& ep, bool ring) {
    if constexpr (Elem<E>::size == 2) {
        if (ring)
            hipLaunchKernelGGL((gemm_kernel_dtl<AK, BK, BB, true, Epi>), grid, dim3(kDtlThreads), 0, stream, A, B, g,
                               ep);
        else
            hipLaunchKernelGGL((gemm_kernel_dtl<AK, BK, BB, false, Epi>), grid, dim3(kDtlThreads), 0, stream, A, B,
                               g, ep);
    } else {
        (void)ring;
        hipLaunchKernelGGL((gemm_kernel<E, AK, BK, Epi>), grid, dim3(kThreads), 0, stream, A, B, g, ep);
    }
}

struct Plan {
    int64_t T, d, V, K, C;
    int es;               // element size of H, W, G
    int64_t V_pad, nst;   // padded vocabulary; (max, sum) partials per row
    float tau;
    int splits;           // grad_H splits over the vocabulary
    bool accumulate;      // grad_W += instead of =
    bool logit_bf16;      // teacher logits are bf16
    size_t off_hdr, off_closs, off_stats, off_G, off_part, off_sparse, off_zc, off_ref, off_fscale, off_dirty, off_Hs, total;
};

// Optional event tables of the profiling hook (kd_topk_kl_set_stage_events).
struct StageEvents {
    void* const* begin = nullptr;
    void* const* end = nullptr;
    int capacity = 0;
    int* recorded = nullptr;
};
static StageEvents g_stage_events[KD_NUM_STAGES];

struct StageScope {
    StageEvents& ev;
    hipStream_t stream;
    int slot;
    StageScope(int stage, hipStream_t s) : ev(g_stage_events[stage]), stream(s), slot(-1) {
        if (ev.begin && *ev.recorded < ev.capacity) {
            slot = (*ev.recorded)++;
            (void)hipEventRecord(reinterpret_cast<hipEvent_t>(ev.begin[slot]), stream);
        }
    }
    ~StageScope() {
        if (slot >= 0) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(ev.end[slot]), stream);
    }
};

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Default rows per chunk.  Larger chunks cut the grad_W read-modify-write
// traffic (once per chunk) at O(C V) workspace; 8192 rows of bf16 logits at a
// 201,088-token vocabulary are 3.3 GB, small next to 288 GB of HBM.
static int64_t default_chunk(int64_t d, int64_t V, int es) {
    (void)d;
    const int64_t V_pad = cdiv(V, BM) * BM;
    int64_t C = 8192;
    if (es == 4)
        while (C > 256 && (C + BN) * V_pad * es >= kOperandLimit) C -= 256;
    return C;
}

static int choose_splits(int64_t tiles, int64_t K, int bk) {
    if (tiles >= 512) return 1;
    int best = 1;
    double best_eff = 0.0;
    for (int s = 1; s <= 16; ++s) {
        if (s > 1 && K / s < 8 * bk) break;
        const int64_t wg = tiles * s;
        const double eff = (double)wg / (double)(cdiv(wg, 256) * 256);
        if (eff >= 0.92) return s;
        if (eff > best_eff + 1e-12) { best_eff = eff; best = s; }
    }
    return best;
}

static kd_status check_problem(const kd_problem* p) {
    if (!p) return KD_ERR_NULL;
    if (p->T < 0 || p->d < 1 || p->V < 1 || p->K < 1 || p->K > p->V || p->chunk < 0) return KD_ERR_SHAPE;
    if (!std::isfinite(p->temperature) || !(p->temperature > 0.f)) return KD_ERR_VALUE;
    if (p->dtype != KD_BF16 && p->dtype != KD_F32) return KD_ERR_UNSUPPORTED;
    // positions and ids are 32-bit inside the kernels
    if (p->d % 8 != 0 || p->K > kMaxK || p->V > ((int64_t)1 << 21) || p->T > 0x7FFFFFFFLL) return KD_ERR_UNSUPPORTED;
    if ((p->flags & ~(KD_FLAG_ACCUMULATE_GRAD_W | KD_FLAG_LOGIT_BF16)) != 0 || p->reserved != 0) return KD_ERR_VALUE;
    return KD_OK;
}

static kd_status make_plan(const kd_problem* p, kd_op op, Plan* pl) {
    kd_status st = check_problem(p);
    if (st != KD_OK) return st;
    if (op != KD_OP_FORWARD && op != KD_OP_BACKWARD && op != KD_OP_FUSED) return KD_ERR_VALUE;
    Plan q{};
    q.T = p->T; q.d = p->d; q.V = p->V; q.K = p->K;
    q.es = p->dtype == KD_BF16 ? 2 : 4;
    q.tau = p->temperature;
    q.accumulate = (p->flags & KD_FLAG_ACCUMULATE_GRAD_W) != 0;
    q.logit_bf16 = (p->flags & KD_FLAG_LOGIT_BF16) != 0;
    q.V_pad = cdiv(q.V, BM) * BM;
    q.nst = q.V_pad / kStatIds;
    q.C = p->chunk > 0 ? p->chunk : default_chunk(q.d, q.V, q.es);
    // The fp32 engine addresses operands with 32-bit buffer offsets (a tile may
    // overhang an operand's end by one tile); the bf16 engine rebases its
    // descriptors per tile and K step and has no such limit.
    if (q.es == 4 && ((q.V_pad + BM) * q.d * q.es >= kOperandLimit || (q.C + BN) * q.V_pad * q.es >= kOperandLimit ||
                      (q.C + BN) * q.d * q.es >= kOperandLimit))
        return KD_ERR_UNSUPPORTED;
    if (q.C > (1 << 20) || q.d > (1 << 20)) return KD_ERR_UNSUPPORTED;
    const int bk = 128 / q.es;
    q.splits = choose_splits(cdiv(q.d, BM) * cdiv(q.C, BN), q.V_pad, bk);
    size_t o = 0;
    q.off_hdr = o;   o += 256;
    q.off_closs = o; o = align256(o + sizeof(float) * (size_t)q.C);
    q.off_stats = o;
    if (op != KD_OP_BACKWARD) o = align256(o + sizeof(f32x2) * (size_t)(q.C * q.nst));
    q.off_G = o;
    if (op != KD_OP_FORWARD) o = align256(o + (size_t)(q.C * q.V_pad * q.es));
    q.off_part = o;
    if (op != KD_OP_FORWARD && q.splits > 1) o = align256(o + sizeof(float) * (size_t)(q.splits * q.C * q.d));
    q.off_sparse = o;
    if (op == KD_OP_FUSED) o = align256(o + sizeof(int2) * (size_t)(q.C * q.K));
    // forward and fused entries: cached-id logits and row references; fused:
    // row factors, dirty flags and the row-scaled copy of the chunk's H (the
    // grad_W operand)
    q.off_zc = o;
    if (op != KD_OP_BACKWARD) o = align256(o + sizeof(float) * (size_t)(q.C * q.K));
    q.off_ref = o;
    if (op != KD_OP_BACKWARD) o = align256(o + sizeof(float) * (size_t)q.C);
    q.off_fscale = o;
    if (op == KD_OP_FUSED) o = align256(o + sizeof(float) * (size_t)q.C);
    q.off_dirty = o;
    if (op == KD_OP_FUSED) o = align256(o + (size_t)q.C);
    q.off_Hs = o;
    if (op == KD_OP_FUSED) o = align256(o + (size_t)(q.C * q.d * q.es));
    q.total = o;
    *pl = q;
    return KD_OK;
}

static inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Tiles walked M-first in groups of `group` M-tiles, so that the 32 tiles an
// XCD runs at once share A and B slices in its L2 (measured best: 4 for the
// logits and grad_H contractions, 8 for grad_W).
static GemmGeom geom(int64_t M, int64_t N, int64_t K, int splits, int bk, int group = 4) {
    GemmGeom g;
    g.M = (int)M; g.N = (int)N; g.K = (int)K;
    g.tiles_m = (int)cdiv(M, BM);
    g.tiles_n = (int)cdiv(N, BN);
    g.k_per_split = (int)(cdiv(cdiv(K, splits), bk) * bk);
    g.group_m = (int)std::min<int64_t>(group, g.tiles_m);
    return g;
}

static dim3 gemm_grid(const GemmGeom& g, int splits) {
    const int64_t tiles = (int64_t)g.tiles_m * g.tiles_n;
    return dim3((unsigned)(cdiv(tiles, 8) * 8), (unsigned)splits, 1);
}

static inline Operand operand(const void* ptr, int64_t ld, int64_t bytes) {
    Operand o;
    o.ptr = ptr; o.ld = ld; o.bytes = (uint64_t)bytes; o.kblock = 0;
    return o;
}

// The chunk's G as an operand: blocked (bf16; ld 64 inside a block of C rows)
// or row-major [C][V_pad] (fp32).
static inline Operand g_operand(const void* G, const Plan& pl) {
    const int64_t bytes = pl.C * pl.V_pad * pl.es;
    if (pl.es == 2) {
        Operand o = operand(G, kGBlock, bytes);
        o.kblock = (uint64_t)pl.C * kGBlock * 2u;
        return o;
    }
    return operand(G, pl.V_pad, bytes);
}

// One op over all chunks.  All pointers already validated.
template <typename E>
static kd_status run(const Plan& pl, kd_op op, const void* H, const void* W, const int32_t* idx,
                     const void* logit, const uint8_t* ignore, const float* grad_loss, float* loss,
                     const float* lse_in, float* lse_out, float* row_loss, void* grad_H, float* grad_W,
                     void* ws, hipStream_t stream) {
    char* wsb = static_cast<char*>(ws);
    WsHeader* hdr = reinterpret_cast<WsHeader*>(wsb + pl.off_hdr);
    float* closs = reinterpret_cast<float*>(wsb + pl.off_closs);
    f32x2* stats = reinterpret_cast<f32x2*>(wsb + pl.off_stats);
    void* G = wsb + pl.off_G;
    float* part = reinterpret_cast<float*>(wsb + pl.off_part);
    float* zc = reinterpret_cast<float*>(wsb + pl.off_zc);
    float* ref = reinterpret_cast<float*>(wsb + pl.off_ref);
    float* fscale = reinterpret_cast<float*>(wsb + pl.off_fscale);
    uint8_t* dirty = reinterpret_cast<uint8_t*>(wsb + pl.off_dirty);
    void* Hs = wsb + pl.off_Hs;
    const bool fused = op == KD_OP_FUSED;
    const int es = pl.es, bk = 128 / es;
    const bool want_grads = op != KD_OP_FORWARD;
    const bool want_loss = op != KD_OP_BACKWARD;

    hipLaunchKernelGGL(prepass_kernel, dim3(1), dim3(kThreads), 0, stream, hdr, ignore, pl.T, grad_loss, pl.tau);
    if (want_grads && pl.T == 0 && !pl.accumulate) {
        const int64_t n16 = pl.V * pl.d * 4 / 16;
        hipLaunchKernelGGL(zero_kernel, dim3(1024), dim3(kThreads), 0, stream, reinterpret_cast<u32x4*>(grad_W), n16);
    }
    const float scale2 = kLog2e / pl.tau;
    for (int64_t t0 = 0; t0 < pl.T; t0 += pl.C) {
        const int64_t rc = pl.T - t0 < pl.C ? pl.T - t0 : pl.C;
        const char* Hc = static_cast<const char*>(H) + t0 * pl.d * es;
        RowParams rp{};
        rp.mode = op == KD_OP_FORWARD ? kStats : (fused ? kFused : kBwd);
        rp.t0 = (int)t0; rp.rows = (int)rc;
        rp.d = (int)pl.d; rp.V = (int)pl.V; rp.V_pad = (int)pl.V_pad; rp.K = (int)pl.K; rp.nst = (int)pl.nst;
        rp.inv_tau = 1.0f / pl.tau;
        rp.H = H; rp.W = W; rp.idx = idx; rp.logit = logit; rp.logit_bf16 = pl.logit_bf16; rp.ignore = ignore;
        rp.stats = stats; rp.lse_in = lse_in; rp.lse_out = lse_out; rp.row_loss = row_loss; rp.C = (int)pl.C;
        rp.chunk_loss = closs; rp.G = G; rp.hdr = hdr;
        rp.sparse = reinterpret_cast<int2*>(wsb + pl.off_sparse);
        rp.zc = zc; rp.ref = ref; rp.fscale = fscale; rp.dirty = dirty;
        if (op != KD_OP_BACKWARD) {
            // ---- dot products at the cached ids and the rows' references
            StageScope scope(KD_STAGE_ROWS, stream);
            rp.pre = 1;
            hipLaunchKernelGGL(row_kernel<E>, dim3((unsigned)rc), dim3(kThreads), 0, stream, rp);
            rp.pre = 0;
        }
        // ---- logits GEMM: Z^T = W H_c^T (M = V_pad, N = rc, K = d)
        {
            StageScope scope(KD_STAGE_LOGITS, stream);
            const Operand A = operand(W, pl.d, pl.V * pl.d * es);
            const Operand B = operand(Hc, pl.d, rc * pl.d * es);
            const GemmGeom g = geom(pl.V_pad, rc, pl.d, 1, bk);
            LogitsParams lp{};
            lp.stats = stats; lp.E = G; lp.V = (int)pl.V; lp.V_pad = (int)pl.V_pad; lp.nst = (int)pl.nst;
            lp.rows = (int)rc; lp.C = (int)pl.C; lp.scale2 = scale2; lp.hdr = hdr;
            lp.lse = lse_in ? lse_in + t0 : nullptr;
            lp.ignore = ignore ? ignore + t0 : nullptr;
            lp.ref = ref;
            const dim3 grid = gemm_grid(g, 1);
            const bool ring = rc <= kRingRows;
            if (op == KD_OP_FORWARD)
                launch_gemm<E, true, true, false, LogitsEpi<E, BM, BN, kStats>>(grid, stream, A, B, g, lp, ring);
            else if (fused)
                launch_gemm<E, true, true, false, LogitsEpi<E, BM, BN, kFused>>(grid, stream, A, B, g, lp, ring);
            else
                launch_gemm<E, true, true, false, LogitsEpi<E, BM, BN, kBwd>>(grid, stream, A, B, g, lp, ring);
        }
        // ---- row kernel
        {
            StageScope scope(KD_STAGE_ROWS, stream);
            hipLaunchKernelGGL(row_kernel<E>, dim3((unsigned)rc), dim3(kThreads), 0, stream, rp);
            if (fused) {
                // dirty rows only: every block brought to the row's largest
                // reference; then the cached entries; then the row-scaled H_c
                const int epc = 16 / es;
                const int64_t nx = es == 2 ? cdiv(pl.C * (kGBlock / epc), (int64_t)kRescaleSpan) : pl.C;
                const int64_t ny = es == 2 ? pl.V_pad / kGBlock : cdiv(pl.V_pad / epc, (int64_t)kRescaleSpan);
                const int64_t nspans = nx * ny;
                hipLaunchKernelGGL(rescale_kernel<E>, dim3((unsigned)std::min<int64_t>(nspans, kRescaleGrid)),
                                   dim3(kThreads), 0, stream, G, stats, dirty, hdr, (int)pl.nst, (int)pl.C,
                                   (int)pl.V_pad, (int)rc, (int)nx, nspans);
                const int64_t n = rc * pl.K;
                hipLaunchKernelGGL(sparse_kernel<E>, dim3((unsigned)cdiv(n, (int64_t)kThreads)), dim3(kThreads), 0,
                                   stream, G, rp.sparse, n, (int)pl.K, (int)pl.C, (int)pl.V_pad);
                if (want_grads)
                    hipLaunchKernelGGL(scale_rows_kernel<E>, dim3((unsigned)cdiv(pl.d / epc, (int64_t)kThreads),
                                                                  (unsigned)rc),
                                       dim3(kThreads), 0, stream, Hc, Hs, fscale, (int)pl.d);
            }
        }
        if (want_loss)
            hipLaunchKernelGGL(loss_chunk_kernel, dim3(1), dim3(kThreads), 0, stream, hdr, closs, (int)rc);
        if (!want_grads) continue;
        // ---- grad_H^T = W^T G^T (M = d, N = rc, K = V_pad)
        {
            const Operand A = operand(W, pl.d, pl.V * pl.d * es);
            const Operand B = g_operand(G, pl);
            const GemmGeom g = geom(pl.d, rc, pl.V_pad, pl.splits, bk);
            GradHParams hp{};
            hp.out = static_cast<char*>(grad_H) + t0 * pl.d * es;
            hp.partial = part; hp.d = (int)pl.d; hp.rows = (int)rc; hp.C = (int)pl.C;
            hp.direct = pl.splits == 1;
            hp.fscale = fused ? fscale : nullptr;
            {
                StageScope scope(KD_STAGE_GRAD_H, stream);
                launch_gemm<E, false, true, true, GradHEpi<E, BM, BN>>(gemm_grid(g, pl.splits), stream, A, B, g, hp,
                                                                       rc <= kRingRows);
            }
            if (pl.splits > 1) {
                const int64_t n4 = rc * pl.d / 4;
                const unsigned blocks = (unsigned)(cdiv(n4, kThreads) < 2048 ? cdiv(n4, kThreads) : 2048);
                hipLaunchKernelGGL(gradh_reduce_kernel<E>, dim3(blocks), dim3(kThreads), 0, stream, hp.out, part,
                                   (int)rc, (int)pl.d, (int)pl.C, pl.splits);
            }
        }
        // ---- grad_W^T (+)= H_c^T G (M = d, N = V_pad, K = rc)
        {
            StageScope scope(KD_STAGE_GRAD_W, stream);
            // fused entry: G = fscale_t * stored values, so the operand is fscale_t * H_t
            const Operand A = operand(fused ? static_cast<const char*>(Hs) : Hc, pl.d, rc * pl.d * es);
            const Operand B = g_operand(G, pl);
            // tiles grouped 8 deep in M (hidden); 12 on the operand ring, where
            // each tile has few K steps (measured on 1,024-row chunks: -2.3%)
            const bool ring = rc <= kRingRowsGradW;
            const GemmGeom g = geom(pl.d, pl.V_pad, rc, 1, bk, ring ? 12 : 8);
            GradWParams wp{};
            wp.gw = grad_W; wp.d = (int)pl.d; wp.V = (int)pl.V; wp.accumulate = t0 > 0 || pl.accumulate;
            launch_gemm<E, false, false, true, GradWEpi<E, BM, BN>>(gemm_grid(g, 1), stream, A, B, g, wp, ring);
        }
    }
    if (want_loss) hipLaunchKernelGGL(loss_final_kernel, dim3(1), dim3(64), 0, stream, hdr, loss);
    return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_HIP;
}

static kd_status dispatch(const Plan& pl, int dtype, kd_op op, const void* H, const void* W, const int32_t* idx,
                          const void* logit, const uint8_t* ignore, const float* grad_loss, float* loss,
                          const float* lse_in, float* lse_out, float* row_loss, void* grad_H, float* grad_W,
                          void* ws, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();   // clear a stale error so the status reflects this call's launches
    if (dtype == KD_BF16)
        return run<bf16_t>(pl, op, H, W, idx, logit, ignore, grad_loss, loss, lse_in, lse_out, row_loss, grad_H,
                           grad_W, ws, s);
    return run<float>(pl, op, H, W, idx, logit, ignore, grad_loss, loss, lse_in, lse_out, row_loss, grad_H, grad_W,
                      ws, s);
}

// Teacher cache from hidden states: per chunk, the logits GEMM writes the
// chunk's fp32 logits [rows][ld] into the workspace and the select kernel
// reduces each row.
struct TeacherPlan {
    int64_t T, d, V, K, C, V_pad, ld;
    int es;
    int64_t nblk;        // 128-id blocks per row (V_pad / 128)
    bool blocks;         // select through the blocks' records (bf16 operands, nblk <= kSelMaxBlocks)
    size_t off_bmax, total;
};

static kd_status teacher_plan(const kd_teacher_problem* p, TeacherPlan* out) {
    if (!p) return KD_ERR_NULL;
    if (p->T < 0 || p->d < 1 || p->V < 1 || p->K < 1 || p->K > p->V || p->chunk < 0) return KD_ERR_SHAPE;
    if (p->reserved != 0) return KD_ERR_VALUE;
    if (p->dtype != KD_BF16 && p->dtype != KD_F32) return KD_ERR_UNSUPPORTED;
    if (p->d % 8 != 0 || p->K > kSelMaxK || p->V > ((int64_t)1 << 21) || p->T > 0x7FFFFFFFLL || p->d > (1 << 20) ||
        p->chunk > (1 << 20))
        return KD_ERR_UNSUPPORTED;
    TeacherPlan q{};
    q.T = p->T; q.d = p->d; q.V = p->V; q.K = p->K;
    q.es = p->dtype == KD_BF16 ? 2 : 4;
    q.C = p->chunk > 0 ? p->chunk : 4096;
    q.V_pad = cdiv(q.V, BM) * BM;
    q.ld = cdiv(q.V, 4) * 4;
    if (q.es == 4 && ((q.V_pad + BM) * q.d * q.es >= kOperandLimit || (q.C + BN) * q.d * q.es >= kOperandLimit))
        return KD_ERR_UNSUPPORTED;
    q.nblk = q.V_pad / kSelBlock;
    q.blocks = q.es == 2 && q.nblk <= kSelMaxBlocks;
    q.off_bmax = align256((size_t)(q.C * q.ld) * sizeof(float));
    q.total = q.off_bmax + (q.blocks ? align256((size_t)(q.C * q.nblk) * sizeof(uint32_t)) : 0);
    *out = q;
    return KD_OK;
}

template <typename E>
static kd_status run_teacher(const TeacherPlan& pl, const void* H, const void* W, int32_t* idx, float* val, void* ws,
                             hipStream_t stream) {
    float* z = static_cast<float*>(ws);
    uint32_t* bmax = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + pl.off_bmax);
    const int bk = 128 / pl.es;
    for (int64_t t0 = 0; t0 < pl.T; t0 += pl.C) {
        const int64_t rc = pl.T - t0 < pl.C ? pl.T - t0 : pl.C;
        const Operand A = operand(W, pl.d, pl.V * pl.d * pl.es);
        const Operand B = operand(static_cast<const char*>(H) + t0 * pl.d * pl.es, pl.d, rc * pl.d * pl.es);
        const GemmGeom g = geom(pl.V_pad, rc, pl.d, 1, bk);
        RawLogitsParams rp{};
        rp.out = z; rp.ld = pl.ld; rp.V = (int)pl.V; rp.rows = (int)rc;
        rp.bmax = pl.blocks ? bmax : nullptr; rp.nblk = (int)pl.nblk;
        launch_gemm<E, true, true, false, RawLogitsEpi<E, BM, BN>>(gemm_grid(g, 1), stream, A, B, g, rp,
                                                                   rc <= kRingRows);
        if (pl.blocks)
            hipLaunchKernelGGL(topk_select_blocks_kernel, dim3((unsigned)rc), dim3(kSelThreads), 0, stream, z, pl.ld,
                               (int)pl.V, (int)pl.K, bmax, (int)pl.nblk, idx + t0 * pl.K, val + t0 * pl.K);
        else
            hipLaunchKernelGGL(topk_select_kernel<float>, dim3((unsigned)rc), dim3(kSelThreads), 0, stream, z, pl.ld,
                               (int)pl.V, (int)pl.K, idx + t0 * pl.K, val + t0 * pl.K);
    }
    return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_HIP;
}

}  // namespace kd

using namespace kd;

// Common argument checks: inputs present and aligned, workspace large enough.
static kd_status check_common(const kd_problem* p, kd_op op, const void* H, const void* W, const int32_t* idx,
                              const void* logit, void* ws, size_t ws_bytes, Plan* pl) {
    kd_status st = make_plan(p, op, pl);
    if (st != KD_OK) return st;
    if (!W) return KD_ERR_NULL;
    if (p->T > 0 && (!H || !idx || !logit)) return KD_ERR_NULL;
    if (pl->total > 0 && !ws) return KD_ERR_NULL;
    if (!aligned(H, 16) || !aligned(W, 16) || !aligned(ws, 16) || !aligned(idx, 4) ||
        !aligned(logit, pl->logit_bf16 ? 2 : 4))
        return KD_ERR_ALIGN;
    if (ws_bytes < pl->total) return KD_ERR_WORKSPACE;
    return KD_OK;
}

// Argument checks of the fused entry that do not involve its workspace.
static kd_status fused_args(const kd_problem* prob, const void* H, const void* W, const int32_t* topk_idx,
                            const void* topk_logit, const float* grad_loss, const float* loss, const float* lse,
                            const float* row_loss, const void* grad_H, const float* grad_W, Plan* pl) {
    kd_status st = make_plan(prob, KD_OP_FUSED, pl);
    if (st != KD_OK) return st;
    if (!W) return KD_ERR_NULL;
    if (prob->T > 0 && (!H || !topk_idx || !topk_logit)) return KD_ERR_NULL;
    if (!loss || !grad_W || (prob->T > 0 && !grad_H)) return KD_ERR_NULL;
    if (!aligned(H, 16) || !aligned(W, 16) || !aligned(topk_idx, 4) || !aligned(topk_logit, pl->logit_bf16 ? 2 : 4))
        return KD_ERR_ALIGN;
    if (!aligned(loss, 4) || !aligned(lse, 4) || !aligned(row_loss, 4) || !aligned(grad_loss, 4) ||
        !aligned(grad_H, 16) || !aligned(grad_W, 16))
        return KD_ERR_ALIGN;
    return KD_OK;
}

// The fused entry's body, shared by the workspace and no-allocation entries.
static kd_status fused_entry(const kd_problem* prob, const void* H, const void* W, const int32_t* topk_idx,
                             const void* topk_logit, const uint8_t* ignore, const float* grad_loss, float* loss,
                             float* lse, float* row_loss, void* grad_H, float* grad_W, void* workspace,
                             size_t workspace_bytes, void* stream) {
    Plan pl;
    kd_status st = fused_args(prob, H, W, topk_idx, topk_logit, grad_loss, loss, lse, row_loss, grad_H, grad_W, &pl);
    if (st != KD_OK) return st;
    if (pl.total > 0 && !workspace) return KD_ERR_NULL;
    if (!aligned(workspace, 16)) return KD_ERR_ALIGN;
    if (workspace_bytes < pl.total) return KD_ERR_WORKSPACE;
    return dispatch(pl, prob->dtype, KD_OP_FUSED, H, W, topk_idx, topk_logit, ignore, grad_loss, loss, nullptr, lse,
                    row_loss, grad_H, grad_W, workspace, stream);
}

// ---------------------------------------------------------------------------
// Scratch of the no-allocation entry: one static array per device, holding
// the fused entry's workspace.  In host code `scratch` names a host-side
// stand-in; its device address is looked up once per device (with that
// device current) and only that address is ever handed to kernels.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)256 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

static kd_status scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KD_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return KD_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return KD_OK;
}

// Largest chunk (at most the default chunk and the positions rounded up to
// 64) whose fused workspace fits the scratch; 0 if none does.
static int64_t scratch_chunk(const kd_problem& p) {
    const int64_t top = std::min<int64_t>(default_chunk(p.d, p.V, p.dtype == KD_BF16 ? 2 : 4),
                                          std::max<int64_t>(64, cdiv(p.T, 64) * 64));
    kd_problem q = p;
    auto fits = [&](int64_t C) {
        q.chunk = C;
        Plan pl;
        return make_plan(&q, KD_OP_FUSED, &pl) == KD_OK && pl.total <= kScratchBytes;
    };
    for (int64_t C = top; C >= 64; C -= 64)
        if (fits(C)) return C;
    for (int64_t C = 63; C >= 1; --C)
        if (fits(C)) return C;
    return 0;
}

extern "C" {

int64_t kd_topk_kl_default_chunk(const kd_problem* prob) {
    if (check_problem(prob) != KD_OK) return 0;
    return default_chunk(prob->d, prob->V, prob->dtype == KD_BF16 ? 2 : 4);
}

kd_status kd_topk_kl_workspace_size(const kd_problem* prob, kd_op op, size_t* bytes) {
    try {
        if (!bytes) return KD_ERR_NULL;
        Plan pl;
        kd_status st = make_plan(prob, op, &pl);
        if (st != KD_OK) return st;
        *bytes = pl.total;
        return KD_OK;
    } catch (...) {
        return KD_ERR_INTERNAL;
    }
}

kd_status kd_topk_kl_forward(const kd_problem* prob, const void* H, const void* W, const int32_t* topk_idx,
                             const void* topk_logit, const uint8_t* ignore, float* loss, float* lse, float* row_loss,
                             void* workspace, size_t workspace_bytes, void* stream) {
    try {
        Plan pl;
        kd_status st = check_common(prob, KD_OP_FORWARD, H, W, topk_idx, topk_logit, workspace, workspace_bytes, &pl);
        if (st != KD_OK) return st;
        if (!loss || (prob->T > 0 && !lse)) return KD_ERR_NULL;
        if (!aligned(loss, 4) || !aligned(lse, 4) || !aligned(row_loss, 4)) return KD_ERR_ALIGN;
        return dispatch(pl, prob->dtype, KD_OP_FORWARD, H, W, topk_idx, topk_logit, ignore, nullptr, loss, nullptr,
                        lse, row_loss, nullptr, nullptr, workspace, stream);
    } catch (...) {
        return KD_ERR_INTERNAL;
    }
}

kd_status kd_topk_kl_backward(const kd_problem* prob, const void* H, const void* W, const int32_t* topk_idx,
                              const void* topk_logit, const uint8_t* ignore, const float* lse,
                              const float* grad_loss, void* grad_H, float* grad_W, void* workspace,
                              size_t workspace_bytes, void* stream) {
    try {
        Plan pl;
        kd_status st = check_common(prob, KD_OP_BACKWARD, H, W, topk_idx, topk_logit, workspace, workspace_bytes, &pl);
        if (st != KD_OK) return st;
        if (!grad_W || (prob->T > 0 && (!lse || !grad_H))) return KD_ERR_NULL;
        if (!aligned(grad_H, 16) || !aligned(grad_W, 16) || !aligned(lse, 4) || !aligned(grad_loss, 4))
            return KD_ERR_ALIGN;
        return dispatch(pl, prob->dtype, KD_OP_BACKWARD, H, W, topk_idx, topk_logit, ignore, grad_loss, nullptr, lse,
                        nullptr, nullptr, grad_H, grad_W, workspace, stream);
    } catch (...) {
        return KD_ERR_INTERNAL;
    }
}

kd_status kd_topk_kl_fused(const kd_problem* prob, const void* H, const void* W, const int32_t* topk_idx,
                           const void* topk_logit, const uint8_t* ignore, const float* grad_loss, float* loss,
                           float* lse, float* row_loss, void* grad_H, float* grad_W, void* workspace,
                           size_t workspace_bytes, void* stream) {
    try {
        return fused_entry(prob, H, W, topk_idx, topk_logit, ignore, grad_loss, loss, lse, row_loss, grad_H, grad_W,
                           workspace, workspace_bytes, stream);
    } catch (...) {
        return KD_ERR_INTERNAL;
    }
}

kd_status kd_topk_kl_fused_noalloc(const kd_problem* prob, const void* H, const void* W, const int32_t* topk_idx,
                                   const void* topk_logit, const uint8_t* ignore, const float* grad_loss,
                                   float* loss, float* lse, float* row_loss, void* grad_H, float* grad_W,
                                   void* stream) {
    try {
        if (!prob) return KD_ERR_NULL;
        kd_problem p = *prob;
        Plan pl;
        kd_status st = fused_args(&p, H, W, topk_idx, topk_logit, grad_loss, loss, lse, row_loss, grad_H, grad_W, &pl);
        if (st != KD_OK) return st;
        if (p.chunk == 0) {
            p.chunk = scratch_chunk(p);
            if (p.chunk == 0) return KD_ERR_WORKSPACE;   // not even one row fits
        } else if (pl.total > kScratchBytes) {
            return KD_ERR_WORKSPACE;
        }
        void* ws = nullptr;
        st = scratch_of_current_device(&ws);
        if (st != KD_OK) return st;
        return fused_entry(&p, H, W, topk_idx, topk_logit, ignore, grad_loss, loss, lse, row_loss, grad_H, grad_W,
                           ws, kScratchBytes, stream);
    } catch (...) {
        return KD_ERR_INTERNAL;
    }
}

kd_status kd_topk_kl_validate(const kd_problem* prob, const int32_t* topk_idx, const void* topk_logit,
                              const uint8_t* ignore, int64_t* bad_count, void* stream) {
    try {
        kd_status st = check_problem(prob);
        if (st != KD_OK) return st;
        if (!bad_count || (prob->T > 0 && (!topk_idx || !topk_logit))) return KD_ERR_NULL;
        const bool lb16 = (prob->flags & KD_FLAG_LOGIT_BF16) != 0;
        if (!aligned(bad_count, 8) || !aligned(topk_idx, 4) || !aligned(topk_logit, lb16 ? 2 : 4)) return KD_ERR_ALIGN;
        if (prob->T > 0x7FFFFFFF) return KD_ERR_UNSUPPORTED;
        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        (void)hipGetLastError();
        unsigned long long* bc = reinterpret_cast<unsigned long long*>(bad_count);
        hipLaunchKernelGGL(set_zero_u64, dim3(1), dim3(64), 0, s, bc);
        if (prob->T > 0)
            hipLaunchKernelGGL(validate_kernel, dim3((unsigned)prob->T), dim3(kThreads), 0, s, topk_idx, topk_logit,
                               (int)lb16, ignore, prob->T, (int)prob->K, (int)prob->V, bc);
        return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_HIP;
    } catch (...) {
        return KD_ERR_INTERNAL;
    }
}

static inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

kd_status kd_topk_kl_scale_grads(const kd_problem* prob, const float* grad_loss, const void* grad_H,
                                 const float* grad_W, void* out_H, void* out_W, int32_t out_w_dtype, void* stream) {
    try {
        kd_status st = check_problem(prob);
        if (st != KD_OK) return st;
        if ((grad_H == nullptr) != (out_H == nullptr) || (grad_W == nullptr) != (out_W == nullptr)) return KD_ERR_NULL;
        if (out_w_dtype != KD_BF16 && out_w_dtype != KD_F32) return KD_ERR_UNSUPPORTED;
        if (!aligned(grad_loss, 4) || !aligned(grad_H, 16) || !aligned(grad_W, 16) || !aligned(out_H, 16) ||
            !aligned(out_W, 16))
            return KD_ERR_ALIGN;
        const int es = prob->dtype == KD_BF16 ? 2 : 4;
        const int64_t nH = prob->T * prob->d, nW = prob->V * prob->d;   // d % 8 == 0: whole groups of 8
        // in place is allowed only for the same element type
        if (grad_H && out_H != grad_H && overlaps(grad_H, (size_t)nH * es, out_H, (size_t)nH * es)) return KD_ERR_VALUE;
        if (grad_W && (out_w_dtype == KD_BF16 || out_W != (const void*)grad_W) &&
            overlaps(grad_W, (size_t)nW * 4, out_W, (size_t)nW * (out_w_dtype == KD_BF16 ? 2 : 4)))
            return KD_ERR_VALUE;
        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        (void)hipGetLastError();
        auto blocks = [](int64_t n) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(n / 8, kThreads), 4096)); };
        if (grad_H && nH > 0) {
            if (es == 2)
                hipLaunchKernelGGL((scale_kernel<bf16_t, bf16_t>), dim3(blocks(nH)), dim3(kThreads), 0, s, grad_H, out_H, nH,
                                   grad_loss);
            else
                hipLaunchKernelGGL((scale_kernel<float, float>), dim3(blocks(nH)), dim3(kThreads), 0, s, grad_H, out_H, nH,
                                   grad_loss);
        }
        if (grad_W && nW > 0) {
            if (out_w_dtype == KD_BF16)
                hipLaunchKernelGGL((scale_kernel<float, bf16_t>), dim3(blocks(nW)), dim3(kThreads), 0, s, grad_W, out_W, nW,
                                   grad_loss);
            else
                hipLaunchKernelGGL((scale_kernel<float, float>), dim3(blocks(nW)), dim3(kThreads), 0, s, grad_W, out_W, nW,
                                   grad_loss);
        }
        return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_HIP;
    } catch (...) {
        return KD_ERR_INTERNAL;
    }
}

kd_status kd_topk_select(const kd_select_problem* prob, const void* logits, int32_t* topk_idx, float* topk_logit,
                         void* stream) {
    try {
        if (!prob) return KD_ERR_NULL;
        const kd_select_problem& p = *prob;
        if (p.T < 0 || p.V < 1 || p.K < 1 || p.K > p.V || p.ld < p.V) return KD_ERR_SHAPE;
        if (p.reserved != 0) return KD_ERR_VALUE;
        if ((p.dtype != KD_BF16 && p.dtype != KD_F32) || p.K > kSelMaxK || p.V > 0x7FFFFFFF || p.T > 0x7FFFFFFF)
            return KD_ERR_UNSUPPORTED;
        if (p.T == 0) return KD_OK;
        if (!logits || !topk_idx || !topk_logit) return KD_ERR_NULL;
        const int es = p.dtype == KD_BF16 ? 2 : 4;
        if (!aligned(logits, es) || !aligned(topk_idx, 4) || !aligned(topk_logit, 4)) return KD_ERR_ALIGN;
        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        (void)hipGetLastError();
        if (es == 2)
            hipLaunchKernelGGL(topk_select_kernel<bf16_t>, dim3((unsigned)p.T), dim3(kSelThreads), 0, s, logits, p.ld,
                               (int)p.V, (int)p.K, topk_idx, topk_logit);
        else
            hipLaunchKernelGGL(topk_select_kernel<float>, dim3((unsigned)p.T), dim3(kSelThreads), 0, s, logits, p.ld,
                               (int)p.V, (int)p.K, topk_idx, topk_logit);
        return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_HIP;
    } catch (...) {
        return KD_ERR_INTERNAL;
    }
}

kd_status kd_teacher_topk_workspace_size(const kd_teacher_problem* prob, size_t* bytes) {
    try {
        if (!bytes) return KD_ERR_NULL;
        TeacherPlan pl;
        const kd_status st = teacher_plan(prob, &pl);
        if (st != KD_OK) return st;
        *bytes = pl.total;
        return KD_OK;
    } catch (...) {
        return KD_ERR_INTERNAL;
    }
}

kd_status kd_teacher_topk(const kd_teacher_problem* prob, const void* H, const void* W, int32_t* topk_idx,
                          float* topk_logit, void* workspace, size_t workspace_bytes, void* stream) {
    try {
        TeacherPlan pl;
        const kd_status st = teacher_plan(prob, &pl);
        if (st != KD_OK) return st;
        if (pl.T == 0) return KD_OK;
        if (!H || !W || !topk_idx || !topk_logit || !workspace) return KD_ERR_NULL;
        if (!aligned(H, 16) || !aligned(W, 16) || !aligned(workspace, 16) || !aligned(topk_idx, 4) ||
            !aligned(topk_logit, 4))
            return KD_ERR_ALIGN;
        if (workspace_bytes < pl.total) return KD_ERR_WORKSPACE;
        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        (void)hipGetLastError();
        if (pl.es == 2) return run_teacher<bf16_t>(pl, H, W, topk_idx, topk_logit, workspace, s);
        return run_teacher<float>(pl, H, W, topk_idx, topk_logit, workspace, s);
    } catch (...) {
        return KD_ERR_INTERNAL;
    }
}

kd_status kd_topk_kl_set_stage_events(int stage, void* const* begin, void* const* end, int capacity,
                                      int* recorded) {
    if (stage < 0 || stage >= KD_NUM_STAGES) return KD_ERR_VALUE;
    StageEvents& ev = g_stage_events[stage];
    if (begin == nullptr) {
        ev = StageEvents{};
        return KD_OK;
    }
    if (!end || !recorded) return KD_ERR_NULL;
    if (capacity < 0) return KD_ERR_VALUE;
    ev.begin = begin;
    ev.end = end;
    ev.capacity = capacity;
    ev.recorded = recorded;
    return KD_OK;
}

const char* kd_status_string(kd_status status) {
    switch (status) {
        case KD_OK: return "ok";
        case KD_ERR_NULL: return "a required pointer is NULL";
        case KD_ERR_SHAPE: return "invalid shape (T, d, V, K or chunk)";
        case KD_ERR_VALUE: return "invalid value (temperature must be finite and > 0; flags known; reserved 0)";
        case KD_ERR_ALIGN: return "misaligned pointer";
        case KD_ERR_WORKSPACE:
            return "workspace too small (below kd_topk_kl_workspace_size, or beyond the 256 MiB static scratch "
                   "of kd_topk_kl_fused_noalloc)";
        case KD_ERR_UNSUPPORTED: return "unsupported problem (dtype, d % 8, K > 1024 or size limits)";
        case KD_ERR_HIP: return "HIP launch failure";
        case KD_ERR_INTERNAL: return "internal error";
    }
    return "unknown status";
}

}  // extern "C"

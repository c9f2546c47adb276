// kd_gemm.hpp -- LDS-tiled MFMA GEMM engine for gfx950 (wave64, CDNA4).
//
// Computes a BM x BN output tile  D[m, n] = sum_k A[m, k] B[k, n]  per
// workgroup of 256 threads (2 x 2 waves, each owning a (BM/2) x (BN/2) block
// of 16 x 16 MFMA accumulators), then hands the fp32 accumulators to an
// epilogue functor.  The three contractions of the loss are instances:
//   logits   Z^T = W  H_c^T   (M = vocab, N = rows, K = hidden)  both operands K-contiguous
//   grad_H   dH^T = W^T G^T   (M = hidden, N = rows, K = vocab)  A hidden-contiguous, B K-contiguous
//   grad_W   dW^T = H_c^T G   (M = hidden, N = vocab, K = rows)  both operands MN-contiguous
// Output rows are mapped to M so that every lane holds four consecutive
// M-indices of one N column: the stores of all three epilogues are then 8- or
// 16-byte vectors along the contiguous dimension of the destination.
//
// Operands reach LDS through registers.  K-contiguous operands are copied as
// 16-byte chunks; MN-contiguous operands are loaded as 16-byte vectors along
// M, transposed in registers (8 x 8 for bf16, 4 x 4 for fp32) and stored as
// K-contiguous chunks, so the MFMA fragment reads are always one ds_read_b128
// per lane.  Tiles are double buffered in LDS with one barrier per K step.
// Raw buffer loads return zero outside each operand's extent, which handles
// all M/N/K tails without branches.
#pragma once

#include "kd_common.hpp"

namespace kd {

template <typename E> struct Elem;
template <> struct Elem<bf16_t> { static constexpr int size = 2; };
template <> struct Elem<float>  { static constexpr int size = 4; };

struct Operand {
    const void* ptr;   // element (m, k) at ptr + (kmajor ? m*ld + k : k*ld + m)
    int64_t ld;        // leading dimension, elements
    uint32_t bytes;    // readable bytes from ptr (loads beyond return 0)
};

struct GemmGeom {
    int M, N, K;          // extents (elements)
    int tiles_m, tiles_n;
    int k_per_split;      // K elements per split (multiple of the K step), grid.y = splits
    int n_fastest;        // 1: consecutive tiles walk N (share the A tile), 0: walk M
};

// ---------------------------------------------------------------------------
// Global -> register -> LDS loaders for a ROWS x 128-byte operand tile
// ---------------------------------------------------------------------------
template <typename E, int ROWS, bool KMAJOR> struct TileLoader;

// K-contiguous operand: thread t copies 16-byte chunk (t & 7) of rows
// (t >> 3) + 32 i.
template <typename E, int ROWS> struct TileLoader<E, ROWS, true> {
    static constexpr int ES = Elem<E>::size;
    static constexpr int EPC = 16 / ES;          // elements per chunk
    static constexpr int NCH = ROWS / 32;        // chunks per thread
    __amdgpu_buffer_rsrc_t rs;
    uint32_t off0;       // byte offset of this thread's first chunk at k = 0
    uint32_t row_bytes;  // ld * ES
    int c, r0;
    u32x4 reg[NCH];

    __device__ __forceinline__ void init(const Operand& op, int m0, int tid) {
        rs = make_rsrc(op.ptr, op.bytes);
        c = tid & 7;
        r0 = tid >> 3;
        row_bytes = (uint32_t)(op.ld * ES);
        off0 = (uint32_t)(((int64_t)(m0 + r0) * op.ld + c * EPC) * ES);
    }
    __device__ __forceinline__ void load(int k0, int kend) {
        const bool ok = (k0 + c * EPC) < kend;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            uint32_t o = off0 + (uint32_t)(32 * i) * row_bytes + (uint32_t)(k0 * ES);
            reg[i] = buf_load16(rs, ok ? o : kOOB);
        }
    }
    __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
        for (int i = 0; i < NCH; ++i)
            *reinterpret_cast<u32x4*>(lds + lds_off(r0 + 32 * i, c)) = reg[i];
    }
};

// MN-contiguous operand: blocks of EPC (k) x EPC (m) elements; thread t owns
// blocks t + 256 i.  Each block is EPC 16-byte loads (one per k) transposed
// into EPC 16-byte chunks (one per m).
template <typename E, int ROWS> struct TileLoader<E, ROWS, false> {
    static constexpr int ES = Elem<E>::size;
    static constexpr int EPC = 16 / ES;
    static constexpr int MB = ROWS / EPC;        // m-blocks per tile
    static constexpr int NBLK = 8 * MB;          // 8 k-chunks per 128-byte row
    static constexpr int BPT = (NBLK + kThreads - 1) / kThreads;
    __amdgpu_buffer_rsrc_t rs;
    uint32_t boff[BPT];  // byte offset of block i at k = 0
    uint32_t k_bytes;    // ld * ES (one k step)
    int mb[BPT], kc[BPT];
    bool live[BPT];
    u32x4 reg[BPT][EPC];

    __device__ __forceinline__ void init(const Operand& op, int m0, int tid) {
        rs = make_rsrc(op.ptr, op.bytes);
        k_bytes = (uint32_t)(op.ld * ES);
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            const int b = tid + kThreads * i;
            live[i] = b < NBLK;
            mb[i] = b % MB;
            kc[i] = b / MB;
            boff[i] = (uint32_t)(((int64_t)kc[i] * EPC * op.ld + m0 + mb[i] * EPC) * ES);
        }
    }
    __device__ __forceinline__ void load(int k0, int kend) {
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                const int k = k0 + kc[i] * EPC + e;
                const uint32_t o = boff[i] + (uint32_t)(k0 + e) * k_bytes;
                reg[i][e] = buf_load16(rs, (live[i] && k < kend) ? o : kOOB);
            }
        }
    }
    __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            if (!live[i]) continue;
            if constexpr (EPC == 8) {
                // 8 x 8 transpose of 16-bit elements: out[mm] holds k = 0..7 of column mm.
#pragma unroll
                for (int mm = 0; mm < 8; ++mm) {
                    u32x4 o;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t lo = reg[i][2 * j][mm >> 1];
                        const uint32_t hi = reg[i][2 * j + 1][mm >> 1];
                        o[j] = (mm & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u))
                                        : ((lo & 0xFFFFu) | (hi << 16));
                    }
                    *reinterpret_cast<u32x4*>(lds + lds_off(mb[i] * 8 + mm, kc[i])) = o;
                }
            } else {
#pragma unroll
                for (int mm = 0; mm < 4; ++mm) {
                    u32x4 o = {reg[i][0][mm], reg[i][1][mm], reg[i][2][mm], reg[i][3][mm]};
                    *reinterpret_cast<u32x4*>(lds + lds_off(mb[i] * 4 + mm, kc[i])) = o;
                }
            }
        }
    }
};

// ---------------------------------------------------------------------------
// MFMA accumulator block of one wave
// ---------------------------------------------------------------------------
template <typename E, int BM, int BN> struct WaveMma {
    static constexpr int FM = BM / 32;   // 16-row fragments per wave (wave covers BM/2 rows)
    static constexpr int FN = BN / 32;
    f32x4 acc[FM][FN];

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // One 128-byte K slab: two halves of four 16-byte chunks each.
    __device__ __forceinline__ void step(const char* la, const char* lb, int wm, int wn, int lane) {
        const int lr = lane & 15, lc = lane >> 4;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            u32x4 a[FM], b[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                a[i] = *reinterpret_cast<const u32x4*>(la + lds_off(wm * (BM / 2) + i * 16 + lr, 4 * h + lc));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                b[j] = *reinterpret_cast<const u32x4*>(lb + lds_off(wn * (BN / 2) + j * 16 + lr, 4 * h + lc));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    if constexpr (Elem<E>::size == 2) {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, a[i]), __builtin_bit_cast(bf16x8, b[j]),
                            acc[i][j], 0, 0, 0);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                __uint_as_float(a[i][e]), __uint_as_float(b[j][e]), acc[i][j], 0, 0, 0);
                    }
                }
        }
    }
};

// Accumulator element (i, j, r) of lane `lane` in wave (wm, wn) sits at tile
// row  wm*BM/2 + 16 i + 4 (lane >> 4) + r  and tile column  wn*BN/2 + 16 j + (lane & 15).

template <int BM, int BN>
constexpr int gemm_lds_bytes() { return 2 * (BM + BN) * 128; }

// ---------------------------------------------------------------------------
// The kernel body
// ---------------------------------------------------------------------------
template <typename E, int BM, int BN, bool A_KMAJOR, bool B_KMAJOR, class Epi>
__device__ __forceinline__ void gemm_body(const Operand& A, const Operand& B, const GemmGeom& g,
                                          const typename Epi::Params& ep, char* smem) {
    constexpr int ES = Elem<E>::size;
    constexpr int BK = 128 / ES;
    // XCD-aware remap: hardware dispatches workgroup b to XCD b % 8; give each
    // XCD a contiguous range of logical tiles so that tiles sharing an operand
    // tile run under the same L2.
    const int total = g.tiles_m * g.tiles_n;
    const int grid = (int)gridDim.x;            // multiple of 8
    const int per_xcd = grid >> 3;
    const int pid = ((int)blockIdx.x & 7) * per_xcd + ((int)blockIdx.x >> 3);
    if (pid >= total) return;
    int tm, tn;
    if (g.n_fastest) { tm = pid / g.tiles_n; tn = pid % g.tiles_n; }
    else             { tn = pid / g.tiles_m; tm = pid % g.tiles_m; }
    const int m0 = tm * BM, n0 = tn * BN;
    const int split = (int)blockIdx.y;
    const int kbeg = split * g.k_per_split;
    const int kend = min(g.K, kbeg + g.k_per_split);
    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    TileLoader<E, BM, A_KMAJOR> la;
    TileLoader<E, BN, B_KMAJOR> lb;
    la.init(A, m0, tid);
    lb.init(B, n0, tid);
    WaveMma<E, BM, BN> mma;
    mma.zero();

    char* stage[2] = {smem, smem + (BM + BN) * 128};
    if (nk > 0) {
        la.load(kbeg, kend);
        lb.load(kbeg, kend);
        la.store(stage[0]);
        lb.store(stage[0] + BM * 128);
    }
    __syncthreads();
    for (int it = 0; it < nk; ++it) {
        const int cur = it & 1;
        const bool more = it + 1 < nk;
        if (more) {
            const int k1 = kbeg + (it + 1) * BK;
            la.load(k1, kend);
            lb.load(k1, kend);
        }
        mma.step(stage[cur], stage[cur] + BM * 128, wm, wn, lane);
        if (more) {
            la.store(stage[cur ^ 1]);
            lb.store(stage[cur ^ 1] + BM * 128);
        }
        __syncthreads();
    }
    Epi::apply(mma, m0, n0, split, wm, wn, lane, tid, smem, ep);
}

}  // namespace kd

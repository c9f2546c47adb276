// kd_gemm.hpp -- shared GEMM definitions (operands, tile order) and the
// register-staged MFMA engine for fp32 operands on gfx950 (wave64, CDNA4).
//
// Computes a BM x BN output tile  D[m, n] = sum_k A[m, k] B[k, n]  per
// workgroup of 256 threads (2 x 2 waves, each owning a (BM/2) x (BN/2) block
// of 32 x 32 MFMA accumulators), then hands the fp32 accumulators to an
// epilogue functor.  The three contractions of the loss are instances:
//   logits   Z^T = W  H_c^T   (M = vocab, N = rows, K = hidden)  both operands K-contiguous
//   grad_H   dH^T = W^T G^T   (M = hidden, N = rows, K = vocab)  A hidden-contiguous, B K-contiguous
//   grad_W   dW^T = H_c^T G   (M = hidden, N = vocab, K = rows)  both operands MN-contiguous
// Output rows are mapped to M so that every lane holds four consecutive
// M-indices of one N column: the stores of all three epilogues are then 8- or
// 16-byte vectors along the contiguous dimension of the destination.
//
// This engine serves fp32 operands only (v_mfma_f32_32x32x2f32); bf16
// operands run on the direct-to-LDS engine of kd_gemm_dtl.hpp.
//
// Operands reach LDS through registers.  K-contiguous operands are copied as
// 16-byte chunks; MN-contiguous operands are loaded as 16-byte vectors along
// M, transposed in registers (4 x 4) and stored as K-contiguous chunks, so
// every MFMA fragment read is one ds_read_b128 per lane.  Tiles are double
// buffered in LDS with one barrier per K step; the per-thread offsets of all
// loads are loop invariant and the K position costs one add per load.  Raw
// buffer loads return zero outside each operand's extent, which handles the
// M/N tails; the K tail of the last step masks offsets explicitly.
#pragma once

#include "kd_common.hpp"

namespace kd {

typedef __attribute__((address_space(3))) char lds_t;

template <typename E> struct Elem;
template <> struct Elem<bf16_t> { static constexpr int size = 2; };
template <> struct Elem<float>  { static constexpr int size = 4; };

struct Operand {
    const void* ptr;   // element (m, k) at ptr + (kmajor ? m*ld + k : k*ld + m)
    int64_t ld;        // leading dimension, elements
    uint64_t bytes;    // readable bytes from ptr (loads beyond return 0)
    uint64_t kblock;   // blocked operands only: bytes from one 64-wide block to the next
};

struct GemmGeom {
    int M, N, K;          // extents (elements)
    int tiles_m, tiles_n;
    int k_per_split;      // K elements per split (multiple of the K step), grid.y = splits
    int group_m;          // tile order: groups of group_m M-tiles, M fastest inside a group, then N
};

// Logical tile of workgroup b.  The hardware dispatches workgroup b to XCD
// b % 8; the remap gives every XCD a contiguous range of logical tiles, and the
// grouped order makes the ~32 workgroups resident on one XCD cover a
// group_m x (32 / group_m) block of tiles, so that each K step's operand slices
// are shared in that XCD's L2.  Returns false for the padding workgroups.
__device__ __forceinline__ bool tile_of(const GemmGeom& g, int& tm, int& tn) {
    const int total = g.tiles_m * g.tiles_n;
    const int per_xcd = (int)gridDim.x >> 3;                 // grid is a multiple of 8
    const int pid = ((int)blockIdx.x & 7) * per_xcd + ((int)blockIdx.x >> 3);
    if (pid >= total) return false;
    const int gsize = g.group_m * g.tiles_n;
    const int grp = pid / gsize;
    const int first_m = grp * g.group_m;
    const int gm = min(g.tiles_m - first_m, g.group_m);
    const int local = pid - grp * gsize;
    tm = first_m + local % gm;
    tn = local / gm;
    return true;
}

__device__ __forceinline__ u32x4 lds_read16(const lds_t* base, int off) {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(base + off);
}
__device__ __forceinline__ void lds_write16(lds_t* base, int off, u32x4 v) {
    *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(base + off) = v;
}

__device__ __forceinline__ u32x4 buf_load16_s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

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
    uint32_t voff[NCH];
    int c, r0;
    u32x4 reg[NCH];

    __device__ __forceinline__ void init(const Operand& op, int m0, int tid) {
        rs = make_rsrc(op.ptr, (uint32_t)op.bytes);
        c = tid & 7;
        r0 = tid >> 3;
#pragma unroll
        for (int i = 0; i < NCH; ++i)
            voff[i] = (uint32_t)(((int64_t)(m0 + r0 + 32 * i) * op.ld + c * EPC) * ES);
    }
    // k0: first K element of the step; full: the whole step lies below kend.
    // The whole byte offset travels in the vector offset (the bounds check
    // then covers it); the scalar offset stays 0.
    __device__ __forceinline__ void load(int k0, int kend, bool full) {
        const uint32_t koff = (uint32_t)(k0 * ES);
        const bool ok = full || (k0 + c * EPC) < kend;
#pragma unroll
        for (int i = 0; i < NCH; ++i) reg[i] = buf_load16_s(rs, ok ? voff[i] + koff : kOOB, 0u);
    }
    __device__ __forceinline__ void store(lds_t* lds) const {
#pragma unroll
        for (int i = 0; i < NCH; ++i) lds_write16(lds, lds_off(r0 + 32 * i, c), reg[i]);
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
    static_assert(NBLK % kThreads == 0, "every thread owns whole blocks");
    __amdgpu_buffer_rsrc_t rs;
    uint32_t boff[BPT];  // byte offset of block i at k = 0
    uint32_t k_bytes;    // ld * ES (one k step)
    int mb[BPT], kc[BPT];
    u32x4 reg[BPT][EPC];

    __device__ __forceinline__ void init(const Operand& op, int m0, int tid) {
        rs = make_rsrc(op.ptr, (uint32_t)op.bytes);
        k_bytes = (uint32_t)(op.ld * ES);
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            const int b = tid + kThreads * i;
            mb[i] = b % MB;
            kc[i] = b / MB;
            boff[i] = (uint32_t)(((int64_t)kc[i] * EPC * op.ld + m0 + mb[i] * EPC) * ES);
        }
    }
    __device__ __forceinline__ void load(int k0, int kend, bool full) {
        const uint32_t koff = (uint32_t)k0 * k_bytes;
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                const uint32_t vo = boff[i] + (uint32_t)e * k_bytes + koff;
                const bool ok = full || (k0 + kc[i] * EPC + e) < kend;
                reg[i][e] = buf_load16_s(rs, ok ? vo : kOOB, 0u);
            }
        }
    }
    __device__ __forceinline__ void store(lds_t* lds) const {
        static_assert(EPC == 4, "fp32 operands: 4 x 4 blocks");
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            // 4 x 4 transpose: out[mm] holds k = 0..3 of column mm
#pragma unroll
            for (int mm = 0; mm < 4; ++mm) {
                u32x4 o = {reg[i][0][mm], reg[i][1][mm], reg[i][2][mm], reg[i][3][mm]};
                lds_write16(lds, lds_off(mb[i] * 4 + mm, kc[i]), o);
            }
        }
    }
};

// ---------------------------------------------------------------------------
// MFMA accumulator block of one wave: (BM/2) x (BN/2) as 32 x 32 fragments.
// Lane l of fragment (i, j) holds tile rows  wm*BM/2 + 32 i + 8 q + 4 (l >> 5) + r
// (accumulator element 4 q + r, q, r in 0..3) of tile column  wn*BN/2 + 32 j + (l & 31).
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(16))) float f32x16;

template <typename E, int BM, int BN> struct WaveMma {
    static constexpr int FM = BM / 64;   // 32-row fragments per wave (wave covers BM/2 rows)
    static constexpr int FN = BN / 64;
    f32x16 acc[FM][FN];

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    }

    // One 128-byte K slab: four sub-steps of two 16-byte chunks each.  Lanes
    // 0..31 read chunk 2s, lanes 32..63 chunk 2s + 1 of their row.
    __device__ __forceinline__ void step(const lds_t* la, const lds_t* lb, int wm, int wn, int lane) {
        const int lr = lane & 31, lc = lane >> 5;
        u32x4 a[2][FM], b[2][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) a[0][i] = lds_read16(la, lds_off(wm * (BM / 2) + i * 32 + lr, lc));
#pragma unroll
        for (int j = 0; j < FN; ++j) b[0][j] = lds_read16(lb, lds_off(wn * (BN / 2) + j * 32 + lr, lc));
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int cur = s & 1;
            if (s + 1 < 4) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    a[cur ^ 1][i] = lds_read16(la, lds_off(wm * (BM / 2) + i * 32 + lr, 2 * (s + 1) + lc));
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    b[cur ^ 1][j] = lds_read16(lb, lds_off(wn * (BN / 2) + j * 32 + lr, 2 * (s + 1) + lc));
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            __uint_as_float(a[cur][i][e]), __uint_as_float(b[cur][j][e]), acc[i][j], 0, 0, 0);
        }
    }

    // tile coordinates of accumulator element (i, j, e) for lane `lane`
    static __device__ __forceinline__ int row(int wm, int i, int q, int lane) {
        return wm * (BM / 2) + 32 * i + 8 * q + 4 * (lane >> 5);
    }
    static __device__ __forceinline__ int col(int wn, int j, int lane) {
        return wn * (BN / 2) + 32 * j + (lane & 31);
    }
};

template <int BM, int BN>
constexpr int gemm_lds_bytes() { return 2 * (BM + BN) * 128; }

// ---------------------------------------------------------------------------
// The kernel body
// ---------------------------------------------------------------------------
template <typename E, int BM, int BN, bool A_KMAJOR, bool B_KMAJOR, class Epi>
__device__ __forceinline__ void gemm_body(const Operand& A, const Operand& B, const GemmGeom& g,
                                          const typename Epi::Params& ep, lds_t* smem) {
    static_assert(Elem<E>::size == 4, "bf16 operands run on the direct-to-LDS engine");
    constexpr int ES = Elem<E>::size;
    constexpr int BK = 128 / ES;
    int tm, tn;
    if (!tile_of(g, tm, tn)) return;
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

    constexpr int kStage = (BM + BN) * 128;
    if (nk > 0) {
        const bool full = kbeg + BK <= kend;
        la.load(kbeg, kend, full);
        lb.load(kbeg, kend, full);
        la.store(smem);
        lb.store(smem + BM * 128);
    }
    __syncthreads();
    for (int it = 0; it < nk; ++it) {
        lds_t* cur = smem + (it & 1) * kStage;
        lds_t* nxt = smem + ((it & 1) ^ 1) * kStage;
        const bool more = it + 1 < nk;
        if (more) {
            const int k1 = kbeg + (it + 1) * BK;
            const bool full = k1 + BK <= kend;
            la.load(k1, kend, full);
            lb.load(k1, kend, full);
        }
        mma.step(cur, cur + BM * 128, wm, wn, lane);
        if (more) {
            la.store(nxt);
            lb.store(nxt + BM * 128);
        }
        __syncthreads();
    }
    Epi::apply(mma, m0, n0, split, wm, wn, lane, tid, smem, ep);
}

}  // namespace kd

// kd_gemm_dtl.hpp -- bf16 MFMA GEMM engine for gfx950 with direct-to-LDS
// operand loads and transposing LDS reads.
//
// Tile BM x BN = 256 x 256 per workgroup of 512 threads: 8 waves as 2 (M) x 4
// (N), each wave owning a 128 x 64 block of v_mfma_f32_32x32x16_bf16
// accumulators (128 registers), so two waves share each SIMD and hide each
// other's LDS and barrier latency.
//
// Operands go from HBM/L2 straight into LDS with buffer_load_dwordx4 ... lds
// (each lane's 16 bytes land at the wave's LDS base + 16 * lane; the global
// address of every lane is chosen so that the LDS image is the swizzled tile).
// Out-of-range lanes of a raw buffer write zeros, which handles every tail.
//   K-contiguous operand: LDS tile [rows][BK] (128-byte rows, 16-byte chunks
//     XOR-swizzled by row); fragments are one ds_read_b128 per lane.
//   MN-contiguous operand: LDS tile [BK][rows] in the operand's own layout
//     (512-byte k-rows, 16-byte chunks XOR-swizzled by k); fragments are two
//     ds_read_b64_tr_b16 per lane, which transpose 4 x 16 blocks across the
//     16 lanes of a quarter-wave.
// Two LDS stages of 64 KiB; each K step waits for its own loads, meets at one
// barrier, issues the next step's loads, then runs 4 MFMA sub-steps.
#pragma once

#include "kd_gemm.hpp"

namespace kd {

constexpr int kDtlThreads = 512;

typedef __attribute__((ext_vector_type(4))) short s16x4;

__device__ __forceinline__ void dtl_load16(__amdgpu_buffer_rsrc_t r, lds_t* lds_wave_base, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16, voff,
                                             0, 0, 0);
}

__device__ __forceinline__ u32x2 lds_read8_tr(const lds_t* base, int off) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(const_cast<lds_t*>(base) + off));
    return __builtin_bit_cast(u32x2, v);
}

// MN-contiguous tile: byte offset of element (k, m) in a [64][256] bf16 tile.
__device__ __forceinline__ int mn_off(int k, int m) {
    return (k << 9) + ((((m >> 3) ^ ((k & 3) << 1))) << 4) + ((m & 7) << 1);
}

// ---------------------------------------------------------------------------
// Direct-to-LDS loaders of one 64-element K step (bf16) of a ROWS-row operand.
// Every wave issues NI instructions of 1 KiB; instruction i of wave w fills
// LDS kilobyte (w * NI + i) of the tile.
// ---------------------------------------------------------------------------
template <int ROWS, bool KMAJOR> struct DtlLoader;

template <int ROWS> struct DtlLoader<ROWS, true> {
    static constexpr int NI = ROWS * 128 / 1024 / (kDtlThreads / 64);   // 4 for 256 rows
    __amdgpu_buffer_rsrc_t rs;
    uint32_t voff[NI];
    int lane_k;          // first element of this lane's chunk within the step
    int lds0;            // LDS byte offset of this wave's first kilobyte

    __device__ __forceinline__ void init(const Operand& op, int m0, int wave, int lane) {
        rs = make_rsrc(op.ptr, op.bytes);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int kb = wave * NI + i;              // kilobyte of the tile = 8 rows
            const int r = kb * 8 + (lane >> 3);
            const int c = (lane & 7) ^ ((r ^ (r >> 3)) & 7);   // logical chunk stored at this lane's slot
            voff[i] = (uint32_t)(((int64_t)(m0 + r) * op.ld + c * 8) * 2);
            if (i == 0) lane_k = c * 8;
        }
        lds0 = wave * NI * 1024;
    }
    __device__ __forceinline__ void issue(lds_t* tile, int k0, int kend, bool full) {
        const uint32_t koff = (uint32_t)(k0 * 2);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            // chunk index differs per instruction (row-dependent swizzle): recompute its k
            bool ok = full;
            if (!full) {
                const int lane = (int)(threadIdx.x & 63);
                const int r = ((int)(threadIdx.x >> 6) * NI + i) * 8 + (lane >> 3);
                const int c = (lane & 7) ^ ((r ^ (r >> 3)) & 7);
                ok = (k0 + c * 8) < kend;
            }
            dtl_load16(rs, tile + lds0 + i * 1024, ok ? voff[i] + koff : kOOB);
        }
    }
    // fragment of 32 rows starting at row r0, sub-step s (k = 16 s .. 16 s + 15)
    static __device__ __forceinline__ u32x4 frag(const lds_t* tile, int r0, int s, int lane) {
        return lds_read16(tile, lds_off(r0 + (lane & 31), 2 * s + (lane >> 5)));
    }
};

template <int ROWS> struct DtlLoader<ROWS, false> {
    static_assert(ROWS == 256, "MN-contiguous tiles are 256 wide (512-byte k-rows)");
    static constexpr int NI = 64 * ROWS * 2 / 1024 / (kDtlThreads / 64);  // 4
    __amdgpu_buffer_rsrc_t rs;
    uint32_t voff[NI];
    uint32_t k_bytes;
    int lds0;

    __device__ __forceinline__ void init(const Operand& op, int m0, int wave, int lane) {
        rs = make_rsrc(op.ptr, op.bytes);
        k_bytes = (uint32_t)(op.ld * 2);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int kb = wave * NI + i;              // kilobyte = 2 k-rows
            const int k = kb * 2 + (lane >> 5);
            const int c = (lane & 31) ^ ((k & 3) << 1);
            voff[i] = (uint32_t)(((int64_t)k * op.ld + m0 + c * 8) * 2);
        }
        lds0 = wave * NI * 1024;
    }
    __device__ __forceinline__ void issue(lds_t* tile, int k0, int kend, bool full) {
        const uint32_t koff = (uint32_t)k0 * k_bytes;
        const int lane = (int)(threadIdx.x & 63);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int k = ((int)(threadIdx.x >> 6) * NI + i) * 2 + (lane >> 5);
            const bool ok = full || (k0 + k) < kend;
            dtl_load16(rs, tile + lds0 + i * 1024, ok ? voff[i] + koff : kOOB);
        }
    }
    // fragment of 32 columns (m) starting at m0, sub-step s: lane l gets
    // m = m0 + (l & 31), k = 16 s + 8 (l >> 5) .. + 7
    static __device__ __forceinline__ u32x4 frag(const lds_t* tile, int m0, int s, int lane) {
        const int g = lane >> 4, i = lane & 15;
        const int mb = m0 + 16 * (g & 1) + 4 * (i & 3);
        const int kb = 16 * s + 8 * (g >> 1) + (i >> 2);
        const u32x2 lo = lds_read8_tr(tile, mn_off(kb, mb));
        const u32x2 hi = lds_read8_tr(tile, mn_off(kb + 4, mb));
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
};

// Accumulators of one wave: (BM/2) x (BN/4) as 32 x 32 fragments.
template <int BM, int BN> struct DtlMma {
    static constexpr int FM = BM / 64;   // 4
    static constexpr int FN = BN / 128;  // 2
    f32x16 acc[FM][FN];
    static __device__ __forceinline__ int row(int wm, int i, int q, int lane) {
        return wm * (BM / 2) + 32 * i + 8 * q + 4 * (lane >> 5);
    }
    static __device__ __forceinline__ int col(int wn, int j, int lane) {
        return wn * (BN / 4) + 32 * j + (lane & 31);
    }
};

template <int BM, int BN, bool A_KMAJOR, bool B_KMAJOR, class Epi>
__device__ __forceinline__ void gemm_body_dtl(const Operand& A, const Operand& B, const GemmGeom& g,
                                              const typename Epi::Params& ep, lds_t* smem) {
    static_assert(BM == 256 && BN == 256, "tile shape");
    constexpr int BK = 64;
    constexpr int kTileA = BM * 128, kTileB = BN * 128, kStage = kTileA + kTileB;
    const int total = g.tiles_m * g.tiles_n;
    const int grid = (int)gridDim.x;
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
    const int wm = wave >> 2, wn = wave & 3;

    DtlLoader<BM, A_KMAJOR> la;
    DtlLoader<BN, B_KMAJOR> lb;
    la.init(A, m0, wave, lane);
    lb.init(B, n0, wave, lane);
    using Mma = DtlMma<BM, BN>;
    Mma mma;
#pragma unroll
    for (int i = 0; i < Mma::FM; ++i)
#pragma unroll
        for (int j = 0; j < Mma::FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) mma.acc[i][j][e] = 0.f;

    if (nk > 0) {
        const bool full = kbeg + BK <= kend;
        la.issue(smem, kbeg, kend, full);
        lb.issue(smem + kTileA, kbeg, kend, full);
    }
    const int am = wm * (BM / 2), bn = wn * (BN / 4);
    for (int it = 0; it < nk; ++it) {
        lds_t* cur = smem + (it & 1) * kStage;
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's loads of step `it` are in LDS
        __syncthreads();                      // every wave's are; step it-1's buffer is free
        if (it + 1 < nk) {
            lds_t* nxt = smem + ((it + 1) & 1) * kStage;
            const int k1 = kbeg + (it + 1) * BK;
            const bool full = k1 + BK <= kend;
            la.issue(nxt, k1, kend, full);
            lb.issue(nxt + kTileA, k1, kend, full);
        }
        const lds_t* ta = cur;
        const lds_t* tb = cur + kTileA;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u32x4 a[Mma::FM], b[Mma::FN];
#pragma unroll
            for (int i = 0; i < Mma::FM; ++i) a[i] = DtlLoader<BM, A_KMAJOR>::frag(ta, am + 32 * i, s, lane);
#pragma unroll
            for (int j = 0; j < Mma::FN; ++j) b[j] = DtlLoader<BN, B_KMAJOR>::frag(tb, bn + 32 * j, s, lane);
#pragma unroll
            for (int i = 0; i < Mma::FM; ++i)
#pragma unroll
                for (int j = 0; j < Mma::FN; ++j)
                    mma.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, a[i]), __builtin_bit_cast(bf16x8, b[j]), mma.acc[i][j], 0, 0, 0);
        }
    }
    __syncthreads();   // LDS is reused by epilogues
    Epi::apply(mma, m0, n0, split, wm, wn, lane, tid, smem, ep);
}

}  // namespace kd

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
//   K-contiguous operand: LDS tile [rows][BK] (16-byte chunks XOR-swizzled by
//     row); fragments are one ds_read_b128 per lane.
//   MN-contiguous operand: LDS tile [BK][rows] in the operand's own layout
//     (512-byte k-rows, 16-byte chunks XOR-swizzled by k); fragments are two
//     ds_read_b64_tr_b16 per lane, which transpose 4 x 16 blocks across the
//     16 lanes of a quarter-wave.
// kDtlStages LDS stages (one K step of kDtlBK each): all but one are in flight
// while one is consumed; each step waits only for its own loads, meets at one
// barrier, issues the step kDtlStages - 1 ahead, then runs kDtlBK / 16 MFMA
// sub-steps.
#pragma once

#include "kd_gemm.hpp"

namespace kd {

constexpr int kDtlThreads = 512;

typedef __attribute__((ext_vector_type(4))) short s16x4;

// Raw buffer descriptor as four dwords (gfx9: 48-bit base, stride 0,
// num_records = bytes, 32-bit data format).
__device__ __forceinline__ u32x4 rsrc_words(uint64_t a, uint32_t bytes) {
    return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}

// Descriptor of the window [base + off, end of operand): the loaders rebase
// every K step so that all per-lane offsets stay far below 2^31 whatever the
// operand size.  Windows that start past the end get no records (all zeros).
__device__ __forceinline__ u32x4 window_rsrc(const Operand& op, uint64_t off) {
    const uint64_t rec = op.bytes > off ? op.bytes - off : 0;
    return rsrc_words(reinterpret_cast<uint64_t>(op.ptr) + off, (uint32_t)(rec < 0x7FFFFFFFull ? rec : 0x7FFFFFFFull));
}

// One direct-to-LDS load: lane l's 16 bytes at byte offset `voff` of the
// buffer land at LDS byte address lds_addr + 16 l (out of range: zeros).  The
// instruction has no destination register; it is issued from asm so that the
// compiler does not add its own conservative vmcnt waits before unrelated LDS
// reads.  Completion is awaited explicitly with s_waitcnt vmcnt(N) before the
// barrier that publishes a stage.
__device__ __forceinline__ void dtl_load16(const u32x4& rsrc, uint32_t lds_addr, uint32_t voff) {
    uint32_t saved;   // m0 is restored, so the compiler's own uses of it are unaffected
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(rsrc), "s"(lds_addr)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_addr_of(const lds_t* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

__device__ __forceinline__ u32x2 lds_read8_tr(const lds_t* base, int off) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(const_cast<lds_t*>(base) + off));
    return __builtin_bit_cast(u32x2, v);
}

// K step of the engine (bf16 elements) and pipeline depth.  A stage holds the
// A and B tiles of one step: 2 * 256 * kDtlBK * 2 bytes.
#ifndef KD_DTL_BK
#define KD_DTL_BK 64
#endif
#ifndef KD_DTL_STAGES
#define KD_DTL_STAGES 2
#endif
constexpr int kDtlBK = KD_DTL_BK;
constexpr int kDtlStages = KD_DTL_STAGES;
constexpr int kDtlTile = 256 * kDtlBK * 2;   // bytes of one operand tile per step
static_assert(kDtlBK == 32 || kDtlBK == 64, "K step");
static_assert(kDtlStages >= 2 && kDtlStages * 2 * kDtlTile <= 160 * 1024, "stages fit in LDS");

// K-contiguous tile of one step: [rows][kDtlBK] bf16, rows of kDtlBK / 8
// 16-byte chunks.  Chunk c of row r is stored at c ^ k_swz(r), chosen so that
// a fragment read (32 consecutive rows, one chunk) touches distinct banks
// whether the LDS serves 8 lanes of a 16-byte read per cycle from 32 banks or
// 16 lanes from 64 banks.
constexpr int kRowBytes = kDtlBK * 2;
__device__ __forceinline__ int k_swz(int r) {
    if constexpr (kDtlBK == 64) return (r ^ (r >> 3)) & 7;
    else return ((r >> 1) ^ (r >> 3)) & 3;
}
__device__ __forceinline__ int k_off(int r, int c) {
    return r * kRowBytes + ((c ^ k_swz(r)) << 4);
}

// MN-contiguous tile of one step: [kDtlBK][256] bf16, 512-byte k-rows of 32
// chunks; chunk c of k-row k is stored at c ^ ((k & 3) << 2) ^ (((k >> 3) & 1) << 4).
// A transposing read touches k-rows {k0..k0+3} (and k0+8.. in the other half
// wave) x four consecutive chunks, which this places in distinct banks.
__device__ __forceinline__ int mn_off(int k, int m) {
    return (k << 9) + (((m >> 3) ^ ((k & 3) << 2) ^ (((k >> 3) & 1) << 4)) << 4) + ((m & 7) << 1);
}

// ---------------------------------------------------------------------------
// Direct-to-LDS loaders of one K step of a 256-row operand.  Only the first
// kLoaderWaves waves (one per SIMD) issue loads: NI instructions of 1 KiB each,
// instruction i of loader wave w filling LDS kilobyte w * NI + i of the tile.
// A wave waiting on a full texture-address queue stalls at issue; keeping the
// other wave of each SIMD free of loads lets it feed the matrix core meanwhile.
// ---------------------------------------------------------------------------
constexpr int kLoaderWaves = 4;
template <int ROWS, bool KMAJOR> struct DtlLoader;

template <int ROWS> struct DtlLoader<ROWS, true> {
    static_assert(ROWS == 256, "tile rows");
    static constexpr int NI = kDtlTile / 1024 / kLoaderWaves;
    static constexpr int RPK = 1024 / kRowBytes;                  // rows per kilobyte
    static constexpr int CPR = kRowBytes / 16;                    // chunks per row
    Operand op;
    uint64_t tile_off;   // byte offset of the tile's first row
    uint32_t voff[NI];   // lane offsets from (tile row 0, step k0)
    int kl[NI];          // element offset of this lane's chunk within the step
    int lds0;            // LDS byte offset of this wave's first kilobyte

    __device__ __forceinline__ void init(const Operand& o, int m0, int wave, int lane) {
        op = o;
        tile_off = (uint64_t)m0 * (uint64_t)o.ld * 2u;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int r = (wave * NI + i) * RPK + lane / CPR;
            const int c = (lane % CPR) ^ k_swz(r);                   // logical chunk at this lane's slot
            kl[i] = c * 8;
            voff[i] = (uint32_t)(((int64_t)r * o.ld + c * 8) * 2);
        }
        lds0 = wave * NI * 1024;
    }
    __device__ __forceinline__ void issue(lds_t* tile, int k0, int kend, bool full) {
        const u32x4 rs = window_rsrc(op, tile_off + (uint64_t)k0 * 2u);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const bool ok = full || (k0 + kl[i]) < kend;
            dtl_load16(rs, lds_addr_of(tile) + (uint32_t)(lds0 + i * 1024), ok ? voff[i] : kOOB);
        }
    }
    // fragment of 32 rows starting at row r0, sub-step s (k = 16 s .. 16 s + 15)
    static __device__ __forceinline__ u32x4 frag(const lds_t* tile, int r0, int s, int lane) {
        return lds_read16(tile, k_off(r0 + (lane & 31), 2 * s + (lane >> 5)));
    }
};

template <int ROWS> struct DtlLoader<ROWS, false> {
    static_assert(ROWS == 256, "MN-contiguous tiles are 256 wide (512-byte k-rows)");
    static constexpr int NI = kDtlTile / 1024 / kLoaderWaves;
    Operand op;
    uint64_t tile_off;   // byte offset of the tile's first column
    uint32_t voff[NI];   // lane offsets from (step k0, tile column 0)
    int kr[NI];          // k-row of this lane within the step
    int lds0;

    __device__ __forceinline__ void init(const Operand& o, int m0, int wave, int lane) {
        op = o;
        tile_off = (uint64_t)m0 * 2u;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int k = (wave * NI + i) * 2 + (lane >> 5);           // 2 k-rows per kilobyte
            const int c = (lane & 31) ^ ((k & 3) << 2) ^ (((k >> 3) & 1) << 4);
            kr[i] = k;
            voff[i] = (uint32_t)(((int64_t)k * o.ld + c * 8) * 2);
        }
        lds0 = wave * NI * 1024;
    }
    __device__ __forceinline__ void issue(lds_t* tile, int k0, int kend, bool full) {
        const u32x4 rs = window_rsrc(op, tile_off + (uint64_t)k0 * (uint64_t)op.ld * 2u);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const bool ok = full || (k0 + kr[i]) < kend;
            dtl_load16(rs, lds_addr_of(tile) + (uint32_t)(lds0 + i * 1024), ok ? voff[i] : kOOB);
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

// Barrier that orders the waves without a memory fence: the caller has
// already waited for exactly the loads it needs, and a fence would make the
// compiler wait for every outstanding load (including the prefetches).
__device__ __forceinline__ void wave_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

// LDS of the engine: one array per pipeline stage.
struct DtlStages {
    lds_t* st[kDtlStages];
};

template <int BM, int BN, bool A_KMAJOR, bool B_KMAJOR, class Epi>
__device__ __forceinline__ void gemm_body_dtl(const Operand& A, const Operand& B, const GemmGeom& g,
                                              const typename Epi::Params& ep, const DtlStages& lds) {
    static_assert(BM == 256 && BN == 256, "tile shape");
    constexpr int BK = kDtlBK;
    constexpr int kStages = kDtlStages;
    int tm, tn;
    if (!tile_of(g, tm, tn)) return;
    const int m0 = tm * BM, n0 = tn * BN;
    const int split = (int)blockIdx.y;
    const int kbeg = split * g.k_per_split;
    const int kend = min(g.K, kbeg + g.k_per_split);
    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;

    const bool loader = wave < kLoaderWaves;
    DtlLoader<BM, A_KMAJOR> la;
    DtlLoader<BN, B_KMAJOR> lb;
    if (loader) {
        la.init(A, m0, wave, lane);
        lb.init(B, n0, wave, lane);
    }
    using Mma = DtlMma<BM, BN>;
    Mma mma;
#pragma unroll
    for (int i = 0; i < Mma::FM; ++i)
#pragma unroll
        for (int j = 0; j < Mma::FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) mma.acc[i][j][e] = 0.f;

    auto issue = [&](lds_t* st, int step) {
        if (!loader) return;
        const int k0 = kbeg + step * BK;
        const bool full = k0 + BK <= kend;
        la.issue(st, k0, kend, full);
        lb.issue(st + kDtlTile, k0, kend, full);
    };
#pragma unroll
    for (int p = 0; p < kStages - 1; ++p)
        if (p < nk) issue(lds.st[p], p);
    const int am = wm * (BM / 2), bn = wn * (BN / 4);

    auto step = [&](int it, const lds_t* ta, lds_t* refill) {
        // this wave's loads of step `it` are in LDS once at most the younger
        // steps' loads are outstanding (2 * NI instructions per step and
        // loader wave; the other waves have none)
        const int younger = min(kStages - 2, nk - 1 - it);
        constexpr int per = 2 * DtlLoader<BM, A_KMAJOR>::NI;
        static_assert(DtlLoader<BM, A_KMAJOR>::NI == DtlLoader<BN, B_KMAJOR>::NI, "loads per step");
        if (younger >= 3)      __builtin_amdgcn_s_waitcnt(0x0F70 | (3 * per));
        else if (younger == 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * per));
        else if (younger == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | per);
        else                   __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        wave_barrier();         // every wave's loads of step `it` landed; step it-1's buffer is free
        if (it + kStages - 1 < nk) issue(refill, it + kStages - 1);
        const lds_t* tb = ta + kDtlTile;
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
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
    };
    // unrolled by the stage count so that every step names its stage arrays statically
    for (int it = 0; it < nk; it += kStages) {
#pragma unroll
        for (int u = 0; u < kStages; ++u)
            if (it + u < nk) step(it + u, lds.st[u], lds.st[(u + kStages - 1) % kStages]);
    }
    __syncthreads();   // LDS is reused by epilogues
    Epi::apply(mma, m0, n0, split, wm, wn, lane, tid, lds.st[0], ep);
}

}  // namespace kd

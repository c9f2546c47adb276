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
// Two schedules (a template switch, chosen per launch by the host): two LDS
// stages of one 64-deep K step each, one consumed while the loads of the other
// are in flight; or an operand ring of three A and two B tiles in the whole
// 160 KiB, which loads A tiles two steps ahead (see the main loops below).
#pragma once

#include <type_traits>

#include "kd_gemm.hpp"

namespace kd {

// Waves per workgroup: 8 (2 x 4, 128 x 64 per wave, two waves per SIMD) or 4
// (2 x 2, 128 x 128 per wave, one wave per SIMD, accumulators in AGPRs).  On
// the GPT-OSS-like step 4 waves measured 12-25% slower: with one wave per SIMD
// nothing covers its LDS waits, load issue and barrier skew.
constexpr int kDtlWaves = 8;
static_assert(kDtlWaves == 8 || kDtlWaves == 4, "waves per workgroup");
constexpr int kDtlThreads = 64 * kDtlWaves;

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
    // records = clamp(bytes - off, 0, 2^31 - 1), with 32-bit compares only (the
    // scalar unit has no 64-bit ordered compare)
    const uint64_t diff = (uint64_t)op.bytes - off;
    const int32_t hi = (int32_t)(diff >> 32);
    const uint32_t lo = (uint32_t)diff;
    const uint32_t rec = hi < 0 ? 0u : ((hi > 0 || lo > 0x7FFFFFFFu) ? 0x7FFFFFFFu : lo);
    return rsrc_words(reinterpret_cast<uint64_t>(op.ptr) + off, rec);
}

// One direct-to-LDS load: lane l's 16 bytes at byte offset `voff` of the
// buffer land at LDS byte address lds_addr + 16 l (out of range: zeros).  The
// instruction has no destination register; it is issued from asm so that the
// compiler does not add its own conservative vmcnt waits before unrelated LDS
// reads.  Completion is awaited explicitly with s_waitcnt vmcnt(N) before the
// barrier that publishes a stage.
__device__ __forceinline__ void dtl_load16(const u32x4& rsrc_in, uint32_t lds_addr_in, uint32_t voff) {
    // the descriptor and the LDS address are wave-uniform; make sure they live
    // in scalar registers (an "s" operand must not be given a vector register)
    const uint32_t lds_addr = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr_in);
    u32x4 rsrc;
#pragma unroll
    for (int w = 0; w < 4; ++w) rsrc[w] = (uint32_t)__builtin_amdgcn_readfirstlane((int)rsrc_in[w]);
    // m0 is declared clobbered: the compiler keeps none of its own values in it
    // across the block (and saves it only where it has one).  An SALU write of
    // m0 needs one wait state before an LDS-DMA load reads it (the compiler pads
    // its own such sequences with s_nop 0 on this target).  Clang warns that a
    // reserved register in a clobber list may not be preserved; the kernels
    // keep no value of their own in m0, which tests/test_static.py checks on
    // the compiled device code (every m0 write is this block's, directly
    // followed by its load, and nothing else reads m0), so only that warning
    // is silenced, here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen lds"
        :
        : "v"(voff), "s"(rsrc), "s"(lds_addr)
        : "memory", "m0");
#pragma clang diagnostic pop
}

// Hides a per-lane value from loop-invariant code motion: the compiler would
// otherwise precompute every load and fragment address of the main loop and
// run out of registers.
template <typename T> __device__ __forceinline__ void opaque(T& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ uint32_t lds_addr_of(const lds_t* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

__device__ __forceinline__ u32x2 lds_read8_tr(const lds_t* base, int off) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(const_cast<lds_t*>(base) + off));
    return __builtin_bit_cast(u32x2, v);
}

// K step of the engine (bf16 elements) and number of LDS stages.  A stage
// holds the A and B tiles of one step, 2 x 256 x BK x 2 bytes.  K step 32 with
// 4 or 5 stages (loads three or four steps ahead, spread evenly over the step)
// measured 3-15% slower than 64 with 2: the per-step barrier and the 64-byte
// row pieces of K-contiguous operands cost more than the deeper prefetch gains.
constexpr int kDtlBK = 64;
constexpr int kDtlStages = 2;
static_assert(kDtlBK == 32 || kDtlBK == 64, "K step");
static_assert(kDtlStages >= 2 && kDtlStages * 2 * 256 * kDtlBK * 2 <= 160 * 1024, "stages fit the LDS");
constexpr int kDtlSub = kDtlBK / 16;          // MFMA sub-steps (k = 16 each) per step
constexpr int kDtlTile = 256 * kDtlBK * 2;    // bytes of one operand tile per step

// K-contiguous tile of one step: [rows][BK] bf16, rows of kCh 16-byte chunks.
// Chunk c of row r is stored at c ^ k_swz(r), chosen so that a fragment read
// (32 consecutive rows, one chunk) touches distinct banks in every group of 16
// lanes (and of 8).
constexpr int kRowBytes = kDtlBK * 2;
constexpr int kCh = kDtlBK / 8;
__device__ __forceinline__ int k_swz(int r) {
    return kCh == 8 ? ((r ^ (r >> 3)) & 7) : (((r >> 1) ^ (r >> 3)) & 3);
}
__device__ __forceinline__ int k_off(int r, int c) {
    return r * kRowBytes + ((c ^ k_swz(r)) << 4);
}

// MN-contiguous tile of one step: [BK][256] bf16, 512-byte k-rows of 32
// chunks; chunk c of k-row k is stored at c ^ ((k & 3) << 2) ^ (((k >> 3) & 1) << 4).
// A transposing read touches k-rows {k0..k0+3} (and k0+8.. in the other half
// wave) x four consecutive chunks, which this places in distinct banks.
__device__ __forceinline__ int mn_off(int k, int m) {
    return (k << 9) + (((m >> 3) ^ ((k & 3) << 2) ^ (((k >> 3) & 1) << 4)) << 4) + ((m & 7) << 1);
}

// ---------------------------------------------------------------------------
// Direct-to-LDS loaders of one K step of a 256-row operand.  The first
// kLoaderWaves waves issue the loads: NI instructions of 1 KiB per operand and
// step, instruction i of loader wave w filling LDS kilobyte w * NI + i of the
// tile.  Instructions are issued one at a time between matrix instructions so
// that a wave waiting for room in the texture-address queue delays at most one
// of its MFMAs.
// ---------------------------------------------------------------------------
constexpr int kLoaderWaves = 4;

// BLOCKED operands are stored in blocks of 64 along one dimension with the
// other dimension's rows 128 bytes apart inside a block (Operand::kblock bytes
// from block to block): K-contiguous blocked = 64 k of every row per block;
// MN-contiguous blocked = 64 m of every k per block.
template <int ROWS, bool KMAJOR, bool BLOCKED = false> struct DtlLoader;

// K-contiguous operand.  An instruction covers RPI = 1024 / kRowBytes rows;
// instruction i of loader wave w covers tile rows RPI u .. RPI u + RPI - 1
// (u = w NI + i); lane l writes slot l % kCh of row RPI u + l / kCh, so it
// reads the logical chunk that the swizzle puts there.
template <int ROWS, bool BLOCKED> struct DtlLoader<ROWS, true, BLOCKED> {
    static_assert(ROWS == 256, "tile rows");
    static constexpr int NI = kDtlTile / 1024 / kLoaderWaves;
    static constexpr int RPI = 1024 / kRowBytes;   // rows per instruction (8 or 16)
    Operand op;
    uint64_t tile_off;   // byte offset of this wave's first row of the tile
    uint32_t lrow;       // byte offset of this lane's row within an instruction's rows
    int zl;              // lane part of the chunk index
    uint32_t voff[NI];   // this lane's byte offset for each instruction (the same every K step)

    __device__ __forceinline__ int chunk(int i, int wave) const {
        if constexpr (kCh == 8) return zl ^ i;
        else return zl ^ (2 * ((wave * NI + i) & 1));
    }
    __device__ __forceinline__ void init(const Operand& o, int m0, int wave, int lane) {
        op = o;
        tile_off = (uint64_t)m0 * (uint64_t)o.ld * 2u + (uint64_t)(wave * NI * RPI) * 2u * (uint64_t)o.ld;
        lrow = (uint32_t)(2 * (lane / kCh) * o.ld);
        // k_swz of row RPI u + l / kCh without the part that depends on u
        if constexpr (kCh == 8) zl = (lane & 7) ^ (lane >> 3) ^ ((wave * NI) & 7);
        else zl = (lane & 3) ^ ((lane >> 3) & 3) ^ (lane >> 5);
#pragma unroll
        for (int i = 0; i < NI; ++i)
            voff[i] = lrow + (uint32_t)(i * RPI * 2 * o.ld) + (uint32_t)(chunk(i, wave) << 4);
    }
    __device__ __forceinline__ u32x4 rsrc(int k0) const {
        // blocked: ld = 64 and k0 lies in block k0 / 64
        if constexpr (BLOCKED) return window_rsrc(op, tile_off + (uint64_t)(k0 >> 6) * op.kblock + (uint64_t)(k0 & 63) * 2u);
        else return window_rsrc(op, tile_off + (uint64_t)k0 * 2u);
    }
    __device__ __forceinline__ void hide() {
        opaque(lrow);
        opaque(zl);
    }
    // instruction i of the step at k0 into the tile at LDS byte address `tile`
    __device__ __forceinline__ void issue1(const u32x4& rs, uint32_t tile, int i, int k0, int kend, bool full,
                                           int wave) const {
        uint32_t v = voff[i];
        if (!full && k0 + chunk(i, wave) * 8 >= kend) v = kOOB;
        dtl_load16(rs, tile + (uint32_t)((wave * NI + i) * 1024), v);
    }
    // Fragment addresses: 32-row fragment f (rows base + 32 f ..) of sub-step
    // s (k = 16 s ..) is at off[s ^ 2 (f & 1)] + 4096 f (K step 64) or
    // off[s] + 2048 f (K step 32) for this lane.
    struct Frag {
        int off[kDtlSub];
    };
    static __device__ __forceinline__ Frag frag_addr(int base, int lane) {
        const int rowb = (base + (lane & 31)) * kRowBytes;
        Frag f;
        if constexpr (kCh == 8) {
            const int x = (lane >> 5) ^ (lane & 7) ^ ((lane >> 3) & 3);
#pragma unroll
            for (int y = 0; y < 4; ++y) f.off[y] = rowb + ((x ^ (2 * y)) << 4);
        } else {
            const int x = (lane >> 5) ^ (((lane >> 1) ^ (lane >> 3)) & 3);
#pragma unroll
            for (int y = 0; y < 2; ++y) f.off[y] = rowb + ((x ^ (2 * y)) << 4);
        }
        return f;
    }
    static __device__ __forceinline__ u32x4 frag(const lds_t* tile, const Frag& fa, int f, int s) {
        if constexpr (kCh == 8) return lds_read16(tile, fa.off[s ^ (2 * (f & 1))] + 4096 * f);
        else return lds_read16(tile, fa.off[s] + 2048 * f);
    }
};

// MN-contiguous operand.  Load instruction i of loader wave w covers k-rows
// 2 u and 2 u + 1 (u = w NI + i); lane l reads the 16 bytes of k-row
// 2 u + (l >> 5) whose chunk lands in slot l & 31 of that row.
template <int ROWS, bool BLOCKED> struct DtlLoader<ROWS, false, BLOCKED> {
    static_assert(ROWS == 256, "MN-contiguous tiles are 256 wide (512-byte k-rows)");
    // bytes between consecutive k-rows, and from one 8-chunk (64-element) group
    // of a k-row to the next
    __device__ __forceinline__ uint64_t krow() const { return BLOCKED ? 128u : (uint64_t)op.ld * 2u; }
    static constexpr int NI = kDtlTile / 1024 / kLoaderWaves;
    Operand op;
    uint64_t tile_off;   // byte offset of the tile's first column at this wave's first k-row
    uint32_t lrow;       // byte offset of this lane's k-row within an instruction
    int zl;              // lane part of the chunk index
    int kw;              // (w NI) / 4, whose parity enters the chunk swizzle
    int kl;              // this lane's k-row within an instruction (0 or 1)
    uint32_t voff[NI];   // this lane's byte offset for each instruction (the same every K step)

    __device__ __forceinline__ void init(const Operand& o, int m0, int wave, int lane) {
        op = o;
        if constexpr (BLOCKED) tile_off = (uint64_t)(m0 >> 6) * o.kblock + (uint64_t)(wave * NI) * 2u * 128u;
        else tile_off = (uint64_t)m0 * 2u + (uint64_t)(wave * NI) * 4u * (uint64_t)o.ld;
        kl = lane >> 5;
        lrow = (uint32_t)(kl * krow());
        zl = (lane & 31) ^ (kl << 2);
        kw = (wave * NI) >> 2;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int c = zl ^ (8 * (i & 1)) ^ (16 * ((kw + (i >> 2)) & 1));
            if constexpr (BLOCKED)
                voff[i] = lrow + (uint32_t)(i * 2 * 128) + (uint32_t)(c >> 3) * (uint32_t)o.kblock + (uint32_t)((c & 7) << 4);
            else
                voff[i] = lrow + (uint32_t)(i * 4 * o.ld) + (uint32_t)(c << 4);
        }
    }
    __device__ __forceinline__ u32x4 rsrc(int k0) const { return window_rsrc(op, tile_off + (uint64_t)k0 * krow()); }
    __device__ __forceinline__ void hide() {
        opaque(lrow);
        opaque(zl);
        opaque(kl);
    }
    __device__ __forceinline__ void issue1(const u32x4& rs, uint32_t tile, int i, int k0, int kend, bool full,
                                           int wave) const {
        uint32_t v = voff[i];
        if (!full && k0 + (wave * NI + i) * 2 + kl >= kend) v = kOOB;
        dtl_load16(rs, tile + (uint32_t)((wave * NI + i) * 1024), v);
    }
    // Fragment f (columns base + 32 f ..) of sub-step s: lane l gets
    // m = base + 32 f + (l & 31), k = 16 s + 8 (l >> 5) .. + 7, as two
    // transposing reads at off[f] + 8192 s and + 2048.
    struct Frag {
        int off[4];
    };
    static __device__ __forceinline__ Frag frag_addr(int base, int lane) {
        const int g = lane >> 4, i = lane & 15;
        Frag fa;
#pragma unroll
        for (int f = 0; f < 4; ++f) fa.off[f] = mn_off(8 * (g >> 1) + (i >> 2), base + 32 * f + 16 * (g & 1) + 4 * (i & 3));
        return fa;
    }
    static __device__ __forceinline__ u32x4 frag(const lds_t* tile, const Frag& fa, int f, int s) {
        const u32x2 lo = lds_read8_tr(tile, fa.off[f] + 8192 * s);
        const u32x2 hi = lds_read8_tr(tile, fa.off[f] + 8192 * s + 2048);
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
};

// Accumulators of one wave: (BM/2) x (BN/WN) as 32 x 32 fragments, the
// waves laid out 2 (M) x WN (N).
template <int BM, int BN> struct DtlMma {
    static constexpr int WN = kDtlWaves / 2;
    static constexpr int FM = BM / 64;          // 4
    static constexpr int FN = BN / WN / 32;     // 2 (8 waves) or 4 (4 waves)
    f32x16 acc[FM][FN];
    static __device__ __forceinline__ int row(int wm, int i, int q, int lane) {
        return wm * (BM / 2) + 32 * i + 8 * q + 4 * (lane >> 5);
    }
    static __device__ __forceinline__ int col(int wn, int j, int lane) {
        return wn * (BN / WN) + 32 * j + (lane & 31);
    }
};

// Barrier that orders the waves without a memory fence: the caller has
// already waited for exactly the loads it needs, and a fence would make the
// compiler wait for every outstanding load.
__device__ __forceinline__ void wave_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

// LDS of the engine's two schedules.
//
// Two-stage (RING = false): kDtlStages pipeline stages of kDtlStage bytes (A
// tile, then B tile); every load of a step has one step to land.
//
// Operand ring (RING = true): the A tiles of kDtlSlotsA consecutive steps, then
// the B tiles of kDtlSlotsB, one tile per slot (160 KiB with 3 + 2).  A tiles
// are loaded two steps ahead of their use, spread over the MFMAs of the
// preceding step's first SUB - 1 sub-steps; B tiles one step ahead, right after
// the barrier that frees their slot.  The deeper prefetch pays where operand
// slices come from HBM with little reuse and the contraction is latency-bound
// (short chunks: fewer rows share each W tile); where the part runs at its
// power limit (long chunks) the two-stage schedule is faster.
constexpr int kDtlStage = 2 * kDtlTile;
constexpr int kDtlLds = kDtlStages * kDtlStage;
static_assert(kDtlLds >= 128 * 1024, "the epilogues stage through 128 KiB of LDS");
constexpr int kDtlSlotsA = 3;
constexpr int kDtlSlotsB = 2;
constexpr int kDtlLdsRing = (kDtlSlotsA + kDtlSlotsB) * kDtlTile;
static_assert(kDtlLdsRing <= 160 * 1024 && kDtlLdsRing >= kDtlLds, "the ring fits the LDS");
template <bool RING> constexpr int dtl_lds_bytes() { return RING ? kDtlLdsRing : kDtlLds; }

// s_waitcnt immediate (gfx9): vmcnt (6 bits, split), expcnt 7, lgkmcnt.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

template <int N, class F> __device__ __forceinline__ void static_for(F&& f) {
    if constexpr (N > 0) {
        static_for<N - 1>(f);
        f(std::integral_constant<int, N - 1>{});
    }
}

// ---------------------------------------------------------------------------
// Main loop.  Per K step a wave runs kDtlSub sub-steps of FM x FN MFMAs; the
// operand fragments of sub-step s + 1 are read from LDS while the MFMAs of
// sub-step s run (two register sets), and the last sub-step's MFMAs run after
// the barrier that publishes the next stage, so they cover the latency of the
// next stage's first fragment reads.
//
// Two-stage schedule: step j lives in stage j mod NS.  The stage of step it is
// free once every wave has passed the barrier that ends step it's reads, so
// the loads of step j are issued partly on the MFMA group after the barrier
// that frees its stage (kPost instructions per loader wave) and the rest on
// the groups of the following step before its barrier; they have NS - 2
// further steps to land before the barrier that publishes step j.  The
// operand ring (RING) is described at its main loop.
// ---------------------------------------------------------------------------
template <int BM, int BN, bool A_KMAJOR, bool B_KMAJOR, bool B_BLOCKED, bool RING, class Epi>
__device__ __forceinline__ void gemm_body_dtl(const Operand& A, const Operand& B, const GemmGeom& g,
                                              const typename Epi::Params& ep, lds_t* smem) {
    static_assert(BM == 256 && BN == 256, "tile shape");
    constexpr int BK = kDtlBK, NS = kDtlStages, SUB = kDtlSub;
    // A and B slots: the two-stage schedule's stages, or the ring's 3 + 2
    constexpr int SA = RING ? kDtlSlotsA : NS, SB = RING ? kDtlSlotsB : NS;
    using LA = DtlLoader<BM, A_KMAJOR>;
    using LB = DtlLoader<BN, B_KMAJOR, B_BLOCKED>;
    using Mma = DtlMma<BM, BN>;
    constexpr int FM = Mma::FM, FN = Mma::FN, WN = Mma::WN;
    constexpr int NA = LA::NI, NB = LB::NI;      // load instructions per step and loader wave
    constexpr int NT = NA + NB;
    static_assert(!RING || 2 * NT <= 63, "vmcnt range");
    // two stages: every load rides on the group right after the barrier (the
    // earliest its stage is free; measured best); more stages: half and half
    constexpr int kPost = NS == 2 ? NT : NT / 2;
    static_assert(kPost >= 0 && kPost <= NT, "load shares");
    constexpr int kPre = NT - kPost;             // spread over the SUB - 1 groups before the barrier
    // loads issued after the last one of step it + 1 when the barrier ending
    // step it is reached in the steady state
    constexpr int kAhead = (NS - 2) * NT;
    static_assert(kAhead + kPost <= 63, "vmcnt range");

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
    const int wm = wave / WN, wn = wave % WN;
    const bool loader = wave < kLoaderWaves;

    LA la;
    LB lb;
    if (loader) {
        la.init(A, m0, wave, lane);
        lb.init(B, n0, wave, lane);
    }
    Mma mma;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) mma.acc[i][j][e] = 0.f;

    // LDS layout: A slot s at s * kDtlTile, B slot s at (SA + s) * kDtlTile
    // (two-stage: stage s holds A slot s and B slot s).  The B fragment offsets
    // carry the SA * kDtlTile, so both operands are read from a slot base plus
    // a per-lane offset and a constant: with the slots known at compile time
    // (the main loop is unrolled over the slots' period) the constants become
    // the LDS instructions' immediate offsets and no address is recomputed per
    // step.
    typename LA::Frag fa = LA::frag_addr(wm * (BM / 2), lane);
    typename LB::Frag fb = LB::frag_addr(wn * (BN / WN), lane);
#pragma unroll
    for (int y = 0; y < (int)(sizeof(fb.off) / sizeof(int)); ++y) fb.off[y] += SA * kDtlTile;
    struct Frags {
        u32x4 a[FM], b[FN];
    };
    auto a_tile = [&](int step) { return smem + (int)((unsigned)step % (unsigned)SA) * kDtlTile; };
    auto b_tile = [&](int step) { return smem + (SA + (int)((unsigned)step % (unsigned)SB)) * kDtlTile; };
    // FMV: fragments of this wave's rows that hold output rows below M (the
    // others are neither read nor multiplied); sa, sb: the step's A and B slots
    // (constants in the unrolled main loop; the B fragment offsets already
    // carry the A slots' extent)
    auto read = [&](Frags& f, int sa, int sb, int s, auto fmv_c) {
        constexpr int FMV = decltype(fmv_c)::value;
        if constexpr (FMV == 0) return;
        const lds_t* base_a = smem + sa * kDtlTile;
        const lds_t* base_b = smem + sb * kDtlTile;
#pragma unroll
        for (int i = 0; i < FMV; ++i) f.a[i] = LA::frag(base_a, fa, i, s);
#pragma unroll
        for (int j = 0; j < FN; ++j) f.b[j] = LB::frag(base_b, fb, j, s);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto mfma1 = [&](const Frags& f, int q) {
        const int i = q / FN, j = q % FN;
        mma.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.a[i]),
                                                               __builtin_bit_cast(bf16x8, f.b[j]), mma.acc[i][j], 0, 0, 0);
    };
    // the loads of one step
    struct Pending {
        u32x4 ra, rb;
        uint32_t tile, tileb;   // LDS byte addresses of the step's A and B tiles
        int k0;
        bool full;
    };
    auto pending_for = [&](int step) {
        Pending p;
        p.k0 = kbeg + step * BK;
        p.full = p.k0 + BK <= kend;
        p.ra = la.rsrc(p.k0);
        p.rb = lb.rsrc(p.k0);
        p.tile = lds_addr_of(a_tile(step));
        p.tileb = lds_addr_of(b_tile(step));
        return p;
    };
    // WHOLE: this workgroup's K range is a whole number of steps, so no load
    // needs the K-tail check (compile-time, so the checks vanish)
    auto load1 = [&](const Pending& p, int q, auto WHOLE) {
        const bool full = decltype(WHOLE)::value || p.full;
        if (q < NA) la.issue1(p.ra, p.tile, q, p.k0, kend, full, wave);
        else        lb.issue1(p.rb, p.tileb, q - NA, p.k0, kend, full, wave);
    };
    // one MFMA group carrying load instructions first .. first + CNT - 1
    auto group = [&](const Frags& f, auto with_loads, const Pending& p, auto first_c, auto cnt_c, auto fmv_c,
                     auto WHOLE) {
        constexpr int first = decltype(first_c)::value, CNT = decltype(cnt_c)::value;
        constexpr int NQ = decltype(fmv_c)::value * FN;
        if constexpr (decltype(with_loads)::value && CNT > 0) {
            if constexpr (NQ == 0) {
#pragma unroll
                for (int t = 0; t < CNT; ++t) load1(p, first + t, WHOLE);
            } else {
                // load t follows MFMA (t * NQ) / CNT
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    mfma1(f, q);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int t = 0; t < CNT; ++t)
                        if ((t * NQ) / CNT == q) load1(p, first + t, WHOLE);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < NQ; ++q) mfma1(f, q);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    using Z = std::integral_constant<int, 0>;

    // Main loop of one wave, two-stage schedule; LOADS: this wave issues loads.
    auto run2 = [&](auto LOADS, auto FMVc, auto WHOLE) {
        constexpr bool loads = decltype(LOADS)::value;
        Frags f0, f1;
        if constexpr (loads) {
            // steps 0 .. NS - 2, and the share of step NS - 1 that would have
            // ridden on the group after the barrier before step 0
#pragma unroll
            for (int j = 0; j + 1 < NS; ++j) {
                if (j < nk) {
                    const Pending p = pending_for(j);
#pragma unroll
                    for (int q = 0; q < NT; ++q) load1(p, q, WHOLE);
                }
            }
            if (NS - 1 < nk) {
                const Pending p = pending_for(NS - 1);
#pragma unroll
                for (int q = 0; q < kPost; ++q) load1(p, q, WHOLE);
                __builtin_amdgcn_s_waitcnt(waitcnt_imm(kAhead + kPost, 15));   // step 0 landed
            } else {
                __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
            }
        }
        wave_barrier();
        read(f0, 0, 0, 0, FMVc);
        // One K step.  PRE / POST: the groups before / after this step's
        // barrier carry loads of step it + NS - 1 / it + NS (compile-time, so
        // the MFMA groups stay free of branches); ps = it mod NS.
        auto body = [&](auto PRE, auto POST, int it, int ps) {
            la.hide();
            lb.hide();
#pragma unroll
            for (int y = 0; y < (int)(sizeof(fa.off) / sizeof(int)); ++y) opaque(fa.off[y]);
#pragma unroll
            for (int y = 0; y < (int)(sizeof(fb.off) / sizeof(int)); ++y) opaque(fb.off[y]);
            constexpr bool pre = decltype(PRE)::value && loads && kPre > 0;
            constexpr bool post = decltype(POST)::value && loads && kPost > 0;
            Pending pp{}, pq{};
            if constexpr (pre) pp = pending_for(it + NS - 1);   // its stage is free since the last barrier
            // sub-steps 0 .. SUB - 2: read the next sub-step's fragments, then
            // the MFMAs of this one with a share of the loads
            static_for<SUB - 1>([&](auto S) {
                constexpr int s = decltype(S)::value;
                constexpr int lo = kPost + (s * kPre) / (SUB - 1);
                constexpr int hi = kPost + ((s + 1) * kPre) / (SUB - 1);
                using First = std::integral_constant<int, lo>;
                using Cnt = std::integral_constant<int, hi - lo>;
                if constexpr (s % 2 == 0) {
                    read(f1, ps, ps, s + 1, FMVc);
                    group(f0, std::integral_constant<bool, pre>{}, pp, First{}, Cnt{}, FMVc, WHOLE);
                } else {
                    read(f0, ps, ps, s + 1, FMVc);
                    group(f1, std::integral_constant<bool, pre>{}, pp, First{}, Cnt{}, FMVc, WHOLE);
                }
            });
            static_assert(SUB % 2 == 0, "the last sub-step uses the second register set");
            if (it + 1 < nk) {
                // this wave's loads of step it + 1 and its reads of `cur` are complete
                if constexpr (decltype(PRE)::value) __builtin_amdgcn_s_waitcnt(waitcnt_imm(kAhead, 0));
                else __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
                wave_barrier();                       // every wave's loads landed; stage ps is free
                const int pn = ps + 1 == NS ? 0 : ps + 1;
                read(f0, pn, pn, 0, FMVc);
            }
            if constexpr (post) pq = pending_for(it + NS);
            // sub-step SUB - 1
            group(f1, std::integral_constant<bool, post>{}, pq, Z{}, std::integral_constant<int, kPost>{}, FMVc, WHOLE);
        };
        const std::true_type yes{};
        const std::false_type no{};
        auto stage_of = [&](int it) { return (int)((unsigned)it % (unsigned)NS); };
        int it = 0;
        for (; it + 2 * NS - 1 < nk; it += NS)
            static_for<NS>([&](auto P) { body(yes, yes, it + decltype(P)::value, decltype(P)::value); });
        for (; it + NS < nk; ++it) body(yes, yes, it, stage_of(it));
        if (it + NS - 1 < nk) {
            body(yes, no, it, stage_of(it));
            ++it;
        }
        for (; it < nk; ++it) body(no, no, it, stage_of(it));
    };

    // Main loop of one wave, operand ring: step j's A tile in A slot j mod SA,
    // its B tile in B slot j mod SB.  The barrier inside step it (after its
    // last fragment reads) frees step it's slots.  The loader waves issue
    // A(it + 2) over the MFMAs of step it's first SUB - 1 sub-steps (its slot
    // was freed by the previous barrier) and B(it + 2) over the last
    // sub-step's, right after the barrier.  At the wait before the barrier of
    // step it everything up to B(it + 1) has landed; only A(it + 2) may still
    // be in flight.
    auto runr = [&](auto LOADS, auto FMVc, auto WHOLE) {
        constexpr bool loads = decltype(LOADS)::value;
        Frags f0, f1;
        if constexpr (loads) {
            // steps 0 and 1 (A then B each), before the first barrier
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (j < nk) {
                    const Pending p = pending_for(j);
#pragma unroll
                    for (int q = 0; q < NT; ++q) load1(p, q, WHOLE);
                }
            }
            // step 0 landed (step 1's loads may be in flight)
            if (1 < nk) __builtin_amdgcn_s_waitcnt(waitcnt_imm(NT, 15));
            else __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
        }
        wave_barrier();
        read(f0, 0, 0, 0, FMVc);
        // One K step.  LD: step it + 2 exists, so this step carries its loads
        // (compile-time, so the MFMA groups stay free of branches); sa, sb:
        // slots of step it.
        auto body = [&](auto LD, int it, int sa, int sb) {
            la.hide();
            lb.hide();
#pragma unroll
            for (int y = 0; y < (int)(sizeof(fa.off) / sizeof(int)); ++y) opaque(fa.off[y]);
#pragma unroll
            for (int y = 0; y < (int)(sizeof(fb.off) / sizeof(int)); ++y) opaque(fb.off[y]);
            constexpr bool ld = decltype(LD)::value && loads;
            Pending pp{};
            if constexpr (ld) pp = pending_for(it + 2);
            // sub-steps 0 .. SUB - 2: read the next sub-step's fragments, then
            // this one's MFMAs with a share of A(it + 2)'s loads
            static_for<SUB - 1>([&](auto S) {
                constexpr int s = decltype(S)::value;
                using First = std::integral_constant<int, (s * NA) / (SUB - 1)>;
                using Cnt = std::integral_constant<int, ((s + 1) * NA) / (SUB - 1) - (s * NA) / (SUB - 1)>;
                if constexpr (s % 2 == 0) {
                    read(f1, sa, sb, s + 1, FMVc);
                    group(f0, std::integral_constant<bool, ld>{}, pp, First{}, Cnt{}, FMVc, WHOLE);
                } else {
                    read(f0, sa, sb, s + 1, FMVc);
                    group(f1, std::integral_constant<bool, ld>{}, pp, First{}, Cnt{}, FMVc, WHOLE);
                }
            });
            static_assert(SUB % 2 == 0, "the last sub-step uses the second register set");
            if (it + 1 < nk) {
                // this wave's loads of step it + 1 and its reads of step it are
                // complete (A(it + 2) may still be in flight)
                if constexpr (decltype(LD)::value) __builtin_amdgcn_s_waitcnt(waitcnt_imm(NA, 0));
                else __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
                wave_barrier();                       // every wave's loads landed; step it's slots are free
                read(f0, sa + 1 == SA ? 0 : sa + 1, sb + 1 == SB ? 0 : sb + 1, 0, FMVc);
            }
            // sub-step SUB - 1 with B(it + 2)'s loads (its slot was freed just now)
            group(f1, std::integral_constant<bool, ld>{}, pp, std::integral_constant<int, NA>{},
                  std::integral_constant<int, NB>{}, FMVc, WHOLE);
        };
        const std::true_type yes{};
        const std::false_type no{};
        constexpr int P = SA * SB;   // both slot indices repeat every SA * SB steps
        int it = 0;
        for (; it + P + 1 < nk; it += P)
            static_for<P>([&](auto Q) {
                constexpr int q = decltype(Q)::value;
                body(yes, it + q, q % SA, q % SB);
            });
        for (; it + 2 < nk; ++it) body(yes, it, it % SA, it % SB);
        for (; it < nk; ++it) body(no, it, it % SA, it % SB);
    };
    auto run = [&](auto LOADS, auto FMVc, auto WHOLE) {
        if constexpr (RING) runr(LOADS, FMVc, WHOLE);
        else run2(LOADS, FMVc, WHOLE);
    };
    if (nk > 0) {
        // rows of this wave's half below M: all (4 fragments), at most 64 (2)
        // or none (0) -- the last is the hidden-size tail of d = 2880 at
        // 256-row tiles, a sixteenth of the two gradient contractions
        const int rem = g.M - m0 - wm * (BM / 2);
        const int fmv = rem > 64 ? 4 : (rem > 0 ? 2 : 0);
        using F4 = std::integral_constant<int, 4>;
        using F2 = std::integral_constant<int, 2>;
        auto dispatch = [&](auto LOADS, auto WHOLE) {
            if (fmv == 4)      run(LOADS, F4{}, WHOLE);
            else if (fmv == 2) run(LOADS, F2{}, WHOLE);
            else               run(LOADS, Z{}, WHOLE);
        };
        const bool whole = (kend - kbeg) % BK == 0;
        if (!loader)    dispatch(std::false_type{}, std::false_type{});
        else if (whole) dispatch(std::true_type{}, std::true_type{});
        else            dispatch(std::true_type{}, std::false_type{});
    }
    // An epilogue that reuses the stage LDS synchronises the workgroup itself
    // before its first LDS write (other waves may still be reading fragments);
    // work before that point overlaps the other waves' last MFMAs.
    Epi::apply(mma, m0, n0, split, wm, wn, lane, tid, smem, ep);
}

}  // namespace kd

// Measurement probe (not part of the loss): the sustained bf16 MFMA rate and
// shader clock of the whole part, with no global memory traffic.
//
// Every workgroup has 8 waves (two per SIMD) and each wave keeps the engine's
// 128 x 64 output block: 8 accumulators of v_mfma_f32_32x32x16_bf16 fed by 4 A
// and 2 B fragments.  The operand bits decide how much the part draws, so the
// probe runs three kinds of operands:
//   mode 0  constant fragments held in registers (random bits, fixed for the
//           whole run: only the accumulators change);
//   mode 1  fragments that change every step in registers: a Weyl sequence per
//           dword (every bit toggles), with bit 14 of each bf16 cleared so the
//           values stay finite;
//   mode 2  random bf16 fragments (random sign and mantissa, exponent 120..127)
//           read from LDS with ds_read_b128 in the engine's pattern, 6 KiB per
//           wave per 8 MFMAs, next step's fragments read while this step's
//           MFMAs run (two register sets);
//   mode 3  constant fragments of few set bits (1.0, 0.5 and 0.25 in bf16)
//           held in registers.
// Each workgroup records its elapsed shader cycles (s_memtime) and real time
// (s_memrealtime, 100 MHz), so the host gets the clock the launch ran at.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace kdprobe {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kThreads = 512;
constexpr int kLds = 65536;

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
    // an integer hash (xor-shift / multiply rounds) for the LDS operand fill
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void mfma_rate_kernel(float* sink, unsigned long long* cycles, int iters) {
    __shared__ __attribute__((aligned(16))) char smem[kLds];
    const int lane = threadIdx.x & 63;
    for (int i = threadIdx.x; i < kLds / 16; i += kThreads) {
        u32x4 v;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t x = mix32((uint32_t)(i * 4 + w) ^ (blockIdx.x * 0x9E3779B9u));
            v[w] = (x & 0x807F807Fu) | 0x3C003C00u | ((x >> 4) & 0x03800380u);
        }
        reinterpret_cast<u32x4*>(smem)[i] = v;
    }
    __syncthreads();

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    auto frag = [&](int step, int f) {   // fragment f (0..5) of a step, 16 bytes per lane
        return *reinterpret_cast<const u32x4*>(smem + (((step * 6 + f) * 1024 + lane * 16) & (kLds - 1)));
    };
    auto mfmas = [&](const u32x4* a, const u32x4* b) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                                   __builtin_bit_cast(bf16x8, b[j]), acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    u32x4 a[4], b[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = frag(0, i);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = frag(0, 4 + j);
    if constexpr (MODE == 3) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = u32x4{0x3F803F80u, 0x3F003F00u, 0x3E803E80u, 0x3F803F00u};
#pragma unroll
        for (int j = 0; j < 2; ++j) b[j] = u32x4{0x3F003F80u, 0x3E803F80u, 0x3F803F80u, 0x3F003E80u};
    }

    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    if constexpr (MODE == 2) {
        u32x4 c[4], e[2];
        for (int it = 0; it < iters; it += 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) c[i] = frag(it + 1, i);
#pragma unroll
            for (int j = 0; j < 2; ++j) e[j] = frag(it + 1, 4 + j);
            __builtin_amdgcn_sched_barrier(0);
            mfmas(a, b);
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = frag(it + 2, i);
#pragma unroll
            for (int j = 0; j < 2; ++j) b[j] = frag(it + 2, 4 + j);
            __builtin_amdgcn_sched_barrier(0);
            mfmas(c, e);
        }
    } else {
        for (int it = 0; it < iters; ++it) {
            mfmas(a, b);
            if constexpr (MODE == 1) {
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = (a[i] + 0x9E3779B9u) & 0xBFFFBFFFu;
#pragma unroll
                for (int j = 0; j < 2; ++j) b[j] = (b[j] + 0x7F4A7C15u) & 0xBFFFBFFFu;
            }
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();

    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) s += acc[i][j][e];
    sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        cycles[2 * blockIdx.x] = t1 - t0;
        cycles[2 * blockIdx.x + 1] = r1 - r0;
    }
}

}  // namespace kdprobe

// Launches the probe on `stream`: `workgroups` workgroups of 512 threads, each
// running `iters` steps of 8 MFMAs per wave (even `iters` for mode 2).  The
// caller owns `sink` (workgroups * 512 floats) and `cycles` (workgroups * 2:
// shader cycles and 100 MHz ticks per workgroup).  FLOP per launch =
// workgroups * 8 waves * iters * 8 MFMAs * 32,768.  Returns a hipError_t.
extern "C" int kd_probe_mfma_launch(int mode, int workgroups, int iters, float* sink, unsigned long long* cycles,
                                    void* stream) {
    if (workgroups < 1 || iters < 2 || (iters & 1) || !sink || !cycles || mode < 0 || mode > 3)
        return (int)hipErrorInvalidValue;
    const hipStream_t s = (hipStream_t)stream;
    const dim3 grid(workgroups), block(kdprobe::kThreads);
    if (mode == 0) hipLaunchKernelGGL(kdprobe::mfma_rate_kernel<0>, grid, block, 0, s, sink, cycles, iters);
    else if (mode == 1) hipLaunchKernelGGL(kdprobe::mfma_rate_kernel<1>, grid, block, 0, s, sink, cycles, iters);
    else if (mode == 2) hipLaunchKernelGGL(kdprobe::mfma_rate_kernel<2>, grid, block, 0, s, sink, cycles, iters);
    else hipLaunchKernelGGL(kdprobe::mfma_rate_kernel<3>, grid, block, 0, s, sink, cycles, iters);
    return (int)hipGetLastError();
}

// calib_mfma.hip -- measurement aid beside the quantized-GEMM library: the
// scaled FP4 MFMA rate the card sustains on random operands under its power
// limit, and the shader clock meanwhile (include/fp4_calib.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4_calib.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// The Wgrad GEMM's wave tile: 7 x 2 accumulator tiles of 32 x 32, two
// fragment sets (even and odd k-steps).
constexpr int FM = 7, FN = 2, NSET = 2;
constexpr int kFrags = NSET * (FM + FN);     // 16-byte fragments per lane
constexpr int kWaves = 4;

__global__ __launch_bounds__(64 * kWaves) void mfma_loop(const v4i* __restrict__ src, int iters,
                                                         float* __restrict__ out,
                                                         uint64_t* __restrict__ clocks) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    const v4i* p = src + wave * kFrags * 64 + lane;
    v4i fa[NSET][FM], fb[NSET][FN];
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[s][i] = p[(s * (FM + FN) + i) * 64];
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[s][j] = p[(s * (FM + FN) + FM + j) * 64];
    }
    v16f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < NSET; ++s)
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const v8i a = __builtin_shufflevector(fa[s][i], v4i{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const v8i b = __builtin_shufflevector(fb[s][j], v4i{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, acc[i][j], 4, 4, 0,
                                                                                127, 0, 127);
                }
            }
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) sum += acc[i][j][r];
    out[wave * 64 + lane] = sum;
    if (lane == 0) {
        clocks[2 * wave] = t1 - t0;
        clocks[2 * wave + 1] = r1 - r0;
    }
}

}  // namespace

extern "C" size_t fp4_calib_mfma_src_bytes(int grid) {
    return grid <= 0 ? 0 : (size_t)grid * kWaves * kFrags * 64 * 16;
}

extern "C" double fp4_calib_mfma_flops(int grid, int iters) {
    if (grid <= 0 || iters <= 0) return 0.0;
    return 2.0 * 32 * 32 * 64 * (double)(NSET * FM * FN) * iters * (double)grid * kWaves;
}

extern "C" int fp4_calib_mfma(const void* src, int grid, int iters, float* out, uint64_t* clocks,
                              void* stream) {
    if (!src || !out || !clocks) return 1;
    if (grid < 1 || grid > 65536 || iters < 1 || iters > (1 << 24)) return 2;
    if (((uintptr_t)src | (uintptr_t)out | (uintptr_t)clocks) & 15) return 3;
    const v4i* s = (const v4i*)src;
    void* args[] = {(void*)&s, (void*)&iters, (void*)&out, (void*)&clocks};
    // the status of this launch alone (not an earlier call's, as hipGetLastError)
    return hipLaunchKernel((const void*)mfma_loop, dim3((unsigned)grid), dim3(64 * kWaves), args, 0,
                           (hipStream_t)stream) == hipSuccess ? 0 : 5;
}

namespace {
// One record per workgroup: shader-clock counter, 100 MHz reference
// counter, and the id of the XCD (accelerator complex die) it ran on -- the
// shader-clock counters of different XCDs are not one clock, so a span is
// read only between two records of the same XCD.
__global__ void clock_stamp(uint64_t* out) {
    if (threadIdx.x == 0) {
        uint64_t* r = out + 4 * blockIdx.x;
        r[0] = __builtin_amdgcn_s_memtime();
        r[1] = __builtin_amdgcn_s_memrealtime();
        r[2] = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 15;   // HW_REG_XCC_ID[3:0]
        r[3] = 0;
    }
}
}  // namespace

extern "C" int fp4_calib_clock_stamp(uint64_t* out, void* stream) {
    if (!out) return 1;
    if ((uintptr_t)out & 7) return 3;
    void* args[] = {(void*)&out};
    return hipLaunchKernel((const void*)clock_stamp, dim3(FP4_CALIB_STAMPS), dim3(64), args, 0,
                           (hipStream_t)stream) == hipSuccess ? 0 : 5;
}

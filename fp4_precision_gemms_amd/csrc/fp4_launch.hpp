// fp4_launch.hpp -- internal launchers behind the C ABI (validated arguments
// only; every pointer and size has been checked by the caller).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

namespace fp4dev {

// Launches kernel k with the arguments converted to its parameter types and
// returns the status of this launch alone (hipLaunchKernel), not an error
// left over from earlier runtime calls as hipGetLastError would.
template <typename... P, typename... A>
inline hipError_t launch(void (*k)(P...), dim3 grid, dim3 block, hipStream_t st, A... a) {
    static_assert(sizeof...(P) == sizeof...(A), "argument count");
    std::tuple<P...> v(static_cast<P>(a)...);
    return std::apply(
        [&](auto&... e) {
            void* args[] = {(void*)&e..., nullptr};
            return hipLaunchKernel((const void*)k, grid, block, args, 0, st);
        },
        v);
}

// MXFP4 quantization of bf16 x[rows, cols] along axis 0 (cols) or 1 (rows).
hipError_t launch_quant_mx(const void* x, int64_t rows, int64_t cols, int axis, int had_n, int had,
                           uint64_t sign_seed, int rnd, uint64_t sr_seed, uint8_t* codes,
                           uint8_t* scales, hipStream_t st);

// Both MXFP4 quantizations of x from one read: along rows (codes_r/scales_r,
// as axis 1) and along cols (codes_c/scales_c, as axis 0), each with its own
// rotation and rounding.  Needs rows % 32 == 0 and cols % 32 == 0.
hipError_t launch_quant_mx_dual(const void* x, int64_t rows, int64_t cols, int had_n_r, int had_r,
                                uint64_t sign_seed_r, int rnd_r, uint64_t sr_seed_r, uint8_t* codes_r,
                                uint8_t* scales_r, int had_n_c, int had_c, uint64_t sign_seed_c,
                                int rnd_c, uint64_t sr_seed_c, uint8_t* codes_c, uint8_t* scales_c,
                                hipStream_t st);

// The two Wgrad operands a [rows, n1] and b [rows, n2] quantized along rows
// with one rotation (own SR seeds), in one launch when it fits.
hipError_t launch_quant_mx_pair(const void* a, int64_t rows, int64_t n1, const void* b, int64_t n2,
                                int had_n, int had, uint64_t sign_seed, int rnd, uint64_t sr_a,
                                uint64_t sr_b, uint8_t* qa, uint8_t* sa, uint8_t* qb, uint8_t* sb,
                                hipStream_t st);

// C[M, N] (row-major; fp32, or bf16 when out_bf16) = A[M, K] B[N, K]^T
// (+ C when accumulate) over MXFP4 operands.
hipError_t launch_gemm_mx(const uint8_t* aq, const uint8_t* as, const uint8_t* bq,
                          const uint8_t* bs, int64_t M, int64_t N, int64_t K, void* c,
                          int out_bf16, int accumulate, hipStream_t st);

// NVFP4 quantization (mode: 0 RTN, 1 renormalized scales by SR, 2 element
// SR); amax_dev is either the caller's amax_in or the workspace the amax pass
// writes.
hipError_t launch_nvfp4(const void* x, int64_t rows, int64_t cols, int had, uint64_t sign_seed,
                        int mode, uint64_t sr_seed, const float* amax_in, uint8_t* codes,
                        uint8_t* scales, float* tensor_scale, void* workspace, hipStream_t st);

// Device address and size of this device's scratch array (the current
// device; looked up once per device, thread-safe).
hipError_t nvfp4_scratch(void** ptr, size_t* bytes);

uint32_t host_sign_word(int had, uint64_t seed);

}  // namespace fp4dev

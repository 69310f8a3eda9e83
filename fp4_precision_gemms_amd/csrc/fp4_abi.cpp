// fp4_abi.cpp -- the C ABI of libfp4.so (declared in include/fp4.h):
// argument validation, then dispatch to the HIP launchers.  No HIP call is
// made before every argument has been checked, so error paths can be
// exercised on machines without a GPU.
#include "fp4.h"

#include <hip/hip_runtime.h>

#include "fp4_launch.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// a * b stays far from int64 overflow (byte counts of bf16 / fp32 tensors)
bool product_ok(int64_t a, int64_t b) { return a > 0 && b > 0 && a <= (INT64_C(1) << 60) / b; }

constexpr int64_t kMaxContraction = INT64_C(1) << 24;
constexpr int64_t kMaxTiles = INT64_C(1) << 24;

fp4_status from_hip(hipError_t e) { return e == hipSuccess ? FP4_OK : FP4_ERR_LAUNCH; }

fp4_status check_gemm(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs,
                      const void* c, int64_t M, int64_t N, int64_t K) {
    if (!aq || !as || !bq || !bs || !c) return FP4_ERR_NULL;
    if (M <= 0 || N <= 0 || K <= 0 || K % 32) return FP4_ERR_SHAPE;
    if (!product_ok(M, K) || !product_ok(N, K) || !product_ok(M, N) || M > INT32_MAX ||
        N > INT32_MAX)
        return FP4_ERR_SHAPE;
    // the kernel addresses a 256-row operand tile with 32-bit byte offsets
    // and launches one workgroup per 256 x 256 output tile
    if (K >= kMaxContraction || ((M + 255) / 256) * ((N + 255) / 256) >= kMaxTiles)
        return FP4_ERR_SHAPE;
    if (!aligned16(aq) || !aligned16(as) || !aligned16(bq) || !aligned16(bs) || !aligned16(c))
        return FP4_ERR_ALIGN;
    return FP4_OK;
}

fp4_status run_gemm(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs,
                    int64_t M, int64_t N, int64_t K, void* c, int out_bf16, int accumulate,
                    void* stream) {
    const fp4_status s = check_gemm(aq, as, bq, bs, c, M, N, K);
    if (s != FP4_OK) return s;
    return from_hip(fp4dev::launch_gemm_mx(aq, as, bq, bs, M, N, K, c, out_bf16, accumulate,
                                           (hipStream_t)stream));
}

}  // namespace

extern "C" {

fp4_status fp4_hadamard_quantize(const void* x_bf16, int64_t rows, int64_t cols, fp4_axis axis,
                                 int had_n, fp4_hadamard had, uint64_t sign_seed, fp4_rounding rnd,
                                 uint64_t sr_seed, uint8_t* codes, uint8_t* scales_e8m0,
                                 void* stream) {
    if (axis != FP4_AXIS_COLS && axis != FP4_AXIS_ROWS) return FP4_ERR_ENUM;
    if (had != FP4_HAD_NONE && had != FP4_HAD_DET && had != FP4_HAD_SIGNED) return FP4_ERR_ENUM;
    if (had != FP4_HAD_NONE && had_n != 16 && had_n != 32) return FP4_ERR_ENUM;
    if (rnd != FP4_RTN && rnd != FP4_SR) return FP4_ERR_ENUM;
    if (!x_bf16 || !codes || !scales_e8m0) return FP4_ERR_NULL;
    if (rows <= 0 || cols <= 0 || !product_ok(rows, cols)) return FP4_ERR_SHAPE;
    const int64_t contraction = axis == FP4_AXIS_COLS ? cols : rows;
    if (contraction % 32) return FP4_ERR_SHAPE;
    if (!aligned16(x_bf16) || !aligned16(codes) || !aligned16(scales_e8m0)) return FP4_ERR_ALIGN;
    return from_hip(fp4dev::launch_quant_mx(x_bf16, rows, cols, (int)axis, had_n, (int)had,
                                            sign_seed, (int)rnd, sr_seed, codes, scales_e8m0,
                                            (hipStream_t)stream));
}

fp4_status fp4_hadamard_quantize_dual(const void* x_bf16, int64_t rows, int64_t cols,
                                      int had_n_rows, fp4_hadamard had_rows, uint64_t sign_seed_rows,
                                      fp4_rounding rnd_rows, uint64_t sr_seed_rows,
                                      uint8_t* codes_rows, uint8_t* scales_rows, int had_n_cols,
                                      fp4_hadamard had_cols, uint64_t sign_seed_cols,
                                      fp4_rounding rnd_cols, uint64_t sr_seed_cols,
                                      uint8_t* codes_cols, uint8_t* scales_cols, void* stream) {
    for (const fp4_hadamard h : {had_rows, had_cols})
        if (h != FP4_HAD_NONE && h != FP4_HAD_DET && h != FP4_HAD_SIGNED) return FP4_ERR_ENUM;
    if (had_rows != FP4_HAD_NONE && had_n_rows != 16 && had_n_rows != 32) return FP4_ERR_ENUM;
    if (had_cols != FP4_HAD_NONE && had_n_cols != 16 && had_n_cols != 32) return FP4_ERR_ENUM;
    for (const fp4_rounding r : {rnd_rows, rnd_cols})
        if (r != FP4_RTN && r != FP4_SR) return FP4_ERR_ENUM;
    if (!x_bf16 || !codes_rows || !scales_rows || !codes_cols || !scales_cols) return FP4_ERR_NULL;
    if (rows <= 0 || cols <= 0 || !product_ok(rows, cols) || rows % 32 || cols % 32)
        return FP4_ERR_SHAPE;
    if (!aligned16(x_bf16) || !aligned16(codes_rows) || !aligned16(scales_rows) ||
        !aligned16(codes_cols) || !aligned16(scales_cols))
        return FP4_ERR_ALIGN;
    return from_hip(fp4dev::launch_quant_mx_dual(
        x_bf16, rows, cols, had_n_rows, (int)had_rows, sign_seed_rows, (int)rnd_rows, sr_seed_rows,
        codes_rows, scales_rows, had_n_cols, (int)had_cols, sign_seed_cols, (int)rnd_cols,
        sr_seed_cols, codes_cols, scales_cols, (hipStream_t)stream));
}

fp4_status fp4_wgrad_quantize(const void* dy_bf16, const void* x_bf16, int64_t T, int64_t N,
                              int64_t K, int had_n, fp4_hadamard had, uint64_t sign_seed,
                              fp4_rounding rnd, uint64_t sr_seed_dy, uint64_t sr_seed_x,
                              uint8_t* dytq, uint8_t* dyts, uint8_t* xtq, uint8_t* xts, void* stream) {
    if (had != FP4_HAD_NONE && had != FP4_HAD_DET && had != FP4_HAD_SIGNED) return FP4_ERR_ENUM;
    if (had != FP4_HAD_NONE && had_n != 16 && had_n != 32) return FP4_ERR_ENUM;
    if (rnd != FP4_RTN && rnd != FP4_SR) return FP4_ERR_ENUM;
    if (!dy_bf16 || !x_bf16 || !dytq || !dyts || !xtq || !xts) return FP4_ERR_NULL;
    if (T <= 0 || N <= 0 || K <= 0 || T % 32 || !product_ok(T, N) || !product_ok(T, K))
        return FP4_ERR_SHAPE;
    if (!aligned16(dy_bf16) || !aligned16(x_bf16) || !aligned16(dytq) || !aligned16(dyts) ||
        !aligned16(xtq) || !aligned16(xts))
        return FP4_ERR_ALIGN;
    return from_hip(fp4dev::launch_quant_mx_pair(dy_bf16, T, N, x_bf16, K, had_n, (int)had, sign_seed,
                                                 (int)rnd, sr_seed_dy, sr_seed_x, dytq, dyts, xtq, xts,
                                                 (hipStream_t)stream));
}

fp4_status fp4_gemm_fprop(const uint8_t* xq, const uint8_t* xs, const uint8_t* wq,
                          const uint8_t* ws, int64_t T, int64_t N, int64_t K, float* y,
                          void* stream) {
    return run_gemm(xq, xs, wq, ws, T, N, K, y, 0, 0, stream);        // [T,K] x [N,K]^T
}

fp4_status fp4_gemm_dgrad(const uint8_t* dyq, const uint8_t* dys, const uint8_t* wtq,
                          const uint8_t* wts, int64_t T, int64_t N, int64_t K, float* dx,
                          void* stream) {
    return run_gemm(dyq, dys, wtq, wts, T, K, N, dx, 0, 0, stream);   // [T,N] x [K,N]^T
}

fp4_status fp4_gemm_wgrad(const uint8_t* dytq, const uint8_t* dyts, const uint8_t* xtq,
                          const uint8_t* xts, int64_t T, int64_t N, int64_t K, float* dw,
                          void* stream) {
    return run_gemm(dytq, dyts, xtq, xts, N, K, T, dw, 0, 0, stream);  // [N,T] x [K,T]^T
}

fp4_status fp4_gemm_mx(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs,
                       int64_t M, int64_t N, int64_t Kc, void* c, fp4_out_dtype out,
                       int accumulate, void* stream) {
    if (out != FP4_OUT_F32 && out != FP4_OUT_BF16) return FP4_ERR_ENUM;
    if (accumulate != 0 && accumulate != 1) return FP4_ERR_ENUM;
    return run_gemm(aq, as, bq, bs, M, N, Kc, c, out == FP4_OUT_BF16 ? 1 : 0, accumulate, stream);
}

size_t nvfp4_workspace_bytes(int64_t rows, int64_t cols) {
    (void)rows;
    (void)cols;
    return 256;   // one 32-bit amax word, padded to the allocation granule
}

namespace {
fp4_status check_nvfp4(const void* x_bf16, int64_t rows, int64_t cols, fp4_hadamard had,
                       nvfp4_mode mode, const float* amax_in, const uint8_t* codes,
                       const uint8_t* scales_e4m3, const float* tensor_scale) {
    if (had != FP4_HAD_NONE && had != FP4_HAD_DET && had != FP4_HAD_SIGNED) return FP4_ERR_ENUM;
    if (mode != NVFP4_RTN && mode != NVFP4_RENORM_SR && mode != NVFP4_ELEMENT_SR) return FP4_ERR_ENUM;
    if (!x_bf16 || !codes || !scales_e4m3 || !tensor_scale) return FP4_ERR_NULL;
    if (rows <= 0 || cols <= 0 || cols % 16 || !product_ok(rows, cols)) return FP4_ERR_SHAPE;
    if (!aligned16(x_bf16) || !aligned16(codes) || !aligned16(scales_e4m3) ||
        !aligned4(tensor_scale) || (amax_in && !aligned4(amax_in)))
        return FP4_ERR_ALIGN;
    return FP4_OK;
}
}  // namespace

fp4_status nvfp4_quantize(const void* x_bf16, int64_t rows, int64_t cols, fp4_hadamard had,
                          uint64_t sign_seed, nvfp4_mode mode, uint64_t sr_seed, const float* amax_in,
                          uint8_t* codes, uint8_t* scales_e4m3, float* tensor_scale,
                          void* workspace, size_t workspace_bytes, void* stream) {
    const fp4_status s = check_nvfp4(x_bf16, rows, cols, had, mode, amax_in, codes, scales_e4m3,
                                     tensor_scale);
    if (s != FP4_OK) return s;
    if (!amax_in) {
        if (!workspace || workspace_bytes < nvfp4_workspace_bytes(rows, cols))
            return FP4_ERR_WORKSPACE;
        if (!aligned16(workspace)) return FP4_ERR_ALIGN;
    }
    return from_hip(fp4dev::launch_nvfp4(x_bf16, rows, cols, (int)had, sign_seed, (int)mode, sr_seed,
                                         amax_in, codes, scales_e4m3, tensor_scale, workspace,
                                         (hipStream_t)stream));
}

fp4_status nvfp4_quantize_noalloc(const void* x_bf16, int64_t rows, int64_t cols, fp4_hadamard had,
                                  uint64_t sign_seed, nvfp4_mode mode, uint64_t sr_seed,
                                  const float* amax_in, uint8_t* codes, uint8_t* scales_e4m3,
                                  float* tensor_scale, void* stream) {
    const fp4_status s = check_nvfp4(x_bf16, rows, cols, had, mode, amax_in, codes, scales_e4m3,
                                     tensor_scale);
    if (s != FP4_OK) return s;
    void* ws = nullptr;
    if (!amax_in) {
        // the amax word in the library's per-device scratch array
        size_t bytes = 0;
        if (fp4dev::nvfp4_scratch(&ws, &bytes) != hipSuccess) return FP4_ERR_LAUNCH;
        if (nvfp4_workspace_bytes(rows, cols) > bytes) return FP4_ERR_WORKSPACE;
    }
    return from_hip(fp4dev::launch_nvfp4(x_bf16, rows, cols, (int)had, sign_seed, (int)mode, sr_seed,
                                         amax_in, codes, scales_e4m3, tensor_scale, ws,
                                         (hipStream_t)stream));
}

const char* fp4_status_string(fp4_status status) {
    switch (status) {
        case FP4_OK: return "FP4_OK";
        case FP4_ERR_NULL: return "FP4_ERR_NULL: a required pointer is NULL";
        case FP4_ERR_SHAPE: return "FP4_ERR_SHAPE: bad size or contraction not a multiple of the block";
        case FP4_ERR_ALIGN: return "FP4_ERR_ALIGN: pointer not 16-byte aligned";
        case FP4_ERR_ENUM: return "FP4_ERR_ENUM: unknown axis, Hadamard mode/size, rounding, output type or flag";
        case FP4_ERR_LAUNCH: return "FP4_ERR_LAUNCH: HIP kernel launch failed";
        case FP4_ERR_WORKSPACE: return "FP4_ERR_WORKSPACE: workspace missing or too small";
    }
    return "FP4_ERR_UNKNOWN";
}

}  // extern "C"

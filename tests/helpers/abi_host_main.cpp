// Host-only test of the C ABI (fp4_abi.cpp) built with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_abi_sanitize.py): the HIP launchers
// are replaced by stubs that record their arguments, so every entry point can
// be driven on a machine without a GPU -- valid calls must reach the right
// launcher with the right operand roles and sizes, invalid ones must be
// refused with the documented status before any launcher is called, and a
// failing launch must come back as FP4_ERR_LAUNCH.  Fake device pointers are
// never dereferenced.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "fp4.h"
#include "fp4_launch.hpp"

namespace {
struct Call {
    std::string fn;
    int64_t a = 0, b = 0, c = 0, d = 0;   // sizes as the launcher received them
    int i0 = 0, i1 = 0, i2 = 0, i3 = 0;   // enums / flags
    const void* p0 = nullptr;
    int count = 0;
};
Call g_call;
hipError_t g_status = hipSuccess;
void* g_scratch = reinterpret_cast<void*>(0x7000);
size_t g_scratch_bytes = 256;

void record(const char* fn, int64_t a, int64_t b, int64_t c, int64_t d, int i0, int i1, int i2, int i3,
            const void* p0) {
    g_call.fn = fn;
    g_call.a = a; g_call.b = b; g_call.c = c; g_call.d = d;
    g_call.i0 = i0; g_call.i1 = i1; g_call.i2 = i2; g_call.i3 = i3;
    g_call.p0 = p0;
    g_call.count++;
}
}  // namespace

namespace fp4dev {
hipError_t launch_quant_mx(const void* x, int64_t rows, int64_t cols, int axis, int had_n, int had,
                           uint64_t, int rnd, uint64_t, uint8_t*, uint8_t*, hipStream_t) {
    record("quant", rows, cols, 0, 0, axis, had_n, had, rnd, x);
    return g_status;
}
hipError_t launch_quant_mx_dual(const void* x, int64_t rows, int64_t cols, int had_n_r, int had_r, uint64_t,
                                int rnd_r, uint64_t, uint8_t*, uint8_t*, int had_n_c, int had_c, uint64_t,
                                int, uint64_t, uint8_t*, uint8_t*, hipStream_t) {
    record("dual", rows, cols, had_n_c, had_c, had_n_r, had_r, rnd_r, 0, x);
    return g_status;
}
hipError_t launch_quant_mx_pair(const void* a, int64_t rows, int64_t n1, const void*, int64_t n2, int had_n,
                                int had, uint64_t, int rnd, uint64_t, uint64_t, uint8_t*, uint8_t*, uint8_t*,
                                uint8_t*, hipStream_t) {
    record("pair", rows, n1, n2, 0, had_n, had, rnd, 0, a);
    return g_status;
}
hipError_t launch_gemm_mx(const uint8_t* aq, const uint8_t*, const uint8_t*, const uint8_t*, int64_t M,
                          int64_t N, int64_t K, void*, int out_bf16, int accumulate, hipStream_t) {
    record("gemm", M, N, K, 0, out_bf16, accumulate, 0, 0, aq);
    return g_status;
}
hipError_t launch_nvfp4(const void* x, int64_t rows, int64_t cols, int had, uint64_t, int mode, uint64_t,
                        const float* amax_in, uint8_t*, uint8_t*, float*, void* workspace, hipStream_t) {
    record("nvfp4", rows, cols, 0, 0, had, mode, amax_in != nullptr, 0, workspace);
    (void)x;
    return g_status;
}
hipError_t nvfp4_scratch(void** ptr, size_t* bytes) {
    *ptr = g_scratch;
    *bytes = g_scratch_bytes;
    return hipSuccess;
}
uint32_t host_sign_word(int, uint64_t) { return 0; }
}  // namespace fp4dev

namespace {
int g_fail = 0;
#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            std::printf("FAIL line %d: %s\n", __LINE__, #cond);            \
            ++g_fail;                                                      \
        }                                                                  \
    } while (0)

template <typename T>
T* P(uintptr_t a) { return reinterpret_cast<T*>(a); }

// a refused call: the status, and no launcher reached
#define REFUSED(expr, st)                         \
    do {                                          \
        const int before = g_call.count;          \
        CHECK((expr) == (st));                    \
        CHECK(g_call.count == before);            \
    } while (0)
}  // namespace

int main() {
    const void* x = P<void>(0x10000);
    uint8_t* q = P<uint8_t>(0x20000);
    uint8_t* s = P<uint8_t>(0x30000);
    float* f = P<float>(0x40000);
    void* odd = P<void>(0x10008);

    // quantize: valid, then each refusal
    CHECK(fp4_hadamard_quantize(x, 64, 96, FP4_AXIS_COLS, 32, FP4_HAD_SIGNED, 5, FP4_SR, 6, q, s, nullptr) == FP4_OK);
    CHECK(g_call.fn == "quant" && g_call.a == 64 && g_call.b == 96 && g_call.i0 == 0 && g_call.i1 == 32 &&
          g_call.i2 == 2 && g_call.i3 == 1 && g_call.p0 == x);
    CHECK(fp4_hadamard_quantize(x, 96, 40, FP4_AXIS_ROWS, 16, FP4_HAD_DET, 0, FP4_RTN, 0, q, s, nullptr) == FP4_OK);
    CHECK(g_call.i0 == 1 && g_call.i1 == 16);
    REFUSED(fp4_hadamard_quantize(x, 64, 96, (fp4_axis)2, 32, FP4_HAD_NONE, 0, FP4_RTN, 0, q, s, nullptr), FP4_ERR_ENUM);
    REFUSED(fp4_hadamard_quantize(x, 64, 96, FP4_AXIS_COLS, 8, FP4_HAD_DET, 0, FP4_RTN, 0, q, s, nullptr), FP4_ERR_ENUM);
    REFUSED(fp4_hadamard_quantize(x, 64, 96, FP4_AXIS_COLS, 32, (fp4_hadamard)3, 0, FP4_RTN, 0, q, s, nullptr), FP4_ERR_ENUM);
    REFUSED(fp4_hadamard_quantize(x, 64, 96, FP4_AXIS_COLS, 32, FP4_HAD_NONE, 0, (fp4_rounding)2, 0, q, s, nullptr), FP4_ERR_ENUM);
    REFUSED(fp4_hadamard_quantize(nullptr, 64, 96, FP4_AXIS_COLS, 32, FP4_HAD_NONE, 0, FP4_RTN, 0, q, s, nullptr), FP4_ERR_NULL);
    REFUSED(fp4_hadamard_quantize(x, 64, 96, FP4_AXIS_COLS, 32, FP4_HAD_NONE, 0, FP4_RTN, 0, q, nullptr, nullptr), FP4_ERR_NULL);
    REFUSED(fp4_hadamard_quantize(x, 64, 100, FP4_AXIS_COLS, 32, FP4_HAD_NONE, 0, FP4_RTN, 0, q, s, nullptr), FP4_ERR_SHAPE);
    REFUSED(fp4_hadamard_quantize(x, 100, 64, FP4_AXIS_ROWS, 32, FP4_HAD_NONE, 0, FP4_RTN, 0, q, s, nullptr), FP4_ERR_SHAPE);
    REFUSED(fp4_hadamard_quantize(x, 0, 64, FP4_AXIS_COLS, 32, FP4_HAD_NONE, 0, FP4_RTN, 0, q, s, nullptr), FP4_ERR_SHAPE);
    REFUSED(fp4_hadamard_quantize(x, INT64_C(1) << 40, INT64_C(1) << 40, FP4_AXIS_COLS, 32, FP4_HAD_NONE, 0, FP4_RTN, 0, q, s, nullptr), FP4_ERR_SHAPE);
    REFUSED(fp4_hadamard_quantize(odd, 64, 96, FP4_AXIS_COLS, 32, FP4_HAD_NONE, 0, FP4_RTN, 0, q, s, nullptr), FP4_ERR_ALIGN);

    // dual and the Wgrad pair
    CHECK(fp4_hadamard_quantize_dual(x, 64, 96, 32, FP4_HAD_DET, 1, FP4_RTN, 2, q, s, 16, FP4_HAD_SIGNED, 3,
                                     FP4_SR, 4, q, s, nullptr) == FP4_OK);
    CHECK(g_call.fn == "dual" && g_call.a == 64 && g_call.b == 96 && g_call.c == 16 && g_call.d == 2 &&
          g_call.i0 == 32 && g_call.i1 == 1);
    REFUSED(fp4_hadamard_quantize_dual(x, 64, 96, 32, FP4_HAD_DET, 1, FP4_RTN, 2, q, s, 16, FP4_HAD_SIGNED, 3,
                                       FP4_SR, 4, nullptr, s, nullptr), FP4_ERR_NULL);
    REFUSED(fp4_hadamard_quantize_dual(x, 60, 96, 32, FP4_HAD_DET, 1, FP4_RTN, 2, q, s, 16, FP4_HAD_SIGNED, 3,
                                       FP4_SR, 4, q, s, nullptr), FP4_ERR_SHAPE);
    CHECK(fp4_wgrad_quantize(x, x, 8192, 14336, 4096, 32, FP4_HAD_DET, 0, FP4_RTN, 0, 0, q, s, q, s, nullptr) == FP4_OK);
    CHECK(g_call.fn == "pair" && g_call.a == 8192 && g_call.b == 14336 && g_call.c == 4096 && g_call.i0 == 32);
    REFUSED(fp4_wgrad_quantize(x, x, 8200, 14336, 4096, 32, FP4_HAD_DET, 0, FP4_RTN, 0, 0, q, s, q, s, nullptr), FP4_ERR_SHAPE);
    REFUSED(fp4_wgrad_quantize(x, x, 8192, 14336, 4096, 32, FP4_HAD_DET, 0, FP4_RTN, 0, 0, q, s, q, P<uint8_t>(0x30004), nullptr), FP4_ERR_ALIGN);

    // the three GEMM roles map (T, N, K) to the one TN product
    CHECK(fp4_gemm_fprop(q, s, q, s, 8192, 14336, 4096, f, nullptr) == FP4_OK);
    CHECK(g_call.fn == "gemm" && g_call.a == 8192 && g_call.b == 14336 && g_call.c == 4096 && g_call.i0 == 0 && g_call.i1 == 0);
    CHECK(fp4_gemm_dgrad(q, s, q, s, 8192, 14336, 4096, f, nullptr) == FP4_OK);
    CHECK(g_call.a == 8192 && g_call.b == 4096 && g_call.c == 14336);
    CHECK(fp4_gemm_wgrad(q, s, q, s, 8192, 14336, 4096, f, nullptr) == FP4_OK);
    CHECK(g_call.a == 14336 && g_call.b == 4096 && g_call.c == 8192);
    CHECK(fp4_gemm_mx(q, s, q, s, 100, 70, 96, f, FP4_OUT_BF16, 1, nullptr) == FP4_OK);
    CHECK(g_call.a == 100 && g_call.b == 70 && g_call.c == 96 && g_call.i0 == 1 && g_call.i1 == 1);
    REFUSED(fp4_gemm_mx(q, s, q, s, 100, 70, 96, f, (fp4_out_dtype)2, 0, nullptr), FP4_ERR_ENUM);
    REFUSED(fp4_gemm_mx(q, s, q, s, 100, 70, 96, f, FP4_OUT_F32, 2, nullptr), FP4_ERR_ENUM);
    REFUSED(fp4_gemm_fprop(q, s, q, s, 64, 64, 48, f, nullptr), FP4_ERR_SHAPE);
    REFUSED(fp4_gemm_fprop(q, s, q, s, 64, 64, INT64_C(1) << 24, f, nullptr), FP4_ERR_SHAPE);
    REFUSED(fp4_gemm_fprop(q, s, q, s, INT64_C(1) << 33, 64, 64, f, nullptr), FP4_ERR_SHAPE);
    REFUSED(fp4_gemm_fprop(q, s, q, s, 64, 64, 64, P<float>(0x40004), nullptr), FP4_ERR_ALIGN);
    REFUSED(fp4_gemm_fprop(q, nullptr, q, s, 64, 64, 64, f, nullptr), FP4_ERR_NULL);

    // NVFP4: workspace, supplied amax, the allocation-free variant
    char ws[512];
    void* wsa = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws) + 15) & ~uintptr_t(15));
    CHECK(nvfp4_workspace_bytes(16384, 8192) == 256);
    CHECK(nvfp4_quantize(x, 48, 80, FP4_HAD_SIGNED, 1, NVFP4_RENORM_SR, 2, nullptr, q, s, f, wsa, 256, nullptr) == FP4_OK);
    CHECK(g_call.fn == "nvfp4" && g_call.a == 48 && g_call.b == 80 && g_call.i0 == 2 && g_call.i1 == 1 &&
          g_call.i2 == 0 && g_call.p0 == wsa);
    CHECK(nvfp4_quantize(x, 48, 80, FP4_HAD_NONE, 1, NVFP4_ELEMENT_SR, 2, f, q, s, f, nullptr, 0, nullptr) == FP4_OK);
    CHECK(g_call.i1 == 2 && g_call.i2 == 1);
    REFUSED(nvfp4_quantize(x, 48, 80, FP4_HAD_SIGNED, 1, NVFP4_RTN, 2, nullptr, q, s, f, nullptr, 0, nullptr), FP4_ERR_WORKSPACE);
    REFUSED(nvfp4_quantize(x, 48, 80, FP4_HAD_SIGNED, 1, NVFP4_RTN, 2, nullptr, q, s, f, wsa, 255, nullptr), FP4_ERR_WORKSPACE);
    REFUSED(nvfp4_quantize(x, 48, 72, FP4_HAD_SIGNED, 1, NVFP4_RTN, 2, f, q, s, f, nullptr, 0, nullptr), FP4_ERR_SHAPE);
    REFUSED(nvfp4_quantize(x, 48, 80, FP4_HAD_SIGNED, 1, (nvfp4_mode)3, 2, f, q, s, f, nullptr, 0, nullptr), FP4_ERR_ENUM);
    REFUSED(nvfp4_quantize(x, 48, 80, FP4_HAD_SIGNED, 1, NVFP4_RTN, 2, P<float>(0x40002), q, s, f, nullptr, 0, nullptr), FP4_ERR_ALIGN);
    CHECK(nvfp4_quantize_noalloc(x, 48, 80, FP4_HAD_SIGNED, 1, NVFP4_RENORM_SR, 2, nullptr, q, s, f, nullptr) == FP4_OK);
    CHECK(g_call.fn == "nvfp4" && g_call.p0 == g_scratch);
    g_scratch_bytes = 128;
    REFUSED(nvfp4_quantize_noalloc(x, 48, 80, FP4_HAD_SIGNED, 1, NVFP4_RENORM_SR, 2, nullptr, q, s, f, nullptr), FP4_ERR_WORKSPACE);
    CHECK(nvfp4_quantize_noalloc(x, 48, 80, FP4_HAD_SIGNED, 1, NVFP4_RENORM_SR, 2, f, q, s, f, nullptr) == FP4_OK);
    g_scratch_bytes = 256;

    // a launch the runtime refuses comes back as FP4_ERR_LAUNCH
    g_status = hipErrorInvalidValue;
    CHECK(fp4_gemm_wgrad(q, s, q, s, 64, 64, 64, f, nullptr) == FP4_ERR_LAUNCH);
    CHECK(fp4_hadamard_quantize(x, 64, 96, FP4_AXIS_COLS, 32, FP4_HAD_NONE, 0, FP4_RTN, 0, q, s, nullptr) == FP4_ERR_LAUNCH);
    CHECK(nvfp4_quantize(x, 48, 80, FP4_HAD_NONE, 1, NVFP4_RTN, 2, f, q, s, f, nullptr, 0, nullptr) == FP4_ERR_LAUNCH);
    g_status = hipSuccess;

    for (int st = 0; st <= 7; ++st) CHECK(fp4_status_string((fp4_status)st) != nullptr);
    CHECK(std::strcmp(fp4_status_string((fp4_status)99), "FP4_ERR_UNKNOWN") == 0);

    if (g_fail) return 1;
    std::printf("ok\n");
    return 0;
}

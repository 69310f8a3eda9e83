// nvfp4.hip -- NVFP4 quantization (16-element blocks, E4M3 block scales, fp32
// tensor scale) with the renormalization folded into the block scales by
// stochastic rounding.
//
// [QUARTET-II] "Quartet II -- обучение в NVFP4 с точными несмещёнными
// градиентами": NVFP4 carries FP8 block scales; a randomly rotated tensor,
// once quantized, is collinear with the original in expectation and a
// renormalization makes it unbiased; the factor is too fine for FP8 scales,
// so it is put into the scales by stochastic rounding -- the scales only,
// not every FP4 element.  [NV-NVFP4] "NVIDIA создала метод обучения
// нейросетей в 4-bit точности", section "Как это работает": 16x16 random
// Hadamard transforms on gradient inputs.
//
// Two passes over x when the tensor amax is not supplied:
//   nv_amax  -- rotate each 16-block (pairs of lanes, 8 elements each) and
//               reduce max |y| into one workspace word (atomic max on the
//               float bits, valid because every value is non-negative);
//   nv_quant -- rotate again, derive s_t from the amax, per block the E4M3
//               scale, the E2M1 codes and, with renorm, the scale rounded
//               stochastically toward |y|^2 / (s_t sum y_i q_i).
#include "fp4_device.hpp"
#include "fp4_launch.hpp"

namespace fp4dev {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float pair_xor1f(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t pair_xor1(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}

// 16-block transform of the 8 elements this lane holds; lane parity q picks
// the half of the block.  Same butterfly order as the MXFP4 kernels.
template <bool HAD>
__device__ __forceinline__ void load_rotate8(const uint4& w, int q, uint32_t sign_word, float* a) {
    a[0] = bf16_lo(w.x); a[1] = bf16_hi(w.x); a[2] = bf16_lo(w.y); a[3] = bf16_hi(w.y);
    a[4] = bf16_lo(w.z); a[5] = bf16_hi(w.z); a[6] = bf16_lo(w.w); a[7] = bf16_hi(w.w);
    if constexpr (HAD) {
#pragma unroll
        for (int t = 0; t < 8; ++t) a[t] = flip_if(a[t], (sign_word >> (8 * q + t)) & 1u);
#pragma unroll
        for (int hh = 1; hh < 8; hh <<= 1) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (i & hh) continue;
                const float x = a[i], y = a[i + hh];
                a[i] = x + y;
                a[i + hh] = x - y;
            }
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float p = pair_xor1f(a[t]);
            a[t] = q ? (p - a[t]) : (a[t] + p);
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) a[t] = a[t] * 0.25f;
    }
}

__global__ void nv_clear(uint32_t* p) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *p = 0u;
}

template <bool HAD>
__global__ __launch_bounds__(kThreads) void nv_amax(const uint4* __restrict__ x, int64_t nchunks,
                                                    uint32_t sign_word, uint32_t* __restrict__ amax) {
    __shared__ uint32_t red[kThreads / 64];
    uint32_t m = 0;
    const int q = threadIdx.x & 1;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < nchunks; g += stride) {
        float a[8];
        load_rotate8<HAD>(x[g], q, sign_word, a);
#pragma unroll
        for (int t = 0; t < 8; ++t) m = max(m, __float_as_uint(a[t]) & 0x7FFFFFFFu);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = red[0];
#pragma unroll
        for (int i = 1; i < kThreads / 64; ++i) r = max(r, red[i]);
        atomicMax(amax, r);
    }
}

__device__ __forceinline__ float e2m1_signed_value(uint32_t code) {
    const uint32_t m = code & 7u, e = m >> 1, mb = m & 1u;
    const uint32_t mag = e == 0u ? (mb ? 0x3F000000u : 0u) : (((e + 126u) << 23) | (mb << 22));
    return __uint_as_float(mag | ((code & 8u) << 28));
}

template <bool HAD, bool RENORM>
__global__ __launch_bounds__(kThreads) void nv_quant(
    const uint4* __restrict__ x, int64_t nchunks, uint32_t sign_word, const float* __restrict__ amax_p,
    uint64_t sr_seed, uint32_t* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ tensor_scale) {
    const float amax = *amax_p;
    const float s_t = amax == 0.0f ? 1.0f : amax / 2688.0f;   // 6 * 448
    const float six_st = 6.0f * s_t;
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (g == 0) *tensor_scale = s_t;
    if (g >= nchunks) return;                                   // uniform per pair
    const int q = threadIdx.x & 1;
    float y[8];
    load_rotate8<HAD>(x[g], q, sign_word, y);
    uint32_t m = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) m = max(m, __float_as_uint(y[t]) & 0x7FFFFFFFu);
    m = max(m, pair_xor1(m));
    const uint32_t sb = e4m3_rne(__uint_as_float(m) / six_st);
    uint32_t word = 0, stored = sb;
    if (sb != 0u) {
        const float inv = 1.0f / (e4m3_value(sb) * s_t);
        uint32_t cq[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            cq[t] = e2m1_rtn(y[t] * inv);
            word |= cq[t] << (4 * t);
        }
        if constexpr (RENORM) {
            // sequential binary32 fmaf chains over the 16 elements in order:
            // the lower lane's partial sums seed the upper lane's chain
            float num = 0.0f, den = 0.0f;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                num = fmaf(y[t], y[t], num);
                den = fmaf(y[t], e2m1_signed_value(cq[t]), den);
            }
            float pnum = pair_xor1f(num), pden = pair_xor1f(den);
            if (q) {
                num = pnum;
                den = pden;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    num = fmaf(y[t], y[t], num);
                    den = fmaf(y[t], e2m1_signed_value(cq[t]), den);
                }
                if (den > 0.0f) {
                    const float target = num / (s_t * den);
                    const uint64_t blk = (uint64_t)g >> 1;
                    const uint32_t u = word_of(stream4(sr_seed, 2u, blk >> 2), (int)(blk & 3));
                    stored = e4m3_sr(target, u);
                }
            }
        }
    }
    codes[g] = word;
    if (q == 1) scales[g >> 1] = (uint8_t)stored;
}

template <bool HAD>
hipError_t launch_nv_had(const void* x, int64_t rows, int64_t cols, uint32_t sw, int renorm,
                         uint64_t sr_seed, const float* amax_in, uint8_t* codes, uint8_t* scales,
                         float* tensor_scale, void* workspace, hipStream_t st) {
    const int64_t nchunks = rows * cols / 8;
    const float* amax_p = amax_in;
    if (!amax_p) {
        uint32_t* ws = (uint32_t*)workspace;
        hipLaunchKernelGGL(nv_clear, dim3(1), dim3(64), 0, st, ws);
        int64_t blocks = (nchunks + kThreads - 1) / kThreads;
        if (blocks > 8192) blocks = 8192;
        hipLaunchKernelGGL((nv_amax<HAD>), dim3((unsigned)blocks), dim3(kThreads), 0, st,
                           (const uint4*)x, nchunks, sw, ws);
        amax_p = (const float*)ws;
    }
    const int64_t qblocks = (nchunks + kThreads - 1) / kThreads;
    if (renorm) {
        hipLaunchKernelGGL((nv_quant<HAD, true>), dim3((unsigned)qblocks), dim3(kThreads), 0, st,
                           (const uint4*)x, nchunks, sw, amax_p, sr_seed, (uint32_t*)codes, scales,
                           tensor_scale);
    } else {
        hipLaunchKernelGGL((nv_quant<HAD, false>), dim3((unsigned)qblocks), dim3(kThreads), 0, st,
                           (const uint4*)x, nchunks, sw, amax_p, sr_seed, (uint32_t*)codes, scales,
                           tensor_scale);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_nvfp4(const void* x, int64_t rows, int64_t cols, int had, uint64_t sign_seed,
                        int renorm, uint64_t sr_seed, const float* amax_in, uint8_t* codes,
                        uint8_t* scales, float* tensor_scale, void* workspace, hipStream_t st) {
    if (had == 0)
        return launch_nv_had<false>(x, rows, cols, 0u, renorm, sr_seed, amax_in, codes, scales,
                                    tensor_scale, workspace, st);
    return launch_nv_had<true>(x, rows, cols, host_sign_word(had, sign_seed), renorm, sr_seed,
                               amax_in, codes, scales, tensor_scale, workspace, st);
}

}  // namespace fp4dev

// nvfp4.hip -- NVFP4 quantization (16-element blocks, E4M3 block scales, fp32
// tensor scale) with the renormalization folded into the block scales by
// stochastic rounding, or with every element rounded stochastically.
//
// [QUARTET-II] "Quartet II -- обучение в NVFP4 с точными несмещёнными
// градиентами": NVFP4 carries FP8 block scales; a randomly rotated tensor,
// once quantized, is collinear with the original in expectation and a
// renormalization makes it unbiased; the factor is too fine for FP8 scales,
// so it is put into the scales by stochastic rounding -- the scales only,
// not every FP4 element as in the recipe it compares against (kept here as
// the element-SR mode).  [NV-NVFP4] "NVIDIA создала метод обучения
// нейросетей в 4-bit точности", section "Как это работает": 16x16 random
// Hadamard transforms on gradient inputs.
//
// Two passes over x when the tensor amax is not supplied:
//   nv_amax  -- rotate each 16-block (pairs of lanes, 8 elements each) and
//               reduce max |y| into one workspace word (atomic max on the
//               float bits, valid because every value is non-negative);
//   nv_quant_renorm (renormalized scales) -- one lane per block: rotate
//               again, derive s_t from the amax, the block's E4M3 scale, the
//               E2M1 codes and the scale rounded stochastically toward
//               |y|^2 / (s_t sum y_i q_i);
//   nv_quant (elements to nearest, or every element stochastically) -- a
//               lane pair per block.
// Codes to nearest come from the hardware FP4 conversion of fl(y_i * inv)
// with scale 1 (round to nearest even, saturating -- the rule the MX
// quantizers check bit-exact), q_i from its inverse; in the element-SR mode
// from the MX quantizers' stochastic rounding with the element stream
// (purpose 0, index = row-major position: two Philox calls per 8-element
// chunk).
#include "fp4_device.hpp"
#include "fp4_launch.hpp"

#include <mutex>

// Scratch memory of the allocation-free entry point (nvfp4_quantize_noalloc):
// the in-library amax word, in a fixed device array instead of a workspace
// the caller passes.  Each GPU the library runs on holds its own copy until
// the process ends; every call on that GPU shares it (the amax pass clears
// it with a kernel first), so calls that overlap on one GPU race.  In host
// code `scratch` is only a symbol: kernels get its device address, looked
// up once per device by nvfp4_scratch below.
static __device__ __align__(256) uint32_t scratch[64];

namespace fp4dev {
namespace {

constexpr int kThreads = 256;
// Loads in flight per thread: 16-byte chunks in nv_amax and nv_quant, whole
// blocks in nv_quant_renorm (four per lane, the four words of a Philox call).
constexpr int kUnroll = 4;
// Workgroups of the amax pass (each ends with one atomic max on the same
// word: 8192 of them serialized behind each other cost 2x the pass).
constexpr int64_t kAmaxBlocks = 1024;

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
    const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
    for (int64_t g0 = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; g0 < nchunks; g0 += stride) {
        uint4 w[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t g = g0 + (int64_t)u * kThreads;
            w[u] = g < nchunks ? x[g] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float a[8];
            load_rotate8<HAD>(w[u], q, sign_word, a);
#pragma unroll
            for (int t = 0; t < 8; ++t) m = max(m, __float_as_uint(a[t]) & 0x7FFFFFFFu);
        }
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

typedef float v2f __attribute__((ext_vector_type(2)));

// The tensor scale of an amax: A / 2688 (6 * 448), 1 for A = 0.  `valid` is
// false when that is not a finite positive number (A NaN, infinite,
// negative, or so small that A / 2688 is zero): the whole tensor is then
// NaN -- tensor scale NaN, every block scale 0x7F (the E4M3 NaN), all codes
// zero.  Non-finite inputs are a reading: the pages are silent on them.
__device__ __forceinline__ float tensor_scale_of(float amax, bool& valid) {
    const float s_t = amax == 0.0f ? 1.0f : amax / 2688.0f;
    valid = (__float_as_uint(s_t) & 0x7FFFFFFFu) < 0x7F800000u && s_t > 0.0f;
    return s_t;
}
constexpr uint32_t kQNaN = 0x7FC00000u;
constexpr uint32_t kE4m3NaN = 0x7Fu;

// E2M1 codes of 8 binary32 values, nearest with ties to even, saturating at
// 6: V_CVT_SCALEF32_PK_FP4_F32 with scale 1 -- the same rounding as the MX
// quantizers' hardware path (there checked bit-exact against the integer
// encoder for power-of-two scales, 1 among them); two values per
// instruction, the first in the low nibble.
__device__ __forceinline__ uint32_t encode8_unit(const float* v) {
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
    return w;
}

// The 8 E2M1 values of a code word (exact; low nibble first).
__device__ __forceinline__ void decode8(uint32_t w, float* out) {
    v2f r;
    r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); out[0] = r.x; out[1] = r.y;
    r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); out[2] = r.x; out[3] = r.y;
    r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); out[4] = r.x; out[5] = r.y;
    r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); out[6] = r.x; out[7] = r.y;
}

// MODE 0: RTN; 2: element SR (the renormalized mode is nv_quant_renorm).
template <bool HAD, int MODE>
__global__ __launch_bounds__(kThreads) void nv_quant(
    const uint4* __restrict__ x, int64_t nchunks, uint32_t sign_word, const float* __restrict__ amax_p,
    uint64_t sr_seed, uint32_t* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ tensor_scale) {
    static_assert(MODE == 0 || MODE == 2, "RTN or element SR");
    bool valid;
    const float s_t = tensor_scale_of(*amax_p, valid);
    const float six_st = 6.0f * s_t;
    if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = valid ? s_t : __uint_as_float(kQNaN);
    const int q = threadIdx.x & 1;
    // Lanes 2p, 2p+1 hold the two 8-element halves of one block; chunk u of
    // a thread is kThreads chunks after chunk u - 1 (every load instruction
    // contiguous).  All chunks are loaded first.
    auto chunk = [&](int u) -> int64_t {
        return ((int64_t)blockIdx.x * kUnroll + u) * kThreads + threadIdx.x;
    };
    uint4 wv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t g = chunk(u);
        wv[u] = g < nchunks ? x[g] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t g = chunk(u);
        if (g >= nchunks) break;                                    // uniform per pair
        float y[8];
        load_rotate8<HAD>(wv[u], q, sign_word, y);
        uint32_t m = 0;
#pragma unroll
        for (int t = 0; t < 8; ++t) m = max(m, __float_as_uint(y[t]) & 0x7FFFFFFFu);
        m = max(m, pair_xor1(m));
        // a NaN or infinite element in the block (m >= the infinity's bits),
        // or a NaN tensor: scale 0x7F, codes zero
        const bool bad = !valid || m >= 0x7F800000u;
        const uint32_t sb = bad ? kE4m3NaN : e4m3_rne(__uint_as_float(m) / six_st);
        uint32_t word = 0;
        const float inv = 1.0f / (e4m3_value(sb) * s_t);
        // (an infinite reciprocal -- s_b s_t below about 2^-128 -- gives zero
        // codes and keeps s_b)
        if (!bad && sb != 0u && __float_as_uint(inv) != 0x7F800000u) {
            float v[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) v[t] = y[t] * inv;
            if constexpr (MODE == 2) {
                // elements 8g .. 8g+7: words of stream counters 2g and 2g + 1
                const uint4 r0 = stream4(sr_seed, 0u, (uint64_t)(2 * g));
                const uint4 r1 = stream4(sr_seed, 0u, (uint64_t)(2 * g + 1));
                const uint32_t uw[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
                for (int t = 0; t < 8; ++t) word |= e2m1_sr(v[t], uw[t]) << (4 * t);
            } else {
                word = encode8_unit(v);
            }
        }
        codes[g] = word;
        if (q == 1) scales[g >> 1] = (uint8_t)sb;
    }
}

// Word (lane mod 4) of the four words lane U of this lane's quad holds:
// four DPP quad broadcasts, then a select.
template <int U>
__device__ __forceinline__ uint32_t quad_word(const uint4& w, int wsel) {
    constexpr int kBroadcast = 0x55 * U;        // quad_perm [U, U, U, U]
    const uint32_t w0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)w.x, kBroadcast, 0xF, 0xF, false);
    const uint32_t w1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)w.y, kBroadcast, 0xF, 0xF, false);
    const uint32_t w2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)w.z, kBroadcast, 0xF, 0xF, false);
    const uint32_t w3 = (uint32_t)__builtin_amdgcn_mov_dpp((int)w.w, kBroadcast, 0xF, 0xF, false);
    return wsel == 0 ? w0 : wsel == 1 ? w1 : wsel == 2 ? w2 : w3;
}

// The renormalized mode with one lane per block: wave w of the grid owns
// blocks 256 w .. 256 w + 255, lane l of it blocks 256 w + 64 u + l for
// u = 0..3 (two 16-byte loads per block, consecutive lanes on consecutive
// blocks).  Each lane then rotates, scales, encodes and sums its whole block
// -- the fmaf chains run over the 16 elements in order in one lane -- so the
// per-block work (three divisions, E4M3 rounding) is done once per block.
// The scale SR words: block blk takes word blk mod 4 of counter blk / 4, so
// the four lanes of a quad need, for each u, the four words of one counter;
// lane j of the quad draws the counter of u = j and DPP broadcasts within
// the quad hand each lane its word.
template <bool HAD>
__global__ __launch_bounds__(kThreads) void nv_quant_renorm(
    const uint4* __restrict__ x, int64_t nblocks, uint32_t sign_word, const float* __restrict__ amax_p,
    uint64_t sr_seed, uint2* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ tensor_scale) {
    bool valid;
    const float s_t = tensor_scale_of(*amax_p, valid);
    const float six_st = 6.0f * s_t;
    if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = valid ? s_t : __uint_as_float(kQNaN);
    const int lane = threadIdx.x & 63;
    const int64_t b0 = ((int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * 256;
    uint4 wv[2 * kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t blk = b0 + 64 * u + lane;
        const bool in = blk < nblocks;
        wv[2 * u] = in ? x[2 * blk] : make_uint4(0, 0, 0, 0);
        wv[2 * u + 1] = in ? x[2 * blk + 1] : make_uint4(0, 0, 0, 0);
    }
    // lane 4k + j: the counter of blocks b0 + 64 j + 4k .. + 3
    const uint4 mine = stream4(sr_seed, 2u, (uint64_t)((b0 >> 2) + 16 * (lane & 3) + (lane >> 2)));
    const int wsel = lane & 3;
    static_assert(kUnroll == 4, "one quad lane per block slot");
    const uint32_t srw[kUnroll] = {quad_word<0>(mine, wsel), quad_word<1>(mine, wsel),
                                   quad_word<2>(mine, wsel), quad_word<3>(mine, wsel)};
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t blk = b0 + 64 * u + lane;
        if (blk >= nblocks) break;                  // only the grid's last wave
        float y[16];
        const uint4 lo = wv[2 * u], hi = wv[2 * u + 1];
        y[0] = bf16_lo(lo.x); y[1] = bf16_hi(lo.x); y[2] = bf16_lo(lo.y); y[3] = bf16_hi(lo.y);
        y[4] = bf16_lo(lo.z); y[5] = bf16_hi(lo.z); y[6] = bf16_lo(lo.w); y[7] = bf16_hi(lo.w);
        y[8] = bf16_lo(hi.x); y[9] = bf16_hi(hi.x); y[10] = bf16_lo(hi.y); y[11] = bf16_hi(hi.y);
        y[12] = bf16_lo(hi.z); y[13] = bf16_hi(hi.z); y[14] = bf16_lo(hi.w); y[15] = bf16_hi(hi.w);
        if constexpr (HAD) {
#pragma unroll
            for (int t = 0; t < 16; ++t) y[t] = flip_if(y[t], (sign_word >> t) & 1u);
#pragma unroll
            for (int hh = 1; hh < 16; hh <<= 1) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    if (i & hh) continue;
                    const float a = y[i], b = y[i + hh];
                    y[i] = a + b;
                    y[i + hh] = a - b;
                }
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) y[t] = y[t] * 0.25f;
        }
        uint32_t m = 0;
#pragma unroll
        for (int t = 0; t < 16; ++t) m = max(m, __float_as_uint(y[t]) & 0x7FFFFFFFu);
        // as in nv_quant: a non-finite block or tensor gives 0x7F and zero
        // codes, an infinite reciprocal scale zero codes with s_b kept
        const bool bad = !valid || m >= 0x7F800000u;
        const uint32_t sb = bad ? kE4m3NaN : e4m3_rne(__uint_as_float(m) / six_st);
        uint32_t c0 = 0, c1 = 0, stored = sb;
        const float inv = 1.0f / (e4m3_value(sb) * s_t);
        if (!bad && sb != 0u && __float_as_uint(inv) != 0x7F800000u) {
            float v[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) v[t] = y[t] * inv;
            c0 = encode8_unit(v);
            c1 = encode8_unit(v + 8);
            float yq[16];
            decode8(c0, yq);
            decode8(c1, yq + 8);
            float num = 0.0f, den = 0.0f;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                num = fmaf(y[t], y[t], num);
                den = fmaf(y[t], yq[t], den);
            }
            // the renormalized scale needs den > 0 and a target that is a
            // number (Inf / Inf when the sums overflow keeps s_b; an
            // infinite target saturates at 448)
            if (den > 0.0f) {
                const float target = num / (s_t * den);
                if (target == target) stored = e4m3_sr(target, srw[u]);
            }
        }
        codes[blk] = make_uint2(c0, c1);
        scales[blk] = (uint8_t)stored;
    }
}

template <bool HAD>
hipError_t launch_nv_had(const void* x, int64_t rows, int64_t cols, uint32_t sw, int mode,
                         uint64_t sr_seed, const float* amax_in, uint8_t* codes, uint8_t* scales,
                         float* tensor_scale, void* workspace, hipStream_t st) {
    const int64_t nchunks = rows * cols / 8;
    const float* amax_p = amax_in;
    if (!amax_p) {
        uint32_t* ws = (uint32_t*)workspace;
        hipError_t e = launch(&nv_clear, dim3(1), dim3(64), st, ws);
        if (e != hipSuccess) return e;
        int64_t blocks = (nchunks + (int64_t)kThreads * kUnroll - 1) / ((int64_t)kThreads * kUnroll);
        if (blocks > kAmaxBlocks) blocks = kAmaxBlocks;
        e = launch(&nv_amax<HAD>, dim3((unsigned)blocks), dim3(kThreads), st, (const uint4*)x, nchunks,
                   sw, ws);
        if (e != hipSuccess) return e;
        amax_p = (const float*)ws;
    }
    const int64_t qblocks = (nchunks + (int64_t)kThreads * kUnroll - 1) / ((int64_t)kThreads * kUnroll);
    if (mode == 1) {
        const int64_t nblocks = nchunks / 2, per_wg = (int64_t)(kThreads / 64) * 256;
        return launch(&nv_quant_renorm<HAD>, dim3((unsigned)((nblocks + per_wg - 1) / per_wg)),
                      dim3(kThreads), st, (const uint4*)x, nblocks, sw, amax_p, sr_seed, (uint2*)codes,
                      scales, tensor_scale);
    }
    if (mode == 2)
        return launch(&nv_quant<HAD, 2>, dim3((unsigned)qblocks), dim3(kThreads), st, (const uint4*)x,
                      nchunks, sw, amax_p, sr_seed, (uint32_t*)codes, scales, tensor_scale);
    return launch(&nv_quant<HAD, 0>, dim3((unsigned)qblocks), dim3(kThreads), st, (const uint4*)x,
                  nchunks, sw, amax_p, sr_seed, (uint32_t*)codes, scales, tensor_scale);
}

}  // namespace

hipError_t nvfp4_scratch(void** ptr, size_t* bytes) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        // with `dev` current: this device's copy of the array
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    *bytes = sizeof(scratch);
    return hipSuccess;
}

hipError_t launch_nvfp4(const void* x, int64_t rows, int64_t cols, int had, uint64_t sign_seed,
                        int mode, uint64_t sr_seed, const float* amax_in, uint8_t* codes,
                        uint8_t* scales, float* tensor_scale, void* workspace, hipStream_t st) {
    if (had == 0)
        return launch_nv_had<false>(x, rows, cols, 0u, mode, sr_seed, amax_in, codes, scales,
                                    tensor_scale, workspace, st);
    return launch_nv_had<true>(x, rows, cols, host_sign_word(had, sign_seed), mode, sr_seed,
                               amax_in, codes, scales, tensor_scale, workspace, st);
}

}  // namespace fp4dev

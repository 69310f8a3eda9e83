// gemm_mx.hip -- scaled MXFP4 GEMM on gfx950 matrix cores.
//
// [AMD-MXFP4] "Pretraining large language models with MXFP4 on Native FP4
// Hardware", section "Поисковая экспериментальная работа: корень
// нестабильности": the three GEMMs of a linear layer (Fprop, Dgrad, Wgrad)
// run in MXFP4 on native FP4 matrix cores.  All three are one "TN" product
//     C[m, n] = sum_k a[m, k] b[n, k]
// of two operands stored along their contraction axis as E2M1 codes (two per
// byte, even k in the low nibble) with one E8M0 scale per 32 k.
//
// Kernel: 256 threads (4 waves as 2 x 2), block tile (64 WM) x (64 WN), each
// wave WM x WN tiles of 32 x 32 computed by V_MFMA_SCALE_F32_32X32X64_F8F6F4
// with both operands in FP4 (format code 4) and fp32 accumulation.  For that
// instruction lane l supplies row (l mod 32) and k-half (l div 32) of a
// 32 x 64 operand slice: 32 consecutive k = one 16-byte code chunk = exactly
// one scale block, so the lane's scale byte is that block's E8M0 scale.
// Stages of 256 k (128 bytes per row) are staged through LDS, double
// buffered; the 16-byte chunks of a row are XOR-swizzled by the row index so
// that the 32 rows one fragment read touches spread over the banks.  Scales
// go straight from global memory to registers, one stage ahead.
#include "fp4_device.hpp"
#include "fp4_launch.hpp"

namespace fp4dev {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBK = 256;             // k elements per stage
constexpr int kRowBytes = kBK / 2;   // code bytes per row per stage
constexpr int kThreads = 256;

__device__ __forceinline__ int swz(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ (row & 7)) << 4);
}

// Scale bytes of blocks 8kt .. 8kt+7 for one row, packed little-endian into
// (lo, hi); blocks at or beyond ks read as 127 (2^0) so that the zero codes
// of a contraction tail contribute exact zeros.
__device__ __forceinline__ void load_scales8(const uint8_t* __restrict__ S, int64_t row, int64_t ks,
                                             int kt, bool vec_ok, uint32_t& lo, uint32_t& hi) {
    const uint8_t* p = S + row * ks + (int64_t)kt * 8;
    if (vec_ok) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        lo = v.x;
        hi = v.y;
        return;
    }
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = ((int64_t)kt * 8 + i < ks) ? (uint32_t)p[i] : 127u;
    lo = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    hi = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
}

template <int WM, int WN>
__global__ __launch_bounds__(kThreads) void gemm_mx_tn(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, int64_t M, int64_t N, int64_t K, float* __restrict__ C,
    int tiles_n) {
    constexpr int BM = 64 * WM, BN = 64 * WN;
    constexpr int CA = BM * 8 / kThreads, CB = BN * 8 / kThreads;   // 16-byte chunks per thread
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + BN) * kRowBytes];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, l32 = lane & 31;
    const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * BM;
    const int64_t n0 = (int64_t)(blockIdx.x % tiles_n) * BN;
    const int64_t kbytes = K / 2, ks = K / 32;
    const int nk = (int)((K + kBK - 1) / kBK);
    const bool svec = (ks % 8) == 0;

    uint4 ra[CA], rb[CB];
    auto gload = [&](int kt) {
        const int64_t k0b = (int64_t)kt * kRowBytes;
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const int c = tid + i * kThreads, row = c >> 3, ch = c & 7;
            const int64_t grow = (m0 + row < M) ? m0 + row : M - 1;
            ra[i] = (k0b + ch * 16 < kbytes)
                        ? *reinterpret_cast<const uint4*>(A + grow * kbytes + k0b + ch * 16)
                        : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int c = tid + i * kThreads, row = c >> 3, ch = c & 7;
            const int64_t grow = (n0 + row < N) ? n0 + row : N - 1;
            rb[i] = (k0b + ch * 16 < kbytes)
                        ? *reinterpret_cast<const uint4*>(B + grow * kbytes + k0b + ch * 16)
                        : make_uint4(0, 0, 0, 0);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const int c = tid + i * kThreads;
            *reinterpret_cast<uint4*>(&lds[buf][swz(c >> 3, c & 7)]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int c = tid + i * kThreads;
            *reinterpret_cast<uint4*>(&lds[buf][BM * kRowBytes + swz(c >> 3, c & 7)]) = rb[i];
        }
    };

    uint32_t sa_lo[WM], sa_hi[WM], sb_lo[WN], sb_hi[WN];
    uint32_t na_lo[WM], na_hi[WM], nb_lo[WN], nb_hi[WN];
    auto sload = [&](int kt, uint32_t* alo, uint32_t* ahi, uint32_t* blo, uint32_t* bhi) {
#pragma unroll
        for (int i = 0; i < WM; ++i) {
            int64_t r = m0 + wm * WM * 32 + i * 32 + l32;
            r = r < M ? r : M - 1;
            load_scales8(SA, r, ks, kt, svec, alo[i], ahi[i]);
        }
#pragma unroll
        for (int j = 0; j < WN; ++j) {
            int64_t r = n0 + wn * WN * 32 + j * 32 + l32;
            r = r < N ? r : N - 1;
            load_scales8(SB, r, ks, kt, svec, blo[j], bhi[j]);
        }
    };

    v16f acc[WM][WN];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    gload(0);
    sload(0, sa_lo, sa_hi, sb_lo, sb_hi);
    lstore(0);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            gload(kt + 1);
            sload(kt + 1, na_lo, na_hi, nb_lo, nb_hi);
        }
        const uint8_t* la = &lds[buf][0];
        const uint8_t* lb = &lds[buf][BM * kRowBytes];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            v8i af[WM], bf[WN];
            uint32_t sca[WM], scb[WN];
            const int shift = 8 * (2 * (s & 1) + h);
#pragma unroll
            for (int i = 0; i < WM; ++i) {
                const uint4 v = *reinterpret_cast<const uint4*>(la + swz(wm * WM * 32 + i * 32 + l32, 2 * s + h));
                af[i] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
                sca[i] = ((s < 2 ? sa_lo[i] : sa_hi[i]) >> shift) & 0xFFu;
            }
#pragma unroll
            for (int j = 0; j < WN; ++j) {
                const uint4 v = *reinterpret_cast<const uint4*>(lb + swz(wn * WN * 32 + j * 32 + l32, 2 * s + h));
                bf[j] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
                scb[j] = ((s < 2 ? sb_lo[j] : sb_hi[j]) >> shift) & 0xFFu;
            }
#pragma unroll
            for (int i = 0; i < WM; ++i)
#pragma unroll
                for (int j = 0; j < WN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        af[i], bf[j], acc[i][j], 4, 4, 0, (int)sca[i], 0, (int)scb[j]);
        }
        if (more) {
            lstore(buf ^ 1);
#pragma unroll
            for (int i = 0; i < WM; ++i) { sa_lo[i] = na_lo[i]; sa_hi[i] = na_hi[i]; }
#pragma unroll
            for (int j = 0; j < WN; ++j) { sb_lo[j] = nb_lo[j]; sb_hi[j] = nb_hi[j]; }
        }
        __syncthreads();
    }

    // accumulator layout of a 32x32 tile: register r of lane l holds
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
    for (int i = 0; i < WM; ++i) {
#pragma unroll
        for (int j = 0; j < WN; ++j) {
            const int64_t col = n0 + wn * WN * 32 + j * 32 + l32;
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * WM * 32 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (row < M) C[row * N + col] = acc[i][j][r];
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_mx(const uint8_t* aq, const uint8_t* as, const uint8_t* bq,
                          const uint8_t* bs, int64_t M, int64_t N, int64_t K, float* c,
                          hipStream_t st) {
    constexpr int WM = 2, WN = 2;
    const int64_t tm = (M + 64 * WM - 1) / (64 * WM), tn = (N + 64 * WN - 1) / (64 * WN);
    hipLaunchKernelGGL((gemm_mx_tn<WM, WN>), dim3((unsigned)(tm * tn)), dim3(kThreads), 0, st,
                       aq, as, bq, bs, M, N, K, c, (int)tn);
    return hipGetLastError();
}

}  // namespace fp4dev

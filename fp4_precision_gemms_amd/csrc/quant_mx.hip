// quant_mx.hip -- Hadamard rotation + MXFP4 quantization kernels for gfx950.
//
// Block format: [AMD-MXFP4] "Pretraining large language models with MXFP4 on
// Native FP4 Hardware", section "Что такое MXFP4": 32-element blocks sharing
// one E8M0 exponent, E2M1 elements rounded to the nearest value.  Rotation:
// same page, section "Поисковая экспериментальная работа: корень
// нестабильности": a Hadamard transform, deterministic or after random sign
// flips, applied before quantization.
//
// Output layouts (those the GEMM loads), for an output of R rows (the
// logical rows of x or x^T) and nb blocks per row:
//   - codes, 32-row tiled: the 16 code bytes of block b of row r at
//     ((r / 32) nb + b) * 512 + 16 (r mod 32), i.e. for each group of 32
//     rows and each block one contiguous 512-byte chunk.  Rows of the last
//     group past R are not written.
//   - scales, k-grouped: block b of row r at byte ((b / 8) R + r) * 8 +
//     b mod 8.  Bytes of the last group past nb are not written.
//
// Kernels, by block axis:
//   quant_mx_along_cols -- blocks run along the contiguous dim.  A workgroup
//     owns 32 rows x 256 columns; a lane owns 8 consecutive elements (one
//     16-byte load); four adjacent lanes own a block.  The first three
//     butterfly stages are in registers, the strides 8 and 16 cross lanes
//     through DPP quad permutes, the block maximum is a two-step DPP
//     reduction, and each lane stores its 8 codes as one dword: the
//     workgroup writes 8 whole 512-byte chunks.
//   quant_mx_along_rows_lds -- blocks run along the strided dim (x^T is
//     quantized, as Wgrad needs: blocks along tokens).  32 x 256 bf16 tiles
//     go global -> LDS by DMA, one thread per column transposes through LDS,
//     and the codes leave through an LDS staging array in column-major
//     store instructions.  Used whenever cols % 8 == 0 and the input is
//     below 2 GiB.
//   quant_mx_along_rows -- the same axis, any column count: a lane owns CPL
//     adjacent columns and RBW consecutive 32-row blocks of each: per block
//     it issues 32 row loads (adjacent lanes read adjacent columns, so every
//     load instruction reads one contiguous 64*CPL*2-byte row segment), then
//     transforms, reduces and encodes each column in registers; its RBW
//     blocks of one column are 16*RBW contiguous code bytes.
//
// Element encoding.  The block maximum is taken on the butterfly outputs a_i
// before the binary32 multiply by c = fl(1/sqrt(n)): rounding is monotone,
// so max_i |fl(c a_i)| = fl(c max_i |a_i|).  With the scale 2^e normal
// (scale byte 1..254) the codes come from V_CVT_SCALEF32_PK_FP4_F32, which
// rounds y / 2^e to the nearest E2M1 value, ties to even, saturating at 6 --
// for a power-of-two scale the same code as rounding the exact binary32
// product y * 2^-e; two elements per instruction, packed even-low.  Scale
// byte 0 (2^-127, not a normal binary32) and stochastic rounding take the
// integer encoders of fp4_device.hpp.
#include "fp4_device.hpp"
#include "fp4_launch.hpp"

namespace fp4dev {
namespace {

// Quad permutes: partner lane q^1 and q^2 inside each group of four lanes.
__device__ __forceinline__ uint32_t quad_xor1(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // [1,0,3,2]
}
__device__ __forceinline__ uint32_t quad_xor2(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);   // [2,3,0,1]
}
__device__ __forceinline__ float quad_xor1f(float v) { return __uint_as_float(quad_xor1(__float_as_uint(v))); }
__device__ __forceinline__ float quad_xor2f(float v) { return __uint_as_float(quad_xor2(__float_as_uint(v))); }

// In-register butterflies with strides 1 .. N/2 over a[0..N-1].
template <int N>
__device__ __forceinline__ void butterflies(float* a) {
#pragma unroll
    for (int h = 1; h < N; h <<= 1) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            if (i & h) continue;
            const float x = a[i], y = a[i + h];
            a[i] = x + y;
            a[i + h] = x - y;
        }
    }
}

// Largest |a_i| of n values as binary32 bits (NaN > Inf > finite).
template <int N>
__device__ __forceinline__ uint32_t max_abs_bits(const float* a) {
    uint32_t m = 0;
#pragma unroll
    for (int t = 0; t < N; ++t) m = max(m, __float_as_uint(a[t]) & 0x7FFFFFFFu);
    return m;
}

// Codes of 8 values y[0..7] under scale byte `byte` (1..254): hardware
// round-to-nearest-even of y / 2^(byte-127), element 2k in nibble 2k.
__device__ __forceinline__ uint32_t encode8_hw(const float* y, uint32_t byte) {
    const float s = __uint_as_float(byte << 23);
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], s, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], s, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], s, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], s, 3);
    return w;
}

// Integer encoders: v_t = y_t * 2^-(byte-127) in binary32, then RTN or SR.
template <bool SR>
__device__ __forceinline__ uint32_t encode8_sw(const float* y, uint32_t byte, uint4 u0, uint4 u1) {
    const float inv = inv_scale_from_e8m0(byte);
    uint32_t w = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const float v = y[t] * inv;
        uint32_t c;
        if constexpr (SR) c = e2m1_sr(v, word_of(t < 4 ? u0 : u1, t & 3));
        else c = e2m1_rtn(v);
        w |= c << (4 * t);
    }
    return w;
}

constexpr int kColsThreads = 256;
constexpr int kColsUnroll = 4;

// Byte offset of the 16 code bytes of (row r, block b) in the 32-row tiled
// layout of an operand with nb blocks per row: chunk (r / 32, b) of 512
// bytes, row r mod 32 at 16 (r mod 32).
__device__ __forceinline__ int64_t tiled_offset(int64_t r, int64_t b, int64_t nb) {
    return ((r >> 5) * nb + b) * 512 + (r & 31) * 16;
}

// Blocks along cols.  A workgroup owns 32 rows x 256 columns (8 blocks per
// row): chunk i = u * 256 + tid of its kColsUnroll x 256 16-byte loads is
// row i / 32, 8-column chunk i mod 32, so each wave load instruction reads
// two 512-byte row segments and a lane quad holds one 32-element block.
// The workgroup's codes are 8 whole chunks of the tiled layout (4 KB).
// HADN: 0 (no rotation), 16 or 32.
template <int HADN, bool SR>
__global__ __launch_bounds__(kColsThreads) void quant_mx_along_cols(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, uint32_t sign_word, float norm,
    uint64_t sr_seed, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    const int64_t nb = cols / 32;
    const int64_t gx = (cols + 255) / 256;           // workgroups per row group (1-D grid)
    const int64_t c0 = ((int64_t)blockIdx.x % gx) * 256, r0 = ((int64_t)blockIdx.x / gx) * 32;
    const int tid = threadIdx.x;
    const int q = tid & 3;                         // lane within the block of 4
    uint4 w[kColsUnroll];
    int64_t row[kColsUnroll], col[kColsUnroll];
    bool in[kColsUnroll];
#pragma unroll
    for (int u = 0; u < kColsUnroll; ++u) {
        const int i = u * kColsThreads + tid;
        row[u] = r0 + (i >> 5);
        col[u] = c0 + (i & 31) * 8;
        in[u] = row[u] < rows && col[u] < cols;    // uniform per quad: cols % 32 == 0
        if (in[u]) w[u] = *reinterpret_cast<const uint4*>(x + row[u] * cols + col[u]);
    }
    // sign-bit masks of the cross-lane butterfly stages: the upper lane of a
    // pair computes partner - own as partner + (-own)
    const uint32_t neg1 = (uint32_t)(q & 1) << 31, neg2 = (uint32_t)((q >> 1) & 1) << 31;
#pragma unroll
    for (int u = 0; u < kColsUnroll; ++u) {
        if (!in[u]) continue;
        float a[8] = {bf16_lo(w[u].x), bf16_hi(w[u].x), bf16_lo(w[u].y), bf16_hi(w[u].y),
                      bf16_lo(w[u].z), bf16_hi(w[u].z), bf16_lo(w[u].w), bf16_hi(w[u].w)};
        if constexpr (HADN != 0) {
            const int sbase = (8 * q) % HADN;
#pragma unroll
            for (int t = 0; t < 8; ++t) a[t] = flip_if(a[t], (sign_word >> (sbase + t)) & 1u);
            butterflies<8>(a);
            // stride 8: pair (i, i+8) lives in lanes (q, q^1)
#pragma unroll
            for (int t = 0; t < 8; ++t)
                a[t] = quad_xor1f(a[t]) + __uint_as_float(__float_as_uint(a[t]) ^ neg1);
            if constexpr (HADN == 32) {
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    a[t] = quad_xor2f(a[t]) + __uint_as_float(__float_as_uint(a[t]) ^ neg2);
            }
        }
        // block maximum of |a| as unsigned bits, then of |c a| (monotone rounding)
        uint32_t m = max_abs_bits<8>(a);
        m = max(m, quad_xor1(m));
        m = max(m, quad_xor2(m));
        if constexpr (HADN != 0) {
            m = __float_as_uint(__uint_as_float(m) * norm) & 0x7FFFFFFFu;
#pragma unroll
            for (int t = 0; t < 8; ++t) a[t] = a[t] * norm;
        }
        const uint32_t byte = e8m0_from_amax_bits(m);
        uint32_t word = 0;
        if (byte != 255u) {
            if (!SR && byte != 0u) {
                word = encode8_hw(a, byte);
            } else {
                uint4 u0 = make_uint4(0, 0, 0, 0), u1 = u0;
                if constexpr (SR) {
                    // elements idx .. idx+7 (idx = row * cols + col): counters idx/4, idx/4 + 1
                    const uint64_t g = ((uint64_t)row[u] * (uint64_t)cols + (uint64_t)col[u]) >> 2;
                    u0 = stream4(sr_seed, 0u, g);
                    u1 = stream4(sr_seed, 0u, g + 1);
                }
                word = encode8_sw<SR>(a, byte, u0, u1);
            }
        }
        const int64_t b = col[u] >> 5;
        *reinterpret_cast<uint32_t*>(codes + tiled_offset(row[u], b, nb) + 4 * q) = word;
        if (q == 0) scales[((b >> 3) * rows + row[u]) * 8 + (b & 7)] = (uint8_t)byte;
    }
}

template <int CPL> struct ColVec;
template <> struct ColVec<1> { using T = uint16_t; };
template <> struct ColVec<2> { using T = uint32_t; };
template <> struct ColVec<4> { using T = uint2; };
template <> struct ColVec<8> { using T = uint4; };

template <int CPL>
__device__ __forceinline__ float col_value(const typename ColVec<CPL>::T& v, int c) {
    if constexpr (CPL == 1) {
        return __uint_as_float((uint32_t)v << 16);
    } else if constexpr (CPL == 2) {
        return c == 0 ? bf16_lo(v) : bf16_hi(v);
    } else if constexpr (CPL == 4) {
        const uint32_t w = c < 2 ? v.x : v.y;
        return (c & 1) ? bf16_hi(w) : bf16_lo(w);
    } else {
        const uint32_t w = c < 2 ? v.x : c < 4 ? v.y : c < 6 ? v.z : v.w;
        return (c & 1) ? bf16_hi(w) : bf16_lo(w);
    }
}

constexpr int kRowsWaves = 4;

// One lane: CPL columns x RBW consecutive 32-row blocks.  The RBW scale
// bytes of a column are contiguous and leave as one RBW-byte store.
template <int CPL, int HADN, bool SR, int RBW>
__global__ __launch_bounds__(64 * kRowsWaves) void quant_mx_along_rows(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, uint32_t sign_word, float norm,
    uint64_t sr_seed, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    static_assert(RBW == 4, "scale bytes of a lane are packed into one word");
    using V = typename ColVec<CPL>::T;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t col0 = ((int64_t)blockIdx.x * 64 + lane) * CPL;
    if (col0 >= cols) return;                      // no cross-lane work in this kernel
    const int64_t nrb = rows / 32;
    const int64_t rb0 = ((int64_t)blockIdx.y * kRowsWaves + wave) * RBW;
    if (rb0 >= nrb) return;
    const int64_t vstride = cols / CPL;
    uint32_t sword[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) sword[c] = 0;
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
        const int64_t rb = rb0 + i;
        if (rb >= nrb) break;
        V v[32];
        const V* src = reinterpret_cast<const V*>(x + rb * 32 * cols + col0);
#pragma unroll
        for (int r = 0; r < 32; ++r) v[r] = src[r * vstride];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            float a[32];
#pragma unroll
            for (int r = 0; r < 32; ++r) a[r] = col_value<CPL>(v[r], c);
            if constexpr (HADN != 0) {
#pragma unroll
                for (int r = 0; r < 32; ++r) a[r] = flip_if(a[r], (sign_word >> (r % HADN)) & 1u);
#pragma unroll
                for (int o = 0; o < 32; o += HADN) butterflies<HADN>(a + o);
            }
            uint32_t m = max_abs_bits<32>(a);
            if constexpr (HADN != 0) {
                m = __float_as_uint(__uint_as_float(m) * norm) & 0x7FFFFFFFu;
#pragma unroll
                for (int r = 0; r < 32; ++r) a[r] = a[r] * norm;
            }
            const uint32_t byte = e8m0_from_amax_bits(m);
            const int64_t col = col0 + c;
            uint4 out = make_uint4(0, 0, 0, 0);
            if (byte != 255u) {
                uint32_t wd[4];
                if (!SR && byte != 0u) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) wd[k] = encode8_hw(a + 8 * k, byte);
                } else {
                    const uint64_t gbase = ((uint64_t)col * (uint64_t)rows + (uint64_t)rb * 32) >> 2;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        uint4 u0 = make_uint4(0, 0, 0, 0), u1 = u0;
                        if constexpr (SR) {
                            u0 = stream4(sr_seed, 0u, gbase + 2 * k);
                            u1 = stream4(sr_seed, 0u, gbase + 2 * k + 1);
                        }
                        wd[k] = encode8_sw<SR>(a + 8 * k, byte, u0, u1);
                    }
                }
                out = make_uint4(wd[0], wd[1], wd[2], wd[3]);
            }
            *reinterpret_cast<uint4*>(codes + tiled_offset(col, rb, nrb)) = out;
            sword[c] |= byte << (8 * i);
        }
    }
    // scale bytes rb0 .. rb0+3 of each column (half of a k-group, rb0 a
    // multiple of 4): one aligned word when all four blocks exist
    const bool word_ok = rb0 + RBW <= nrb;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        uint8_t* dst = scales + ((rb0 >> 3) * cols + col0 + c) * 8 + (rb0 & 7);
        if (word_ok) {
            *reinterpret_cast<uint32_t*>(dst) = sword[c];
        } else {
            for (int i = 0; i < RBW && rb0 + i < nrb; ++i) dst[i] = (uint8_t)(sword[c] >> (8 * i));
        }
    }
}


typedef __attribute__((address_space(3))) void lds_void_t;

// Wave-wide DMA: each lane's 16 bytes at voff of the buffer go to LDS at
// lds_dst + 16 * lane (lds_dst wave-uniform).  The input is read once, so the
// load is marked non-temporal (cache policy bit 1, NT).  Measured on the
// Wgrad pair dY[8192x14336] + X[8192x4096]: 64 us instead of 70 us back to
// back, and the whole Llama-3.1-8B gate/up linear layer 5 % faster.  Marking
// the code stores non-temporal too speeds the quantizer alike but slows the
// GEMM that reads the codes next (they then miss the caches); the same hint
// on the along-cols and NVFP4 kernels' plain loads measured no gain.
__device__ __forceinline__ void dma16_to_lds(__amdgpu_buffer_rsrc_t rsrc, void* lds_dst, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds_dst, 16, voff, 0, 0, 2);
}

constexpr int kTileCols = 256;           // columns per block, one per thread

// Rotation, scale and codes of one 32-element block held by one thread: a[]
// holds the block's values in order; gbase is the logical index (in the
// quantized [R, C] layout) of the block's first element divided by 4, the SR
// counter of its first four elements.  Returns the scale byte; wd gets the
// 16 code bytes (zero for a NaN / infinite block).
template <int HADN, bool SR>
__device__ __forceinline__ uint32_t quant_block32(float* a, uint32_t sign_word, float norm,
                                                  uint64_t sr_seed, uint64_t gbase, uint32_t* wd) {
    if constexpr (HADN != 0) {
#pragma unroll
        for (int r = 0; r < 32; ++r) a[r] = flip_if(a[r], (sign_word >> (r % HADN)) & 1u);
#pragma unroll
        for (int o = 0; o < 32; o += HADN) butterflies<HADN>(a + o);
    }
    uint32_t m = max_abs_bits<32>(a);
    if constexpr (HADN != 0) {
        m = __float_as_uint(__uint_as_float(m) * norm) & 0x7FFFFFFFu;
#pragma unroll
        for (int r = 0; r < 32; ++r) a[r] = a[r] * norm;
    }
    const uint32_t byte = e8m0_from_amax_bits(m);
#pragma unroll
    for (int k = 0; k < 4; ++k) wd[k] = 0;
    if (byte != 255u) {
        if (!SR && byte != 0u) {
#pragma unroll
            for (int k = 0; k < 4; ++k) wd[k] = encode8_hw(a + 8 * k, byte);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                uint4 u0 = make_uint4(0, 0, 0, 0), u1 = u0;
                if constexpr (SR) {
                    u0 = stream4(sr_seed, 0u, gbase + 2 * k);
                    u1 = stream4(sr_seed, 0u, gbase + 2 * k + 1);
                }
                wd[k] = encode8_sw<SR>(a + 8 * k, byte, u0, u1);
            }
        }
    }
    return byte;
}

// s_waitcnt vmcnt(N) (N <= 63), leaving the other counters alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// Waits until at most 4 (TB - 1 - t) DMA instructions are outstanding: the
// four of tile t and all before it have landed (t < TB <= 8).
template <int TB>
__device__ __forceinline__ void wait_tile(int t) {
    switch (t) {
    case 0: wait_vmcnt<(TB > 0 ? 4 * (TB - 1) : 0)>(); break;
    case 1: wait_vmcnt<(TB > 1 ? 4 * (TB - 2) : 0)>(); break;
    case 2: wait_vmcnt<(TB > 2 ? 4 * (TB - 3) : 0)>(); break;
    case 3: wait_vmcnt<(TB > 3 ? 4 * (TB - 4) : 0)>(); break;
    case 4: wait_vmcnt<(TB > 4 ? 4 * (TB - 5) : 0)>(); break;
    case 5: wait_vmcnt<(TB > 5 ? 4 * (TB - 6) : 0)>(); break;
    case 6: wait_vmcnt<(TB > 6 ? 4 * (TB - 7) : 0)>(); break;
    default: wait_vmcnt<0>(); break;
    }
}

// Blocks along rows, staged through LDS: a workgroup owns 256 adjacent
// columns and TB consecutive 32-row blocks.  All TB 32 x 256 bf16 tiles go
// global -> LDS by DMA up front (each wave instruction moves two 512-byte
// row segments); tile t is processed once its DMA has landed.  Thread c
// owns column c: it reads the column's 32 values of a tile from LDS
// (consecutive lanes, consecutive columns: conflict-free), transforms and
// encodes them; at the end the TB blocks' codes of a column (16 TB
// contiguous bytes) leave through LDS in column-major store instructions and
// the TB scale bytes as one word.  Needs cols % 8 == 0.
//
// HADN_C >= 0 adds a second output from the same tiles: x quantized along
// cols (blocks of 32 consecutive columns, rotation size HADN_C, 0 = none,
// rounding to nearest), one (row, 32-column block) of each tile per thread,
// read as four 16-byte LDS loads.  Needs cols % 32 == 0 then.
//
// A second input (x2 [rows, cols2], its own outputs and SR seed) may share
// the launch: the grid is then 1-D, its first n_first workgroups (gx1 wide)
// work on x and the rest (gx2 wide) on x2 -- the two Wgrad operands, same
// rows, same rotation.
struct RowsLdsSecond {
    const uint16_t* x;
    int64_t cols;
    uint64_t sr_seed;
    uint8_t* codes;
    uint8_t* scales;
    int64_t n_first, gx1, gx2;   // n_first = 0: single input, 2-D grid
};

template <int HADN, bool SR, int TB, int HADN_C>
__global__ __launch_bounds__(kTileCols) void quant_mx_along_rows_lds(
    const uint16_t* __restrict__ x_in, int64_t rows, int64_t cols_in, uint32_t sign_word, float norm,
    uint64_t sr_seed_in, uint8_t* __restrict__ codes_in, uint8_t* __restrict__ scales_in,
    uint32_t sign_word_c, float norm_c, uint64_t sr_seed_c, uint8_t* __restrict__ codes_c,
    uint8_t* __restrict__ scales_c, RowsLdsSecond second) {
    static_assert(TB == 2, "two blocks per workgroup: one 64-element k-step of the tiled codes");
    constexpr int kTileBlocks = TB;
    __shared__ __attribute__((aligned(1024))) uint16_t tile[kTileBlocks][32 * kTileCols];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // which input and which (column strip, row-block group) this workgroup owns
    int64_t bx = blockIdx.x, by = blockIdx.y;
    const uint16_t* x = x_in;
    int64_t cols = cols_in;
    uint64_t sr_seed = sr_seed_in;
    uint8_t* codes = codes_in;
    uint8_t* scales = scales_in;
    if (second.n_first > 0) {
        const int64_t w = blockIdx.x;
        if (w < second.n_first) {
            bx = w % second.gx1;
            by = w / second.gx1;
        } else {
            bx = (w - second.n_first) % second.gx2;
            by = (w - second.n_first) / second.gx2;
            x = second.x; cols = second.cols; sr_seed = second.sr_seed;
            codes = second.codes; scales = second.scales;
        }
    }
    const int64_t c0 = (int64_t)__builtin_amdgcn_readfirstlane((int)bx) * kTileCols;
    const int64_t nrb = rows / 32;
    const int64_t rb0 = (int64_t)__builtin_amdgcn_readfirstlane((int)by) * kTileBlocks;
    const int nt = (int)((nrb - rb0) < kTileBlocks ? (nrb - rb0) : kTileBlocks);
    // the whole input as one buffer: offsets are 32-bit, the caller bounds
    // rows * cols * 2 below 2^31; segments past the last row read as zero
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)x, (short)0, (int)(rows * cols * 2), 0x00020000);
    // DMA instruction j of a tile (4 per wave) covers rows 2j, 2j+1:
    // lane i -> row 2j + i / 32, LDS slot i mod 32 of the row segment, which
    // holds 16-byte chunk (i mod 32) XOR (row mod 4): the swizzle keeps the
    // per-column reads conflict-free and makes the per-row 16-byte reads of
    // the along-cols output conflict-free too.
    // Every tile is issued, also those past the last row (they read zeros),
    // so that the wait counts below are the same for every workgroup.
    const int64_t nbytes = rows * cols * 2;
#pragma unroll
    for (int t = 0; t < kTileBlocks; ++t) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int j = wave * 4 + k;
            const int64_t row = (rb0 + t) * 32 + 2 * j + (lane >> 5);
            const int64_t o = (row * cols + c0) * 2 + (int64_t)((((lane & 31) ^ (int)(row & 3))) * 16);
            dma16_to_lds(rx, (uint8_t*)tile[t] + j * 1024, o < nbytes ? (uint32_t)o : 0x80000000u);
        }
    }
    const int64_t col = c0 + tid;
    // LDS position (bf16 units, within a row) of this thread's column for row
    // mod 4 = q: its 8-column chunk XOR q
    int colpos[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) colpos[q] = (((tid >> 3) ^ q) << 3) | (tid & 7);
    uint32_t wd[kTileBlocks][4] = {};
    uint64_t sword = 0;
#pragma unroll
    for (int t = 0; t < kTileBlocks; ++t) {
        if (t >= nt) break;
        // this wave's DMA of tiles 0..t has landed (4 instructions per tile,
        // issued in order); the barrier publishes every wave's part
        wait_tile<TB>(t);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float a[32];
#pragma unroll
        for (int r = 0; r < 32; ++r) a[r] = __uint_as_float((uint32_t)tile[t][r * kTileCols + colpos[r & 3]] << 16);
        const uint64_t gbase = ((uint64_t)col * (uint64_t)rows + (uint64_t)(rb0 + t) * 32) >> 2;
        const uint32_t byte = quant_block32<HADN, SR>(a, sign_word, norm, sr_seed, gbase, wd[t]);
        if constexpr (HADN_C >= 0) {
            // the same tile along cols: each 16-lane group of a wave takes 4
            // rows x 4 blocks, so with the chunk swizzle its 16-byte reads of
            // chunk k hit 16 different bank groups
            const int grp = lane >> 4;
            const int r = 8 * wave + 4 * (grp & 1) + ((lane >> 2) & 3), b = 4 * (grp >> 1) + (lane & 3);
            const int64_t row = (rb0 + t) * 32 + r, cb = c0 + 32 * b;
            if (cb < cols) {
                float ar[32];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint4 v = *reinterpret_cast<const uint4*>(
                        &tile[t][r * kTileCols + (((4 * b + k) ^ (r & 3)) << 3)]);
                    ar[8 * k + 0] = bf16_lo(v.x); ar[8 * k + 1] = bf16_hi(v.x);
                    ar[8 * k + 2] = bf16_lo(v.y); ar[8 * k + 3] = bf16_hi(v.y);
                    ar[8 * k + 4] = bf16_lo(v.z); ar[8 * k + 5] = bf16_hi(v.z);
                    ar[8 * k + 6] = bf16_lo(v.w); ar[8 * k + 7] = bf16_hi(v.w);
                }
                uint32_t wc[4];
                const uint64_t gb = ((uint64_t)row * (uint64_t)cols + (uint64_t)cb) >> 2;
                const uint32_t bc = quant_block32<HADN_C, false>(ar, sign_word_c, norm_c, sr_seed_c, gb, wc);
                *reinterpret_cast<uint4*>(codes_c + tiled_offset(row, cb / 32, cols / 32)) =
                    make_uint4(wc[0], wc[1], wc[2], wc[3]);
                const int64_t blk = cb / 32;
                scales_c[((blk >> 3) * rows + row) * 8 + (blk & 7)] = (uint8_t)bc;
            }
        }
        sword |= (uint64_t)byte << (8 * t);
    }
    // DMA into tiles past the last row must land before the tiles are reused
    // (and before the workgroup ends)
    __builtin_amdgcn_s_waitcnt(0x0F70);
    // Codes leave through LDS: thread c's 16 TB bytes go to row c of a
    // [256][16 TB + 16 byte] staging array (the 16-byte pad makes both the
    // row writes and the chunk reads below conflict-free), then each wave
    // stores 64 / TB columns x 16 TB bytes per instruction (TB lanes per
    // column) instead of 64 columns x 16 bytes.  The staging array overlays
    // the tiles.
    __syncthreads();                                   // every tile has been read
    constexpr int kStageRow = 16 * TB + 16;
    static_assert(kTileCols * kStageRow <= (int)sizeof(tile), "staging fits the tiles");
    uint8_t* stg = reinterpret_cast<uint8_t*>(&tile[0][0]);
#pragma unroll
    for (int t = 0; t < kTileBlocks; ++t)
        *reinterpret_cast<uint4*>(stg + tid * kStageRow + 16 * t) =
            make_uint4(wd[t][0], wd[t][1], wd[t][2], wd[t][3]);
    __syncthreads();
    // lane = 32 chunk + (column mod 32): with TB = 2 the two chunks of a
    // 32-column group are adjacent 512-byte chunks of the tiled layout, so
    // each store instruction writes 1 KB contiguous
#pragma unroll
    for (int i = 0; i < TB; ++i) {
        const int c = wave * 64 + i * 32 + (lane & 31), chunk = lane >> 5;
        const uint4 v = *reinterpret_cast<const uint4*>(stg + c * kStageRow + 16 * chunk);
        if (chunk < nt && c0 + c < cols)
            *reinterpret_cast<uint4*>(codes + tiled_offset(c0 + c, rb0 + chunk, nrb)) = v;
    }
    if (col >= cols) return;
    // rb0 is a multiple of TB: blocks rb0 .. rb0+TB-1 lie in one k-group
    uint8_t* sdst = scales + ((rb0 >> 3) * cols + col) * 8 + (rb0 & 7);
    if (nt == kTileBlocks) {
        if constexpr (TB == 2) *reinterpret_cast<uint16_t*>(sdst) = (uint16_t)sword;
        else if constexpr (TB == 4) *reinterpret_cast<uint32_t*>(sdst) = (uint32_t)sword;
        else *reinterpret_cast<uint64_t*>(sdst) = sword;
    } else {
        for (int t = 0; t < nt; ++t) sdst[t] = (uint8_t)(sword >> (8 * t));
    }
}

template <int HADN, bool SR>
hipError_t launch_cols(const void* x, int64_t rows, int64_t cols, uint32_t sign_word, float norm,
                       uint64_t sr_seed, uint8_t* codes, uint8_t* scales, hipStream_t st) {
    const int64_t blocks = ((cols + 255) / 256) * ((rows + 31) / 32);
    return launch(&quant_mx_along_cols<HADN, SR>, dim3((unsigned)blocks), dim3(kColsThreads), st,
                  (const uint16_t*)x, rows, cols, sign_word, norm, sr_seed, codes, scales);
}

template <int CPL, int HADN, bool SR>
hipError_t launch_rows(const void* x, int64_t rows, int64_t cols, uint32_t sign_word, float norm,
                       uint64_t sr_seed, uint8_t* codes, uint8_t* scales, hipStream_t st) {
    constexpr int RBW = 4;
    const int64_t nrb = rows / 32;
    const int64_t gx = (cols + 64 * CPL - 1) / (64 * CPL);
    const int64_t gy = (nrb + kRowsWaves * RBW - 1) / (kRowsWaves * RBW);
    return launch(&quant_mx_along_rows<CPL, HADN, SR, RBW>, dim3((unsigned)gx, (unsigned)gy),
                  dim3(64 * kRowsWaves), st, (const uint16_t*)x, rows, cols, sign_word, norm, sr_seed,
                  codes, scales);
}

// 32-row blocks per workgroup of the LDS kernel: two (32 KB of LDS) keeps
// five workgroups' DMA in flight per CU; measured on dY[8192x14336] and
// X[8192x4096], two is as fast as four on the large input and 10 % faster on
// the small one, and eight (one workgroup per CU) is 1.5-1.8x slower.
constexpr int kRowsLdsBlocks = 2;

template <int HADN, bool SR>
hipError_t dispatch_rows_cpl(const void* x, int64_t rows, int64_t cols, uint32_t sign_word,
                             float norm, uint64_t sr_seed, uint8_t* codes, uint8_t* scales,
                             hipStream_t st) {
    if (cols % 8 == 0 && rows * cols * 2 < (INT64_C(1) << 31)) {
        const int64_t gx = (cols + kTileCols - 1) / kTileCols;
        constexpr int TB = kRowsLdsBlocks;
        const int64_t gy = (rows / 32 + TB - 1) / TB;
        return launch(&quant_mx_along_rows_lds<HADN, SR, TB, -1>, dim3((unsigned)gx, (unsigned)gy),
                      dim3(kTileCols), st, (const uint16_t*)x, rows, cols, sign_word, norm, sr_seed,
                      codes, scales, 0u, 1.0f, (uint64_t)0, (uint8_t*)nullptr, (uint8_t*)nullptr,
                      RowsLdsSecond{});
    }
    if (cols % 4 == 0) return launch_rows<4, HADN, SR>(x, rows, cols, sign_word, norm, sr_seed, codes, scales, st);
    if (cols % 2 == 0) return launch_rows<2, HADN, SR>(x, rows, cols, sign_word, norm, sr_seed, codes, scales, st);
    return launch_rows<1, HADN, SR>(x, rows, cols, sign_word, norm, sr_seed, codes, scales, st);
}

template <int HADN>
hipError_t dispatch_rnd(int axis, bool sr, const void* x, int64_t rows, int64_t cols,
                        uint32_t sign_word, float norm, uint64_t sr_seed, uint8_t* codes,
                        uint8_t* scales, hipStream_t st) {
    if (axis == 0) {
        return sr ? launch_cols<HADN, true>(x, rows, cols, sign_word, norm, sr_seed, codes, scales, st)
                  : launch_cols<HADN, false>(x, rows, cols, sign_word, norm, sr_seed, codes, scales, st);
    }
    return sr ? dispatch_rows_cpl<HADN, true>(x, rows, cols, sign_word, norm, sr_seed, codes, scales, st)
              : dispatch_rows_cpl<HADN, false>(x, rows, cols, sign_word, norm, sr_seed, codes, scales, st);
}

// Both outputs from one pass over the tiles (the rows output is the one the
// kernel's template arguments HADN / SR describe).
template <int HADN, bool SR, int HADN_C>
hipError_t launch_dual(const void* x, int64_t rows, int64_t cols, uint32_t sign_word, float norm,
                       uint64_t sr_seed, uint8_t* codes, uint8_t* scales, uint32_t sign_word_c,
                       float norm_c, uint64_t sr_seed_c, uint8_t* codes_c,
                       uint8_t* scales_c, hipStream_t st) {
    constexpr int TB = kRowsLdsBlocks;
    const int64_t gx = (cols + kTileCols - 1) / kTileCols;
    const int64_t gy = (rows / 32 + TB - 1) / TB;
    return launch(&quant_mx_along_rows_lds<HADN, SR, TB, HADN_C>, dim3((unsigned)gx, (unsigned)gy),
                  dim3(kTileCols), st, (const uint16_t*)x, rows, cols, sign_word, norm, sr_seed, codes,
                  scales, sign_word_c, norm_c, sr_seed_c, codes_c, scales_c, RowsLdsSecond{});
}

template <int HADN, bool SR>
hipError_t dispatch_dual_c(int hadn_c, const void* x, int64_t rows, int64_t cols, uint32_t sign_word,
                           float norm, uint64_t sr_seed, uint8_t* codes, uint8_t* scales,
                           uint32_t sign_word_c, float norm_c, uint64_t sr_seed_c,
                           uint8_t* codes_c, uint8_t* scales_c, hipStream_t st) {
    if (hadn_c == 0)
        return launch_dual<HADN, SR, 0>(x, rows, cols, sign_word, norm, sr_seed, codes, scales,
                                        sign_word_c, norm_c, sr_seed_c, codes_c, scales_c, st);
    if (hadn_c == 16)
        return launch_dual<HADN, SR, 16>(x, rows, cols, sign_word, norm, sr_seed, codes, scales,
                                         sign_word_c, norm_c, sr_seed_c, codes_c, scales_c, st);
    return launch_dual<HADN, SR, 32>(x, rows, cols, sign_word, norm, sr_seed, codes, scales,
                                     sign_word_c, norm_c, sr_seed_c, codes_c, scales_c, st);
}

// Both Wgrad operands (dY [rows, n1] and X [rows, n2], blocks along rows,
// the same rotation) in one launch.
template <int HADN, bool SR>
hipError_t launch_pair(const void* a, int64_t rows, int64_t n1, const void* b, int64_t n2,
                       uint32_t sign_word, float norm, uint64_t sr_a, uint64_t sr_b, uint8_t* qa,
                       uint8_t* sa, uint8_t* qb, uint8_t* sb, hipStream_t st) {
    constexpr int TB = kRowsLdsBlocks;
    const int64_t gy = (rows / 32 + TB - 1) / TB;
    const int64_t gx1 = (n1 + kTileCols - 1) / kTileCols, gx2 = (n2 + kTileCols - 1) / kTileCols;
    const RowsLdsSecond second{(const uint16_t*)b, n2, sr_b, qb, sb, gx1 * gy, gx1, gx2};
    return launch(&quant_mx_along_rows_lds<HADN, SR, TB, -1>, dim3((unsigned)((gx1 + gx2) * gy)),
                  dim3(kTileCols), st, (const uint16_t*)a, rows, n1, sign_word, norm, sr_a, qa, sa, 0u,
                  1.0f, (uint64_t)0, (uint8_t*)nullptr, (uint8_t*)nullptr, second);
}

// Rotation size and the binary32 factor fl(1/sqrt(n)) of a (had, had_n) pair.
int rot_size(int had, int had_n) { return had == 0 ? 0 : had_n; }
float rot_norm(int n) {
    return n == 0 ? 1.0f : n == 16 ? 0.25f : __builtin_bit_cast(float, 0x3E3504F3u);
}

}  // namespace

// Host-side sign word of the randomized transform: bit j of word 0 of the
// purpose-1 Philox stream (host copy of the device generator, same rounds).
uint32_t host_sign_word(int had, uint64_t seed) {
    if (had != 2) return 0u;
    uint32_t c[4] = {0u, 0u, 1u, 0u};
    uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    for (int r = 0; r < 10; ++r) {
        if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0, n1 = (uint32_t)p1;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1, n3 = (uint32_t)p0;
        c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
    }
    return c[0];
}

hipError_t launch_quant_mx_dual(const void* x, int64_t rows, int64_t cols, int had_n_r, int had_r,
                                uint64_t sign_seed_r, int rnd_r, uint64_t sr_seed_r, uint8_t* codes_r,
                                uint8_t* scales_r, int had_n_c, int had_c, uint64_t sign_seed_c,
                                int rnd_c, uint64_t sr_seed_c, uint8_t* codes_c, uint8_t* scales_c,
                                hipStream_t st) {
    if (rows * cols * 2 >= (INT64_C(1) << 31) || rnd_c == 1) {
        // beyond the fused kernel's 32-bit buffer offsets, or stochastic
        // rounding on the along-cols output (the fused kernel rounds that
        // output to nearest only): two passes
        const hipError_t e = launch_quant_mx(x, rows, cols, 1, had_n_r, had_r, sign_seed_r, rnd_r,
                                             sr_seed_r, codes_r, scales_r, st);
        if (e != hipSuccess) return e;
        return launch_quant_mx(x, rows, cols, 0, had_n_c, had_c, sign_seed_c, rnd_c, sr_seed_c,
                               codes_c, scales_c, st);
    }
    const int nr = rot_size(had_r, had_n_r), nc = rot_size(had_c, had_n_c);
    const uint32_t sw_r = host_sign_word(had_r, sign_seed_r), sw_c = host_sign_word(had_c, sign_seed_c);
    const float fr = rot_norm(nr), fc = rot_norm(nc);
#define FP4_DUAL(HR, SRR)                                                                        \
    return dispatch_dual_c<HR, SRR>(nc, x, rows, cols, sw_r, fr, sr_seed_r, codes_r, scales_r, \
                                    sw_c, fc, sr_seed_c, codes_c, scales_c, st)
    if (rnd_r == 1) {
        if (nr == 0) FP4_DUAL(0, true);
        if (nr == 16) FP4_DUAL(16, true);
        FP4_DUAL(32, true);
    }
    if (nr == 0) FP4_DUAL(0, false);
    if (nr == 16) FP4_DUAL(16, false);
    FP4_DUAL(32, false);
#undef FP4_DUAL
}

hipError_t launch_quant_mx_pair(const void* a, int64_t rows, int64_t n1, const void* b, int64_t n2,
                                int had_n, int had, uint64_t sign_seed, int rnd, uint64_t sr_a,
                                uint64_t sr_b, uint8_t* qa, uint8_t* sa, uint8_t* qb, uint8_t* sb,
                                hipStream_t st) {
    if (n1 % 8 || n2 % 8 || rows * n1 * 2 >= (INT64_C(1) << 31) || rows * n2 * 2 >= (INT64_C(1) << 31) ||
        (rows / 32) * ((n1 + 255) / 256 + (n2 + 255) / 256) >= (INT64_C(1) << 31)) {
        // outside the fused launch's limits: one call per operand
        const hipError_t e = launch_quant_mx(a, rows, n1, 1, had_n, had, sign_seed, rnd, sr_a, qa, sa, st);
        if (e != hipSuccess) return e;
        return launch_quant_mx(b, rows, n2, 1, had_n, had, sign_seed, rnd, sr_b, qb, sb, st);
    }
    const int n = rot_size(had, had_n);
    const uint32_t sw = host_sign_word(had, sign_seed);
    const float f = rot_norm(n);
    const bool sr = rnd == 1;
#define FP4_PAIR(HN)                                                                                 \
    return sr ? launch_pair<HN, true>(a, rows, n1, b, n2, sw, f, sr_a, sr_b, qa, sa, qb, sb, st)    \
              : launch_pair<HN, false>(a, rows, n1, b, n2, sw, f, sr_a, sr_b, qa, sa, qb, sb, st)
    if (n == 0) FP4_PAIR(0);
    if (n == 16) FP4_PAIR(16);
    FP4_PAIR(32);
#undef FP4_PAIR
}

hipError_t launch_quant_mx(const void* x, int64_t rows, int64_t cols, int axis, int had_n, int had,
                           uint64_t sign_seed, int rnd, uint64_t sr_seed, uint8_t* codes,
                           uint8_t* scales, hipStream_t st) {
    const uint32_t sw = host_sign_word(had, sign_seed);
    const bool sr = rnd == 1;
    if (had == 0) return dispatch_rnd<0>(axis, sr, x, rows, cols, 0u, 1.0f, sr_seed, codes, scales, st);
    if (had_n == 16) {
        return dispatch_rnd<16>(axis, sr, x, rows, cols, sw, 0.25f, sr_seed, codes, scales, st);
    }
    // fl(1/sqrt(32)) = 0x3E3504F3
    return dispatch_rnd<32>(axis, sr, x, rows, cols, sw, __builtin_bit_cast(float, 0x3E3504F3u),
                            sr_seed, codes, scales, st);
}

}  // namespace fp4dev

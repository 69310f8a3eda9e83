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
// Kernel layout (256 threads = 4 waves as 2 x 2, block tile BM x BN, wave
// tile BM/2 x BN/2 made of 32 x 32 MFMA tiles):
//   - V_MFMA_SCALE_F32_32X32X64_F8F6F4 with both operands FP4 (format 4) and
//     fp32 accumulation.  Operand lane l supplies row (l mod 32) and k-half
//     (l div 32) of a 32 x 64 slice: 32 consecutive k = one 16-byte code
//     chunk = exactly one scale block, so the lane's scale byte is that
//     block's E8M0 scale.  The B tile is passed as the instruction's first
//     operand, so the accumulator holds C^T: lane l owns row m = l mod 32 of
//     C and four runs of four consecutive n, each stored as one 16-byte write.
//   - A stage is 256 k: 128 code bytes and 8 scale bytes per row.  Both go
//     global -> LDS by buffer_load ... lds (no VGPR round trip), double
//     buffered.  One dwordx4 instruction fills 8 rows x 128 code bytes, lane
//     i writing slot i mod 8 of row i div 8; the lane fetches chunk
//     (slot XOR row mod 8), so chunk c of row r sits at slot c XOR (r mod 8)
//     and the 32 rows a fragment read touches spread over all banks.  One
//     dword instruction fills the 8 scale bytes of 32 rows.  Rows past M
//     (or N) lie outside the buffer range and read as zero.
//   - Per stage a wave waits at one barrier, reads all its fragments and
//     scales of the stage into registers, issues the next stage's DMA into
//     the other buffer, then runs the stage's MFMAs while that DMA lands.
//   - A contraction that is not a multiple of 256 (KTAIL) zero-fills the
//     missing code chunks through out-of-range offsets and loads the last
//     stage's scales through registers with the missing blocks set to 127.
//   - Block order: workgroups are dispatched round-robin over the 8 XCDs;
//     the block index is remapped so that each XCD works on a contiguous run
//     of tiles, ordered in groups of GM tile-rows, so tiles that share A and
//     B rows meet in the same L2.
#include "fp4_device.hpp"
#include "fp4_launch.hpp"

namespace fp4dev {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kBK = 256;              // k elements per stage
constexpr int kRowBytes = kBK / 2;    // code bytes per row per stage
constexpr int kScaleBytes = kBK / 32; // scale bytes per row per stage
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int kBufferWord3 = 0x00020000;   // raw buffer, 32-bit data format
constexpr int kWaitVmcnt0 = 0x0F70;        // s_waitcnt vmcnt(0), expcnt/lgkmcnt unchanged

__device__ __forceinline__ int swz(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ (row & 7)) << 4);
}

// Wave-wide DMA: each lane's 16 (or 4) bytes at (voff + soff) of the buffer
// go to LDS at lds_dst + 16 (or 4) * lane; lds_dst must be wave-uniform.
__device__ __forceinline__ void dma16_to_lds(__amdgpu_buffer_rsrc_t rsrc, void* lds_dst,
                                             uint32_t voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds_dst, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4_to_lds(__amdgpu_buffer_rsrc_t rsrc, void* lds_dst,
                                            uint32_t voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds_dst, 4, voff, soff, 0, 0);
}

// Maps the hardware block index to a (tile_m, tile_n) pair: XCD-contiguous
// runs of logical tiles, grouped GM tile-rows at a time.
template <int GM>
__device__ __forceinline__ void tile_of_block(int b, int nb, int tm, int tn, int& tile_m, int& tile_n) {
    const int xcd = b % kXcds, idx = b / kXcds;
    const int full = nb / kXcds, rem = nb % kXcds;
    const int t = xcd * full + (xcd < rem ? xcd : rem) + idx;
    const int per_group = GM * tn;
    const int group = t / per_group, first_m = group * GM;
    const int gm = (tm - first_m) < GM ? (tm - first_m) : GM;
    const int r = t - group * per_group;
    tile_m = first_m + r % gm;
    tile_n = r / gm;
}

// The 8 scale bytes of stage kt of one row, blocks at or past ks read as
// 127 (2^0; their codes are zero), packed little-endian.
__device__ __forceinline__ uint2 scales8_masked(const uint8_t* __restrict__ S, int64_t row,
                                                int64_t ks, int kt) {
    const int64_t b0 = (int64_t)kt * kScaleBytes;
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t c = b0 + i < ks ? b0 + i : ks - 1;
        const uint32_t v = S[row * ks + c];
        b[i] = b0 + i < ks ? v : 127u;
    }
    return make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                      b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
}

template <int BM, int BN, int GM, bool KTAIL>
__global__ __launch_bounds__(kThreads) void gemm_mx_tn(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, int64_t M, int64_t N, int64_t K, float* __restrict__ C,
    int tiles_m, int tiles_n) {
    constexpr int FM = BM / 64, FN = BN / 64;          // 32x32 tiles per wave
    constexpr int LA = BM / 32, LB = BN / 32;          // code DMA instructions per wave per stage
    constexpr int SLA = BM / 128, SLB = BN / 128;      // scale DMA instructions per wave per stage
    constexpr int kCodesA = 0, kCodesB = BM * kRowBytes;
    constexpr int kScA = (BM + BN) * kRowBytes, kScB = kScA + BM * kScaleBytes;
    constexpr int kStage = kScB + BN * kScaleBytes;
    static_assert(BM % 128 == 0 && BN % 128 == 0, "tile sizes");
    // Two stage buffers as distinct arrays: the compiler can then tell that
    // fragment reads of one do not depend on DMA still landing in the other.
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStage];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, l32 = lane & 31;
    int tile_m, tile_n;
    tile_of_block<GM>(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tile_m, tile_n);
    tile_m = __builtin_amdgcn_readfirstlane(tile_m);
    tile_n = __builtin_amdgcn_readfirstlane(tile_n);
    const int64_t m0 = (int64_t)tile_m * BM, n0 = (int64_t)tile_n * BN;
    const int64_t kbytes = K / 2, ks = K / 32;
    const int nk = (int)((K + kBK - 1) / kBK);

    // Buffer views of this block's rows: rows past M / N are out of range.
    const int64_t rows_a = (M - m0) < BM ? (M - m0) : BM;
    const int64_t rows_b = (N - n0) < BN ? (N - n0) : BN;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(A + m0 * kbytes), (short)0, (int)(rows_a * kbytes), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(B + n0 * kbytes), (short)0, (int)(rows_b * kbytes), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(SA + m0 * ks), (short)0, (int)(rows_a * ks), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(SB + n0 * ks), (short)0, (int)(rows_b * ks), kBufferWord3);

    // Per-lane DMA offsets within the stage at k = 0; the stage's k offset
    // goes in the scalar offset.  Codes: row lane/8 of an 8-row group, chunk
    // (lane mod 8) XOR (lane / 8).  Scales: row lane/2 of a 32-row group,
    // bytes 4 (lane mod 2) .. +3.
    const int drow = lane >> 3, dchunk = (lane & 7) ^ drow;
    uint32_t offa[LA], offb[LB], offsa[SLA], offsb[SLB];
#pragma unroll
    for (int i = 0; i < LA; ++i) offa[i] = (uint32_t)(((wave * LA + i) * 8 + drow) * kbytes + dchunk * 16);
#pragma unroll
    for (int i = 0; i < LB; ++i) offb[i] = (uint32_t)(((wave * LB + i) * 8 + drow) * kbytes + dchunk * 16);
#pragma unroll
    for (int i = 0; i < SLA; ++i) offsa[i] = (uint32_t)(((wave * SLA + i) * 32 + (lane >> 1)) * ks + (lane & 1) * 4);
#pragma unroll
    for (int i = 0; i < SLB; ++i) offsb[i] = (uint32_t)(((wave * SLB + i) * 32 + (lane >> 1)) * ks + (lane & 1) * 4);

    // A stage kt outside [0, nk) is an all-zero stage (every offset out of
    // range, zero codes and scale bytes).  Stage -1 lets an odd stage count
    // run in the loop below, which takes stages two at a time; stage nk is the
    // (unused) prefetch of the last stage, which keeps every stage one
    // straight-line block.
    auto load_stage = [&](int kt, uint8_t* base) {
        const bool zero = kt < 0 || kt >= nk;
        const int kcode = zero ? 0 : kt * kRowBytes;
        // a chunk past the contraction end gets an offset out of range
        uint32_t oob = zero ? 0x80000000u : 0u;
        if (KTAIL && !zero) oob = (uint32_t)(kcode + dchunk * 16 >= kbytes) << 31;
#pragma unroll
        for (int i = 0; i < LA; ++i)
            dma16_to_lds(ra, base + kCodesA + (wave * LA + i) * 8 * kRowBytes, offa[i] | oob, kcode);
#pragma unroll
        for (int i = 0; i < LB; ++i)
            dma16_to_lds(rb, base + kCodesB + (wave * LB + i) * 8 * kRowBytes, offb[i] | oob, kcode);
        if constexpr (!KTAIL) {
            const int kscale = zero ? 0 : kt * kScaleBytes;
#pragma unroll
            for (int i = 0; i < SLA; ++i)
                dma4_to_lds(rsa, base + kScA + (wave * SLA + i) * 32 * kScaleBytes, offsa[i] | oob, kscale);
#pragma unroll
            for (int i = 0; i < SLB; ++i)
                dma4_to_lds(rsb, base + kScB + (wave * SLB + i) * 32 * kScaleBytes, offsb[i] | oob, kscale);
        } else {
            for (int r = tid; r < BM; r += kThreads) {
                const int64_t g = m0 + r < M ? m0 + r : M - 1;
                *reinterpret_cast<uint2*>(base + kScA + r * kScaleBytes) =
                    zero ? make_uint2(0u, 0u) : scales8_masked(SA, g, ks, kt);
            }
            for (int r = tid; r < BN; r += kThreads) {
                const int64_t g = n0 + r < N ? n0 + r : N - 1;
                *reinterpret_cast<uint2*>(base + kScB + r * kScaleBytes) =
                    zero ? make_uint2(0u, 0u) : scales8_masked(SB, g, ks, kt);
            }
        }
    };

    v16f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // One stage from buffer `base` while stage kt+1 streams into `nbase`:
    // every wave waits for its own DMA into `base`, then the barrier makes
    // all of it visible (and frees `nbase`, read one stage earlier).  The
    // next stage's DMA is issued right after the first fragment reads; the
    // fragment reads of k-step s+1 are issued ahead of the MFMAs of k-step s.
    auto run_stage = [&](const uint8_t* base, int kt, uint8_t* nbase) {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        const uint8_t* la = base + kCodesA + wm * (BM / 2) * kRowBytes;
        const uint8_t* lb = base + kCodesB + wn * (BN / 2) * kRowBytes;
        // fragments of k-step s live in register set s mod 2
        uint4 fa[2][FM], fb[2][FN];
        uint2 sa[FM], sb[FN];
        auto read_frags = [&](int s) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[s & 1][i] = *reinterpret_cast<const uint4*>(la + swz(i * 32 + l32, 2 * s + h));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                fb[s & 1][j] = *reinterpret_cast<const uint4*>(lb + swz(j * 32 + l32, 2 * s + h));
        };
        auto mfmas = [&](int s) {
            const int shift = 8 * (2 * (s & 1) + h);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const uint4 a = fa[s & 1][i];
                const v8i af = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
                const int sca = (int)(((s < 2 ? sa[i].x : sa[i].y) >> shift) & 0xFFu);
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const uint4 b = fb[s & 1][j];
                    const v8i bf = v8i{(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
                    const int scb = (int)(((s < 2 ? sb[j].x : sb[j].y) >> shift) & 0xFFu);
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        bf, af, acc[i][j], 4, 4, 0, scb, 0, sca);
                }
            }
        };
#pragma unroll
        for (int i = 0; i < FM; ++i)
            sa[i] = *reinterpret_cast<const uint2*>(base + kScA + (wm * (BM / 2) + i * 32 + l32) * kScaleBytes);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            sb[j] = *reinterpret_cast<const uint2*>(base + kScB + (wn * (BN / 2) + j * 32 + l32) * kScaleBytes);
        read_frags(0);
        __builtin_amdgcn_sched_barrier(0);
        load_stage(kt + 1, nbase);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3) read_frags(s + 1);
            mfmas(s);
        }
        // Issue order: each MFMA is followed by at most one DMA instruction
        // of the next stage and, every other MFMA, one fragment read of the
        // next k-step, so neither the DMA burst nor the LDS reads hold up
        // the matrix pipe.
        int dma_left = LA + LB + (KTAIL ? 0 : SLA + SLB);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int t = 0; t < FM * FN; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
                if (s < 3 && (t & 1) == 0 && t / 2 < FM + FN)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
                if (dma_left > 0) {
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
                    --dma_left;
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    const int kfirst = -(nk & 1);
    load_stage(kfirst, lds0);
    for (int kt = kfirst; kt < nk; kt += 2) {
        run_stage(lds0, kt, lds1);
        run_stage(lds1, kt + 1, lds0);
    }

    // acc[i][j] holds C^T of a 32x32 tile: register r of lane l is
    // n = 8 (r / 4) + 4 (l / 32) + r mod 4, m = l mod 32.
    const bool vec_store = (N % 4) == 0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int64_t m = m0 + wm * (BM / 2) + i * 32 + l32;
        if (m >= M) continue;
        float* crow = C + m * N;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = n0 + wn * (BN / 2) + j * 32 + 8 * q + 4 * h;
                const float4 v = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                             acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                if (vec_store && n + 4 <= N) {
                    *reinterpret_cast<float4*>(crow + n) = v;
                } else {
                    if (n < N) crow[n] = v.x;
                    if (n + 1 < N) crow[n + 1] = v.y;
                    if (n + 2 < N) crow[n + 2] = v.z;
                    if (n + 3 < N) crow[n + 3] = v.w;
                }
            }
        }
    }
}

template <int BM, int BN, int GM, bool KTAIL>
hipError_t launch_tiles(const uint8_t* aq, const uint8_t* as, const uint8_t* bq,
                        const uint8_t* bs, int64_t M, int64_t N, int64_t K, float* c,
                        hipStream_t st) {
    const int64_t tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    hipLaunchKernelGGL((gemm_mx_tn<BM, BN, GM, KTAIL>), dim3((unsigned)(tm * tn)), dim3(kThreads),
                       0, st, aq, as, bq, bs, M, N, K, c, (int)tm, (int)tn);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mx(const uint8_t* aq, const uint8_t* as, const uint8_t* bq,
                          const uint8_t* bs, int64_t M, int64_t N, int64_t K, float* c,
                          hipStream_t st) {
    if (K % kBK == 0) return launch_tiles<256, 256, 8, false>(aq, as, bq, bs, M, N, K, c, st);
    return launch_tiles<256, 256, 8, true>(aq, as, bq, bs, M, N, K, c, st);
}

}  // namespace fp4dev

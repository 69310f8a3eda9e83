// gemm_mx.hip -- scaled MXFP4 GEMM on gfx950 matrix cores.
//
// [AMD-MXFP4] "Pretraining large language models with MXFP4 on Native FP4
// Hardware", section "Поисковая экспериментальная работа: корень
// нестабильности": the three GEMMs of a linear layer (Fprop, Dgrad, Wgrad)
// run in MXFP4 on native FP4 matrix cores.  All three are one "TN" product
//     C[m, n] = sum_k a[m, k] b[n, k]
// of two operands stored along their contraction axis as E2M1 codes (two per
// byte, even k in the low nibble) with one E8M0 scale per 32 k.  The scales
// of an operand with R rows are k-grouped: the 8 bytes of blocks 8g .. 8g+7
// of row r sit at (g R + r) * 8, so the scales of one 256-k stage of
// consecutive rows are one contiguous run.
//
// Kernel layout (WM x WN waves of 64 lanes -- 4 in the shapes launched,
// 2 x 2 for 256 x 256, 1 x 4 for 224 x 256, 4 x 1 for 256 x 224; the
// template also builds 8 -- block tile BM x BN, wave tile BM/WM x BN/WN made
// of 32 x 32 MFMA tiles):
//   - V_MFMA_SCALE_F32_32X32X64_F8F6F4 with both operands FP4 (format 4) and
//     fp32 accumulation.  Operand lane l supplies row (l mod 32) and k-half
//     (l div 32) of a 32 x 64 slice: 32 consecutive k = one 16-byte code
//     chunk = exactly one scale block, so the lane's scale byte is that
//     block's E8M0 scale.  The B tile is passed as the instruction's first
//     operand, so the accumulator holds C^T: lane l owns row m = l mod 32 of
//     C and four runs of four consecutive n, each stored as one 16-byte write.
//   - A stage is BK = 256 k: 128 code bytes and one 8-byte scale group per
//     row.  Both go global -> LDS by buffer_load ... lds (no VGPR round trip) into a
//     ring of NBUF stage buffers, NBUF - 1 stages ahead of the MFMAs.  One
//     dwordx4 instruction fills 64 16-byte slots of consecutive rows, lane i
//     writing slot i; the lane fetches the chunk that belongs in that slot.
//     Chunk c of row r sits in slot c XOR ((r / (16 / CPR)) mod CPR), CPR the
//     chunks per row: the 16 lanes the LDS serves per clock (rows r..r+15 of
//     one chunk) then hit all 64 banks once.  A dword instruction copies the
//     contiguous scale groups of 32 rows.  Rows past M (or N) lie outside
//     the buffer range and read as zero.
//   - Per stage a wave issues the DMA of stage kt + NBUF - 1 and the fragment
//     reads of its k-steps 1.. between the MFMAs of its k-steps 0.., then
//     waits for its own DMA of stage kt + 1; one barrier makes that stage
//     visible to all waves and frees buffer kt; the scales and k-step 0
//     fragments of stage kt + 1 are read while the last k-step's MFMAs run.
//   - A contraction that is not a multiple of BK (KTAIL) zero-fills the
//     missing code chunks through out-of-range offsets and loads the scales
//     through registers with the blocks past the end set to 127.
//   - Block order: workgroups are dispatched round-robin over the 8 XCDs;
//     the block index is remapped so that each XCD works on a contiguous run
//     of tiles, ordered in groups of GM tile-rows, so tiles that share A and
//     B rows meet in the same L2.
//   - Persistent workgroups (one per CU) loop over their tiles.  The output
//     leaves through LDS in whole rows per store instruction; when a tile and
//     the workgroup's next tile are both full, the next tile's first stage is
//     issued before the epilogue (into stage buffer 0, the epilogue staging
//     in buffer 1), so its latency hides behind the stores.
#include "fp4_device.hpp"
#include "fp4_launch.hpp"

namespace fp4dev {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kXcds = 8;
constexpr int kBufferWord3 = 0x00020000;   // raw buffer, 32-bit data format

// s_waitcnt immediate: vmcnt(n) with lgkmcnt(0).
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0070; }

// Workgroup barrier without the workgroup-scope release fence of
// __syncthreads(), which would wait for every outstanding LDS DMA: the caller
// has already waited (s_waitcnt) for exactly the DMA the barrier publishes.
// The wavefront-scope fences emit no code; they keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void barrier_after_wait() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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

// Scaled FP4 MFMA (32x32x64, both operands E2M1, fp32 accumulate) taking the
// E8M0 scales from byte 0 or byte 2 of the scale registers.
__device__ __forceinline__ v16f mfma_fp4_byte0(v8i b, v8i a, v16f c, uint32_t sb, uint32_t sa) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 4, 4, 0, (int)sb, 0, (int)sa);
}
__device__ __forceinline__ v16f mfma_fp4_byte2(v8i b, v8i a, v16f c, uint32_t sb, uint32_t sa) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 4, 4, 2, (int)sb, 2, (int)sa);
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

// Scale word w (bytes 4w .. 4w+3 of group kt) of one row of an operand with
// R rows and ks blocks per row, k-grouped; blocks at or past ks (the unused
// tail of the last group) read as 127 (2^0; their codes are zero).
__device__ __forceinline__ uint32_t scale_word_masked(const uint8_t* __restrict__ S, int64_t R,
                                                      int64_t row, int64_t ks, int kt, int w) {
    const int64_t b0 = (int64_t)kt * 8 + 4 * w;
    const uint8_t* p = S + ((int64_t)kt * R + row) * 8 + 4 * w;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) word |= (b0 + i < ks ? (uint32_t)p[i] : 127u) << (8 * i);
    return word;
}

// Round-to-nearest-even binary32 -> bfloat16 (NaN -> the quiet NaN 0x7FC0).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_value(uint32_t b) { return __uint_as_float(b << 16); }

// A 16-byte store of C marked non-temporal: with whole 128-byte lines per
// instruction the output streams to HBM during the GEMM instead of sitting
// dirty in the caches until the next kernel's traffic evicts it (measured:
// the quantizer that follows ran 14 us longer on dY[8192x14336]).  Partial
// lines must not take this path: non-temporal 16-byte pieces of a line are
// written to memory one by one.
typedef float v4f __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_c_line_part(float* p, float4 v) {
    __builtin_nontemporal_store(v4f{v.x, v.y, v.z, v.w}, reinterpret_cast<v4f*>(p));
}

// OBF16: C is bfloat16 (else fp32); ACC: C = A B^T + C (else C = A B^T), the
// sum formed in fp32 before the output rounding.
template <int BM, int BN, int WM, int WN, int BK, int NBUF, int GM, bool KTAIL, bool OBF16, bool ACC>
__global__ __launch_bounds__(64 * WM * WN) void gemm_mx_tn(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, int64_t M, int64_t N, int64_t K, void* __restrict__ C,
    int tiles_m, int tiles_n) {
    constexpr int RB = BK / 2;                     // code bytes per row per stage
    constexpr int CPR = RB / 16;                   // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;                  // rows per code DMA instruction
    constexpr int SWZ = 16 / CPR;                  // rows sharing a swizzle value
    constexpr int SBY = BK / 32;                   // scale bytes per row per stage (one group)
    constexpr int SW = SBY / 4;                    // scale words per row per stage
    constexpr int SRPI = 64 / SW;                  // rows per scale DMA instruction
    constexpr int KS = BK / 64;                    // MFMA k-steps per stage
    constexpr int TM = BM / WM, TN = BN / WN;     // wave tile
    constexpr int FM = TM / 32, FN = TN / 32;      // 32x32 MFMA tiles per wave
    // scale rows are fetched for BM / BN rounded up to whole instructions
    // over the four waves (the extra rows are never read)
    constexpr int NW = WM * WN, NT = 64 * NW;      // waves, threads
    constexpr int BMP = (BM + NW * SRPI - 1) / (NW * SRPI) * (NW * SRPI);
    constexpr int BNP = (BN + NW * SRPI - 1) / (NW * SRPI) * (NW * SRPI);
    constexpr int LA = BM / RPI / NW, LB = BN / RPI / NW;        // code DMAs per wave per stage
    constexpr int SLA = BMP / SRPI / NW, SLB = BNP / SRPI / NW;  // scale DMAs per wave per stage
    constexpr int DMA_PER_STAGE = LA + LB + (KTAIL ? 0 : SLA + SLB);
    constexpr int kCodesA = 0, kCodesB = BM * RB;
    constexpr int kScA = (BM + BN) * RB, kScB = kScA + BMP * SBY;
    constexpr int kStage = kScB + BNP * SBY;
    constexpr int D = NBUF - 1;                    // stages of DMA in flight
    static_assert(BK == 256, "a stage is one 8-block scale group");
    static_assert(NBUF == 2 || NBUF == 4, "stage ring");
    static_assert((NW == 4 || NW == 8) && TM % 32 == 0 && TN % 32 == 0, "wave layout");
    static_assert(BM % (NW * RPI) == 0 && BN % (NW * RPI) == 0, "code DMA split over the waves");
    static_assert(NBUF * kStage <= 160 * 1024, "LDS");
    // Stage buffers as distinct arrays: the compiler can then tell that
    // fragment reads of one do not wait on DMA still landing in another.
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[NBUF > 2 ? kStage : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds3[NBUF > 2 ? kStage : 16];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wm = wave / WN, wn = wave % WN, h = lane >> 5, l32 = lane & 31;
    // Persistent workgroups: tile t, t + gridDim.x, ... (the grid is at most
    // one workgroup per CU, so consecutive tile indices still land on the
    // XCDs round-robin).
    const int ntiles = tiles_m * tiles_n;
    const int64_t kbytes = K / 2, ks = K / 32;
    const int nk = (int)((K + BK - 1) / BK);
    // The current tile: origin and buffer views of its rows (rows past M / N
    // are out of range).  Set before the tile's first DMA, which for all but
    // a workgroup's first tile may be issued during the previous tile's
    // epilogue.
    int64_t m0 = 0, n0 = 0, rows_a = 0, rows_b = 0;
    __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, 0, kBufferWord3);
    __amdgpu_buffer_rsrc_t rb = ra;
    auto set_tile = [&](int t) {
        int tile_m, tile_n;
        tile_of_block<GM>(t, ntiles, tiles_m, tiles_n, tile_m, tile_n);
        tile_m = __builtin_amdgcn_readfirstlane(tile_m);
        tile_n = __builtin_amdgcn_readfirstlane(tile_n);
        m0 = (int64_t)tile_m * BM;
        n0 = (int64_t)tile_n * BN;
        rows_a = (M - m0) < BM ? (M - m0) : BM;
        rows_b = (N - n0) < BN ? (N - n0) : BN;
        ra = __builtin_amdgcn_make_buffer_rsrc((void*)(A + m0 * kbytes), (short)0, (int)(rows_a * kbytes),
                                               kBufferWord3);
        rb = __builtin_amdgcn_make_buffer_rsrc((void*)(B + n0 * kbytes), (short)0, (int)(rows_b * kbytes),
                                               kBufferWord3);
    };
    // Epilogue staging: with kEarly each wave stages its rows in a quarter of
    // stage buffer 1 only, so the next tile's first stage can land in stage
    // buffer 0 meanwhile; otherwise in 32 KB spread over both buffers.
    constexpr int kRowBytes = TN * 4 + 16;
    constexpr int kLanesPerRow = TN / 4;
    constexpr int kRowsPerInst = kLanesPerRow >= 64 ? 1 : 64 / kLanesPerRow;
    constexpr bool kEarly = !KTAIL && !ACC && NBUF == 2 && 32 * kRowBytes <= kStage / 4 &&
                            kRowsPerInst * kLanesPerRow == 64;
    constexpr int kRegion = kEarly ? kStage / 4 / 16 * 16 : 32768;
    // store instructions of a full tile's epilogue (they follow the next
    // tile's first DMA in the wave's memory counter)
    constexpr int kEpiStores = FM * 32 / kRowsPerInst;
    bool early = false;   // this tile's first stage was issued during the previous epilogue
    for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
        if (!early) {
            // every wave is done with the previous tile's LDS before it is refilled
            if (t != (int)blockIdx.x) {
                __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
                barrier_after_wait();
            }
            set_tile(t);
        }

        // Per-lane DMA offsets within the stage at k = 0; the stage's k offset
        // goes in the scalar offset.  Codes: row lane / CPR of an RPI-row group,
        // the chunk that belongs in slot lane mod CPR of that row.  Scales: the
        // contiguous groups of an SRPI-row run, one word per lane.
        const int drow = lane / CPR, dslot = lane % CPR;
        uint32_t offa[LA], offb[LB], offsa[SLA], offsb[SLB];
        int chka[LA], chkb[LB];   // byte offset of the fetched chunk within the row
    #pragma unroll
        for (int i = 0; i < LA; ++i) {
            const int row = (wave * LA + i) * RPI + drow;
            chka[i] = (dslot ^ ((row / SWZ) % CPR)) * 16;
            offa[i] = (uint32_t)(row * kbytes + chka[i]);
        }
    #pragma unroll
        for (int i = 0; i < LB; ++i) {
            const int row = (wave * LB + i) * RPI + drow;
            chkb[i] = (dslot ^ ((row / SWZ) % CPR)) * 16;
            offb[i] = (uint32_t)(row * kbytes + chkb[i]);
        }
    #pragma unroll
        for (int i = 0; i < SLA; ++i)
            offsa[i] = (uint32_t)(((wave * SLA + i) * SRPI * SBY) + lane * 4);
    #pragma unroll
        for (int i = 0; i < SLB; ++i)
            offsb[i] = (uint32_t)(((wave * SLB + i) * SRPI * SBY) + lane * 4);

        // A stage kt outside [0, nk) is an all-zero stage (every offset out of
        // range, zero codes and scale bytes).  Leading zero stages round the
        // stage count up to a multiple of NBUF for the loop below; trailing ones
        // are the (unused) prefetches past the last stage, which keep every
        // stage one straight-line block.
        auto load_stage = [&](int kt, uint8_t* base) {
            const bool zero = kt < 0 || kt >= nk;
            const int kcode = __builtin_amdgcn_readfirstlane(zero ? 0 : kt * RB);
            // a chunk past the contraction end gets an offset out of range
            const uint32_t oob = zero ? 0x80000000u : 0u;
    #pragma unroll
            for (int i = 0; i < LA; ++i) {
                const uint32_t tail = KTAIL ? (uint32_t)(kcode + chka[i] >= kbytes) << 31 : 0u;
                dma16_to_lds(ra, base + kCodesA + (wave * LA + i) * RPI * RB, offa[i] | oob | tail, kcode);
            }
    #pragma unroll
            for (int i = 0; i < LB; ++i) {
                const uint32_t tail = KTAIL ? (uint32_t)(kcode + chkb[i] >= kbytes) << 31 : 0u;
                dma16_to_lds(rb, base + kCodesB + (wave * LB + i) * RPI * RB, offb[i] | oob | tail, kcode);
            }
            if constexpr (!KTAIL) {
                // group kt of this tile's rows: one contiguous run per operand
                const int64_t g = zero ? 0 : kt;
                const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
                    (void*)(SA + (g * M + m0) * SBY), (short)0, (int)(rows_a * SBY), kBufferWord3);
                const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
                    (void*)(SB + (g * N + n0) * SBY), (short)0, (int)(rows_b * SBY), kBufferWord3);
    #pragma unroll
                for (int i = 0; i < SLA; ++i)
                    dma4_to_lds(rsa, base + kScA + (wave * SLA + i) * SRPI * SBY, offsa[i] | oob, 0);
    #pragma unroll
                for (int i = 0; i < SLB; ++i)
                    dma4_to_lds(rsb, base + kScB + (wave * SLB + i) * SRPI * SBY, offsb[i] | oob, 0);
            } else {
                for (int r = tid; r < BM; r += NT) {
                    const int64_t g = m0 + r < M ? m0 + r : M - 1;
    #pragma unroll
                    for (int w = 0; w < SW; ++w)
                        reinterpret_cast<uint32_t*>(base + kScA + r * SBY)[w] =
                            zero ? 0u : scale_word_masked(SA, M, g, ks, kt, w);
                }
                for (int r = tid; r < BN; r += NT) {
                    const int64_t g = n0 + r < N ? n0 + r : N - 1;
    #pragma unroll
                    for (int w = 0; w < SW; ++w)
                        reinterpret_cast<uint32_t*>(base + kScB + r * SBY)[w] =
                            zero ? 0u : scale_word_masked(SB, N, g, ks, kt, w);
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

        // Register state: the fragments of two k-steps (k-step s in set s mod 2)
        // and the scale words of two stages (word w of a fragment row holds the
        // blocks of k-steps 2w and 2w+1).  Shifted right by 8 h, word s / 2 holds
        // this lane's block of k-step s in byte 0 (even s) or byte 2 (odd s),
        // which the MFMA selects by op_sel.
        struct Scales { uint32_t a[FM][SW], b[FN][SW]; };
        // native vectors (not HIP's uint4 struct): one 16-byte LDS load each
        v4i fa[2][FM], fb[2][FN];
        auto read_frags = [&](const uint8_t* base, int s) {
            const uint8_t* la = base + kCodesA + wm * TM * RB;
            const uint8_t* lb = base + kCodesB + wn * TN * RB;
    #pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = i * 32 + l32;
                fa[s & 1][i] = *reinterpret_cast<const v4i*>(
                    la + row * RB + (((2 * s + h) ^ ((row / SWZ) % CPR)) << 4));
            }
    #pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = j * 32 + l32;
                fb[s & 1][j] = *reinterpret_cast<const v4i*>(
                    lb + row * RB + (((2 * s + h) ^ ((row / SWZ) % CPR)) << 4));
            }
        };
        auto read_scales = [&](const uint8_t* base, Scales& sc) {
    #pragma unroll
            for (int i = 0; i < FM; ++i) {
                const uint8_t* p = base + kScA + (wm * TM + i * 32 + l32) * SBY;
    #pragma unroll
                for (int w = 0; w < SW; ++w) sc.a[i][w] = reinterpret_cast<const uint32_t*>(p)[w];
            }
    #pragma unroll
            for (int j = 0; j < FN; ++j) {
                const uint8_t* p = base + kScB + (wn * TN + j * 32 + l32) * SBY;
    #pragma unroll
                for (int w = 0; w < SW; ++w) sc.b[j][w] = reinterpret_cast<const uint32_t*>(p)[w];
            }
        };
        auto mfmas = [&](int s, const Scales& sc) {
    #pragma unroll
            for (int i = 0; i < FM; ++i) {
                const v8i af = __builtin_shufflevector(fa[s & 1][i], v4i{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
                const uint32_t wa = sc.a[i][s >> 1] >> (8 * h);
    #pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const v8i bf = __builtin_shufflevector(fb[s & 1][j], v4i{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
                    const uint32_t wb = sc.b[j][s >> 1] >> (8 * h);
                    acc[i][j] = (s & 1) ? mfma_fp4_byte2(bf, af, acc[i][j], wb, wa)
                                        : mfma_fp4_byte0(bf, af, acc[i][j], wb, wa);
                }
            }
        };

        // One stage from buffer `cur` (its k-step 0 fragments and scales already
        // in registers as `sc`); `ahead` receives stage kt + D, `next` holds
        // stage kt + 1.
        auto run_stage = [&](const uint8_t* cur, int kt, uint8_t* ahead, const uint8_t* next,
                             const Scales& sc, Scales& nsc) {
            load_stage(kt + D, ahead);
    #pragma unroll
            for (int s = 0; s < KS - 1; ++s) {
                read_frags(cur, s + 1);
                mfmas(s, sc);
            }
            constexpr int kMfma1 = (KS - 1) * FM * FN, kDs1 = (KS - 1) * (FM + FN);
            int dma_left = DMA_PER_STAGE;
    #pragma unroll
            for (int t = 0; t < kMfma1; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
                if (dma_left > 0) {
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read (DMA)
                    --dma_left;
                }
                // fragment reads spread evenly over the MFMAs
                if ((t + 1) * kDs1 / kMfma1 > t * kDs1 / kMfma1)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
            }
            __builtin_amdgcn_sched_barrier(0);
            // this wave's DMA of stage kt + 1 has landed (only the D - 1 younger
            // stages may still be in flight) and its reads of `cur` are done
            if constexpr (KTAIL) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
            else __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((D - 1) * DMA_PER_STAGE));
            barrier_after_wait();
            read_scales(next, nsc);
            read_frags(next, 0);
            mfmas(KS - 1, sc);
            constexpr int kMfma2 = FM * FN, kDs2 = (FM + FN) * (1 + SW);
    #pragma unroll
            for (int t = 0; t < kMfma2; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
                if ((t + 1) * kDs2 / kMfma2 > t * kDs2 / kMfma2)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
                if ((t + 1) * kDs2 / kMfma2 > t * kDs2 / kMfma2 + 1)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
            }
            __builtin_amdgcn_sched_barrier(0);
        };

        uint8_t* const bufs[4] = {lds0, lds1, lds2, lds3};
        const int kfirst = -((NBUF - nk % NBUF) % NBUF);
        if (!early) {
    #pragma unroll
            for (int d = 0; d < D; ++d) load_stage(kfirst + d, bufs[d]);
            if constexpr (KTAIL) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
            else __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((D - 1) * DMA_PER_STAGE));
        } else {
            // the first stage went out before the previous tile's kEpiStores
            // stores (the memory counter completes in order)
            __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(kEpiStores < 63 ? kEpiStores : 63));
        }
        barrier_after_wait();
        Scales sc0, sc1;
        read_scales(bufs[0], sc0);
        read_frags(bufs[0], 0);
        for (int kt = kfirst; kt < nk; kt += NBUF) {
    #pragma unroll
            for (int b = 0; b < NBUF; ++b) {
                if (b & 1)
                    run_stage(bufs[b], kt + b, bufs[(b + D) % NBUF], bufs[(b + 1) % NBUF], sc1, sc0);
                else
                    run_stage(bufs[b], kt + b, bufs[(b + D) % NBUF], bufs[(b + 1) % NBUF], sc0, sc1);
            }
        }

        // the prefetches past the last stage must land before the workgroup
        // (and its LDS) goes away
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
        __syncthreads();                                // all fragment reads of the tile are done
        const int64_t em0 = m0, en0 = n0;               // the tile the epilogue writes
        const bool vec_store = (N % 4) == 0;
        const bool full_tile = vec_store && em0 + BM <= M && en0 + BN <= N;   // workgroup-uniform
        early = false;
        if constexpr (kEarly) {
            // The next tile's first stage goes out now, into stage buffer 0
            // (this epilogue stages in buffer 1 only); it is waited for at
            // the start of the next tile.
            const int tn = t + (int)gridDim.x;
            if (full_tile && tn < ntiles) {
                set_tile(tn);
    #pragma unroll
                for (int d = 0; d < D; ++d) load_stage(kfirst + d, bufs[d]);
                early = true;
            }
        }

        // acc[i][j] holds C^T of a 32x32 tile: register r of lane l is
        // n = 8 (r / 4) + 4 (l / 32) + r mod 4, m = l mod 32.  The wave's rows
        // go out through LDS: the stage buffers are free once every wave is
        // past its last fragment read; each wave stages a few 32-row pieces of
        // its tile at a time in its own region (rows padded by 16 bytes:
        // conflict-free writes of the accumulator layout and row reads), then
        // reads back four consecutive n of a row per lane, TN / 4 lanes per
        // row, so that a store instruction covers whole rows of the tile.
        // fp32 rows are whole 128-byte lines, written non-temporally; with
        // N % 4 != 0 (rows not 16-byte aligned) elements go one by one.
        static_assert(NW == 4 && kStage >= 65536 && 32 * kRowBytes <= kRegion && kLanesPerRow <= 64,
                      "each wave stages at least 32 rows of its tile");
        constexpr int ICH = (kRegion / kRowBytes) / 32 < FM ? (kRegion / kRowBytes) / 32 : FM;
        uint8_t* const reg = kEarly ? lds1 + wave * kRegion : ((wave >> 1) ? lds1 : lds0) + (wave & 1) * 32768;
    #pragma unroll
        for (int i0 = 0; i0 < FM; i0 += ICH) {
    #pragma unroll
            for (int ii = 0; ii < ICH; ++ii) {
                if (i0 + ii >= FM) break;
    #pragma unroll
                for (int j = 0; j < FN; ++j)
    #pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int row = ii * 32 + l32, cn = j * 32 + 8 * q + 4 * h;
                        *reinterpret_cast<float4*>(reg + row * kRowBytes + cn * 4) =
                            make_float4(acc[i0 + ii][j][4 * q], acc[i0 + ii][j][4 * q + 1],
                                        acc[i0 + ii][j][4 * q + 2], acc[i0 + ii][j][4 * q + 3]);
                    }
            }
            const int nrows = (FM - i0 < ICH ? FM - i0 : ICH) * 32;
            const int lr = lane / kLanesPerRow, c4 = (lane % kLanesPerRow) * 4;
            const bool lane_on = lr < kRowsPerInst;
            if (full_tile) {
                // every row and column in range: batches of kBatch row
                // reads go out back to back, then their stores
                constexpr int kBatch = 8;
    #pragma unroll
                for (int rb = 0; rb < ICH * 32; rb += kBatch * kRowsPerInst) {
                    if (rb >= nrows) break;
                    float4 f[kBatch];
    #pragma unroll
                    for (int k = 0; k < kBatch; ++k)
                        f[k] = *reinterpret_cast<const float4*>(
                            reg + (lane_on ? rb + k * kRowsPerInst + lr : 0) * kRowBytes + c4 * 4);
                    if (lane_on) {
    #pragma unroll
                        for (int k = 0; k < kBatch; ++k) {
                            const int64_t m = em0 + wm * TM + i0 * 32 + rb + k * kRowsPerInst + lr;
                            const int64_t n = en0 + wn * TN + c4;
                            float v[4] = {f[k].x, f[k].y, f[k].z, f[k].w};
                            if constexpr (OBF16) {
                                uint2* p = reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(C) + m * N + n);
                                if constexpr (ACC) {
                                    const uint2 o = *p;
                                    v[0] += bf16_value(o.x & 0xFFFFu); v[1] += bf16_value(o.x >> 16);
                                    v[2] += bf16_value(o.y & 0xFFFFu); v[3] += bf16_value(o.y >> 16);
                                }
                                *p = make_uint2(bf16_rne(v[0]) | (bf16_rne(v[1]) << 16),
                                                bf16_rne(v[2]) | (bf16_rne(v[3]) << 16));
                            } else {
                                float* p = reinterpret_cast<float*>(C) + m * N + n;
                                if constexpr (ACC) {
                                    const float4 o = *reinterpret_cast<const float4*>(p);
                                    v[0] += o.x; v[1] += o.y; v[2] += o.z; v[3] += o.w;
                                }
                                store_c_line_part(p, make_float4(v[0], v[1], v[2], v[3]));
                            }
                        }
                    }
                }
                continue;
            }
    #pragma unroll
            for (int rr = 0; rr < ICH * 32; rr += kRowsPerInst) {
                if (rr >= nrows) break;
                const int row = rr + lr;
                const float4 f = *reinterpret_cast<const float4*>(reg + (lane_on ? row : 0) * kRowBytes + c4 * 4);
                const int64_t m = em0 + wm * TM + i0 * 32 + row, n = en0 + wn * TN + c4;
                if (!lane_on || m >= M) continue;
                float v[4] = {f.x, f.y, f.z, f.w};
                if constexpr (OBF16) {
                    uint16_t* crow = reinterpret_cast<uint16_t*>(C) + m * N;
                    if (vec_store && n + 4 <= N) {
                        uint2* p = reinterpret_cast<uint2*>(crow + n);
                        if constexpr (ACC) {
                            const uint2 o = *p;
                            v[0] += bf16_value(o.x & 0xFFFFu); v[1] += bf16_value(o.x >> 16);
                            v[2] += bf16_value(o.y & 0xFFFFu); v[3] += bf16_value(o.y >> 16);
                        }
                        *p = make_uint2(bf16_rne(v[0]) | (bf16_rne(v[1]) << 16),
                                        bf16_rne(v[2]) | (bf16_rne(v[3]) << 16));
                    } else {
                        for (int e = 0; e < 4; ++e) {
                            if (n + e >= N) break;
                            const float old = ACC ? bf16_value(crow[n + e]) : 0.0f;
                            crow[n + e] = (uint16_t)bf16_rne(ACC ? v[e] + old : v[e]);
                        }
                    }
                } else {
                    float* crow = reinterpret_cast<float*>(C) + m * N;
                    if (vec_store && n + 4 <= N) {
                        if constexpr (ACC) {
                            const float4 o = *reinterpret_cast<const float4*>(crow + n);
                            v[0] += o.x; v[1] += o.y; v[2] += o.z; v[3] += o.w;
                        }
                        store_c_line_part(crow + n, make_float4(v[0], v[1], v[2], v[3]));
                    } else {
                        for (int e = 0; e < 4; ++e) {
                            if (n + e >= N) break;
                            crow[n + e] = ACC ? v[e] + crow[n + e] : v[e];
                        }
                    }
                }
            }
        }
    }
}

// Compute units of the current device (queried once per device).
int cu_count() {
    static int counts[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (counts[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        counts[dev] = n;
    }
    return counts[dev];
}

template <int BM, int BN, int WM, int WN, int BK, int NBUF, int GM, bool OBF16, bool ACC>
void launch_kernel(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs,
                   int64_t M, int64_t N, int64_t K, void* c, hipStream_t st) {
    const int64_t tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    const int64_t grid = tm * tn < cu_count() ? tm * tn : cu_count();
    if (K % BK == 0) {
        hipLaunchKernelGGL((gemm_mx_tn<BM, BN, WM, WN, BK, NBUF, GM, false, OBF16, ACC>),
                           dim3((unsigned)grid), dim3(64 * WM * WN), 0, st, aq, as, bq, bs, M, N, K,
                           c, (int)tm, (int)tn);
    } else {
        hipLaunchKernelGGL((gemm_mx_tn<BM, BN, WM, WN, BK, NBUF, GM, true, OBF16, ACC>),
                           dim3((unsigned)grid), dim3(64 * WM * WN), 0, st, aq, as, bq, bs, M, N, K,
                           c, (int)tm, (int)tn);
    }
}

template <int BM, int BN, int WM, int WN, int BK, int NBUF, int GM>
hipError_t launch_tiles(const uint8_t* aq, const uint8_t* as, const uint8_t* bq,
                        const uint8_t* bs, int64_t M, int64_t N, int64_t K, void* c, int out_bf16,
                        int accumulate, hipStream_t st) {
    if (out_bf16) {
        if (accumulate) launch_kernel<BM, BN, WM, WN, BK, NBUF, GM, true, true>(aq, as, bq, bs, M, N, K, c, st);
        else launch_kernel<BM, BN, WM, WN, BK, NBUF, GM, true, false>(aq, as, bq, bs, M, N, K, c, st);
    } else {
        if (accumulate) launch_kernel<BM, BN, WM, WN, BK, NBUF, GM, false, true>(aq, as, bq, bs, M, N, K, c, st);
        else launch_kernel<BM, BN, WM, WN, BK, NBUF, GM, false, false>(aq, as, bq, bs, M, N, K, c, st);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mx(const uint8_t* aq, const uint8_t* as, const uint8_t* bq,
                          const uint8_t* bs, int64_t M, int64_t N, int64_t K, void* c,
                          int out_bf16, int accumulate, hipStream_t st) {
    // Tile shape: the persistent grid runs ceil(tiles / CUs) rounds of one
    // tile per CU, each costing about the tile's area, so pick the shape with
    // the least rounds x area (256 x 256 unless a 224-row or -column tile
    // removes a partly idle last round, e.g. M = 14336 = 64 x 224).
    const int64_t cus = cu_count();
    // Tile-rows per group of the block order.  Measured on the gate/up and
    // q_proj shapes (each XCD runs 32 tiles at a time): groups of 2 to 4
    // rows beat 8 by 2-5 % and 16 by more; 4 is the best on average.
    constexpr int kGroupRows = 4;
    auto cost = [&](int64_t bm, int64_t bn) {
        const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
        return ((tiles + cus - 1) / cus) * bm * bn;
    };
    const int64_t c256 = cost(256, 256), cm = cost(224, 256), cn = cost(256, 224);
    if (cm < c256 && cm <= cn)
        return launch_tiles<224, 256, 1, 4, 256, 2, kGroupRows>(aq, as, bq, bs, M, N, K, c, out_bf16, accumulate, st);
    if (cn < c256)
        return launch_tiles<256, 224, 4, 1, 256, 2, kGroupRows>(aq, as, bq, bs, M, N, K, c, out_bf16, accumulate, st);
    return launch_tiles<256, 256, 2, 2, 256, 2, kGroupRows>(aq, as, bq, bs, M, N, K, c, out_bf16, accumulate, st);
}

}  // namespace fp4dev

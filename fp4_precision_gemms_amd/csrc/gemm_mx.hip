// gemm_mx.hip -- scaled MXFP4 GEMM on gfx950 matrix cores.
//
// [AMD-MXFP4] "Pretraining large language models with MXFP4 on Native FP4
// Hardware", section "Поисковая экспериментальная работа: корень
// нестабильности": the three GEMMs of a linear layer (Fprop, Dgrad, Wgrad)
// run in MXFP4 on native FP4 matrix cores.  All three are one "TN" product
//     C[m, n] = sum_k a[m, k] b[n, k]
// of two operands stored along their contraction axis as E2M1 codes with one
// E8M0 scale per 32 k.
//
// Operand layouts (written so by the quantizers):
//   - codes, "32-row tiled": for each group of 32 rows and each 32-element
//     block, the 32 rows' 16 code bytes (two per byte, even k in the low
//     nibble) are one contiguous 512-byte chunk, row r of the group at
//     16 * (r mod 32); chunk (g, b) of an operand with nb blocks per row sits
//     at (g * nb + b) * 512.  Two consecutive chunks of a row group are then
//     exactly the 1 KB operand of one 32 x 32 x 64 MFMA k-step in lane order.
//   - scales, k-grouped: the 8 bytes of blocks 8q .. 8q+7 of row r at
//     (q R + r) * 8, so one 256-k stage of consecutive rows is one run.
//
// Kernel (one workgroup of 4 waves per CU, persistent over tiles):
//   - block tile BM x 256 (BM = 32 FM, FM = 7 or 8), wave w computes all BM
//     rows x columns 64 w .. 64 w + 63 with V_MFMA_SCALE_F32_32X32X64_F8F6F4
//     (FP4 x FP4, fp32 accumulation).  The B operand is the instruction's
//     first source, so an accumulator holds a 32 x 32 tile of C^T: lane l
//     owns row m = l mod 32 and four runs of four consecutive n.
//   - A (shared by the four waves) goes global -> LDS by buffer_load ... lds
//     into a ring of four 256-k stage slots; the DMA of stage kt + 3 is
//     spread over the k-steps of stage kt, and the wait for a stage is issued
//     two stages after its DMA.  Measured on this chip: issuing a stage's DMA
//     in one burst stalls the in-order MFMA issue behind the per-CU load
//     path, and a wait one stage after the issue exposes the load latency.
//   - B (private to each wave: its 64 rows) goes global -> registers: each
//     k-step's two 1 KB fragments are one contiguous load each (the tiled
//     layout), issued 8 k-steps ahead into a register ring; B scales come
//     from HBM one stage group per load, two stages ahead.
//   - Scales: when a stage starts, each lane turns its rows' 8 block scales
//     of the stage into one word by a byte permute (the 4 blocks its lane
//     half uses), and k-step s reads byte s of it through the MFMA's scale
//     byte select -- no per-MFMA arithmetic on the operand path.
//   - A contraction that is not a multiple of 256 (KTAIL) zero-fills chunks
//     past the end through out-of-range buffer offsets and sets the scale
//     bytes of blocks past the end to 127 (2^0).
//   - Block order: workgroups are dispatched round-robin over the 8 XCDs;
//     the tile index is remapped so that each XCD works on a contiguous run
//     of tiles, ordered in groups of GM tile-rows.
//   - Epilogue: each wave stages 32 rows of its 64 columns at a time in one
//     LDS slot and stores whole rows per instruction.  When the tile and the
//     workgroup's next tile are both full, the next tile's first stages are
//     issued before the epilogue (into the other three slots).
//   - Launches of several rounds start their workgroups staggered, so that
//     the tile boundaries of the 256 workgroups do not coincide.
#include "fp4_device.hpp"
#include "fp4_launch.hpp"

#include <atomic>

namespace fp4dev {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kXcds = 8;
constexpr int kBufferWord3 = 0x00020000;   // raw buffer, 32-bit data format
constexpr uint32_t kOob = 0x80000000u;     // a buffer offset past any range: reads zero

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
// E8M0 scales from byte S of the scale registers.
template <int S>
__device__ __forceinline__ v16f mfma_fp4(v8i b, v8i a, v16f c, uint32_t sb, uint32_t sa) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 4, 4, S, (int)sb, S, (int)sa);
}

// The scale word a lane feeds the MFMAs of one 256-k stage: the stage's 8
// block scales of its row are bytes 0..7 of (hi:lo); k-step s uses block
// 2 s + (lane / 32), so lane half h keeps bytes h, 2 + h, 4 + h, 6 + h, and
// k-step s reads byte s of the word -- one byte permute per stage instead of
// a shift before every MFMA.  Formed when the stage starts: at load time it
// would wait for loads issued stages ahead.
__device__ __forceinline__ uint32_t stage_scale_word(uint32_t lo, uint32_t hi, int h) {
    return __builtin_amdgcn_perm(hi, lo, h ? 0x07050301u : 0x06040200u);
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

// Bytes of a scale word for blocks first .. first+3 that lie at or past nb
// (the unused tail of the last k-group) set to 127 (2^0; their codes are
// zero).
__device__ __forceinline__ uint32_t mask_scale_word(uint32_t w, int64_t first, int64_t nb) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (first + i >= nb) w = (w & ~(0xFFu << (8 * i))) | (127u << (8 * i));
    return w;
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
// dirty in the caches until the next kernel's traffic evicts it.  Partial
// lines must not take this path: non-temporal 16-byte pieces of a line are
// written to memory one by one.
__device__ __forceinline__ void store_c_line_part(float* p, float4 v) {
    __builtin_nontemporal_store(v4f{v.x, v.y, v.z, v.w}, reinterpret_cast<v4f*>(p));
}

constexpr int kWaves = 4, kThreads = 64 * kWaves;
constexpr int kBN = 256;            // tile columns: 64 per wave
constexpr int kKS = 4;              // MFMA k-steps (64 k each) per 256-k stage
constexpr int kSlots = 4;           // A stage ring
constexpr int kRing = 8;            // B register ring depth, in k-steps
constexpr int kEpiRow = 64 * 4 + 16;            // a staged row of a wave's 64 fp32 columns, padded
constexpr int kEpiRegion = 32 * kEpiRow;        // 32 rows per wave

// OBF16: C is bfloat16 (else fp32); ACC: C = A B^T + C (else C = A B^T), the
// sum formed in fp32 before the output rounding.  FAST: every tile is full
// and the contraction is a multiple of 1024 (the stage count a multiple of
// the ring), so no lane ever reads out of range; the prefetches past the
// last stage re-load the last stage (never read) and each stage's offset is
// a scalar added to per-tile descriptors.
template <int FM, int GM, bool FAST, bool KTAIL, bool OBF16, bool ACC>
__global__ __launch_bounds__(kThreads) void gemm_mx_tn(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, int64_t M, int64_t N, int64_t K, void* __restrict__ C,
    int tiles_m, int tiles_n) {
    constexpr int BM = 32 * FM, FN = 2;
    constexpr int kACodes = FM * 4096;                 // FM row groups x 8 chunks of 512 B
    constexpr int kAScales = 2048;                     // 8 scale DMAs of 32 rows x 8 B
    constexpr int kSlot = (kACodes + kAScales) > kWaves * kEpiRegion ? (kACodes + kAScales)
                                                                     : kWaves * kEpiRegion;
    // VMEM instructions per wave per stage: A codes (FM) and scales (2) by
    // DMA, B codes (two per k-step) and B scales (two)
    // (the fast path moves A's scales with one 16-byte DMA per wave)
    constexpr int kVmStage = FM + (FAST ? 1 : 2) + 2 * kKS + 2;
    static_assert(FM >= 4 && FM <= 8, "tile rows");
    static_assert(!(FAST && KTAIL), "the fast path has no contraction tail");
    constexpr int kWaitStage = 2 * kVmStage - 2;
    static_assert(kWaitStage <= 63, "vmcnt range");
    static_assert(kSlots * kSlot <= 160 * 1024, "LDS");
    // Stage slots as distinct arrays: the compiler can then tell that
    // fragment reads of one do not wait on DMA still landing in another.
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[kSlot];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[kSlot];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[kSlot];
    __shared__ __attribute__((aligned(1024))) uint8_t lds3[kSlot];
    uint8_t* const slots[kSlots] = {lds0, lds1, lds2, lds3};

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int h = lane >> 5, l32 = lane & 31;
    const int ntiles = tiles_m * tiles_n;
    const int64_t nb = K / 32;                         // blocks per row
    const int nks = (int)((nb + 1) / 2);               // MFMA k-steps (K < 2^24)
    const int nk = (int)((nb + 7) / 8);                // 256-k stages
    // leading all-zero stages round the stage count up to a multiple of the
    // ring (the loop below handles four stages per iteration)
    const int kfirst = -((kSlots - nk % kSlots) % kSlots);
    const uint32_t gstride = (uint32_t)(nb * 512);     // bytes per 32-row group of codes

    // Per-lane parts of the buffer offsets (the stage / k-step part goes in
    // the scalar offset): A chunk d of this wave's k-step (wave) of a stage,
    // B fragment j (row group 2 wave + j) of a k-step.
    uint32_t offa[FM], offb[FN];
#pragma unroll
    for (int d = 0; d < FM; ++d) offa[d] = (uint32_t)d * gstride + (uint32_t)lane * 16;
#pragma unroll
    for (int j = 0; j < FN; ++j) offb[j] = (uint32_t)(2 * wave + j) * gstride + (uint32_t)lane * 16;
    // the upper half of a k-step past the last block (nb odd) reads zero
    const bool half_tail = KTAIL && (nb & 1) && h == 1;

    int64_t m0 = 0, n0 = 0, rows_a = 0, rows_b = 0;
    __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, 0, kBufferWord3);
    __amdgpu_buffer_rsrc_t rb = ra, rsa = ra, rsb = ra;   // rsa, rsb: FAST scale descriptors
    // FAST: lane parts of the scale offsets (A: 16 bytes of this wave's
    // 128-row run, B: this lane's row of fragment j)
    const uint32_t offsa0 = (uint32_t)(((wave & 1) ? (BM - 128) * 8 : 0) + lane * 16);
    uint32_t offsb[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) offsb[j] = (uint32_t)((64 * wave + 32 * j + l32) * 8);
    auto set_tile = [&](int t) {
        int tile_m, tile_n;
        tile_of_block<GM>(t, ntiles, tiles_m, tiles_n, tile_m, tile_n);
        tile_m = __builtin_amdgcn_readfirstlane(tile_m);
        tile_n = __builtin_amdgcn_readfirstlane(tile_n);
        m0 = (int64_t)tile_m * BM;
        n0 = (int64_t)tile_n * kBN;
        rows_a = (M - m0) < BM ? (M - m0) : BM;
        rows_b = (N - n0) < kBN ? (N - n0) : kBN;
        // the tile's row groups of each operand; groups past the operand's
        // last one are out of range and read as zero
        ra = __builtin_amdgcn_make_buffer_rsrc((void*)(A + (m0 / 32) * (int64_t)gstride), (short)0,
                                               (int)(((rows_a + 31) / 32) * (int64_t)gstride), kBufferWord3);
        rb = __builtin_amdgcn_make_buffer_rsrc((void*)(B + (n0 / 32) * (int64_t)gstride), (short)0,
                                               (int)(((rows_b + 31) / 32) * (int64_t)gstride), kBufferWord3);
        if constexpr (FAST) {
            // stage q of the tile's rows starts q R 8 bytes further on
            rsa = __builtin_amdgcn_make_buffer_rsrc((void*)(SA + m0 * 8), (short)0,
                                                    (int)(((int64_t)nk * M - m0) * 8), kBufferWord3);
            rsb = __builtin_amdgcn_make_buffer_rsrc((void*)(SB + n0 * 8), (short)0,
                                                    (int)(((int64_t)nk * N - n0) * 8), kBufferWord3);
        }
    };

    // ---- loads ---------------------------------------------------------
    // A DMA of stage kt into `slot`: chunk d (row group d, k-step `wave` of
    // the stage) for d in [d0, d1), and the scale runs (two per wave) when
    // `scales`.  A stage outside [0, nk) is all zero.
    auto dma_a = [&](int kt, uint8_t* slot, int d0, int d1, bool scales) {
        if constexpr (FAST) {
            const int kc = kt < nk ? kt : nk - 1;
            const int soff = __builtin_amdgcn_readfirstlane((4 * kc + wave) * 1024);
#pragma unroll
            for (int d = 0; d < FM; ++d)
                if (d >= d0 && d < d1) dma16_to_lds(ra, slot + d * 4096 + wave * 1024, offa[d], soff);
            // the scale run of the stage's BM rows (8 bytes each) by
            // 16-byte-per-lane DMAs of 128 rows: rows 0..127 (waves 0, 2) and
            // the last 128 rows of the tile (waves 1, 3; the repeated DMA
            // writes the same bytes and keeps every wave's instruction count,
            // hence its waits, identical).  4-byte DMAs cost several times
            // more per byte on the load path.
            if (scales) {
                const int ss = __builtin_amdgcn_readfirstlane((int)((int64_t)kc * M * 8));
                dma16_to_lds(rsa, slot + kACodes + ((wave & 1) ? (BM - 128) * 8 : 0), offsa0, ss);
            }
            return;
        }
        const bool zero = kt < 0 || kt >= nk;
        const int ks = 4 * kt + wave;                  // this wave's k-step
        bool dead = zero;
        if constexpr (KTAIL) dead = dead || ks >= nks;
        const int soff = __builtin_amdgcn_readfirstlane(dead ? 0 : ks * 1024);
        const uint32_t oob = dead ? kOob : 0u;
        const uint32_t hoob = (KTAIL && !dead && ks == nks - 1 && half_tail) ? kOob : 0u;
#pragma unroll
        for (int d = 0; d < FM; ++d)
            if (d >= d0 && d < d1)
                dma16_to_lds(ra, slot + d * 4096 + wave * 1024, offa[d] | oob | hoob, soff);
        if (scales) {
            const int64_t q = zero ? 0 : kt;
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(SA + (q * M + m0) * 8), (short)0, (int)(rows_a * 8), kBufferWord3);
            const uint32_t zoob = zero ? kOob : 0u;
            dma4_to_lds(rs, slot + kACodes + wave * 256, (uint32_t)(wave * 256 + lane * 4) | zoob, 0);
            dma4_to_lds(rs, slot + kACodes + (wave + 4) * 256,
                        (uint32_t)((wave + 4) * 256 + lane * 4) | zoob, 0);
        }
    };
    // B fragment j of k-step s (global index) into registers.
    auto load_b = [&](int s, int j) -> v4i {
        if constexpr (FAST) {
            const int soff = __builtin_amdgcn_readfirstlane((s < nks ? s : nks - 1) * 1024);
            return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rb, offb[j], soff, 0));
        }
        bool dead = s < 0 || s >= nks;
        const int soff = __builtin_amdgcn_readfirstlane(dead ? 0 : s * 1024);
        uint32_t off = offb[j] | (dead ? kOob : 0u);
        if constexpr (KTAIL) off |= (!dead && s == nks - 1 && half_tail) ? kOob : 0u;
        return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rb, off, soff, 0));
    };
    // B scales of stage kt: this lane's row of fragment j, 8 bytes (blocks
    // past the contraction's end already set to 2^0).
    struct BSc { uint32_t w[FN][2]; };
    auto load_bsc = [&](int kt) -> BSc {
        if constexpr (FAST) {
            const int kc = kt < nk ? kt : nk - 1;
            const int ss = __builtin_amdgcn_readfirstlane((int)((int64_t)kc * N * 8));
            BSc r;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b64(rsb, offsb[j], ss, 0);
                r.w[j][0] = v[0];
                r.w[j][1] = v[1];
            }
            return r;
        }
        const bool zero = kt < 0 || kt >= nk;
        const int64_t q = zero ? 0 : kt;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(SB + (q * N + n0) * 8), (short)0, (int)(rows_b * 8), kBufferWord3);
        BSc r;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const uint32_t off = (uint32_t)((64 * wave + 32 * j + l32) * 8) | (zero ? kOob : 0u);
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
            r.w[j][0] = v[0];
            r.w[j][1] = v[1];
        }
        return r;
    };

    // ---- registers -----------------------------------------------------
    v16f acc[FM][FN];
    v4i fa[2][FM];                 // A fragments of two k-steps (k-step parity)
    v4i fb[kRing][FN];             // B fragments, k-step s in fb[s mod 8]
    BSc bsc[kSlots];               // B scales, stage kt in bsc[(kt - kfirst) mod 4]
    struct ASc { uint32_t w[FM][2]; };
    ASc asc[2];                    // A scales of the current and next stage

    // Per-slot lane bases of the LDS reads (this lane's 16 bytes of a
    // fragment; its row's 8 scale bytes): the rest of each address then fits
    // the LDS read's 16-bit immediate also in the slots past 64 KB, instead
    // of costing an OR before every read.  The lane offsets pass through an
    // empty asm statement so that the bases are not folded back into them.
    uint32_t lo16 = (uint32_t)lane * 16, lo8 = (uint32_t)l32 * 8;
    asm volatile("" : "+v"(lo16), "+v"(lo8));
    const uint8_t* fbase[kSlots];
    const uint8_t* sbase[kSlots];
#pragma unroll
    for (int q = 0; q < kSlots; ++q) {
        fbase[q] = slots[q] + lo16;
        sbase[q] = slots[q] + kACodes + lo8;
    }
    auto read_afrags = [&](int q, int s, int set) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
            fa[set][i] = *reinterpret_cast<const v4i*>(fbase[q] + i * 4096 + s * 1024);
    };
    auto read_ascales = [&](int q, int kt, ASc& sc) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const uint2 v = *reinterpret_cast<const uint2*>(sbase[q] + i * 32 * 8);
            sc.w[i][0] = v.x;
            sc.w[i][1] = v.y;
        }
    };
    // MFMAs of k-step s (0..3) of a stage: A fragments set, B ring slot r.
    // The stage's scale words (stage_scale_word) from its raw A and B scales;
    // blocks past the contraction's end take 2^0.
    struct SWords { uint32_t a[FM], b[FN]; };
    auto stage_words = [&](const ASc& sa, const BSc& sb, int kt) -> SWords {
        SWords w;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            uint32_t lo = sa.w[i][0], hi = sa.w[i][1];
            if constexpr (KTAIL) {
                lo = mask_scale_word(lo, (int64_t)kt * 8, nb);
                hi = mask_scale_word(hi, (int64_t)kt * 8 + 4, nb);
            }
            w.a[i] = stage_scale_word(lo, hi, h);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            uint32_t lo = sb.w[j][0], hi = sb.w[j][1];
            if constexpr (KTAIL) {
                lo = mask_scale_word(lo, (int64_t)kt * 8, nb);
                hi = mask_scale_word(hi, (int64_t)kt * 8 + 4, nb);
            }
            w.b[j] = stage_scale_word(lo, hi, h);
        }
        return w;
    };
    auto mfmas = [&](int s, int set, int r, const SWords& sw) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const v8i af = __builtin_shufflevector(fa[set][i], v4i{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
            const uint32_t wa = sw.a[i];
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const v8i bf = __builtin_shufflevector(fb[r][j], v4i{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
                const uint32_t wb = sw.b[j];
                switch (s) {
                    case 0: acc[i][j] = mfma_fp4<0>(bf, af, acc[i][j], wb, wa); break;
                    case 1: acc[i][j] = mfma_fp4<1>(bf, af, acc[i][j], wb, wa); break;
                    case 2: acc[i][j] = mfma_fp4<2>(bf, af, acc[i][j], wb, wa); break;
                    default: acc[i][j] = mfma_fp4<3>(bf, af, acc[i][j], wb, wa); break;
                }
            }
        }
    };

    // A chunk DMAs of a stage are spread over k-steps 0..2: k-step s issues
    // chunks [kDma(s), kDma(s + 1)) (the scale runs go with k-step 0).
    auto kdma = [](int s) { return s * FM / 3 < FM ? s * FM / 3 : FM; };

    // One stage from slot u (its k-step 0 fragments and scales already in
    // registers).  Stage kt + 3 is loaded into slot (u + 3) mod 4, B scales
    // of stage kt + 2 into the B scale ring, B k-steps 8 ahead into the B ring.
    auto run_stage = [&](int u, int kt) {
        uint8_t* const ahead = slots[(u + 3) % kSlots];
        ASc& nsa = asc[(u + 1) & 1];
        const SWords sw = stage_words(asc[u & 1], bsc[u], kt);
#pragma unroll
        for (int s = 0; s < kKS - 1; ++s) {
            read_afrags(u, s + 1, (s + 1) & 1);
            mfmas(s, s & 1, (4 * u + s) % kRing, sw);
#pragma unroll
            for (int j = 0; j < FN; ++j) fb[(4 * u + s) % kRing][j] = load_b(4 * kt + s + kRing, j);
            dma_a(kt + 3, ahead, kdma(s), kdma(s + 1), s == 0);
            if (s == 0) bsc[(u + 2) % kSlots] = load_bsc(kt + 2);
            // interleave: one MFMA, then a DS read and a VMEM op spread evenly
            constexpr int kM = FM * FN;
            const int nvm = FN + (kdma(s + 1) - kdma(s)) + (s == 0 ? (FAST ? 1 : 2) + FN : 0);
#pragma unroll
            for (int t = 0; t < kM; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA
                if ((t + 1) * FM / kM > t * FM / kM)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // DS read
                if ((t + 1) * nvm / kM > t * nvm / kM)
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);    // VMEM read
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // this wave's DMA of stage kt + 1 (issued two stages ago) has landed,
        // and its fragment reads of `cur` are done; the barrier publishes
        // every wave's part of stage kt + 1.  At least 2 kVmStage - 2 VMEM
        // instructions follow the last one of stage kt + 1: all of stage
        // kt - 1, stage kt up to here, the B loads closing stage kt - 2 (the
        // prologue's order gives exactly that count for the first stages).
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(kWaitStage));
        barrier_after_wait();
        read_ascales((u + 1) % kSlots, kt + 1, nsa);
        read_afrags((u + 1) % kSlots, 0, 0);
        mfmas(kKS - 1, 1, (4 * u + 3) % kRing, sw);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[(4 * u + 3) % kRing][j] = load_b(4 * kt + 3 + kRing, j);
        constexpr int kM = FM * FN, kDs = 2 * FM;
#pragma unroll
        for (int t = 0; t < kM; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // MFMA
            if ((t + 1) * kDs / kM > t * kDs / kM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if ((t + 1) * kDs / kM > t * kDs / kM + 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if ((t + 1) * FN / kM > t * FN / kM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // The first stages of a tile: A stages kfirst .. kfirst+2 into slots
    // 0..2, B scales of the first two stages, B k-steps of the first two
    // stages.  Issued in stage order so that the wait for stage kfirst
    // counts everything after its A part.
    // (The scheduling barriers keep this order: the waits the compiler puts
    // before the first MFMAs of every loop iteration are the deeper of the
    // loop's own distance and this prologue's.)
    auto prologue = [&]() {
        dma_a(kfirst, slots[0], 0, FM, true);
        __builtin_amdgcn_sched_barrier(0);
        bsc[0] = load_bsc(kfirst);
#pragma unroll
        for (int s = 0; s < kKS; ++s)
#pragma unroll
            for (int j = 0; j < FN; ++j) fb[s][j] = load_b(4 * kfirst + s, j);
        __builtin_amdgcn_sched_barrier(0);
        dma_a(kfirst + 1, slots[1], 0, FM, true);
        __builtin_amdgcn_sched_barrier(0);
        bsc[1] = load_bsc(kfirst + 1);
#pragma unroll
        for (int s = kKS; s < 2 * kKS; ++s)
#pragma unroll
            for (int j = 0; j < FN; ++j) fb[s][j] = load_b(4 * kfirst + s, j);
        __builtin_amdgcn_sched_barrier(0);
        dma_a(kfirst + 2, slots[2], 0, FM, true);
        __builtin_amdgcn_sched_barrier(0);
    };
    // VMEM issued after stage kfirst's A part in the prologue: its B scales,
    // the B loads of two stages, two more A stages and one more B scale load
    constexpr int kPro = FN + 2 * kKS * FN + 2 * (FM + (FAST ? 1 : 2)) + FN;
    // stores of a full tile's epilogue per wave (32-row pieces, 4 rows per
    // store instruction)
    constexpr int kEpiStores = FM * 8;

    bool early = false;   // this tile's prologue was issued during the previous epilogue
    // Staggered start: workgroup b begins b x 64 cycles late (about 8 us for
    // 256 workgroups), so that their tile boundaries -- an epilogue writing
    // the finished tile while the next tile's first stages load -- do not
    // all fall at the same moment: measured 1.6-2.4 % faster on launches of
    // several rounds.  A single round would only pay the delay.
    if (ntiles > (int)gridDim.x) {
        for (int q = 0; q < (int)blockIdx.x; ++q) __builtin_amdgcn_s_sleep(1);
    }
    if constexpr (FAST) {
        // Every tile is full: the first tile's prologue goes out here and
        // every later one during the previous tile's epilogue (accumulation
        // aside), so the loop below has a single prologue site (with two, the
        // compiler moved the prologue's B fragments between registers in the
        // middle of the epilogue, waiting for them there).
        set_tile(blockIdx.x);
        prologue();
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
        early = true;
    }
    for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
        // (an accumulating fast-path launch issues no prologue during its
        // epilogues, which read C: its later tiles take theirs here)
        if ((!FAST || ACC) && !early) {
            if (t != (int)blockIdx.x) {
                // every wave is done with the previous tile's LDS before it is refilled
                __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
                barrier_after_wait();
            }
            set_tile(t);
            prologue();
            // (a full drain, once per tile issued this way: the compiler's
            // own waits before the first MFMAs of each loop iteration then
            // follow the loop's steady state, not this prologue's order)
            __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
        } else {
            // the prologue went out before the previous tile's kEpiStores stores
            // (the memory counter completes in order)
            __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(kPro + kEpiStores < 63 ? kPro + kEpiStores : 63));
        }
        barrier_after_wait();
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
        read_ascales(0, kfirst, asc[0]);
        read_afrags(0, 0, 0);
        for (int kt = kfirst; kt < nk; kt += kSlots) {
            run_stage(0, kt);
            run_stage(1, kt + 1);
            run_stage(2, kt + 2);
            run_stage(3, kt + 3);
        }

        // the prefetches past the last stage must land before the slots are
        // refilled (and before the workgroup goes away)
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
        __syncthreads();                                // all fragment reads of the tile are done
        const int64_t em0 = m0, en0 = n0;               // the tile the epilogue writes
        const bool vec_store = (N % 4) == 0;
        // workgroup-uniform; constant on the fast path, whose tiles are all
        // full: the epilogue then has no partial-tile branch, whose zero-store
        // path made the compiler wait for most of these stores before the
        // next tile's first fragment moves
        const bool full_tile = FAST || (vec_store && em0 + BM <= M && en0 + kBN <= N);
        early = false;
        if constexpr (!KTAIL && !ACC) {
            // The next tile's first stages go out now, into slots 0..2 (this
            // epilogue stages in slot 3); waited for at the next tile's start.
            const int tn = t + (int)gridDim.x;
            if (full_tile && tn < ntiles) {
                set_tile(tn);
                prologue();
                early = true;
            }
        }

        // acc[i][j] holds C^T of a 32x32 tile: register r of lane l is
        // n = 8 (r / 4) + 4 (l / 32) + r mod 4, m = l mod 32.  Each wave
        // stages 32 rows x its 64 columns at a time in its quarter of slot 3
        // (rows padded by 16 bytes: conflict-free writes of the accumulator
        // layout and row reads), then reads back four consecutive n of a row
        // per lane, 16 lanes per row, so that one store instruction writes
        // four whole rows of the wave's columns (fp32: two 128-byte lines
        // each, written non-temporally); with N % 4 != 0 (rows not 16-byte
        // aligned) elements go one by one.
        uint8_t* const reg = lds3 + wave * kEpiRegion;
        const int lr = lane >> 4, c4 = (lane & 15) * 4;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int cn = j * 32 + 8 * q + 4 * h;
                    *reinterpret_cast<float4*>(reg + l32 * kEpiRow + cn * 4) =
                        make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                    acc[i][j][4 * q + 3]);
                }
            if (full_tile) {
                float4 f[8];
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    f[k] = *reinterpret_cast<const float4*>(reg + (4 * k + lr) * kEpiRow + c4 * 4);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int64_t m = em0 + i * 32 + 4 * k + lr;
                    const int64_t n = en0 + 64 * wave + c4;
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
                continue;
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int row = 4 * k + lr;
                const float4 f = *reinterpret_cast<const float4*>(reg + row * kEpiRow + c4 * 4);
                const int64_t m = em0 + i * 32 + row, n = en0 + 64 * wave + c4;
                if (m >= M || n >= N) continue;
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

// Compute units of each device, queried once per device (concurrent first
// calls may both query; they store the same value).
int cu_count() {
    static std::atomic<int> counts[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = counts[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        counts[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Tile-rows per group of the block order (each XCD runs 32 tiles at a time):
// groups of 2 to 4 rows measured best on the gate/up and q_proj shapes.
constexpr int kGroupRows = 4;

template <int FM, bool FAST, bool KTAIL, bool OBF16, bool ACC>
hipError_t launch_one(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs,
                      int64_t M, int64_t N, int64_t K, void* c, dim3 grid, int tm, int tn, hipStream_t st) {
    void (*k)(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, int64_t, int64_t, int64_t,
              void*, int, int) = gemm_mx_tn<FM, kGroupRows, FAST, KTAIL, OBF16, ACC>;
    void* args[] = {(void*)&aq, (void*)&as, (void*)&bq, (void*)&bs, (void*)&M, (void*)&N,
                    (void*)&K, (void*)&c, (void*)&tm, (void*)&tn};
    return hipLaunchKernel((const void*)k, grid, dim3(kThreads), args, 0, st);
}

template <int FM, bool OBF16, bool ACC>
hipError_t launch_kernel(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs,
                         int64_t M, int64_t N, int64_t K, void* c, hipStream_t st) {
    const int64_t tm = (M + 32 * FM - 1) / (32 * FM), tn = (N + kBN - 1) / kBN;
    const int64_t cus = cu_count();
    const dim3 grid((unsigned)(tm * tn < cus ? tm * tn : cus));
    // the fast path: full tiles, K a multiple of 1024, and every scale
    // offset (stage q of row r at (q R + r) 8) within 31 bits
    const bool fast = M % (32 * FM) == 0 && N % kBN == 0 && K % 1024 == 0 &&
                      (K / 256) * (M > N ? M : N) * 8 < (INT64_C(1) << 31);
    if (fast) return launch_one<FM, true, false, OBF16, ACC>(aq, as, bq, bs, M, N, K, c, grid, (int)tm, (int)tn, st);
    if (K % 256 == 0)
        return launch_one<FM, false, false, OBF16, ACC>(aq, as, bq, bs, M, N, K, c, grid, (int)tm, (int)tn, st);
    return launch_one<FM, false, true, OBF16, ACC>(aq, as, bq, bs, M, N, K, c, grid, (int)tm, (int)tn, st);
}

template <int FM>
hipError_t launch_out(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs,
                      int64_t M, int64_t N, int64_t K, void* c, int out_bf16, int accumulate,
                      hipStream_t st) {
    if (out_bf16)
        return accumulate ? launch_kernel<FM, true, true>(aq, as, bq, bs, M, N, K, c, st)
                          : launch_kernel<FM, true, false>(aq, as, bq, bs, M, N, K, c, st);
    return accumulate ? launch_kernel<FM, false, true>(aq, as, bq, bs, M, N, K, c, st)
                      : launch_kernel<FM, false, false>(aq, as, bq, bs, M, N, K, c, st);
}

}  // namespace

hipError_t launch_gemm_mx(const uint8_t* aq, const uint8_t* as, const uint8_t* bq,
                          const uint8_t* bs, int64_t M, int64_t N, int64_t K, void* c,
                          int out_bf16, int accumulate, hipStream_t st) {
    // Tile rows: the persistent grid runs ceil(tiles / CUs) rounds of one
    // tile per CU, each costing about the tile's area, so take the height
    // with the least rounds x height (256 unless 224 removes a partly idle
    // last round, e.g. M = 14336 = 64 x 224).
    const int64_t cus = cu_count();
    const int64_t tn = (N + kBN - 1) / kBN;
    auto cost = [&](int64_t bm) {
        const int64_t tiles = ((M + bm - 1) / bm) * tn;
        return ((tiles + cus - 1) / cus) * bm;
    };
    if (cost(224) < cost(256)) return launch_out<7>(aq, as, bq, bs, M, N, K, c, out_bf16, accumulate, st);
    return launch_out<8>(aq, as, bq, bs, M, N, K, c, out_bf16, accumulate, st);
}

}  // namespace fp4dev

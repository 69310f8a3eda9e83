/*
 * fp4_calib.h -- C ABI of libfp4calib.so, a measurement aid that sits beside
 * libfp4.so and is not part of the quantized-GEMM path.
 *
 * The scaled FP4 GEMM's roofline is the chip's dense MXFP4 matrix peak, a
 * figure for the nominal 2.4 GHz clock.  Under a sustained MFMA load the
 * card runs at a lower clock set by its power limit, and that clock depends
 * on the data: random E2M1 operands toggle more bits than constant ones.
 * fp4_calib_mfma measures the rate a GEMM could at best reach on this card:
 * every wave of a persistent grid issues nothing but independent
 * V_MFMA_SCALE_F32_32X32X64_F8F6F4 instructions (both operands FP4, fp32
 * accumulation) on random operands held in registers -- the wave tile of the
 * Wgrad GEMM (7 x 2 accumulator tiles of 32 x 32) and its two fragment sets,
 * alternated every k-step as the GEMM does -- with no memory traffic and no
 * LDS use in the loop.  It also reads the shader clock counter and the
 * 100 MHz reference clock around the loop, so the caller can derive the
 * shader clock the loop ran at.
 *
 * Conventions as in fp4.h: device pointers owned by the caller, work
 * enqueued on `stream` (a hipStream_t), arguments checked before any HIP
 * call, the return value is the only error channel (0 ok, 1 NULL pointer,
 * 2 bad size, 3 misaligned pointer, 5 launch refused).
 */
#ifndef FP4_CALIB_H_
#define FP4_CALIB_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of operand data one fp4_calib_mfma call with `grid` workgroups reads
 * (once, before its loop): 18 fragments of 16 bytes per lane, 256 lanes per
 * workgroup.  0 for grid <= 0. */
size_t fp4_calib_mfma_src_bytes(int grid);

/* Floating-point operations of one call: 2 * 32 * 32 * 64 per MFMA, 28 MFMAs
 * per wave per iteration, 4 waves per workgroup. */
double fp4_calib_mfma_flops(int grid, int iters);

/* Runs `grid` workgroups of 4 waves, each wave `iters` iterations of 28
 * independent scaled FP4 MFMAs (E8M0 scales 127, i.e. 2^0).
 *   src     device, fp4_calib_mfma_src_bytes(grid) bytes of operand codes
 *           (the caller fills them, e.g. with uniform random bytes), 16-byte
 *           aligned
 *   out     device, grid * 256 floats: each lane's sum of its accumulators
 *           (keeps the work observable; the values are not meaningful)
 *   clocks  device, grid * 4 * 2 uint64: per wave, the shader clock counter
 *           ticks and the 100 MHz reference clock ticks its loop took
 * grid in [1, 65536], iters in [1, 2^24].  Returns 0 when the launch was
 * enqueued. */
int fp4_calib_mfma(const void* src, int grid, int iters, float* out, uint64_t* clocks, void* stream);

/* Workgroups launched by one fp4_calib_clock_stamp call. */
#define FP4_CALIB_STAMPS 32

/* Enqueues FP4_CALIB_STAMPS one-wave workgroups on `stream`; workgroup i
 * writes record i of `out` (device, FP4_CALIB_STAMPS * 4 uint64, 8-byte
 * aligned): the shader clock counter, the 100 MHz reference counter, and the
 * id of the XCD it ran on (0..7), then a zero.  Two stamps around a stretch
 * of work on the same stream give the average shader clock over it, ticks /
 * reference ticks * 100 MHz, from any pair of records of the same XCD (each
 * XCD counts its own clock).  Returns 0 when enqueued, 1 for a null `out`,
 * 3 if it is misaligned, 5 if the launch failed. */
int fp4_calib_clock_stamp(uint64_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4_CALIB_H_ */

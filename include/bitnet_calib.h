/*
 * bitnet_calib.h -- calibration kernels of the MI355X (gfx950) BitLinear
 * library: the measured ceilings its kernels are reported against, next to
 * the chip's nominal peaks.  Not part of the BitLinear hot path; the
 * benchmark runs them on the same device and in the same process.
 *
 * A bandwidth-bound BitLinear call (the packed decode GEMV, the quantizers)
 * reads a known byte count in one launch, so its practical ceiling is the
 * plainest one-launch read of that many bytes, launch, ramp and drain
 * included ("1.58-bit量化技术突破AI算力与内存墙限制", section 1: decode is
 * bound by the weight stream, the memory wall).  A contraction on the matrix
 * cores is compared with back-to-back MFMAs on random operands at the clock
 * the part holds under that load.
 *
 * Conventions as include/bitnet.h: device pointers, the caller owns every
 * buffer, calls only enqueue on `stream` (hipStream_t as void*; NULL = the
 * null stream), arguments are checked before any launch and a failure
 * returns a negative bitnet_status with nothing enqueued.
 */
#ifndef BITNET_CALIB_H_
#define BITNET_CALIB_H_

#include <stddef.h>
#include <stdint.h>

#include "bitnet.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BITNET_CALIB_MFMA_I8 = 0,          /* int8 x int8, both random bytes            */
    BITNET_CALIB_MFMA_BF16 = 1,        /* bf16 x bf16, both random in +-[1, 2)       */
    BITNET_CALIB_MFMA_I8_TERNARY = 2,  /* random int8 x ternary codes (0, +1, -1)    */
    BITNET_CALIB_MFMA_BF16_TERNARY = 3 /* random bf16 x ternary codes as bf16        */
} bitnet_calib_mfma_kind;

/*
 * Read `bytes` bytes at `src` once: 16-byte global loads, grid-stride
 * over `workgroups` workgroups of 256 threads, four loads in flight per
 * thread.  Nothing is written except, for one 2^-32 chance per workgroup in
 * the XOR of the data, one word of `sink`.
 *   src   device, 16-byte aligned, bytes % 16 == 0, bytes >= 16
 *   sink  device, 4 bytes, 4-byte aligned
 *   workgroups in [1, 2^20]
 * Errors: BITNET_E_ARG, BITNET_E_SHAPE, BITNET_E_ALIGN, BITNET_E_HIP.
 */
int bitnet_calib_stream_read(const void *src, int64_t bytes, int workgroups, uint32_t *sink, void *stream);

/*
 * `iters` iterations of eight dependent-free MFMAs per wave (four
 * accumulators, each fed twice per iteration), 4 waves per workgroup:
 * the int8 kinds run v_mfma_i32_32x32x32_i8 (65536 int8 ops each), the bf16
 * kinds v_mfma_f32_32x32x16_bf16 (32768 flops each), on pseudo-random
 * operands held in registers.  The ternary kinds draw the second operand as
 * the BitLinear codes (0 with probability about 0.35, else +1 or -1), the
 * operand mix of the ternary x int8 forward and of the grad_x product: with
 * fewer bits toggling the part holds a higher clock than on two random
 * operands.
 *   sink    device, 4 bytes (written only if the folded result hits one
 *           32-bit value)
 *   clocks  device, [workgroups][2] uint64, written: wave 0's shader clock
 *           cycles and 100 MHz real-time ticks over its loop, so that
 *           cycles / ticks * 100 MHz is the clock the part held
 * Errors: BITNET_E_ARG (NULL pointer, unknown kind), BITNET_E_SHAPE
 * (workgroups outside [1, 2^20], iters < 1), BITNET_E_ALIGN, BITNET_E_HIP.
 */
int bitnet_calib_mfma(int kind, int workgroups, int iters, uint32_t *sink, uint64_t *clocks, void *stream);

/* Operations one bitnet_calib_mfma launch performs (0 for bad arguments). */
double bitnet_calib_mfma_ops(int kind, int workgroups, int iters);

#ifdef __cplusplus
}
#endif

#endif /* BITNET_CALIB_H_ */

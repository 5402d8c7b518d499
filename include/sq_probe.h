/*
 * sq_probe.h - C ABI of libsq_probe, the measurement probe that bench.py
 * uses to price the INT8 GEMM against what the chip's matrix cores sustain.
 *
 * The INT8 GEMM's speed rests on the integer matrix instructions running at
 * about twice the 16-bit rate ("SmoothQuant" explainer, "How it works",
 * Step 7). The dense peak on paper assumes the top shader clock; under a
 * long MFMA load the clock settles lower and depends on the operands (how
 * many bits toggle), so the practical ceiling is measured here: a kernel of
 * INT8 MFMAs only (no memory traffic in the timed loop), with the GEMM's
 * occupancy, and the shader clock it runs at.
 *
 * Not part of the hot path; no call here is used by libsq.
 */
#ifndef SQ_PROBE_H
#define SQ_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Launches `blocks` workgroups of 8 waves (two per SIMD, as the GEMM's
 * 256x256 tiles run), each wave holding 8 independent 32x32 INT32
 * accumulators and issuing `iters` x 64 V_MFMA_I32_32X32X32_I8 from
 * registers (65536 integer operations each). Operands: mode 0 - the same
 * constant fragment in every MFMA; mode 1 - eight random fragments per
 * operand, loaded once from `rnd` (device, at least blocks * 512 * 64
 * int32 words), paired differently in each MFMA so the operands change
 * every instruction, as in a GEMM. clk: device [blocks, 2] uint64, written
 * by each block's wave 0 with the shader-clock (S_MEMTIME) and 100 MHz
 * reference-clock (S_MEMREALTIME) ticks its timed loop took. sink: device
 * [blocks * 512] int32, written (keeps the accumulators live).
 * Returns 0, or -1 for bad arguments, -6 for a launch error. Asynchronous on
 * `stream` (hipStream_t as void*). */
int sq_probe_mfma_i8(int mode, int blocks, int iters, const int32_t* rnd, uint64_t* clk,
                     int32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SQ_PROBE_H */

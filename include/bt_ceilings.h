/*
 * bt_ceilings.h — what the hardware itself reaches, measured on the part the
 * library runs on: the rate at which the int8 matrix-core instruction the
 * ternary matmul is built on (v_mfma_i32_16x16x64_i8) retires, the shader
 * clock while it runs, and the bandwidth of a plain streaming read at a given
 * size. They give the library's kernels denominators that are
 * measured rather than only published values.
 *
 * A separate library (libbt_ceilings.so): nothing here is part of the matmul
 * path, and the matmul library does not depend on it.
 *
 * All calls are asynchronous on the given stream; the caller times them with
 * events on that stream. Every status is 0 on success, 2 for a size or grid
 * outside the stated range, 1 for a null pointer and 5 when the launch fails
 * (hipGetLastError after the launch); nothing is launched on an argument error.
 */
#ifndef BT_CEILINGS_H
#define BT_CEILINGS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Matrix-core issue rate. `blocks` workgroups of four waves (1 <= blocks <=
 * 65536) each run `iters` (1 <= iters <= 1 << 20) rounds of eight independent
 * v_mfma_i32_16x16x64_i8 on operands held in registers (every A byte
 * `a_byte`, every B byte `b_byte`); no memory is touched inside the loop.
 * That is blocks * 4 * iters * 8 instructions of 16 * 16 * 64 multiply-adds
 * (2 ops each).
 *   out     int32[blocks * 256] (device): thread t writes the sum of the four
 *           elements of its eight accumulators, which is exactly
 *           32 * 64 * iters * a_byte * b_byte in int32 arithmetic (wrapping),
 *           the same for every thread: a check that every instruction ran.
 *   clocks  int64[4] (device): workgroup 0's first wave writes clock64() and
 *           wall_clock64() at the start of its loop (clocks[0], clocks[1]) and
 *           at its end (clocks[2], clocks[3]). With the wall clock's rate
 *           (hipDeviceAttributeWallClockRate, kHz) this gives the shader clock
 *           while the instructions ran.
 */
int btc_mfma_i8_issue(int blocks, int iters, int8_t a_byte, int8_t b_byte, int32_t* out,
                      int64_t* clocks, hipStream_t stream);

/* Rate of wall_clock64() on `device` in kHz (hipDeviceAttributeWallClockRate);
 * -1 if the runtime cannot tell. Synchronous, launches nothing. */
int btc_wall_clock_khz(int device);

/*
 * Streaming read of `bytes` bytes at `p` (device; p and out 16-byte aligned; bytes a
 * positive multiple of 16, at most 2^40) by `blocks` workgroups of 256
 * threads (1 <= blocks <= 65536) in a grid-stride loop of 16-byte
 * non-temporal loads, eight in flight per thread.
 *   out  uint32[blocks * 4 * 4] (device): each wave writes the XOR of every
 *        16-byte vector it read (4 words); the XOR of all of them is the XOR
 *        of the whole buffer, which checks that every byte was read.
 */
int btc_stream_read(const void* p, int64_t bytes, int blocks, uint32_t* out,
                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BT_CEILINGS_H */

/*
 * lstm_peaks.h -- C ABI of the measured-peak microbenchmarks that the
 * stacked-LSTM forward library's rooflines are read against.
 *
 * The forward pass is bound, depending on the shape, by the matrix cores
 * (grouped input projection, "Optimizing Performance of Recurrent Neural
 * Networks on GPUs", proposed method), by the rate at which weights kept on
 * chip can be re-read every step ("Persistent RNNs: Stashing Recurrent Weights
 * On-Chip", citing quotes on caching weights across timesteps), or by the
 * latency of making h_t visible to every workgroup before step t+1 (the same
 * page: one launch for the whole sequence).  These kernels measure each of
 * those limits on the device they run on, so a kernel's fraction can be given
 * against the measured rate as well as the published one.
 *
 * Every entry point enqueues its kernel(s) on `stream` between the two
 * caller-created events `ev0` and `ev1` (recorded by the library) and returns
 * without waiting; the caller synchronises and reads the elapsed time.  No
 * entry point allocates memory.  Errors: 0 on success, 1 for a bad argument
 * (NULL pointer, size out of range), 2 for a failed HIP call or launch.
 */
#ifndef LSTM_PEAKS_H
#define LSTM_PEAKS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Matrix-core rate: `grid` workgroups of 256 threads, every wave issuing
 * `iters` rounds of 8 independent MFMAs on register operands.
 *   kind 0: v_mfma_f32_16x16x32_bf16   (16384 FLOPs each)
 *   kind 1: v_mfma_f32_32x32x16_bf16   (32768 FLOPs each)
 *   kind 2: v_mfma_f32_16x16x4_f32     (2048 FLOPs each)
 * `out` (device, >= 1 float) receives a value only if `sink` is non-zero (it
 * keeps the products live).  FLOPs = grid * 4 * iters * 8 * (FLOPs each).
 */
int lstm_peak_mfma(int kind, int grid, int iters, float *out, int sink, hipStream_t stream, hipEvent_t ev0,
                   hipEvent_t ev1);

/*
 * Memory rate over a device buffer `buf` of `bytes` bytes (a multiple of 16,
 * 16-byte aligned): mode 0 reads it once (16-byte loads, grid-stride);
 * mode 1 copies its first half onto its second half.  `out` (>= 16 bytes)
 * receives a value only if `sink` is non-zero.  Bytes moved: `bytes` for
 * mode 0 and for mode 1 (half read, half written).
 */
int lstm_peak_memory(int mode, void *buf, size_t bytes, int grid, void *out, int sink, hipStream_t stream,
                     hipEvent_t ev0, hipEvent_t ev1);

/*
 * LDS read rate: `grid` workgroups of 256 threads, each lane issuing `iters`
 * rounds of 8 conflict-free 16-byte LDS reads (ds_read_b128; a wave reads
 * 1 KiB contiguous per read).  LDS bytes read = grid * 256 * iters * 8 * 16.
 * `out` (>= 16 bytes) receives a value only if `sink` is non-zero.
 */
int lstm_peak_lds(int grid, int iters, void *out, int sink, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);

/*
 * Step-exchange latency: one cooperative launch of `grid` workgroups (one per
 * CU, 256 threads) runs `steps` steps of the forward kernels' step protocol
 * among the workgroups whose id is a multiple of `stride` (stride 1: every
 * workgroup; stride 8: every 8th, which the dispatcher places on one XCD):
 *   each active workgroup writes its `slice_bytes` (a multiple of 1024) of the
 *   step's slot, waits for those stores, bumps its step counter; then polls
 *   every active counter and reads the whole slot (active * slice_bytes).
 *   scope 0: agent-scope (write-through) stores and device-coherent polls, as
 *            the forward kernels use -- correct across XCDs;
 *   scope 1: ordinary stores and L2-level polls (the L1 bypassed, the L2
 *            not), correct only when every active workgroup shares one XCD.
 * `ws` (device) holds: 256 B error word | 256 x 128 B counters | `steps`
 * slots of active * slice_bytes -- lstm_peak_step_ws_bytes() bytes.  Its
 * contents on entry are ignored (the first kernel clears it).  Every wait is
 * bounded by `timeout_us`; a timeout sets the error word (read it with
 * hipMemcpy after the stream is done: non-zero means the run is invalid).
 * `xcc` (device, >= grid ints, may be NULL) receives each workgroup's XCD id.
 */
size_t lstm_peak_step_ws_bytes(int grid, int stride, int slice_bytes, int steps);
int lstm_peak_step(int grid, int stride, int scope, int slice_bytes, int steps, int64_t timeout_us, void *ws,
                   int *xcc, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);

#ifdef __cplusplus
}
#endif

#endif /* LSTM_PEAKS_H */

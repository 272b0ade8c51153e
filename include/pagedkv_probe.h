/* pagedkv_probe.h -- a measurement aid shipped with libpagedkv.
 *
 * Not an operation of the attention path, and no part of the pages' method:
 * it measures the HBM gather a decode step makes, without the decode.  A
 * benchmark hands it the K and V runs a decode reads (16 KiB each for the
 * four adjacent kv-head tiles of one block with bf16, head_dim 128) and times
 * it beside the decode call: the ratio of the two rates says how much of the
 * achievable gather bandwidth the decode reaches.
 *
 * Conventions are those of pagedkv.h (kv_status returns, kv_last_error,
 * caller-owned device memory, asynchronous work on the caller's stream).
 */
#ifndef PAGEDKV_PROBE_H
#define PAGEDKV_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Device: read run_bytes bytes at k_base + k_offsets[i] and at
 * v_base + v_offsets[i] for every i < n_runs, with 16-byte loads, on a grid of
 * `workgroups` workgroups of 256 threads; workgroup c takes runs
 * [c*n_runs/workgroups, (c+1)*n_runs/workgroups).  sink (device uint32
 * [workgroups]) receives each workgroup's XOR of the 32-bit words it read, so
 * the XOR over sink is the XOR of every word of every run.
 * k_offsets, v_offsets: device int64 [n_runs], multiples of 16; the runs must
 * lie inside the caller's buffers (device-resident offsets are a caller
 * contract, not checked).  Errors: KV_E_INVALID for NULL pointers, a negative
 * n_runs, run_bytes not a positive multiple of 16, or workgroups outside
 * [1, 65535]; KV_E_HIP if the launch fails. */
int kv_probe_gather(const void* k_base, const void* v_base, const int64_t* k_offsets,
                    const int64_t* v_offsets, int32_t n_runs, int32_t run_bytes, uint32_t* sink,
                    int32_t workgroups, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif

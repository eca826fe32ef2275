/*
 * crosscu debug hooks: an in-kernel timeline of the persistent decode launch.
 *
 * With a timeline buffer set, every workgroup of a later cc_decode /
 * cc_decode_variant launch on any stream records eight uint64 words at
 * buf[8 * w .. 8 * w + 7], times on the constant 100 MHz clock
 * (s_memrealtime):
 *   [0] start,
 *   [1] all its waves have finished streaming KV,
 *   [2] its items shared by waves or split across workgroups are merged and
 *       written (outputs, or partials for split units),
 *   [3] its arrival counters are updated (equal to [2] without the in-kernel
 *       merge),
 *   [4] exit, after merging the units it completed,
 *   [5] the id of the XCD (accelerator complex die) it ran on,
 *   [6], [7] GQA kernel: its merge-slot scan, then the per-head (max, sum)
 *       pass of [2] are done; MLA kernel: unused (0).
 * The MLA kernel publishes its pieces' partials inside its stream and
 * arrives after it, so its [2] equals [1]; between [1] and [4] it arrives,
 * waits for its split units to complete and merges head slices of them, and
 * its [3] equals [4].
 * Workgroups with no work record [0] == [1] == ... == [4] (and [6], [7]).  From these the caller
 * computes the busy fraction of the compute units over the launch and checks
 * the workgroup-to-XCD placement the planner assumes (workgroup w on XCD
 * w mod num_xcds).
 */
#ifndef CROSSCU_DEBUG_H
#define CROSSCU_DEBUG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Sets (buf != NULL) or clears (buf == NULL) the timeline buffer for this
 * process.  buf: device memory of `bytes` bytes; launches whose worker count
 * exceeds bytes / 64 record nothing.  The library only writes to it from
 * kernels; the caller owns it and must keep it alive while set.  Returns
 * CC_OK. */
int cc_debug_timeline(void* buf, size_t bytes);

/* Sets (both non-NULL) or clears (both NULL) a pair of HIP events
 * (hipEvent_t, created by the caller with timing enabled) that later
 * cc_decode / cc_decode_variant / cc_probe_read / cc_probe_mfma / cc_indexer_topk / cc_moe_gemm calls on
 * any stream record
 * through hipExtLaunchKernel: start_event when the call's first kernel
 * begins, stop_event when its last kernel ends.  The time between them covers the
 * call's kernels (both kernels of the split-then-combine variant, and the gap
 * between them), without the queue markers an ordinary event record adds
 * around a launch.  The caller owns the events and must keep them alive while
 * set.  Returns CC_OK, or CC_ERR_INVALID when only one event is given. */
int cc_debug_kernel_events(void* start_event, void* stop_event);

/* MLA in-kernel merge: once a workgroup has finished its chunk, it polls each
 * split unit it holds a piece of until every piece has arrived, then merges
 * head slices of it.  After `polls` polls it stops waiting and leaves those
 * slices to the unit's other pieces (the last piece to arrive never waits and
 * merges whatever is left).  This sets the poll limit for later launches on
 * the current device; polls < 0 restores the default (512).  Lowering it
 * exercises the path where pieces stop waiting; the result is the same.
 * Returns CC_OK or CC_ERR_HIP. */
int cc_debug_merge_poll_limit(int polls);

/* Streaming-read probe: reads `bytes` (a multiple of 16 KiB, >= 16 KiB) of
 * device memory `buf` once with `workgroups` persistent workgroups of 512
 * threads, asynchronously on `stream`, so the caller can time the practical
 * HBM read ceiling of a load path.
 *   method 0: 128-bit loads into registers, 8 per lane in flight;
 *   method 1: 128-bit loads straight into LDS, one 16 KiB slot per wave;
 *   method 2: the same into two 8 KiB slots per wave, one refilling while
 *             the other is read;
 *   methods 3, 4: methods 0 and 2 with the non-temporal cache policy (nt),
 *             the policy the decode kernels read the KV cache with.
 * pages: optional device int32[num_pages], a read order of page_bytes-sized
 * pages (page_bytes a multiple of 16 KiB); NULL reads contiguously.  sink:
 * device uint32[workgroups * 512], written.  Returns CC_OK, CC_ERR_INVALID or
 * CC_ERR_HIP. */
int cc_probe_read(const void* buf, long long bytes, int method, const int32_t* pages, int page_bytes,
                  int num_pages, int workgroups, void* sink, void* stream);

/* MFMA ceiling probe: `workgroups` x `waves_per_workgroup` waves (1..8 per
 * workgroup) each run `iters` rounds of 8 independent
 * v_mfma_f32_32x32x16_bf16 accumulations (32768 flops each) on register
 * operands, with no memory traffic, asynchronously on `stream`; the rate the
 * caller times is the practical dense bf16 MFMA ceiling the MLA and MoE
 * kernels' MFMA fractions can be placed against.  Flops of one call:
 * workgroups * waves_per_workgroup * iters * 8 * 32768.  sink: device
 * uint32[workgroups * waves_per_workgroup * 64], written.  Returns CC_OK,
 * CC_ERR_INVALID or CC_ERR_HIP. */
int cc_probe_mfma(int workgroups, int waves_per_workgroup, int iters, void* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CROSSCU_DEBUG_H */

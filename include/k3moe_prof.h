/* k3moe profiling entry: the whole layer with every kernel launch timed by its own pair
 * of events. For measurement tools only; the result is identical to k3moe_layer. */
#ifndef K3MOE_PROF_H
#define K3MOE_PROF_H

#include <stddef.h>
#include <stdint.h>

#include "k3moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* As k3moe_layer. events[0 .. max_events-1] are hipEvent_t handles created by the
 * caller (timing enabled). Kernel launch i of the call takes the pair events[2 i] and
 * events[2 i + 1], which the HIP runtime binds to that kernel's own start and end
 * (hipExtLaunchKernel), so their interval is the kernel's duration without the launch
 * gaps around it. Launches beyond max_events / 2 (at most 64) run untimed. *n_kernels
 * receives the number of timed launches; k3moe_prof_name(i) names the step launch i
 * belongs to (static storage; a step such as the dispatch may take several launches).
 * The binding of events to launches is per host thread: a profiled call times the
 * launches its own thread makes, and plain calls on other threads meanwhile take no
 * events. k3moe_prof_name reads the calling thread's last profiled call. */
int k3moe_layer_profiled(const k3moe_dims *d, int32_t T, const uint16_t *x, const k3moe_weights *w,
                         float *y, int32_t *topk_idx_out, float *topk_w_out, void *ws, size_t ws_bytes,
                         void *stream, void **events, int max_events, int *n_kernels);
const char *k3moe_prof_name(int i);

/* As k3moe_shared_glu_bf16, its launches timed as in k3moe_layer_profiled. */
int k3moe_shared_profiled(const k3moe_dims *d, int32_t n_shared, int32_t T, const uint16_t *x,
                          const uint16_t *sh1, const uint16_t *sh3, const uint16_t *sh2, float *y,
                          void *ws, size_t ws_bytes, void *stream, void **events, int max_events,
                          int *n_kernels);

/* TESTS AND MEASUREMENT ONLY. Which kernels run the expert passes, for tests and
 * measurement that compare the two forms on the same inputs: 0 = by batch size (the
 * default: the grouped GEMM form when the batch averages at least 6.25 token-expert pairs
 * per expert), 1 = always the grouped GEMV form, 2 = the grouped GEMM form wherever its
 * shape limits allow (the pass's K a multiple of 128 and its activation records under
 * 2 GiB). Both forms give the same result up to fp32 summation order. The mode is per
 * host thread: it applies to the later calls of the thread that set it and to no other
 * thread's. Returns the thread's previous mode, or K3MOE_EINVAL for another value. */
int k3moe_set_expert_path(int mode);

/* MEASUREMENT ONLY. The grouped GEMM form's tiling, for load-balance reports: the most
 * tokens per column tile, and rows per block of the gate/up pass (of w1 and of w3 each) and
 * of the down pass. An expert's n tokens take ceil(n / tile_tokens) column tiles of
 * ceil(n / tiles) tokens rounded up to a multiple of 32 (the last tile takes the rest).
 * Entry q of the (column tile, row block) list, tiles in expert order, runs on XCD
 * q / ceil(entries / 8). In the GEMM form chosen by batch size (not a forced one), the
 * experts of at most *small_pairs pairs take no tiles: the grouped GEMV's decode kernel
 * runs them. */
int k3moe_prof_gemm_tiling(int *tile_tokens, int *rows_gateup, int *rows_down, int *small_pairs);

#ifdef __cplusplus
}
#endif
#endif

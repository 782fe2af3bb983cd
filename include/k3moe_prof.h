/* k3moe profiling entry: the whole layer with an event mark after every kernel.
 * For measurement tools only; the result is identical to k3moe_layer. */
#ifndef K3MOE_PROF_H
#define K3MOE_PROF_H

#include <stddef.h>
#include <stdint.h>

#include "k3moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* As k3moe_layer. events[0 .. max_events-1] are hipEvent_t handles created by the
 * caller (timing enabled); events[0] is recorded on the stream before the first kernel
 * and events[i] right after kernel i-1, for as many kernels as fit. *n_kernels receives
 * the number of kernels marked; k3moe_prof_name(i) names kernel i of that call (static
 * storage). Not reentrant: one profiled call at a time per process. */
int k3moe_layer_profiled(const k3moe_dims *d, int32_t T, const uint16_t *x, const k3moe_weights *w,
                         float *y, int32_t *topk_idx_out, float *topk_w_out, void *ws, size_t ws_bytes,
                         void *stream, void **events, int max_events, int *n_kernels);
const char *k3moe_prof_name(int i);

/* Which kernels run the expert passes, for tests and measurement that compare the two
 * forms on the same inputs: 0 = by batch size (the default: the grouped GEMM form when
 * the batch averages at least two token-expert pairs per expert), 1 = always the
 * grouped GEMV form, 2 = the grouped GEMM form wherever its shape limits allow (the
 * pass's K a multiple of 128 and its activation records under 2 GiB). Both forms give
 * the same result up to fp32 summation order. Process-wide, not synchronised with calls
 * in flight on other threads. Returns the previous mode, or K3MOE_EINVAL for another
 * value. */
int k3moe_set_expert_path(int mode);

#ifdef __cplusplus
}
#endif
#endif

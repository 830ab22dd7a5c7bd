/*
 * ttt_prof.h - kernel timing hooks of the TTT-E2E library (measurement only).
 *
 * ttt_prof_begin selects one kernel class. Every launch of that class made by
 * the following ttt_prefill / ttt_decode calls is bracketed by two hipEvents
 * recorded on the caller's stream (the stream the kernels run on), and the
 * launch's algorithmic work is accumulated:
 *   TTT_PROF_GEMM      2*M*N*K flops per launch (all MFMA GEMMs)
 *   TTT_PROF_ATTN_FWD  4*hd*H*(visible query-key pairs) flops per launch
 *   TTT_PROF_ATTN_BWD  4*hd*H*(pairs + in-chunk pairs) flops (dQ, dK, dV)
 *   TTT_PROF_CE        bytes: 4*V read (+ element size * V written) per row
 *   TTT_PROF_MLP_UP    2*M*N*K flops, only the MLP up-projection GEMM with
 *                      the activation in its epilogue over a full prefill
 *                      span (frozen blocks, M = batch * span: one kernel
 *                      instance)
 * ttt_prof_end waits for the recorded events and returns the summed event
 * time (ms), the launch count and the summed work, then switches timing off.
 * Timing adds event records between launches; leave it off for throughput.
 * Errors: TTT_EINVAL (NULL model, unknown class), TTT_EHIP.
 */
#ifndef TTT_PROF_H
#define TTT_PROF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TTT_PROF_GEMM 0
#define TTT_PROF_ATTN_FWD 1
#define TTT_PROF_ATTN_BWD 2
#define TTT_PROF_CE 3
#define TTT_PROF_MLP_UP 4

struct ttt_model;
int ttt_prof_begin(struct ttt_model* m, int32_t kernel_class);
int ttt_prof_end(struct ttt_model* m, double* total_ms, int64_t* launches, double* total_work);

#ifdef __cplusplus
}
#endif

#endif /* TTT_PROF_H */

/*
 * ttt_prof.h - kernel timing hooks of the TTT-E2E library (measurement only).
 *
 * ttt_prof_begin selects a kernel class. Every launch of that class made by
 * the following ttt_prefill / ttt_decode calls is timed by two hipEvents
 * attached to the dispatches of its own kernels (the first kernel records the
 * start, the last the end; hipExtLaunchKernelGGL), and the launch's algorithmic work (flops
 * and HBM bytes of what the step must compute, not of what a kernel happens
 * to re-read or recompute) is accumulated. The classes:
 *   TTT_PROF_GEMM        every matrix product (the union of 5, 6 and 7)
 *   TTT_PROF_ATTN_FWD    sliding-window attention forward (with its key-split
 *                        merge): 4*hd*H*(visible query-key pairs) flops
 *   TTT_PROF_ATTN_BWD    attention backward (the union of 8 and 9)
 *   TTT_PROF_CE          fused softmax / cross entropy / logit gradient:
 *                        4*V bytes read (+ element size * V written) per row
 *   TTT_PROF_MLP_UP      the frozen blocks' MLP up-projection with the
 *                        activation fused, over a full prefill span (one
 *                        kernel instance; a subset of 5)
 *   TTT_PROF_GEMM_SPAN   products of the frozen-prefix passes
 *   TTT_PROF_GEMM_CHUNK  forward and input-gradient products of the chunk loop
 *   TTT_PROF_GEMM_SGD    weight-gradient products with the SGD step fused
 *                        (flops 2*M*N*K; bytes: operands, the fp32 master
 *                        read and written and one compute copy written)
 *   TTT_PROF_ATTN_DQ     dQ over the window: 4*hd*H*pairs flops (dP, dQ)
 *   TTT_PROF_ATTN_DKDV   dK, dV of the chunk's own keys: 4*hd*H*(in-chunk
 *                        pairs) flops
 *   TTT_PROF_NORM        RMSNorm forward and backward (bytes)
 *   TTT_PROF_OTHER       the remaining row / elementwise kernels: embedding,
 *                        activations, RoPE backward, attention delta, copies,
 *                        transposes (bytes)
 * Every product's flops are 2*M*N*K; its bytes are its operands read once
 * and its output written once. GEMM launches include their split-K reduce.
 * TTT_PROF_ALL times every launch, each under exactly one of the disjoint
 * classes 1, 3 and 5..11 (read back with ttt_prof_end_classes).
 * ttt_prof_sample(m, every), after ttt_prof_begin, times only every
 * `every`-th launch of the selected class (in launch order, starting with the
 * first; 1 = every launch): the sums then cover those launches, and their
 * ratio (work per time) estimates the class's rate at a fraction of the cost.
 * ttt_prof_end waits for the recorded events and returns the summed event
 * time (ms), the launch count and the summed flops (bytes for CE, NORM and
 * OTHER), then switches timing off. A timed dispatch still costs its stream a
 * few microseconds; sample, or leave timing off, for throughput.
 * Errors: TTT_EINVAL (NULL model, unknown class, every < 1), TTT_EHIP.
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
#define TTT_PROF_GEMM_SPAN 5
#define TTT_PROF_GEMM_CHUNK 6
#define TTT_PROF_GEMM_SGD 7
#define TTT_PROF_ATTN_DQ 8
#define TTT_PROF_ATTN_DKDV 9
#define TTT_PROF_NORM 10
#define TTT_PROF_OTHER 11
#define TTT_PROF_NCLASS 12
#define TTT_PROF_ALL 12

struct ttt_model;
int ttt_prof_begin(struct ttt_model* m, int32_t kernel_class);
int ttt_prof_sample(struct ttt_model* m, int32_t every);
int ttt_prof_end(struct ttt_model* m, double* total_ms, int64_t* launches, double* total_work);
/* Per-class totals (arrays of n entries, class index = array index; n <=
 * TTT_PROF_NCLASS): summed event time (ms), launches, flops and bytes of the
 * launches timed since ttt_prof_begin; then switches timing off. NULL arrays
 * are skipped. */
int ttt_prof_end_classes(struct ttt_model* m, int32_t n, double* ms, int64_t* launches, double* flops,
                         double* bytes);

#ifdef __cplusplus
}
#endif

#endif /* TTT_PROF_H */

/*
 * ttt_kernels.h - single-kernel entry points of the TTT-E2E library, used by
 * the kernel-level parity tests. Each runs one kernel of the hot path on
 * `stream` (async) with plain device pointers; dtype is 0 (fp32) or 1
 * (bf16) for the storage type of the non-fp32 operands. Return 0 or a
 * negative TTT_E* code (TTT_EINVAL for unsupported sizes / layouts,
 * TTT_EHIP for launch errors); ttt_last_error() explains.
 */
#ifndef TTT_KERNELS_H
#define TTT_KERNELS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Thread-local message of the last failed ttt_k_* call ("" if none). */
const char* ttt_k_last_error(void);

/* MFMA GEMM, C[m][n] (epi)= sum_k A[m*lda+k] B[n*ldb+k] (both operands
 * K-contiguous; K a multiple of 8 for bf16, 4 for fp32), batched over
 * `batch` with element strides sA, sB, sC (sC2, sR, sW for the epilogue).
 * epi 0: C = acc (fp32 if out_f32 else dtype); 1: C = R + acc (fp32);
 *     2: Wm -= lr * acc (fp32 master, ld ldw), then C[m][n] = cast(Wm) if C
 *        and C2[n*ldc2+m] = cast(Wm) if C2 (the inner SGD step, technical
 *        review section 5, Eq. 9, with both compute layouts refreshed).
 *        For bf16, sr_seed != 0 rounds the copies stochastically (unbiased,
 *        bits from a hash of (sr_seed, batch, m, n)); 0 rounds to nearest.
 *     3: SwiGLU MLP up-projection with the activation applied to the fp32
 *        accumulators: B's rows come in blocks of 64, 32 gate rows then the
 *        32 up rows of the same hidden units (N a multiple of 64), and
 *        C[m][u] = silu(gate_u) * up_u for hidden unit u < N/2 (C has N/2
 *        columns; fp32 if out_f32 else dtype).
 *     4: C = gelu(acc), exact erf form (fp32 if out_f32 else dtype).
 *     The activations are the block MLPs of the workloads' configurations.
 * ws: fp32 workspace of ws_elems elements for split-K partial sums (may be
 *     NULL; the kernel then runs without splitting K). */
int ttt_k_gemm(int32_t dtype, int32_t epi, int32_t out_f32, int32_t M, int32_t N, int32_t K, const void* A,
               int64_t lda, int64_t sA, const void* B, int64_t ldb, int64_t sB, void* C, int64_t ldc, int64_t sC,
               void* C2, int64_t ldc2, int64_t sC2, const float* R, int64_t ldr, int64_t sR, float* Wm, int64_t ldw,
               int64_t sW, float lr, uint32_t sr_seed, int32_t batch, float* ws, int64_t ws_elems, void* stream);

/* bf16 Q/K/V projection of an attention block with the rotary embedding
 * (RoPE: pairs (i, i + hd/2) rotated by angle pos * theta^(-2i/hd); the
 * positions are absolute, as the sliding-window attention of the technical
 * review's section 5 keys its cache by position) applied to the fp32
 * accumulators, and the split into q and the K/V ring caches.
 * A: [rows][K] bf16 (ld lda); row r = s*S + i is position p0 + i of
 * sequence s. Bp: [3*H*hd][K] bf16, the rows (output columns) of W_q, W_k,
 * W_v (each [K][H*hd] as y = x W) transposed, each head's hd rows permuted
 * in 32-row blocks into the order [0, nb/2, 1, nb/2 + 1, ...] with
 * nb = hd/32 (hd a multiple of 64). tab: device float2 [p0 + S][hd/2]
 * (cos, sin) of the angles, or NULL for no rotation. Outputs (bf16, each
 * rounded once after the rotation): q [rows][H*hd]; k and v of position p of
 * sequence s at kc / vc + s*cap*H*hd + (p % cap)*H*hd (cap a multiple of 64,
 * >= S). */
int ttt_k_qkv_rope(int32_t rows, int32_t S, int32_t H, int32_t hd, int32_t K, const void* A, int64_t lda,
                   const void* Bp, const void* tab, int64_t p0, void* q, void* kc, void* vc, int32_t cap,
                   void* stream);

/* Test hook: force the GEMM block tile (0 automatic, 1 = 256x256, 2 = 256x128,
 * 3 = 128x128, 4 = 256x256 with operands loaded straight into a two-stage LDS
 * ring (bf16, K a multiple of 64, not epi 2), 5 = the same with a four-stage
 * ring (K a multiple of 32), 6 / 7 = 128x128 direct-to-LDS with a two / three
 * stage ring (bf16, K a multiple of 64), 8 / 9 = 128x128 with a four-stage
 * ring of 64 / 32 deep K tiles; each splits K when the tile count is low and
 * a workspace is given; 4 and 5 fall back to 1, 6 to 9 to 3 where they do
 * not apply). cfg >> 8, when non-zero, forces the number of K splits (1 when
 * the workspace is too small or K has fewer tiles). Process-wide. */
void ttt_k_gemm_tile(int32_t cfg);

/* Test hook: mn = 1 makes ttt_k_gemm read both operands MN-major, element
 * (m, k) at A[k*lda + m] and (n, k) at B[k*ldb + n] (bf16, epi 0 or 2, M and
 * N multiples of 128, K of 64, no split; the layout the weight-gradient
 * products read their activations in). 0 restores K-contiguous operands.
 * Process-wide. */
void ttt_k_gemm_operands(int32_t mn);

/* Sliding-window attention forward over a ring cache (query p sees keys
 * p-window < j <= p; technical review section 2.1 Eq. 1 and section 5).
 * q, o: [B*M][H*hd] rows (row s*M+i = position pos0+i of sequence s);
 * kc, vc: [B][cap][H*hd], key position j at slot j % cap (cap multiple of 64);
 * lse: fp32 [B][H][M] natural-log sum of exp of the scaled scores.
 * nsplit (1..16) splits each query block's key range over workgroups; with
 * nsplit > 1, H <= 64 and ws is an fp32 workspace of nsplit*B*M*(H*hd + 2*H)
 * elements. Every slot of a 64-key tile that holds a visible key must hold
 * finite K and V values (the tile's other keys get weight exactly 0). */
int ttt_k_attn_fwd(int32_t dtype, const void* q, const void* kc, const void* vc, int32_t cap, void* o,
                   float* lse, int32_t B, int32_t M, int32_t H, int32_t hd, int64_t pos0, int32_t window,
                   float scale, int32_t nsplit, float* ws, void* stream);

/* ttt_k_attn_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and arguments without `ws`. The split partials go to a
 * fixed 64 MiB device array (16 Mi floats) that the library holds on every
 * device it runs on until the process ends; the call allocates and frees
 * nothing. nsplit * B * M * (H*hd + 2*H) must not exceed 16 Mi floats
 * (nsplit = 1 needs none), else TTT_EINVAL with the size in the message and
 * nothing launched. Every partial the merge reads is written by the same call,
 * so nothing needs clearing; calls that overlap on one device (other streams,
 * other threads) share the array and race. */
int ttt_k_attn_fwd_noalloc(int32_t dtype, const void* q, const void* kc, const void* vc, int32_t cap, void* o,
                           float* lse, int32_t B, int32_t M, int32_t H, int32_t hd, int64_t pos0, int32_t window,
                           float scale, int32_t nsplit, void* stream);

/* Backward of ttt_k_attn_fwd: dq (fp32, nsplit slices of [B*M][H*hd] whose
 * sum is the gradient; each query's window split as in the forward); dk, dv
 * (fp32 [B*M][H*hd]) for the keys at positions pos0..pos0+M-1 only (earlier
 * cached keys are constants). dout like q; delta = fp32 [B][H][M] row sums
 * of dout * o (see ttt_k_attn_delta). */
int ttt_k_attn_bwd(int32_t dtype, const void* q, const void* kc, const void* vc, int32_t cap, const float* lse,
                   const void* dout, const float* delta, float* dq, float* dk, float* dv, int32_t B, int32_t M,
                   int32_t H, int32_t hd, int64_t pos0, int32_t window, float scale, int32_t nsplit, void* stream);

/* Test hook: 0 runs bf16 head-dim-128 attention (forward, dQ, dK/dV) on the
 * register-staged kernels (those of the other head dims), 1 (default) on the
 * direct-to-LDS ones, with the forward of at most 8 queries per sequence on
 * the one-query streaming kernel; 2 as 1 but the forward always on the
 * direct-to-LDS tile kernel. Process-wide. */
void ttt_k_attn_fwd_kernel(int32_t dl);

/* The library's choice of key-range splits for M queries per sequence. */
int32_t ttt_k_attn_splits(int32_t M, int32_t H, int32_t B, int64_t keys_per_query);
int ttt_k_attn_delta(int32_t dtype, const void* o, const void* dout, int32_t B, int32_t M, int32_t H, int32_t hd,
                     float* delta, void* stream);

/* Fused softmax / cross entropy / logit gradient over fp32 logits [rows][V]
 * (loss l = -log softmax(z)[label], natural log: b-lab.team summary, loss
 * function; technical review section 2.2). ids2: device int32 [rows][2] with
 * ids2[r][1] the label of row r.
 * labelled != 0: losses[r] = lse - z[label] and, if dz != NULL,
 *   dz[r] = (softmax - onehot) * scale in dtype.
 * labelled == 0: lse[r], mx[r] and argmax[r] (lowest index among maxima). */
int ttt_k_ce(int32_t dtype, const float* logits, int32_t rows, int32_t V, const int32_t* ids2, int32_t labelled,
             float* losses, void* dz, float scale, float* lse, float* mx, int32_t* argmax, void* stream);

/* RMSNorm y = x * (mean(x^2)+eps)^(-1/2) * g (x fp32 [rows][d], y dtype) and
 * its backward dres (+)= r*g*dn - x*r^3*mean(x*g*dn) (fp32). */
int ttt_k_rmsnorm_fwd(int32_t dtype, const float* x, int32_t rows, int32_t d, const void* g, float eps, void* y,
                      float* rstd, void* stream);
int ttt_k_rmsnorm_bwd(int32_t dtype, const float* x, const float* rstd, const void* g, const float* dn, int32_t rows,
                      int32_t d, float* dres, int32_t accumulate, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TTT_KERNELS_H */

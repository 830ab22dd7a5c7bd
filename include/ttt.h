/*
 * ttt.h - C ABI of the MI355X (gfx950) TTT-E2E prefill / decode library.
 *
 * The method ("End-to-End Test-Time Training for Long Context"): a Transformer
 * with causal sliding-window attention (window k >= b) reads its context in
 * mini-batches ("chunks") of b positions. For each chunk it scores every
 * position with the current fast weights W, then takes one SGD step
 *     W_i = W_{i-1} - eta * (1/b) * sum over the chunk of grad l_p(W_{i-1})
 * where l_p is the next-token cross entropy (natural log). Only the MLPs of
 * the last quarter of the blocks are fast weights; embeddings, norms,
 * attention, the LM head and a second, static MLP branch in each of those
 * blocks stay frozen but are differentiated through.
 * Sources: b-lab.team summary, "Test-Time Training (Inner Loop)" and
 * "Implementation Details for TTT"; technical review "TTT-E2E: Learning a Long
 * Context into Weights", section 5 (Eq. 9), section 6, section 7 (Algorithms
 * 1 and 3).
 *
 * Conventions for every call:
 *   - Device pointers are HIP device addresses on the current device; host
 *     pointers are ordinary process memory. Which is which is stated per
 *     argument.
 *   - `stream` is a hipStream_t cast to void* (NULL = the null stream).
 *     Calls marked "async" only enqueue work on `stream`; the caller keeps its
 *     buffers alive until that work completes.
 *   - Return 0 on success or a negative TTT_E* code. Arguments are validated
 *     before any work is enqueued, so a call that fails validation leaves the
 *     model unchanged. After a HIP runtime error the model is "poisoned": all
 *     calls except ttt_reset / ttt_model_destroy / ttt_last_error return
 *     TTT_ESTATE until ttt_reset succeeds. ttt_last_error() returns a
 *     thread-local message for the last failure.
 *   - Non-finite values: the cross-entropy kernel raises a device status flag
 *     when a logit row's log-sum-exp or a loss is not finite (the fast
 *     weights or the initial weights then hold non-finite values). The next
 *     ttt_prefill / ttt_decode reads the flag, poisons the model and returns
 *     TTT_ESTATE; the losses of the call that produced them are already in
 *     the caller's buffer.
 *   - Matrices passed in are row-major [in][out] (y = x @ W).
 */
#ifndef TTT_H
#define TTT_H

#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TTT_OK 0
#define TTT_EINVAL (-1)  /* invalid argument or configuration */
#define TTT_ENOMEM (-2)  /* device allocation failed or over max_device_bytes */
#define TTT_EHIP (-3)    /* HIP runtime error (model is poisoned) */
#define TTT_ESTATE (-4)  /* call not valid in this state (e.g. decode before prefill) */

enum ttt_dtype { TTT_FP32 = 0, TTT_BF16 = 1 };
enum ttt_mlp { TTT_GELU = 0, TTT_SWIGLU = 1 };
enum ttt_mat { TTT_UP = 0, TTT_GATE = 1, TTT_DOWN = 2 };

/* Model shape and inner-loop hyper-parameters.
 * n_ttt_blocks tail blocks (the last ones) carry fast MLP weights of hidden
 * size ttt_hidden plus a static branch of hidden size static_hidden; the other
 * blocks have one frozen MLP of hidden size mlp_hidden. Attention is
 * multi-head with n_heads * head_dim columns per projection. RMSNorm with
 * norm_eps everywhere (pre-attention, pre-MLP, final). RoPE (if rope != 0) on
 * pairs (i, i + head_dim/2) at absolute positions, base rope_theta.
 * window = k, mini_batch = b (k >= b is required), lr = eta.
 * batch = number of independent sequences, each with its own fast weights,
 * attention cache and position counter. max_positions bounds the stream
 * length (ids) per sequence. prefill_span bounds how many positions the
 * frozen lower blocks process per pass (0 = library default: four
 * mini-batches, at least 2048).
 * max_device_bytes (0 = unlimited) caps the library's allocation.
 * forward_only != 0 turns the inner loop off: every position is scored at
 * the initial weights and no backward or SGD step runs (the static model;
 * with window >= the stream length it is the full-attention Transformer whose
 * prefill time the technical review compares TTT-E2E with: its Figure 1 and
 * section 11).
 * mh_heads > 1 selects the "TTT-E2E all layers MH" variant (b-lab.team
 * summary, "Alternative Derivation", step 4; technical review, section 8 and
 * its Table 1): the fast MLP of each tail block is split into mh_heads
 * independent heads, head i mapping columns [i*dh, (i+1)*dh) of the
 * normalised state (dh = d_model / mh_heads) through its own MLP of hidden
 * ttt_hidden / mh_heads back to the same columns; with n_ttt_blocks =
 * n_blocks every block has one, beside its static MLP of hidden
 * static_hidden. 0 or 1: the dense fast MLP of the final design. */
typedef struct ttt_config {
  int32_t vocab, d_model, n_blocks, n_heads, head_dim;
  int32_t mlp_kind;          /* enum ttt_mlp */
  int32_t mlp_hidden, n_ttt_blocks, ttt_hidden, static_hidden;
  int32_t rope;
  float rope_theta, norm_eps;
  int32_t window, mini_batch;
  float lr;
  int32_t dtype;             /* enum ttt_dtype: storage and GEMM operand type */
  int32_t batch;
  int64_t max_positions;
  int32_t prefill_span;
  int64_t max_device_bytes;
  int32_t forward_only;
  int32_t mh_heads;
} ttt_config;

/* Initial weights, all device pointers in cfg.dtype, row-major [in][out].
 * Per-block arrays are HOST arrays of n_blocks device pointers.
 *   embed [V][d], final_norm [d], lm_head [d][V]
 *   attn_norm[l], mlp_norm[l]: [d]
 *   wq[l], wk[l], wv[l]: [d][H*hd];  wo[l]: [H*hd][d]
 *   w_up[l], w_gate[l] (SwiGLU only, else NULL): [d][h];  w_down[l]: [h][d]
 *     with h = ttt_hidden for tail blocks (the fast, trainable branch) and
 *     mlp_hidden otherwise; with mh_heads = nh > 1 the tail blocks' fast
 *     matrices are per head: w_up[l], w_gate[l] [nh][d/nh][h/nh], w_down[l]
 *     [nh][h/nh][d/nh]
 *   s_up[l], s_gate[l], s_down[l]: static branch of tail blocks ([d][hs],
 *     [d][hs], [hs][d]); NULL (or ignored) for other blocks. */
typedef struct ttt_weights {
  const void* embed;
  const void* final_norm;
  const void* lm_head;
  const void* const* attn_norm;
  const void* const* wq;
  const void* const* wk;
  const void* const* wv;
  const void* const* wo;
  const void* const* mlp_norm;
  const void* const* w_up;
  const void* const* w_gate;
  const void* const* w_down;
  const void* const* s_up;
  const void* const* s_gate;
  const void* const* s_down;
} ttt_weights;

typedef struct ttt_model ttt_model;

/* Create a model: validates cfg, allocates library-owned storage (frozen
 * weights, per-sequence fast weights - an fp32 master plus the cfg.dtype copy
 * the GEMMs read - attention caches and workspace) and copies `init` into it
 * (the copy runs on `stream` and is complete when the call returns). The
 * caller's weight buffers may be freed afterwards. Every sequence starts from
 * a fresh copy of the initial fast weights (review, Algorithm 1 step 1).
 * Errors: TTT_EINVAL (k < b, d_model or n_heads or head_dim < 1, n_ttt_blocks
 * not in [1, n_blocks], odd head_dim with rope, mini_batch not a multiple of
 * 8 (bf16) or 4 (fp32) - the weight-gradient products contract over the b
 * positions of a chunk -, NULL pointers), TTT_ENOMEM (a device allocation
 * failed, or the model would need more than max_device_bytes), TTT_EHIP.
 * On error *out is NULL and nothing stays allocated. */
int ttt_model_create(const ttt_config* cfg, const ttt_weights* init, void* stream,
                     ttt_model** out);

/* Create a session of `base`: another model that shares base's frozen
 * weights and initial fast weights (by reference, not copied) and has its own
 * sequences, fast weights, attention caches, positions and workspace - the
 * per-session terms of the serving budget of the technical review, section
 * 11.2, Eq. 13, M(S) = M_shared + S (M_fast + M_local cache + M_update work).
 * batch, max_positions, prefill_span and max_device_bytes (which caps only
 * what this call allocates) are the session's own; every other configuration
 * field is base's. Sessions are independent: each can be reset, fed and
 * destroyed on its own, and each starts from a fresh copy of the initial
 * fast weights (Algorithm 1 step 1). The shared part is freed with the last
 * model that uses it, so base may be destroyed before its sessions.
 * Synchronous on `stream`. Errors: TTT_EINVAL (base NULL, invalid sizes),
 * TTT_ENOMEM, TTT_EHIP; on error *out is NULL. */
int ttt_model_create_session(const ttt_model* base, int32_t batch, int64_t max_positions, int32_t prefill_span,
                             int64_t max_device_bytes, void* stream, ttt_model** out);

/* Prefill (review, section 7, Algorithm 1). Async.
 * tokens: device int32 [batch][n], the next n ids of every sequence.
 * losses: device float [batch][n] or NULL. Entry [s][i] receives the loss of
 *   predicting new id i of sequence s, i.e. of position (n_before + i - 1)
 *   where n_before is the stream length before this call; on the first call
 *   of a stream entry 0 has no predecessor and is set to NaN.
 * Every position is scored with the fast weights current for its chunk
 * (before the update that chunk produces). Whenever chunk c = positions
 * [c*b, (c+1)*b) has all of its labels (ids up to (c+1)*b), the library runs
 * the chunk's backward and SGD step. Positions of an incomplete chunk are
 * scored at the current W and wait for the rest of their chunk.
 * Validation reads the n new ids of every sequence back to the host, so the
 * call waits for `stream` to reach it (earlier work on `stream`, such as the
 * kernel that wrote `tokens`, completes first); everything after the check is
 * enqueued asynchronously.
 * Errors: TTT_EINVAL (n < 1, stream would exceed max_positions, an id outside
 * [0, vocab): nothing is enqueued and the model is unchanged), TTT_ESTATE
 * (poisoned, or an earlier call produced non-finite logits), TTT_EHIP. */
int ttt_prefill(ttt_model* m, const int32_t* tokens, int64_t n, float* losses, void* stream);

/* Greedy decode with periodic adaptation (review, section 7, Algorithm 3;
 * summary, "Decoding Multiple Tokens"). Async.
 * Generates n_new ids per sequence: each is the argmax (lowest id on ties)
 * of the logits of the last position, computed with the current W. After the
 * id is appended, if it completes a chunk of b labelled positions, that
 * chunk's SGD step runs before the next position is computed.
 * tokens_out: device int32 [batch][n_new]. losses: device float
 * [batch][n_new] or NULL; entry i = -log p(chosen id i).
 * Waits for `stream` to reach the call (to read the non-finite status flag);
 * the generation itself is enqueued asynchronously. A row whose logits have
 * no finite maximum yields id 0 and raises the status flag.
 * Errors: TTT_ESTATE (no prefill yet, poisoned, or an earlier call produced
 * non-finite logits), TTT_EINVAL (n_new < 1, exceeds max_positions),
 * TTT_EHIP. */
int ttt_decode(ttt_model* m, int64_t n_new, int32_t* tokens_out, float* losses, void* stream);

/* Copy the current fp32 fast weights of one trainable matrix of one sequence
 * into dst (device float, row-major [in][out]: UP/GATE [d][ttt_hidden],
 * DOWN [ttt_hidden][d]; with mh_heads = nh > 1, [nh][d/nh][ttt_hidden/nh] and
 * [nh][ttt_hidden/nh][d/nh]). Async on `stream`. Reflects every completed chunk:
 * the adapted weights W that the review's section 7, Algorithm 1 returns
 * after its last update (the summary's W_{T/b}, "Test-Time Training (Inner
 * Loop)"); an incomplete chunk has not changed them.
 * Errors: TTT_EINVAL (seq out of range, block not a tail block, GATE without
 * SwiGLU, dst NULL). */
int ttt_get_weights(const ttt_model* m, int32_t seq, int32_t block, int32_t mat, float* dst,
                    void* stream);

/* Reset every sequence: fast weights <- initial weights, empty caches and
 * streams (review, Algorithm 2 step 7: per-sequence state is discarded).
 * Synchronous on `stream`. Clears the poisoned flag if it succeeds. */
int ttt_reset(ttt_model* m, void* stream);

/* Free everything the model owns (after synchronising the device). NULL ok. */
void ttt_model_destroy(ttt_model* m);

/* Thread-local description of the last error ("" if none). */
const char* ttt_last_error(void);

/* Number of positions already in sequence streams (ids appended). */
int64_t ttt_stream_length(const ttt_model* m);

/* Device memory in bytes the model uses: its own allocations plus the shared
 * part (frozen weights and initial fast weights), which sessions of one base
 * model hold in common. */
int64_t ttt_device_bytes(const ttt_model* m);

/* The same bytes by part, the terms of the review's Eq. 13 (section 11.2):
 * out[0] the shared part (frozen weights and the initial fast weights; the
 * same memory for every session of one base), out[1] the fast weights of the
 * model's sequences (compute copies in both layouts and, for bf16, the fp32
 * master), out[2] the local attention caches and stream state (K/V rings,
 * ids, the residual hand-off of the frozen prefix, the RoPE table), out[3]
 * the workspace of the forward and update passes. Errors: TTT_EINVAL. */
int ttt_device_bytes_by_part(const ttt_model* m, int64_t* out);

#ifdef __cplusplus
}
#endif

#endif /* TTT_H */

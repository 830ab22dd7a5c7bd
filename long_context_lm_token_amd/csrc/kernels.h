// Internal launchers of the gfx950 kernels (host side). All pointers are
// device pointers; `dt` is 0 for fp32 storage, 1 for bf16 storage.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// EPI_SWIGLU: B's rows (output columns) come in blocks of 32 gate / 32 up
// columns; C[m][u] = silu(gate_u) * up_u for hidden unit u, C has N/2 columns.
// EPI_GELU: C = gelu(acc).
// EPI_ROPE: the attention's Q/K/V projection with the rotary embedding and
// the split applied to the fp32 accumulators (GemmArgs::rope). B's rows (the
// output columns) are the q, k, v parts of each head, each permuted in
// 32-row blocks so that every 64-column block holds dims 32s.. 32s+31 and
// then their rotation partners hd/2 + 32s..: with nb = hd/32 blocks, block
// order [0, nb/2, 1, nb/2 + 1, ...] (hd a multiple of 64). Outputs in the
// compute dtype: q [rows][H*hd], k and v into ring caches at slot pos % cap.
// Never split over K.
enum { EPI_STORE = 0, EPI_ADD = 1, EPI_SGD = 2, EPI_SWIGLU = 3, EPI_GELU = 4, EPI_ROPE = 5 };

// outputs of EPI_ROPE: row s*S + i of the product is position p0 + i of
// sequence s; tab: [pos][hd/2] (cos, sin), or null for no rotation
struct RopeOut {
  void* q;
  void* kc;
  void* vc;
  const float2* tab;
  int64_t ldq, seq_stride, p0;
  int cap, S, H, hd;
};

// C[m][n] (epilogue)= sum_k A[m*lda + k] * B[n*ldb + k], batched over z.
struct GemmArgs {
  const void* A;
  const void* B;
  void* C;
  int64_t lda, ldb, ldc;
  int64_t sA, sB, sC;  // batch strides in elements
  int M, N, K;
  const float* R;      // EPI_ADD: C = R + acc (R may alias C)
  int64_t ldr, sR;
  float* Wm;           // EPI_SGD: Wm -= lr * acc; C[m][n] and C2[n][m] (if non-null) = cast(Wm)
  int64_t ldw, sW;
  void* C2;
  int64_t ldc2, sC2;
  float lr;
  // EPI_SGD with a bf16 compute copy: if nonzero, the copies are rounded
  // stochastically from the fp32 master with a counter-based hash of
  // (sr_seed, batch, row, col); 0 = round to nearest even
  uint32_t sr_seed;
  RopeOut rope;  // EPI_ROPE
  // bf16 only: A and B stored MN-major, element (m, k) at A[k * lda + m] and
  // (n, k) at B[k * ldb + n] (M, N multiples of 128, K of 64; no split)
  int mn;
  // skinny products only (bf16, at most GEMV_MAX_ROWS rows of A, not SGD):
  // if nx is set, A is not read; row m of batch z is the RMSNorm of the fp32
  // row nx[z * snx + m * ldnx ..] with gain ng (compute dtype) rounded to the
  // compute dtype, as rmsnorm_fwd_launch writes it. Other kernels reject it.
  const float* nx;
  int64_t ldnx, snx;
  const void* ng;
  float neps;
  // EPI_STORE / EPI_ADD with fp32 output: if set (a host pointer), a product
  // split over K leaves its partial sums in the workspace for the consumer to
  // add, in split order (then R, for EPI_ADD): split s of output row r (rows
  // of all batches counted together) at ws + (s * batch * M + r) * N. The
  // number of splits is written here (1: no split, C holds the result).
  int* split_out;
};
constexpr int GEMV_MAX_ROWS = 8;  // products with at most this many rows of A stream B once

// Timing of launches. While `start` and `stop` are set (the runtime sets them
// around the launches of a timed class), every kernel is launched with them
// attached to its own dispatch (hipExtLaunchKernelGGL): the first kernel of
// the group records `start` when it begins, each kernel records `stop` when
// it ends (the last one wins), so the pair spans the group with no marker
// packets between kernels. Unset (null), a launch is a plain launch. Per host
// thread; defined in runtime.cpp.
struct LaunchEvents {
  hipEvent_t start;
  hipEvent_t stop;
};
LaunchEvents& launch_events();

// ws: fp32 split-K workspace of ws_elems elements (may be null: no split)
hipError_t gemm_launch(const GemmArgs& p, int dt, int epi, bool out_f32, int batch, float* ws,
                       int64_t ws_elems, hipStream_t st);
void gemm_force_tile(int cfg);  // test hook (0 = automatic choice)

// Attention over a ring cache. Queries: rows [s*M + i] of q (row stride ldq,
// head h at column h*hd), position pos0 + i. Keys/values of sequence s at
// absolute position j live in kc/vc + s*seq_stride + (j % cap)*ldk + h*hd.
struct AttnArgs {
  const void* q; int64_t ldq;
  const void* kc; const void* vc; int64_t ldk; int64_t seq_stride; int cap;
  void* o; int64_t ldo;          // output rows like q
  float* lse;                    // [B][H][M] natural-log sum exp of scaled scores
  int M, H, hd, B;
  int64_t pos0;
  int window;
  float scale;
  // backward
  const void* dout; int64_t lddo;   // dO rows like q
  const float* delta;               // [B][H][M] rowsum(dO * O)
  float* dq; int64_t lddq;          // fp32 rows like q, nsplit slices of B*M rows (summed by the caller)
  float* dk; float* dv; int64_t lddk;  // fp32 [B*M][H*hd] for keys at pos0..pos0+M-1
  // key-range splits (forward and dq): partial outputs of the forward
  int nsplit;
  float* part_o;                    // [nsplit][B*M][ldo]
  float* part_m; float* part_l;     // [nsplit][B][H][M]
  // backward: which kernels attn_bwd_launch runs (0 both, 1 dQ only, 2 dK/dV only)
  int parts;
};

hipError_t attn_fwd_launch(const AttnArgs& a, int dt, hipStream_t st);
hipError_t attn_bwd_launch(const AttnArgs& a, int dt, hipStream_t st);
void attn_force_fwd_kernel(int dl);  // test hook: 0 register-staged, 1 default, 2 no one-query forward (bf16 hd 128)
// number of key-range splits that keeps the CUs busy for M queries per sequence
int attn_splits(int M, int H, int B, int64_t keys_per_query);

// elementwise / row kernels
hipError_t embed_launch(const int32_t* ids, int64_t ids_seq_stride, int64_t p0, int S, int B,
                        const void* E, int d, int vocab, float* x, int dt, hipStream_t st);
// x_splits > 1: x holds that many partial sums of an EPI_ADD product's output
// (split s at x + s * x_ss, x_ss >= rows * d; GemmArgs::split_out) and x_res
// its residual; the row, sum of the partials in order plus x_res, is also
// stored to x_out (all rows of stride d)
hipError_t rmsnorm_fwd_launch(const float* x, int rows, int d, const void* g, float eps, void* y,
                              float* rstd, int dt, hipStream_t st, int x_splits = 1, int64_t x_ss = 0,
                              const float* x_res = nullptr, float* x_out = nullptr);
// dn_splits > 1: dn holds that many partial sums of the gradient (split s at
// dn + s * dn_ss, dn_ss >= rows * d), added in order (GemmArgs::split_out)
hipError_t rmsnorm_bwd_launch(const float* x, const float* rstd, const void* g, const float* dn,
                              int rows, int d, float* dres, void* dres_c, bool accumulate, int dt,
                              hipStream_t st, int dn_splits = 1, int64_t dn_ss = 0);
hipError_t rope_split_launch(const float* qkv, int rows, int S, int H, int hd, int64_t p0,
                             const float2* rope_tab, void* q, void* kc, void* vc, int cap,
                             int64_t seq_stride, int dt, hipStream_t st);
// dq holds nsplit slices of rows x H*hd (summed here)
hipError_t rope_bwd_pack_launch(const float* dq, int nsplit, const float* dk, const float* dv, int rows, int S,
                                int H, int hd, int64_t p0, const float2* rope_tab, void* dqkv,
                                int dt, hipStream_t st);
hipError_t act_fwd_launch(const float* z, int rows, int h, int64_t ldz, int glu, void* a, int64_t lda,
                          int dt, hipStream_t st);
hipError_t act_bwd_launch(const float* z, const float* da, int rows, int hcols, int64_t ldz,
                          int64_t ldda, int64_t up_off, int glu, void* dz, int64_t lddz, int dt,
                          hipStream_t st);
hipError_t attn_delta_launch(const void* o, const void* dout, int rows, int H, int hd, int64_t ld,
                             int S, float* delta, int dt, hipStream_t st);

// Cross entropy over rows of fp32 logits. Row r = s*S + i is position p0+i of
// sequence s; its label is ids[s][p0+i+1] when p0+i+1 < n_ids.
struct CEArgs {
  const float* logits; int rows, S, V;
  const int32_t* ids; int64_t ids_seq_stride; int64_t p0, n_ids;
  void* dz; float dz_scale;            // NULL: no gradient
  float* losses; int64_t loss_base, loss_ld, loss_n;  // losses[s*loss_ld + (p - loss_base)]
  float* last_lse; float* last_max; int32_t* last_arg;  // per sequence, row of position n_ids-1
  int32_t* status;                     // if set: *status = 1 when a row's lse or loss is not finite
};
hipError_t ce_launch(const CEArgs& a, int dt, hipStream_t st);

// dst[z][c][r] = src[z][r][c] for r < rows, c < cols (strides in elements)
hipError_t transpose_launch(const void* src, int rows, int cols, int64_t lds, int src_dt, void* dst,
                            int64_t ldd, int dst_dt, hipStream_t st, int batch = 1, int64_t s_src = 0,
                            int64_t s_dst = 0);
hipError_t copy_rows_f32_launch(const float* src, int64_t src_seq_stride, float* dst,
                                int64_t dst_seq_stride, int S, int d, int B, hipStream_t st);
hipError_t fill_f32_launch(float* p, int64_t n, float v, hipStream_t st);
// Appends the greedy ids next[s] at position pos; an id outside [0, vocab)
// (the argmax of a row with no finite maximum) is written as 0 and sets
// *status |= 2.
hipError_t decode_emit_launch(const int32_t* next, const float* lse, const float* mx, int B, int vocab,
                              int32_t* ids, int64_t ids_seq_stride, int64_t pos, int32_t* tokens_out,
                              int64_t out_ld, int64_t i, float* losses, int32_t* status, hipStream_t st);

// Host runtime of the TTT-E2E library: model state, memory layout, the
// prefill chunk scheduler and decode loop, weight upload and read-back.
//
// The inner loop (technical review "TTT-E2E: Learning a Long Context into
// Weights", section 7, Algorithm 1; section 5, Eq. 9):
//   for each chunk of b positions, in order: score every position with the
//   current fast weights W (causal sliding-window attention), record the
//   losses, differentiate their mean with respect to W, apply
//   W <- W - eta * grad, keep only the K/V rows the window still needs.
//
// Layout (all device memory owned by the model):
//   * frozen blocks 0 .. t0-1 and the attention of block t0 do not depend on
//     W, so their forward runs over long spans of new positions at once
//     ("span pass": GEMMs with M = batch * span); it ends by storing the
//     residual after block t0's attention for every position (ystage). The
//     span passes of a prefill run on their own stream, at most two spans
//     ahead of the chunk loop, whose small chunk-sized kernels leave compute
//     units free for them;
//   * the tail (MLP of block t0, blocks t0+1 .. L-1, final norm, head, CE)
//     runs per chunk: forward at W_c, backward through the tail, and the SGD
//     step fused into each trainable matrix's weight-gradient GEMM;
//   * every block keeps a ring cache of K/V rows indexed by absolute position
//     modulo its capacity (>= window + rows written per pass);
//   * weights are stored transposed, [out][in], so the forward GEMM reads
//     both operands K-contiguous; tail MLPs are stored per sequence with the
//     trainable and static branches concatenated along the hidden dim (one
//     GEMM per projection), the trainable rows/columns first; an fp32 master
//     of the trainable part is kept for bf16 models.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <memory>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/ttt.h"
#include "../../include/ttt_prof.h"
#include "kernels.h"

LaunchEvents& launch_events() {
  static thread_local LaunchEvents le{nullptr, nullptr};
  return le;
}

namespace {

thread_local std::string g_err;

// Events that only order work between the library's streams on one device:
// no timing, and a device-scope release instead of a system-scope fence (the
// waiting kernels run on the same device; nothing on the host reads the data
// they publish), which spares a cache writeback per record.
constexpr unsigned kOrderEventFlags = hipEventDisableTiming | hipEventDisableSystemFence;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

struct Prof {
  int cls = -1;  // kernel class being timed (TTT_PROF_ALL: every launch), -1 = off
  int every = 1;     // time every `every`-th launch of the class
  int64_t seen = 0;  // launches of the class so far
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<int> cls_of;     // per timed launch: its (disjoint) class
  std::vector<double> flops;   // per timed launch: algorithmic flops
  std::vector<double> bytes;   // per timed launch: algorithmic HBM bytes
};

// Is a launch of disjoint class `cls` (also a member of `alias`, or -1) timed?
bool prof_wants(const Prof& p, int cls, int alias) {
  if (p.cls < 0) return false;
  if (p.cls == TTT_PROF_ALL || p.cls == cls || p.cls == alias) return true;
  if (p.cls == TTT_PROF_GEMM)
    return cls == TTT_PROF_GEMM_SPAN || cls == TTT_PROF_GEMM_CHUNK || cls == TTT_PROF_GEMM_SGD;
  if (p.cls == TTT_PROF_ATTN_BWD) return cls == TTT_PROF_ATTN_DQ || cls == TTT_PROF_ATTN_DKDV;
  return false;
}

// Device memory that several models (sessions) may share: the frozen weights
// and the initial fast weights. Freed with the last model that uses it.
struct Shared {
  std::vector<void*> allocs;
  int64_t bytes = 0;
  ~Shared() {
    for (void* p : allocs) (void)hipFree(p);
  }
};

// parts of a model's device memory (the terms of the serving budget M(S))
enum { PART_SHARED = 0, PART_FAST = 1, PART_CACHE = 2, PART_WORK = 3, NPART = 4 };

}  // namespace

struct ttt_model {
  ttt_config cfg;
  int dt;             // 0 fp32, 1 bf16
  size_t es;          // element size of the compute dtype
  int L, t0, nt, H, hd, HD, d, V, h, ht, hs, hf, mg;  // mg = 2 for SwiGLU
  int64_t maxpos;
  int span;
  int cap_s, cap_t;
  float scale;

  // frozen weights
  void* embed = nullptr;
  void* gfin = nullptr;
  void* wout_t = nullptr;  // [V][d]
  void* wout_b = nullptr;  // [d][V] (input-grad layout)
  std::vector<void*> g_attn, g_mlp, wqkv_t, wo_t, wgu_t, wd_t;  // wgu_t/wd_t: frozen blocks only
  std::vector<void*> wqkv_b, wo_b;  // tail blocks t0+1..L-1: [d][3HD], [HD][d] (input-grad layout)

  // fast weights, per tail block j: [B][...] compute copies in both layouts
  // (forward [out][in], input-grad [in][out]) and fp32 masters
  std::vector<void*> f_gu, f_d;      // [B][mg*hf][d], [B][d][hf]
  std::vector<void*> fb_gu, fb_d;    // [B][d][mg*hf], [B][hf][d]
  std::vector<float*> m_gu, m_d;     // [B][mg*ht][d], [B][d][ht] (bf16 models only)
  std::vector<void*> i_gu, i_d, ib_gu, ib_d;  // initial copies (one sequence)
  std::vector<float*> im_gu, im_d;
  // multi-head fast MLPs (mh_heads > 1; the dense fast part above is then
  // empty, ht = 0): per tail block, nhm heads of width dhm and hidden hhm,
  // [B][mg][nhm][hhm][dhm] (gate/up, forward layout), [B][nhm][dhm][hhm]
  // (down, forward layout), the input-grad layouts [B][mg][nhm][dhm][hhm] and
  // [B][nhm][hhm][dhm], fp32 masters (bf16) in the forward layouts, initial copies
  bool mh = false;
  int nhm = 0, dhm = 0, hhm = 0, htm = 0;
  std::vector<void*> f_mg, f_md, fb_mg, fb_md, i_mg, i_md, ib_mg, ib_md;
  std::vector<float*> m_mg, m_md, im_mg, im_md;
  std::vector<float*> tz_m;      // fp32 pre-activations [B*b][mg*htm] per tail block
  std::vector<void*> ta_m;       // activations [B*b][htm] per tail block
  float* dA_m = nullptr;         // [B*b][htm]
  void* dz_m = nullptr;          // [B*b][mg*htm]
  void *T_dres = nullptr, *T_am = nullptr, *T_dzm = nullptr, *T_n = nullptr;  // token-contiguous copies

  // caches and stream state
  std::vector<void*> kc, vc;
  int32_t* ids = nullptr;     // [B][maxpos]
  float* ystage = nullptr;    // [B][maxpos][d]
  float2* rope = nullptr;     // [maxpos][hd/2]
  int64_t n_ids = 0;
  int64_t chunk = 0;
  float *last_lse = nullptr, *last_max = nullptr;
  int32_t* last_arg = nullptr;
  // device status word: non-zero once a logit row was non-finite (CE) or a
  // greedy id was not a valid id; read at the start of the next call
  int32_t* status = nullptr;

  // span-pass workspace (rows = B * span)
  float *sX = nullptr, *sR = nullptr, *sL = nullptr;
  void *sU = nullptr, *sQ = nullptr, *sO = nullptr, *sA = nullptr;
  float* sQKV = nullptr;
  // bf16 with hd % 64 == 0: the QKV projection takes the rotary embedding and
  // the split into q / the K, V caches in its epilogue (EPI_ROPE); wqkv_t's
  // rows are then permuted in 32-row blocks (see EPI_ROPE)
  bool qkv_rope = false;

  // tail workspace (rows = B * b), per tail block where saved for the backward
  std::vector<float*> tx, ty, tr1, tr2, tlse;
  std::vector<void*> tn, tq, to, ta;
  std::vector<float*> tz;  // fp32 pre-activations of the tail MLPs (kept for the backward)
  float *txL = nullptr, *trf = nullptr, *tlog = nullptr;
  void *tf = nullptr, *tdz = nullptr, *tU = nullptr;
  float* tQKV = nullptr;
  float *dres = nullptr, *dn = nullptr, *dA = nullptr, *delta = nullptr, *dq = nullptr, *dk = nullptr,
        *dv = nullptr;
  void *dres_c = nullptr, *dO = nullptr, *dqkv = nullptr;
  // per tail block: the bf16 gradient at its MLP output and the activation
  // gradient dZ, which the side stream's weight-gradient products read while
  // the chunk loop moves on to the blocks below
  std::vector<void*> dres_b, dZ_b;
  // the weight-gradient products read their operands MN-major (bf16 with
  // d and the trainable width multiples of 128, b of 64); otherwise from the
  // token-contiguous copies below
  bool mn_dw = false;
  // token-contiguous operands of the weight-gradient GEMMs, per tail block: [B][cols][b]
  std::vector<void*> Tdres, Ta, Tdz, Tn;  // token-contiguous copies (when !mn_dw)
  // the weight-gradient + SGD GEMMs run on a second stream (default priority),
  // ordered after the input-gradient GEMMs that read W_c; joined per chunk
  hipStream_t side = nullptr;
  std::vector<hipEvent_t> ev;  // pool of ordering events
  // the frozen prefix of a prefill runs on its own stream (default priority),
  // overlapping the chunk loop: one event per span, one for the id upload
  hipStream_t pre = nullptr;
  std::vector<hipEvent_t> span_ev, reach_ev;  // span done (prefix) / span reached (chunk loop)
  hipEvent_t ev_ids = nullptr;
  float* ws = nullptr;  // split-K partials
  int64_t ws_elems = 0;
  // key-range splits of the chunk attention: forward partials (dq slices use dq)
  static constexpr int kMaxSplit = 16;
  float *part_o = nullptr, *part_m = nullptr, *part_l = nullptr;
  // the same for span passes of at most one chunk of rows (decode, the last
  // rows of a prefill): their own buffers, as span passes run on the prefix
  // stream beside the chunk loop
  float *spart_o = nullptr, *spart_m = nullptr, *spart_l = nullptr;

  bool poisoned = false;
  int64_t bytes = 0;                // allocated by this model's create call (shared part included if it made it)
  int64_t part_bytes[NPART] = {0, 0, 0, 0};
  std::vector<void*> allocs;        // this model's own allocations
  std::shared_ptr<Shared> shared;   // frozen + initial fast weights (possibly another model's)
  Prof prof;
};

namespace {

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// ---------- allocation ----------
// Allocations are charged to the part set in `part`; shared-part allocations
// belong to m->shared, the others to the model.
struct Alloc {
  ttt_model* m;
  int part = PART_WORK;
  bool ok = true;
  std::string why;
  void* get(int64_t bytes) {
    if (!ok) return nullptr;
    bytes = round_up(std::max<int64_t>(bytes, 256), 256);
    if (m->cfg.max_device_bytes > 0 && m->bytes + bytes > m->cfg.max_device_bytes) {
      ok = false;
      why = "allocation exceeds max_device_bytes";
      return nullptr;
    }
    void* p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess) {
      (void)hipGetLastError();
      ok = false;
      why = "hipMalloc failed";
      return nullptr;
    }
    if (part == PART_SHARED) {
      m->shared->allocs.push_back(p);
      m->shared->bytes += bytes;
    } else {
      m->allocs.push_back(p);
    }
    m->bytes += bytes;
    m->part_bytes[part] += bytes;
    return p;
  }
  float* f32(int64_t n) { return static_cast<float*>(get(n * 4)); }
  void* el(int64_t n) { return get(n * (int64_t)m->es); }
};

// ---------- timing hooks (HIP events on the launches of selected classes) ----------
// The events ride on the kernels' own dispatches (launch_events(), kernels.h):
// events recorded between the kernels of a stream would each add a marker
// packet, and the stream would idle for it between the kernels.
hipEvent_t prof_begin(ttt_model* m, hipStream_t) {
  Prof& p = m->prof;
  if (p.used + 2 > p.pool.size()) {
    for (int i = 0; i < 256; ++i) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      p.pool.push_back(e);
    }
  }
  LaunchEvents& le = launch_events();
  le.start = p.pool[p.used];
  le.stop = p.pool[p.used + 1];
  return le.start;
}
void prof_end(ttt_model* m, hipStream_t st, int cls, double flops, double bytes) {
  Prof& p = m->prof;
  LaunchEvents& le = launch_events();
  if (le.start) {  // no kernel was launched: an empty interval at this point of the stream
    (void)hipEventRecord(p.pool[p.used], st);
    (void)hipEventRecord(p.pool[p.used + 1], st);
  }
  le.start = le.stop = nullptr;
  p.used += 2;
  p.cls_of.push_back(cls);
  p.flops.push_back(flops);
  p.bytes.push_back(bytes);
}

// ---------- thin wrappers that launch and check ----------
struct Ctx {
  ttt_model* m;
  hipStream_t st;
  bool own_ws = true;  // the split-K workspace belongs to the caller's stream
  hipError_t err = hipSuccess;
  const char* where = "";
  void chk(hipError_t e, const char* w) {
    if (err == hipSuccess && e != hipSuccess) {
      err = e;
      where = w;
    }
  }
  // Run `f` (one or more launches on stream s, default st); when the timing
  // hooks select class `cls` (or `alias`), bracket it with events and record
  // its algorithmic flops and HBM bytes.
  template <class F>
  void run(int cls, double flops, double bytes, F&& f, hipStream_t s = nullptr, int alias = -1) {
    hipStream_t ss = s ? s : st;
    if (!prof_wants(m->prof, cls, alias) || m->prof.seen++ % m->prof.every != 0) {
      f();
      return;
    }
    hipEvent_t e0 = prof_begin(m, ss);
    f();
    if (e0) prof_end(m, ss, cls, flops, bytes);
  }
  // C = A . B^T-ish per GemmArgs, optionally batched over sequences. cls: the
  // timing class (span pass, chunk loop or weight gradient + SGD).
  void gemm(int epi, bool out_f32, const GemmArgs& a, int batch = 1, hipStream_t on = nullptr,
            int cls = TTT_PROF_GEMM_CHUNK) {
    if (epi == EPI_SGD) cls = TTT_PROF_GEMM_SGD;
    // the frozen blocks' MLP up-projection with the activation fused, over a full prefill span
    const int alias = ((epi == EPI_SWIGLU || epi == EPI_GELU) && a.M == m->cfg.batch * m->span) ? TTT_PROF_MLP_UP
                                                                                              : -1;
    hipStream_t s = on ? on : st;
    // the split-K workspace belongs to the caller's stream
    const bool use_ws = !on && own_ws;
    float* ws = use_ws ? m->ws : nullptr;
    const double es = (double)m->es;
    const double flops = 2.0 * a.M * a.N * (double)a.K * batch;
    double bytes = ((double)a.M * a.K + (double)a.N * a.K) * es * batch;  // operands once
    if (epi == EPI_SGD) {
      // fp32 master read + written, one compute copy written (a second layout is a choice)
      bytes += (double)a.M * a.N * batch * (m->dt == 1 ? 8.0 + es : 8.0);
    } else if (epi == EPI_ROPE) {
      bytes += (double)a.M * a.N * es;
    } else {
      const int nout = (epi == EPI_SWIGLU) ? a.N / 2 : a.N;
      bytes += (double)a.M * nout * batch * ((out_f32 || epi == EPI_ADD) ? 4.0 : es) + (epi == EPI_ADD ? 4.0 * a.M * nout * batch : 0.0);
    }
    run(cls, flops, bytes,
        [&] { chk(gemm_launch(a, m->dt, epi, out_f32, batch, ws, use_ws ? m->ws_elems : 0, s), "gemm"); }, s, alias);
  }
  // `to` waits for everything enqueued so far on `from`
  void order(hipStream_t from, hipStream_t to, hipEvent_t e) {
    chk(hipEventRecord(e, from), "event record");
    chk(hipStreamWaitEvent(to, e, 0), "stream wait");
  }
  void transpose(const void* src, int rows, int cols, int64_t lds, void* dst, int64_t ldd, int batch,
                 int64_t s_src, int64_t s_dst) {
    run(TTT_PROF_OTHER, 0, 2.0 * rows * cols * batch * m->es, [&] {
      chk(transpose_launch(src, rows, cols, lds, m->dt, dst, ldd, m->dt, st, batch, s_src, s_dst), "transpose");
    });
  }
};

GemmArgs ga(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, int M, int N,
            int K) {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.C = C; g.ldc = ldc;
  g.M = M; g.N = N; g.K = K;
  return g;
}

inline char* off(void* p, int64_t elems, size_t es) { return static_cast<char*>(p) + elems * (int64_t)es; }

// nonzero seed of the stochastic rounding of one update (chunk, tail block, matrix)
inline uint32_t sr_seed(int64_t chunk, int j, int mat) {
  return (uint32_t)(chunk * 1024 + j * 8 + mat) * 2654435761u | 1u;
}

// The RMSNorm of fp32 rows x (gain gn) as the A operand of a skinny product,
// computed inside it: forward-only passes of at most GEMV_MAX_ROWS rows per
// product (bf16) skip the norm kernel and its output
void fold_norm(GemmArgs& g, const float* x, int64_t ldx, int64_t sx, const void* gn, float eps) {
  g.nx = x; g.ldnx = ldx; g.snx = sx; g.ng = gn; g.neps = eps;
}

// Q/K/V of block l for R = B*S rows (positions p0.. of each sequence): q into
// q_out, k and v into the block's ring caches (slot pos % cap), RoPE applied;
// in one product with the rotation in its epilogue, or through fp32 qkv. With
// nx set, A is the RMSNorm of nx (gain ng) instead of u.
void qkv(Ctx& c, const void* u, int l, int R, int S, int64_t p0, float* qkv32, void* q_out, int cap,
         const float* nx, const void* ng, int cls) {
  ttt_model* m = c.m;
  const int d = m->d, HD = m->HD;
  const float2* tab = m->cfg.rope ? m->rope : nullptr;
  if (m->qkv_rope) {
    GemmArgs g = ga(u, d, m->wqkv_t[l], d, nullptr, 0, R, 3 * HD, d);
    if (nx) fold_norm(g, nx, d, 0, ng, m->cfg.norm_eps);
    g.rope.q = q_out; g.rope.kc = m->kc[l]; g.rope.vc = m->vc[l]; g.rope.tab = tab;
    g.rope.ldq = HD; g.rope.seq_stride = (int64_t)cap * HD; g.rope.p0 = p0;
    g.rope.cap = cap; g.rope.S = S; g.rope.H = m->H; g.rope.hd = m->hd;
    c.gemm(EPI_ROPE, false, g, 1, nullptr, cls);
    return;
  }
  GemmArgs g = ga(u, d, m->wqkv_t[l], d, qkv32, 3 * HD, R, 3 * HD, d);
  if (nx) fold_norm(g, nx, d, 0, ng, m->cfg.norm_eps);
  c.gemm(EPI_STORE, true, g, 1, nullptr, cls);
  c.run(TTT_PROF_OTHER, 0, (double)R * 3 * HD * (4.0 + m->es), [&] {
    c.chk(rope_split_launch(qkv32, R, S, m->H, m->hd, p0, tab, q_out, m->kc[l], m->vc[l], cap, (int64_t)cap * HD,
                            m->dt, c.st),
          "rope");
  });
}

// RMSNorm forward of R rows of width d (fp32 in, compute dtype out, rstd).
// x_splits > 1: the rows are the output of an EPI_ADD product (residual
// x_res) that was split over K and left its partial sums in this stream's
// split-K workspace (GemmArgs::split_out); the norm adds them, in split
// order, then x_res, and stores the rows to x.
void norm_fwd(Ctx& c, float* x, int R, const void* g, void* y, float* rstd, int x_splits = 1,
              const float* x_res = nullptr) {
  ttt_model* m = c.m;
  const int d = m->d;
  const double bytes = (double)R * d * (x_splits > 1 ? 4.0 * x_splits + 8.0 : 4.0) + (double)R * d * m->es + 4.0 * R;
  c.run(TTT_PROF_NORM, 0, bytes, [&] {
    if (x_splits > 1)
      c.chk(rmsnorm_fwd_launch(m->ws, R, d, g, m->cfg.norm_eps, y, rstd, m->dt, c.st, x_splits, (int64_t)R * d,
                               x_res, x),
            "norm");
    else
      c.chk(rmsnorm_fwd_launch(x, R, d, g, m->cfg.norm_eps, y, rstd, m->dt, c.st), "norm");
  });
}

// dn: the gradient at the norm's output. dn_splits > 1: the product that
// made it was split over K and left its partial sums in this stream's split-K
// workspace (GemmArgs::split_out); the norm adds them, in split order.
void norm_bwd(Ctx& c, const float* x, const float* rstd, const void* g, const float* dn, int R, float* dres,
              void* dres_c, bool accumulate, int dn_splits = 1) {
  ttt_model* m = c.m;
  const int d = m->d;
  const double bytes =
      (double)R * d * (4.0 * (1 + dn_splits) + (accumulate ? 8.0 : 4.0) + (dres_c ? m->es : 0.0)) + 4.0 * R;
  const float* src = dn_splits > 1 ? m->ws : dn;
  c.run(TTT_PROF_NORM, 0, bytes, [&] {
    c.chk(rmsnorm_bwd_launch(x, rstd, g, src, R, d, dres, dres_c, accumulate, m->dt, c.st, dn_splits,
                             (int64_t)R * d),
          "norm_bwd");
  });
}

// visible (query, key) pairs of M queries at positions p0.. (per sequence)
double window_pairs(const ttt_model* m, int64_t p0, int M) {
  double pairs = 0;
  for (int i = 0; i < M; ++i) pairs += std::min<int64_t>(p0 + i + 1, m->cfg.window);
  return pairs;
}

void attn_fwd(Ctx& c, const AttnArgs& a) {
  ttt_model* m = c.m;
  c.run(TTT_PROF_ATTN_FWD, 4.0 * m->hd * m->H * window_pairs(m, a.pos0, a.M) * a.B,
        // q, o, the window's K and V rows once
        (double)a.B * (2.0 * a.M * m->HD * m->es + 2.0 * std::min<int64_t>(a.pos0 + a.M, m->cfg.window + a.M) * m->HD * m->es),
        [&] { c.chk(attn_fwd_launch(a, m->dt, c.st), "attn_fwd"); });
}

// ---------- the span pass: frozen prefix over positions [p0, p0+S) ----------
void span_pass(Ctx& c, int64_t p0, int S) {
  ttt_model* m = c.m;
  const int B = m->cfg.batch, d = m->d, HD = m->HD, R = B * S;
  const size_t es = m->es;
  c.run(TTT_PROF_OTHER, 0, (double)R * d * (4.0 + m->es), [&] {
    c.chk(embed_launch(m->ids, m->maxpos, p0, S, B, m->embed, d, m->V, m->sX, m->dt, c.st), "embed");
  });
  const bool fold = m->dt == 1 && R <= GEMV_MAX_ROWS;  // norms inside the skinny products
  const int GS = TTT_PROF_GEMM_SPAN;
  for (int l = 0; l <= m->t0; ++l) {
    if (!fold) norm_fwd(c, m->sX, R, m->g_attn[l], m->sU, m->sR);
    qkv(c, m->sU, l, R, S, p0, m->sQKV, m->sQ, m->cap_s, fold ? m->sX : nullptr, m->g_attn[l], GS);
    AttnArgs a;
    memset(&a, 0, sizeof(a));
    a.q = m->sQ; a.ldq = HD; a.kc = m->kc[l]; a.vc = m->vc[l]; a.ldk = HD;
    a.seq_stride = (int64_t)m->cap_s * HD; a.cap = m->cap_s; a.o = m->sO; a.ldo = HD; a.lse = m->sL;
    a.M = S; a.H = m->H; a.hd = m->hd; a.B = B; a.pos0 = p0; a.window = m->cfg.window; a.scale = m->scale;
    if (S <= m->cfg.mini_batch) {
      // few queries (decode, the last rows of a prefill): split each query
      // block's key range over workgroups
      a.nsplit = std::min(ttt_model::kMaxSplit,
                          attn_splits(S, m->H, B, std::min<int64_t>(m->cfg.window, p0 + S)));
      a.part_o = m->spart_o; a.part_m = m->spart_m; a.part_l = m->spart_l;
    }
    attn_fwd(c, a);
    GemmArgs g = ga(m->sO, HD, m->wo_t[l], HD, m->sX, d, R, d, HD);
    g.R = m->sX; g.ldr = d;
    c.gemm(EPI_ADD, true, g, 1, nullptr, GS);
    if (l == m->t0) break;
    if (!fold) norm_fwd(c, m->sX, R, m->g_mlp[l], m->sU, m->sR);
    // up-projection with the activation in its epilogue (SwiGLU weights are
    // stored with gate / up rows interleaved in blocks of 32)
    const int h = m->h, zw = m->mg * h;
    GemmArgs gu = ga(m->sU, d, m->wgu_t[l], d, m->sA, h, R, zw, d);
    if (fold) fold_norm(gu, m->sX, d, 0, m->g_mlp[l], m->cfg.norm_eps);
    c.gemm(m->mg == 2 ? EPI_SWIGLU : EPI_GELU, false, gu, 1, nullptr, GS);
    g = ga(m->sA, h, m->wd_t[l], h, m->sX, d, R, d, h);
    g.R = m->sX; g.ldr = d;
    c.gemm(EPI_ADD, true, g, 1, nullptr, GS);
  }
  (void)es;
  c.run(TTT_PROF_OTHER, 0, 8.0 * R * d, [&] {
    c.chk(copy_rows_f32_launch(m->sX, (int64_t)S * d, m->ystage + p0 * d, m->maxpos * d, S, d, B, c.st), "copy");
  });
}

// ---------- multi-head fast MLPs (mh_heads > 1) ----------
// Head h of sequence s: columns [h*dh, (h+1)*dh) of the block's normalised
// state through its own MLP back to the same columns of the residual. Every
// product is batched over the heads (batch strides dh / hh / the head's weight
// block), one launch per sequence.
void mh_forward(Ctx& c, int j, int M, float* xo) {
  ttt_model* m = c.m;
  const int B = m->cfg.batch, d = m->d, nh = m->nhm, dh = m->dhm, hh = m->hhm, htm = m->htm, mg = m->mg;
  const size_t es = m->es;
  const int64_t blk = (int64_t)nh * hh * dh;  // one part of one sequence's heads
  const int R = B * M;
  for (int s = 0; s < B; ++s)
    for (int part = 0; part < mg; ++part) {
      // z[:, part*htm + h*hh ..] = n_h . W_part_h^T   (fp32 pre-activations)
      GemmArgs g = ga(off(m->tn[j], (int64_t)s * M * d, es), d, off(m->f_mg[j], ((int64_t)s * mg + part) * blk, es), dh,
                      m->tz_m[j] + (int64_t)s * M * mg * htm + part * htm, mg * htm, M, hh, dh);
      g.sA = dh; g.sB = (int64_t)hh * dh; g.sC = hh;
      c.gemm(EPI_STORE, true, g, nh);
    }
  c.run(TTT_PROF_OTHER, 0, (double)R * (4.0 * mg * htm + es * htm), [&] {
    c.chk(act_fwd_launch(m->tz_m[j], R, htm, mg * htm, mg == 2, m->ta_m[j], htm, m->dt, c.st), "act");
  });
  for (int s = 0; s < B; ++s) {
    // x_out[:, h*dh ..] += a_h . W_down_h^T
    float* xs = xo + (int64_t)s * M * d;
    GemmArgs g = ga(off(m->ta_m[j], (int64_t)s * M * htm, es), htm, off(m->f_md[j], (int64_t)s * nh * dh * hh, es), hh,
                    xs, d, M, dh, hh);
    g.sA = hh; g.sB = (int64_t)dh * hh; g.sC = dh;
    g.R = xs; g.ldr = d; g.sR = dh;
    c.gemm(EPI_ADD, true, g, nh);
  }
}

// Backward of block j's multi-head MLP from drc (gradient at the block's
// MLP output, compute dtype, [B*M][d]): the head-batched input gradients
// (added to m->dn when need_dn), then the weight gradients with the SGD step,
// all on the chunk loop's stream after the products that read W_c.
void mh_backward(Ctx& c, int j, int M, void* drc, bool need_dn, int64_t chunk) {
  ttt_model* m = c.m;
  const int B = m->cfg.batch, d = m->d, nh = m->nhm, dh = m->dhm, hh = m->hhm, htm = m->htm, mg = m->mg;
  const size_t es = m->es;
  const int64_t blk = (int64_t)nh * hh * dh;
  const int R = B * M;
  const bool master = m->dt == 1;
  for (int s = 0; s < B; ++s) {
    // dA[:, h*hh ..] = dres_h . W_down_h   (input-grad layout [hh][dh])
    GemmArgs g = ga(off(drc, (int64_t)s * M * d, es), d, off(m->fb_md[j], (int64_t)s * blk, es), dh,
                    m->dA_m + (int64_t)s * M * htm, htm, M, hh, dh);
    g.sA = dh; g.sB = (int64_t)hh * dh; g.sC = hh;
    c.gemm(EPI_STORE, true, g, nh);
  }
  c.run(TTT_PROF_OTHER, 0, (double)R * htm * (4.0 * (mg + 1) + es * mg), [&] {
    c.chk(act_bwd_launch(m->tz_m[j], m->dA_m, R, htm, mg * htm, htm, htm, mg == 2, m->dz_m, mg * htm, m->dt, c.st),
          "act_bwd");
  });
  if (need_dn)
    for (int s = 0; s < B; ++s)
      for (int part = 0; part < mg; ++part) {
        // dn[:, h*dh ..] += dZ_part_h . W_part_h   (input-grad layout [dh][hh])
        float* dns = m->dn + (int64_t)s * M * d;
        GemmArgs g = ga(off(m->dz_m, (int64_t)s * M * mg * htm + part * htm, es), mg * htm,
                        off(m->fb_mg[j], ((int64_t)s * mg + part) * blk, es), hh, dns, d, M, dh, hh);
        g.sA = hh; g.sB = (int64_t)dh * hh; g.sC = dh;
        g.R = dns; g.ldr = d; g.sR = dh;
        c.gemm(EPI_ADD, true, g, nh);
      }
  // weight gradients from token-contiguous copies (K = the chunk's positions)
  c.transpose(drc, M, d, d, m->T_dres, M, B, (int64_t)M * d, (int64_t)d * M);
  c.transpose(m->ta_m[j], M, htm, htm, m->T_am, M, B, (int64_t)M * htm, (int64_t)htm * M);
  c.transpose(m->dz_m, M, mg * htm, mg * htm, m->T_dzm, M, B, (int64_t)M * mg * htm, (int64_t)mg * htm * M);
  c.transpose(m->tn[j], M, d, d, m->T_n, M, B, (int64_t)M * d, (int64_t)d * M);
  const float lr = m->cfg.lr;
  for (int s = 0; s < B; ++s) {
    // W_down_h [dh][hh] -= lr * dres_h^T . a_h
    const int64_t wd = (int64_t)s * nh * dh * hh;
    GemmArgs g = ga(off(m->T_dres, (int64_t)s * d * M, es), M, off(m->T_am, (int64_t)s * htm * M, es), M,
                    master ? off(m->f_md[j], wd, es) : nullptr, hh, dh, hh, M);
    g.sA = (int64_t)dh * M; g.sB = (int64_t)hh * M; g.sC = (int64_t)dh * hh;
    g.Wm = master ? m->m_md[j] + wd : reinterpret_cast<float*>(off(m->f_md[j], wd, es));
    g.ldw = hh; g.sW = (int64_t)dh * hh;
    g.C2 = off(m->fb_md[j], wd, es); g.ldc2 = dh; g.sC2 = (int64_t)hh * dh;
    g.lr = lr;
    g.sr_seed = (sr_seed(chunk, j, 4) ^ (uint32_t)(s * 0x9E3779B9u)) | 1u;
    c.gemm(EPI_SGD, false, g, nh);
    for (int part = 0; part < mg; ++part) {
      // W_part_h [hh][dh] -= lr * dZ_part_h^T . n_h
      const int64_t wg = ((int64_t)s * mg + part) * blk;
      g = ga(off(m->T_dzm, ((int64_t)s * mg * htm + part * htm) * M, es), M, off(m->T_n, (int64_t)s * d * M, es), M,
             master ? off(m->f_mg[j], wg, es) : nullptr, dh, hh, dh, M);
      g.sA = (int64_t)hh * M; g.sB = (int64_t)dh * M; g.sC = (int64_t)hh * dh;
      g.Wm = master ? m->m_mg[j] + wg : reinterpret_cast<float*>(off(m->f_mg[j], wg, es));
      g.ldw = dh; g.sW = (int64_t)hh * dh;
      g.C2 = off(m->fb_mg[j], wg, es); g.ldc2 = hh; g.sC2 = (int64_t)dh * hh;
      g.lr = lr;
      g.sr_seed = (sr_seed(chunk, j, 5 + part) ^ (uint32_t)(s * 0x9E3779B9u)) | 1u;
      c.gemm(EPI_SGD, false, g, nh);
    }
  }
}

// ---------- the tail over positions [P0, P0+M) of every sequence ----------
// bwd: run the backward and the SGD step (a complete chunk, M == b).
void tail_pass(Ctx& c, int64_t P0, int M, bool bwd, float* losses, int64_t loss_base, int64_t loss_n) {
  ttt_model* m = c.m;
  const int B = m->cfg.batch, d = m->d, HD = m->HD, R = B * M, V = m->V;
  const int hf = m->hf, ht = m->ht, mg = m->mg, zw = mg * hf;
  const size_t es = m->es;
  const float eps = m->cfg.norm_eps;
  // forward-only passes of few rows take their norms inside the skinny
  // products (the backward would read the norms' outputs)
  const bool fold_r = !bwd && m->dt == 1 && R <= GEMV_MAX_ROWS;  // one product over all rows
  // (not with multi-head fast MLPs, whose head-batched products read the norm's output)
  const bool fold_m = !bwd && m->dt == 1 && M <= GEMV_MAX_ROWS && !m->mh;  // batched over the sequences
  const int64_t sgu = (int64_t)zw * d, sd = (int64_t)d * hf;        // per-seq fast strides
  const int64_t smgu = (int64_t)mg * ht * d, smd = (int64_t)d * ht;  // per-seq master strides

  c.run(TTT_PROF_OTHER, 0, 8.0 * R * d, [&] {
    c.chk(copy_rows_f32_launch(m->ystage + P0 * d, m->maxpos * d, m->tx[0], (int64_t)M * d, M, d, B, c.st), "copy");
  });
  // the down projection of each tail block leaves its K splits (x_sp) and
  // residual (x_res) to the norm that reads its output
  int x_sp = 1;
  const float* x_res = nullptr;
  for (int j = 0; j < m->nt; ++j) {
    const int l = m->t0 + j;
    float* y = m->tx[j];  // block t0: the residual after its attention
    if (j >= 1) {
      y = m->ty[j];
      if (!fold_r) norm_fwd(c, m->tx[j], R, m->g_attn[l], m->tU, m->tr1[j], x_sp, x_res);
      qkv(c, m->tU, l, R, M, P0, m->tQKV, m->tq[j], m->cap_t, fold_r ? m->tx[j] : nullptr, m->g_attn[l],
          TTT_PROF_GEMM_CHUNK);
      AttnArgs a;
      memset(&a, 0, sizeof(a));
      a.q = m->tq[j]; a.ldq = HD; a.kc = m->kc[l]; a.vc = m->vc[l]; a.ldk = HD;
      a.seq_stride = (int64_t)m->cap_t * HD; a.cap = m->cap_t; a.o = m->to[j]; a.ldo = HD;
      a.lse = m->tlse[j]; a.M = M; a.H = m->H; a.hd = m->hd; a.B = B; a.pos0 = P0;
      a.window = m->cfg.window; a.scale = m->scale;
      a.nsplit = std::min(ttt_model::kMaxSplit,
                          attn_splits(M, m->H, B, std::min<int64_t>(m->cfg.window, P0 + M)));
      a.part_o = m->part_o; a.part_m = m->part_m; a.part_l = m->part_l;
      attn_fwd(c, a);
      GemmArgs g = ga(m->to[j], HD, m->wo_t[l], HD, y, d, R, d, HD);
      g.R = m->tx[j]; g.ldr = d;
      c.gemm(EPI_ADD, true, g);
    }
    if (!fold_m) norm_fwd(c, y, R, m->g_mlp[l], m->tn[j], m->tr2[j]);
    GemmArgs g = ga(m->tn[j], d, m->f_gu[j], d, m->tz[j], zw, M, zw, d);
    g.sA = (int64_t)M * d; g.sB = sgu; g.sC = (int64_t)M * zw;
    if (fold_m) fold_norm(g, y, d, (int64_t)M * d, m->g_mlp[l], eps);
    c.gemm(EPI_STORE, true, g, B);
    c.run(TTT_PROF_OTHER, 0, (double)R * (4.0 * zw + es * hf), [&] {
      c.chk(act_fwd_launch(m->tz[j], R, hf, zw, mg == 2, m->ta[j], hf, m->dt, c.st), "act");
    });
    float* xo = (j + 1 < m->nt) ? m->tx[j + 1] : m->txL;
    g = ga(m->ta[j], hf, m->f_d[j], hf, xo, d, M, d, hf);
    g.sA = (int64_t)M * hf; g.sB = sd; g.sC = (int64_t)M * d;
    g.R = y; g.ldr = d; g.sR = (int64_t)M * d;
    // (the multi-head fast MLP adds its output to xo itself)
    x_sp = 1;
    x_res = y;
    if (!fold_r && !m->mh) g.split_out = &x_sp;
    c.gemm(EPI_ADD, true, g, B);
    if (m->mh) mh_forward(c, j, M, xo);
  }
  if (!fold_r) norm_fwd(c, m->txL, R, m->gfin, m->tf, m->trf, x_sp, x_res);
  {
    GemmArgs g = ga(m->tf, d, m->wout_t, d, m->tlog, V, R, V, d);
    if (fold_r) fold_norm(g, m->txL, d, 0, m->gfin, eps);
    c.gemm(EPI_STORE, true, g);
  }
  {
    CEArgs a;
    memset(&a, 0, sizeof(a));
    a.logits = m->tlog; a.rows = R; a.S = M; a.V = V;
    a.ids = m->ids; a.ids_seq_stride = m->maxpos; a.p0 = P0; a.n_ids = m->n_ids;
    a.dz = bwd ? m->tdz : nullptr; a.dz_scale = 1.f / m->cfg.mini_batch;
    a.losses = losses; a.loss_base = loss_base; a.loss_ld = loss_n; a.loss_n = loss_n;
    a.last_lse = m->last_lse; a.last_max = m->last_max; a.last_arg = m->last_arg;
    a.status = m->status;
    c.run(TTT_PROF_CE, 0, (double)R * V * (4.0 + (bwd ? es : 0)), [&] { c.chk(ce_launch(a, m->dt, c.st), "ce"); });
  }
  if (!bwd) return;

  // ---------------- backward ----------------
  // every product below reads both operands K-contiguous, except the weight
  // gradients: input grads use the [in][out] copies of the weights; weight
  // grads read the activations and output gradients token-major (MN-major
  // operands), or token-contiguous copies of them
  // each input-gradient product that feeds a norm backward leaves its K
  // splits to it (dn_sp: the split count)
  int dn_sp = 1;
  {
    GemmArgs g = ga(m->tdz, V, m->wout_b, V, m->dn, d, R, d, V);
    g.split_out = &dn_sp;
    c.gemm(EPI_STORE, true, g);
  }
  norm_bwd(c, m->txL, m->trf, m->gfin, m->dn, R, m->dres, m->dres_b[m->nt - 1], false, dn_sp);
  const bool master = m->dt == 1, mnw = m->mn_dw;
  const int64_t sbgu = (int64_t)d * zw, sbd = (int64_t)hf * d;  // per-seq strides of the [in][out] copies
  for (int j = m->nt - 1; j >= 0; --j) {
    const int l = m->t0 + j;
    const int hcols = j == 0 ? ht : hf;
    void* drc = m->dres_b[j];  // gradient at this block's MLP output (compute dtype)
    void* dz = m->dZ_b[j];
    // dA = dres . W_down^T  (reads W_c before its update below)
    GemmArgs g = ga(drc, d, m->fb_d[j], d, m->dA, hf, M, hcols, d);
    g.sA = (int64_t)M * d; g.sB = sbd; g.sC = (int64_t)M * hf;
    c.gemm(EPI_STORE, true, g, B);
    // W_down trainable columns: W^T[d][ht] -= eta * dres^T . A_t  (side stream,
    // after the dA GEMM above has read W_c)
    if (mnw) {
      c.order(c.st, m->side, m->ev[2 * j]);
      g = ga(drc, d, m->ta[j], hf, master ? m->f_d[j] : nullptr, hf, d, ht, M);
      g.sA = (int64_t)M * d; g.sB = (int64_t)M * hf; g.mn = 1;
    } else {
      c.transpose(drc, M, d, d, m->Tdres[j], M, B, (int64_t)M * d, (int64_t)d * M);
      c.transpose(m->ta[j], M, ht, hf, m->Ta[j], M, B, (int64_t)M * hf, (int64_t)ht * M);
      c.order(c.st, m->side, m->ev[2 * j]);
      g = ga(m->Tdres[j], M, m->Ta[j], M, master ? m->f_d[j] : nullptr, hf, d, ht, M);
      g.sA = (int64_t)d * M; g.sB = (int64_t)ht * M;
    }
    g.sC = sd;
    g.Wm = master ? m->m_d[j] : static_cast<float*>(m->f_d[j]);
    g.ldw = master ? ht : hf; g.sW = master ? smd : sd;
    g.C2 = m->fb_d[j]; g.ldc2 = d; g.sC2 = sbd;
    g.lr = m->cfg.lr;
    g.sr_seed = sr_seed(P0 / m->cfg.mini_batch, j, 2);
    c.gemm(EPI_SGD, false, g, B, m->side);
    c.run(TTT_PROF_OTHER, 0, (double)R * hcols * (4.0 * (mg + 1) + es * mg), [&] {
      c.chk(act_bwd_launch(m->tz[j], m->dA, R, hcols, zw, hf, hf, mg == 2, dz, zw, m->dt, c.st), "act_bwd");
    });
    if (j >= 1) {
      // dn = dZ . W_gu^T (reads W_c before its update below)
      g = ga(dz, zw, m->fb_gu[j], zw, m->dn, d, M, d, zw);
      g.sA = (int64_t)M * zw; g.sB = sbgu; g.sC = (int64_t)M * d;
      // (the multi-head fast MLP adds its part to dn itself)
      dn_sp = 1;
      if (!m->mh) g.split_out = &dn_sp;
      c.gemm(EPI_STORE, true, g, B);
    }
    // multi-head fast MLP: its input gradient added to dn, then its update
    if (m->mh) mh_backward(c, j, M, drc, j >= 1, P0 / m->cfg.mini_batch);
    // W_gate / W_up trainable rows: W^T[ht][d] -= eta * dZ_t^T . n. On the
    // side stream, except for the first tail block: its update is the last
    // one the next chunk waits for, so it runs on this stream at once rather
    // than behind the side stream's queue. With one sequence the gate and up
    // parts are one launch batched over the part (the part index then also
    // separates their stochastic-rounding streams).
    if (!mnw) {
      c.transpose(m->tn[j], M, d, d, m->Tn[j], M, B, (int64_t)M * d, (int64_t)d * M);
      for (int part = 0; part < mg; ++part) {
        void* tdz = off(m->Tdz[j], (int64_t)part * B * ht * M, es);
        c.transpose(off(dz, (int64_t)part * hf, es), M, ht, zw, tdz, M, B, (int64_t)M * zw, (int64_t)ht * M);
      }
    }
    hipStream_t gu_st = j == 0 ? nullptr : m->side;
    if (j > 0) c.order(c.st, m->side, m->ev[2 * j + 1]);
    const bool by_part = B == 1 && mg > 1;
    for (int part = 0; part < (by_part ? 1 : mg); ++part) {
      const int64_t zoff = (int64_t)part * hf;      // column of dZ / row of the forward copy
      const int64_t moff = (int64_t)part * ht * d;  // row block of the master
      void* fcopy = master ? off(m->f_gu[j], zoff * d, es) : nullptr;
      if (mnw) {
        g = ga(off(dz, zoff, es), zw, m->tn[j], d, fcopy, d, ht, d, M);
        g.sA = by_part ? (int64_t)hf : (int64_t)M * zw; g.sB = by_part ? 0 : (int64_t)M * d; g.mn = 1;
      } else {
        void* tdz = off(m->Tdz[j], (int64_t)part * B * ht * M, es);
        g = ga(tdz, M, m->Tn[j], M, fcopy, d, ht, d, M);
        g.sA = (int64_t)ht * M; g.sB = by_part ? 0 : (int64_t)d * M;
      }
      g.sC = by_part ? (int64_t)hf * d : sgu;
      g.Wm = master ? m->m_gu[j] + moff : reinterpret_cast<float*>(off(m->f_gu[j], zoff * d, es));
      g.ldw = d; g.sW = by_part ? (int64_t)(master ? ht : hf) * d : (master ? smgu : sgu);
      g.C2 = off(m->fb_gu[j], zoff, es); g.ldc2 = zw; g.sC2 = by_part ? (int64_t)hf : sbgu;
      g.lr = m->cfg.lr;
      g.sr_seed = sr_seed(P0 / m->cfg.mini_batch, j, part);
      c.gemm(EPI_SGD, false, g, by_part ? mg : B, gu_st);
    }
    if (j == 0) break;
    norm_bwd(c, m->ty[j], m->tr2[j], m->g_mlp[l], m->dn, R, m->dres, m->dres_c, true, dn_sp);
    // attention sublayer
    c.gemm(EPI_STORE, false, ga(m->dres_c, d, m->wo_b[l], d, m->dO, HD, R, HD, d));
    c.run(TTT_PROF_OTHER, 0, (double)R * (2.0 * HD * es + 4.0 * m->H), [&] {
      c.chk(attn_delta_launch(m->to[j], m->dO, R, m->H, m->hd, HD, M, m->delta, m->dt, c.st), "delta");
    });
    AttnArgs a;
    memset(&a, 0, sizeof(a));
    a.q = m->tq[j]; a.ldq = HD; a.kc = m->kc[l]; a.vc = m->vc[l]; a.ldk = HD;
    a.seq_stride = (int64_t)m->cap_t * HD; a.cap = m->cap_t; a.o = m->to[j]; a.ldo = HD;
    a.lse = m->tlse[j]; a.M = M; a.H = m->H; a.hd = m->hd; a.B = B; a.pos0 = P0;
    a.window = m->cfg.window; a.scale = m->scale;
    a.dout = m->dO; a.lddo = HD; a.delta = m->delta; a.dq = m->dq; a.lddq = HD;
    a.dk = m->dk; a.dv = m->dv; a.lddk = HD;
    a.nsplit = std::min(ttt_model::kMaxSplit, attn_splits(M, m->H, B, std::min<int64_t>(m->cfg.window, P0 + M)));
    {
      // dQ over the window, then dK / dV of the chunk's own keys (two launches)
      const double pairs = window_pairs(m, P0, M), inchunk = (double)M * (M + 1) / 2.0;
      const double kv = (double)B * std::min<int64_t>(P0 + M, m->cfg.window + M) * HD * es * 2.0;
      a.parts = 1;
      c.run(TTT_PROF_ATTN_DQ, 4.0 * pairs * m->hd * m->H * B, kv + (double)R * HD * (3.0 * es + 4.0 * a.nsplit),
            [&] { c.chk(attn_bwd_launch(a, m->dt, c.st), "attn_bwd_dq"); });
      a.parts = 2;
      c.run(TTT_PROF_ATTN_DKDV, 4.0 * inchunk * m->hd * m->H * B, (double)R * HD * (4.0 * es + 8.0),
            [&] { c.chk(attn_bwd_launch(a, m->dt, c.st), "attn_bwd_dkdv"); });
    }
    c.run(TTT_PROF_OTHER, 0, (double)R * HD * (4.0 * (a.nsplit + 2) + 3.0 * es), [&] {
      c.chk(rope_bwd_pack_launch(m->dq, a.nsplit, m->dk, m->dv, R, M, m->H, m->hd, P0,
                                 m->cfg.rope ? m->rope : nullptr, m->dqkv, m->dt, c.st),
            "rope_bwd");
    });
    g = ga(m->dqkv, 3 * HD, m->wqkv_b[l], 3 * HD, m->dn, d, R, d, 3 * HD);
    g.split_out = &dn_sp;
    c.gemm(EPI_STORE, true, g);
    // the gradient at block j's input is the one at block j-1's MLP output
    norm_bwd(c, m->tx[j], m->tr1[j], m->g_attn[l], m->dn, R, m->dres, m->dres_b[j - 1], true, dn_sp);
  }
  // the next use of the fast weights (and of the per-block operand copies) waits
  // for every SGD step of this chunk
  c.order(m->side, c.st, m->ev[2 * m->nt]);
}

// Wait for `st` and read the status word the kernels of earlier calls set.
// A non-finite logit row means the fast weights (or the inputs) hold
// non-finite values: the model is poisoned until ttt_reset.
int check_status(ttt_model* m, hipStream_t st, std::vector<int32_t>* ids_out = nullptr,
                 const int32_t* ids_dev = nullptr, int64_t n_ids = 0) {
  int32_t flag = 0;
  hipError_t e = hipSuccess;
  if (ids_out) {
    ids_out->resize((size_t)n_ids);
    e = hipMemcpyAsync(ids_out->data(), ids_dev, n_ids * 4, hipMemcpyDeviceToHost, st);
  }
  if (e == hipSuccess) e = hipMemcpyAsync(&flag, m->status, 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(TTT_EHIP, std::string("reading the ids / status: ") + hipGetErrorString(e));
  }
  if (flag) {
    m->poisoned = true;
    return fail(TTT_ESTATE, flag & 2 ? "an earlier call produced a greedy id from non-finite logits; call ttt_reset"
                                     : "an earlier call produced non-finite logits; call ttt_reset");
  }
  return TTT_OK;
}

int finish(Ctx& c) {
  if (c.err != hipSuccess) {
    c.m->poisoned = true;
    return fail(TTT_EHIP, std::string("HIP error in ") + c.where + ": " + hipGetErrorString(c.err));
  }
  return TTT_OK;
}

int validate(const ttt_config* c) {
  if (!c) return fail(TTT_EINVAL, "cfg is NULL");
  if (c->vocab < 1 || c->d_model < 1 || c->n_blocks < 1 || c->n_heads < 1 || c->head_dim < 1)
    return fail(TTT_EINVAL, "sizes must be positive");
  if (c->n_ttt_blocks < 1 || c->n_ttt_blocks > c->n_blocks) return fail(TTT_EINVAL, "n_ttt_blocks out of range");
  if (c->window < c->mini_batch) return fail(TTT_EINVAL, "window k must be >= mini_batch b");
  if (c->mini_batch < 1) return fail(TTT_EINVAL, "mini_batch must be >= 1");
  // the weight-gradient products contract over the chunk's b positions (K = b)
  if (c->dtype == TTT_BF16 && c->mini_batch % 8)
    return fail(TTT_EINVAL, "mini_batch must be a multiple of 8 for bf16 (K of the weight-gradient products)");
  if (c->dtype == TTT_FP32 && c->mini_batch % 4)
    return fail(TTT_EINVAL, "mini_batch must be a multiple of 4 for fp32 (K of the weight-gradient products)");
  if (c->dtype != TTT_FP32 && c->dtype != TTT_BF16) return fail(TTT_EINVAL, "dtype");
  if (c->mlp_kind != TTT_GELU && c->mlp_kind != TTT_SWIGLU) return fail(TTT_EINVAL, "mlp_kind");
  if (c->batch < 1 || c->max_positions < 2) return fail(TTT_EINVAL, "batch / max_positions");
  const int hd = c->head_dim;
  if (c->dtype == TTT_BF16 && hd != 16 && hd != 32 && hd != 64 && hd != 128)
    return fail(TTT_EINVAL, "head_dim must be 16, 32, 64 or 128 for bf16");
  if (c->dtype == TTT_FP32 && hd != 16 && hd != 32 && hd != 64)
    return fail(TTT_EINVAL, "head_dim must be 16, 32 or 64 for fp32");
  if (c->rope && (hd % 2)) return fail(TTT_EINVAL, "rope needs an even head_dim");
  const int vec = 8;  // every contiguous extent a multiple of 8 elements
  const int tail_h = c->ttt_hidden + c->static_hidden;
  if (c->d_model % vec || (c->n_heads * hd) % vec || c->vocab % vec || c->mlp_hidden % vec ||
      c->ttt_hidden % vec || c->static_hidden < 0 || tail_h % vec)
    return fail(TTT_EINVAL, "d_model, n_heads*head_dim, vocab and hidden sizes must be multiples of 8");
  if (c->mlp_kind == TTT_SWIGLU && c->mlp_hidden % 32)
    return fail(TTT_EINVAL, "mlp_hidden must be a multiple of 32 for SwiGLU");
  if (c->vocab > 32768) return fail(TTT_EINVAL, "vocab above 32768 is not supported");
  if (c->ttt_hidden < 8) return fail(TTT_EINVAL, "ttt_hidden must be >= 8");
  if (c->mh_heads < 0) return fail(TTT_EINVAL, "mh_heads must be >= 0");
  if (c->mh_heads > 1) {
    const int nh = c->mh_heads;
    if (c->d_model % nh || c->ttt_hidden % nh || (c->d_model / nh) % vec || (c->ttt_hidden / nh) % vec)
      return fail(TTT_EINVAL, "mh_heads must divide d_model and ttt_hidden into multiples of 8");
    if (c->static_hidden < 8) return fail(TTT_EINVAL, "the multi-head variant needs a static MLP (static_hidden >= 8)");
  }
  return TTT_OK;
}

// transpose an [in][out] user matrix into rows [row0, row0+out) of a [.][in]
// buffer (ld = in) or into columns (ldd given)
hipError_t put_t(const void* src, int in, int out, void* dst, int64_t ldd, int sdt, int ddt, hipStream_t st) {
  return transpose_launch(src, in, out, out, sdt, dst, ldd, ddt, st);
}

}  // namespace

// ============================ C ABI ============================

extern "C" {

const char* ttt_last_error(void) { return g_err.c_str(); }

int64_t ttt_stream_length(const ttt_model* m) { return m ? m->n_ids : 0; }
int64_t ttt_device_bytes(const ttt_model* m) {
  if (!m) return 0;
  int64_t t = m->shared ? m->shared->bytes : 0;
  for (int k = 1; k < NPART; ++k) t += m->part_bytes[k];
  return t;
}

int ttt_device_bytes_by_part(const ttt_model* m, int64_t* out) {
  if (!m || !out) return fail(TTT_EINVAL, "model or out is NULL");
  out[0] = m->shared ? m->shared->bytes : 0;
  for (int k = 1; k < NPART; ++k) out[k] = m->part_bytes[k];
  return TTT_OK;
}

void ttt_model_destroy(ttt_model* m) {
  if (!m) return;
  (void)hipDeviceSynchronize();
  for (void* p : m->allocs) (void)hipFree(p);
  m->shared.reset();  // the shared part goes with the last model that holds it
  for (hipEvent_t e : m->prof.pool) (void)hipEventDestroy(e);
  for (hipEvent_t e : m->ev) (void)hipEventDestroy(e);
  if (m->side) (void)hipStreamDestroy(m->side);
  if (m->pre) (void)hipStreamDestroy(m->pre);
  for (hipEvent_t e : m->span_ev) (void)hipEventDestroy(e);
  for (hipEvent_t e : m->reach_ev) (void)hipEventDestroy(e);
  if (m->ev_ids) (void)hipEventDestroy(m->ev_ids);
  delete m;
}

static int reset_state(ttt_model* m, hipStream_t st) {
  const int B = m->cfg.batch;
  hipError_t e = hipSuccess;
  auto ck = [&](hipError_t x) { if (e == hipSuccess) e = x; };
  for (int j = 0; j < m->nt; ++j) {
    const int64_t ngu = (int64_t)m->mg * m->hf * m->d, nd = (int64_t)m->d * m->hf;
    for (int s = 0; s < B; ++s) {
      ck(hipMemcpyAsync(off(m->f_gu[j], s * ngu, m->es), m->i_gu[j], ngu * m->es, hipMemcpyDeviceToDevice, st));
      ck(hipMemcpyAsync(off(m->f_d[j], s * nd, m->es), m->i_d[j], nd * m->es, hipMemcpyDeviceToDevice, st));
      ck(hipMemcpyAsync(off(m->fb_gu[j], s * ngu, m->es), m->ib_gu[j], ngu * m->es, hipMemcpyDeviceToDevice, st));
      ck(hipMemcpyAsync(off(m->fb_d[j], s * nd, m->es), m->ib_d[j], nd * m->es, hipMemcpyDeviceToDevice, st));
      if (m->dt == 1 && m->ht) {
        const int64_t mgu = (int64_t)m->mg * m->ht * m->d, md = (int64_t)m->d * m->ht;
        ck(hipMemcpyAsync(m->m_gu[j] + s * mgu, m->im_gu[j], mgu * 4, hipMemcpyDeviceToDevice, st));
        ck(hipMemcpyAsync(m->m_d[j] + s * md, m->im_d[j], md * 4, hipMemcpyDeviceToDevice, st));
      }
      if (m->mh) {
        const int64_t mgu = (int64_t)m->mg * m->nhm * m->hhm * m->dhm, md = (int64_t)m->nhm * m->dhm * m->hhm;
        ck(hipMemcpyAsync(off(m->f_mg[j], s * mgu, m->es), m->i_mg[j], mgu * m->es, hipMemcpyDeviceToDevice, st));
        ck(hipMemcpyAsync(off(m->f_md[j], s * md, m->es), m->i_md[j], md * m->es, hipMemcpyDeviceToDevice, st));
        ck(hipMemcpyAsync(off(m->fb_mg[j], s * mgu, m->es), m->ib_mg[j], mgu * m->es, hipMemcpyDeviceToDevice, st));
        ck(hipMemcpyAsync(off(m->fb_md[j], s * md, m->es), m->ib_md[j], md * m->es, hipMemcpyDeviceToDevice, st));
        if (m->dt == 1) {
          ck(hipMemcpyAsync(m->m_mg[j] + s * mgu, m->im_mg[j], mgu * 4, hipMemcpyDeviceToDevice, st));
          ck(hipMemcpyAsync(m->m_md[j] + s * md, m->im_md[j], md * 4, hipMemcpyDeviceToDevice, st));
        }
      }
    }
  }
  // caches hold finite values (zeros): masked keys multiply by exactly zero
  for (int l = 0; l < m->L; ++l) {
    const int cap = l < m->t0 + 1 ? m->cap_s : m->cap_t;
    const int64_t n = (int64_t)B * cap * m->HD;
    ck(hipMemsetAsync(m->kc[l], 0, n * m->es, st));
    ck(hipMemsetAsync(m->vc[l], 0, n * m->es, st));
  }
  ck(hipMemsetAsync(m->status, 0, 4, st));
  ck(hipStreamSynchronize(st));
  m->n_ids = 0;
  m->chunk = 0;
  if (e != hipSuccess) {
    m->poisoned = true;
    return fail(TTT_EHIP, std::string("reset: ") + hipGetErrorString(e));
  }
  m->poisoned = false;
  return TTT_OK;
}

int ttt_reset(ttt_model* m, void* stream) {
  if (!m) return fail(TTT_EINVAL, "model is NULL");
  return reset_state(m, static_cast<hipStream_t>(stream));
}

// Shapes and derived sizes of a model from m->cfg (already validated).
static void init_shape(ttt_model* m) {
  const ttt_config* cfg = &m->cfg;
  const bool glu = cfg->mlp_kind == TTT_SWIGLU;
  const int L = cfg->n_blocks, t0 = L - cfg->n_ttt_blocks;
  m->dt = cfg->dtype == TTT_BF16 ? 1 : 0;
  m->es = m->dt ? 2 : 4;
  m->L = L; m->t0 = t0; m->nt = cfg->n_ttt_blocks; m->H = cfg->n_heads; m->hd = cfg->head_dim;
  m->HD = m->H * m->hd; m->d = cfg->d_model; m->V = cfg->vocab; m->h = cfg->mlp_hidden;
  m->ht = cfg->ttt_hidden; m->hs = cfg->static_hidden; m->hf = m->ht + m->hs; m->mg = glu ? 2 : 1;
  m->maxpos = cfg->max_positions;
  const int b = cfg->mini_batch;
  // default span: four mini-batches (at least 2048 positions). Shorter
  // passes interleave more finely with the chunk loop on the other stream;
  // at the 3B shape (b = 1024, k = 8192) 3072..4096 measured fastest (2048
  // and 16384 about 2-3% slower, 1024 25% slower), and the frozen blocks'
  // K/V rings (window + span slots) shrink with it
  int span = cfg->prefill_span > 0 ? cfg->prefill_span : std::max(4 * b, 2048);
  span = (int)std::min<int64_t>(span, m->maxpos);
  span = std::max(span, 1);
  m->span = span;
  m->cap_s = (int)round_up(cfg->window + span, 64);
  m->cap_t = (int)round_up(cfg->window + b, 64);
  m->scale = 1.f / std::sqrt((float)m->hd);
  m->qkv_rope = m->dt == 1 && m->hd % 64 == 0;
  if (cfg->mh_heads > 1) {
    // the fast part is multi-head; the dense tail products carry the static branch only
    m->mh = true;
    m->nhm = cfg->mh_heads;
    m->dhm = m->d / m->nhm;
    m->htm = cfg->ttt_hidden;
    m->hhm = m->htm / m->nhm;
    m->ht = 0;
    m->hf = m->hs;
  }
}

// The shared part: frozen weights and the initial fast weights.
static void alloc_shared(ttt_model* m, Alloc& A) {
  const int L = m->L, t0 = m->t0;
  const int d = m->d, HD = m->HD, V = m->V, hf = m->hf, ht = m->ht, mg = m->mg, h = m->h;
  A.part = PART_SHARED;
  // frozen weights
  m->embed = A.el((int64_t)V * d);
  m->gfin = A.el(d);
  m->wout_t = A.el((int64_t)V * d);
  m->wout_b = A.el((int64_t)V * d);
  m->g_attn.resize(L); m->g_mlp.resize(L); m->wqkv_t.resize(L); m->wo_t.resize(L);
  m->wgu_t.assign(L, nullptr); m->wd_t.assign(L, nullptr);
  m->wqkv_b.assign(L, nullptr); m->wo_b.assign(L, nullptr);
  for (int l = 0; l < L; ++l) {
    m->g_attn[l] = A.el(d);
    m->g_mlp[l] = A.el(d);
    m->wqkv_t[l] = A.el((int64_t)3 * HD * d);
    m->wo_t[l] = A.el((int64_t)d * HD);
    if (l < t0) {
      m->wgu_t[l] = A.el((int64_t)mg * h * d);
      m->wd_t[l] = A.el((int64_t)d * h);
    }
    if (l > t0) {
      m->wqkv_b[l] = A.el((int64_t)3 * HD * d);
      m->wo_b[l] = A.el((int64_t)d * HD);
    }
  }
  m->i_gu.resize(m->nt); m->i_d.resize(m->nt); m->ib_gu.resize(m->nt); m->ib_d.resize(m->nt);
  m->im_gu.assign(m->nt, nullptr); m->im_d.assign(m->nt, nullptr);
  if (m->mh) {
    const int64_t ngu = (int64_t)mg * m->nhm * m->hhm * m->dhm, nd = (int64_t)m->nhm * m->dhm * m->hhm;
    m->i_mg.resize(m->nt); m->i_md.resize(m->nt); m->ib_mg.resize(m->nt); m->ib_md.resize(m->nt);
    m->im_mg.assign(m->nt, nullptr); m->im_md.assign(m->nt, nullptr);
    for (int j = 0; j < m->nt; ++j) {
      m->i_mg[j] = A.el(ngu); m->i_md[j] = A.el(nd); m->ib_mg[j] = A.el(ngu); m->ib_md[j] = A.el(nd);
      if (m->dt == 1) { m->im_mg[j] = A.f32(ngu); m->im_md[j] = A.f32(nd); }
    }
  }
  for (int j = 0; j < m->nt; ++j) {
    m->i_gu[j] = A.el((int64_t)mg * hf * d);
    m->i_d[j] = A.el((int64_t)d * hf);
    m->ib_gu[j] = A.el((int64_t)mg * hf * d);
    m->ib_d[j] = A.el((int64_t)d * hf);
    if (m->dt == 1) {
      m->im_gu[j] = A.f32((int64_t)mg * ht * d);
      m->im_d[j] = A.f32((int64_t)d * ht);
    }
  }
}

// Per-model state: fast weights, caches and stream state, workspace.
static void alloc_state(ttt_model* m, Alloc& A) {
  const ttt_config* cfg = &m->cfg;
  const int L = m->L, t0 = m->t0, B = cfg->batch, b = cfg->mini_batch, span = m->span;
  const int d = m->d, HD = m->HD, V = m->V, hf = m->hf, ht = m->ht, mg = m->mg, h = m->h;
  A.part = PART_FAST;
  m->f_gu.resize(m->nt); m->f_d.resize(m->nt);
  m->fb_gu.resize(m->nt); m->fb_d.resize(m->nt);
  m->m_gu.assign(m->nt, nullptr); m->m_d.assign(m->nt, nullptr);
  for (int j = 0; j < m->nt; ++j) {
    m->f_gu[j] = A.el((int64_t)B * mg * hf * d);
    m->f_d[j] = A.el((int64_t)B * d * hf);
    m->fb_gu[j] = A.el((int64_t)B * mg * hf * d);
    m->fb_d[j] = A.el((int64_t)B * d * hf);
    if (m->dt == 1) {
      m->m_gu[j] = A.f32((int64_t)B * mg * ht * d);
      m->m_d[j] = A.f32((int64_t)B * d * ht);
    }
  }
  if (m->mh) {
    const int64_t ngu = (int64_t)mg * m->nhm * m->hhm * m->dhm, nd = (int64_t)m->nhm * m->dhm * m->hhm;
    m->f_mg.resize(m->nt); m->f_md.resize(m->nt); m->fb_mg.resize(m->nt); m->fb_md.resize(m->nt);
    m->m_mg.assign(m->nt, nullptr); m->m_md.assign(m->nt, nullptr);
    for (int j = 0; j < m->nt; ++j) {
      m->f_mg[j] = A.el(B * ngu); m->f_md[j] = A.el(B * nd); m->fb_mg[j] = A.el(B * ngu); m->fb_md[j] = A.el(B * nd);
      if (m->dt == 1) { m->m_mg[j] = A.f32(B * ngu); m->m_md[j] = A.f32(B * nd); }
    }
  }
  A.part = PART_CACHE;
  m->kc.resize(L); m->vc.resize(L);
  for (int l = 0; l < L; ++l) {
    const int cap = l <= t0 ? m->cap_s : m->cap_t;
    m->kc[l] = A.el((int64_t)B * cap * HD);
    m->vc[l] = A.el((int64_t)B * cap * HD);
  }
  m->ids = static_cast<int32_t*>(A.get((int64_t)B * m->maxpos * 4));
  m->ystage = A.f32((int64_t)B * m->maxpos * d);
  if (cfg->rope) m->rope = static_cast<float2*>(A.get(m->maxpos * (m->hd / 2) * 8));
  m->last_lse = A.f32(B); m->last_max = A.f32(B);
  m->last_arg = static_cast<int32_t*>(A.get(B * 4));
  m->status = static_cast<int32_t*>(A.get(4));
  A.part = PART_WORK;
  // span workspace
  const int64_t Rs = (int64_t)B * span;
  m->sX = A.f32(Rs * d); m->sR = A.f32(Rs); m->sL = A.f32(Rs * m->H);
  m->sU = A.el(Rs * d); m->sQKV = m->qkv_rope ? nullptr : A.f32(Rs * 3 * HD); m->sQ = A.el(Rs * HD); m->sO = A.el(Rs * HD);
  m->sA = A.el(Rs * h);
  // tail workspace
  const int64_t Rt = (int64_t)B * b;
  const int nt = m->nt;
  m->tx.resize(nt); m->ty.assign(nt, nullptr); m->tr1.assign(nt, nullptr); m->tr2.resize(nt);
  m->tlse.assign(nt, nullptr); m->tn.resize(nt); m->tq.assign(nt, nullptr); m->to.assign(nt, nullptr);
  m->tz.resize(nt); m->ta.resize(nt);
  for (int j = 0; j < nt; ++j) {
    m->tx[j] = A.f32(Rt * d);
    if (j >= 1) {
      m->ty[j] = A.f32(Rt * d); m->tr1[j] = A.f32(Rt); m->tlse[j] = A.f32(Rt * m->H);
      m->tq[j] = A.el(Rt * HD); m->to[j] = A.el(Rt * HD);
    }
    m->tr2[j] = A.f32(Rt); m->tn[j] = A.el(Rt * d);
    m->tz[j] = A.f32(Rt * mg * hf); m->ta[j] = A.el(Rt * hf);
  }
  m->txL = A.f32(Rt * d); m->trf = A.f32(Rt); m->tlog = A.f32(Rt * V);
  m->tf = A.el(Rt * d); m->tdz = A.el(Rt * V); m->tU = A.el(Rt * d); m->tQKV = m->qkv_rope ? nullptr : A.f32(Rt * 3 * HD);
  m->dres = A.f32(Rt * d); m->dn = A.f32(Rt * d); m->dA = A.f32(Rt * hf); m->delta = A.f32(Rt * m->H);
  m->dq = A.f32(ttt_model::kMaxSplit * Rt * HD); m->dk = A.f32(Rt * HD); m->dv = A.f32(Rt * HD);
  m->part_o = A.f32(ttt_model::kMaxSplit * Rt * HD);
  m->part_m = A.f32(ttt_model::kMaxSplit * Rt * m->H);
  m->part_l = A.f32(ttt_model::kMaxSplit * Rt * m->H);
  m->spart_o = A.f32(ttt_model::kMaxSplit * Rt * HD);
  m->spart_m = A.f32(ttt_model::kMaxSplit * Rt * m->H);
  m->spart_l = A.f32(ttt_model::kMaxSplit * Rt * m->H);
  m->dres_c = A.el(Rt * d); m->dO = A.el(Rt * HD); m->dqkv = A.el(Rt * 3 * HD);
  m->mn_dw = m->dt == 1 && d % 128 == 0 && ht % 128 == 0 && m->cfg.mini_batch % 64 == 0 && hf % 8 == 0;
  m->dres_b.resize(nt); m->dZ_b.resize(nt);
  if (!m->mn_dw) { m->Tdres.resize(nt); m->Ta.resize(nt); m->Tdz.resize(nt); m->Tn.resize(nt); }
  for (int j = 0; j < nt; ++j) {
    m->dres_b[j] = A.el(Rt * d); m->dZ_b[j] = A.el(Rt * mg * hf);
    if (!m->mn_dw) {
      m->Tdres[j] = A.el(Rt * d); m->Ta[j] = A.el(Rt * ht); m->Tdz[j] = A.el(Rt * mg * ht); m->Tn[j] = A.el(Rt * d);
    }
  }
  if (m->mh) {
    const int htm = m->htm;
    m->tz_m.resize(nt); m->ta_m.resize(nt);
    for (int j = 0; j < nt; ++j) { m->tz_m[j] = A.f32(Rt * mg * htm); m->ta_m[j] = A.el(Rt * htm); }
    m->dA_m = A.f32(Rt * htm); m->dz_m = A.el(Rt * mg * htm);
    m->T_dres = A.el(Rt * d); m->T_am = A.el(Rt * htm); m->T_dzm = A.el(Rt * mg * htm); m->T_n = A.el(Rt * d);
  }
  m->ws_elems = std::min<int64_t>((int64_t)1 << 26, 8 * Rt * std::max({d, 3 * HD, hf}));
  m->ws = A.f32(m->ws_elems);
}

// Streams, events, the RoPE table and a reset: the last steps of creating a
// model (its state allocated; the shared part uploaded).
static int finish_create(ttt_model* m, hipStream_t st) {
  const ttt_config* cfg = &m->cfg;
  const int B = cfg->batch, nt = m->nt;
  int rc = TTT_OK;
  if (hipStreamCreateWithFlags(&m->side, hipStreamNonBlocking) != hipSuccess) {
    m->side = nullptr;
    rc = fail(TTT_EHIP, "side stream creation failed");
    return rc;
  }
  for (int i = 0; i < 2 * nt + 2; ++i) {
    hipEvent_t e;
    if (hipEventCreateWithFlags(&e, kOrderEventFlags) != hipSuccess) {
      rc = fail(TTT_EHIP, "event creation failed");
      return rc;
    }
    m->ev.push_back(e);
  }
  if (hipStreamCreateWithFlags(&m->pre, hipStreamNonBlocking) != hipSuccess) {
    m->pre = nullptr;
    rc = fail(TTT_EHIP, "prefix stream creation failed");
    return rc;
  }
  {
    const int64_t nspan = (m->maxpos + m->span - 1) / m->span + 1;
    for (int64_t i = 0; i <= 2 * nspan; ++i) {
      hipEvent_t e;
      if (hipEventCreateWithFlags(&e, kOrderEventFlags) != hipSuccess) {
        rc = fail(TTT_EHIP, "event creation failed");
        return rc;
      }
      if (i == 2 * nspan) m->ev_ids = e;
      else if (i < nspan) m->span_ev.push_back(e);
      else m->reach_ev.push_back(e);
    }
  }

  hipError_t e = hipSuccess;
  auto ck = [&](hipError_t x) { if (e == hipSuccess) e = x; };
  if (cfg->rope) {
    const int half = m->hd / 2;
    // angles p * theta^(-2i/hd) in fp64 (an fp32 product loses ~1e-2 rad at p ~ 1e5)
    std::vector<double> inv(half);
    for (int i = 0; i < half; ++i) inv[i] = std::pow((double)cfg->rope_theta, -2.0 * i / m->hd);
    std::vector<float2> tab((size_t)m->maxpos * half);
    for (int64_t p = 0; p < m->maxpos; ++p)
      for (int i = 0; i < half; ++i) {
        const double a = (double)p * inv[i];
        tab[p * half + i] = make_float2((float)std::cos(a), (float)std::sin(a));
      }
    ck(hipMemcpyAsync(m->rope, tab.data(), tab.size() * 8, hipMemcpyHostToDevice, st));
    ck(hipStreamSynchronize(st));
  }
  ck(hipMemsetAsync(m->ids, 0, (int64_t)B * m->maxpos * 4, st));
  if (e != hipSuccess) {
    rc = fail(TTT_EHIP, std::string("create: ") + hipGetErrorString(e));
    return rc;
  }
  rc = reset_state(m, st);
  return rc;
}

// copy [in][out] user weights into the shared part's internal layouts
static hipError_t upload_shared(ttt_model* m, const ttt_weights* w, hipStream_t st) {
  const ttt_config* cfg = &m->cfg;
  const bool glu = cfg->mlp_kind == TTT_SWIGLU;
  const int L = m->L, t0 = m->t0;
  const int d = m->d, HD = m->HD, V = m->V, hf = m->hf, ht = m->ht, hs = m->hs, mg = m->mg, h = m->h;
  const size_t es = m->es;
  hipError_t e = hipSuccess;
  auto ck = [&](hipError_t x) { if (e == hipSuccess) e = x; };
  const int dt = m->dt;
  ck(hipMemcpyAsync(m->embed, w->embed, (int64_t)V * d * es, hipMemcpyDeviceToDevice, st));
  ck(hipMemcpyAsync(m->gfin, w->final_norm, d * es, hipMemcpyDeviceToDevice, st));
  ck(put_t(w->lm_head, d, V, m->wout_t, d, dt, dt, st));
  ck(hipMemcpyAsync(m->wout_b, w->lm_head, (int64_t)V * d * es, hipMemcpyDeviceToDevice, st));
  for (int l = 0; l < L; ++l) {
    ck(hipMemcpyAsync(m->g_attn[l], w->attn_norm[l], d * es, hipMemcpyDeviceToDevice, st));
    ck(hipMemcpyAsync(m->g_mlp[l], w->mlp_norm[l], d * es, hipMemcpyDeviceToDevice, st));
    if (m->qkv_rope) {
      // each head part's 32-column blocks of W^T to their permuted row blocks
      // (block b -> 2b in the first half, 2(b - nb/2) + 1 in the second),
      // batched over the heads
      const int hd = m->hd, nb = hd / 32;
      const void* src3[3] = {w->wq[l], w->wk[l], w->wv[l]};
      for (int part = 0; part < 3; ++part)
        for (int b = 0; b < nb; ++b) {
          const int k = b < nb / 2 ? 2 * b : 2 * (b - nb / 2) + 1;
          ck(transpose_launch(static_cast<const char*>(src3[part]) + (int64_t)32 * b * es, d, 32, HD, dt,
                              off(m->wqkv_t[l], ((int64_t)part * HD + 32 * k) * d, es), d, dt, st, m->H, hd,
                              (int64_t)hd * d));
        }
    } else {
      ck(put_t(w->wq[l], d, HD, m->wqkv_t[l], d, dt, dt, st));
      ck(put_t(w->wk[l], d, HD, off(m->wqkv_t[l], (int64_t)HD * d, es), d, dt, dt, st));
      ck(put_t(w->wv[l], d, HD, off(m->wqkv_t[l], (int64_t)2 * HD * d, es), d, dt, dt, st));
    }
    ck(put_t(w->wo[l], HD, d, m->wo_t[l], HD, dt, dt, st));
    if (l > t0) {
      const void* qkv[3] = {w->wq[l], w->wk[l], w->wv[l]};
      for (int i = 0; i < 3; ++i)
        ck(hipMemcpy2DAsync(off(m->wqkv_b[l], (int64_t)i * HD, es), 3 * HD * es, qkv[i], HD * es, HD * es, d,
                            hipMemcpyDeviceToDevice, st));
      ck(hipMemcpyAsync(m->wo_b[l], w->wo[l], (int64_t)HD * d * es, hipMemcpyDeviceToDevice, st));
    }
    if (l < t0) {
      if (glu) {
        // rows 64c .. 64c+31: gate units 32c .. 32c+31; rows 64c+32 .. 64c+63: up units
        for (int i = 0; i < 2; ++i)
          ck(transpose_launch(i ? w->w_up[l] : w->w_gate[l], d, 32, h, dt, off(m->wgu_t[l], (int64_t)i * 32 * d, es),
                              d, dt, st, h / 32, 32, (int64_t)64 * d));
      } else {
        ck(put_t(w->w_up[l], d, h, m->wgu_t[l], d, dt, dt, st));
      }
      ck(put_t(w->w_down[l], h, d, m->wd_t[l], h, dt, dt, st));
    } else {
      const int j = l - t0;
      // concatenated [gate_t | gate_s | up_t | up_s] rows (SwiGLU) or [up_t | up_s]
      const void* tr[2] = {glu ? w->w_gate[l] : w->w_up[l], w->w_up[l]};
      const void* sr[2] = {glu ? w->s_gate[l] : (hs ? w->s_up[l] : nullptr), hs ? w->s_up[l] : nullptr};
      const int zw = mg * hf;
      for (int part = 0; part < mg; ++part) {
        void* base = off(m->i_gu[j], (int64_t)part * hf * d, es);
        void* bb = off(m->ib_gu[j], (int64_t)part * hf, es);
        if (ht) {
          ck(put_t(tr[part], d, ht, base, d, dt, dt, st));
          if (dt == 1) ck(put_t(tr[part], d, ht, m->im_gu[j] + (int64_t)part * ht * d, d, dt, 0, st));
          // input-grad layout [d][zw]: columns [part*hf, part*hf + ht) trainable, then static
          ck(hipMemcpy2DAsync(bb, zw * es, tr[part], ht * es, ht * es, d, hipMemcpyDeviceToDevice, st));
        }
        if (hs) {
          ck(put_t(sr[part], d, hs, off(base, (int64_t)ht * d, es), d, dt, dt, st));
          ck(hipMemcpy2DAsync(off(bb, ht, es), zw * es, sr[part], hs * es, hs * es, d, hipMemcpyDeviceToDevice, st));
        }
      }
      if (ht) {
        ck(put_t(w->w_down[l], ht, d, m->i_d[j], hf, dt, dt, st));
        ck(hipMemcpyAsync(m->ib_d[j], w->w_down[l], (int64_t)ht * d * es, hipMemcpyDeviceToDevice, st));
        if (dt == 1) ck(put_t(w->w_down[l], ht, d, m->im_d[j], ht, dt, 0, st));
      }
      if (hs) {
        ck(put_t(w->s_down[l], hs, d, off(m->i_d[j], ht, es), hf, dt, dt, st));
        ck(hipMemcpyAsync(off(m->ib_d[j], (int64_t)ht * d, es), w->s_down[l], (int64_t)hs * d * es,
                          hipMemcpyDeviceToDevice, st));
      }
      if (m->mh) {
        // per head: user [nh][dh][hh] (gate / up) and [nh][hh][dh] (down); the
        // forward layouts are the per-head transposes, the input-grad layouts copies
        const int nh = m->nhm, dh = m->dhm, hh = m->hhm;
        const int64_t blk = (int64_t)nh * dh * hh;
        for (int part = 0; part < mg; ++part) {
          ck(transpose_launch(tr[part], dh, hh, hh, dt, off(m->i_mg[j], part * blk, es), dh, dt, st, nh,
                              (int64_t)dh * hh, (int64_t)hh * dh));
          if (dt == 1)
            ck(transpose_launch(tr[part], dh, hh, hh, dt, m->im_mg[j] + part * blk, dh, 0, st, nh, (int64_t)dh * hh,
                                (int64_t)hh * dh));
          ck(hipMemcpyAsync(off(m->ib_mg[j], part * blk, es), tr[part], blk * es, hipMemcpyDeviceToDevice, st));
        }
        ck(transpose_launch(w->w_down[l], hh, dh, dh, dt, m->i_md[j], hh, dt, st, nh, (int64_t)hh * dh,
                            (int64_t)dh * hh));
        if (dt == 1)
          ck(transpose_launch(w->w_down[l], hh, dh, dh, dt, m->im_md[j], hh, 0, st, nh, (int64_t)hh * dh,
                              (int64_t)dh * hh));
        ck(hipMemcpyAsync(m->ib_md[j], w->w_down[l], blk * es, hipMemcpyDeviceToDevice, st));
      }
    }
  }
  return e;
}

static int check_weights(const ttt_config* cfg, const ttt_weights* w) {
  if (!w || !w->embed || !w->final_norm || !w->lm_head || !w->attn_norm || !w->wq || !w->wk || !w->wv ||
      !w->wo || !w->mlp_norm || !w->w_up || !w->w_down)
    return fail(TTT_EINVAL, "weights: NULL pointer");
  const bool glu = cfg->mlp_kind == TTT_SWIGLU;
  const int L = cfg->n_blocks, t0 = L - cfg->n_ttt_blocks;
  for (int l = 0; l < L; ++l) {
    if (!w->attn_norm[l] || !w->wq[l] || !w->wk[l] || !w->wv[l] || !w->wo[l] || !w->mlp_norm[l] || !w->w_up[l] ||
        !w->w_down[l] || (glu && (!w->w_gate || !w->w_gate[l])))
      return fail(TTT_EINVAL, "weights: NULL block pointer");
    if (l >= t0 && cfg->static_hidden > 0 &&
        (!w->s_up || !w->s_down || !w->s_up[l] || !w->s_down[l] || (glu && (!w->s_gate || !w->s_gate[l]))))
      return fail(TTT_EINVAL, "weights: NULL static-branch pointer");
  }
  return TTT_OK;
}

int ttt_model_create(const ttt_config* cfg, const ttt_weights* w, void* stream, ttt_model** out) {
  if (!out) return fail(TTT_EINVAL, "out is NULL");
  *out = nullptr;
  int rc = validate(cfg);
  if (rc) return rc;
  rc = check_weights(cfg, w);
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  ttt_model* m = new ttt_model();
  m->cfg = *cfg;
  init_shape(m);
  m->shared = std::make_shared<Shared>();
  Alloc A{m};
  alloc_shared(m, A);
  alloc_state(m, A);
  if (!A.ok) {
    rc = fail(TTT_ENOMEM, A.why);
    ttt_model_destroy(m);
    return rc;
  }
  hipError_t e = upload_shared(m, w, st);
  if (e != hipSuccess) {
    rc = fail(TTT_EHIP, std::string("create: ") + hipGetErrorString(e));
    ttt_model_destroy(m);
    return rc;
  }
  rc = finish_create(m, st);
  if (rc) {
    ttt_model_destroy(m);
    return rc;
  }
  *out = m;
  return TTT_OK;
}

int ttt_model_create_session(const ttt_model* base, int32_t batch, int64_t max_positions, int32_t prefill_span,
                             int64_t max_device_bytes, void* stream, ttt_model** out) {
  if (!out) return fail(TTT_EINVAL, "out is NULL");
  *out = nullptr;
  if (!base) return fail(TTT_EINVAL, "base model is NULL");
  ttt_config cfg = base->cfg;
  cfg.batch = batch;
  cfg.max_positions = max_positions;
  cfg.prefill_span = prefill_span;
  cfg.max_device_bytes = max_device_bytes;
  int rc = validate(&cfg);
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  ttt_model* m = new ttt_model();
  m->cfg = cfg;
  init_shape(m);
  // the shared part is base's: pointers copied, ownership shared
  m->shared = base->shared;
  m->embed = base->embed; m->gfin = base->gfin; m->wout_t = base->wout_t; m->wout_b = base->wout_b;
  m->g_attn = base->g_attn; m->g_mlp = base->g_mlp; m->wqkv_t = base->wqkv_t; m->wo_t = base->wo_t;
  m->wgu_t = base->wgu_t; m->wd_t = base->wd_t; m->wqkv_b = base->wqkv_b; m->wo_b = base->wo_b;
  m->i_gu = base->i_gu; m->i_d = base->i_d; m->ib_gu = base->ib_gu; m->ib_d = base->ib_d;
  m->im_gu = base->im_gu; m->im_d = base->im_d;
  m->i_mg = base->i_mg; m->i_md = base->i_md; m->ib_mg = base->ib_mg; m->ib_md = base->ib_md;
  m->im_mg = base->im_mg; m->im_md = base->im_md;
  Alloc A{m};
  alloc_state(m, A);
  if (!A.ok) {
    rc = fail(TTT_ENOMEM, A.why);
    ttt_model_destroy(m);
    return rc;
  }
  rc = finish_create(m, st);
  if (rc) {
    ttt_model_destroy(m);
    return rc;
  }
  *out = m;
  return TTT_OK;
}

int ttt_prefill(ttt_model* m, const int32_t* tokens, int64_t n, float* losses, void* stream) {
  if (!m) return fail(TTT_EINVAL, "model is NULL");
  if (m->poisoned) return fail(TTT_ESTATE, "model is poisoned by an earlier HIP error; call ttt_reset");
  if (!tokens || n < 1) return fail(TTT_EINVAL, "tokens NULL or n < 1");
  if (m->n_ids + n > m->maxpos) return fail(TTT_EINVAL, "stream would exceed max_positions");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int B = m->cfg.batch, b = m->cfg.mini_batch;
  {
    // the new ids are read back once the caller's stream reaches this call,
    // and checked before any work is enqueued
    std::vector<int32_t> h;
    int rc = check_status(m, st, &h, tokens, (int64_t)B * n);
    if (rc) return rc;
    for (size_t i = 0; i < h.size(); ++i)
      if (h[i] < 0 || h[i] >= m->V)
        return fail(TTT_EINVAL, "token id " + std::to_string(h[i]) + " of sequence " + std::to_string(i / n) +
                                    " at new position " + std::to_string(i % n) + " is outside [0, vocab)");
  }
  Ctx c{m, st};
  const int64_t n0 = m->n_ids;
  c.chk(hipMemcpy2DAsync(m->ids + n0, m->maxpos * 4, tokens, n * 4, n * 4, B, hipMemcpyDeviceToDevice, st),
        "copy ids");
  if (losses && n0 == 0) {
    // the first id of a stream has no predecessor
    for (int s = 0; s < B; ++s) c.chk(fill_f32_launch(losses + s * n, 1, NAN, st), "fill");
  }
  // frozen prefix over the new positions, on the prefix stream after the id
  // upload. The chunk loop waits only for the span that holds its last row;
  // the prefix stream stays at most two spans ahead of the chunk loop, so its
  // work spreads over the loop instead of crowding its start.
  Ctx cp{m, m->pre};
  cp.own_ws = false;
  cp.chk(hipEventRecord(m->ev_ids, st), "event record");
  cp.chk(hipStreamWaitEvent(cp.st, m->ev_ids, 0), "stream wait");
  std::vector<int64_t> span_start;
  for (int64_t p = n0; p < n0 + n; p += m->span) span_start.push_back(p);
  const size_t nsp = span_start.size();
  size_t issued = 0, waited = 0;
  auto issue = [&](size_t k) {
    const int64_t p = span_start[k];
    if (k >= 2) cp.chk(hipStreamWaitEvent(cp.st, m->reach_ev[k - 2], 0), "stream wait");
    span_pass(cp, p, (int)std::min<int64_t>(m->span, n0 + n - p));
    cp.chk(hipEventRecord(m->span_ev[k], cp.st), "event record");
  };
  while (issued < std::min<size_t>(2, nsp)) issue(issued++);
  auto need = [&](int64_t last_pos) {
    while (waited < nsp && span_start[waited] <= last_pos) {
      c.chk(hipStreamWaitEvent(st, m->span_ev[waited], 0), "stream wait");
      // the chunk loop has reached span `waited`: release the one two ahead
      c.chk(hipEventRecord(m->reach_ev[waited], st), "event record");
      ++waited;
      if (issued < nsp && issued <= waited + 1) issue(issued++);
    }
  };
  m->n_ids = n0 + n;
  const int64_t n_lab = m->n_ids - 1;
  const int64_t loss_base = n0 - 1;
  while ((m->chunk + 1) * b <= n_lab && c.err == hipSuccess && cp.err == hipSuccess) {
    need(m->chunk * b + b - 1);
    tail_pass(c, m->chunk * b, b, !m->cfg.forward_only, losses, loss_base, n);
    ++m->chunk;
  }
  const int64_t p0 = m->chunk * b;
  need(m->n_ids - 1);
  if (p0 < m->n_ids) tail_pass(c, p0, (int)(m->n_ids - p0), false, losses, loss_base, n);
  need(INT64_MAX);  // the caller's stream covers all work of the call
  if (c.err == hipSuccess && cp.err != hipSuccess) {
    c.err = cp.err;
    c.where = cp.where;
  }
  return finish(c);
}

int ttt_decode(ttt_model* m, int64_t n_new, int32_t* tokens_out, float* losses, void* stream) {
  if (!m) return fail(TTT_EINVAL, "model is NULL");
  if (m->poisoned) return fail(TTT_ESTATE, "model is poisoned by an earlier HIP error; call ttt_reset");
  if (m->n_ids < 1) return fail(TTT_ESTATE, "decode before any prefill");
  if (n_new < 1) return fail(TTT_EINVAL, "n_new < 1");
  if (m->n_ids + n_new > m->maxpos) return fail(TTT_EINVAL, "decode would exceed max_positions");
  hipStream_t st = static_cast<hipStream_t>(stream);
  {
    int rc = check_status(m, st);
    if (rc) return rc;
  }
  Ctx c{m, st};
  const int B = m->cfg.batch, b = m->cfg.mini_batch;
  for (int64_t i = 0; i < n_new && c.err == hipSuccess; ++i) {
    const int64_t pos = m->n_ids;  // the new id lands here
    c.chk(decode_emit_launch(m->last_arg, m->last_lse, m->last_max, B, m->V, m->ids, m->maxpos, pos, tokens_out,
                             n_new, i, losses, m->status, st),
          "emit");
    m->n_ids = pos + 1;
    const int64_t n_lab = m->n_ids - 1;
    // a completed chunk is applied before the next position is computed
    while ((m->chunk + 1) * b <= n_lab && c.err == hipSuccess) {
      tail_pass(c, m->chunk * b, b, !m->cfg.forward_only, nullptr, 0, 0);
      ++m->chunk;
    }
    // forward of the new position with the current W: its logits pick the next id
    span_pass(c, pos, 1);
    tail_pass(c, pos, 1, false, nullptr, 0, 0);
  }
  return finish(c);
}

int ttt_get_weights(const ttt_model* m, int32_t seq, int32_t block, int32_t mat, float* dst, void* stream) {
  if (!m) return fail(TTT_EINVAL, "model is NULL");
  if (!dst) return fail(TTT_EINVAL, "dst is NULL");
  if (seq < 0 || seq >= m->cfg.batch) return fail(TTT_EINVAL, "seq out of range");
  if (block < m->t0 || block >= m->L) return fail(TTT_EINVAL, "block is not a tail (fast-weight) block");
  if (mat != TTT_UP && mat != TTT_GATE && mat != TTT_DOWN) return fail(TTT_EINVAL, "mat");
  if (mat == TTT_GATE && m->mg != 2) return fail(TTT_EINVAL, "GATE needs a SwiGLU model");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int j = block - m->t0, d = m->d, ht = m->ht, hf = m->hf, mg = m->mg;
  hipError_t e;
  if (m->mh) {
    // forward layouts per head: gate/up [nh][hh][dh] -> user [nh][dh][hh];
    // down [nh][dh][hh] -> user [nh][hh][dh]
    const int nh = m->nhm, dh = m->dhm, hh = m->hhm;
    const int64_t blk = (int64_t)nh * dh * hh;
    if (mat == TTT_DOWN) {
      const void* src = m->dt == 1 ? (const void*)(m->m_md[j] + seq * blk) : off(m->f_md[j], seq * blk, 4);
      e = transpose_launch(src, dh, hh, hh, 0, dst, dh, 0, st, nh, (int64_t)dh * hh, (int64_t)hh * dh);
    } else {
      const int part = (mat == TTT_GATE || mg == 1) ? 0 : 1;
      const int64_t o = ((int64_t)seq * mg + part) * blk;
      const void* src = m->dt == 1 ? (const void*)(m->m_mg[j] + o) : off(m->f_mg[j], o, 4);
      e = transpose_launch(src, hh, dh, dh, 0, dst, hh, 0, st, nh, (int64_t)hh * dh, (int64_t)dh * hh);
    }
    if (e != hipSuccess) return fail(TTT_EHIP, hipGetErrorString(e));
    return TTT_OK;
  }
  if (mat == TTT_DOWN) {
    // stored [d][ht] -> user [ht][d]
    if (m->dt == 1)
      e = transpose_launch(m->m_d[j] + (int64_t)seq * d * ht, d, ht, ht, 0, dst, d, 0, st);
    else
      e = transpose_launch(off(m->f_d[j], (int64_t)seq * d * hf, 4), d, ht, hf, 0, dst, d, 0, st);
  } else {
    const int part = (mat == TTT_GATE || mg == 1) ? 0 : 1;
    // stored rows [ht][d] -> user [d][ht]
    if (m->dt == 1)
      e = transpose_launch(m->m_gu[j] + (int64_t)seq * mg * ht * d + (int64_t)part * ht * d, ht, d, d, 0, dst, ht, 0,
                           st);
    else
      e = transpose_launch(off(m->f_gu[j], (int64_t)seq * mg * hf * d + (int64_t)part * hf * d, 4), ht, d, d, 0, dst,
                           ht, 0, st);
  }
  if (e != hipSuccess) return fail(TTT_EHIP, hipGetErrorString(e));
  return TTT_OK;
}

// ---- kernel timing (HIP events around each launch of the selected classes) ----
int ttt_prof_begin(ttt_model* m, int32_t kernel_class) {
  if (!m) return fail(TTT_EINVAL, "model is NULL");
  if (kernel_class < 0 || kernel_class > TTT_PROF_ALL) return fail(TTT_EINVAL, "kernel_class");
  Prof& p = m->prof;
  p.cls = kernel_class;
  p.every = 1;
  p.seen = 0;
  p.used = 0;
  p.cls_of.clear();
  p.flops.clear();
  p.bytes.clear();
  return TTT_OK;
}

int ttt_prof_sample(ttt_model* m, int32_t every) {
  if (!m) return fail(TTT_EINVAL, "model is NULL");
  if (every < 1) return fail(TTT_EINVAL, "every must be >= 1");
  m->prof.every = every;
  m->prof.seen = 0;
  return TTT_OK;
}

static int prof_collect(ttt_model* m, int n, double* ms, int64_t* launches, double* flops, double* bytes) {
  Prof& p = m->prof;
  for (int c = 0; c < n; ++c) {
    if (ms) ms[c] = 0;
    if (launches) launches[c] = 0;
    if (flops) flops[c] = 0;
    if (bytes) bytes[c] = 0;
  }
  int rc = TTT_OK;
  for (size_t i = 0; i + 1 < p.used && rc == TTT_OK; i += 2) {
    const size_t k = i / 2;
    float t = 0;
    if (hipEventSynchronize(p.pool[i + 1]) != hipSuccess) rc = fail(TTT_EHIP, "event sync");
    else if (hipEventElapsedTime(&t, p.pool[i], p.pool[i + 1]) != hipSuccess) rc = fail(TTT_EHIP, "event time");
    const int c = p.cls_of[k];
    if (rc != TTT_OK || c < 0 || c >= n) continue;
    if (ms) ms[c] += t;
    if (launches) launches[c] += 1;
    if (flops) flops[c] += p.flops[k];
    if (bytes) bytes[c] += p.bytes[k];
  }
  p.cls = -1;
  p.used = 0;
  p.cls_of.clear();
  p.flops.clear();
  p.bytes.clear();
  return rc;
}

int ttt_prof_end(ttt_model* m, double* total_ms, int64_t* launches, double* total_work) {
  if (!m) return fail(TTT_EINVAL, "model is NULL");
  double ms[TTT_PROF_NCLASS], fl[TTT_PROF_NCLASS], by[TTT_PROF_NCLASS];
  int64_t n[TTT_PROF_NCLASS];
  int rc = prof_collect(m, TTT_PROF_NCLASS, ms, n, fl, by);
  if (rc) return rc;
  double t = 0, w = 0;
  int64_t k = 0;
  for (int c = 0; c < TTT_PROF_NCLASS; ++c) {
    t += ms[c];
    k += n[c];
    // bytes for the memory-bound classes, flops otherwise
    w += (c == TTT_PROF_CE || c == TTT_PROF_NORM || c == TTT_PROF_OTHER) ? by[c] : fl[c];
  }
  if (total_ms) *total_ms = t;
  if (launches) *launches = k;
  if (total_work) *total_work = w;
  return TTT_OK;
}

int ttt_prof_end_classes(ttt_model* m, int32_t n, double* ms, int64_t* launches, double* flops, double* bytes) {
  if (!m) return fail(TTT_EINVAL, "model is NULL");
  if (n < 0 || n > TTT_PROF_NCLASS) return fail(TTT_EINVAL, "n");
  return prof_collect(m, n, ms, launches, flops, bytes);
}

}  // extern "C"

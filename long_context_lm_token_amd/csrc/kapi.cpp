// Single-kernel C entry points (include/ttt_kernels.h) for kernel-level tests.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/ttt.h"
#include "../../include/ttt_kernels.h"
#include "kernels.h"

// Split partials of ttt_k_attn_fwd_noalloc: a fixed device array, so that
// the call allocates nothing. Each device holds its own copy, at its own
// address, for the life of the process; host code reaches it only through the
// per-device address hipGetSymbolAddress returns.
constexpr int64_t kScratchFloats = (int64_t)16 << 20;  // 64 MiB
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {
thread_local std::string k_err;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device.
hipError_t scratch_ptr(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_dev[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

int g_gemm_mn = 0;  // test hook: operands of ttt_k_gemm stored MN-major
int kfail(int code, const char* msg) {
  k_err = msg;
  return code;
}
int kdone(hipError_t e) {
  if (e == hipErrorInvalidValue) return kfail(TTT_EINVAL, "unsupported size or layout");
  if (e != hipSuccess) return kfail(TTT_EHIP, hipGetErrorString(e));
  return TTT_OK;
}
}  // namespace

extern "C" {

const char* ttt_k_last_error(void) { return k_err.c_str(); }

int ttt_k_gemm(int32_t dtype, int32_t epi, int32_t out_f32, int32_t M, int32_t N, int32_t K, const void* A,
               int64_t lda, int64_t sA, const void* B, int64_t ldb, int64_t sB, void* C, int64_t ldc, int64_t sC,
               void* C2, int64_t ldc2, int64_t sC2, const float* R, int64_t ldr, int64_t sR, float* Wm, int64_t ldw,
               int64_t sW, float lr, uint32_t sr_seed, int32_t batch, float* ws, int64_t ws_elems, void* stream) {
  if (epi < 0 || epi > 4 || M < 0 || N < 0 || K < 0 || batch < 1) return kfail(TTT_EINVAL, "bad gemm arguments");
  const int v = dtype == 1 ? 8 : 4;
  if (K % v) return kfail(TTT_EINVAL, "K must be a multiple of the vector width");
  if (epi == 1 && !R) return kfail(TTT_EINVAL, "EPI_ADD needs R");
  if (epi == 2 && !Wm) return kfail(TTT_EINVAL, "EPI_SGD needs Wm");
  if (epi == 3 && N % 64) return kfail(TTT_EINVAL, "EPI_SWIGLU needs N a multiple of 64");
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.A = A; g.lda = lda; g.sA = sA; g.B = B; g.ldb = ldb; g.sB = sB; g.C = C; g.ldc = ldc; g.sC = sC;
  g.C2 = C2; g.ldc2 = ldc2; g.sC2 = sC2;
  g.M = M; g.N = N; g.K = K; g.R = R; g.ldr = ldr; g.sR = sR; g.Wm = Wm; g.ldw = ldw; g.sW = sW; g.lr = lr;
  g.sr_seed = sr_seed;
  g.mn = g_gemm_mn;
  return kdone(gemm_launch(g, dtype, epi, out_f32 != 0, batch, ws, ws_elems, static_cast<hipStream_t>(stream)));
}

int ttt_k_qkv_rope(int32_t rows, int32_t S, int32_t H, int32_t hd, int32_t K, const void* A, int64_t lda,
                   const void* Bp, const void* tab, int64_t p0, void* q, void* kc, void* vc, int32_t cap,
                   void* stream) {
  if (rows < 1 || S < 1 || rows % S || H < 1 || hd % 64 || K < 8 || K % 8 || lda < K || cap < S || cap % 64 ||
      p0 < 0 || !A || !Bp || !q || !kc || !vc)
    return kfail(TTT_EINVAL, "bad rotary Q/K/V arguments");
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  const int64_t HD = (int64_t)H * hd;
  g.A = A; g.lda = lda; g.B = Bp; g.ldb = K; g.M = rows; g.N = (int)(3 * HD); g.K = K;
  g.rope.q = q; g.rope.kc = kc; g.rope.vc = vc; g.rope.tab = static_cast<const float2*>(tab);
  g.rope.ldq = HD; g.rope.seq_stride = (int64_t)cap * HD; g.rope.p0 = p0; g.rope.cap = cap; g.rope.S = S;
  g.rope.H = H; g.rope.hd = hd;
  return kdone(gemm_launch(g, 1, EPI_ROPE, false, 1, nullptr, 0, static_cast<hipStream_t>(stream)));
}

void ttt_k_gemm_tile(int32_t cfg) { gemm_force_tile(cfg); }

void ttt_k_gemm_operands(int32_t mn) { g_gemm_mn = mn != 0; }

static AttnArgs mk(const void* q, const void* kc, const void* vc, int32_t cap, int32_t B, int32_t M, int32_t H,
                   int32_t hd, int64_t pos0, int32_t window, float scale) {
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  const int64_t HD = (int64_t)H * hd;
  a.q = q; a.ldq = HD; a.kc = kc; a.vc = vc; a.ldk = HD; a.seq_stride = (int64_t)cap * HD; a.cap = cap;
  a.M = M; a.H = H; a.hd = hd; a.B = B; a.pos0 = pos0; a.window = window; a.scale = scale;
  return a;
}

static int64_t attn_ws_floats(int32_t B, int32_t M, int32_t H, int32_t hd, int32_t nsplit) {
  return nsplit > 1 ? (int64_t)nsplit * B * M * ((int64_t)H * hd + 2 * H) : 0;
}

static int attn_fwd_ws(int32_t dtype, const void* q, const void* kc, const void* vc, int32_t cap, void* o, float* lse,
                       int32_t B, int32_t M, int32_t H, int32_t hd, int64_t pos0, int32_t window, float scale,
                       int32_t nsplit, float* ws, void* stream) {
  AttnArgs a = mk(q, kc, vc, cap, B, M, H, hd, pos0, window, scale);
  a.o = o; a.ldo = (int64_t)H * hd; a.lse = lse;
  a.nsplit = nsplit;
  if (nsplit > 1) {
    a.part_o = ws;
    a.part_m = ws + (int64_t)nsplit * B * M * H * hd;
    a.part_l = a.part_m + (int64_t)nsplit * B * H * M;
  }
  return kdone(attn_fwd_launch(a, dtype, static_cast<hipStream_t>(stream)));
}

int ttt_k_attn_fwd(int32_t dtype, const void* q, const void* kc, const void* vc, int32_t cap, void* o,
                   float* lse, int32_t B, int32_t M, int32_t H, int32_t hd, int64_t pos0, int32_t window,
                   float scale, int32_t nsplit, float* ws, void* stream) {
  if (cap % 64 || cap < window + M || window < 1 || B < 1 || M < 0)
    return kfail(TTT_EINVAL, "cap must be a multiple of 64 and >= window + M");
  if (nsplit < 1 || nsplit > 16 || (nsplit > 1 && !ws)) return kfail(TTT_EINVAL, "nsplit in 1..16, ws for > 1");
  return attn_fwd_ws(dtype, q, kc, vc, cap, o, lse, B, M, H, hd, pos0, window, scale, nsplit, ws, stream);
}

int ttt_k_attn_fwd_noalloc(int32_t dtype, const void* q, const void* kc, const void* vc, int32_t cap, void* o,
                           float* lse, int32_t B, int32_t M, int32_t H, int32_t hd, int64_t pos0, int32_t window,
                           float scale, int32_t nsplit, void* stream) {
  if (cap % 64 || cap < window + M || window < 1 || B < 1 || M < 0 || H < 1 || hd < 1)
    return kfail(TTT_EINVAL, "cap must be a multiple of 64 and >= window + M");
  if (nsplit < 1 || nsplit > 16) return kfail(TTT_EINVAL, "nsplit in 1..16");
  const int64_t need = attn_ws_floats(B, M, H, hd, nsplit);
  if (need > kScratchFloats) {
    k_err = "the split partials need " + std::to_string(need) + " floats; the static scratch holds " +
            std::to_string(kScratchFloats) + " (fewer splits, rows or heads per call)";
    return TTT_EINVAL;
  }
  float* ws = nullptr;
  if (need > 0) {
    hipError_t e = scratch_ptr(&ws);
    if (e != hipSuccess) return kfail(TTT_EHIP, hipGetErrorString(e));
  }
  return attn_fwd_ws(dtype, q, kc, vc, cap, o, lse, B, M, H, hd, pos0, window, scale, nsplit, ws, stream);
}

int ttt_k_attn_bwd(int32_t dtype, const void* q, const void* kc, const void* vc, int32_t cap, const float* lse,
                   const void* dout, const float* delta, float* dq, float* dk, float* dv, int32_t B, int32_t M,
                   int32_t H, int32_t hd, int64_t pos0, int32_t window, float scale, int32_t nsplit, void* stream) {
  if (cap % 64 || cap < window + M || window < 1 || B < 1 || M < 0)
    return kfail(TTT_EINVAL, "cap must be a multiple of 64 and >= window + M");
  if (nsplit < 1 || nsplit > 16) return kfail(TTT_EINVAL, "nsplit in 1..16");
  AttnArgs a = mk(q, kc, vc, cap, B, M, H, hd, pos0, window, scale);
  const int64_t HD = (int64_t)H * hd;
  a.lse = const_cast<float*>(lse); a.dout = dout; a.lddo = HD; a.delta = delta;
  a.dq = dq; a.lddq = HD; a.dk = dk; a.dv = dv; a.lddk = HD;
  a.nsplit = nsplit;
  return kdone(attn_bwd_launch(a, dtype, static_cast<hipStream_t>(stream)));
}

void ttt_k_attn_fwd_kernel(int32_t dl) { attn_force_fwd_kernel(dl); }

int32_t ttt_k_attn_splits(int32_t M, int32_t H, int32_t B, int64_t keys_per_query) {
  return attn_splits(M, H, B, keys_per_query);
}

int ttt_k_attn_delta(int32_t dtype, const void* o, const void* dout, int32_t B, int32_t M, int32_t H, int32_t hd,
                     float* delta, void* stream) {
  return kdone(attn_delta_launch(o, dout, B * M, H, hd, (int64_t)H * hd, M, delta, dtype,
                                 static_cast<hipStream_t>(stream)));
}

int ttt_k_ce(int32_t dtype, const float* logits, int32_t rows, int32_t V, const int32_t* ids2, int32_t labelled,
             float* losses, void* dz, float scale, float* lse, float* mx, int32_t* argmax, void* stream) {
  // each row is a one-position "sequence" at position 0 whose label is ids2[r][1]
  CEArgs a;
  memset(&a, 0, sizeof(a));
  a.logits = logits; a.rows = rows; a.S = 1; a.V = V;
  a.ids = ids2; a.ids_seq_stride = 2; a.p0 = 0; a.n_ids = labelled ? 2 : 1;
  a.dz = labelled ? dz : nullptr; a.dz_scale = scale;
  a.losses = labelled ? losses : nullptr; a.loss_base = 0; a.loss_ld = 1; a.loss_n = 1;
  if (!labelled) { a.last_lse = lse; a.last_max = mx; a.last_arg = argmax; }
  return kdone(ce_launch(a, dtype, static_cast<hipStream_t>(stream)));
}

int ttt_k_rmsnorm_fwd(int32_t dtype, const float* x, int32_t rows, int32_t d, const void* g, float eps, void* y,
                      float* rstd, void* stream) {
  return kdone(rmsnorm_fwd_launch(x, rows, d, g, eps, y, rstd, dtype, static_cast<hipStream_t>(stream)));
}

int ttt_k_rmsnorm_bwd(int32_t dtype, const float* x, const float* rstd, const void* g, const float* dn, int32_t rows,
                      int32_t d, float* dres, int32_t accumulate, void* stream) {
  return kdone(rmsnorm_bwd_launch(x, rstd, g, dn, rows, d, dres, nullptr, accumulate != 0, dtype,
                                  static_cast<hipStream_t>(stream)));
}

}  // extern "C"

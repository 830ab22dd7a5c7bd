// Row-wise and elementwise kernels for gfx950 (HBM-bound): embedding gather,
// RMSNorm forward/backward, RoPE split/pack, MLP activations, fused
// softmax / cross-entropy / logit-gradient, copies and decode bookkeeping.
// Each thread moves 16-byte vectors where the row length allows it; a row is
// owned by one workgroup so that its reductions stay in LDS.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int NT = 256;

template <typename T> __host__ __device__ inline const T* cp(const void* p) { return reinterpret_cast<const T*>(p); }
template <typename T> __host__ __device__ inline T* mp(void* p) { return reinterpret_cast<T*>(p); }

template <typename T> struct V8;
template <> struct V8<bf16> {
  typedef bf16x8 type;
  TTT_DEV static type load(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
  TTT_DEV static void store(bf16* p, const float (&v)[8]) {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16)v[e];
    *reinterpret_cast<bf16x8*>(p) = o;
  }
  TTT_DEV static void get(const bf16* p, float (&v)[8]) {
    const bf16x8 x = load(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
  }
};
template <> struct V8<float> {
  TTT_DEV static void store(float* p, const float (&v)[8]) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
  TTT_DEV static void get(const float* p, float (&v)[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};


// 4 consecutive values of T as floats (8-byte bf16 / 16-byte fp32 accesses)
TTT_DEV void get4(const bf16* p, float (&v)[4]) {
  const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (float)x[e];
}
TTT_DEV void get4(const float* p, float (&v)[4]) {
  const float4 x = *reinterpret_cast<const float4*>(p);
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
}
TTT_DEV void put4(bf16* p, const float (&v)[4]) {
  bf16x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = (bf16)v[e];
  *reinterpret_cast<bf16x4*>(p) = o;
}
TTT_DEV void put4(float* p, const float (&v)[4]) { *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]); }

// ------------------------------- embedding -------------------------------
template <typename T>
__global__ void embed_kernel(const int32_t* ids, int64_t ids_ss, int64_t p0, int S, const T* E,
                             int d, int vocab, float* x) {
  const int i = blockIdx.x, s = blockIdx.y;
  int id = ids[s * ids_ss + p0 + i];
  // ids are checked on the host before any launch (TTT_EINVAL); the clamp
  // only keeps a corrupted id from reading outside the table
  id = id < 0 ? 0 : (id >= vocab ? vocab - 1 : id);
  const T* e = E + (int64_t)id * d;
  float* o = x + ((int64_t)s * S + i) * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) o[c] = to_f32(e[c]);
}

// ------------------------------- RMSNorm ---------------------------------
// Where the norm's input row comes from. Plain: x (row stride d). Split
// (splits > 1): x holds the K-split partial sums of the product whose output
// is the row (split s at x + s * ss) and `res` the residual that product's
// epilogue adds; the norm adds the partials in split order, then the
// residual, as a split-K reduce does, and stores the row to `out`.
struct NormIn {
  const float* x;
  int splits;
  int64_t ss;
  const float* res;
  float* out;
};

// four consecutive columns (offset o of the row block) of the input row
TTT_DEV void norm_in4(const NormIn& in, int64_t o, float (&v)[4]) {
  get4(in.x + o, v);
  if (in.splits > 1) {
    for (int s = 1; s < in.splits; ++s) {
      float t[4];
      get4(in.x + s * in.ss + o, t);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += t[e];
    }
    float t[4];
    get4(in.res + o, t);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] += t[e];
    put4(in.out + o, v);
  }
}

// y = x * (mean(x^2) + eps)^(-1/2) * g ; rstd saved for the backward.
template <typename T>
__global__ void rmsnorm_fwd_kernel(NormIn in, int d, const T* g, float eps, T* y, float* rstd) {
  __shared__ float red[16];
  const int64_t r = blockIdx.x;
  float ss = 0.f;
  for (int c = threadIdx.x * 4; c < d; c += blockDim.x * 4) {
    float v[4];
    norm_in4(in, r * d + c, v);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = block_sum(ss, red);
  const float rs = rsqrtf(ss / d + eps);
  // the second pass reads the row back where the first pass left it (each
  // thread its own columns)
  const float* xr = (in.splits > 1 ? in.out : in.x) + r * d;
  T* yr = y + r * d;
  for (int c = threadIdx.x * 4; c < d; c += blockDim.x * 4) {
    float v[4], gg[4];
    get4(xr + c, v);
    get4(g + c, gg);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] *= rs * gg[e];
    put4(yr + c, v);
  }
  if (threadIdx.x == 0) rstd[r] = rs;
}

// The same with the row held in registers (C float4 per thread, d <= C*4*NT):
// x is read once.
template <typename T, int C>
__global__ void rmsnorm_fwd_reg_kernel(NormIn in, int d, const T* g, float eps, T* y, float* rstd) {
  __shared__ float red[16];
  const int64_t r = blockIdx.x;
  float v[C][4];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < C; ++k) {
    const int c = (k * NT + threadIdx.x) * 4;
    if (c < d) {
      norm_in4(in, r * d + c, v[k]);
#pragma unroll
      for (int e = 0; e < 4; ++e) ss += v[k][e] * v[k][e];
    }
  }
  ss = block_sum(ss, red);
  const float rs = rsqrtf(ss / d + eps);
  T* yr = y + r * d;
#pragma unroll
  for (int k = 0; k < C; ++k) {
    const int c = (k * NT + threadIdx.x) * 4;
    if (c < d) {
      float gg[4];
      get4(g + c, gg);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[k][e] *= rs * gg[e];
      put4(yr + c, v[k]);
    }
  }
  if (threadIdx.x == 0) rstd[r] = rs;
}

// Four consecutive columns of dn: with splits > 1, dn arrives as the K-split
// partial sums of the product that made it (split s at dn + s * ss), added
// here in split order, the order a split-K reduce adds them in.
TTT_DEV void get_dn4(const float* dr, int splits, int64_t ss, float (&v)[4]) {
  get4(dr, v);
  for (int s = 1; s < splits; ++s) {
    float t[4];
    get4(dr + s * ss, t);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] += t[e];
  }
}

// dx = r*g*dn - x * r^3 * mean(x*g*dn); dres (+)= dx; optional compute copy.
// Four consecutive columns per thread (d % 4 == 0).
template <typename T>
__global__ void rmsnorm_bwd_kernel(const float* x, const float* rstd, const T* g, const float* dn,
                                   int dn_splits, int64_t dn_ss, int d, float* dres, T* dres_c, bool accumulate) {
  __shared__ float red[16];
  const int64_t r = blockIdx.x;
  const float* xr = x + r * d;
  const float* dr = dn + r * d;
  float dot = 0.f;
  for (int c = threadIdx.x * 4; c < d; c += blockDim.x * 4) {
    float xv[4], gv[4], dv[4];
    get4(xr + c, xv);
    get4(g + c, gv);
    get_dn4(dr + c, dn_splits, dn_ss, dv);
#pragma unroll
    for (int e = 0; e < 4; ++e) dot += xv[e] * gv[e] * dv[e];
  }
  dot = block_sum(dot, red);
  const float rs = rstd[r];
  const float k = rs * rs * rs * dot / d;
  float* o = dres + r * d;
  T* oc = dres_c ? dres_c + r * d : nullptr;
  for (int c = threadIdx.x * 4; c < d; c += blockDim.x * 4) {
    float xv[4], gv[4], dv[4], v[4];
    get4(xr + c, xv);
    get4(g + c, gv);
    get_dn4(dr + c, dn_splits, dn_ss, dv);
    if (accumulate) get4(o + c, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = rs * gv[e] * dv[e] - xv[e] * k + (accumulate ? v[e] : 0.f);
    put4(o + c, v);
    if (oc) put4(oc + c, v);
  }
}

// The same with the row's x, dn (and dres) held in registers (d <= C*4*NT).
template <typename T, int C>
__global__ void rmsnorm_bwd_reg_kernel(const float* x, const float* rstd, const T* g, const float* dn,
                                       int dn_splits, int64_t dn_ss, int d, float* dres, T* dres_c,
                                       bool accumulate) {
  __shared__ float red[16];
  const int64_t r = blockIdx.x;
  const float* xr = x + r * d;
  const float* dr = dn + r * d;
  float xv[C][4], gd[C][4];
  float dot = 0.f;
#pragma unroll
  for (int k = 0; k < C; ++k) {
    const int c = (k * NT + threadIdx.x) * 4;
    if (c < d) {
      float gv[4], dv[4];
      get4(xr + c, xv[k]);
      get4(g + c, gv);
      get_dn4(dr + c, dn_splits, dn_ss, dv);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gd[k][e] = gv[e] * dv[e];
        dot += xv[k][e] * gd[k][e];
      }
    }
  }
  dot = block_sum(dot, red);
  const float rs = rstd[r];
  const float kk = rs * rs * rs * dot / d;
  float* o = dres + r * d;
  T* oc = dres_c ? dres_c + r * d : nullptr;
#pragma unroll
  for (int k = 0; k < C; ++k) {
    const int c = (k * NT + threadIdx.x) * 4;
    if (c < d) {
      float v[4];
      if (accumulate) get4(o + c, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = rs * gd[k][e] - xv[k][e] * kk + (accumulate ? v[e] : 0.f);
      put4(o + c, v);
      if (oc) put4(oc + c, v);
    }
  }
}

// ------------------------------- RoPE ------------------------------------
// fp32 qkv rows [rows][3*H*hd] (q | k | v), as the projection GEMM leaves
// them, so q and k are rounded to T once, after the rotation. Row r = s*S + i
// is position p0 + i. q -> q out (rotated), k (rotated), v -> ring caches at
// slot pos % cap.
// Each thread rotates 4 consecutive pairs (e, e + hd/2), e = 4t .. 4t+3.
template <typename T>
__global__ void rope_split_kernel(const float* qkv, int S, int H, int hd, int64_t p0, const float2* tab,
                                  T* q, T* kc, T* vc, int cap, int64_t seq_stride) {
  const int64_t r = blockIdx.x;
  const int s = r / S, i = r % S;
  const int64_t pos = p0 + i;
  const int HD = H * hd, half = hd / 2;
  const float* src = qkv + r * 3 * HD;
  T* kdst = kc + s * seq_stride + (pos % cap) * HD;
  T* vdst = vc + s * seq_stride + (pos % cap) * HD;
  T* qdst = q + r * HD;
  for (int t = threadIdx.x; t < HD / 8; t += blockDim.x) {
    const int hh = (t * 4) / half, e = (t * 4) % half;
    const int c1 = hh * hd + e, c2 = c1 + half;
    float q1[4], q2[4], k1[4], k2[4], v1[4], v2[4];
    get4(src + c1, q1); get4(src + c2, q2);
    get4(src + HD + c1, k1); get4(src + HD + c2, k2);
    get4(src + 2 * HD + c1, v1); get4(src + 2 * HD + c2, v2);
    if (tab) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float2 cs = tab[pos * half + e + u];
        const float a = q1[u], b = q2[u], ka = k1[u], kb = k2[u];
        q1[u] = a * cs.x - b * cs.y;
        q2[u] = a * cs.y + b * cs.x;
        k1[u] = ka * cs.x - kb * cs.y;
        k2[u] = ka * cs.y + kb * cs.x;
      }
    }
    put4(qdst + c1, q1); put4(qdst + c2, q2);
    put4(kdst + c1, k1); put4(kdst + c2, k2);
    put4(vdst + c1, v1); put4(vdst + c2, v2);
  }
}

// inverse rotation of dq (sum of nsplit slices), dk (fp32 rows [rows][H*hd]);
// pack [dq | dk | dv] in T. Each thread handles 4 consecutive pairs.
template <typename T>
__global__ void rope_bwd_pack_kernel(const float* dq, int nsplit, int64_t rows, const float* dk, const float* dv,
                                     int S, int H, int hd, int64_t p0, const float2* tab, T* out) {
  const int64_t r = blockIdx.x;
  const int i = r % S;
  const int64_t pos = p0 + i;
  const int HD = H * hd, half = hd / 2;
  const float* a = dq + r * HD;
  const float* b = dk + r * HD;
  const float* v = dv + r * HD;
  T* o = out + r * 3 * HD;
  for (int t = threadIdx.x; t < HD / 8; t += blockDim.x) {
    const int hh = (t * 4) / half, e = (t * 4) % half;
    const int c1 = hh * hd + e, c2 = c1 + half;
    float x1[4], x2[4], y1[4], y2[4], v1[4], v2[4];
    get4(a + c1, x1); get4(a + c2, x2);
    for (int sp = 1; sp < nsplit; ++sp) {
      float t1[4], t2[4];
      get4(a + sp * rows * HD + c1, t1);
      get4(a + sp * rows * HD + c2, t2);
#pragma unroll
      for (int u = 0; u < 4; ++u) { x1[u] += t1[u]; x2[u] += t2[u]; }
    }
    get4(b + c1, y1); get4(b + c2, y2);
    get4(v + c1, v1); get4(v + c2, v2);
    if (tab) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float2 cs = tab[pos * half + e + u];
        const float xa = x1[u], xb = x2[u], ya = y1[u], yb = y2[u];
        x1[u] = xa * cs.x + xb * cs.y;
        x2[u] = -xa * cs.y + xb * cs.x;
        y1[u] = ya * cs.x + yb * cs.y;
        y2[u] = -ya * cs.y + yb * cs.x;
      }
    }
    put4(o + c1, x1); put4(o + c2, x2);
    put4(o + HD + c1, y1); put4(o + HD + c2, y2);
    put4(o + 2 * HD + c1, v1); put4(o + 2 * HD + c2, v2);
  }
}

// ----------------------------- activations -------------------------------
TTT_DEV float gelu_f(float x) { return 0.5f * x * (1.f + erff(x * 0.70710678118654752f)); }
TTT_DEV float gelu_g(float x) {
  return 0.5f * (1.f + erff(x * 0.70710678118654752f)) + x * 0.3989422804014327f * __expf(-0.5f * x * x);
}
TTT_DEV float sigm(float x) { return 1.f / (1.f + __expf(-x)); }

// GELU: a = gelu(z[:, j]); SwiGLU: a = silu(z[:, j]) * z[:, h + j], z in fp32
// (the pre-activations kept for the backward). Each thread handles 8
// consecutive columns (16-byte bf16 / 2x16-byte fp32 accesses).
template <typename T>
__global__ void act_fwd_kernel(const float* z, int h, int64_t ldz, int glu, T* a, int64_t lda) {
  const int64_t r = blockIdx.y;
  const int j = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (j >= h) return;
  const float* zr = z + r * ldz;
  float g[8], o[8];
  V8<float>::get(zr + j, g);
  if (glu) {
    float u[8];
    V8<float>::get(zr + h + j, u);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = g[e] * sigm(g[e]) * u[e];
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = gelu_f(g[e]);
  }
  V8<T>::store(a + r * lda + j, o);
}

template <typename T>
__global__ void act_bwd_kernel(const float* z, const float* da, int hcols, int64_t ldz, int64_t ldda,
                               int64_t up_off, int glu, T* dz, int64_t lddz) {
  const int64_t r = blockIdx.y;
  const int j = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (j >= hcols) return;
  const float* zr = z + r * ldz;
  float g[8], zg[8], o1[8];
  V8<float>::get(da + r * ldda + j, g);
  V8<float>::get(zr + j, zg);
  T* out = dz + r * lddz;
  if (glu) {
    float zu[8], o2[8];
    V8<float>::get(zr + up_off + j, zu);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sg = sigm(zg[e]);
      o1[e] = g[e] * zu[e] * sg * (1.f + zg[e] * (1.f - sg));
      o2[e] = g[e] * zg[e] * sg;
    }
    V8<T>::store(out + up_off + j, o2);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) o1[e] = g[e] * gelu_g(zg[e]);
  }
  V8<T>::store(out + j, o1);
}

// delta[s][h][i] = sum_d dO * O for row s*S+i, head h
// 8 consecutive elements per thread; the hd/8 lanes of a head (2..16, a
// power of two) reduce with butterflies. Whole waves iterate together.
template <typename T>
__global__ void attn_delta_kernel(const T* o, const T* dout, int H, int hd, int64_t ld, int S,
                                  float* delta) {
  const int64_t r = blockIdx.x;
  const int s = r / S, i = r % S;
  const int nv = H * hd / 8, g = hd / 8;
  const int iters = (nv + blockDim.x - 1) / blockDim.x;
  for (int it = 0; it < iters; ++it) {
    const int t = it * blockDim.x + threadIdx.x;
    float acc = 0.f;
    if (t < nv) {
      float a[8], b[8];
      V8<T>::get(o + r * ld + t * 8, a);
      V8<T>::get(dout + r * ld + t * 8, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += a[e] * b[e];
    }
    for (int off = g >> 1; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (t < nv && t % g == 0) delta[((int64_t)s * H + t / g) * S + i] = acc;
  }
}

// -------------------------- cross entropy --------------------------------
// One workgroup per row: max / argmax / sum-exp over V fp32 logits read once
// into registers; loss = lse - z[label]; dz = (softmax - onehot)*scale.
// Each thread owns runs of 8 consecutive logits (two 16-byte loads, one
// 16-byte bf16 store of the gradient); the exponentials of the sum pass stay
// in registers for the gradient.
constexpr int CE_NT = 512;
constexpr int CE_IT = 8;  // runs of 8 per thread -> up to 32768 logits

template <typename T>
__global__ __launch_bounds__(CE_NT) void ce_kernel(CEArgs a) {
  __shared__ float red[16];
  __shared__ int redi[16];
  const int64_t row = blockIdx.x;
  const int s = row / a.S, i = row % a.S;
  const int64_t pos = a.p0 + i;
  const float* z = a.logits + row * a.V;
  const int n8 = a.V / 8;
  float v[CE_IT][8];
  float mx = -INFINITY;
  int am = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < CE_IT; ++k) {
    const int idx = k * CE_NT + threadIdx.x;
    if (idx < n8) {
      V8<float>::get(z + idx * 8, v[k]);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (v[k][c] > mx) { mx = v[k][c]; am = idx * 8 + c; }
    }
  }
  // block argmax (lowest index among maxima)
  {
    float m = mx;
    int ai = am;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float om = __shfl_xor(m, o, 64);
      const int oi = __shfl_xor(ai, o, 64);
      if (om > m || (om == m && oi < ai)) { m = om; ai = oi; }
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { red[w] = m; redi[w] = ai; }
    __syncthreads();
    m = red[0];
    ai = redi[0];
    for (int k = 1; k < CE_NT / 64; ++k)
      if (red[k] > m || (red[k] == m && redi[k] < ai)) { m = red[k]; ai = redi[k]; }
    mx = m;
    am = ai;
    __syncthreads();
  }
  float se = 0.f;
#pragma unroll
  for (int k = 0; k < CE_IT; ++k) {
    const int idx = k * CE_NT + threadIdx.x;
    if (idx < n8) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        v[k][c] = __expf(v[k][c] - mx);
        se += v[k][c];
      }
    }
  }
  se = block_sum(se, red);
  const float lse = mx + logf(se);
  const bool has_label = pos + 1 < a.n_ids;
  int label = -1;
  if (has_label) {
    // ids are checked on the host before any launch; the clamp only keeps a
    // corrupted id from reading outside the row
    label = a.ids[s * a.ids_seq_stride + pos + 1];
    label = label < 0 ? 0 : (label >= a.V ? a.V - 1 : label);
  }
  if (threadIdx.x == 0) {
    const float loss = has_label ? lse - z[label] : 0.f;
    if (a.status && !(isfinite(lse) && isfinite(loss))) a.status[0] = 1;
    if (has_label && a.losses) {
      const int64_t li = pos - a.loss_base;
      if (li >= 0 && li < a.loss_n) a.losses[s * a.loss_ld + li] = loss;
    }
    if (pos == a.n_ids - 1 && a.last_lse) {
      a.last_lse[s] = lse;
      a.last_max[s] = mx;
      a.last_arg[s] = am;
    }
  }
  if (a.dz) {
    T* dz = reinterpret_cast<T*>(a.dz) + row * a.V;
    const float sc = has_label ? a.dz_scale / se : 0.f;
    const float sl = has_label ? a.dz_scale : 0.f;
#pragma unroll
    for (int k = 0; k < CE_IT; ++k) {
      const int idx = k * CE_NT + threadIdx.x;
      if (idx < n8) {
        float o[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c] = v[k][c] * sc - (idx * 8 + c == label ? sl : 0.f);
        V8<T>::store(dz + idx * 8, o);
      }
    }
  }
}

// ------------------------------- copies ----------------------------------
template <typename S, typename D>
__global__ void transpose_kernel(const S* src, int rows, int cols, int64_t lds, D* dst, int64_t ldd, int64_t s_src,
                                 int64_t s_dst) {
  __shared__ float tile[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  src += blockIdx.z * s_src;
  dst += blockIdx.z * s_dst;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 256 threads: 64 x 4
  for (int k = ty; k < 64; k += 4) {
    const int r = r0 + k, c = c0 + tx;
    tile[k][tx] = (r < rows && c < cols) ? to_f32(src[(int64_t)r * lds + c]) : 0.f;
  }
  __syncthreads();
  for (int k = ty; k < 64; k += 4) {
    const int c = c0 + k, r = r0 + tx;
    if (r < rows && c < cols) dst[(int64_t)c * ldd + r] = from_f32<D>(tile[tx][k]);
  }
}

// 8-element vectors along the source rows and along the destination rows
// (rows, cols, strides multiples of 8, 16-byte aligned bases).
template <typename S, typename D>
__global__ void transpose8_kernel(const S* src, int rows, int cols, int64_t lds, D* dst, int64_t ldd, int64_t s_src,
                                  int64_t s_dst) {
  __shared__ float tile[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  src += blockIdx.z * s_src;
  dst += blockIdx.z * s_dst;
  for (int v = threadIdx.x; v < 512; v += blockDim.x) {
    const int r = v >> 3, cv = (v & 7) * 8;
    float x[8];
    if (r0 + r < rows && c0 + cv < cols) {
      V8<S>::get(src + (int64_t)(r0 + r) * lds + c0 + cv, x);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[r][cv + e] = x[e];
  }
  __syncthreads();
  for (int v = threadIdx.x; v < 512; v += blockDim.x) {
    const int c = v >> 3, rv = (v & 7) * 8;
    if (c0 + c < cols && r0 + rv < rows) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = tile[rv + e][c];
      V8<D>::store(dst + (int64_t)(c0 + c) * ldd + r0 + rv, x);
    }
  }
}

__global__ void copy_rows_kernel(const float* src, int64_t sss, float* dst, int64_t dss, int S, int d) {
  const int i = blockIdx.x, s = blockIdx.y;
  const float* a = src + s * sss + (int64_t)i * d;
  float* b = dst + s * dss + (int64_t)i * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) b[c] = a[c];
}

__global__ void fill_kernel(float* p, int64_t n, float v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void decode_emit_kernel(const int32_t* next, const float* lse, const float* mx, int B, int vocab,
                                   int32_t* ids, int64_t ids_ss, int64_t pos, int32_t* out,
                                   int64_t out_ld, int64_t i, float* losses, int32_t* status) {
  const int s = threadIdx.x;
  if (s >= B) return;
  int32_t t = next[s];
  if (t < 0 || t >= vocab) {
    t = 0;
    if (status) status[0] = 2;
  }
  ids[s * ids_ss + pos] = t;
  if (out) out[s * out_ld + i] = t;
  if (losses) losses[s * out_ld + i] = lse[s] - mx[s];
}

}  // namespace

#define DT_DISPATCH(dt, KERNEL_CALL_BF16, KERNEL_CALL_F32) \
  do {                                                     \
    if ((dt) == 1) { KERNEL_CALL_BF16; }                   \
    else { KERNEL_CALL_F32; }                              \
  } while (0)

hipError_t embed_launch(const int32_t* ids, int64_t ids_ss, int64_t p0, int S, int B, const void* E,
                        int d, int vocab, float* x, int dt, hipStream_t st) {
  if (S <= 0 || B <= 0) return hipSuccess;
  dim3 g(S, B);
  DT_DISPATCH(dt,
      TTT_LAUNCH(embed_kernel<bf16>, g, dim3(NT), 0, st, ids, ids_ss, p0, S, cp<bf16>(E), d, vocab, x),
      TTT_LAUNCH(embed_kernel<float>, g, dim3(NT), 0, st, ids, ids_ss, p0, S, cp<float>(E), d, vocab, x));
  return hipGetLastError();
}

hipError_t rmsnorm_fwd_launch(const float* x, int rows, int d, const void* g, float eps, void* y,
                              float* rstd, int dt, hipStream_t st, int x_splits, int64_t x_ss,
                              const float* x_res, float* x_out) {
  if (rows <= 0) return hipSuccess;
  if (d % 4 || x_splits < 1) return hipErrorInvalidValue;
  if (x_splits > 1 && (x_ss < (int64_t)rows * d || !x_res || !x_out)) return hipErrorInvalidValue;
  const NormIn in{x, x_splits, x_ss, x_res, x_out};
  // rows of up to 4096 columns stay in registers (x read once)
  const int C = (d + 4 * NT - 1) / (4 * NT);
#define TTT_NORM_FWD(TT, CC) \
  TTT_LAUNCH((rmsnorm_fwd_reg_kernel<TT, CC>), dim3(rows), dim3(NT), 0, st, in, d, cp<TT>(g), eps, mp<TT>(y), rstd)
  if (C <= 4) {
    if (dt == 1) {
      if (C == 1) TTT_NORM_FWD(bf16, 1); else if (C == 2) TTT_NORM_FWD(bf16, 2);
      else if (C == 3) TTT_NORM_FWD(bf16, 3); else TTT_NORM_FWD(bf16, 4);
    } else {
      if (C == 1) TTT_NORM_FWD(float, 1); else if (C == 2) TTT_NORM_FWD(float, 2);
      else if (C == 3) TTT_NORM_FWD(float, 3); else TTT_NORM_FWD(float, 4);
    }
    return hipGetLastError();
  }
#undef TTT_NORM_FWD
  DT_DISPATCH(dt,
      TTT_LAUNCH(rmsnorm_fwd_kernel<bf16>, dim3(rows), dim3(NT), 0, st, in, d, cp<bf16>(g), eps, mp<bf16>(y), rstd),
      TTT_LAUNCH(rmsnorm_fwd_kernel<float>, dim3(rows), dim3(NT), 0, st, in, d, cp<float>(g), eps, mp<float>(y), rstd));
  return hipGetLastError();
}

hipError_t rmsnorm_bwd_launch(const float* x, const float* rstd, const void* g, const float* dn, int rows,
                              int d, float* dres, void* dres_c, bool accumulate, int dt, hipStream_t st,
                              int dn_splits, int64_t dn_ss) {
  if (rows <= 0) return hipSuccess;
  if (d % 4 || dn_splits < 1 || (dn_splits > 1 && dn_ss < (int64_t)rows * d)) return hipErrorInvalidValue;
  const int C = (d + 4 * NT - 1) / (4 * NT);
#define TTT_NORM_BWD(TT, CC)                                                                                       \
  TTT_LAUNCH((rmsnorm_bwd_reg_kernel<TT, CC>), dim3(rows), dim3(NT), 0, st, x, rstd, cp<TT>(g), dn, dn_splits,      \
             dn_ss, d, dres, mp<TT>(dres_c), accumulate)
  if (C <= 4) {
    if (dt == 1) {
      if (C == 1) TTT_NORM_BWD(bf16, 1); else if (C == 2) TTT_NORM_BWD(bf16, 2);
      else if (C == 3) TTT_NORM_BWD(bf16, 3); else TTT_NORM_BWD(bf16, 4);
    } else {
      if (C == 1) TTT_NORM_BWD(float, 1); else if (C == 2) TTT_NORM_BWD(float, 2);
      else if (C == 3) TTT_NORM_BWD(float, 3); else TTT_NORM_BWD(float, 4);
    }
    return hipGetLastError();
  }
#undef TTT_NORM_BWD
  DT_DISPATCH(dt,
      TTT_LAUNCH(rmsnorm_bwd_kernel<bf16>, dim3(rows), dim3(NT), 0, st, x, rstd, cp<bf16>(g), dn, dn_splits, dn_ss, d,
                 dres, mp<bf16>(dres_c), accumulate),
      TTT_LAUNCH(rmsnorm_bwd_kernel<float>, dim3(rows), dim3(NT), 0, st, x, rstd, cp<float>(g), dn, dn_splits, dn_ss,
                 d, dres, mp<float>(dres_c), accumulate));
  return hipGetLastError();
}

hipError_t rope_split_launch(const float* qkv, int rows, int S, int H, int hd, int64_t p0,
                             const float2* tab, void* q, void* kc, void* vc, int cap,
                             int64_t seq_stride, int dt, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (hd % 8) return hipErrorInvalidValue;
  DT_DISPATCH(dt,
      TTT_LAUNCH(rope_split_kernel<bf16>, dim3(rows), dim3(NT), 0, st, qkv, S, H, hd, p0, tab, mp<bf16>(q), mp<bf16>(kc), mp<bf16>(vc), cap, seq_stride),
      TTT_LAUNCH(rope_split_kernel<float>, dim3(rows), dim3(NT), 0, st, qkv, S, H, hd, p0, tab, mp<float>(q), mp<float>(kc), mp<float>(vc), cap, seq_stride));
  return hipGetLastError();
}

hipError_t rope_bwd_pack_launch(const float* dq, int nsplit, const float* dk, const float* dv, int rows, int S,
                                int H, int hd, int64_t p0, const float2* tab, void* dqkv, int dt, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (hd % 8) return hipErrorInvalidValue;
  const int64_t R = rows;
  DT_DISPATCH(dt,
      TTT_LAUNCH(rope_bwd_pack_kernel<bf16>, dim3(rows), dim3(NT), 0, st, dq, nsplit, R, dk, dv, S, H, hd, p0, tab, mp<bf16>(dqkv)),
      TTT_LAUNCH(rope_bwd_pack_kernel<float>, dim3(rows), dim3(NT), 0, st, dq, nsplit, R, dk, dv, S, H, hd, p0, tab, mp<float>(dqkv)));
  return hipGetLastError();
}

hipError_t act_fwd_launch(const float* z, int rows, int h, int64_t ldz, int glu, void* a, int64_t lda,
                          int dt, hipStream_t st) {
  if (rows <= 0 || h <= 0) return hipSuccess;
  if (h % 8 || ldz % 8 || lda % 8) return hipErrorInvalidValue;
  dim3 g((h / 8 + NT - 1) / NT, rows);
  DT_DISPATCH(dt,
      TTT_LAUNCH(act_fwd_kernel<bf16>, g, dim3(NT), 0, st, z, h, ldz, glu, mp<bf16>(a), lda),
      TTT_LAUNCH(act_fwd_kernel<float>, g, dim3(NT), 0, st, z, h, ldz, glu, mp<float>(a), lda));
  return hipGetLastError();
}

hipError_t act_bwd_launch(const float* z, const float* da, int rows, int hcols, int64_t ldz, int64_t ldda,
                          int64_t up_off, int glu, void* dz, int64_t lddz, int dt, hipStream_t st) {
  if (rows <= 0 || hcols <= 0) return hipSuccess;
  if (hcols % 8 || ldz % 8 || ldda % 8 || up_off % 8 || lddz % 8) return hipErrorInvalidValue;
  dim3 g((hcols / 8 + NT - 1) / NT, rows);
  DT_DISPATCH(dt,
      TTT_LAUNCH(act_bwd_kernel<bf16>, g, dim3(NT), 0, st, z, da, hcols, ldz, ldda, up_off, glu, mp<bf16>(dz), lddz),
      TTT_LAUNCH(act_bwd_kernel<float>, g, dim3(NT), 0, st, z, da, hcols, ldz, ldda, up_off, glu, mp<float>(dz), lddz));
  return hipGetLastError();
}

hipError_t attn_delta_launch(const void* o, const void* dout, int rows, int H, int hd, int64_t ld, int S,
                             float* delta, int dt, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (hd % 8 || hd / 8 > 64 || ((hd / 8) & (hd / 8 - 1))) return hipErrorInvalidValue;
  DT_DISPATCH(dt,
      TTT_LAUNCH(attn_delta_kernel<bf16>, dim3(rows), dim3(NT), 0, st, cp<bf16>(o), cp<bf16>(dout), H, hd, ld, S, delta),
      TTT_LAUNCH(attn_delta_kernel<float>, dim3(rows), dim3(NT), 0, st, cp<float>(o), cp<float>(dout), H, hd, ld, S, delta));
  return hipGetLastError();
}

hipError_t ce_launch(const CEArgs& a, int dt, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  if (a.V % 8 || a.V > CE_NT * CE_IT * 8) return hipErrorInvalidValue;
  DT_DISPATCH(dt,
      TTT_LAUNCH(ce_kernel<bf16>, dim3(a.rows), dim3(CE_NT), 0, st, a),
      TTT_LAUNCH(ce_kernel<float>, dim3(a.rows), dim3(CE_NT), 0, st, a));
  return hipGetLastError();
}

hipError_t transpose_launch(const void* src, int rows, int cols, int64_t lds, int sdt, void* dst, int64_t ldd,
                            int ddt, hipStream_t st, int batch, int64_t s_src, int64_t s_dst) {
  if (rows <= 0 || cols <= 0 || batch <= 0) return hipSuccess;
  dim3 g((cols + 63) / 64, (rows + 63) / 64, batch);
  const bool v8 = rows % 8 == 0 && cols % 8 == 0 && lds % 8 == 0 && ldd % 8 == 0 && s_src % 8 == 0 &&
                  s_dst % 8 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0 &&
                  reinterpret_cast<uintptr_t>(dst) % 16 == 0;
  if (v8) {
    if (sdt == 1 && ddt == 1)
      TTT_LAUNCH((transpose8_kernel<bf16, bf16>), g, dim3(256), 0, st, cp<bf16>(src), rows, cols, lds, mp<bf16>(dst), ldd, s_src, s_dst);
    else if (sdt == 1 && ddt == 0)
      TTT_LAUNCH((transpose8_kernel<bf16, float>), g, dim3(256), 0, st, cp<bf16>(src), rows, cols, lds, mp<float>(dst), ldd, s_src, s_dst);
    else if (sdt == 0 && ddt == 1)
      TTT_LAUNCH((transpose8_kernel<float, bf16>), g, dim3(256), 0, st, cp<float>(src), rows, cols, lds, mp<bf16>(dst), ldd, s_src, s_dst);
    else
      TTT_LAUNCH((transpose8_kernel<float, float>), g, dim3(256), 0, st, cp<float>(src), rows, cols, lds, mp<float>(dst), ldd, s_src, s_dst);
    return hipGetLastError();
  }
  if (sdt == 1 && ddt == 1)
    TTT_LAUNCH((transpose_kernel<bf16, bf16>), g, dim3(256), 0, st, cp<bf16>(src), rows, cols, lds, mp<bf16>(dst), ldd, s_src, s_dst);
  else if (sdt == 1 && ddt == 0)
    TTT_LAUNCH((transpose_kernel<bf16, float>), g, dim3(256), 0, st, cp<bf16>(src), rows, cols, lds, mp<float>(dst), ldd, s_src, s_dst);
  else if (sdt == 0 && ddt == 1)
    TTT_LAUNCH((transpose_kernel<float, bf16>), g, dim3(256), 0, st, cp<float>(src), rows, cols, lds, mp<bf16>(dst), ldd, s_src, s_dst);
  else
    TTT_LAUNCH((transpose_kernel<float, float>), g, dim3(256), 0, st, cp<float>(src), rows, cols, lds, mp<float>(dst), ldd, s_src, s_dst);
  return hipGetLastError();
}

hipError_t copy_rows_f32_launch(const float* src, int64_t sss, float* dst, int64_t dss, int S, int d, int B,
                                hipStream_t st) {
  if (S <= 0 || B <= 0) return hipSuccess;
  TTT_LAUNCH(copy_rows_kernel, dim3(S, B), dim3(NT), 0, st, src, sss, dst, dss, S, d);
  return hipGetLastError();
}

hipError_t fill_f32_launch(float* p, int64_t n, float v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + NT - 1) / NT;
  if (blocks > 65536) blocks = 65536;
  TTT_LAUNCH(fill_kernel, dim3((unsigned)blocks), dim3(NT), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t decode_emit_launch(const int32_t* next, const float* lse, const float* mx, int B, int vocab,
                              int32_t* ids, int64_t ids_ss, int64_t pos, int32_t* out, int64_t out_ld, int64_t i,
                              float* losses, int32_t* status, hipStream_t st) {
  TTT_LAUNCH(decode_emit_kernel, dim3(1), dim3(((B + 63) / 64) * 64), 0, st, next, lse, mx, B, vocab, ids,
                     ids_ss, pos, out, out_ld, i, losses, status);
  return hipGetLastError();
}

// Causal sliding-window attention for gfx950: flash-style forward and the
// activation-gradient backward.
//
// Query p sees key j iff p - window < j <= p (exactly min(p+1, window) keys:
// the N_window <= T*k count of Eq. 1 in the technical review "TTT-E2E:
// Learning a Long Context into Weights", section 2.1; causal masking inside
// a chunk, section 5). Keys and values live in a per-layer ring cache indexed
// by absolute position modulo `cap` (a multiple of 64), which holds the K/V
// of earlier chunks as they were computed; the current chunk writes its own
// rows before attention runs.
//
// Every product is an MFMA 32x32 tile with the query index on the lanes:
//   S^T[key][q] = K . Q^T     (K tile from LDS, Q fragments held in registers)
//   O^T[d][q]  += V^T . P^T   (V staged transposed in LDS, P from registers)
// so each lane owns one query's softmax row (two half-waves split the keys):
// the online-softmax max and sum need only one cross-half shuffle. The P
// fragments are fed to the second MFMA straight from the first one's
// accumulator registers; the keys of the 16-wide contraction are permuted
// consistently on both operands, which the sum over keys does not see.
//
// Backward (only the gradients the inner loop needs): dQ for every query over
// its whole window; dK and dV only for keys of the current chunk (cached keys
// are constants of the gradient). Two kernels, no atomics:
//   dq kernel   (query-owned):  P, dP^T = V . dO^T, dS = P (dP - delta),
//                               dQ^T += K^T . dS^T
//   dkdv kernel (key-owned):    S = Q . K^T, P, dV^T += dO^T . P,
//                               dP = dO . V^T, dK^T += Q^T . dS
#include "common.h"
#include "kernels.h"

namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr int NT = 256;
constexpr int BKEY = 64;  // key tile
constexpr int WQ = 32;    // queries (or keys) per wave
constexpr float NEG_BIG = -1e30f;

template <typename T> struct AT;
template <> struct AT<bf16> {
  static constexpr int KS = 16, PAD = 8, VEC = 8;
  typedef bf16x8 frag;
  typedef bf16x8 vec;
};
template <> struct AT<float> {
  static constexpr int KS = 2, PAD = 1, VEC = 4;
  typedef float frag;
  typedef f32x4 vec;
};

TTT_DEV f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
TTT_DEV f32x16 mfma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Number of MFMA k-steps that cover 32 keys, and the key index (0..31 in a
// 32-key accumulator tile) of fragment element e at k-step u for half-wave h.
template <typename T> struct KeyPerm;
template <> struct KeyPerm<bf16> {
  static constexpr int STEPS = 2;
  TTT_DEV static int key(int u, int h, int e) { return u * 16 + (e >> 2) * 8 + h * 4 + (e & 3); }
};
template <> struct KeyPerm<float> {
  static constexpr int STEPS = 16;
  TTT_DEV static int key(int u, int h, int) { return (u >> 2) * 8 + h * 4 + (u & 3); }
};

// accumulator register r of a 32x32 tile -> row within the tile (lane half h)
TTT_DEV int acc_row(int r, int h) { return (r >> 2) * 8 + h * 4 + (r & 3); }

// fragment of a row-major LDS tile s[row][ld] at (row, k..): rows on lanes
template <typename T>
TTT_DEV typename AT<T>::frag lds_frag(const T* s, int ld, int row, int k) {
  return *reinterpret_cast<const typename AT<T>::frag*>(s + row * ld + k);
}

// Build the fragment of a transposed LDS tile st[d][key] for MFMA A-operand
// rows d, keys permuted as KeyPerm for the 32-key group g and step u.
template <typename T>
TTT_DEV typename AT<T>::frag lds_frag_perm(const T* st, int ld, int d, int g, int u, int h) {
  typename AT<T>::frag f;
  if constexpr (sizeof(T) == 2) {
    const T* p = st + d * ld + g * 32 + u * 16 + h * 4;
    bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
    bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 8);
    f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
    f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
  } else {
    f = st[d * ld + g * 32 + KeyPerm<float>::key(u, h, 0)];
  }
  return f;
}

// B-operand fragment from accumulator registers (P or dS), step u.
template <typename T>
TTT_DEV typename AT<T>::frag acc_frag(const f32x16& acc, int u) {
  typename AT<T>::frag f;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (bf16)acc[u * 8 + e];
  } else {
    f = acc[u];
  }
  return f;
}

// Cooperative copy of `rows` rows (rows of length HD, global row stride ld)
// into LDS as row-major [rows][HD+PAD] and/or transposed [HD][rows+PAD].
// Global rows come from row_ptr(i) (nullptr = zero row).
template <typename T, int HD, int ROWS, bool ROWMAJ, bool TRANS, typename F>
TTT_DEV void stage_rows(T* s_row, T* s_tr, F row_ptr) {
  typedef AT<T> A;
  typedef typename A::vec V;
  constexpr int VPR = HD / A::VEC;
  constexpr int NV = ROWS * VPR;
  for (int vi = threadIdx.x; vi < NV; vi += NT) {
    const int r = vi / VPR, c = (vi % VPR) * A::VEC;
    const T* src = row_ptr(r);
    V v = src ? *reinterpret_cast<const V*>(src + c) : V{};
    if constexpr (ROWMAJ) *reinterpret_cast<V*>(s_row + r * (HD + A::PAD) + c) = v;
    if constexpr (TRANS) {
#pragma unroll
      for (int e = 0; e < A::VEC; ++e) s_tr[(c + e) * (ROWS + A::PAD) + r] = v[e];
    }
  }
}

// ============================== forward ==============================

template <typename T, int HD>
__global__ __launch_bounds__(NT) void attn_fwd_kernel(AttnArgs a) {
  typedef AT<T> A;
  constexpr int LDK = HD + A::PAD, LDV = BKEY + A::PAD;
  constexpr int NKS = HD / A::KS;               // k-steps over the head dim
  constexpr int DB = HD >= 32 ? HD / 32 : 1;    // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) T sK[BKEY * LDK];
  __shared__ __attribute__((aligned(16))) T sVt[HD * LDV];

  const int s = blockIdx.z, h = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hl = lane >> 5;
  const int M = a.M;
  const int qb0 = blockIdx.x * (4 * WQ);
  const int qw0 = qb0 + w * WQ;
  const int q = qw0 + (lane & 31);
  const bool qvalid = q < M;
  const int64_t pq = a.pos0 + (qvalid ? q : M - 1);
  const int64_t win = a.window;
  const T* Q = reinterpret_cast<const T*>(a.q);
  const T* Kc = reinterpret_cast<const T*>(a.kc) + s * a.seq_stride + h * a.hd;
  const T* Vc = reinterpret_cast<const T*>(a.vc) + s * a.seq_stride + h * a.hd;

  // Q fragments (B operand: query on lanes)
  typename A::frag qf[NKS];
  {
    const T* qrow = Q + ((int64_t)s * M + (qvalid ? q : 0)) * a.ldq + h * a.hd;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if constexpr (sizeof(T) == 2) {
        qf[ks] = qvalid ? *reinterpret_cast<const bf16x8*>(qrow + ks * 16 + hl * 8) : bf16x8{};
      } else {
        qf[ks] = qvalid ? qrow[ks * 2 + hl] : 0.f;
      }
    }
  }

  const int qlast_blk = min(qb0 + 4 * WQ, M) - 1;
  const int64_t lo = max((int64_t)0, a.pos0 + qb0 - win + 1);
  const int64_t hi = a.pos0 + qlast_blk;
  const int64_t j_start = lo & ~(int64_t)(BKEY - 1);
  const bool wactive = qw0 < M;
  const int64_t wfirst = a.pos0 + qw0;
  const int64_t wlast = a.pos0 + min(qw0 + WQ, M) - 1;

  const float c2 = a.scale * LOG2E;
  float m_i = NEG_BIG, l_i = 0.f;
  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x16{};

  for (int64_t j0 = j_start; j0 <= hi; j0 += BKEY) {
    __syncthreads();
    {
      auto rp = [&](int r) -> const T* {
        const int64_t j = j0 + r;
        if (j < 0 || j > hi) return nullptr;
        return Kc + (j % a.cap) * a.ldk;
      };
      stage_rows<T, HD, BKEY, true, false>(sK, nullptr, rp);
      auto rv = [&](int r) -> const T* {
        const int64_t j = j0 + r;
        if (j < 0 || j > hi) return nullptr;
        return Vc + (j % a.cap) * a.ldk;
      };
      stage_rows<T, HD, BKEY, false, true>(nullptr, sVt, rv);
    }
    __syncthreads();
    if (!wactive) continue;
    if (j0 > wlast || j0 + BKEY - 1 <= wfirst - win) continue;
    const bool full = (j0 + BKEY - 1 <= wfirst) && (j0 > wlast - win);

    f32x16 st[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      st[g] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        typename A::frag kf = lds_frag<T>(sK, LDK, g * 32 + (lane & 31), ks * A::KS + hl * (A::KS / 2));
        st[g] = mfma(kf, qf[ks], st[g]);
      }
    }
    float mx = NEG_BIG;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = st[g][r] * c2;
        if (!full) {
          const int64_t j = j0 + g * 32 + acc_row(r, hl);
          if (!(j <= pq && j > pq - win)) v = -INFINITY;
        }
        st[g][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_i, mx);
    const float alpha = exp2f(m_i - m_new);
    float rs = 0.f;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = exp2f(st[g][r] - m_new);
        st[g][r] = pv;
        rs += pv;
      }
    l_i = l_i * alpha + rs;
    m_i = m_new;
#pragma unroll
    for (int i = 0; i < DB; ++i) o[i] *= alpha;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int u = 0; u < KeyPerm<T>::STEPS; ++u) {
        typename A::frag pf = acc_frag<T>(st[g], u);
#pragma unroll
        for (int i = 0; i < DB; ++i) {
          const int d = i * 32 + (lane & 31);
          typename A::frag vf = d < HD ? lds_frag_perm<T>(sVt, LDV, d, g, u, hl) : typename A::frag{};
          o[i] = mfma(vf, pf, o[i]);
        }
      }
  }

  if (!wactive || !qvalid) return;
  const float l_tot = l_i + __shfl_xor(l_i, 32, 64);
  const float inv = 1.f / l_tot;
  T* O = reinterpret_cast<T*>(a.o) + ((int64_t)s * M + q) * a.ldo + h * a.hd;
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = i * 32 + acc_row(r, hl);
      if (d < HD) O[d] = from_f32<T>(o[i][r] * inv);
    }
  if (hl == 0) a.lse[((int64_t)s * a.H + h) * M + q] = m_i * LN2 + logf(l_tot);
}

// ============================== backward: dQ ==============================

template <typename T, int HD>
__global__ __launch_bounds__(NT) void attn_bwd_dq_kernel(AttnArgs a) {
  typedef AT<T> A;
  constexpr int LDK = HD + A::PAD, LDT = BKEY + A::PAD;
  constexpr int NKS = HD / A::KS;
  constexpr int DB = HD >= 32 ? HD / 32 : 1;
  __shared__ __attribute__((aligned(16))) T sK[BKEY * LDK];
  __shared__ __attribute__((aligned(16))) T sV[BKEY * LDK];
  __shared__ __attribute__((aligned(16))) T sKt[HD * LDT];

  const int s = blockIdx.z, h = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hl = lane >> 5;
  const int M = a.M;
  const int qb0 = blockIdx.x * (4 * WQ);
  const int qw0 = qb0 + w * WQ;
  const int q = qw0 + (lane & 31);
  const bool qvalid = q < M;
  const int64_t pq = a.pos0 + (qvalid ? q : M - 1);
  const int64_t win = a.window;
  const T* Kc = reinterpret_cast<const T*>(a.kc) + s * a.seq_stride + h * a.hd;
  const T* Vc = reinterpret_cast<const T*>(a.vc) + s * a.seq_stride + h * a.hd;

  typename A::frag qf[NKS], df[NKS];
  {
    const T* qrow = reinterpret_cast<const T*>(a.q) + ((int64_t)s * M + (qvalid ? q : 0)) * a.ldq + h * a.hd;
    const T* drow = reinterpret_cast<const T*>(a.dout) + ((int64_t)s * M + (qvalid ? q : 0)) * a.lddo + h * a.hd;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if constexpr (sizeof(T) == 2) {
        qf[ks] = qvalid ? *reinterpret_cast<const bf16x8*>(qrow + ks * 16 + hl * 8) : bf16x8{};
        df[ks] = qvalid ? *reinterpret_cast<const bf16x8*>(drow + ks * 16 + hl * 8) : bf16x8{};
      } else {
        qf[ks] = qvalid ? qrow[ks * 2 + hl] : 0.f;
        df[ks] = qvalid ? drow[ks * 2 + hl] : 0.f;
      }
    }
  }
  const int64_t li = ((int64_t)s * a.H + h) * M + (qvalid ? q : 0);
  const float lse2 = qvalid ? a.lse[li] * LOG2E : 0.f;
  const float dlt = qvalid ? a.delta[li] : 0.f;

  const int qlast_blk = min(qb0 + 4 * WQ, M) - 1;
  const int64_t lo = max((int64_t)0, a.pos0 + qb0 - win + 1);
  const int64_t hi = a.pos0 + qlast_blk;
  const int64_t j_start = lo & ~(int64_t)(BKEY - 1);
  const bool wactive = qw0 < M;
  const int64_t wfirst = a.pos0 + qw0;
  const int64_t wlast = a.pos0 + min(qw0 + WQ, M) - 1;
  const float c2 = a.scale * LOG2E;

  f32x16 dq[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dq[i] = f32x16{};

  for (int64_t j0 = j_start; j0 <= hi; j0 += BKEY) {
    __syncthreads();
    {
      auto rk = [&](int r) -> const T* {
        const int64_t j = j0 + r;
        if (j < 0 || j > hi) return nullptr;
        return Kc + (j % a.cap) * a.ldk;
      };
      stage_rows<T, HD, BKEY, true, true>(sK, sKt, rk);
      auto rv = [&](int r) -> const T* {
        const int64_t j = j0 + r;
        if (j < 0 || j > hi) return nullptr;
        return Vc + (j % a.cap) * a.ldk;
      };
      stage_rows<T, HD, BKEY, true, false>(sV, nullptr, rv);
    }
    __syncthreads();
    if (!wactive) continue;
    if (j0 > wlast || j0 + BKEY - 1 <= wfirst - win) continue;
    const bool full = (j0 + BKEY - 1 <= wfirst) && (j0 > wlast - win);

    f32x16 p[2], dp[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      p[g] = f32x16{};
      dp[g] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int row = g * 32 + (lane & 31), kk = ks * A::KS + hl * (A::KS / 2);
        p[g] = mfma(lds_frag<T>(sK, LDK, row, kk), qf[ks], p[g]);
        dp[g] = mfma(lds_frag<T>(sV, LDK, row, kk), df[ks], dp[g]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float sv = p[g][r] * c2;
        if (!full) {
          const int64_t j = j0 + g * 32 + acc_row(r, hl);
          if (!(j <= pq && j > pq - win)) sv = -INFINITY;
        }
        const float pr = exp2f(sv - lse2);
        p[g][r] = pr * (dp[g][r] - dlt);  // dS
      }
    }
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int u = 0; u < KeyPerm<T>::STEPS; ++u) {
        typename A::frag sf = acc_frag<T>(p[g], u);
#pragma unroll
        for (int i = 0; i < DB; ++i) {
          const int d = i * 32 + (lane & 31);
          typename A::frag kf = d < HD ? lds_frag_perm<T>(sKt, LDT, d, g, u, hl) : typename A::frag{};
          dq[i] = mfma(kf, sf, dq[i]);
        }
      }
  }
  if (!wactive || !qvalid) return;
  float* out = a.dq + ((int64_t)s * M + q) * a.lddq + h * a.hd;
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = i * 32 + acc_row(r, hl);
      if (d < HD) out[d] = dq[i][r] * a.scale;
    }
}

// ============================== backward: dK, dV ==============================

constexpr int BQT = 64;  // query tile of the key-owned kernel

template <typename T, int HD>
__global__ __launch_bounds__(NT) void attn_bwd_dkdv_kernel(AttnArgs a) {
  typedef AT<T> A;
  constexpr int LDR = HD + A::PAD, LDT = BQT + A::PAD;
  constexpr int NKS = HD / A::KS;
  constexpr int DB = HD >= 32 ? HD / 32 : 1;
  __shared__ __attribute__((aligned(16))) T sQ[BQT * LDR];
  __shared__ __attribute__((aligned(16))) T sD[BQT * LDR];
  __shared__ __attribute__((aligned(16))) T sQt[HD * LDT];
  __shared__ __attribute__((aligned(16))) T sDt[HD * LDT];
  __shared__ float sL[BQT], sDl[BQT];

  const int s = blockIdx.z, h = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hl = lane >> 5;
  const int M = a.M;
  const int kb0 = blockIdx.x * (4 * WQ);
  const int kw0 = kb0 + w * WQ;
  const int kr = kw0 + (lane & 31);     // key row within the chunk
  const bool kvalid = kr < M;
  const int64_t pk = a.pos0 + (kvalid ? kr : M - 1);
  const int64_t win = a.window;
  const T* Kc = reinterpret_cast<const T*>(a.kc) + s * a.seq_stride + h * a.hd;
  const T* Vc = reinterpret_cast<const T*>(a.vc) + s * a.seq_stride + h * a.hd;
  const T* Q = reinterpret_cast<const T*>(a.q) + (int64_t)s * M * a.ldq + h * a.hd;
  const T* DO = reinterpret_cast<const T*>(a.dout) + (int64_t)s * M * a.lddo + h * a.hd;

  typename A::frag kf[NKS], vf[NKS];
  {
    const T* krow = Kc + (pk % a.cap) * a.ldk;
    const T* vrow = Vc + (pk % a.cap) * a.ldk;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if constexpr (sizeof(T) == 2) {
        kf[ks] = kvalid ? *reinterpret_cast<const bf16x8*>(krow + ks * 16 + hl * 8) : bf16x8{};
        vf[ks] = kvalid ? *reinterpret_cast<const bf16x8*>(vrow + ks * 16 + hl * 8) : bf16x8{};
      } else {
        kf[ks] = kvalid ? krow[ks * 2 + hl] : 0.f;
        vf[ks] = kvalid ? vrow[ks * 2 + hl] : 0.f;
      }
    }
  }
  const float c2 = a.scale * LOG2E;
  const int klast_blk = min(kb0 + 4 * WQ, M) - 1;
  const bool wactive = kw0 < M;
  const int wk_first = kw0, wk_last = min(kw0 + WQ, M) - 1;
  // queries (rows) that can see keys of this block: [kb0, klast_blk + win - 1]
  const int q_end = (int)min((int64_t)M, (int64_t)klast_blk + win);
  const int q_start = kb0 & ~(BQT - 1);

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) { dk[i] = f32x16{}; dv[i] = f32x16{}; }

  for (int q0 = q_start; q0 < q_end; q0 += BQT) {
    __syncthreads();
    {
      auto rq = [&](int r) -> const T* {
        const int qi = q0 + r;
        return qi < M ? Q + (int64_t)qi * a.ldq : nullptr;
      };
      stage_rows<T, HD, BQT, true, true>(sQ, sQt, rq);
      auto rd = [&](int r) -> const T* {
        const int qi = q0 + r;
        return qi < M ? DO + (int64_t)qi * a.lddo : nullptr;
      };
      stage_rows<T, HD, BQT, true, true>(sD, sDt, rd);
      for (int r = threadIdx.x; r < BQT; r += NT) {
        const int qi = q0 + r;
        const int64_t li = ((int64_t)s * a.H + h) * M + qi;
        sL[r] = qi < M ? a.lse[li] * LOG2E : 0.f;
        sDl[r] = qi < M ? a.delta[li] : 0.f;
      }
    }
    __syncthreads();
    if (!wactive) continue;
    // does any (query in tile, key in wave) pair satisfy pk <= pq < pk + win ?
    if (q0 + BQT - 1 < wk_first || q0 > wk_last + win - 1) continue;

    f32x16 p[2], dp[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {   // 32-query groups of the tile
      p[g] = f32x16{};
      dp[g] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int row = g * 32 + (lane & 31), kk = ks * A::KS + hl * (A::KS / 2);
        p[g] = mfma(lds_frag<T>(sQ, LDR, row, kk), kf[ks], p[g]);
        dp[g] = mfma(lds_frag<T>(sD, LDR, row, kk), vf[ks], dp[g]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = g * 32 + acc_row(r, hl);
        const int qi = q0 + qr;
        const int64_t pq = a.pos0 + qi;
        float sv = p[g][r] * c2;
        if (!(kvalid && qi < M && pk <= pq && pk > pq - win)) sv = -INFINITY;
        const float pr = exp2f(sv - sL[qr]);
        p[g][r] = pr;
        dp[g][r] = pr * (dp[g][r] - sDl[qr]);  // dS
      }
    }
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int u = 0; u < KeyPerm<T>::STEPS; ++u) {
        typename A::frag pf = acc_frag<T>(p[g], u);
        typename A::frag sf = acc_frag<T>(dp[g], u);
#pragma unroll
        for (int i = 0; i < DB; ++i) {
          const int d = i * 32 + (lane & 31);
          typename A::frag dof = d < HD ? lds_frag_perm<T>(sDt, LDT, d, g, u, hl) : typename A::frag{};
          typename A::frag qtf = d < HD ? lds_frag_perm<T>(sQt, LDT, d, g, u, hl) : typename A::frag{};
          dv[i] = mfma(dof, pf, dv[i]);
          dk[i] = mfma(qtf, sf, dk[i]);
        }
      }
  }
  if (!wactive || !kvalid) return;
  float* dko = a.dk + ((int64_t)s * M + kr) * a.lddk + h * a.hd;
  float* dvo = a.dv + ((int64_t)s * M + kr) * a.lddk + h * a.hd;
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = i * 32 + acc_row(r, hl);
      if (d < HD) {
        dko[d] = dk[i][r] * a.scale;
        dvo[d] = dv[i][r];
      }
    }
}

template <typename T, int HD>
hipError_t fwd_t(const AttnArgs& a, hipStream_t st) {
  dim3 grid((a.M + 4 * WQ - 1) / (4 * WQ), a.H, a.B);
  hipLaunchKernelGGL((attn_fwd_kernel<T, HD>), grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}
template <typename T, int HD>
hipError_t bwd_t(const AttnArgs& a, hipStream_t st) {
  dim3 grid((a.M + 4 * WQ - 1) / (4 * WQ), a.H, a.B);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, HD>), grid, dim3(NT), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, HD>), grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace

// head dims: bf16 16..128, fp32 16..64 (fp32 tiles above 64 exceed the LDS budget)
#define TTT_HD_SWITCH(FN)                                                   \
  if (dt == 1) {                                                            \
    switch (a.hd) {                                                         \
      case 16: return FN<bf16, 16>(a, st);                                  \
      case 32: return FN<bf16, 32>(a, st);                                  \
      case 64: return FN<bf16, 64>(a, st);                                  \
      case 128: return FN<bf16, 128>(a, st);                                \
    }                                                                       \
  } else {                                                                  \
    switch (a.hd) {                                                         \
      case 16: return FN<float, 16>(a, st);                                 \
      case 32: return FN<float, 32>(a, st);                                 \
      case 64: return FN<float, 64>(a, st);                                 \
    }                                                                       \
  }                                                                         \
  return hipErrorInvalidValue;

hipError_t attn_fwd_launch(const AttnArgs& a, int dt, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  TTT_HD_SWITCH(fwd_t)
}

hipError_t attn_bwd_launch(const AttnArgs& a, int dt, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  TTT_HD_SWITCH(bwd_t)
}

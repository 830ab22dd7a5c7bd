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
//   S^T[key][q] = K . Q^T     (K fragments from LDS, Q fragments in registers)
//   O^T[d][q]  += V^T . P^T   (V^T fragments from LDS, P from registers)
// so each lane owns one query's softmax row (two half-waves split the keys):
// the online-softmax max and sum need one cross-half shuffle. P is fed to the
// second MFMA straight from the first one's accumulator registers; the keys
// of the 16-wide contraction are permuted consistently on both operands,
// which the sum over keys does not see. All tiles sit in LDS row-major
// (copied with 16-byte loads and stores, double-buffered so the next tile's
// global loads overlap the current tile's MFMAs); operands that need the
// transposed view (V^T, K^T, Q^T, dO^T) are read with gfx950's transposing
// LDS read ds_read_b64_tr_b16 (fp32: plain reads, one element per lane).
//
// Backward (only the gradients the inner loop needs): dQ for every query over
// its whole window; dK and dV only for keys of the current chunk (cached keys
// are constants of the gradient). Two kernels, no atomics:
//   dq kernel   (query-owned):  P, dP^T = V . dO^T, dS = P (dP - delta),
//                               dQ^T += K^T . dS^T
//   dkdv kernel (key-owned):    S = Q . K^T, P, dV^T += dO^T . P,
//                               dP = dO . V^T, dK^T += Q^T . dS
// When few queries are in flight (a chunk of b rows), the forward and the dq
// kernel split each query block's key range over several workgroups
// ("splits"); partial results are merged in a fixed order.
#include "common.h"
#include "kernels.h"

namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr int NT = 256;
constexpr int BKEY = 64;  // key tile
constexpr int WQ = 32;    // queries (or keys) per wave
constexpr int QB = 4 * WQ;  // queries per workgroup
constexpr float NEG_BIG = -1e30f;
// The running row max of the online softmax is raised only when a tile's max
// exceeds it by more than RESCALE_SLACK (log2 units): probabilities are then
// bounded by 2^RESCALE_SLACK and the O accumulators are rescaled rarely.
constexpr float RESCALE_SLACK = 8.f;

// 2^x with the hardware instruction (flushes results below 2^-126 to zero,
// which a softmax weight never needs)
TTT_DEV float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T> struct AT;
// Row padding of the LDS tiles: PADR for tiles read only row-wise (16-byte
// fragment reads, conflict-free at a stride of 4 mod 64 dwords), PADT for
// tiles also read transposed (a 16-lane transposing read touches 4 rows, which
// a stride of 8 mod 64 dwords spreads over distinct banks).
template <> struct AT<bf16> {
  static constexpr int KS = 16, PADR = 8, PADT = 16, VEC = 8;
  typedef bf16x8 frag;
  typedef bf16x8 vec;
};
template <> struct AT<float> {
  static constexpr int KS = 2, PADR = 1, PADT = 1, VEC = 4;
  typedef float frag;
  typedef f32x4 vec;
};

TTT_DEV f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
TTT_DEV f32x16 mfma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Number of MFMA k-steps that cover 32 keys.
template <typename T> struct KSteps;
template <> struct KSteps<bf16> { static constexpr int N = 2; };
template <> struct KSteps<float> { static constexpr int N = 16; };

// accumulator register r of a 32x32 tile -> row within the tile (lane half h)
TTT_DEV int acc_row(int r, int h) { return (r >> 2) * 8 + h * 4 + (r & 3); }

// fragment (rows on lanes, KS consecutive k) of a row-major LDS tile s[row][ld]
template <typename T>
TTT_DEV typename AT<T>::frag lds_frag(const T* s, int ld, int row, int k) {
  return *reinterpret_cast<const typename AT<T>::frag*>(s + row * ld + k);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Fragment of the TRANSPOSED view of a row-major LDS tile s[key][d]: MFMA
// operand rows = d (d0 .. d0+31 on the lanes), contraction over the 32 keys
// of group g at k-step u, in the key order of the accumulator registers
// (key(u, h, e) = 16u + 8*(e/4) + 4h + e%4 for bf16; (u/4)*8 + 4h + u%4 fp32).
// bf16: two ds_read_b64_tr_b16. Within a 16-lane group a transposing read
// returns to lane i element e the (i%4)-th 16-bit value at the address of
// lane i/4 + 4e, so lane X supplies the 4 values of key row
// (base + 8r + (X%16)/4), columns d0 + 16*((X/16)%2) + 4*(X%4) .. +3.
template <typename T>
TTT_DEV typename AT<T>::frag lds_frag_tr(const T* s, int ld, int d0, int g, int u, int lane, int dmax) {
  typename AT<T>::frag f;
  if constexpr (sizeof(T) == 2) {
    const int h = lane >> 5;
    const int key = g * 32 + u * 16 + h * 4 + ((lane & 15) >> 2);
    const int col = d0 + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
    typedef __attribute__((address_space(3))) s16x4 lds_v4;
    // generic -> LDS address-space casts (the tiles live in __shared__ memory)
    lds_v4* p0 = (lds_v4*)(T*)(s + key * ld + col);
    lds_v4* p1 = (lds_v4*)(T*)(s + (key + 8) * ld + col);
    s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p0);
    s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p1);
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 v;
    v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
    v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
    f = __builtin_bit_cast(bf16x8, v);
  } else {
    const int h = lane >> 5;
    const int key = g * 32 + (u >> 2) * 8 + h * 4 + (u & 3);
    const int d = d0 + (lane & 31);
    f = d < dmax ? s[key * ld + d] : 0.f;
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

// Registers holding one ROWS x HD tile between its global load and its LDS
// store (LDS row stride LD). Rows r < nvalid come from base + r*ld, the others
// are zero.
template <typename T, int HD, int ROWS, int LD>
struct Stage {
  typedef AT<T> A;
  typedef typename A::vec V;
  static constexpr int VPR = HD / A::VEC;
  static constexpr int NV = (ROWS * VPR + NT - 1) / NT;
  V v[NV];
  TTT_DEV void load(const T* base, int64_t ld, int nvalid) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = i * NT + threadIdx.x;
      if (vi < ROWS * VPR) {
        const int r = vi / VPR;
        v[i] = r < nvalid ? *reinterpret_cast<const V*>(base + r * ld + (vi % VPR) * A::VEC) : V{};
      }
    }
  }
  TTT_DEV void store(T* s) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = i * NT + threadIdx.x;
      if (vi < ROWS * VPR)
        *reinterpret_cast<V*>(s + (vi / VPR) * LD + (vi % VPR) * A::VEC) = v[i];
    }
  }
};

// Workgroup coordinates with an XCD-aware remap. Workgroups go round-robin to
// the 8 XCDs in launch order (x fastest); the query (or key) blocks of one
// head and split are consecutive in x and read the same K/V, so each XCD is
// given a contiguous run of logical workgroups and those blocks share its L2.
struct Blk { int x, y, z; };
TTT_DEV Blk blk() {
  const int nx = gridDim.x, ny = gridDim.y, n = nx * ny * gridDim.z;
  int p = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  if ((n & 7) == 0) p = (p & 7) * (n >> 3) + (p >> 3);
  Blk b;
  b.x = p % nx;
  b.y = (p / nx) % ny;
  b.z = p / (nx * ny);
  return b;
}

// key-tile range [jb, je) (positions, multiples of BKEY) of split `sp`
TTT_DEV void split_range(int j_start, int hi, int nsplit, int sp, int* jb, int* je) {
  const int ntiles = (hi - j_start) / BKEY + 1;
  const int per = (ntiles + nsplit - 1) / nsplit;
  const int t0 = min(ntiles, per * sp), t1 = min(ntiles, per * (sp + 1));
  *jb = j_start + t0 * BKEY;
  *je = j_start + t1 * BKEY;  // exclusive
}

// ============================== forward ==============================

template <typename T, int HD>
__global__ __launch_bounds__(NT, 2) void attn_fwd_kernel(AttnArgs a) {
  typedef AT<T> A;
  constexpr int LDK = HD + A::PADR, LDV = HD + A::PADT;
  constexpr int NKS = HD / A::KS;               // k-steps over the head dim
  constexpr int DB = HD >= 32 ? HD / 32 : 1;    // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) T sK[2][BKEY * LDK];
  __shared__ __attribute__((aligned(16))) T sV[2][BKEY * LDV];

  const int nsplit = a.nsplit > 0 ? a.nsplit : 1;
  const Blk bk = blk();
  const int s = bk.z / nsplit, sp = bk.z % nsplit, h = bk.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hl = lane >> 5;
  const int M = a.M;
  const int qb0 = bk.x * QB;
  const int qw0 = qb0 + w * WQ;
  const int q = qw0 + (lane & 31);
  const bool qvalid = q < M;
  const int pos0 = (int)a.pos0;                // positions fit in 31 bits
  const int pq = pos0 + (qvalid ? q : M - 1);
  const int win = a.window;
  const T* Kc = reinterpret_cast<const T*>(a.kc) + s * a.seq_stride + h * a.hd;
  const T* Vc = reinterpret_cast<const T*>(a.vc) + s * a.seq_stride + h * a.hd;

  typename A::frag qf[NKS];
  {
    const T* qrow = reinterpret_cast<const T*>(a.q) + ((int64_t)s * M + (qvalid ? q : 0)) * a.ldq + h * a.hd;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if constexpr (sizeof(T) == 2)
        qf[ks] = qvalid ? *reinterpret_cast<const bf16x8*>(qrow + ks * 16 + hl * 8) : bf16x8{};
      else
        qf[ks] = qvalid ? qrow[ks * 2 + hl] : 0.f;
    }
  }

  const int qlast_blk = min(qb0 + QB, M) - 1;
  const int lo = max(0, pos0 + qb0 - win + 1);
  const int hi = pos0 + qlast_blk;
  int jb, je;
  split_range(lo & ~(BKEY - 1), hi, nsplit, sp, &jb, &je);
  const bool wactive = qw0 < M;
  const int wfirst = pos0 + qw0;
  const int wlast = pos0 + min(qw0 + WQ, M) - 1;

  const float c2 = a.scale * LOG2E;
  float m_i = NEG_BIG, l_i = 0.f;
  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x16{};

  Stage<T, HD, BKEY, LDK> stK;
  Stage<T, HD, BKEY, LDV> stV;
  // a 64-aligned key tile occupies consecutive ring slots (cap % 64 == 0)
  auto load_tile = [&](int j0) {
    const int64_t off = (int64_t)(j0 % a.cap) * a.ldk;
    const int nvalid = min(BKEY, hi - j0 + 1);
    stK.load(Kc + off, a.ldk, nvalid);
    stV.load(Vc + off, a.ldk, nvalid);
  };
  if (jb < je) {
    load_tile(jb);
    stK.store(sK[0]);
    stV.store(sV[0]);
  }
  __syncthreads();

  int buf = 0;
  for (int j0 = jb; j0 < je; j0 += BKEY, buf ^= 1) {
    const bool more = j0 + BKEY < je;
    if (more) load_tile(j0 + BKEY);
    const T* cK = sK[buf];
    const T* cV = sV[buf];
    if (wactive && !(j0 > wlast || j0 + BKEY - 1 <= wfirst - win)) {
      const bool full = (j0 + BKEY - 1 <= wfirst) && (j0 > wlast - win);
      // S^T for the two 32-key groups: the two accumulation chains interleave
      // and the K fragments of step ks+1 are read while step ks multiplies
      f32x16 st[2] = {f32x16{}, f32x16{}};
      {
        typename A::frag kf[2][2];
        const int kr = lane & 31, kc = hl * (A::KS / 2);
        kf[0][0] = lds_frag<T>(cK, LDK, kr, kc);
        kf[0][1] = lds_frag<T>(cK, LDK, 32 + kr, kc);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          if (ks + 1 < NKS) {
            kf[(ks + 1) & 1][0] = lds_frag<T>(cK, LDK, kr, (ks + 1) * A::KS + kc);
            kf[(ks + 1) & 1][1] = lds_frag<T>(cK, LDK, 32 + kr, (ks + 1) * A::KS + kc);
          }
          st[0] = mfma(kf[ks & 1][0], qf[ks], st[0]);
          st[1] = mfma(kf[ks & 1][1], qf[ks], st[1]);
        }
      }
      if (!full) {
        // visible iff pq - win < j <= pq, i.e. 0 <= pq - j < win
        const int dj = pq - (j0 + hl * 4);
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const unsigned t = (unsigned)(dj - g * 32 - (r >> 2) * 8 - (r & 3));
            if (t >= (unsigned)win) st[g][r] = -INFINITY;
          }
      }
      // max of the raw scores, then one fma per score into exp2
      float mx = -INFINITY;
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[g][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c2;
      if (__any(mx > m_i + RESCALE_SLACK)) {   // wave-uniform branch
        const float m_new = fmaxf(m_i, mx);
        const float alpha = ex2(m_i - m_new);
        l_i *= alpha;
        m_i = m_new;
#pragma unroll
        for (int i = 0; i < DB; ++i) o[i] *= alpha;
      }
      float rs = 0.f;
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = ex2(fmaf(st[g][r], c2, -m_i));
          st[g][r] = pv;
          rs += pv;
        }
      l_i += rs;
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int u = 0; u < KSteps<T>::N; ++u) {
          // all V^T fragments of this key step first, then their MFMAs
          typename A::frag vf[DB];
#pragma unroll
          for (int i = 0; i < DB; ++i)
            vf[i] = (i * 32 < HD) ? lds_frag_tr<T>(cV, LDV, i * 32, g, u, lane, HD) : typename A::frag{};
          typename A::frag pf = acc_frag<T>(st[g], u);
#pragma unroll
          for (int i = 0; i < DB; ++i) o[i] = mfma(vf[i], pf, o[i]);
        }
    }
    if (more) {
      stK.store(sK[buf ^ 1]);
      stV.store(sV[buf ^ 1]);
    }
    __syncthreads();
  }

  if (!wactive || !qvalid) return;
  const float l_tot = l_i + __shfl_xor(l_i, 32, 64);
  if (nsplit == 1) {
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
  } else {
    // partial: normalized O_s (fp32), row max (log2 units) and row sum
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t row = (int64_t)s * M + q;
    float* O = a.part_o + ((int64_t)sp * a.B * M + row) * a.ldo + h * a.hd;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = i * 32 + acc_row(r, hl);
        if (d < HD) O[d] = o[i][r] * inv;
      }
    if (hl == 0) {
      const int64_t li = (((int64_t)sp * a.B + s) * a.H + h) * M + q;
      a.part_m[li] = m_i;
      a.part_l[li] = l_tot;
    }
  }
}

// ---- forward, bf16 with head dim 128: direct-to-LDS tiles, pipelined scores ----
// The same computation as attn_fwd_kernel with three changes:
//  * K and V tiles go from global memory straight into LDS (global_load_lds,
//    16 bytes per lane): no staging registers, no per-element copy code. The
//    rows are unpadded (256 bytes); their 16-byte chunks are XOR-swizzled
//    (fd_swz) so that K's row-wise fragment reads and V's transposing reads
//    hit distinct banks.
//  * Keys past the last query of the block are read as stored: their scores
//    are masked to -inf, so their weights are exactly 0; the caches hold
//    finite values, so 0 * V adds nothing.
//  * K and V have separate two-slot rings. Iteration t multiplies S(t+1) =
//    K(t+1) Q^T while it exponentiates tile t (one basic block, so the
//    scheduler interleaves the MFMAs with the softmax VALU work), then
//    accumulates V(t)^T P(t)^T. Its loads (K(t+2), V(t+1)) overlap the whole
//    iteration.
constexpr int FD_HD = 128;
typedef __attribute__((address_space(3))) void fd_lds_t;

// Row r of a tile keeps its 16-byte chunk c at chunk c ^ swz<Z>(r):
//  Z = 0: r % 16, for tiles read row-wise (a 16-lane fragment read takes one
//         chunk of 16 consecutive rows);
//  Z = 1: 4 (r % 4), for tiles read transposed (a 16-lane transposing read
//         takes 2 chunks of 4 consecutive rows, 4-aligned);
//  Z = 2: 4 (r % 4) + (r / 4) % 4, for tiles read both ways (a bijection on
//         16 consecutive rows that also keeps the 4-row groups apart).
template <int Z>
TTT_DEV int fd_swz(int r) {
  if constexpr (Z == 0) return r & 15;
  else if constexpr (Z == 1) return (r & 3) << 2;
  else return ((r & 3) << 2) | ((r >> 2) & 3);
}

// this wave's 4 of the 16 one-KB loads of a 64-row tile whose row 0 is `base`:
// load i of wave w fills LDS bytes [1 KB (4w + i), +1 KB), rows 4(4w+i) ..
// +3; `off` holds each lane's element offset from `base` (swizzled chunk)
TTT_DEV void fd_issue(const bf16* base, const uint32_t (&off)[4], bf16* tile, int w) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(base + off[i]), (fd_lds_t*)(tile + (w * 4 + i) * 512), 16, 0, 0);
}
template <int Z>
TTT_DEV void fd_offsets(int64_t ld, int w, int lane, uint32_t (&off)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (w * 4 + i) * 4 + (lane >> 4);
    const int c = (lane & 15) ^ fd_swz<Z>(r);
    off[i] = (uint32_t)(r * ld + c * 8);
  }
}

// wait until none of this wave's vector-memory loads (LDS-DMA included) is in flight
TTT_DEV void fd_wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// row-wise fragment: row r, 8 elements from chunk c
template <int Z>
TTT_DEV bf16x8 fd_frag(const bf16* t, int r, int c) {
  return *reinterpret_cast<const bf16x8*>(t + r * FD_HD + ((c ^ fd_swz<Z>(r)) << 3));
}

// transposed-view fragment (see lds_frag_tr) of a swizzled tile
template <int Z>
TTT_DEV bf16x8 fd_frag_tr(const bf16* t, int d0, int g, int u, int lane) {
  const int key = g * 32 + u * 16 + (lane >> 5) * 4 + ((lane & 15) >> 2);
  const int col = d0 + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
  const int c = col >> 3;
  const int o0 = key * FD_HD + ((c ^ fd_swz<Z>(key)) << 3) + (col & 7);
  const int o1 = (key + 8) * FD_HD + ((c ^ fd_swz<Z>(key + 8)) << 3) + (col & 7);
  typedef __attribute__((address_space(3))) s16x4 lds_v4;
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(bf16*)(t + o0));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(bf16*)(t + o1));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  return __builtin_bit_cast(bf16x8, v);
}

__global__ __launch_bounds__(NT, 2) void attn_fwd_dl_kernel(AttnArgs a) {
  constexpr int NKS = FD_HD / 16, DB = FD_HD / 32;
  // K and V slots in one array. With an array per operand the compiler gives
  // each its own alias scope and then waits for every LDS-DMA load in flight
  // (vmcnt(0)) before each LDS read of that operand, which drains the step's
  // prefetch; the kernel's own waits and barriers order every slot it reads.
  __shared__ __attribute__((aligned(1024))) bf16 sKV[4][BKEY * FD_HD];
  bf16(*const sK)[BKEY * FD_HD] = sKV;
  bf16(*const sV)[BKEY * FD_HD] = sKV + 2;

  const int nsplit = a.nsplit > 0 ? a.nsplit : 1;
  const Blk bk = blk();
  const int s = bk.z / nsplit, sp = bk.z % nsplit, h = bk.y;
  const int lane = threadIdx.x & 63, hl = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int M = a.M;
  const int qb0 = bk.x * QB;
  const int qw0 = qb0 + w * WQ;
  const int q = qw0 + (lane & 31);
  const bool qvalid = q < M;
  const int pos0 = (int)a.pos0;
  const int pq = pos0 + (qvalid ? q : M - 1);
  const int win = a.window;
  const bf16* Kc = reinterpret_cast<const bf16*>(a.kc) + s * a.seq_stride + h * FD_HD;
  const bf16* Vc = reinterpret_cast<const bf16*>(a.vc) + s * a.seq_stride + h * FD_HD;

  bf16x8 qf[NKS];
  {
    const bf16* qrow = reinterpret_cast<const bf16*>(a.q) + ((int64_t)s * M + (qvalid ? q : 0)) * a.ldq + h * FD_HD;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = qvalid ? *reinterpret_cast<const bf16x8*>(qrow + ks * 16 + hl * 8) : bf16x8{};
  }

  const int qlast_blk = min(qb0 + QB, M) - 1;
  const int lo = max(0, pos0 + qb0 - win + 1);
  const int hi = pos0 + qlast_blk;
  int jb, je;
  split_range(lo & ~(BKEY - 1), hi, nsplit, sp, &jb, &je);
  const int nt = (je - jb) / BKEY;
  const bool wactive = qw0 < M;
  const int wfirst = pos0 + qw0;
  const int wlast = pos0 + min(qw0 + WQ, M) - 1;

  const float c2 = a.scale * LOG2E;
  float m_i = NEG_BIG, l_i = 0.f;
  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x16{};

  // a 64-aligned key tile occupies 64 consecutive ring slots (cap % 64 == 0);
  // tile t starts at ring row (jb + 64 t) mod cap, and nt * 64 <= cap
  uint32_t koff[4], voff[4];
  fd_offsets<0>(a.ldk, w, lane, koff);
  fd_offsets<1>(a.ldk, w, lane, voff);
  const int r0 = jb % a.cap;
  auto row = [&](int t) {
    const int r = r0 + t * BKEY;
    return (int64_t)(r >= a.cap ? r - a.cap : r) * a.ldk;
  };
  auto scores = [&](const bf16* cK, f32x16 (&st)[2]) {
    st[0] = f32x16{};
    st[1] = f32x16{};
    const int kr = lane & 31;
    bf16x8 kf[2][2];
    kf[0][0] = fd_frag<0>(cK, kr, hl);
    kf[0][1] = fd_frag<0>(cK, 32 + kr, hl);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (ks + 1 < NKS) {
        kf[(ks + 1) & 1][0] = fd_frag<0>(cK, kr, (ks + 1) * 2 + hl);
        kf[(ks + 1) & 1][1] = fd_frag<0>(cK, 32 + kr, (ks + 1) * 2 + hl);
      }
      st[0] = mfma(kf[ks & 1][0], qf[ks], st[0]);
      st[1] = mfma(kf[ks & 1][1], qf[ks], st[1]);
    }
  };
  // one key tile: cur = S(t) in, nxt = S(t+1) out
  auto step = [&](int t, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
    // this wave's loads of K(t+1) and V(t) are the only ones in flight; after
    // the barrier every wave's are in LDS and K(t) / V(t-1) are no longer read
    fd_wait_loads();
    __syncthreads();
    if (t + 2 < nt) fd_issue(Kc + row(t + 2), koff, sK[t & 1], w);
    if (t + 1 < nt) fd_issue(Vc + row(t + 1), voff, sV[(t + 1) & 1], w);
    if (!wactive) return;
    const int j0 = jb + t * BKEY;
    // masking and the running max of tile t
    if (!((j0 + BKEY - 1 <= wfirst) && (j0 > wlast - win))) {
      // visible iff pq - win < j <= pq, i.e. 0 <= pq - j < win
      const int dj = pq - (j0 + hl * 4);
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const unsigned tt = (unsigned)(dj - g * 32 - (r >> 2) * 8 - (r & 3));
          if (tt >= (unsigned)win) cur[g][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, cur[g][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c2;
    if (__any(mx > m_i + RESCALE_SLACK)) {   // wave-uniform branch
      const float m_new = fmaxf(m_i, mx);
      const float alpha = ex2(m_i - m_new);
      l_i *= alpha;
      m_i = m_new;
#pragma unroll
      for (int i = 0; i < DB; ++i) o[i] *= alpha;
    }
    // S(t+1) (the last step computes an unused one from a stale slot)
    // alongside the exponentials of tile t
    scores(sK[(t + 1) & 1], nxt);
    bf16x8 pf[2][2];
    float rs = 0.f;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = ex2(fmaf(cur[g][u * 8 + e], c2, -m_i));
          rs += pv;
          pf[g][u][e] = (bf16)pv;
        }
    l_i += rs;
    const bf16* cV = sV[t & 1];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8 vf[DB];
#pragma unroll
        for (int i = 0; i < DB; ++i) vf[i] = fd_frag_tr<1>(cV, i * 32, g, u, lane);
#pragma unroll
        for (int i = 0; i < DB; ++i) o[i] = mfma(vf[i], pf[g][u], o[i]);
      }
  };

  f32x16 sa[2], sb[2];
  if (nt > 0) {
    fd_issue(Kc + row(0), koff, sK[0], w);
    fd_issue(Vc + row(0), voff, sV[0], w);
    if (nt > 1) fd_issue(Kc + row(1), koff, sK[1], w);
    fd_wait_loads();
    __syncthreads();
    if (wactive) scores(sK[0], sa);
  }
  // two steps per trip, so the score tiles swap roles without copies
  for (int t = 0; t < nt; t += 2) {
    step(t, sa, sb);
    if (t + 1 < nt) step(t + 1, sb, sa);
  }

  if (!wactive || !qvalid) return;
  const float l_tot = l_i + __shfl_xor(l_i, 32, 64);
  if (nsplit == 1) {
    const float inv = 1.f / l_tot;
    bf16* O = reinterpret_cast<bf16*>(a.o) + ((int64_t)s * M + q) * a.ldo + h * FD_HD;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) O[i * 32 + acc_row(r, hl)] = from_f32<bf16>(o[i][r] * inv);
    if (hl == 0) a.lse[((int64_t)s * a.H + h) * M + q] = m_i * LN2 + logf(l_tot);
  } else {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t row = (int64_t)s * M + q;
    float* O = a.part_o + ((int64_t)sp * a.B * M + row) * a.ldo + h * FD_HD;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) O[i * 32 + acc_row(r, hl)] = o[i][r] * inv;
    if (hl == 0) {
      const int64_t li = (((int64_t)sp * a.B + s) * a.H + h) * M + q;
      a.part_m[li] = m_i;
      a.part_l[li] = l_tot;
    }
  }
}

// Forward for a few queries (decode; the last rows of a prefill), bf16, head
// dim 128: one workgroup per (query, head, sequence, key split) streams the
// split's K and V rows from the ring once. A row is 256 bytes, one 16-byte
// load per lane of a 16-lane group, so a wave reads 4 keys per instruction
// and the 16 groups of a workgroup take keys jb + g, jb + g + 16, ... Each
// group keeps its own online softmax (max in log2 units, sum, 128 output
// columns over its 16 lanes); the groups are merged through LDS at the end.
// Outputs as the tile kernels: o and lse, or the split partials (normalised
// O, max, sum) that attn_combine_head_kernel merges.
constexpr int ONE_MAXM = 8;  // queries per sequence served by this kernel
constexpr int ONE_U = 4;     // keys per group with loads in flight
__global__ __launch_bounds__(256) void attn_fwd_one_kernel(AttnArgs a) {
  __shared__ float gm[16], gl[16];
  __shared__ float go[16][FD_HD];
  const int nsplit = a.nsplit > 0 ? a.nsplit : 1;
  const Blk bk = blk();
  const int s = bk.z / nsplit, sp = bk.z % nsplit, h = bk.y, q = bk.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = w * 4 + (lane >> 4);  // key group
  const int c8 = (lane & 15) * 8;     // this lane's 8 columns
  const int pq = (int)a.pos0 + q;     // positions fit in 31 bits
  const int win = a.window;
  int jb, je;
  split_range(max(0, pq - win + 1) & ~(BKEY - 1), pq, nsplit, sp, &jb, &je);
  const float c2 = a.scale * LOG2E;
  float qf[8];
  {
    const bf16x8 qv =
        *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(a.q) + ((int64_t)s * a.M + q) * a.ldq +
                                         h * FD_HD + c8);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[e] = (float)qv[e] * c2;
  }
  const bf16* Kc = reinterpret_cast<const bf16*>(a.kc) + s * a.seq_stride + h * FD_HD + c8;
  const bf16* Vc = reinterpret_cast<const bf16*>(a.vc) + s * a.seq_stride + h * FD_HD + c8;
  float m = NEG_BIG, l = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  // ring slot of this group's next key (cap is a multiple of 64)
  int slot = (jb + g) % a.cap;
  for (int j0 = jb + g; j0 < je; j0 += 16 * ONE_U) {
    bf16x8 kv[ONE_U], vv[ONE_U];
#pragma unroll
    for (int u = 0; u < ONE_U; ++u) {
      if (j0 + 16 * u < je) {
        kv[u] = *reinterpret_cast<const bf16x8*>(Kc + (int64_t)slot * a.ldk);
        vv[u] = *reinterpret_cast<const bf16x8*>(Vc + (int64_t)slot * a.ldk);
      }
      slot += 16;
      if (slot >= a.cap) slot -= a.cap;
    }
#pragma unroll
    for (int u = 0; u < ONE_U; ++u) {
      const int j = j0 + 16 * u;
      if (j >= je) break;  // uniform over the 16 lanes of a group
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(qf[e], (float)kv[u][e], d);
      d += __shfl_xor(d, 1, 64);
      d += __shfl_xor(d, 2, 64);
      d += __shfl_xor(d, 4, 64);
      d += __shfl_xor(d, 8, 64);
      // visible iff pq - win < j <= pq
      const float sc = (unsigned)(pq - j) < (unsigned)win ? d : -INFINITY;
      const float mn = fmaxf(m, sc);
      const float al = ex2(m - mn), p = ex2(sc - mn);
      l = fmaf(l, al, p);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fmaf(o[e], al, p * (float)vv[u][e]);
      m = mn;
    }
  }
  if ((lane & 15) == 0) {
    gm[g] = m;
    gl[g] = l;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) go[g][c8 + e] = o[e];
  __syncthreads();
  const int c = threadIdx.x;
  if (c >= FD_HD) return;
  float mx = NEG_BIG;
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = fmaxf(mx, gm[i]);
  float L = 0.f, acc = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float wg = ex2(gm[i] - mx);
    L = fmaf(gl[i], wg, L);
    acc = fmaf(go[i][c], wg, acc);
  }
  const int64_t row = (int64_t)s * a.M + q;
  if (nsplit == 1) {
    reinterpret_cast<bf16*>(a.o)[row * a.ldo + h * FD_HD + c] = (bf16)(acc / L);
    if (c == 0) a.lse[((int64_t)s * a.H + h) * a.M + q] = mx * LN2 + logf(L);
  } else {
    a.part_o[((int64_t)sp * a.B * a.M + row) * a.ldo + h * FD_HD + c] = L > 0.f ? acc / L : 0.f;
    if (c == 0) {
      const int64_t li = (((int64_t)sp * a.B + s) * a.H + h) * a.M + q;
      a.part_m[li] = mx;
      a.part_l[li] = L;
    }
  }
}

// merge split partials: O = sum_s w_s O_s / sum_s w_s, w_s = l_s 2^(m_s - m).
// One workgroup per row: the normalised weights of every (split, head) go to
// LDS first, then each thread combines 4 consecutive columns.
constexpr int COMBINE_MAX_H = 64;
// test hook: 0 keeps bf16 head-dim-128 attention on the register-staged kernels
int g_attn_dl = 1;
template <typename T>
__global__ void attn_combine_kernel(AttnArgs a) {
  __shared__ float wgt[16][COMBINE_MAX_H];
  const int64_t row = blockIdx.x;  // s*M + q
  const int s = row / a.M, q = row % a.M;
  const int HD = a.H * a.hd;
  for (int h = threadIdx.x; h < a.H; h += blockDim.x) {
    float m = NEG_BIG;
    for (int sp = 0; sp < a.nsplit; ++sp) m = fmaxf(m, a.part_m[(((int64_t)sp * a.B + s) * a.H + h) * a.M + q]);
    float wsum = 0.f;
    for (int sp = 0; sp < a.nsplit; ++sp) {
      const int64_t li = (((int64_t)sp * a.B + s) * a.H + h) * a.M + q;
      const float w = a.part_l[li] * ex2(a.part_m[li] - m);
      wgt[sp][h] = w;
      wsum += w;
    }
    const float inv = 1.f / wsum;
    for (int sp = 0; sp < a.nsplit; ++sp) wgt[sp][h] *= inv;
    a.lse[((int64_t)s * a.H + h) * a.M + q] = m * LN2 + logf(wsum);
  }
  __syncthreads();
  for (int c = threadIdx.x * 4; c < HD; c += blockDim.x * 4) {
    const int h = c / a.hd;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < a.nsplit; ++sp) {
      const float4 v = *reinterpret_cast<const float4*>(a.part_o + ((int64_t)sp * a.B * a.M + row) * a.ldo + c);
      const float w = wgt[sp][h];
      acc[0] += w * v.x; acc[1] += w * v.y; acc[2] += w * v.z; acc[3] += w * v.w;
    }
    T* o = reinterpret_cast<T*>(a.o) + row * a.ldo + c;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = from_f32<T>(acc[k]);
  }
}

// The same merge for a few rows (decode): one wave per (row, head), so the
// split partials of a row are read by many workgroups at once. Every load
// (split maxima, sums and this thread's partial rows) is issued before any
// arithmetic, in one round trip.
template <typename T>
__global__ __launch_bounds__(64) void attn_combine_head_kernel(AttnArgs a) {
  const int64_t row = blockIdx.x;  // s*M + q
  const int h = blockIdx.y;
  const int s = row / a.M, q = row % a.M;
  for (int c0 = 0; c0 < a.hd; c0 += 64 * 4) {
    const int c = c0 + threadIdx.x * 4;
    const bool col = c < a.hd;
    float pm[16], pl[16];
    float4 v[16];
#pragma unroll
    for (int sp = 0; sp < 16; ++sp) {
      pm[sp] = NEG_BIG;
      pl[sp] = 0.f;
      v[sp] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (sp < a.nsplit) {
        const int64_t li = (((int64_t)sp * a.B + s) * a.H + h) * a.M + q;
        pm[sp] = a.part_m[li];
        pl[sp] = a.part_l[li];
        if (col) v[sp] = *reinterpret_cast<const float4*>(a.part_o + ((int64_t)sp * a.B * a.M + row) * a.ldo + h * a.hd + c);
      }
    }
    float m = NEG_BIG;
#pragma unroll
    for (int sp = 0; sp < 16; ++sp) m = fmaxf(m, pm[sp]);
    float wsum = 0.f;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sp = 0; sp < 16; ++sp) {
      const float w = pl[sp] * ex2(pm[sp] - m);  // 0 for the absent splits
      wsum += w;
      acc[0] += w * v[sp].x; acc[1] += w * v[sp].y; acc[2] += w * v[sp].z; acc[3] += w * v[sp].w;
    }
    const float inv = 1.f / wsum;
    if (c0 == 0 && threadIdx.x == 0) a.lse[((int64_t)s * a.H + h) * a.M + q] = m * LN2 + logf(wsum);
    if (col) {
      T* o = reinterpret_cast<T*>(a.o) + row * a.ldo + h * a.hd + c;
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = from_f32<T>(acc[k] * inv);
    }
  }
}

// ============================== backward: dQ ==============================

template <typename T, int HD>
__global__ __launch_bounds__(NT, 2) void attn_bwd_dq_kernel(AttnArgs a) {
  typedef AT<T> A;
  constexpr int LDK = HD + A::PADT, LDV = HD + A::PADR;
  constexpr int NKS = HD / A::KS;
  constexpr int DB = HD >= 32 ? HD / 32 : 1;
  __shared__ __attribute__((aligned(16))) T sK[2][BKEY * LDK];
  __shared__ __attribute__((aligned(16))) T sV[2][BKEY * LDV];

  const int nsplit = a.nsplit > 0 ? a.nsplit : 1;
  const Blk bk = blk();
  const int s = bk.z / nsplit, sp = bk.z % nsplit, h = bk.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hl = lane >> 5;
  const int M = a.M;
  const int qb0 = bk.x * QB;
  const int qw0 = qb0 + w * WQ;
  const int q = qw0 + (lane & 31);
  const bool qvalid = q < M;
  const int pos0 = (int)a.pos0;
  const int pq = pos0 + (qvalid ? q : M - 1);
  const int win = a.window;
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

  const int qlast_blk = min(qb0 + QB, M) - 1;
  const int lo = max(0, pos0 + qb0 - win + 1);
  const int hi = pos0 + qlast_blk;
  int jb, je;
  split_range(lo & ~(BKEY - 1), hi, nsplit, sp, &jb, &je);
  const bool wactive = qw0 < M;
  const int wfirst = pos0 + qw0;
  const int wlast = pos0 + min(qw0 + WQ, M) - 1;
  const float c2 = a.scale * LOG2E;

  f32x16 dq[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dq[i] = f32x16{};

  Stage<T, HD, BKEY, LDK> stK;
  Stage<T, HD, BKEY, LDV> stV;
  auto load_tile = [&](int j0) {
    const int64_t off = (int64_t)(j0 % a.cap) * a.ldk;
    const int nvalid = min(BKEY, hi - j0 + 1);
    stK.load(Kc + off, a.ldk, nvalid);
    stV.load(Vc + off, a.ldk, nvalid);
  };
  if (jb < je) {
    load_tile(jb);
    stK.store(sK[0]);
    stV.store(sV[0]);
  }
  __syncthreads();

  int buf = 0;
  for (int j0 = jb; j0 < je; j0 += BKEY, buf ^= 1) {
    const bool more = j0 + BKEY < je;
    if (more) load_tile(j0 + BKEY);
    const T* cK = sK[buf];
    const T* cV = sV[buf];
    if (wactive && !(j0 > wlast || j0 + BKEY - 1 <= wfirst - win)) {
      const bool full = (j0 + BKEY - 1 <= wfirst) && (j0 > wlast - win);
      f32x16 p[2], dp[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        p[g] = f32x16{};
        dp[g] = f32x16{};
        // S and dP^T chains interleaved; the K / V fragments of step ks+1 are
        // read while step ks multiplies
        const int row = g * 32 + (lane & 31), kc = hl * (A::KS / 2);
        typename A::frag kf[2], vf[2];
        kf[0] = lds_frag<T>(cK, LDK, row, kc);
        vf[0] = lds_frag<T>(cV, LDV, row, kc);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          if (ks + 1 < NKS) {
            kf[(ks + 1) & 1] = lds_frag<T>(cK, LDK, row, (ks + 1) * A::KS + kc);
            vf[(ks + 1) & 1] = lds_frag<T>(cV, LDV, row, (ks + 1) * A::KS + kc);
          }
          p[g] = mfma(kf[ks & 1], qf[ks], p[g]);
          dp[g] = mfma(vf[ks & 1], df[ks], dp[g]);
        }
        const int dj = pq - (j0 + g * 32 + hl * 4);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pr = ex2(fmaf(p[g][r], c2, -lse2));
          if (!full && (unsigned)(dj - (r >> 2) * 8 - (r & 3)) >= (unsigned)win) pr = 0.f;
          p[g][r] = pr * (dp[g][r] - dlt);  // dS
        }
      }
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int u = 0; u < KSteps<T>::N; ++u) {
          // every K^T fragment of this key step first, then their MFMAs
          typename A::frag kt[DB];
#pragma unroll
          for (int i = 0; i < DB; ++i)
            kt[i] = (i * 32 < HD) ? lds_frag_tr<T>(cK, LDK, i * 32, g, u, lane, HD) : typename A::frag{};
          typename A::frag sf = acc_frag<T>(p[g], u);
#pragma unroll
          for (int i = 0; i < DB; ++i) dq[i] = mfma(kt[i], sf, dq[i]);
        }
    }
    if (more) {
      stK.store(sK[buf ^ 1]);
      stV.store(sV[buf ^ 1]);
    }
    __syncthreads();
  }
  if (!wactive || !qvalid) return;
  // split sp writes its own slice of dq (the slices are summed by the caller's pack)
  float* out = a.dq + (int64_t)sp * a.B * M * a.lddq + ((int64_t)s * M + q) * a.lddq + h * a.hd;
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = i * 32 + acc_row(r, hl);
      if (d < HD) out[d] = dq[i][r] * a.scale;
    }
}

// dQ kernel for bf16 with head dim 128: the computation of attn_bwd_dq_kernel
// with K and V tiles loaded straight into swizzled LDS (two-slot rings, tile
// t+1 in flight during tile t), K swizzled for both its row-wise reads (S) and
// its transposed reads (dQ^T += K^T dS^T), and the window mask applied only
// on tiles that cross a window edge. Keys past the last query are read as
// stored: their weights are masked to 0, and the caches hold finite values.
__global__ __launch_bounds__(NT, 2) void attn_bwd_dq_dl_kernel(AttnArgs a) {
  constexpr int NKS = FD_HD / 16, DB = FD_HD / 32;
  // K and V slots in one array (see attn_fwd_dl_kernel: no compiler waits on
  // the LDS-DMA loads in flight before the reads of the other slot)
  __shared__ __attribute__((aligned(1024))) bf16 sKV[4][BKEY * FD_HD];
  bf16(*const sK)[BKEY * FD_HD] = sKV;
  bf16(*const sV)[BKEY * FD_HD] = sKV + 2;

  const int nsplit = a.nsplit > 0 ? a.nsplit : 1;
  const Blk bk = blk();
  const int s = bk.z / nsplit, sp = bk.z % nsplit, h = bk.y;
  const int lane = threadIdx.x & 63, hl = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int M = a.M;
  const int qb0 = bk.x * QB;
  const int qw0 = qb0 + w * WQ;
  const int q = qw0 + (lane & 31);
  const bool qvalid = q < M;
  const int pos0 = (int)a.pos0;
  const int pq = pos0 + (qvalid ? q : M - 1);
  const int win = a.window;
  const bf16* Kc = reinterpret_cast<const bf16*>(a.kc) + s * a.seq_stride + h * FD_HD;
  const bf16* Vc = reinterpret_cast<const bf16*>(a.vc) + s * a.seq_stride + h * FD_HD;

  bf16x8 qf[NKS], df[NKS];
  {
    const bf16* qrow = reinterpret_cast<const bf16*>(a.q) + ((int64_t)s * M + (qvalid ? q : 0)) * a.ldq + h * FD_HD;
    const bf16* drow = reinterpret_cast<const bf16*>(a.dout) + ((int64_t)s * M + (qvalid ? q : 0)) * a.lddo + h * FD_HD;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qf[ks] = qvalid ? *reinterpret_cast<const bf16x8*>(qrow + ks * 16 + hl * 8) : bf16x8{};
      df[ks] = qvalid ? *reinterpret_cast<const bf16x8*>(drow + ks * 16 + hl * 8) : bf16x8{};
    }
  }
  const int64_t li = ((int64_t)s * a.H + h) * M + (qvalid ? q : 0);
  const float lse2 = qvalid ? a.lse[li] * LOG2E : 0.f;
  const float dlt = qvalid ? a.delta[li] : 0.f;

  const int qlast_blk = min(qb0 + QB, M) - 1;
  const int lo = max(0, pos0 + qb0 - win + 1);
  const int hi = pos0 + qlast_blk;
  int jb, je;
  split_range(lo & ~(BKEY - 1), hi, nsplit, sp, &jb, &je);
  const int nt = (je - jb) / BKEY;
  const bool wactive = qw0 < M;
  const int wfirst = pos0 + qw0;
  const int wlast = pos0 + min(qw0 + WQ, M) - 1;
  const float c2 = a.scale * LOG2E;

  f32x16 dq[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dq[i] = f32x16{};

  uint32_t koff[4], voff[4];
  fd_offsets<2>(a.ldk, w, lane, koff);
  fd_offsets<0>(a.ldk, w, lane, voff);
  const int r0 = jb % a.cap;
  auto row = [&](int t) {
    const int r = r0 + t * BKEY;
    return (int64_t)(r >= a.cap ? r - a.cap : r) * a.ldk;
  };
  if (nt > 0) {
    fd_issue(Kc + row(0), koff, sK[0], w);
    fd_issue(Vc + row(0), voff, sV[0], w);
  }
  for (int t = 0; t < nt; ++t) {
    // this wave's loads of tile t are the only ones in flight; after the
    // barrier every wave's are in LDS and tile t-1 is no longer read
    fd_wait_loads();
    __syncthreads();
    if (t + 1 < nt) {
      fd_issue(Kc + row(t + 1), koff, sK[(t + 1) & 1], w);
      fd_issue(Vc + row(t + 1), voff, sV[(t + 1) & 1], w);
    }
    const int j0 = jb + t * BKEY;
    if (!wactive || j0 > wlast || j0 + BKEY - 1 <= wfirst - win) continue;
    const bf16* cK = sK[t & 1];
    const bf16* cV = sV[t & 1];
    const bool full = (j0 + BKEY - 1 <= wfirst) && (j0 > wlast - win);
    // the two 32-key halves one after the other (one half's S and dP live)
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      f32x16 p = f32x16{}, dp = f32x16{};
      // S and dP^T chains interleaved; the K / V fragments of step ks+1 are
      // read while step ks multiplies
      const int r = g * 32 + (lane & 31);
      bf16x8 kf[2], vf[2];
      kf[0] = fd_frag<2>(cK, r, hl);
      vf[0] = fd_frag<0>(cV, r, hl);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if (ks + 1 < NKS) {
          kf[(ks + 1) & 1] = fd_frag<2>(cK, r, (ks + 1) * 2 + hl);
          vf[(ks + 1) & 1] = fd_frag<0>(cV, r, (ks + 1) * 2 + hl);
        }
        p = mfma(kf[ks & 1], qf[ks], p);
        dp = mfma(vf[ks & 1], df[ks], dp);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) p[e] = ex2(fmaf(p[e], c2, -lse2));
      if (!full) {
        // a real branch (tiles crossing a window edge are few): the empty
        // volatile asm keeps the compiler from turning it into selects
        asm volatile("" ::: "memory");
        // visible iff 0 <= pq - j < win
        const int dj = pq - (j0 + g * 32 + hl * 4);
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if ((unsigned)(dj - (e >> 2) * 8 - (e & 3)) >= (unsigned)win) p[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) p[e] *= dp[e] - dlt;  // dS
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8 kt[DB];
#pragma unroll
        for (int i = 0; i < DB; ++i) kt[i] = fd_frag_tr<2>(cK, i * 32, g, u, lane);
        const bf16x8 sf = acc_frag<bf16>(p, u);
#pragma unroll
        for (int i = 0; i < DB; ++i) dq[i] = mfma(kt[i], sf, dq[i]);
      }
    }
  }
  if (!wactive || !qvalid) return;
  // split sp writes its own slice of dq (the slices are summed by the caller's pack)
  float* out = a.dq + (int64_t)sp * a.B * M * a.lddq + ((int64_t)s * M + q) * a.lddq + h * FD_HD;
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) out[i * 32 + acc_row(e, hl)] = dq[i][e] * a.scale;
}

// ============================== backward: dK, dV ==============================

constexpr int BQT = 64;  // query tile of the key-owned kernel

template <typename T, int HD>
__global__ __launch_bounds__(NT) void attn_bwd_dkdv_kernel(AttnArgs a) {
  typedef AT<T> A;
  constexpr int LD = HD + A::PADT;
  constexpr int NKS = HD / A::KS;
  constexpr int DB = HD >= 32 ? HD / 32 : 1;
  __shared__ __attribute__((aligned(16))) T sQ[2][BQT * LD];
  __shared__ __attribute__((aligned(16))) T sD[2][BQT * LD];
  __shared__ float sL[2][BQT], sDl[2][BQT];

  const Blk bk = blk();
  const int s = bk.z, h = bk.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hl = lane >> 5;
  const int M = a.M;
  const int kb0 = bk.x * QB;
  const int kw0 = kb0 + w * WQ;
  const int kr = kw0 + (lane & 31);     // key row within the chunk
  const bool kvalid = kr < M;
  const int pos0 = (int)a.pos0;
  const int pk = pos0 + (kvalid ? kr : M - 1);
  const int win = a.window;
  const T* Kc = reinterpret_cast<const T*>(a.kc) + s * a.seq_stride + h * a.hd;
  const T* Vc = reinterpret_cast<const T*>(a.vc) + s * a.seq_stride + h * a.hd;
  const T* Q = reinterpret_cast<const T*>(a.q) + (int64_t)s * M * a.ldq + h * a.hd;
  const T* DO = reinterpret_cast<const T*>(a.dout) + (int64_t)s * M * a.lddo + h * a.hd;
  const float* LSE = a.lse + ((int64_t)s * a.H + h) * M;
  const float* DLT = a.delta + ((int64_t)s * a.H + h) * M;

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
  const int klast_blk = min(kb0 + QB, M) - 1;
  const bool wactive = kw0 < M;
  const int wk_first = kw0, wk_last = min(kw0 + WQ, M) - 1;
  // queries (rows) that can see keys of this block: [kb0, klast_blk + win - 1]
  const int q_end = min(M, klast_blk + win);
  const int q_start = kb0 & ~(BQT - 1);

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) { dk[i] = f32x16{}; dv[i] = f32x16{}; }

  Stage<T, HD, BQT, LD> stQ, stD;
  float nl = 0.f, nd = 0.f;

  auto ld_stats = [&](int q0) {
    const int r = threadIdx.x, qi = q0 + r;
    if (r < BQT) {
      nl = qi < M ? LSE[qi] * LOG2E : 0.f;
      nd = qi < M ? DLT[qi] : 0.f;
    }
  };
  auto st_stats = [&](int b) {
    if (threadIdx.x < BQT) { sL[b][threadIdx.x] = nl; sDl[b][threadIdx.x] = nd; }
  };
  if (q_start < q_end) {
    stQ.load(Q + (int64_t)q_start * a.ldq, a.ldq, M - q_start);
    stD.load(DO + (int64_t)q_start * a.lddo, a.lddo, M - q_start);
    ld_stats(q_start);
    stQ.store(sQ[0]);
    stD.store(sD[0]);
    st_stats(0);
  }
  __syncthreads();

  int buf = 0;
  for (int q0 = q_start; q0 < q_end; q0 += BQT, buf ^= 1) {
    const bool more = q0 + BQT < q_end;
    if (more) {
      stQ.load(Q + (int64_t)(q0 + BQT) * a.ldq, a.ldq, M - q0 - BQT);
      stD.load(DO + (int64_t)(q0 + BQT) * a.lddo, a.lddo, M - q0 - BQT);
      ld_stats(q0 + BQT);
    }
    const T* cQ = sQ[buf];
    const T* cD = sD[buf];
    // does any (query in tile, key in wave) pair satisfy pk <= pq < pk + win ?
    if (wactive && !(q0 + BQT - 1 < wk_first || q0 > wk_last + win - 1)) {
      f32x16 p[2], dp[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {   // 32-query groups of the tile
        p[g] = f32x16{};
        dp[g] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const int row = g * 32 + (lane & 31), kk = ks * A::KS + hl * (A::KS / 2);
          p[g] = mfma(lds_frag<T>(cQ, LD, row, kk), kf[ks], p[g]);
          dp[g] = mfma(lds_frag<T>(cD, LD, row, kk), vf[ks], dp[g]);
        }
        // visible iff 0 <= pq - pk < win, pq = pos0 + q0 + qr, and the query row exists
        const int dq0 = pos0 + q0 + g * 32 + hl * 4 - pk;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qr = g * 32 + acc_row(r, hl);
          float pr = ex2(fmaf(p[g][r], c2, -sL[buf][qr]));
          if ((unsigned)(dq0 + (r >> 2) * 8 + (r & 3)) >= (unsigned)win || q0 + qr >= M || !kvalid) pr = 0.f;
          p[g][r] = pr;
          dp[g][r] = pr * (dp[g][r] - sDl[buf][qr]);  // dS
        }
      }
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int u = 0; u < KSteps<T>::N; ++u) {
          typename A::frag pf = acc_frag<T>(p[g], u);
          typename A::frag sf = acc_frag<T>(dp[g], u);
#pragma unroll
          for (int i = 0; i < DB; ++i) {
            if (i * 32 >= HD) continue;
            dv[i] = mfma(lds_frag_tr<T>(cD, LD, i * 32, g, u, lane, HD), pf, dv[i]);
            dk[i] = mfma(lds_frag_tr<T>(cQ, LD, i * 32, g, u, lane, HD), sf, dk[i]);
          }
        }
    }
    if (more) {
      stQ.store(sQ[buf ^ 1]);
      stD.store(sD[buf ^ 1]);
      st_stats(buf ^ 1);
    }
    __syncthreads();
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

// workgroup barrier that orders LDS only: this wave's LDS accesses are done,
// global loads and stores may still be in flight (__syncthreads would wait
// for them too)
TTT_DEV void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// base + a 32-bit byte offset (lets the load take a scalar base address)
TTT_DEV const void* gaddr(const void* base, uint32_t bytes) { return static_cast<const char*>(base) + bytes; }

// dK / dV kernel for bf16 with head dim 128: the computation of
// attn_bwd_dkdv_kernel, balanced. The chunk's keys form blocks of 64; a
// workgroup takes block x and block nkb-1-x in turn (nkb = blocks in the
// chunk), so an early block, which many queries see, rides with a late one,
// which few do: with a window of at least the chunk every workgroup walks the
// same number of query tiles. Eight waves: wave w owns keys 32 (w % 2) .. +31
// of the block (K fragments in registers, the block's V rows in LDS) and
// queries 32 (w / 2) .. +31 of every 128-query tile; Q and dO tiles go
// straight into a two-stage LDS ring (read both row-wise and transposed:
// swizzle 2), the per-query statistics by 4-byte DMA. The four waves that
// share keys sum their partial dK, dV through LDS, in a fixed order, once per
// block, while the next block's first tile is loading.
constexpr int DKDV_NT = 512;
constexpr int DK_KB = 64;   // keys per block
constexpr int DK_QT = 128;  // queries per tile
__global__ __launch_bounds__(DKDV_NT) void attn_bwd_dkdv_dl_kernel(AttnArgs a) {
  constexpr int NKS = FD_HD / 16, DB = FD_HD / 32;
  constexpr int XF = DB * 16 * 64;  // floats of one wave's dK (or dV) partial
  // [stage][Q, dO][128 rows]: 128 KB; a stage doubles as the exchange buffer
  // one array for every tile the LDS-DMA loads fill (see attn_fwd_dl_kernel:
  // no compiler waits on the loads in flight before the reads of other parts)
  constexpr int QD_B = 2 * 2 * DK_QT * FD_HD * 2, VK_B = DK_KB * FD_HD * 2, ST_B = 2 * DK_QT * 4;
  __shared__ __attribute__((aligned(1024))) char lds[QD_B + VK_B + 2 * ST_B];
  bf16(*const sQD)[2][DK_QT * FD_HD] = reinterpret_cast<bf16(*)[2][DK_QT * FD_HD]>(lds);
  bf16* const sVk = reinterpret_cast<bf16*>(lds + QD_B);  // the block's V rows
  float(*const sL)[DK_QT] = reinterpret_cast<float(*)[DK_QT]>(lds + QD_B + VK_B);
  float(*const sDl)[DK_QT] = reinterpret_cast<float(*)[DK_QT]>(lds + QD_B + VK_B + ST_B);

  const Blk bk = blk();
  const int s = bk.z, h = bk.y;
  const int lane = threadIdx.x & 63, hl = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int kq = w & 1, qg = w >> 1;  // key half, query quarter
  const int M = a.M;
  const int nkb = (M + DK_KB - 1) / DK_KB;
  const int pos0 = (int)a.pos0;
  const int win = a.window;
  const bf16* Kc = reinterpret_cast<const bf16*>(a.kc) + s * a.seq_stride + h * FD_HD;
  const bf16* Vc = reinterpret_cast<const bf16*>(a.vc) + s * a.seq_stride + h * FD_HD;
  const bf16* Q = reinterpret_cast<const bf16*>(a.q) + (int64_t)s * M * a.ldq + h * FD_HD;
  const bf16* DO = reinterpret_cast<const bf16*>(a.dout) + (int64_t)s * M * a.lddo + h * FD_HD;
  const float* LSE = a.lse + ((int64_t)s * a.H + h) * M;
  const float* DLT = a.delta + ((int64_t)s * a.H + h) * M;
  const float c2 = a.scale * LOG2E;

  // the (one or two) key blocks of this workgroup and their query tiles
  // [qs, qs + 128 n): the queries that can see a key of block x lie in
  // [64 x, min(M, last key + win))
  int xb[2], qs[2], nq[2];
  const int nblk = (bk.x == nkb - 1 - bk.x) ? 1 : 2;
  xb[0] = bk.x;
  xb[1] = nkb - 1 - bk.x;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int k0 = xb[b] * DK_KB, klast = min(k0 + DK_KB, M) - 1;
    const int q_end = min(M, klast + win);
    qs[b] = k0 & ~(DK_QT - 1);
    nq[b] = (b < nblk && q_end > qs[b]) ? (q_end - qs[b] + DK_QT - 1) / DK_QT : 0;
  }
  const int nt = nq[0] + nq[1];

  // this wave's 4 + 4 of the 64 one-KB loads of a tile (rows past the last
  // query read the last row: their weights are masked to 0); waves 0..3 also
  // bring 64 of the tile's log-sum-exps or deltas (4 bytes a lane)
  // (offsets recomputed at each issue: registers are the scarce resource)
  auto issue = [&](int t) __attribute__((always_inline)) {
    const int q0 = t < nq[0] ? qs[0] + t * DK_QT : qs[1] + (t - nq[0]) * DK_QT;
    const int st = t & 1;
    // addresses as a uniform base + a 32-bit byte offset per lane (the
    // launcher checks that the operands span less than 4 GiB): 64-bit
    // addresses per row would cost 16 registers
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rt = (w * 4 + i) * 4 + (lane >> 4);
      const uint32_t c8 = (uint32_t)(((lane & 15) ^ fd_swz<2>(rt)) * 8);
      const uint32_t r = (uint32_t)min(q0 + rt, M - 1);
      __builtin_amdgcn_global_load_lds(gaddr(Q, (r * (uint32_t)a.ldq + c8) * 2),
                                       (fd_lds_t*)(sQD[st][0] + (w * 4 + i) * 512), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(gaddr(DO, (r * (uint32_t)a.lddo + c8) * 2),
                                       (fd_lds_t*)(sQD[st][1] + (w * 4 + i) * 512), 16, 0, 0);
    }
    if (w < 4) {
      const uint32_t r = (uint32_t)min(q0 + (w >> 1) * 64 + lane, M - 1);
      __builtin_amdgcn_global_load_lds(gaddr((w & 1) ? DLT : LSE, r * 4),
                                       (fd_lds_t*)(((w & 1) ? sDl[st] : sL[st]) + (w >> 1) * 64), 4, 0, 0);
    }
  };
  // K fragments of this lane's key (registers) and the block's 64 V rows
  // (ring slots; past the last key the last one), 2 one-KB loads per wave
  bf16x8 kf[NKS];
  int kb0 = 0, kr = 0;
  bool kvalid = false;
  auto load_keys = [&](int b) __attribute__((always_inline)) {
    kb0 = xb[b] * DK_KB;
    kr = kb0 + kq * WQ + (lane & 31);
    kvalid = kr < M;
    const int pk = pos0 + (kvalid ? kr : M - 1);
    const bf16* krow = Kc + (int64_t)(pk % a.cap) * a.ldk;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) kf[ks] = kvalid ? *reinterpret_cast<const bf16x8*>(krow + ks * 16 + hl * 8) : bf16x8{};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = (w * 2 + i) * 4 + (lane >> 4);
      const uint32_t slot = (uint32_t)((pos0 + min(kb0 + r, M - 1)) % a.cap);
      __builtin_amdgcn_global_load_lds(
          gaddr(Vc, (slot * (uint32_t)a.ldk + (uint32_t)(((lane & 15) ^ fd_swz<0>(r)) * 8)) * 2),
          (fd_lds_t*)(sVk + (w * 2 + i) * 512), 16, 0, 0);
    }
  };

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) { dk[i] = f32x16{}; dv[i] = f32x16{}; }

  // Sum the four query quarters' partials of each key half through one stage
  // of the ring (64 KB: [2 slots][2 key halves][XF], lane-contiguous), in a
  // fixed order, (v0 + v2) + (v1 + v3), ending in slot 0; then all 512
  // threads store the block's rows from there, 16 bytes at a time (each
  // takes 4 consecutive columns of one key). dK first, then dV. Each step
  // touches one of the two register arrays only (steps that pick between
  // them by a condition get merged into one by address, which takes both
  // out of registers).
  auto reduce_store = [&](float* X, f32x16 (&v)[DB], float* outp, float sc, int kbase)
                          __attribute__((always_inline)) {
    if (qg >= 2) {
      float* x = X + ((qg - 2) * 2 + kq) * XF;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) x[(i * 16 + e) * 64 + lane] = v[i][e];
    }
    lds_sync();
    if (qg < 2) {
      const float* x = X + (qg * 2 + kq) * XF;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) v[i][e] += x[(i * 16 + e) * 64 + lane];
    }
    lds_sync();
    if (qg == 1) {
      float* x = X + kq * XF;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) x[(i * 16 + e) * 64 + lane] = v[i][e];
    }
    lds_sync();
    if (qg == 0) {
      float* x = X + kq * XF;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) x[(i * 16 + e) * 64 + lane] += v[i][e];
    }
    lds_sync();
    // slot 0 element (i, e) of lane l is key 32 kh + l % 32, column
    // 32 i + acc_row(e, l / 32); e = 4 g + 0..3 are 4 consecutive columns
#pragma unroll
    for (int j = 0; j < 2 * XF / 4 / DKDV_NT; ++j) {
      const int g = j * DKDV_NT + (int)threadIdx.x;
      const int l = g & 63, grp = (g >> 6) & (XF / 256 - 1), kh = g / (XF / 4);
      const int i = grp >> 2, eg = grp & 3;
      const float* x = X + kh * XF + (i * 16 + eg * 4) * 64 + l;
      const f32x4 val = {x[0] * sc, x[64] * sc, x[128] * sc, x[192] * sc};
      const int r = kh * WQ + (l & 31);
      if (kbase + r < M)
        *reinterpret_cast<f32x4*>(outp + ((int64_t)s * M + kbase + r) * a.lddk + h * FD_HD + i * 32 + eg * 8 +
                                  (l >> 5) * 4) = val;
    }
    lds_sync();  // slot 0 is read before it is written again
  };
  // the block's dK (scaled) and dV; `next` >= 0 loads that block's K
  // fragments and V rows meanwhile (sVk is free: every wave is past this
  // block's tiles)
  auto finish = [&](int st, int next) __attribute__((always_inline)) {
    float* X = reinterpret_cast<float*>(&sQD[st][0][0]);
    lds_sync();  // every wave is past its last tile of this block
    const int kb_done = kb0;
    reduce_store(X, dk, a.dk, a.scale, kb_done);
    if (next >= 0) load_keys(next);
    reduce_store(X, dv, a.dv, 1.f, kb_done);
#pragma unroll
    for (int i = 0; i < DB; ++i) { dk[i] = f32x16{}; dv[i] = f32x16{}; }
  };

  load_keys(0);
  issue(0);  // (nt >= 1: see the end)
  int t = 0;
#pragma nounroll
  for (int blkno = 0; blkno < nblk; ++blkno) {
    const int tend = blkno == 0 ? nq[0] : nt;
    for (; t < tend; ++t) {
      // this wave's loads of tile t (and of the block's V rows) are the only
      // ones in flight; after the barrier every wave's are in LDS and tile
      // t-1 is no longer read
      fd_wait_loads();
      __syncthreads();
      if (t + 1 < nt) issue(t + 1);
      const int b = t & 1;
      const int q0 = t < nq[0] ? qs[0] + t * DK_QT : qs[1] + (t - nq[0]) * DK_QT;
      const int qa = q0 + qg * WQ;  // this wave's 32 queries: qa ..
      const int kw0 = kb0 + kq * WQ;
      const int wk_first = kw0, wk_last = min(kw0 + WQ, M) - 1;
      // does any (query, key) pair satisfy 0 <= q - k < win ?
      if (kw0 < M && !(qa + WQ - 1 < wk_first || qa > wk_last + win - 1)) {
        const bf16* cQ = sQD[b][0];
        const bf16* cD = sQD[b][1];
        f32x16 p = f32x16{}, dp = f32x16{};
        const int row = qg * WQ + (lane & 31);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          p = mfma(fd_frag<2>(cQ, row, ks * 2 + hl), kf[ks], p);
          dp = mfma(fd_frag<2>(cD, row, ks * 2 + hl), fd_frag<0>(sVk, kq * WQ + (lane & 31), ks * 2 + hl), dp);
          if (ks & 1) __builtin_amdgcn_sched_barrier(0);
        }
        // accumulator rows are queries: acc_row(e, hl) = 8 (e/4) + 4 hl + e%4
        const float* Lq = &sL[b][qg * WQ + hl * 4];
        const float* Dq = &sDl[b][qg * WQ + hl * 4];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(Lq + k4 * 8);
#pragma unroll
          for (int e = 0; e < 4; ++e) p[k4 * 4 + e] = ex2(fmaf(p[k4 * 4 + e], c2, -l4[e] * LOG2E));
        }
        const bool full =
            qa - wk_last >= 0 && qa + WQ - 1 - wk_first < win && qa + WQ - 1 < M && wk_last == kw0 + WQ - 1;
        if (!full) {
          asm volatile("" ::: "memory");  // a real branch, not selects
          // visible iff 0 <= q - k < win, the query row exists and the key does
          const int dq0 = qa + hl * 4 - kr;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int dqe = dq0 + (e >> 2) * 8 + (e & 3);
            if ((unsigned)dqe >= (unsigned)win || qa + (e >> 2) * 8 + hl * 4 + (e & 3) >= M || !kvalid) p[e] = 0.f;
          }
        }
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(Dq + k4 * 8);
#pragma unroll
          for (int e = 0; e < 4; ++e) dp[k4 * 4 + e] = p[k4 * 4 + e] * (dp[k4 * 4 + e] - d4[e]);  // dS
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bf16x8 pf = acc_frag<bf16>(p, u), sf = acc_frag<bf16>(dp, u);
#pragma unroll
          for (int i = 0; i < DB; ++i) dv[i] = mfma(fd_frag_tr<2>(cD, i * 32, qg, u, lane), pf, dv[i]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < DB; ++i) dk[i] = mfma(fd_frag_tr<2>(cQ, i * 32, qg, u, lane), sf, dk[i]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // the block's sums use the stage of its last tile (the next block's first
    // tile, if any, is loading into the other one)
    finish((t - 1) & 1, blkno + 1 < nblk ? 1 : -1);
  }
  // (every key sees at least its own query when window >= 1, so each block
  // has a tile and every key's dK, dV are written above)
}

template <typename T, int HD>
hipError_t fwd_t(const AttnArgs& a, hipStream_t st) {
  const int ns = a.nsplit > 0 ? a.nsplit : 1;
  dim3 grid((a.M + QB - 1) / QB, a.H, a.B * ns);
  const auto al16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  const bool dl = sizeof(T) == 2 && HD == FD_HD && g_attn_dl && al16(a.kc) && al16(a.vc) && a.ldk % 8 == 0 &&
                  a.seq_stride % 8 == 0;
  if (dl && g_attn_dl == 1 && a.M <= ONE_MAXM && al16(a.q) && a.ldq % 8 == 0)
    TTT_LAUNCH(attn_fwd_one_kernel, dim3(a.M, a.H, a.B * ns), dim3(256), 0, st, a);
  else if (dl)
    TTT_LAUNCH(attn_fwd_dl_kernel, grid, dim3(NT), 0, st, a);
  else
    TTT_LAUNCH((attn_fwd_kernel<T, HD>), grid, dim3(NT), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ns == 1) return e;
  if (a.M <= ONE_MAXM)
    TTT_LAUNCH((attn_combine_head_kernel<T>), dim3(a.B * a.M, a.H), dim3(64), 0, st, a);
  else
    TTT_LAUNCH((attn_combine_kernel<T>), dim3(a.B * a.M), dim3(256), 0, st, a);
  return hipGetLastError();
}
template <typename T, int HD>
hipError_t bwd_t(const AttnArgs& a, hipStream_t st) {
  const int ns = a.nsplit > 0 ? a.nsplit : 1;
  dim3 grid((a.M + QB - 1) / QB, a.H, a.B * ns);
  const auto al16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  if (a.parts != 2) {
    if (sizeof(T) == 2 && HD == FD_HD && g_attn_dl && al16(a.kc) && al16(a.vc) && a.ldk % 8 == 0 &&
        a.seq_stride % 8 == 0)
      TTT_LAUNCH(attn_bwd_dq_dl_kernel, grid, dim3(NT), 0, st, a);
    else
      TTT_LAUNCH((attn_bwd_dq_kernel<T, HD>), grid, dim3(NT), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.parts == 1) return e;
  }
  // (the direct-to-LDS kernel addresses one sequence's q, dO rows and ring
  // slots with 32-bit byte offsets)
  const bool small = (int64_t)a.M * std::max(a.ldq, a.lddo) * 2 < (1ll << 32) &&
                     (int64_t)a.cap * a.ldk * 2 < (1ll << 32);
  const bool dl = sizeof(T) == 2 && HD == FD_HD && g_attn_dl && al16(a.kc) && al16(a.vc) && al16(a.q) &&
                  al16(a.dout) && al16(a.dk) && al16(a.dv) && a.ldk % 8 == 0 && a.seq_stride % 8 == 0 &&
                  a.ldq % 8 == 0 && a.lddo % 8 == 0 && a.lddk % 4 == 0 && small;
  if (dl) {
    // key blocks of 64 in pairs
    const int nkb = (a.M + DK_KB - 1) / DK_KB;
    TTT_LAUNCH(attn_bwd_dkdv_dl_kernel, dim3((nkb + 1) / 2, a.H, a.B), dim3(DKDV_NT), 0, st, a);
  } else {
    TTT_LAUNCH((attn_bwd_dkdv_kernel<T, HD>), dim3((a.M + QB - 1) / QB, a.H, a.B), dim3(NT), 0, st, a);
  }
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

int attn_splits(int M, int H, int B, int64_t keys_per_query) {
  // enough waves to cover the CUs twice, each split keeping >= 8 key tiles
  const int64_t waves = (int64_t)((M + WQ - 1) / WQ) * H * B;
  int ns = 1;
  while (waves * ns < 2048 && keys_per_query / (BKEY * ns * 2) >= 8 && ns < 16) ns *= 2;
  return ns;
}

hipError_t attn_fwd_launch(const AttnArgs& a, int dt, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  if (a.nsplit > 1 && (!a.part_o || !a.part_m || !a.part_l)) return hipErrorInvalidValue;
  if (a.nsplit > 16 || (a.nsplit > 1 && (a.H > COMBINE_MAX_H || a.ldo % 4))) return hipErrorInvalidValue;
  TTT_HD_SWITCH(fwd_t)
}

void attn_force_fwd_kernel(int dl) { g_attn_dl = dl; }

hipError_t attn_bwd_launch(const AttnArgs& a, int dt, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  TTT_HD_SWITCH(bwd_t)
}

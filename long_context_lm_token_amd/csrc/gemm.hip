// MFMA GEMM for gfx950: C[m][n] (epilogue)= sum_k A(m,k) * B(n,k).
//
// A(m,k) is read from a row-major array either K-contiguous (A[m*lda+k]) or
// M-contiguous (A[k*lda+m]); B(n,k) likewise (B[n*ldb+k] or B[k*ldb+n]).
// This covers the three products of a linear layer y = x W:
//   forward   y  = x  . W      (A K-contiguous, B = W^T stored [out][in])
//   input grad dx = dy . W^T   (A K-contiguous, B = the same [out][in] array
//                               read N-contiguous)
//   weight grad dW^T = dy^T . x (A and B both read M/N-contiguous; the
//                               reduction runs over the tokens of a chunk)
// and the weight-grad epilogue applies the inner SGD step
// W <- W - eta * G directly to the fp32 master (review "TTT-E2E: Learning a
// Long Context into Weights", section 5, Eq. 9), refreshing the compute copy.
//
// Tiling: 256 threads = 4 wave64s, block tile 128x128, each wave 64x64 as
// 2x2 MFMA 32x32 tiles (bf16: v_mfma_f32_32x32x16_bf16, fp32:
// v_mfma_f32_32x32x2f32), fp32 accumulation. Operands are staged through LDS
// K-contiguous with a padded row stride (conflict-free 16-byte fragment
// reads); M/N-contiguous operands are transposed in registers on the way in.
// Two LDS stages; global loads of tile k+1 are in flight during the MFMAs of
// tile k. Block ids are remapped so that each XCD gets a contiguous run of
// tiles in grouped-M order (L2 reuse of A rows and B columns).
#include "common.h"
#include "kernels.h"

namespace {

template <typename T> struct GT;
template <> struct GT<bf16> {
  static constexpr int BK = 64, KS = 16, VEC = 8, PAD = 8;
  typedef bf16x8 frag;
};
template <> struct GT<float> {
  static constexpr int BK = 16, KS = 2, VEC = 4, PAD = 2;
  typedef float frag;
};

constexpr int BM = 128, BN = 128, NT = 256;

template <typename T> struct Vec;
template <> struct Vec<bf16> { typedef bf16x8 type; };
template <> struct Vec<float> { typedef f32x4 type; };

TTT_DEV f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
TTT_DEV f32x16 mfma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Stage one 128 x BK operand tile into registers.
// KMAJ: array [rows][ld] with k contiguous; else array [k][ld] with rows contiguous.
template <typename T, bool KMAJ>
struct TileLoader {
  typedef GT<T> G;
  typedef typename Vec<T>::type V;
  static constexpr int NV = BM * G::BK / (NT * G::VEC);  // vectors per thread
  V v[NV];

  TTT_DEV void load(const T* __restrict__ base, int64_t ld, int row0, int nrows, int k0, int K) {
    const int t = threadIdx.x;
    if constexpr (KMAJ) {
      constexpr int VPR = G::BK / G::VEC;  // vectors per row
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int vi = i * NT + t;
        const int r = vi / VPR, kc = (vi % VPR) * G::VEC;
        const int gr = row0 + r, gk = k0 + kc;
        if (gr < nrows && gk < K)
          v[i] = *reinterpret_cast<const V*>(base + (int64_t)gr * ld + gk);
        else
          v[i] = V{};
      }
    } else {
      constexpr int TPR = BM / G::VEC;  // threads per k-row group
      const int kb = t / TPR, mb = t % TPR;
      const int gr = row0 + mb * G::VEC;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int gk = k0 + kb * NV + j;
        if (gk < K && gr < nrows)
          v[j] = *reinterpret_cast<const V*>(base + (int64_t)gk * ld + gr);
        else
          v[j] = V{};
      }
    }
  }

  // write into LDS tile s[BM][BK+PAD] (k contiguous)
  TTT_DEV void store(T* s) {
    constexpr int LS = G::BK + G::PAD;
    const int t = threadIdx.x;
    if constexpr (KMAJ) {
      constexpr int VPR = G::BK / G::VEC;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int vi = i * NT + t;
        const int r = vi / VPR, kc = (vi % VPR) * G::VEC;
        *reinterpret_cast<V*>(s + r * LS + kc) = v[i];
      }
    } else {
      constexpr int TPR = BM / G::VEC;
      const int kb = t / TPR, mb = t % TPR;
#pragma unroll
      for (int e = 0; e < G::VEC; ++e) {
        T* dst = s + (mb * G::VEC + e) * LS + kb * NV;
        if constexpr (NV == 4) {
          bf16x4 w;
          w[0] = v[0][e]; w[1] = v[1][e]; w[2] = v[2][e]; w[3] = v[3][e];
          *reinterpret_cast<bf16x4*>(dst) = w;
        } else {
          float2 w;
          w.x = v[0][e]; w.y = v[1][e];
          *reinterpret_cast<float2*>(dst) = w;
        }
      }
    }
  }
};

template <typename T>
TTT_DEV typename GT<T>::frag read_frag(const T* s, int row, int k) {
  constexpr int LS = GT<T>::BK + GT<T>::PAD;
  return *reinterpret_cast<const typename GT<T>::frag*>(s + row * LS + k);
}

template <typename T, bool AK, bool BKM, int EPI, typename OutT>
__global__ __launch_bounds__(NT) void gemm_kernel(GemmArgs p) {
  typedef GT<T> G;
  constexpr int LS = G::BK + G::PAD;
  __shared__ __attribute__((aligned(16))) T smem[2][(BM + BN) * LS];

  // ---- tile schedule: XCD-contiguous remap, then grouped-M order ----
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
  int t = blockIdx.x;
  if ((ntiles & 7) == 0) t = (t & 7) * (ntiles >> 3) + (t >> 3);
  constexpr int GROUP = 8;
  const int group = t / (GROUP * tiles_n);
  const int first_m = group * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (t % (GROUP * tiles_n)) % gsz;
  const int tn = (t % (GROUP * tiles_n)) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  const int z = blockIdx.z;
  const T* A = reinterpret_cast<const T*>(p.A) + z * p.sA;
  const T* B = reinterpret_cast<const T*>(p.B) + z * p.sB;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;

  TileLoader<T, AK> la;
  TileLoader<T, BKM> lb;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = (p.K + G::BK - 1) / G::BK;
  la.load(A, p.lda, m0, p.M, 0, p.K);
  lb.load(B, p.ldb, n0, p.N, 0, p.K);
  la.store(smem[0]);
  lb.store(smem[0] + BM * LS);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      la.load(A, p.lda, m0, p.M, (kt + 1) * G::BK, p.K);
      lb.load(B, p.ldb, n0, p.N, (kt + 1) * G::BK, p.K);
    }
    const T* sa = smem[cur];
    const T* sb = smem[cur] + BM * LS;
#pragma unroll
    for (int ks = 0; ks < G::BK / G::KS; ++ks) {
      const int kk = ks * G::KS + (lane >> 5) * (G::KS / 2);
      typename G::frag fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = read_frag(sa, wm * 64 + i * 32 + (lane & 31), kk);
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = read_frag(sb, wn * 64 + j * 32 + (lane & 31), kk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma(fa[i], fb[j], acc[i][j]);
    }
    if (kt + 1 < nk) {
      la.store(smem[cur ^ 1]);
      lb.store(smem[cur ^ 1] + BM * LS);
    }
    __syncthreads();
  }

  // ---- epilogue ----
  OutT* C = p.C ? reinterpret_cast<OutT*>(p.C) + z * p.sC : nullptr;
  const float* R = p.R ? p.R + z * p.sR : nullptr;
  float* Wm = p.Wm ? p.Wm + z * p.sW : nullptr;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + (lane & 31);
      if (col >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (row >= p.M) continue;
        const float v = acc[i][j][r];
        if constexpr (EPI == EPI_STORE) {
          C[(int64_t)row * p.ldc + col] = from_f32<OutT>(v);
        } else if constexpr (EPI == EPI_ADD) {
          C[(int64_t)row * p.ldc + col] = from_f32<OutT>(R[(int64_t)row * p.ldr + col] + v);
        } else {  // EPI_SGD: fp32 master step, refresh the compute copy
          float* wp = Wm + (int64_t)row * p.ldw + col;
          const float nw = *wp - p.lr * v;
          *wp = nw;
          if (C) C[(int64_t)row * p.ldc + col] = from_f32<OutT>(nw);
        }
      }
    }
}

template <typename T, bool AK, bool BKM, int EPI, typename OutT>
hipError_t launch_t(const GemmArgs& p, int batch, hipStream_t st) {
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_kernel<T, AK, BKM, EPI, OutT>), dim3(tiles, 1, batch), dim3(NT), 0, st, p);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const GemmArgs& p, int layout, int epi, bool out_f32, int batch, hipStream_t st) {
  // layout: 0 = A K-contig / B K-contig, 1 = A K-contig / B N-contig, 2 = A M-contig / B N-contig
#define TTT_EPI_CASES(AK, BKM)                                                              \
  if (epi == EPI_STORE)                                                                    \
    return out_f32 ? launch_t<T, AK, BKM, EPI_STORE, float>(p, batch, st)                  \
                   : launch_t<T, AK, BKM, EPI_STORE, T>(p, batch, st);                     \
  if (epi == EPI_ADD) return launch_t<T, AK, BKM, EPI_ADD, float>(p, batch, st);           \
  if (epi == EPI_SGD) return launch_t<T, AK, BKM, EPI_SGD, T>(p, batch, st);
  if (layout == 0) { TTT_EPI_CASES(true, true) }
  if (layout == 1) { TTT_EPI_CASES(true, false) }
  if (layout == 2) { TTT_EPI_CASES(false, false) }
#undef TTT_EPI_CASES
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t gemm_launch(const GemmArgs& p, int dtype, int layout, int epi, bool out_f32, int batch,
                       hipStream_t st) {
  if (p.M <= 0 || p.N <= 0 || batch <= 0) return hipSuccess;
  if (dtype == 1) return dispatch<bf16>(p, layout, epi, out_f32, batch, st);
  return dispatch<float>(p, layout, epi, out_f32, batch, st);
}

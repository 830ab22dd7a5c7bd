// MFMA GEMM for gfx950: C[m][n] (epilogue)= sum_k A[m][k] * B[n][k].
//
// Both operands are read K-contiguous (row-major [rows][ld]). Every product
// of a linear layer y = x W is brought to this form by the data layout:
//   forward      y  = x . W      A = x [t][in],    B = W stored [out][in]
//   input grad   dx = dy . W^T   A = dy [t][out],  B = W stored [in][out]
//   weight grad  dW^T = dy^T . x A = dy^T [out][t], B = x^T [in][t]
// (the weight grad reduces over the tokens of a chunk). The weight-grad
// epilogue applies the inner SGD step W <- W - eta * G to the fp32 master
// and refreshes the compute copies (technical review "TTT-E2E: Learning a
// Long Context into Weights", section 5, Eq. 9). The MLP up-projection
// epilogues apply the activation to the fp32 accumulators (GELU, or SwiGLU
// with gate and up columns interleaved in 32-column blocks so that a lane
// holds both operands of a hidden unit), so the pre-activation never makes a
// round trip through HBM or a bf16 rounding.
//
// Tiling: block tile BM x BN computed by a WGM x WGN grid of wave64s, each
// owning a (BM/WGM) x (BN/WGN) tile of 32x32 MFMA tiles (bf16:
// v_mfma_f32_32x32x16_bf16, fp32: v_mfma_f32_32x32x2f32), fp32 accumulation.
// Configurations: 256x256 with 8 waves (128x64 wave tiles, two waves per
// SIMD) for large M*N, 128x128 with 4 waves (64x64 wave tiles) otherwise.
// Larger wave tiles reuse each LDS fragment for more MFMAs (LDS bandwidth is
// the limit of 64x64 wave tiles). Operands are
// staged global -> registers -> LDS (two stages, loads of tile k+1 in flight
// during the MFMAs of tile k) with a padded row stride that keeps the 16-byte
// fragment reads conflict-free. Block ids are remapped so that each XCD runs
// a contiguous run of tiles in grouped-M order (L2 reuse).
//
// Split-K: with `splits` > 1 every block handles a K range and writes fp32
// partial tiles to a workspace; gemm_reduce sums them in a fixed order and
// applies the epilogue (deterministic, no atomics).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace {

template <typename T> struct GT;
template <> struct GT<bf16> {
  static constexpr int BK = 64, KS = 16, VEC = 8, PAD = 8;
  typedef bf16x8 frag;
  typedef bf16x8 vec;
};
template <> struct GT<float> {
  static constexpr int BK = 16, KS = 2, VEC = 4, PAD = 2;
  typedef float frag;
  typedef f32x4 vec;
};


TTT_DEV f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
TTT_DEV f32x16 mfma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// One ROWS x BK operand tile, K-contiguous in global memory and in LDS,
// loaded by NT threads.
template <typename T, int ROWS, int NT>
struct TileLoader {
  typedef GT<T> G;
  typedef typename G::vec V;
  static constexpr int VPR = G::BK / G::VEC;          // vectors per row
  static constexpr int NV = ROWS * VPR / NT;          // vectors per thread
  V v[NV];

  TTT_DEV void load(const T* __restrict__ base, int64_t ld, int row0, int nrows, int k0, int k1) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = i * NT + threadIdx.x;
      const int r = vi / VPR, kc = (vi % VPR) * G::VEC;
      const int gr = row0 + r, gk = k0 + kc;
      if (gr < nrows && gk < k1)
        v[i] = *reinterpret_cast<const V*>(base + (int64_t)gr * ld + gk);
      else
        v[i] = V{};
    }
  }
  TTT_DEV void store(T* s) const {
    constexpr int LS = G::BK + G::PAD;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = i * NT + threadIdx.x;
      const int r = vi / VPR, kc = (vi % VPR) * G::VEC;
      *reinterpret_cast<V*>(s + r * LS + kc) = v[i];
    }
  }
};

template <typename T>
TTT_DEV typename GT<T>::frag read_frag(const T* s, int row, int k) {
  constexpr int LS = GT<T>::BK + GT<T>::PAD;
  return *reinterpret_cast<const typename GT<T>::frag*>(s + row * LS + k);
}

// tile index -> (tm, tn): XCD-contiguous remap, then grouped-M order
TTT_DEV void tile_coords(int t, int tiles_m, int tiles_n, int* tm, int* tn) {
  const int ntiles = tiles_m * tiles_n;
  if ((ntiles & 7) == 0) t = (t & 7) * (ntiles >> 3) + (t >> 3);
  constexpr int GROUP = 4;
  const int group = t / (GROUP * tiles_n);
  const int first_m = group * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  *tm = first_m + (t % (GROUP * tiles_n)) % gsz;
  *tn = (t % (GROUP * tiles_n)) / gsz;
}

// Unbiased (stochastic) rounding of the fp32 master to the bf16 compute copy.
// A fast weight starts exactly on the bf16 grid and an inner step moves it by
// less than half a bf16 ulp, so round-to-nearest would return it to W_0 and the
// forward would never see the update; stochastic rounding keeps the copy an
// unbiased estimate of W. The random bits come from a counter-based hash.
TTT_DEV uint32_t mix32(uint32_t h) {
  h ^= h >> 16; h *= 0x7feb352du; h ^= h >> 15; h *= 0x846ca68bu; h ^= h >> 16;
  return h;
}
template <typename T>
TTT_DEV T round_copy(float x, uint32_t seed, int z, int row, int col) {
  if constexpr (sizeof(T) == 2) {
    if (seed) {
      const uint32_t h = mix32(seed * 0x9E3779B1u ^ mix32((uint32_t)row * 0x85EBCA77u ^ (uint32_t)col * 0xC2B2AE3Du
                                                          ^ (uint32_t)z * 0x27D4EB2Fu));
      const uint32_t u = (__float_as_uint(x) + (h & 0xFFFFu)) & 0xFFFF0000u;
      return __builtin_bit_cast(bf16, (uint16_t)(u >> 16));
    }
  }
  return from_f32<T>(x);
}

// MLP activations applied to fp32 accumulators (exact GELU; SiLU gate)
TTT_DEV float gelu_acc(float x) { return 0.5f * x * (1.f + erff(x * 0.70710678118654752f)); }
// silu(g) * u with the hardware reciprocal (1 ulp; the result is rounded to
// the compute dtype) instead of an IEEE division sequence
TTT_DEV float swiglu_acc(float g, float u) { return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u; }

// interleaved column of hidden unit u's gate (its up column is 32 further)
TTT_DEV int gate_col(int u) { return (u >> 5) * 64 + (u & 31); }

// Apply the epilogue to one element (row, col) of batch z (not EPI_SWIGLU).
template <int EPI, typename OutT, typename T>
TTT_DEV void apply(const GemmArgs& p, int z, int row, int col, float v) {
  static_assert(EPI != EPI_ROPE, "the rotary epilogue needs column pairs");
  if constexpr (EPI == EPI_GELU) {
    OutT* C = reinterpret_cast<OutT*>(p.C) + z * p.sC;
    C[(int64_t)row * p.ldc + col] = from_f32<OutT>(gelu_acc(v));
  } else if constexpr (EPI == EPI_STORE) {
    OutT* C = reinterpret_cast<OutT*>(p.C) + z * p.sC;
    C[(int64_t)row * p.ldc + col] = from_f32<OutT>(v);
  } else if constexpr (EPI == EPI_ADD) {
    float* C = reinterpret_cast<float*>(p.C) + z * p.sC;
    C[(int64_t)row * p.ldc + col] = p.R[z * p.sR + (int64_t)row * p.ldr + col] + v;
  } else {
    // EPI_SGD: fp32 master step, then the compute copies [row][col] and [col][row]
    float* wp = p.Wm + z * p.sW + (int64_t)row * p.ldw + col;
    const float nw = *wp - p.lr * v;
    *wp = nw;
    const T cv = round_copy<T>(nw, p.sr_seed, z, row, col);
    if (p.C) reinterpret_cast<T*>(p.C)[z * p.sC + (int64_t)row * p.ldc + col] = cv;
    if (p.C2) reinterpret_cast<T*>(p.C2)[z * p.sC2 + (int64_t)col * p.ldc2 + row] = cv;
  }
}

// Epilogue store when the operand (residual / master value) is already loaded.
template <int EPI, typename OutT, typename T>
TTT_DEV void store_out(const GemmArgs& p, int z, int row, int col, float v, float in) {
  static_assert(EPI != EPI_ROPE, "the rotary epilogue needs column pairs");
  if constexpr (EPI == EPI_GELU) {
    reinterpret_cast<OutT*>(p.C)[z * p.sC + (int64_t)row * p.ldc + col] = from_f32<OutT>(gelu_acc(v));
  } else if constexpr (EPI == EPI_STORE) {
    reinterpret_cast<OutT*>(p.C)[z * p.sC + (int64_t)row * p.ldc + col] = from_f32<OutT>(v);
  } else if constexpr (EPI == EPI_ADD) {
    reinterpret_cast<float*>(p.C)[z * p.sC + (int64_t)row * p.ldc + col] = in + v;
  } else {
    const float nw = in - p.lr * v;
    p.Wm[z * p.sW + (int64_t)row * p.ldw + col] = nw;
    const T cv = round_copy<T>(nw, p.sr_seed, z, row, col);
    if (p.C) reinterpret_cast<T*>(p.C)[z * p.sC + (int64_t)row * p.ldc + col] = cv;
    if (p.C2) reinterpret_cast<T*>(p.C2)[z * p.sC2 + (int64_t)col * p.ldc2 + row] = cv;
  }
}

// SGD epilogue with the transposed compute copy written through LDS: the
// tile's new weights go to LDS as [col][row] (4 consecutive rows per 8-byte
// store), then each [col] row segment leaves in 16-byte stores. The fp32
// master and the row-major copy are updated directly (lanes along columns).
template <typename T, int BM, int BN, int WGM, int WGN>
TTT_DEV void sgd_epilogue_staged(const GemmArgs& p, int z, int m0, int n0, const f32x16 (&acc)[BM / WGM / 32][BN / WGN / 32],
                                 T* lds, const float (&pre)[BM / WGM / 32][BN / WGN / 32][16], bool use_pre) {
  constexpr int WTM = BM / WGM, WTN = BN / WGN, TI = WTM / 32, TJ = WTN / 32;
  constexpr int NT = WGM * WGN * 64;
  constexpr int LT = BM + 8;  // row stride of the [col][row] staging tile
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / WGN, wn = w % WGN, hl = lane >> 5;
  float* Wm = p.Wm + z * p.sW;
  T* C = p.C ? reinterpret_cast<T*>(p.C) + z * p.sC : nullptr;
  __syncthreads();  // the main loop's last reads of the operand tiles are done
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    // all master loads of this row block first, so they are in flight together
    float mv[TJ][16];
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int col = n0 + wn * WTN + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * WTM + i * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
        mv[j][r] = use_pre ? pre[i][j][r] : (row < p.M && col < p.N) ? Wm[(int64_t)row * p.ldw + col] : 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int cl = wn * WTN + j * 32 + (lane & 31);
      const int col = n0 + cl;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rl = wm * WTM + i * 32 + q * 8 + hl * 4;
        bf16x4 nv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + rl + e;
          const float nw = mv[j][q * 4 + e] - p.lr * acc[i][j][q * 4 + e];
          const T cv = round_copy<T>(nw, p.sr_seed, z, row, col);
          if (row < p.M && col < p.N) {
            Wm[(int64_t)row * p.ldw + col] = nw;
            if (C) C[(int64_t)row * p.ldc + col] = cv;
          }
          nv[e] = cv;
        }
        *reinterpret_cast<bf16x4*>(lds + cl * LT + rl) = nv;
      }
    }
  }
  __syncthreads();
  T* C2 = reinterpret_cast<T*>(p.C2) + z * p.sC2;
  constexpr int CH = BM / 8;  // 16-byte chunks per column
  for (int v = threadIdx.x; v < BN * CH; v += NT) {
    const int cl = v / CH, r0 = (v % CH) * 8;
    const int col = n0 + cl, row = m0 + r0;
    if (col >= p.N || row >= p.M) continue;
    T* dst = C2 + (int64_t)col * p.ldc2 + row;
    const T* src = lds + cl * LT + r0;
    if (row + 8 <= p.M && ((uintptr_t)dst & 15) == 0) {
      *reinterpret_cast<bf16x8*>(dst) = *reinterpret_cast<const bf16x8*>(src);
    } else {
      for (int e = 0; e < 8 && row + e < p.M; ++e) dst[e] = src[e];
    }
  }
}

// Epilogue body of one block for the non-staged operations. CHECK = false
// for tiles inside the matrix: the stores then run without per-element
// bounds branches (which would otherwise make the compiler move large
// accumulator sets through scratch).
template <bool CHECK, typename T, int BM, int BN, int WGM, int WGN, int EPI, typename OutT>
TTT_DEV void epi_body(const GemmArgs& p, int z, int m0, int n0, int wm, int wn, int lane,
                      const f32x16 (&acc)[BM / WGM / 32][BN / WGN / 32], int splits, float* part,
                      const float (&pre)[BM / WGM / 32][BN / WGN / 32][16], bool use_pre) {
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TI = WTM / 32, TJ = WTN / 32;
  if (splits > 1) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int col = n0 + wn * WTN + j * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * WTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          if (!CHECK || (row < p.M && col < p.N))
            part[(((int64_t)blockIdx.y * gridDim.z + z) * p.M + row) * p.N + col] = acc[i][j][r];
        }
      }
    return;
  }
  if constexpr (EPI == EPI_ROPE) {
    // acc[i][2jj] holds dims e = 32 sb + u of a head part, acc[i][2jj+1] their
    // rotation partners e + hd/2
    static_assert(TJ % 2 == 0, "the rotary epilogue pairs 32-column blocks");
    const RopeOut& ro = p.rope;
    const int hd = ro.hd, half = hd / 2, HDm = ro.H * hd;
    // with S % 32 == 0 a 32-row block is one run of positions of one
    // sequence (its position and ring slot follow from its first row);
    // otherwise (the few rows that end a stream) every row is placed itself
    const int S = ro.S, cap = ro.cap;
    const bool runs = S % 32 == 0;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int rb = m0 + wm * WTM + i * 32;  // first row of this 32-row block
      const int sq0 = rb / S;
      const int pos0 = (int)ro.p0 + rb % S;   // positions fit in 31 bits
      const int slot0 = pos0 % cap;
#pragma unroll
      for (int jj = 0; jj < TJ / 2; ++jj) {
        const int cb = n0 + wn * WTN + jj * 64;  // multiple of 64
        if (CHECK && cb >= p.N) continue;
        const int hp = cb / hd, part = hp / ro.H, h = hp % ro.H;
        const int e1 = ((cb % hd) / 64) * 32 + (lane & 31);
        OutT* const qb = reinterpret_cast<OutT*>(ro.q) + h * hd + e1;
        OutT* const cb_ = reinterpret_cast<OutT*>(part == 1 ? ro.kc : ro.vc) + h * hd + e1;
        // the block's 16 cos/sin pairs are loaded before any store: a load
        // after a store that may alias it cannot be hoisted, which would make
        // the 16 loads 16 round trips one after the other
        const bool rot = part < 2 && ro.tab;
        float2 cs[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const int row = rb + rr;
          cs[r] = make_float2(1.f, 0.f);
          if (rot && !(CHECK && row >= p.M)) {
            const int pos = runs ? pos0 + rr : (int)ro.p0 + row % S;
            cs[r] = ro.tab[(int64_t)pos * half + e1];
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);  // row within the block
          const int row = rb + rr;
          if (CHECK && row >= p.M) continue;
          int pos, slot, sq;
          if (runs) {
            pos = pos0 + rr;
            slot = slot0 + rr;
            if (slot >= cap) slot -= cap;
            sq = sq0;
          } else {
            sq = row / S;
            pos = (int)ro.p0 + row % S;
            slot = pos % cap;
          }
          (void)pos;
          float y1 = acc[i][2 * jj][r], y2 = acc[i][2 * jj + 1][r];
          if (rot) {
            const float a = y1, b = y2;
            y1 = a * cs[r].x - b * cs[r].y;
            y2 = a * cs[r].y + b * cs[r].x;
          }
          OutT* dst = part == 0 ? qb + (int64_t)row * ro.ldq : cb_ + sq * ro.seq_stride + (int64_t)slot * HDm;
          dst[0] = from_f32<OutT>(y1);
          dst[half] = from_f32<OutT>(y2);
        }
      }
    }
    return;
  } else if constexpr (EPI == EPI_SWIGLU) {
    // acc[i][2jj] holds gate columns and acc[i][2jj+1] the matching up columns
    static_assert(TJ % 2 == 0, "SwiGLU epilogue pairs 32-column blocks");
    OutT* C = reinterpret_cast<OutT*>(p.C) + z * p.sC;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int jj = 0; jj < TJ / 2; ++jj) {
        const int cb = n0 + wn * WTN + jj * 64;  // multiple of 64
        if (CHECK && cb >= p.N) continue;
        const int u = cb / 2 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * WTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          if (!CHECK || row < p.M)
            C[(int64_t)row * p.ldc + u] = from_f32<OutT>(swiglu_acc(acc[i][2 * jj][r], acc[i][2 * jj + 1][r]));
        }
      }
    return;
  } else {
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      // epilogue operands (residual or master) of this row block loaded first
      float in[TJ][16];
      if constexpr (EPI == EPI_ADD || EPI == EPI_SGD) {
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int col = n0 + wn * WTN + j * 32 + (lane & 31);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * WTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            in[j][r] = 0.f;
            if (use_pre)
              in[j][r] = pre[i][j][r];
            else if (!CHECK || (row < p.M && col < p.N))
              in[j][r] = EPI == EPI_ADD ? p.R[z * p.sR + (int64_t)row * p.ldr + col]
                                        : p.Wm[z * p.sW + (int64_t)row * p.ldw + col];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int col = n0 + wn * WTN + j * 32 + (lane & 31);
        if (CHECK && col >= p.N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * WTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          if (CHECK && row >= p.M) continue;
          store_out<EPI, OutT, T>(p, z, row, col, acc[i][j][r], in[j][r]);
        }
      }
    }
  }
}

// Epilogue of one block: split-K partials, or the EPI operation on the
// accumulators of wave (wm, wn). smem: the block's LDS (staged SGD copy).
// The SGD epilogue of a full 128 x 128 bf16 tile (2 x 2 waves of 64 x 64)
// with wide memory accesses: the fp32 master is read as float4 rows (512
// bytes per row of the tile); per half of 64 rows, the owning waves stage
// lr * acc in LDS ([64][132] fp32), and each thread updates 4 consecutive
// columns of 8 rows: the master written back with 16-byte stores, the
// row-major bf16 copy with 8-byte stores, and the transposed copy staged
// ([128 cols][72] bf16) for 16-byte stores of 8 rows. The update is that of
// sgd_epilogue_staged with lr * acc rounded to fp32 before the subtraction
// (the other path may fuse the two: the results differ by at most an ulp).
constexpr int SGDV_LA = 128 + 4, SGDV_LT = 64 + 8;
constexpr int SGDV_LDS = 64 * SGDV_LA * 4 + 128 * SGDV_LT * 2;
TTT_DEV bool sgd_vec_ok(const GemmArgs& p, int m0, int n0) {
  const auto al = [](const void* q, int b) { return reinterpret_cast<uintptr_t>(q) % b == 0; };
  return m0 + 128 <= p.M && n0 + 128 <= p.N && p.ldw % 4 == 0 && p.sW % 4 == 0 && al(p.Wm, 16) &&
         (!p.C || (p.ldc % 4 == 0 && p.sC % 4 == 0 && al(p.C, 8))) && p.ldc2 % 8 == 0 && p.sC2 % 8 == 0 &&
         al(p.C2, 16);
}
TTT_DEV void sgd_epilogue_vec(const GemmArgs& p, int z, int m0, int n0, const f32x16 (&acc)[2][2], void* lds) {
  float* A = reinterpret_cast<float*>(lds);
  bf16* Tt = reinterpret_cast<bf16*>(A + 64 * SGDV_LA);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1, hl = lane >> 5;
  const int c4 = tid & 31, rr = tid >> 5;  // 4 columns from 4 c4; rows rr, rr + 8, ...
  float* Wm = p.Wm + z * p.sW;
  bf16* C = p.C ? reinterpret_cast<bf16*>(p.C) + z * p.sC : nullptr;
  bf16* C2 = reinterpret_cast<bf16*>(p.C2) + z * p.sC2;
  const int col = n0 + c4 * 4;
  // one half's master values at a time (two would lift the kernel past 256
  // registers): the second half's loads go out as soon as the first half's
  // are consumed, ahead of the first half's transposed stores
  f32x4 mv[8];
  auto load_master = [&](int h) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      mv[k] = *reinterpret_cast<const f32x4*>(Wm + (int64_t)(m0 + h * 64 + k * 8 + rr) * p.ldw + col);
  };
  load_master(0);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            A[(i * 32 + (e >> 2) * 8 + hl * 4 + (e & 3)) * SGDV_LA + wn * 64 + j * 32 + (lane & 31)] =
                p.lr * acc[i][j][e];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = k * 8 + rr, row = m0 + h * 64 + r;
      const f32x4 g = *reinterpret_cast<const f32x4*>(A + r * SGDV_LA + c4 * 4);
      f32x4 nw;
      bf16x4 cv;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        nw[q] = mv[k][q] - g[q];
        cv[q] = round_copy<bf16>(nw[q], p.sr_seed, z, row, col + q);
        Tt[(c4 * 4 + q) * SGDV_LT + r] = cv[q];
      }
      *reinterpret_cast<f32x4*>(Wm + (int64_t)row * p.ldw + col) = nw;
      if (C) *reinterpret_cast<bf16x4*>(C + (int64_t)row * p.ldc + col) = cv;
    }
    if (h == 0) load_master(1);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ch = q * 256 + tid, cl = ch >> 3, rs = (ch & 7) * 8;
      *reinterpret_cast<bf16x8*>(C2 + (int64_t)(n0 + cl) * p.ldc2 + m0 + h * 64 + rs) =
          *reinterpret_cast<const bf16x8*>(Tt + cl * SGDV_LT + rs);
    }
    __syncthreads();
  }
}

// pre / use_pre: the epilogue operand (residual or fp32 master) of this
// lane's accumulators, already loaded (see prefetch_operand)
// LDS: the block's operand ring, LDS_BYTES long (free once the main loop is done)
template <typename T, int BM, int BN, int WGM, int WGN, int EPI, typename OutT, int LDS_BYTES = 0>
TTT_DEV void gemm_epilogue(const GemmArgs& p, int z, int m0, int n0, int wm, int wn, int lane,
                           const f32x16 (&acc)[BM / WGM / 32][BN / WGN / 32], int splits, float* part, T* smem,
                           const float (&pre)[BM / WGM / 32][BN / WGN / 32][16], bool use_pre) {
  if constexpr (EPI == EPI_SGD && sizeof(T) == 2 && BM == 128 && BN == 128 && WGM == 2 && WGN == 2 &&
                LDS_BYTES >= SGDV_LDS) {
    if (splits == 1 && p.C2 && sgd_vec_ok(p, m0, n0)) {
      sgd_epilogue_vec(p, z, m0, n0, acc, smem);
      return;
    }
  }
  if constexpr (EPI == EPI_SGD && sizeof(T) == 2) {
    if (splits == 1 && p.C2) {
      sgd_epilogue_staged<T, BM, BN, WGM, WGN>(p, z, m0, n0, acc, smem, pre, use_pre);
      return;
    }
  }
  if (m0 + BM <= p.M && n0 + BN <= p.N)
    epi_body<false, T, BM, BN, WGM, WGN, EPI, OutT>(p, z, m0, n0, wm, wn, lane, acc, splits, part, pre, use_pre);
  else
    epi_body<true, T, BM, BN, WGM, WGN, EPI, OutT>(p, z, m0, n0, wm, wn, lane, acc, splits, part, pre, use_pre);
}

// The residual of an unsplit EPI_ADD tile at this lane's accumulator
// positions, loaded before the main loop so that the epilogue does not wait
// for it; only for wave tiles of at most 4 MFMA tiles (64 more registers,
// which keeps two waves per SIMD). The SGD epilogue's fp32 master is not
// prefetched: holding it lifts that kernel past 256 registers, one wave per
// SIMD, and measured twice as slow.
template <int BM, int BN, int WGM, int WGN, int EPI>
TTT_DEV bool prefetch_operand(const GemmArgs& p, int z, int m0, int n0, int wm, int wn, int lane, int splits,
                              float (&pre)[BM / WGM / 32][BN / WGN / 32][16]) {
  constexpr int WTM = BM / WGM, WTN = BN / WGN, TI = WTM / 32, TJ = WTN / 32;
  if constexpr (EPI == EPI_ADD && TI * TJ <= 4) {
    if (splits != 1) return false;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int col = n0 + wn * WTN + j * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * WTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          pre[i][j][r] = 0.f;
          if (row < p.M && col < p.N)
            pre[i][j][r] = p.R[z * p.sR + (int64_t)row * p.ldr + col];
        }
      }
    return true;
  } else {
    return false;
  }
}


template <typename T, int BM, int BN, int WGM, int WGN, int EPI, typename OutT>
__global__ __launch_bounds__(WGM * WGN * 64) void gemm_kernel(GemmArgs p, int splits, float* part) {
  typedef GT<T> G;
  constexpr int NT = WGM * WGN * 64;
  constexpr int LS = G::BK + G::PAD;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;   // wave tile
  constexpr int TI = WTM / 32, TJ = WTN / 32;     // MFMA tiles per wave
  __shared__ __attribute__((aligned(16))) T smem[2][(BM + BN) * LS];

  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int z = blockIdx.z;
  const T* A = reinterpret_cast<const T*>(p.A) + z * p.sA;
  const T* B = reinterpret_cast<const T*>(p.B) + z * p.sB;

  // K range of this split (multiples of BK)
  const int nk_all = (p.K + G::BK - 1) / G::BK;
  const int per = (nk_all + splits - 1) / splits;
  const int kt0 = blockIdx.y * per;
  const int kt1 = min(nk_all, kt0 + per);
  const int k_end = min(p.K, kt1 * G::BK);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / WGN, wn = w % WGN;

  TileLoader<T, BM, NT> la;
  TileLoader<T, BN, NT> lb;
  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16{};

  if (kt0 < kt1) {
    la.load(A, p.lda, m0, p.M, kt0 * G::BK, k_end);
    lb.load(B, p.ldb, n0, p.N, kt0 * G::BK, k_end);
    la.store(smem[0]);
    lb.store(smem[0] + BM * LS);
  }
  __syncthreads();

  for (int kt = kt0; kt < kt1; ++kt) {
    const int cur = (kt - kt0) & 1;
    const bool more = kt + 1 < kt1;
    if (more) {
      la.load(A, p.lda, m0, p.M, (kt + 1) * G::BK, k_end);
      lb.load(B, p.ldb, n0, p.N, (kt + 1) * G::BK, k_end);
    }
    const T* sa = smem[cur] + wm * WTM * LS;
    const T* sb = smem[cur] + BM * LS + wn * WTN * LS;
#pragma unroll
    for (int ks = 0; ks < G::BK / G::KS; ++ks) {
      const int kk = ks * G::KS + (lane >> 5) * (G::KS / 2);
      typename G::frag fa[TI], fb[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) fa[i] = read_frag(sa, i * 32 + (lane & 31), kk);
#pragma unroll
      for (int j = 0; j < TJ; ++j) fb[j] = read_frag(sb, j * 32 + (lane & 31), kk);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = mfma(fa[i], fb[j], acc[i][j]);
    }
    if (more) {
      la.store(smem[cur ^ 1]);
      lb.store(smem[cur ^ 1] + BM * LS);
    }
    __syncthreads();
  }

  float pre[TI][TJ][16];
  const bool use_pre = prefetch_operand<BM, BN, WGM, WGN, EPI>(p, z, m0, n0, wm, wn, lane, splits, pre);
  gemm_epilogue<T, BM, BN, WGM, WGN, EPI, OutT>(p, z, m0, n0, wm, wn, lane, acc, splits, part, &smem[0][0], pre,
                                                use_pre);
}

// ---------------- direct-to-LDS variant (bf16, K % BK == 0) ----------------
// Operand tiles go from global memory straight into an S-stage LDS ring
// (global_load_lds: 16 bytes per lane, no register staging), so S-1 tiles are
// in flight while one is multiplied. Rows hold BK elements; their 16-byte
// chunks are XOR-swizzled by row so that the fragment reads of consecutive
// rows hit distinct banks. 128x128 wave tiles (16 MFMA tiles per wave) halve
// the LDS reads per MFMA of the 128x64 tiles above.
typedef __attribute__((address_space(3))) void lds_void_t;

template <int BK>
struct DL {
  static constexpr int CPR = BK / 8;            // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;          // rows per 1 KB load instruction
  static constexpr int RP256 = 256 / (BK * 2);  // rows per 256 bytes of LDS
  TTT_DEV static int swz(int r) { return (r / RP256) % CPR; }
};

// issue one ROWS x BK tile (rows row0.., k0..k0+BK) into `tile`; rows past
// nrows read row nrows-1 (their results are never stored)
template <int ROWS, int NW, int BK>
TTT_DEV void dl_issue(const bf16* __restrict__ base, int64_t ld, int row0, int nrows, int k0, bf16* tile, int w,
                      int lane) {
  typedef DL<BK> D;
  constexpr int NQ = ROWS / D::RPI;
  static_assert(NQ % NW == 0, "whole load instructions per wave");
  constexpr int PER = NQ / NW;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int q = w * PER + i;
    const int r = q * D::RPI + lane / D::CPR;
    const int c = (lane % D::CPR) ^ D::swz(r);
    const int gr = min(row0 + r, nrows - 1);
    const bf16* g = base + (int64_t)gr * ld + k0 + c * 8;
    __builtin_amdgcn_global_load_lds((const void*)g, (lds_void_t*)(tile + q * 512), 16, 0, 0);
  }
}

// The same loads with each lane's byte offset from the tile's first column
// computed once (`off`, see dl_offsets) and a uniform base per K tile: a load
// is then an M0 write and the load, with no 64-bit address arithmetic
// (operands must span less than 4 GiB; the launcher checks).
template <int ROWS, int NW, int BK>
TTT_DEV void dl_offsets(int64_t ld, int row0, int nrows, int w, int lane, uint32_t (&off)[ROWS / DL<BK>::RPI / NW]) {
  typedef DL<BK> D;
  constexpr int PER = ROWS / D::RPI / NW;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int q = w * PER + i;
    const int r = q * D::RPI + lane / D::CPR;
    const int c = (lane % D::CPR) ^ D::swz(r);
    const int gr = min(row0 + r, nrows - 1);
    off[i] = (uint32_t)(((int64_t)gr * ld + c * 8) * 2);
  }
}
template <int ROWS, int NW, int BK>
TTT_DEV void dl_issue_off(const bf16* __restrict__ base_k0, const uint32_t (&off)[ROWS / DL<BK>::RPI / NW], bf16* tile,
                          int w) {
  constexpr int PER = ROWS / DL<BK>::RPI / NW;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(reinterpret_cast<const char*>(base_k0) + off[i]),
                                     (lds_void_t*)(tile + (w * PER + i) * 512), 16, 0, 0);
}

template <int BK>
TTT_DEV bf16x8 dl_frag(const bf16* tile, int r, int c) {
  return *reinterpret_cast<const bf16x8*>(tile + r * BK + ((c ^ DL<BK>::swz(r)) << 3));
}

// wait until at most n of this wave's vector-memory operations are in flight
template <int N>
TTT_DEV void wait_vm() {
  static_assert(N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// MN-major operands (128-wide tiles, 64 K rows): K row r of a tile keeps its
// 16-byte chunk c at chunk c ^ 4 (r % 4), so the 4 rows x 2 chunks of a
// 16-lane transposing read hit distinct banks
TTT_DEV int mn_swz(int r) { return (r & 3) << 2; }

// this wave's 4 of the 16 one-KB loads of the 64 x 128 tile (K rows k0..,
// columns c0..c0+127)
TTT_DEV void mn_issue(const bf16* __restrict__ base, int64_t ld, int c0, int k0, bf16* tile, int w, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = w * 4 + i;
    const int r = q * 4 + (lane >> 4);
    const int c = (lane & 15) ^ mn_swz(r);
    const bf16* g = base + (int64_t)(k0 + r) * ld + c0 + c * 8;
    __builtin_amdgcn_global_load_lds((const void*)g, (lds_void_t*)(tile + q * 512), 16, 0, 0);
  }
}

// MFMA operand (32 rows d0.. on the lanes, K step ks of 16) of a [k][128]
// tile, read with two transposing reads. The K order within the step is
// permuted (k = 16 ks' + 8 (e / 4) + 4 (lane / 32) + e % 4 for element e);
// both operands are read this way, so the products pair up unchanged.
TTT_DEV bf16x8 mn_frag(const bf16* t, int d0, int ks, int lane) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_v4;
  const int k = ks * 16 + (lane >> 5) * 4 + ((lane & 15) >> 2);
  const int col = d0 + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
  const int c = col >> 3;
  const int o0 = k * 128 + ((c ^ mn_swz(k)) << 3) + (col & 7);
  const int o1 = (k + 8) * 128 + ((c ^ mn_swz(k + 8)) << 3) + (col & 7);
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(bf16*)(t + o0));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(bf16*)(t + o1));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  return __builtin_bit_cast(bf16x8, v);
}

template <int BM, int BN, int WGM, int WGN, int BK, int S, int EPI, typename OutT, bool MN = false>
__global__ __launch_bounds__(WGM * WGN * 64, WGM * WGN == 4 && EPI == EPI_SGD ? 2 : 1) void gemm_dl_kernel(GemmArgs p, int splits, float* part) {
  static_assert(!MN || (BM == 128 && BN == 128 && BK == 64), "MN-major operands: 128 x 128 tiles, 64 deep");
  static_assert(EPI != EPI_SGD || BN * (BM + 8) <= S * (BM + BN) * BK, "the staged SGD tile must fit in the ring");
  static_assert(S >= 2 && S <= 4, "ring depth");
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN, TI = WTM / 32, TJ = WTN / 32;
  constexpr int L = (BM + BN) / DL<BK>::RPI / NW;  // load instructions per wave per tile
  __shared__ __attribute__((aligned(1024))) bf16 smem[S][(BM + BN) * BK];

  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int z = blockIdx.z;
  const bf16* A = reinterpret_cast<const bf16*>(p.A) + z * p.sA;
  const bf16* B = reinterpret_cast<const bf16*>(p.B) + z * p.sB;
  const int nk_all = p.K / BK;
  const int per = (nk_all + splits - 1) / splits;
  const int kt0 = blockIdx.y * per;
  const int kt1 = min(nk_all, kt0 + per);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / WGN, wn = w % WGN;
  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16{};

  // each tile walks its K range from its own starting point ((tm + tn) mod
  // the range): tiles that share an operand panel then ask for a given K
  // slice an iteration or more apart, so one takes the miss beyond L2 and the
  // others find the slice in L2, instead of all waiting on the same miss
  // the epilogue's residual / master values, in flight during the main loop
  float pre[TI][TJ][16];
  const bool use_pre = prefetch_operand<BM, BN, WGM, WGN, EPI>(p, z, m0, n0, wm, wn, lane, splits, pre);
  const int nkt = kt1 - kt0;
  const int rot = nkt > 0 ? (tm + tn) % nkt : 0;
  // per-lane byte offsets of this wave's tile loads (K-contiguous operands)
  uint32_t offa[MN ? 1 : BM / DL<BK>::RPI / NW], offb[MN ? 1 : BN / DL<BK>::RPI / NW];
  if constexpr (!MN) {
    dl_offsets<BM, NW, BK>(p.lda, m0, p.M, w, lane, offa);
    dl_offsets<BN, NW, BK>(p.ldb, n0, p.N, w, lane, offb);
  }
  auto issue = [&](int kt, int st) {
    int kp = kt - kt0 + rot;
    kp = kt0 + (kp >= nkt ? kp - nkt : kp);
    if constexpr (MN) {
      mn_issue(A, p.lda, m0, kp * BK, smem[st], w, lane);
      mn_issue(B, p.ldb, n0, kp * BK, smem[st] + BM * BK, w, lane);
    } else {
      dl_issue_off<BM, NW, BK>(A + kp * BK, offa, smem[st], w);
      dl_issue_off<BN, NW, BK>(B + kp * BK, offb, smem[st] + BM * BK, w);
    }
  };
#pragma unroll
  for (int st = 0; st < S - 1; ++st)
    if (kt0 + st < kt1) issue(kt0 + st, st);

  for (int kt = kt0; kt < kt1; ++kt) {
    const int it = kt - kt0;
    // this wave's loads of tile kt are complete once at most the younger
    // tiles' loads are outstanding; the barrier then publishes every wave's
    // part and retires the reads of tile kt-1, whose stage is refilled next
    const int young = min(S - 2, kt1 - 1 - kt);
    if (young >= 2) wait_vm<2 * L>();
    else if (young == 1) wait_vm<L>();
    else wait_vm<0>();
    // a plain barrier: a fenced one would also drain the younger tiles' loads
    asm volatile("s_barrier" ::: "memory");
    const bf16* sa = smem[it % S] + (MN ? 0 : wm * WTM * BK);
    const bf16* sb = smem[it % S] + BM * BK + (MN ? 0 : wn * WTN * BK);
    // (K-contiguous operands) fragments double-buffered in registers: step
    // ks+1 is read from LDS while the MFMAs of step ks run
    bf16x8 fa[2][TI], fb[2][TJ];
    auto read = [&](int ks, int b) {
      const int c = ks * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < TI; ++i) fa[b][i] = dl_frag<BK>(sa, i * 32 + (lane & 31), c);
#pragma unroll
      for (int j = 0; j < TJ; ++j) fb[b][j] = dl_frag<BK>(sb, j * 32 + (lane & 31), c);
    };
    if constexpr (MN) {
      // every fragment of the tile is read before this wave issues its loads
      // of the tile S-1 ahead: the compiler makes a transposing LDS read wait
      // for all LDS-DMA loads in flight (it carries no alias information), so
      // a read after the issue would drain the prefetch before the tile's
      // MFMAs had run
      bf16x8 ga[BK / 16][TI], gb[BK / 16][TJ];
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
#pragma unroll
        for (int i = 0; i < TI; ++i) ga[ks][i] = mn_frag(sa, wm * WTM + i * 32, ks, lane);
#pragma unroll
        for (int j = 0; j < TJ; ++j) gb[ks][j] = mn_frag(sb, wn * WTN + j * 32, ks, lane);
      }
      if (kt + S - 1 < kt1) issue(kt + S - 1, (it + S - 1) % S);
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j) acc[i][j] = mfma(ga[ks][i], gb[ks][j], acc[i][j]);
      continue;
    }
    // the first step's fragments are read before this wave issues its loads
    // of the tile S-1 ahead (into the other stage), so their LDS latency
    // passes during that issue instead of before the first MFMA
    read(0, 0);
    if (kt + S - 1 < kt1) issue(kt + S - 1, (it + S - 1) % S);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks + 1 < BK / 16) read(ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = mfma(fa[ks & 1][i], fb[ks & 1][j], acc[i][j]);
    }
    // schedule: each step's MFMAs alternate with the next step's reads (mask
    // 0x8 = MFMA, 0x100 = LDS read)
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks + 1 < BK / 16) {
#pragma unroll
        for (int q = 0; q < TI + TJ; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x8, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x8, TI * TJ - (TI + TJ), 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x8, TI * TJ, 0);
      }
    }
  }
  __syncthreads();
  gemm_epilogue<bf16, BM, BN, WGM, WGN, EPI, OutT, (int)sizeof(smem)>(p, z, m0, n0, wm, wn, lane, acc, splits, part,
                                                                     &smem[0][0], pre, use_pre);
}

// sum split-K partials in order and apply the epilogue
template <typename T, int EPI, typename OutT>
__global__ void gemm_reduce(GemmArgs p, int splits, int batch, const float* __restrict__ part) {
  const int64_t MN = (int64_t)p.M * p.N;
  const int z = blockIdx.y;
  if constexpr (EPI == EPI_SWIGLU) {
    const int H = p.N / 2;
    OutT* C = reinterpret_cast<OutT*>(p.C) + z * p.sC;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < (int64_t)p.M * H;
         e += (int64_t)gridDim.x * blockDim.x) {
      const int row = (int)(e / H), u = (int)(e % H);
      const int64_t gi = (int64_t)row * p.N + gate_col(u);
      float g = 0.f, up = 0.f;
      for (int s = 0; s < splits; ++s) {
        g += part[((int64_t)s * batch + z) * MN + gi];
        up += part[((int64_t)s * batch + z) * MN + gi + 32];
      }
      C[(int64_t)row * p.ldc + u] = from_f32<OutT>(swiglu_acc(g, up));
    }
    return;
  } else if constexpr (EPI != EPI_SGD) {
    // four consecutive columns per thread (the launcher checks alignment)
    const int N4 = p.N / 4;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < MN / 4;
         e += (int64_t)gridDim.x * blockDim.x) {
      float4 v = reinterpret_cast<const float4*>(part + (int64_t)z * MN)[e];
      for (int s = 1; s < splits; ++s) {
        const float4 t = reinterpret_cast<const float4*>(part + ((int64_t)s * batch + z) * MN)[e];
        v.x += t.x; v.y += t.y; v.z += t.z; v.w += t.w;
      }
      const int row = (int)(e / N4), col = (int)(e % N4) * 4;
      float o[4] = {v.x, v.y, v.z, v.w};
      if constexpr (EPI == EPI_ADD) {
        const float4 r = *reinterpret_cast<const float4*>(p.R + z * p.sR + (int64_t)row * p.ldr + col);
        o[0] += r.x; o[1] += r.y; o[2] += r.z; o[3] += r.w;
      } else if constexpr (EPI == EPI_GELU) {
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = gelu_acc(o[k]);
      }
      OutT* C = reinterpret_cast<OutT*>(p.C) + z * p.sC + (int64_t)row * p.ldc + col;
      if constexpr (sizeof(OutT) == 4) {
        *reinterpret_cast<float4*>(C) = make_float4(o[0], o[1], o[2], o[3]);
      } else {
        bf16x4 b;
#pragma unroll
        for (int k = 0; k < 4; ++k) b[k] = (bf16)o[k];
        *reinterpret_cast<bf16x4*>(C) = b;
      }
    }
  } else {
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < MN; e += (int64_t)gridDim.x * blockDim.x) {
      float v = 0.f;
      for (int s = 0; s < splits; ++s) v += part[((int64_t)s * batch + z) * MN + e];
      apply<EPI, OutT, T>(p, z, (int)(e / p.N), (int)(e % p.N), v);
    }
  }
}

// ---------------- skinny products (M <= 8 rows of A, bf16) ----------------
// Memory-bound on B (the weights): each wave streams whole rows of B with
// 16-byte loads per lane and forms the M dot products against the rows of A
// (small, cache-resident), then reduces them across the wave. SwiGLU: a wave
// takes one hidden unit, i.e. its interleaved gate and up rows.
constexpr int GV_MAXM = GEMV_MAX_ROWS;
TTT_DEV float dot8(bf16x8 a, bf16x8 b) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s += (float)a[e] * (float)b[e];
  return s;
}

// EPI_ROPE for one row and one rotation pair: 64-column block cb, offset u < 32
template <typename OutT>
TTT_DEV void rope_store(const RopeOut& ro, int row, int cb, int u, float y1, float y2) {
  const int hd = ro.hd, half = hd / 2;
  const int hp = cb / hd, part = hp / ro.H, h = hp % ro.H;
  const int e1 = ((cb % hd) / 64) * 32 + u;
  const int sq = row / ro.S;
  const int64_t pos = ro.p0 + row % ro.S;
  if (part < 2 && ro.tab) {
    const float2 cs = ro.tab[pos * half + e1];
    const float a = y1, b = y2;
    y1 = a * cs.x - b * cs.y;
    y2 = a * cs.y + b * cs.x;
  }
  OutT* dst = part == 0 ? reinterpret_cast<OutT*>(ro.q) + (int64_t)row * ro.ldq
                        : reinterpret_cast<OutT*>(part == 1 ? ro.kc : ro.vc) + sq * ro.seq_stride +
                              (pos % ro.cap) * (int64_t)(ro.H * hd);
  dst += h * hd + e1;
  dst[0] = from_f32<OutT>(y1);
  dst[half] = from_f32<OutT>(y2);
}

template <int EPI, typename OutT>
__global__ __launch_bounds__(256) void gemv_kernel(GemmArgs p) {
  // each wave streams GV_ROWS outputs at once (more loads in flight)
  constexpr int GV_ROWS = 2;
  // SwiGLU and the rotary split both pair column c with c + 32 (64-column blocks)
  constexpr bool GLU = EPI == EPI_SWIGLU || EPI == EPI_ROPE;
  constexpr int NB = GLU ? 2 * GV_ROWS : GV_ROWS;  // rows of B per wave step
  const int z = blockIdx.z;
  const bf16* A = reinterpret_cast<const bf16*>(p.A) + z * p.sA;
  const bf16* B = reinterpret_cast<const bf16*>(p.B) + z * p.sB;
  const int lane = threadIdx.x & 63;
  const int nw = gridDim.x * 4;
  const int nout = GLU ? p.N / 2 : p.N;
  // RMSNorm folded into the A operand: each wave takes its rows' 1/rms itself
  const float* X = p.nx ? p.nx + z * p.snx : nullptr;
  const bf16* G = reinterpret_cast<const bf16*>(p.ng);
  float rs[GV_MAXM];
#pragma unroll
  for (int m = 0; m < GV_MAXM; ++m) {
    rs[m] = 0.f;
    if (X && m < p.M) {
      float ss = 0.f;
      for (int k = lane * 8; k < p.K; k += 512) {
        const float4 x0 = *reinterpret_cast<const float4*>(X + m * p.ldnx + k);
        const float4 x1 = *reinterpret_cast<const float4*>(X + m * p.ldnx + k + 4);
        ss += x0.x * x0.x + x0.y * x0.y + x0.z * x0.z + x0.w * x0.w;
        ss += x1.x * x1.x + x1.y * x1.y + x1.z * x1.z + x1.w * x1.w;
      }
      rs[m] = rsqrtf(wave_sum(ss) / p.K + p.neps);
    }
  }
  for (int o0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * GV_ROWS; o0 < nout; o0 += nw * GV_ROWS) {
    const bf16* brow[NB];
#pragma unroll
    for (int q = 0; q < GV_ROWS; ++q) {
      const int o = min(o0 + q, nout - 1);  // a tail wave repeats the last output (not stored)
      const int n = GLU ? gate_col(o) : o;
      brow[q] = B + (int64_t)n * p.ldb;
      if constexpr (GLU) brow[GV_ROWS + q] = brow[q] + 32 * p.ldb;  // the matching up row
    }
    float acc[NB][GV_MAXM];
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
      for (int m = 0; m < GV_MAXM; ++m) acc[q][m] = 0.f;
    for (int k = lane * 8; k < p.K; k += 512) {
      bf16x8 bv[NB];
#pragma unroll
      for (int q = 0; q < NB; ++q) bv[q] = *reinterpret_cast<const bf16x8*>(brow[q] + k);
      bf16x8 gv;
      if (X) gv = *reinterpret_cast<const bf16x8*>(G + k);
#pragma unroll
      for (int m = 0; m < GV_MAXM; ++m) {
        if (m < p.M) {
          bf16x8 av;
          if (X) {
            const float4 x0 = *reinterpret_cast<const float4*>(X + m * p.ldnx + k);
            const float4 x1 = *reinterpret_cast<const float4*>(X + m * p.ldnx + k + 4);
            const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) av[e] = (bf16)(xv[e] * (rs[m] * (float)gv[e]));
          } else {
            av = *reinterpret_cast<const bf16x8*>(A + (int64_t)m * p.lda + k);
          }
#pragma unroll
          for (int q = 0; q < NB; ++q) acc[q][m] += dot8(av, bv[q]);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
      for (int m = 0; m < GV_MAXM; ++m)
        if (m < p.M) acc[q][m] = wave_sum(acc[q][m]);
    // lane m writes row m of each output
    if (lane < p.M) {
#pragma unroll
      for (int q = 0; q < GV_ROWS; ++q) {
        const int o = o0 + q;
        if (o >= nout) break;
        float v = 0.f, v2 = 0.f;
#pragma unroll
        for (int m = 0; m < GV_MAXM; ++m)
          if (lane == m) { v = acc[q][m]; if constexpr (GLU) v2 = acc[GV_ROWS + q][m]; }
        if constexpr (EPI == EPI_ROPE)
          rope_store<OutT>(p.rope, lane, (o >> 5) * 64, o & 31, v, v2);
        else if constexpr (GLU)
          reinterpret_cast<OutT*>(p.C)[z * p.sC + (int64_t)lane * p.ldc + o] = from_f32<OutT>(swiglu_acc(v, v2));
        else
          apply<EPI, OutT, bf16>(p, z, lane, o, v);
      }
    }
  }
}

template <int EPI, typename OutT>
hipError_t launch_gemv(const GemmArgs& p, int batch, hipStream_t st) {
  if (p.nx && (p.ldnx % 4 || p.snx % 4 || !p.ng || reinterpret_cast<uintptr_t>(p.nx) % 16 ||
               reinterpret_cast<uintptr_t>(p.ng) % 16))
    return hipErrorInvalidValue;
  const int nout = (EPI == EPI_SWIGLU || EPI == EPI_ROPE) ? p.N / 2 : p.N;
  const int blocks = std::min((nout + 7) / 8, 4096);  // 4 waves of 2 outputs
  TTT_LAUNCH((gemv_kernel<EPI, OutT>), dim3(blocks, 1, batch), dim3(256), 0, st, p);
  return hipGetLastError();
}

// test hook: 0 auto, 1 = 256x256, 2 = 256x128, 3 = 128x128, 4 = 256x256 direct-to-LDS
// (BK 64, two stages), 5 = the same with BK 32 and four stages, 6 / 7 = 128x128
// direct-to-LDS with two / three stages, 8 / 9 = 128x128 with four stages of BK
// 64 / 32 (each + split-K); bits 8.. force the number of K splits (0: chosen)
int g_force_tile = 0;
int g_force_splits = 0;

template <int BM, int BN, int WGM, int WGN, int BK, int S, int EPI, typename OutT, bool MN = false>
hipError_t launch_dl(const GemmArgs& p, int batch, int splits, float* ws, hipStream_t st) {
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  TTT_LAUNCH((gemm_dl_kernel<BM, BN, WGM, WGN, BK, S, EPI, OutT, MN>), dim3(tiles, splits, batch),
                     dim3(WGM * WGN * 64), 0, st, p, splits, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  if constexpr (EPI == EPI_ROPE) return hipErrorInvalidValue;  // never split
  if constexpr ((EPI == EPI_STORE || EPI == EPI_ADD) && sizeof(OutT) == 4) {
    if (p.split_out) {  // the consumer adds the partials
      *p.split_out = splits;
      return hipSuccess;
    }
  }
  const int64_t elems = (int64_t)p.M * p.N;
  int blocks = (int)std::min<int64_t>((elems + 255) / 256, 4096);
  TTT_LAUNCH((gemm_reduce<bf16, EPI, OutT>), dim3(blocks, batch), dim3(256), 0, st, p, splits, batch, ws);
  return hipGetLastError();
}

template <typename T, int BM, int BN, int WGM, int WGN, int EPI, typename OutT>
hipError_t launch_t(const GemmArgs& p, int batch, int splits, float* ws, hipStream_t st) {
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  TTT_LAUNCH((gemm_kernel<T, BM, BN, WGM, WGN, EPI, OutT>), dim3(tiles, splits, batch),
                     dim3(WGM * WGN * 64), 0, st, p, splits, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  if constexpr (EPI == EPI_ROPE) return hipErrorInvalidValue;  // never split
  if constexpr ((EPI == EPI_STORE || EPI == EPI_ADD) && sizeof(OutT) == 4) {
    if (p.split_out) {  // the consumer adds the partials
      *p.split_out = splits;
      return hipSuccess;
    }
  }
  const int64_t MN = (int64_t)p.M * p.N;
  int blocks = (int)std::min<int64_t>((MN + 255) / 256, 4096);
  TTT_LAUNCH((gemm_reduce<T, EPI, OutT>), dim3(blocks, batch), dim3(256), 0, st, p, splits, batch, ws);
  return hipGetLastError();
}

// K splits that bring `tiles` blocks up to `target` (at least 8 K tiles per
// split); with max_kt > 0, also until a split has at most max_kt K tiles
template <typename T>
int k_splits(const GemmArgs& p, int batch, int64_t tiles, int64_t target, int64_t ws_elems, int max_kt = 0) {
  // the reduce of plain / residual / GELU outputs moves 4 columns per thread
  const auto al = [](const void* q) { return reinterpret_cast<uintptr_t>(q) % 16 == 0; };
  if (!(p.N % 4 == 0 && p.ldc % 4 == 0 && p.sC % 4 == 0 && al(p.C) &&
        (!p.R || (p.ldr % 4 == 0 && p.sR % 4 == 0 && al(p.R)))))
    return 1;
  int splits = 1;
  const int nk = (p.K + GT<T>::BK - 1) / GT<T>::BK;
  if (g_force_splits > 0)
    return (int64_t)g_force_splits * batch * p.M * p.N <= ws_elems && nk >= g_force_splits ? g_force_splits : 1;
  while ((tiles * splits < target || (max_kt > 0 && tiles * splits < 2 * target && nk / splits > max_kt)) &&
         nk / (splits * 2) >= 8 && splits < 8 && (int64_t)(splits * 2) * batch * p.M * p.N <= ws_elems)
    splits *= 2;
  return splits;
}

// K splits of the 256x256 direct-to-LDS kernel (one block per CU): with
// fewer tiles than half the CUs, as many splits as fill the CUs in one round
// (a second, partial round costs more than it spreads); otherwise only a long
// K (over 128 K tiles), halved down to at most 128 K tiles per split.
template <int BK>
int dl_splits(const GemmArgs& p, int batch, int64_t tiles, int64_t slots, int64_t ws_elems) {
  const auto al = [](const void* q) { return reinterpret_cast<uintptr_t>(q) % 16 == 0; };
  if (!(p.N % 4 == 0 && p.ldc % 4 == 0 && p.sC % 4 == 0 && al(p.C) &&
        (!p.R || (p.ldr % 4 == 0 && p.sR % 4 == 0 && al(p.R)))))
    return 1;
  const int nk = p.K / BK;
  const auto fits = [&](int sp) { return (int64_t)sp * batch * p.M * p.N <= ws_elems && nk / sp >= 8; };
  if (g_force_splits > 0) return fits(g_force_splits) ? g_force_splits : 1;
  int sp = 1;
  if (tiles < 128) {
    while (sp < 8 && tiles * (sp + 1) <= slots && fits(sp + 1)) ++sp;
  } else {
    while (nk / sp > 128 && sp < 8 && fits(sp * 2)) sp *= 2;
  }
  return sp;
}

template <typename T, int EPI, typename OutT>
hipError_t pick(const GemmArgs& p, int batch, float* ws, int64_t ws_elems, hipStream_t st) {
  // 256x256 tiles (8 waves, one block per CU) when they give >= 2 blocks per
  // CU; 256x128 (4 waves) when M is a multiple of 256 and those fill the CUs;
  // otherwise 128x128 (4 waves, two blocks per CU). Each splits K when the
  // tile count alone leaves CUs idle.
  constexpr int CUS = 256;
  const int64_t t256 = (int64_t)((p.M + 255) / 256) * ((p.N + 255) / 256) * batch;
  const int64_t t2x1 = (int64_t)((p.M + 255) / 256) * ((p.N + 127) / 128) * batch;
  const int64_t t128 = (int64_t)((p.M + 127) / 128) * ((p.N + 127) / 128) * batch;
  if (!ws) ws_elems = 0;
  if constexpr (sizeof(T) == 2 && (EPI == EPI_SGD || EPI == EPI_STORE)) {
    if (p.mn) {
      const auto al = [](const void* q) { return reinterpret_cast<uintptr_t>(q) % 16 == 0; };
      if (p.nx || p.M % 128 || p.N % 128 || p.K % 64 || p.lda % 8 || p.ldb % 8 || p.sA % 8 || p.sB % 8 || !al(p.A) ||
          !al(p.B))
        return hipErrorInvalidValue;
      return launch_dl<128, 128, 2, 2, 64, 2, EPI, OutT, true>(p, batch, 1, nullptr, st);
    }
  }
  if (p.mn) return hipErrorInvalidValue;
  int cfg = g_force_tile;
  if constexpr (sizeof(T) == 2 && EPI != EPI_SGD) {
    // a few rows of A (decode): one streaming pass over B
    if (!cfg && p.M <= GV_MAXM) return launch_gemv<EPI, OutT>(p, batch, st);
  }
  if (p.nx) return hipErrorInvalidValue;  // a folded RMSNorm needs the skinny kernel
  // the direct-to-LDS kernels address each operand with 32-bit byte offsets
  const bool small32 = (int64_t)p.M * p.lda * 2 < (1ll << 32) && (int64_t)p.N * p.ldb * 2 < (1ll << 32) &&
                       (int64_t)p.K * 2 < (1ll << 31);
  if (!cfg) {
    // direct-to-LDS 256x256 when there are enough large tiles (or K >= 8192,
    // long enough for split-K over few tiles to fill the CUs in one round);
    // register-staged kernels otherwise
    // (also when a short K leaves 128x128 tiles unsplit over more than one
    // round of block slots, and the large tiles alone cover over half the CUs)
    const bool dl = sizeof(T) == 2 && p.K % 64 == 0 && small32;
    const bool ragged128 = t256 > CUS / 2 && t128 > 2 * CUS && p.K <= 48 * 64;
    if (dl && EPI != EPI_SGD && (t256 >= CUS || ragged128 || p.K >= 8192)) cfg = 4;
    else if (dl) cfg = 6;
    else cfg = t256 >= 2 * CUS ? 1 : 3;
  }
  if (cfg == 1) {
    const int sp = k_splits<T>(p, batch, t256, CUS, ws_elems);
    return launch_t<T, 256, 256, 2, 4, EPI, OutT>(p, batch, sp, sp > 1 ? ws : nullptr, st);
  }
  if (!small32 && cfg >= 4) cfg = (cfg == 4 || cfg == 5) ? 1 : 3;
  if constexpr (sizeof(T) == 2) {
    if ((cfg == 6 || cfg == 7) && p.K % 64 == 0) {
      // 128x128, two blocks per CU: at least 3/4 of the 512 slots, and short K
      // ranges per split (long ones keep splitting while the blocks fit twice)
      // (a short K over >= 128 tiles gains nothing from a split and its reduce)
      const int sp = cfg == 6 && t128 >= 128 && p.K <= 48 * 64
                         ? 1
                         : k_splits<T>(p, batch, t128, cfg == 6 ? 3 * CUS / 2 : CUS, ws_elems, cfg == 6 ? 48 : 0);
      float* w = sp > 1 ? ws : nullptr;
      if (cfg == 6) return launch_dl<128, 128, 2, 2, 64, 2, EPI, OutT>(p, batch, sp, w, st);
      return launch_dl<128, 128, 2, 2, 64, 3, EPI, OutT>(p, batch, sp, w, st);
    }
    if ((cfg == 8 && p.K % 64 == 0) || (cfg == 9 && p.K % 32 == 0)) {
      const int sp = k_splits<T>(p, batch, t128, cfg == 8 ? CUS : 2 * CUS, ws_elems);
      float* w = sp > 1 ? ws : nullptr;
      if (cfg == 8) return launch_dl<128, 128, 2, 2, 64, 4, EPI, OutT>(p, batch, sp, w, st);
      return launch_dl<128, 128, 2, 2, 32, 4, EPI, OutT>(p, batch, sp, w, st);
    }
    if (EPI != EPI_SGD && ((cfg == 4 && p.K % 64 == 0) || (cfg == 5 && p.K % 32 == 0))) {
      const int sp = cfg == 4 ? dl_splits<64>(p, batch, t256, CUS, ws_elems) : k_splits<T>(p, batch, t256, CUS, ws_elems);
      float* w = sp > 1 ? ws : nullptr;
      if constexpr (EPI != EPI_SGD) {
        if (cfg == 4) return launch_dl<256, 256, 2, 4, 64, 2, EPI, OutT>(p, batch, sp, w, st);
        return launch_dl<256, 256, 2, 4, 32, 4, EPI, OutT>(p, batch, sp, w, st);
      }
    }
  }
  if (cfg >= 6) cfg = 3;  // 6..9 where they do not apply
  if (cfg >= 4) cfg = 1;
  if (cfg == 2) {
    const int sp = k_splits<T>(p, batch, t2x1, CUS, ws_elems);
    return launch_t<T, 256, 128, 2, 2, EPI, OutT>(p, batch, sp, sp > 1 ? ws : nullptr, st);
  }
  const int sp = k_splits<T>(p, batch, t128, 2 * CUS, ws_elems);
  return launch_t<T, 128, 128, 2, 2, EPI, OutT>(p, batch, sp, sp > 1 ? ws : nullptr, st);
}

template <typename T>
hipError_t dispatch(const GemmArgs& p, int epi, bool out_f32, int batch, float* ws, int64_t ws_elems,
                    hipStream_t st) {
  if (epi == EPI_STORE)
    return out_f32 ? pick<T, EPI_STORE, float>(p, batch, ws, ws_elems, st)
                   : pick<T, EPI_STORE, T>(p, batch, ws, ws_elems, st);
  if (epi == EPI_ADD) return pick<T, EPI_ADD, float>(p, batch, ws, ws_elems, st);
  if (epi == EPI_SGD) return pick<T, EPI_SGD, T>(p, batch, ws, ws_elems, st);
  if (epi == EPI_SWIGLU)
    return out_f32 ? pick<T, EPI_SWIGLU, float>(p, batch, ws, ws_elems, st)
                   : pick<T, EPI_SWIGLU, T>(p, batch, ws, ws_elems, st);
  if (epi == EPI_GELU)
    return out_f32 ? pick<T, EPI_GELU, float>(p, batch, ws, ws_elems, st)
                   : pick<T, EPI_GELU, T>(p, batch, ws, ws_elems, st);
  if (epi == EPI_ROPE) return pick<T, EPI_ROPE, T>(p, batch, nullptr, 0, st);  // never split
  return hipErrorInvalidValue;
}

}  // namespace

void gemm_force_tile(int cfg) {
  g_force_tile = cfg & 255;
  g_force_splits = cfg >> 8;
}

hipError_t gemm_launch(const GemmArgs& p, int dtype, int epi, bool out_f32, int batch, float* ws, int64_t ws_elems,
                       hipStream_t st) {
  if (p.split_out) *p.split_out = 1;
  if (p.M <= 0 || p.N <= 0 || batch <= 0) return hipSuccess;
  if (p.K % (dtype == 1 ? 8 : 4)) return hipErrorInvalidValue;
  if (epi == EPI_SWIGLU && p.N % 64) return hipErrorInvalidValue;
  if (epi == EPI_ROPE) {
    const RopeOut& r = p.rope;
    if (batch != 1 || r.hd % 64 || r.H < 1 || p.N != 3 * r.H * r.hd || r.S < 1 || r.cap < 32 || !r.q || !r.kc ||
        !r.vc || r.ldq < r.H * r.hd || p.M % r.S || r.p0 < 0 || r.p0 + r.S > ((int64_t)1 << 31))
      return hipErrorInvalidValue;
  }
  if (dtype == 1) return dispatch<bf16>(p, epi, out_f32, batch, ws, ws_elems, st);
  return dispatch<float>(p, epi, out_f32, batch, ws, ws_elems, st);
}

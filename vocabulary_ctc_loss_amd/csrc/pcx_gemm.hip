// Head projections on the CDNA4 matrix cores, with the loss-specific epilogues.
//
// "Pruned CTC for Memory-Efficient Large-Vocabulary ASR Training":
//  * Sec. 3.1: logits Z = X W^T + 1 b^T; Eq. 1: normalizer lambda_m =
//    log sum_v exp Z[m][v] over the whole vocabulary.
//  * App. B.1: the vocabulary is processed in chunks; the normalizer is
//    accumulated in FP64 and subtracted in FP64 before S = Z[:, U] - lambda is
//    rounded once to FP32; the backward pass recomputes each chunk, combines
//    the sparse (selected-class) and dense terms before the products, writes
//    the chunk's own weight-gradient rows and adds its contribution to the
//    input gradient.
//  * App. B.2 (Table 5 strategy): FP64 normalization, reuse of S for the
//    selected classes in the backward pass, FP32 gradient products and sums;
//    the recomputed probabilities of the other classes subtract an FP32 copy
//    of the normalizer.
//
// One GEMM core serves all four products.  A work-group of 256 threads
// (4 wavefronts of 64) computes a 128 x 128 fp32 tile as 2 x 2 wavefront
// tiles of 2 x 2 MFMA 32x32 blocks: v_mfma_f32_32x32x2f32 for fp32 inputs,
// v_mfma_f32_32x32x16_bf16 for bf16 inputs, fp32 accumulation in both.  Each
// k-tile is 128 bytes of every operand row, staged through double-buffered
// LDS; within a k-tile, lane half h (lanes 32h..32h+31) feeds the k values of
// the half-row it owns, which is just a fixed relabelling of the reduction
// index shared by both operands.  Operands are K-contiguous (row-major along
// the reduction) or MN-contiguous.  fp32 MN-contiguous tiles are staged as
// they lie ([k][mn]) and read one k row per MFMA; for bf16 the one product
// with an MN-contiguous operand on the hot path (dX = dZ W_c) reads a
// transposed copy of the chunk's weight rows instead.
#include <float.h>
#include <math.h>

#include "pcx_common.h"

namespace pcx {

namespace {

constexpr int BM = GEMM_BM;
constexpr int BN = GEMM_BN;
constexpr int NT = GEMM_THREADS;
constexpr int ROW_BYTES = 128;  // one operand row of a k-tile
constexpr int PAD_BYTES = 16;   // LDS row padding
constexpr int TILE_LD = BM + 4; // accumulator tile in LDS, column-major [col][row]
constexpr int EPI_BYTES = BN * TILE_LD * 4;

template <typename T>
struct Geo {
  static constexpr int VEC = Elem<T>::VEC;
  static constexpr int BK = ROW_BYTES / (int)sizeof(T);                 // 32 fp32 / 64 bf16
  static constexpr int LDK = (ROW_BYTES + PAD_BYTES) / (int)sizeof(T);  // LDS row stride
  static constexpr int OPER = 128 * LDK;                                // one operand buffer
  static constexpr int STAGE_BYTES = 2 * 2 * OPER * (int)sizeof(T);
};

constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int SMEM_BYTES = cmax(cmax(Geo<float>::STAGE_BYTES, Geo<bf16_t>::STAGE_BYTES), EPI_BYTES);

union Vec16 {
  uint4 u;
  float f[4];
  bf16_t h[8];
};

// Logical tile id for hardware work-group id `bid`: consecutive ids are
// dispatched round-robin over the 8 XCDs, so give every XCD a contiguous run
// of logical tiles (which then share operand rows in that XCD's L2).
__device__ __forceinline__ int xcd_tile(int bid, int nblocks) {
  const int X = 8;
  const int per = nblocks / X, rem = nblocks % X;
  const int xcd = bid % X, local = bid / X;
  return xcd * per + min(xcd, rem) + local;
}

// LDS layouts of one staged 128 (mn) x BK (k) operand tile:
//  * row layout [mn][LDK], k contiguous: K-contiguous operands, and bf16
//    MN-contiguous operands (transposed element by element on the way in);
//  * column layout [k][LDM], mn contiguous: fp32 MN-contiguous operands,
//    written straight from the 16-byte global loads.
constexpr int LDM = 128 + 4;

template <typename T, bool KMAJOR>
struct ColLayout {
  static constexpr bool value = !KMAJOR && sizeof(T) == 4;
};

// Global -> registers -> LDS staging of one operand tile.
// KMAJOR: element (mn, k) is g[mn * ld + k]; otherwise g[k * ld + mn].
template <typename T, bool KMAJOR>
struct Stage {
  static constexpr int VEC = Geo<T>::VEC;
  static constexpr int BK = Geo<T>::BK;
  static constexpr int LDK = Geo<T>::LDK;
  static constexpr bool COL = ColLayout<T, KMAJOR>::value;

  __device__ static __forceinline__ void coords(int q, int& mn, int& k) {
    const int v = threadIdx.x + NT * q;
    if (KMAJOR) {
      mn = v / (BK / VEC);
      k = (v % (BK / VEC)) * VEC;
    } else {
      k = v / (128 / VEC);
      mn = (v % (128 / VEC)) * VEC;
    }
  }

  __device__ static __forceinline__ void load(const T* __restrict__ g, long long ld, int mn0,
                                              int mn_lim, int k0, int k_lim, bool vec_ok,
                                              Vec16 (&r)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int mn, k;
      coords(q, mn, k);
      const int gm = mn0 + mn, gk = k0 + k;
      if (KMAJOR) {
        if (vec_ok && gm < mn_lim && gk + VEC <= k_lim) {
          r[q].u = *reinterpret_cast<const uint4*>(g + (long long)gm * ld + gk);
        } else {
          Vec16 t;
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            T x = T(0);
            if (gm < mn_lim && gk + e < k_lim) x = g[(long long)gm * ld + gk + e];
            reinterpret_cast<T*>(&t)[e] = x;
          }
          r[q] = t;
        }
      } else {
        if (vec_ok && gk < k_lim && gm + VEC <= mn_lim) {
          r[q].u = *reinterpret_cast<const uint4*>(g + (long long)gk * ld + gm);
        } else {
          Vec16 t;
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            T x = T(0);
            if (gk < k_lim && gm + e < mn_lim) x = g[(long long)gk * ld + gm + e];
            reinterpret_cast<T*>(&t)[e] = x;
          }
          r[q] = t;
        }
      }
    }
  }

  __device__ static __forceinline__ void store(T* __restrict__ s, const Vec16 (&r)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int mn, k;
      coords(q, mn, k);
      if (KMAJOR) {
        *reinterpret_cast<uint4*>(s + mn * LDK + k) = r[q].u;
      } else if (COL) {
        *reinterpret_cast<uint4*>(s + k * LDM + mn) = r[q].u;
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) s[(mn + e) * LDK + k] = reinterpret_cast<const T*>(&r[q])[e];
      }
    }
  }
};

// MFMA work on one staged k-tile for this wavefront's 64 x 64 block.
//
// fp32: a k-tile holds 32 k values; the 16 v_mfma_f32_32x32x2f32 steps s of
// a lane in half h consume k = 16*(s/8) + 8*h + s%8.  Four consecutive steps
// read four consecutive k, so a row-layout fragment is one 16-byte LDS read,
// and in the column layout the two lane halves read rows 8 apart, which lands
// them on disjoint LDS banks.
template <typename T, bool ACOL, bool BCOL>
struct Mma;

template <bool COL>
__device__ __forceinline__ f32x4 frag_f32(const float* __restrict__ S, int row, int h, int kc) {
  constexpr int LDK = Geo<float>::LDK;
  const int k0 = ((kc >> 1) << 4) + (h << 3) + ((kc & 1) << 2);
  if (!COL) return *reinterpret_cast<const f32x4*>(S + row * LDK + k0);
  f32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = S[(k0 + e) * LDM + row];
  return v;
}

template <bool ACOL, bool BCOL>
struct Mma<float, ACOL, BCOL> {
  __device__ static __forceinline__ void run(const float* __restrict__ As,
                                             const float* __restrict__ Bs, f32x16 (&acc)[2][2],
                                             int wm, int wn) {
    const int lane = threadIdx.x & 63, i = lane & 31, h = lane >> 5;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      f32x4 a[2], b[2];
      a[0] = frag_f32<ACOL>(As, wm * 64 + i, h, kc);
      a[1] = frag_f32<ACOL>(As, wm * 64 + 32 + i, h, kc);
      b[0] = frag_f32<BCOL>(Bs, wn * 64 + i, h, kc);
      b[1] = frag_f32<BCOL>(Bs, wn * 64 + 32 + i, h, kc);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[mi][e], b[ni][e], acc[mi][ni],
                                                               0, 0, 0);
    }
  }
};

// bf16: a k-tile holds 64 k values; lane half h feeds k in [32h, 32h + 32),
// eight per v_mfma_f32_32x32x16_bf16 (row layout only).
template <>
struct Mma<bf16_t, false, false> {
  static constexpr int LDK = Geo<bf16_t>::LDK;
  __device__ static __forceinline__ void run(const bf16_t* __restrict__ As,
                                             const bf16_t* __restrict__ Bs, f32x16 (&acc)[2][2],
                                             int wm, int wn) {
    const int lane = threadIdx.x & 63, i = lane & 31, h = lane >> 5;
    const bf16_t* a0 = As + (wm * 64 + i) * LDK + h * 32;
    const bf16_t* b0 = Bs + (wn * 64 + i) * LDK + h * 32;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 a[2], b[2];
      a[0] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(a0 + j * 8));
      a[1] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(a0 + 32 * LDK + j * 8));
      b[0] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(b0 + j * 8));
      b[1] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(b0 + 32 * LDK + j * 8));
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
  }
};

// acc = A[m0:m0+128, k] . B[n0:n0+128, k]^T over k in [k_begin, k_end).
// Rows/columns past the limits and k past k_end read as zero.  Ends with a
// barrier, so the caller may reuse `smem` right away.
template <typename T, bool AK, bool BK_>
__device__ __forceinline__ void gemm_tile(const T* __restrict__ A, long long lda, int m0, int m_lim,
                                          const T* __restrict__ B, long long ldb, int n0, int n_lim,
                                          int k_begin, int k_end, bool a_vec, bool b_vec,
                                          f32x16 (&acc)[2][2], char* smem) {
  constexpr int BK = Geo<T>::BK;
  constexpr int OPER = Geo<T>::OPER;
  constexpr bool ACOL = ColLayout<T, AK>::value;
  constexpr bool BCOL = ColLayout<T, BK_>::value;
  T* As = reinterpret_cast<T*>(smem);
  T* Bs = As + 2 * OPER;
  const int w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
  const int nk = (k_end - k_begin + BK - 1) / BK;
  if (nk <= 0) return;
  Vec16 ra[4], rb[4];
  Stage<T, AK>::load(A, lda, m0, m_lim, k_begin, k_end, a_vec, ra);
  Stage<T, BK_>::load(B, ldb, n0, n_lim, k_begin, k_end, b_vec, rb);
  Stage<T, AK>::store(As, ra);
  Stage<T, BK_>::store(Bs, rb);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k0 = k_begin + (kt + 1) * BK;
      Stage<T, AK>::load(A, lda, m0, m_lim, k0, k_end, a_vec, ra);
      Stage<T, BK_>::load(B, ldb, n0, n_lim, k0, k_end, b_vec, rb);
    }
    Mma<T, ACOL, BCOL>::run(As + cur * OPER, Bs + cur * OPER, acc, wm, wn);
    if (more) {
      Stage<T, AK>::store(As + (cur ^ 1) * OPER, ra);
      Stage<T, BK_>::store(Bs + (cur ^ 1) * OPER, rb);
    }
    __syncthreads();
  }
}

// Accumulator element (mi, ni, r) of lane l sits at tile row
// wm*64 + mi*32 + 8*(r/4) + 4*(l/32) + r%4 and tile column wn*64 + ni*32 + l%32.
__device__ __forceinline__ void acc_to_lds(const f32x16 (&acc)[2][2], float* __restrict__ Zt) {
  const int lane = threadIdx.x & 63, i = lane & 31, h = lane >> 5;
  const int w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int col = wn * 64 + ni * 32 + i;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int row = wm * 64 + mi * 32 + rg * 8 + h * 4;
        f32x4 v = {acc[mi][ni][rg * 4 + 0], acc[mi][ni][rg * 4 + 1], acc[mi][ni][rg * 4 + 2],
                   acc[mi][ni][rg * 4 + 3]};
        *reinterpret_cast<f32x4*>(Zt + col * TILE_LD + row) = v;
      }
    }
}

// (m1, s1) <- fold of two log-sum-exp partials (max, sum of exp(z - max)).
__device__ __forceinline__ void lse_fold(float& m1, double& s1, float m2, double s2) {
  if (m2 == -INFINITY) return;
  if (m1 == -INFINITY) {
    m1 = m2;
    s1 = s2;
  } else if (m2 > m1) {
    s1 = s1 * exp((double)m1 - (double)m2) + s2;
    m1 = m2;
  } else {
    s1 = s1 + s2 * exp((double)m2 - (double)m1);
  }
}

template <typename T>
__device__ __forceinline__ float load_f32(const T* p, long long i) {
  return Elem<T>::to_f32(p[i]);
}

// ------------------------------------------------------------- forward
// One work-group: 128 frames x one LSE_SPAN-wide vocabulary span, walked in
// 128-column tiles.  Per tile: MFMA logits, + bias, then per row the FP64
// sum of exp(z - tile-row max) folded into the row's running partial, and a
// gather of the selected columns into Zsel (class-major, K x M).
template <typename T>
__global__ __launch_bounds__(NT, 2) void k_fwd_lse(const T* __restrict__ X, const T* __restrict__ W,
                                                   const T* __restrict__ bias, int M, int D, int V,
                                                   const int* __restrict__ col2sel,
                                                   float* __restrict__ Zsel,
                                                   double2* __restrict__ part, int nspan,
                                                   int mtiles, int vec_ok) {
  __shared__ __attribute__((aligned(16))) char smem[SMEM_BYTES];
  __shared__ int s_sel[BN];
  __shared__ float s_bias[BN];
  __shared__ float s_pm[BM];
  __shared__ double s_ps[BM];
  const int lin = xcd_tile(blockIdx.x, gridDim.x);
  const int mt = lin % mtiles, sp = lin / mtiles;
  const int m0 = mt * BM;
  const int c_begin = sp * LSE_SPAN, c_end = min(V, c_begin + LSE_SPAN);
  const int r = threadIdx.x & (BM - 1), hh = threadIdx.x >> 7;
  const int m = m0 + r;
  float run_m = -INFINITY;
  double run_s = 0.0;
  float* Zt = reinterpret_cast<float*>(smem);
  for (int n0 = c_begin; n0 < c_end; n0 += BN) {
    f32x16 acc[2][2];
    gemm_tile<T, true, true>(X, D, m0, M, W, D, n0, c_end, 0, D, vec_ok, vec_ok, acc, smem);
    acc_to_lds(acc, Zt);
    if (threadIdx.x < BN) {
      const int v = n0 + threadIdx.x;
      s_sel[threadIdx.x] = v < c_end ? col2sel[v] : -1;
      s_bias[threadIdx.x] = (bias != nullptr && v < c_end) ? load_f32(bias, v) : 0.f;
    }
    __syncthreads();
    const int ncol = min(BN, c_end - n0);
    const int cb = hh * 64, ce = min(cb + 64, ncol);
    if (m < M && ce > cb) {
      float mx = -INFINITY;
      for (int c = cb; c < ce; ++c) mx = fmaxf(mx, Zt[c * TILE_LD + r] + s_bias[c]);
      double s = 0.0;
      const double dmx = (double)mx;
      for (int c = cb; c < ce; ++c) {
        const float z = Zt[c * TILE_LD + r] + s_bias[c];
        s += exp((double)z - dmx);
        const int sel = s_sel[c];
        if (sel >= 0) Zsel[(long long)sel * M + m] = z;
      }
      lse_fold(run_m, run_s, mx, s);
    }
    __syncthreads();
  }
  if (hh == 1) {
    s_pm[r] = run_m;
    s_ps[r] = run_s;
  }
  __syncthreads();
  if (hh == 0 && m < M) {
    lse_fold(run_m, run_s, s_pm[r], s_ps[r]);
    part[(long long)m * nspan + sp] = make_double2((double)run_m, run_s);
  }
}

// lambda_m = max + log(sum_spans s * exp(m_span - max)), spans in order.
__global__ void k_lambda(const double2* __restrict__ part, int M, int nspan,
                         double* __restrict__ lam, float* __restrict__ lamf) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= M) return;
  const double2* p = part + (long long)m * nspan;
  double mx = -INFINITY;
  for (int i = 0; i < nspan; ++i) mx = fmax(mx, p[i].x);
  double s = 0.0;
  for (int i = 0; i < nspan; ++i)
    if (p[i].x != -INFINITY) s += p[i].y * exp(p[i].x - mx);
  const double l = mx + log(s);
  lam[m] = l;
  lamf[m] = (float)l;
}

// S[j][m] = fp32(Zsel[j][m] - lambda_m), subtraction in FP64, one rounding.
__global__ void k_scores(float* __restrict__ S, const double* __restrict__ lam, int K, int M) {
  const long long n = (long long)K * M;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x) {
    const int m = (int)(i % M);
    S[i] = (float)((double)S[i] - lam[m]);
  }
}

// ------------------------------------------------------------- backward
// Recompute one 128 x 128 tile of chunk logits and form the logit gradient
//   v not selected:  dZ = (grad g_m) * exp(fp32(z - fp32(lambda_m)))
//   v = U[j]:        dZ = fp32(grad * (g_m exp(S[j][m]) - Gamma[j][m]))
// (g_m = sum_j gamma_j(m), zero on excluded rows).  dZ goes to the chunk
// block (row-major, leading dimension ldz) and the tile's column sums to
// dbpart[mtile][col].
template <typename T>
__global__ __launch_bounds__(NT, 2) void k_recompute(
    const T* __restrict__ X, const T* __restrict__ W, const T* __restrict__ bias, int M, int D,
    int c0, int c1, const int* __restrict__ col2sel, const float* __restrict__ lamf,
    const double* __restrict__ g, const float* __restrict__ S, const float* __restrict__ Gam,
    double grad, T* __restrict__ dZ, int ldz, float* __restrict__ dbpart, int mtiles,
    int vec_ok) {
  __shared__ __attribute__((aligned(16))) char smem[SMEM_BYTES];
  __shared__ int s_sel[BN];
  __shared__ float s_bias[BN];
  __shared__ float s_lam[BM];
  __shared__ float s_rs[BM];
  __shared__ double s_g[BM];
  __shared__ float s_db[BN];
  const int lin = xcd_tile(blockIdx.x, gridDim.x);
  const int mt = lin % mtiles, nt = lin / mtiles;
  const int m0 = mt * BM, n0 = c0 + nt * BN;
  f32x16 acc[2][2];
  gemm_tile<T, true, true>(X, D, m0, M, W, D, n0, c1, 0, D, vec_ok, vec_ok, acc, smem);
  float* Zt = reinterpret_cast<float*>(smem);
  acc_to_lds(acc, Zt);
  if (threadIdx.x < BN) {
    const int v = n0 + threadIdx.x;
    s_sel[threadIdx.x] = v < c1 ? col2sel[v] : -1;
    s_bias[threadIdx.x] = (bias != nullptr && v < c1) ? load_f32(bias, v) : 0.f;
    const int mm = m0 + threadIdx.x;
    const double gm = mm < M ? g[mm] : 0.0;
    s_g[threadIdx.x] = gm;
    s_rs[threadIdx.x] = (float)(grad * gm);
    s_lam[threadIdx.x] = mm < M ? lamf[mm] : 0.f;
  }
  __syncthreads();
  const int c = threadIdx.x & (BN - 1), hh = threadIdx.x >> 7;
  const int v = n0 + c;
  float colsum = 0.f;
  if (v < c1) {
    const int sel = s_sel[c];
    const float bv = s_bias[c];
    const int rend = min(hh * 64 + 64, M - m0);
    for (int rr = hh * 64; rr < rend; ++rr) {
      const int mm = m0 + rr;
      const float z = Zt[c * TILE_LD + rr] + bv;
      float dz;
      if (sel < 0) {
        dz = s_rs[rr] * expf(z - s_lam[rr]);
      } else {
        const long long o = (long long)sel * M + mm;
        dz = (float)(grad * (s_g[rr] * exp((double)S[o]) - (double)Gam[o]));
      }
      dZ[(long long)mm * ldz + (v - c0)] = Elem<T>::from_f32(dz);
      colsum += dz;
    }
  }
  if (hh == 1) s_db[c] = colsum;
  __syncthreads();
  if (hh == 0 && v < c1) dbpart[(long long)mt * ldz + (v - c0)] = colsum + s_db[c];
}

// dXacc[m][d] (+)= sum_{c in chunk} dZ[m][c] W[c0 + c][d].  With BKM the
// weight operand is the transposed chunk Wt[d][c] (leading dimension ldb),
// otherwise the chunk's rows W[c0 + c][d] (leading dimension D).
template <typename T, bool BKM>
__global__ __launch_bounds__(NT, 2) void k_dx(const T* __restrict__ dZ, int ldz,
                                              const T* __restrict__ Wc, int ldb, int M, int D,
                                              int Cc, float* __restrict__ dXacc, int first,
                                              int mtiles, int a_vec, int b_vec) {
  __shared__ __attribute__((aligned(16))) char smem[SMEM_BYTES];
  const int lin = xcd_tile(blockIdx.x, gridDim.x);
  const int mt = lin % mtiles, nt = lin / mtiles;
  const int m0 = mt * BM, n0 = nt * BN;
  f32x16 acc[2][2];
  gemm_tile<T, true, BKM>(dZ, ldz, m0, M, Wc, ldb, n0, D, 0, Cc, a_vec, b_vec, acc, smem);
  const int lane = threadIdx.x & 63, i = lane & 31, h = lane >> 5;
  const int w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int col = n0 + wn * 64 + ni * 32 + i;
      if (col >= D) continue;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int row = m0 + wm * 64 + mi * 32 + (rr >> 2) * 8 + h * 4 + (rr & 3);
        if (row < M) {
          float* p = dXacc + (long long)row * D + col;
          *p = first ? acc[mi][ni][rr] : *p + acc[mi][ni][rr];
        }
      }
    }
}

// part[s][i][d] = sum_{m in split s} dZ[m][i] X[m][d]  (i = chunk column).
template <typename T>
__global__ __launch_bounds__(NT, 2) void k_dw(const T* __restrict__ dZ, int ldz,
                                              const T* __restrict__ X, int M, int D, int Cc,
                                              float* __restrict__ part, int itiles, int ntiles,
                                              int kchunk, int a_vec, int b_vec) {
  __shared__ __attribute__((aligned(16))) char smem[SMEM_BYTES];
  const int lin = xcd_tile(blockIdx.x, gridDim.x);
  const int per = itiles * ntiles;
  const int s = lin / per, rem = lin % per;
  const int it = rem % itiles, nt = rem / itiles;
  const int i0 = it * BM, n0 = nt * BN;
  const int kb = s * kchunk, ke = min(M, kb + kchunk);
  f32x16 acc[2][2];
  gemm_tile<T, false, false>(dZ, ldz, i0, Cc, X, D, n0, D, kb, ke, a_vec, b_vec, acc, smem);
  const int lane = threadIdx.x & 63, li = lane & 31, h = lane >> 5;
  const int w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int col = n0 + wn * 64 + ni * 32 + li;
      if (col >= D) continue;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int row = i0 + wm * 64 + mi * 32 + (rr >> 2) * 8 + h * 4 + (rr & 3);
        if (row < Cc) part[((long long)s * Cc + row) * D + col] = acc[mi][ni][rr];
      }
    }
}

template <typename T>
__global__ void k_dw_reduce(const float* __restrict__ part, int splitk, int rows, int D,
                            T* __restrict__ dW, long long row_base) {
  const long long n = (long long)rows * D;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x) {
    float s = 0.f;
    for (int k = 0; k < splitk; ++k) s += part[(long long)k * n + i];
    dW[row_base * D + i] = Elem<T>::from_f32(s);
  }
}

template <typename T>
__global__ void k_db_reduce(const float* __restrict__ dbpart, int mtiles, int cols, int ld,
                            T* __restrict__ db, long long col_base) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= cols) return;
  float s = 0.f;
  for (int k = 0; k < mtiles; ++k) s += dbpart[(long long)k * ld + i];
  db[col_base + i] = Elem<T>::from_f32(s);
}

// dst[d][c] = src[c][d] for a rows x D block (64 x 64 tiles through LDS).
template <typename T>
__global__ void k_transpose(const T* __restrict__ src, int rows, int D, T* __restrict__ dst,
                            int ldd) {
  __shared__ T t[64][65];
  const int r0 = blockIdx.y * 64, d0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int rr = r0 + r, dd = d0 + tx;
    t[r][tx] = (rr < rows && dd < D) ? src[(long long)rr * D + dd] : T(0);
  }
  __syncthreads();
  for (int d = ty; d < 64; d += 4) {
    const int dd = d0 + d, rr = r0 + tx;
    if (dd < D && rr < rows) dst[(long long)dd * ldd + rr] = t[tx][d];
  }
}

__global__ void k_cast_bf16(const float* __restrict__ src, bf16_t* __restrict__ dst, long long n) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x)
    dst[i] = f32_to_bf16(src[i]);
}

int grid_cap(long long n, int threads, int cap = 8192) {
  long long g = (n + threads - 1) / threads;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

}  // namespace

hipError_t launch_fwd_lse(hipStream_t st, int dtype, const void* X, const void* W, const void* b,
                          int M, int D, int V, const int* col2sel, float* Zsel, double2* part,
                          int nspan) {
  const int mtiles = ceil_div(M, BM);
  const int grid = mtiles * nspan;
  if (grid == 0) return hipSuccess;
  if (dtype == 0) {
    const int vec = (D % 4 == 0) && aligned16(X) && aligned16(W);
    k_fwd_lse<float><<<grid, NT, 0, st>>>((const float*)X, (const float*)W, (const float*)b, M, D,
                                          V, col2sel, Zsel, part, nspan, mtiles, vec);
  } else {
    const int vec = (D % 8 == 0) && aligned16(X) && aligned16(W);
    k_fwd_lse<bf16_t><<<grid, NT, 0, st>>>((const bf16_t*)X, (const bf16_t*)W, (const bf16_t*)b,
                                           M, D, V, col2sel, Zsel, part, nspan, mtiles, vec);
  }
  return hipGetLastError();
}

hipError_t launch_lambda(hipStream_t st, const double2* part, int M, int nspan, double* lam,
                         float* lamf) {
  if (M == 0) return hipSuccess;
  k_lambda<<<ceil_div(M, 256), 256, 0, st>>>(part, M, nspan, lam, lamf);
  return hipGetLastError();
}

hipError_t launch_scores(hipStream_t st, float* S, const double* lam, int K, int M) {
  const long long n = (long long)K * M;
  if (n == 0) return hipSuccess;
  k_scores<<<grid_cap(n, 256), 256, 0, st>>>(S, lam, K, M);
  return hipGetLastError();
}

hipError_t launch_recompute(hipStream_t st, int dtype, const void* X, const void* W, const void* b,
                            int M, int D, int c0, int c1, const int* col2sel, const float* lamf,
                            const double* g, const float* S, const float* Gam, double grad,
                            void* dZ, int ldz, float* dbpart) {
  const int mtiles = ceil_div(M, BM);
  const int grid = mtiles * ceil_div(c1 - c0, BN);
  if (grid == 0) return hipSuccess;
  if (dtype == 0) {
    const int vec = (D % 4 == 0) && aligned16(X) && aligned16(W);
    k_recompute<float><<<grid, NT, 0, st>>>((const float*)X, (const float*)W, (const float*)b, M,
                                            D, c0, c1, col2sel, lamf, g, S, Gam, grad,
                                            (float*)dZ, ldz, dbpart, mtiles, vec);
  } else {
    const int vec = (D % 8 == 0) && aligned16(X) && aligned16(W);
    k_recompute<bf16_t><<<grid, NT, 0, st>>>((const bf16_t*)X, (const bf16_t*)W,
                                             (const bf16_t*)b, M, D, c0, c1, col2sel, lamf, g, S,
                                             Gam, grad, (bf16_t*)dZ, ldz, dbpart, mtiles, vec);
  }
  return hipGetLastError();
}

hipError_t launch_dx(hipStream_t st, int dtype, const void* dZ, int ldz, const void* W, int M,
                     int D, int c0, int c1, float* dXacc, int first, void* wt) {
  const int mtiles = ceil_div(M, BM);
  const int grid = mtiles * ceil_div(D, BN);
  if (grid == 0) return hipSuccess;
  const int Cc = c1 - c0;
  if (dtype == 0) {
    const float* Wc = (const float*)W + (long long)c0 * D;
    const int av = (ldz % 4 == 0) && aligned16(dZ);
    const int bv = (D % 4 == 0) && aligned16(Wc);
    k_dx<float, false><<<grid, NT, 0, st>>>((const float*)dZ, ldz, Wc, D, M, D, Cc, dXacc, first,
                                            mtiles, av, bv);
  } else {
    // bf16: stage W_c^T (D x Cc, leading dimension ldz) so both operands are
    // K-contiguous.
    const bf16_t* Wc = (const bf16_t*)W + (long long)c0 * D;
    dim3 tg(ceil_div(D, 64), ceil_div(Cc, 64));
    k_transpose<bf16_t><<<tg, 256, 0, st>>>(Wc, Cc, D, (bf16_t*)wt, ldz);
    const int av = (ldz % 8 == 0) && aligned16(dZ);
    const int bv = (ldz % 8 == 0) && aligned16(wt);
    k_dx<bf16_t, true><<<grid, NT, 0, st>>>((const bf16_t*)dZ, ldz, (const bf16_t*)wt, ldz, M, D,
                                            Cc, dXacc, first, mtiles, av, bv);
  }
  return hipGetLastError();
}

hipError_t launch_dw(hipStream_t st, int dtype, const void* dZ, int ldz, const void* X, int M,
                     int D, int c0, int c1, float* part, int splitk) {
  const int Cc = c1 - c0;
  const int itiles = ceil_div(Cc, BM), ntiles = ceil_div(D, BN);
  const int grid = itiles * ntiles * splitk;
  if (grid == 0) return hipSuccess;
  const int kchunk = ceil_div(ceil_div(M, splitk), 64) * 64;
  if (dtype == 0) {
    const int av = (ldz % 4 == 0) && aligned16(dZ);
    const int bv = (D % 4 == 0) && aligned16(X);
    k_dw<float><<<grid, NT, 0, st>>>((const float*)dZ, ldz, (const float*)X, M, D, Cc, part,
                                     itiles, ntiles, kchunk, av, bv);
  } else {
    const int av = (ldz % 8 == 0) && aligned16(dZ);
    const int bv = (D % 8 == 0) && aligned16(X);
    k_dw<bf16_t><<<grid, NT, 0, st>>>((const bf16_t*)dZ, ldz, (const bf16_t*)X, M, D, Cc, part,
                                      itiles, ntiles, kchunk, av, bv);
  }
  return hipGetLastError();
}

hipError_t launch_dw_reduce(hipStream_t st, int dtype, const float* part, int splitk, int rows,
                            int D, void* dW, long long row_base) {
  const long long n = (long long)rows * D;
  if (n == 0) return hipSuccess;
  if (dtype == 0)
    k_dw_reduce<float><<<grid_cap(n, 256), 256, 0, st>>>(part, splitk, rows, D, (float*)dW,
                                                          row_base);
  else
    k_dw_reduce<bf16_t><<<grid_cap(n, 256), 256, 0, st>>>(part, splitk, rows, D, (bf16_t*)dW,
                                                           row_base);
  return hipGetLastError();
}

hipError_t launch_db_reduce(hipStream_t st, int dtype, const float* dbpart, int mtiles, int cols,
                            int ld, void* db, long long col_base) {
  if (cols == 0) return hipSuccess;
  if (dtype == 0)
    k_db_reduce<float><<<ceil_div(cols, 256), 256, 0, st>>>(dbpart, mtiles, cols, ld, (float*)db,
                                                            col_base);
  else
    k_db_reduce<bf16_t><<<ceil_div(cols, 256), 256, 0, st>>>(dbpart, mtiles, cols, ld,
                                                             (bf16_t*)db, col_base);
  return hipGetLastError();
}

hipError_t launch_cast_out(hipStream_t st, int dtype, const float* src, void* dst, long long n) {
  if (n == 0 || dtype == 0) return hipSuccess;
  k_cast_bf16<<<grid_cap(n, 256), 256, 0, st>>>(src, (bf16_t*)dst, n);
  return hipGetLastError();
}

}  // namespace pcx

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

constexpr int cmax(int a, int b) { return a > b ? a : b; }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

// Grouped order of an (mtiles x ntiles) tile grid: GM consecutive row tiles
// form a group whose tiles are enumerated row-fastest, so the work-groups an
// XCD runs at the same time cover a compact GM x (concurrent / GM) block and
// share both operands' tiles in its L2.
template <int GM>
__device__ __forceinline__ void grouped_tile(int lin, int mtiles, int ntiles, int& mt, int& nt) {
  const int per_group = GM * ntiles;
  const int g = lin / per_group, j = lin % per_group;
  const int gm = min(GM, mtiles - g * GM);
  mt = g * GM + j % gm;
  nt = j / gm;
}

// Tile configuration of one GEMM kernel: a BM x BN work-group tile computed
// by (BM/WM) x (BN/WN) wavefronts of WM x WN, each a grid of MFMA 32 x 32
// blocks; KB bytes of every operand row are staged per k step.
template <typename T, int BM_, int BN_, int WM_, int WN_, int KB_, int MINWG_, int DEPTH_ = 1>
struct Cfg {
  using type = T;
  // Stages in flight between global memory and LDS: 1 = the next stage is
  // loaded during this stage's MFMAs; 2 = the one after it (for short MFMA
  // phases, where one stage of matrix work does not cover the load latency).
  static constexpr int DEPTH = DEPTH_;
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int WGM = BM / WM, WGN = BN / WN;
  static constexpr int WAVES = WGM * WGN;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int VEC = Elem<T>::VEC;
  static constexpr int BK = KB_ / (int)sizeof(T);          // k values per stage
  static constexpr int LDK = (KB_ + 16) / (int)sizeof(T);  // row-layout stride
  static constexpr int LDMA = BM + 4, LDMB = BN + 4;       // column-layout strides
  static constexpr int OPA = cmax(BM * LDK, BK * LDMA);    // one A buffer (elements)
  static constexpr int OPB = cmax(BN * LDK, BK * LDMB);
  static constexpr int STAGE_BYTES = 2 * (OPA + OPB) * (int)sizeof(T);
  static constexpr int MINWG = MINWG_;
  static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0, "tile shape");
  static_assert(sizeof(T) == 4 ? BK % 16 == 0 : BK % 32 == 0, "k step");
};

// LDS layouts of one staged ROWS (mn) x BK (k) operand tile:
//  * row layout [mn][LDK], k contiguous: K-contiguous operands, and bf16
//    MN-contiguous operands (transposed element by element on the way in);
//  * column layout [k][ROWS + 4], mn contiguous: fp32 MN-contiguous operands,
//    written straight from the 16-byte global loads.
template <typename T, bool KMAJOR>
struct ColLayout {
  static constexpr bool value = !KMAJOR && sizeof(T) == 4;
};

// Global -> registers -> LDS staging of one operand tile.
// KMAJOR: element (mn, k) is g[mn * ld + k]; otherwise g[k * ld + mn].
template <class C, int ROWS, bool KMAJOR>
struct Stage {
  using T = typename C::type;
  static constexpr int VEC = C::VEC;
  static constexpr int BK = C::BK;
  static constexpr int LDK = C::LDK;
  static constexpr int LDM = ROWS + 4;
  static constexpr bool COL = ColLayout<T, KMAJOR>::value;
  static constexpr int NV = ROWS * BK / VEC;  // 16-byte vectors per tile
  static constexpr int Q = NV / C::THREADS;    // per thread
  static_assert(NV % C::THREADS == 0, "staging split");

  __device__ static __forceinline__ void coords(int q, int& mn, int& k) {
    const int v = threadIdx.x + C::THREADS * q;
    if (KMAJOR) {
      mn = v / (BK / VEC);
      k = (v % (BK / VEC)) * VEC;
    } else {
      k = v / (ROWS / VEC);
      mn = (v % (ROWS / VEC)) * VEC;
    }
  }

  // FULL: the whole tile is in bounds and 16-byte aligned (no checks).
  template <bool FULL>
  __device__ static __forceinline__ void load(const T* g, long long ld, int mn0,
                                              int mn_lim, int k0, int k_lim, bool vec_ok,
                                              Vec16 (&r)[Q]) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      int mn, k;
      coords(q, mn, k);
      const int gm = mn0 + mn, gk = k0 + k;
      if (FULL) {
        const long long off = KMAJOR ? (long long)gm * ld + gk : (long long)gk * ld + gm;
        r[q].u = __builtin_bit_cast(uint4, *reinterpret_cast<const volatile u32x4*>(g + off));
      } else if (KMAJOR) {
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

  __device__ static __forceinline__ void store(T* __restrict__ s, const Vec16 (&r)[Q]) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
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

// One fp32 operand fragment: the values lane (i, h) feeds to four
// consecutive MFMA steps.  Within a stage of BK k values, step s of lane half
// h consumes k = 16*(s/8) + 8*h + s%8: four consecutive steps read four
// consecutive k (one 16-byte read in the row layout), and in the column
// layout the two lane halves read rows 8 apart, on disjoint LDS banks.
template <bool COL, int LDK, int LDM>
__device__ __forceinline__ f32x4 frag_f32(const float* __restrict__ S, int row, int h, int kc) {
  const int k0 = ((kc >> 1) << 4) + (h << 3) + ((kc & 1) << 2);
  if (!COL) return *reinterpret_cast<const f32x4*>(S + row * LDK + k0);
  f32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = S[(k0 + e) * LDM + row];
  return v;
}

// MFMA work of one staged k step for this wavefront's WM x WN block.
template <class C, bool ACOL, bool BCOL>
__device__ __forceinline__ void mma_stage(const typename C::type* __restrict__ As,
                                          const typename C::type* __restrict__ Bs,
                                          f32x16 (&acc)[C::FM][C::FN], int wm, int wn) {
  using T = typename C::type;
  const int lane = threadIdx.x & 63, i = lane & 31, h = lane >> 5;
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int kc = 0; kc < C::BK / 8; ++kc) {
      f32x4 a[C::FM], b[C::FN];
#pragma unroll
      for (int fi = 0; fi < C::FM; ++fi)
        a[fi] = frag_f32<ACOL, C::LDK, C::LDMA>(As, wm * C::WM + fi * 32 + i, h, kc);
#pragma unroll
      for (int fj = 0; fj < C::FN; ++fj)
        b[fj] = frag_f32<BCOL, C::LDK, C::LDMB>(Bs, wn * C::WN + fj * 32 + i, h, kc);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int fi = 0; fi < C::FM; ++fi)
#pragma unroll
          for (int fj = 0; fj < C::FN; ++fj)
            acc[fi][fj] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[fi][e], b[fj][e], acc[fi][fj],
                                                               0, 0, 0);
    }
  } else {
    // bf16 (row layout only): lane half h feeds k in [h*BK/2, (h+1)*BK/2),
    // eight per v_mfma_f32_32x32x16_bf16.
    static_assert(!ACOL && !BCOL, "bf16 operands use the row layout");
    // All fragments of the stage are read before its MFMAs: the short bf16
    // MFMA phase cannot cover one LDS round trip per k step.
    constexpr int KS = C::BK / 16;
    bf16x8 a[KS][C::FM], b[KS][C::FN];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
#pragma unroll
      for (int fi = 0; fi < C::FM; ++fi)
        a[j][fi] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(As + (wm * C::WM + fi * 32 + i) * C::LDK +
                                                    h * (C::BK / 2) + j * 8));
#pragma unroll
      for (int fj = 0; fj < C::FN; ++fj)
        b[j][fj] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(Bs + (wn * C::WN + fj * 32 + i) * C::LDK +
                                                    h * (C::BK / 2) + j * 8));
    }
#pragma unroll
    for (int j = 0; j < KS; ++j)
#pragma unroll
      for (int fi = 0; fi < C::FM; ++fi)
#pragma unroll
        for (int fj = 0; fj < C::FN; ++fj)
          acc[fi][fj] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j][fi], b[j][fj], acc[fi][fj], 0, 0, 0);
  }
}

// First k stage of a tile, loaded into registers ahead of time so that a
// caller walking several tiles can overlap it with the previous epilogue.
template <class C, bool AK, bool BK_>
struct Prefetch {
  Vec16 ra[Stage<C, C::BM, AK>::Q];
  Vec16 rb[Stage<C, C::BN, BK_>::Q];
  bool full;
};

template <class C, bool AK, bool BK_>
__device__ __forceinline__ void gemm_prefetch(Prefetch<C, AK, BK_>& p,
                                              const typename C::type* A, long long lda, int m0,
                                              int m_lim, const typename C::type* B,
                                              long long ldb, int n0, int n_lim, int k_begin,
                                              int k_end, bool a_vec, bool b_vec) {
  using SA = Stage<C, C::BM, AK>;
  using SB = Stage<C, C::BN, BK_>;
  p.full = a_vec && b_vec && m0 + C::BM <= m_lim && n0 + C::BN <= n_lim &&
           (k_end - k_begin) % C::BK == 0;
  if (k_end <= k_begin) return;
  if (p.full) {
    SA::template load<true>(A, lda, m0, m_lim, k_begin, k_end, a_vec, p.ra);
    SB::template load<true>(B, ldb, n0, n_lim, k_begin, k_end, b_vec, p.rb);
  } else {
    SA::template load<false>(A, lda, m0, m_lim, k_begin, k_end, a_vec, p.ra);
    SB::template load<false>(B, ldb, n0, n_lim, k_begin, k_end, b_vec, p.rb);
  }
}

template <class C, bool AK, bool BK_, bool FULL>
__device__ __forceinline__ void gemm_tile_impl(Prefetch<C, AK, BK_>& p,
                                               const typename C::type* A,
                                               long long lda, int m0, int m_lim,
                                               const typename C::type* B,
                                               long long ldb, int n0, int n_lim, int k_begin,
                                               int k_end, bool a_vec, bool b_vec,
                                               f32x16 (&acc)[C::FM][C::FN], char* smem) {
  using T = typename C::type;
  using SA = Stage<C, C::BM, AK>;
  using SB = Stage<C, C::BN, BK_>;
  T* As = reinterpret_cast<T*>(smem);
  T* Bs = As + 2 * C::OPA;
  const int w = threadIdx.x >> 6, wm = w / C::WGN, wn = w % C::WGN;
  const int nk = (k_end - k_begin + C::BK - 1) / C::BK;
  SA::store(As, p.ra);
  SB::store(Bs, p.rb);
  if constexpr (C::DEPTH == 2) {
    // Two register stages alternate; stage indices past the end are clamped
    // (harmless reloads into a buffer that is never read).
    Vec16 qa[SA::Q], qb[SB::Q];
    auto kof = [&](int kt) { return k_begin + min(kt, nk - 1) * C::BK; };
    SA::template load<FULL>(A, lda, m0, m_lim, kof(1), k_end, a_vec, p.ra);
    SB::template load<FULL>(B, ldb, n0, n_lim, kof(1), k_end, b_vec, p.rb);
    lds_barrier();
    for (int kt = 0; kt < nk; kt += 2) {
      SA::template load<FULL>(A, lda, m0, m_lim, kof(kt + 2), k_end, a_vec, qa);
      SB::template load<FULL>(B, ldb, n0, n_lim, kof(kt + 2), k_end, b_vec, qb);
      asm volatile("" ::: "memory");
      mma_stage<C, SA::COL, SB::COL>(As, Bs, acc, wm, wn);
      SA::store(As + C::OPA, p.ra);
      SB::store(Bs + C::OPB, p.rb);
      lds_barrier();
      if (kt + 1 >= nk) break;
      SA::template load<FULL>(A, lda, m0, m_lim, kof(kt + 3), k_end, a_vec, p.ra);
      SB::template load<FULL>(B, ldb, n0, n_lim, kof(kt + 3), k_end, b_vec, p.rb);
      asm volatile("" ::: "memory");
      mma_stage<C, SA::COL, SB::COL>(As + C::OPA, Bs + C::OPB, acc, wm, wn);
      SA::store(As, qa);
      SB::store(Bs, qb);
      lds_barrier();
    }
    return;
  }
  lds_barrier();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    // The last step reloads its own (in-bounds) stage into the idle buffer,
    // which keeps the loop body free of branches.
    const int k0 = k_begin + min(kt + 1, nk - 1) * C::BK;
    SA::template load<FULL>(A, lda, m0, m_lim, k0, k_end, a_vec, p.ra);
    SB::template load<FULL>(B, ldb, n0, n_lim, k0, k_end, b_vec, p.rb);
    // Keep the next stage's global loads ahead of this stage's MFMAs so their
    // latency hides behind the matrix work (a compiler-only memory fence: no
    // memory operation moves across it, and the MFMAs wait on the LDS reads
    // below it).
    asm volatile("" ::: "memory");
    mma_stage<C, SA::COL, SB::COL>(As + cur * C::OPA, Bs + cur * C::OPB, acc, wm, wn);
    SA::store(As + (cur ^ 1) * C::OPA, p.ra);
    SB::store(Bs + (cur ^ 1) * C::OPB, p.rb);
    lds_barrier();
  }
}

// acc = A[m0:m0+BM, k] . B[n0:n0+BN, k]^T over k in [k_begin, k_end), with
// the first stage already in `p` (from gemm_prefetch on the same tile).
// Rows/columns past the limits and k past k_end read as zero.  Ends with a
// barrier, so the caller may reuse `smem` right away.
template <class C, bool AK, bool BK_>
__device__ __forceinline__ void gemm_tile_run(Prefetch<C, AK, BK_>& p,
                                              const typename C::type* A, long long lda, int m0,
                                              int m_lim, const typename C::type* B,
                                              long long ldb, int n0, int n_lim, int k_begin,
                                              int k_end, bool a_vec, bool b_vec,
                                              f32x16 (&acc)[C::FM][C::FN], char* smem) {
#pragma unroll
  for (int fi = 0; fi < C::FM; ++fi)
#pragma unroll
    for (int fj = 0; fj < C::FN; ++fj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[fi][fj][r] = 0.f;
  if (k_end <= k_begin) return;
  if (p.full)
    gemm_tile_impl<C, AK, BK_, true>(p, A, lda, m0, m_lim, B, ldb, n0, n_lim, k_begin, k_end,
                                     a_vec, b_vec, acc, smem);
  else
    gemm_tile_impl<C, AK, BK_, false>(p, A, lda, m0, m_lim, B, ldb, n0, n_lim, k_begin, k_end,
                                      a_vec, b_vec, acc, smem);
}

// One tile, no cross-tile overlap.
template <class C, bool AK, bool BK_>
__device__ __forceinline__ void gemm_tile(const typename C::type* __restrict__ A, long long lda,
                                          int m0, int m_lim,
                                          const typename C::type* __restrict__ B, long long ldb,
                                          int n0, int n_lim, int k_begin, int k_end, bool a_vec,
                                          bool b_vec, f32x16 (&acc)[C::FM][C::FN], char* smem) {
  Prefetch<C, AK, BK_> p;
  gemm_prefetch<C, AK, BK_>(p, A, lda, m0, m_lim, B, ldb, n0, n_lim, k_begin, k_end, a_vec,
                            b_vec);
  gemm_tile_run<C, AK, BK_>(p, A, lda, m0, m_lim, B, ldb, n0, n_lim, k_begin, k_end, a_vec,
                            b_vec, acc, smem);
}

// Accumulator element (fi, fj, r) of lane l in wave (wm, wn) sits at tile row
// wm*WM + fi*32 + 8*(r/4) + 4*(l/32) + r%4 and tile column wn*WN + fj*32 + l%32.
template <class C>
__device__ __forceinline__ int acc_row(int fi, int r) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  return (w / C::WGN) * C::WM + fi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}
template <class C>
__device__ __forceinline__ int acc_col(int fj) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  return (w % C::WGN) * C::WN + fj * 32 + (lane & 31);
}

// A tile partial with a NaN or infinite logit (chk is then NaN) becomes
// (finite max, NaN sum): every later fold, and the normalizer built from it,
// is then NaN, so the frame's utterance comes out nonfinite and is excluded.
// (The max alone would drop a NaN, and the clamped exp maps it to 0.)
__device__ __forceinline__ void nonfinite_partial(float chk, float& mx, double& sum) {
  if (chk != chk) {
    mx = (mx == -INFINITY || mx == INFINITY) ? 0.f : mx;
    sum = __builtin_nan("");
  }
}

// (m1, s1) <- fold of two log-sum-exp partials (max, sum of exp(z - max)).
__device__ __forceinline__ void lse_fold(float& m1, double& s1, float m2, double s2) {
  if (m2 == -INFINITY) return;
  if (m1 == -INFINITY) {
    m1 = m2;
    s1 = s2;
  } else if (m2 > m1) {
    s1 = s1 * exp_nonpos((double)m1 - (double)m2) + s2;
    m1 = m2;
  } else {
    s1 = s1 + s2 * exp_nonpos((double)m2 - (double)m1);
  }
}


// Tile configurations of the four head products, chosen by sweeps of tile /
// wave shapes on the V = 180k (fp32) and LLM (bf16) heads.  fp32: 128 x 128
// work-group tiles with 16-k stages; the forward (whose epilogue ends every
// short K = D product) gains from 32-k stages, the dX product from eight
// 64 x 32 wavefronts.
using CfgF32 = Cfg<float, 128, 128, 64, 64, 64, 2>;
using CfgF32Fwd = Cfg<float, 128, 128, 64, 64, 128, 2>;
using CfgF32Dx = Cfg<float, 128, 128, 64, 32, 128, 2>;
using CfgB16 = Cfg<bf16_t, 128, 128, 64, 64, 128, 2>;
using CfgB16W8 = Cfg<bf16_t, 128, 128, 32, 64, 128, 2>;
using CfgB16Wide = Cfg<bf16_t, 128, 256, 64, 128, 64, 2>;
template <typename T> struct Pick;
template <> struct Pick<float> {
  using fwd = CfgF32Fwd;
  using rec = CfgF32;
  using dx = CfgF32Dx;
  using dw = CfgF32;
};
// bf16 (heads the 256 x 256 core does not take): the
// recompute product takes 128 x 256 tiles of four 64 x 128 wavefronts (fewer
// LDS bytes per MFMA at the bf16 rate); dX, whose epilogue is a fp32
// accumulator update, runs eight 32 x 64 wavefronts.
template <> struct Pick<bf16_t> {
  using fwd = CfgB16;
  using rec = CfgB16Wide;
  using dx = CfgB16W8;
  using dw = CfgB16;
};

// ------------------------------------------------------------- forward
// The forward tile is computed transposed: BM vocabulary rows (operand A =
// W) by BN frames (operand B = X), so each lane holds FM x 16 vocabulary
// values of each of its FN frames and the per-frame log-sum-exp of a tile
// needs no cross-lane step.  One work-group: BN frames x one span-wide
// vocabulary span, walked in BM-row tiles, the next tile's first k stage
// loaded before the current tile's epilogue.  Per tile and frame each lane
// folds the max and the FP64 sum of exp(z - max) over its values into a
// running partial; at the end of the span the two lane halves and the WGM
// wave rows are folded in a fixed order.  Selected vocabulary rows are
// gathered into Zsel (class-major, K x M), 32 frames per coalesced store.
template <class C, bool MASKED>
__global__ __launch_bounds__(C::THREADS, C::MINWG) void k_fwd_lse(
    const typename C::type* __restrict__ X, const typename C::type* __restrict__ W,
    const typename C::type* __restrict__ bias, int M, int D, int V,
    const int* __restrict__ col2sel, float* __restrict__ Zsel, double2* __restrict__ part,
    int nspan, int ftiles, int vec_ok, int span0, int part_ld, int span) {
  using T = typename C::type;
  __shared__ __attribute__((aligned(16))) char smem[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) int s_sel[2][C::BM];
  __shared__ __attribute__((aligned(16))) float s_bias[2][C::BM];
  __shared__ float f_m[C::WGM][C::BN];
  __shared__ double f_s[C::WGM][C::BN];
  __shared__ int s_any[2][C::WAVES];  // per wavefront: a selected row among its loads

  int ft, sp;
  grouped_tile<8>(xcd_tile(blockIdx.x, gridDim.x), ftiles, nspan, ft, sp);
  const int f0 = ft * C::BN;
  const int c_begin = sp * span, c_end = min(V, c_begin + span);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w / C::WGN;
  float run_m[C::FN];
  double run_s[C::FN];
#pragma unroll
  for (int fj = 0; fj < C::FN; ++fj) {
    run_m[fj] = -INFINITY;
    run_s[fj] = 0.0;
  }
  Prefetch<C, true, true> pf;
  gemm_prefetch<C, true, true>(pf, W, D, c_begin, c_end, X, D, f0, M, 0, D, vec_ok, vec_ok);
  int par = 0;
  for (int v0 = c_begin; v0 < c_end; v0 += C::BM, par ^= 1) {
    // this tile's row data: visible after the GEMM's barriers; the buffer
    // written here was last read two tiles ago
    bool any_sel = false;
    for (int r = threadIdx.x; r < C::BM; r += C::THREADS) {
      const int v = v0 + r;
      const int sl = v < c_end ? col2sel[v] : -2;  // -2: past the span
      s_sel[par][r] = sl;
      s_bias[par][r] = (bias != nullptr && v < c_end) ? Elem<T>::to_f32(bias[v]) : 0.f;
      any_sel |= sl >= 0;
    }
    {
      const unsigned long long b = __ballot(any_sel);
      if (lane == 0) s_any[par][w] = b != 0ull;
    }
    f32x16 acc[C::FM][C::FN];
    gemm_tile_run<C, true, true>(pf, W, D, v0, c_end, X, D, f0, M, 0, D, vec_ok, vec_ok, acc,
                                 smem);
    if (v0 + C::BM < c_end)
      gemm_prefetch<C, true, true>(pf, W, D, v0 + C::BM, c_end, X, D, f0, M, 0, D, vec_ok,
                                   vec_ok);
    // selected vocabulary rows of this tile into Zsel (most tiles of a large
    // vocabulary have none, and skip this as a whole)
    bool tile_sel = false;
#pragma unroll
    for (int q = 0; q < C::WAVES; ++q) tile_sel |= s_any[par][q] != 0;
    if (tile_sel) {
#pragma unroll
      for (int fj = 0; fj < C::FN; ++fj) {
        const int frame = f0 + acc_col<C>(fj);
#pragma unroll
        for (int fi = 0; fi < C::FM; ++fi)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r0 = acc_row<C>(fi, 4 * q);
            const int4 sel4 = *reinterpret_cast<const int4*>(&s_sel[par][r0]);
            const f32x4 b4 = *reinterpret_cast<const f32x4*>(&s_bias[par][r0]);
            const int sl[4] = {sel4.x, sel4.y, sel4.z, sel4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (sl[e] >= 0 && frame < M)
                Zsel[(long long)sl[e] * M + frame] = acc[fi][fj][4 * q + e] + b4[e];
          }
      }
    }
#pragma unroll
    for (int fj = 0; fj < C::FN; ++fj) {
      float mx = -INFINITY;
      float chk = 0.f;  // stays 0 unless a logit is NaN or infinite
#pragma unroll
      for (int fi = 0; fi < C::FM; ++fi)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r0 = acc_row<C>(fi, 4 * q);
          const int4 sel4 = *reinterpret_cast<const int4*>(&s_sel[par][r0]);
          const f32x4 b4 = *reinterpret_cast<const f32x4*>(&s_bias[par][r0]);
          const int sl[4] = {sel4.x, sel4.y, sel4.z, sel4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float z = acc[fi][fj][4 * q + e] + b4[e];
            chk = fmaf(z, 0.f, chk);
            // in the sum: every vocabulary row of the span, or (masked)
            // only the unselected ones
            acc[fi][fj][4 * q + e] = (MASKED ? sl[e] == -1 : sl[e] >= -1) ? z : -INFINITY;
            mx = fmaxf(mx, acc[fi][fj][4 * q + e]);
          }
        }
      double sum = 0.0;
      if (mx != -INFINITY) {
#pragma unroll
        for (int fi = 0; fi < C::FM; ++fi)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sum += exp_nonpos((double)acc[fi][fj][r] - (double)mx);
      }
      nonfinite_partial(chk, mx, sum);
      lse_fold(run_m[fj], run_s[fj], mx, sum);
    }
  }
  // lane halves (lower half first), then wave rows in order
#pragma unroll
  for (int fj = 0; fj < C::FN; ++fj) {
    const float om = __shfl_xor(run_m[fj], 32, 64);
    const double os = __shfl_xor(run_s[fj], 32, 64);
    float m1 = lane < 32 ? run_m[fj] : om;
    double s1 = lane < 32 ? run_s[fj] : os;
    lse_fold(m1, s1, lane < 32 ? om : run_m[fj], lane < 32 ? os : run_s[fj]);
    if (lane < 32) {
      f_m[wm][acc_col<C>(fj)] = m1;
      f_s[wm][acc_col<C>(fj)] = s1;
    }
  }
  lds_barrier();
  for (int c = threadIdx.x; c < C::BN; c += C::THREADS) {
    const int frame = f0 + c;
    if (frame >= M) continue;
    float fm = f_m[0][c];
    double fs = f_s[0][c];
#pragma unroll
    for (int q = 1; q < C::WGM; ++q) lse_fold(fm, fs, f_m[q][c], f_s[q][c]);
    part[(long long)frame * part_ld + span0 + sp] = make_double2((double)fm, fs);
  }
}

// lambda_m = max + log(sum_spans s * exp(m_span - max)).  Eight lanes per
// frame: lane j takes the spans j, j + 8, ... (the eight lanes of a frame
// read 128 consecutive bytes at a time); the maximum is exact in any order
// and the eight partial sums are added in a fixed butterfly (IEEE addition is
// commutative, so both lanes of a pair hold the same sum).
constexpr int LAM_LANES = 8;
__global__ __launch_bounds__(256) void k_lambda(const double2* __restrict__ part, int M,
                                                int nspan, double* __restrict__ lam,
                                                float* __restrict__ lamf) {
  const long long gt = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int m = (int)(gt / LAM_LANES), j = (int)(gt % LAM_LANES);
  const bool in = m < M;
  const double2* p = part + (long long)(in ? m : 0) * nspan;
  double mx = -INFINITY;
  if (in)
    for (int i = j; i < nspan; i += LAM_LANES) mx = fmax(mx, p[i].x);
#pragma unroll
  for (int o = 1; o < LAM_LANES; o <<= 1) mx = fmax(mx, __shfl_xor(mx, o, 64));
  double s = 0.0;
  if (in)
    for (int i = j; i < nspan; i += LAM_LANES)
      if (p[i].x != -INFINITY) s += p[i].y * exp_nonpos(p[i].x - mx);
#pragma unroll
  for (int o = 1; o < LAM_LANES; o <<= 1) s += __shfl_xor(s, o, 64);
  if (in && j == 0) {
    const double l = mx + log(s);
    lam[m] = l;
    lamf[m] = (float)l;
  }
}

// Grouped logits R = [Z[:, U], o] with o_m = log sum over the unselected
// classes of exp Z[m][v] ("other" column, Eq. 4): lambda_m = log-sum-exp of
// the K + 1 entries of R_m (FP64; the selected logits are the fp32 values
// gathered in Zsel).  o_m = -inf when every class is selected.
__global__ void k_lambda_grouped(const float* __restrict__ Zsel, const double* __restrict__ other,
                                 int K, int M, double* __restrict__ lam,
                                 float* __restrict__ lamf) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= M) return;
  double mx = other[m];
  for (int j = 0; j < K; ++j) mx = fmax(mx, (double)Zsel[(long long)j * M + m]);
  double s = other[m] == -INFINITY ? 0.0 : exp_nonpos(other[m] - mx);
  for (int j = 0; j < K; ++j) s += exp_nonpos((double)Zsel[(long long)j * M + m] - mx);
  double l = mx + log(s);
  // a nonfinite logit in the frame made the other column NaN: so is lambda
  if (other[m] != other[m]) l = other[m];
  lam[m] = l;
  lamf[m] = (float)l;
}

// Row factor of the unselected classes in the grouped backward: the "other"
// column's gradient grad * g_m * p_other(m) (its occupancy is zero), spread
// over the unselected classes by the log-sum-exp Jacobian exp(z - o_m)
// (App. B.1, Eq. 11); gu_m = g_m exp(o_m - lambda_m).
__global__ void k_grouped_rowscale(const double* __restrict__ g, const double* __restrict__ other,
                                   const double* __restrict__ lam, int M,
                                   double* __restrict__ gu, float* __restrict__ ou) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= M) return;
  const bool empty = other[m] == -INFINITY;  // no unselected class
  gu[m] = empty ? 0.0 : g[m] * exp_nonpos(other[m] - lam[m]);
  ou[m] = empty ? 0.f : (float)other[m];
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
// Above this many selected columns in one wavefront's tile (of 32 FN), the
// recompute epilogue lets every lane handle its own selected columns instead
// of sharing each selected column among all 64 lanes.
constexpr int SEL_DENSE = 8;
// On the 256 x 256 core with eight wavefronts the per-wavefront limit of
// that cooperative pass, whose S and Gamma values are loaded into a 24 KiB LDS
// region beside the operand stages (the registers are taken by the
// accumulators); with sixteen wavefronts (half the columns each) half of it.
constexpr int SEL_PRE_BIG = 6;
// Elements per thread whose loads the dense selected-class pass keeps in
// flight together.
constexpr int DENSE_ILP = 8;

// ------------------------------------------------------ gradient reduction
// The two head-gradient reductions of one chunk, in work-groups of 256
// threads: the first nb_db reduce the bias partials, 16 columns each
// (db[col] = sum over row tiles of dbpart[tile][col]: sixteen fixed groups of
// consecutive tiles, the group sums added in group order); the others reduce
// the dW split partials (dW[row_base + r][d] = sum over k, in order, of
// part[k][r][d]).  The db part is latency-bound and the dW part HBM-bound, so
// they share a launch: their own, or the next chunk's recompute launch, whose
// last partial wave of tiles leaves CUs free for them.
constexpr int DB_GROUPS = 16;
constexpr int DB_COLS = 256 / DB_GROUPS;

// Work-group bid (0 .. rj.nb - 1) of the reduction; gs: DB_GROUPS x DB_COLS
// floats of LDS.  Every thread of the work-group calls it.
template <typename T>
__device__ __forceinline__ void grad_reduce_wg(const ReduceJob& rj, int bid, float* gs) {
  const float* __restrict__ part = rj.part;
  const int splitk = rj.splitk, D = rj.D;
  if (bid < rj.nb_db) {
    const int lc = threadIdx.x % DB_COLS, q = threadIdx.x / DB_COLS;
    const int c = bid * DB_COLS + lc;
    const int per = (rj.mtiles + DB_GROUPS - 1) / DB_GROUPS;
    const int k1 = min(rj.mtiles, (q + 1) * per);
    float s = 0.f;
    if (c < rj.cols) {
#pragma unroll 8
      for (int k = q * per; k < k1; ++k) s += rj.dbpart[(long long)k * rj.ld + c];
    }
    gs[q * DB_COLS + lc] = s;
    lds_barrier();
    if (q == 0 && c < rj.cols) {
      float t = gs[lc];
#pragma unroll
      for (int g = 1; g < DB_GROUPS; ++g) t += gs[g * DB_COLS + lc];
      static_cast<T*>(rj.db)[rj.col_base + c] = Elem<T>::from_f32(t);
    }
    return;
  }
  T* __restrict__ dW = static_cast<T*>(rj.dW);
  const long long n = (long long)rj.rows * D;
  const long long stride = (long long)(rj.nb - rj.nb_db) * 256;
  const long long i0 = (long long)(bid - rj.nb_db) * 256 + threadIdx.x;
  if (rj.vec4) {
    // four consecutive elements per thread (16-byte partial loads); the
    // same split order per element
    for (long long i = i0; i < n / 4; i += stride) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
      // eight splits' loads in flight together (clamped split index, the
      // extra ones not added), summed in split order
      for (int k0 = 0; k0 < splitk; k0 += 8) {
        f32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = *reinterpret_cast<const f32x4*>(part + (long long)min(k0 + u, splitk - 1) * n +
                                                 4 * i);
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (k0 + u < splitk) s += v[u];
      }
      T o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = Elem<T>::from_f32(s[e]);
      T* dst = dW + rj.row_base * D + 4 * i;
      if (sizeof(T) == 4)
        *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<const f32x4*>(o);
      else
        *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(o);
    }
    return;
  }
  for (long long i = i0; i < n; i += stride) {
    float s = 0.f;
    for (int k0 = 0; k0 < splitk; k0 += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(long long)min(k0 + u, splitk - 1) * n + i];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (k0 + u < splitk) s += v[u];
    }
    dW[rj.row_base * D + i] = Elem<T>::from_f32(s);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_grad_reduce(ReduceJob rj) {
  __shared__ float gs[DB_GROUPS * DB_COLS];
  grad_reduce_wg<T>(rj, blockIdx.x, gs);
}

// Selected columns of one wavefront's tile block for the cooperative pass
// (at most SEL_DENSE of them), in (fragment column, lane) order, with the S
// and Gamma values of the wavefront's rows (WM / 64 per lane).  They do not
// depend on the product, so they are loaded before it and their latency
// hides behind the matrix work.  n > SEL_DENSE: the dense pass runs instead.
template <class C>
struct SelPre {
  static constexpr int RPL = C::WM / 64;
  int n;
  int col[SEL_DENSE];
  float s[SEL_DENSE][RPL], g[SEL_DENSE][RPL];
};

// s_sel[c]: selected index of tile column c (or -1); columns at or past c1
// are never selected.  S and Gamma are class-major with leading dimension ldS.
template <class C>
__device__ __forceinline__ void sel_prefetch(SelPre<C>& p, const int* s_sel, int n0, int c1,
                                             int m0, int M, const float* __restrict__ S,
                                             const float* __restrict__ Gam, long long ldS) {
  static_assert(C::WM % 64 == 0, "selected-class pass: whole rows per lane");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w / C::WGN, wn = w % C::WGN;
  unsigned long long mk[C::FN];
  int cs[C::FN];
  int total = 0;
#pragma unroll
  for (int fj = 0; fj < C::FN; ++fj) {
    const int col = acc_col<C>(fj);
    cs[fj] = s_sel[col];
    mk[fj] = __ballot(lane < 32 && n0 + col < c1 && cs[fj] >= 0);
    total += __popcll(mk[fj]);
  }
  p.n = total;
  if (total > SEL_DENSE) return;
#pragma unroll
  for (int k = 0; k < SEL_DENSE; ++k) {
    int sel = 0, col = 0;
    bool found = false;
#pragma unroll
    for (int fj = 0; fj < C::FN; ++fj) {
      if (!found && mk[fj] != 0ull) {
        const int src = __ffsll((long long)mk[fj]) - 1;
        mk[fj] &= mk[fj] - 1;
        sel = __builtin_amdgcn_readlane(cs[fj], src);
        col = wn * C::WN + fj * 32 + src;
        found = true;
      }
    }
    p.col[k] = col;
#pragma unroll
    for (int t = 0; t < SelPre<C>::RPL; ++t) {
      const int row = wm * C::WM + SelPre<C>::RPL * lane + t;
      const bool ok = found && m0 + row < M;
      p.s[k][t] = ok ? S[sel * ldS + m0 + row] : 0.f;
      p.g[k][t] = ok ? Gam[sel * ldS + m0 + row] : 0.f;
    }
  }
}

// dZ of the prefetched selected columns, grad (g_m exp(S) - Gamma) formed in
// FP64 and rounded once; each column's sum over the wavefront's rows (a
// fixed-order wave sum) goes to s_db_w[column].
template <class C, typename T>
__device__ __forceinline__ void sel_finish(const SelPre<C>& p, const double* s_g, int m0, int M,
                                           const int* s_col, double grad, T* __restrict__ dZ,
                                           int ldz, float* s_db_w) {
  const int lane = threadIdx.x & 63, wm = (threadIdx.x >> 6) / C::WGN;
#pragma unroll
  for (int k = 0; k < SEL_DENSE; ++k) {
    if (k < p.n) {
      float sum = 0.f;
#pragma unroll
      for (int t = 0; t < SelPre<C>::RPL; ++t) {
        const int row = wm * C::WM + SelPre<C>::RPL * lane + t;
        if (m0 + row < M) {
          // S <= 0 (a log-probability)
          const float dz =
              (float)(grad * (s_g[row] * exp_nonpos((double)p.s[k][t]) - (double)p.g[k][t]));
          dZ[(long long)(m0 + row) * ldz + s_col[p.col[k]]] = Elem<T>::from_f32(dz);
          sum += dz;
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
      if (lane == 0) s_db_w[p.col[k]] = sum;
    }
  }
}

// Recompute one BM x BN tile of chunk logits and form the logit gradient
//   v not selected:  dZ = (grad g_m) * exp(z - fp32(lambda_m)), evaluated in
//                    fp32 as exp2(z log2e - fp32(lambda_m log2e)) with one
//                    fused multiply-add for the argument;
//   v = U[j]:        dZ = fp32(grad * (g_m exp(S[j][m]) - Gamma[j][m]))
//                    (S reused; the difference formed in FP64, one rounding)
// (g_m = sum_j gamma_j(m), zero on excluded rows).  The epilogue works on the
// MFMA accumulators in place: dZ goes to the chunk block (row-major,
// leading dimension ldz) and the tile's column sums to dbpart[mtile][col].
//
// cmap (optional): the tiles walk the chunk's columns in the order
// cmap[0 .. c1 - c0) (the unselected classes first, see k_colperm; *nu of
// them), so that the selected classes fill whole tiles, which need no
// product and are left to k_dz_sel; the product of the other tiles reads
// head rows from Wg, where row i holds the head row of column cmap[i].  Without cmap the tiles walk the columns in order and
// read the head itself.
template <class C>
__global__ __launch_bounds__(C::THREADS, C::MINWG) void k_recompute(
    const typename C::type* __restrict__ X, const typename C::type* __restrict__ W,
    const typename C::type* __restrict__ bias, int M, int D, int c0, int c1,
    const int* __restrict__ col2sel, const float* __restrict__ lamf,
    const double* __restrict__ g, const float* __restrict__ S, const float* __restrict__ Gam,
    double grad, typename C::type* __restrict__ dZ, int ldz, float* __restrict__ dbpart,
    int mtiles, int vec_ok, const double* __restrict__ gu, const float* __restrict__ lamu,
    long long ldS, const int* __restrict__ cmap, const typename C::type* __restrict__ Wg,
    const int* __restrict__ nu, ReduceJob rj, int ntile) {
  using T = typename C::type;
  constexpr int BM = C::BM, BN = C::BN;
  static_assert(C::THREADS == 256, "the appended reduction takes 256-thread work-groups");
  constexpr float LOG2E = 1.44269504088896340736f;
  __shared__ __attribute__((aligned(16))) char smem[C::STAGE_BYTES];
  __shared__ int s_sel[BN];
  __shared__ float s_bias[BN];
  __shared__ float s_lam2[BM];
  __shared__ float s_rs[BM];
  __shared__ double s_g[BM];
  __shared__ float s_db[C::WGM][BN];
  __shared__ int s_list[BN], s_pos[BN], s_cnt[BN / 64];
  __shared__ int s_col[BN];  // dZ column (within the chunk) of each tile column
  if ((int)blockIdx.x >= ntile) {
    // a work-group of the appended reduction (another chunk's gradients;
    // nothing this launch's tiles read or write)
    float* gs = reinterpret_cast<float*>(smem);
    if (rj.out_bf16)
      grad_reduce_wg<bf16_t>(rj, (int)blockIdx.x - ntile, gs);
    else
      grad_reduce_wg<float>(rj, (int)blockIdx.x - ntile, gs);
    return;
  }
  int mt, nt;
  grouped_tile<8>(xcd_tile(blockIdx.x, ntile), mtiles, (c1 - c0 + BN - 1) / BN, mt, nt);
  const int m0 = mt * BM, n0 = c0 + nt * BN;
  // in the unselected-first order the tiles of selected classes alone are
  // k_dz_sel's
  if (cmap != nullptr && n0 - c0 >= *nu) return;
  // End of the places this tile forms: in the unselected-first order only the
  // unselected ones (the selected places of a tile that also holds unselected
  // ones are k_dz_sel's too, so this tile's epilogue has no selected class).
  const int c1e = cmap != nullptr ? c0 + *nu : c1;
  // head rows of the product: the gathered rows (from row 0) or the head
  const T* Bh = cmap != nullptr ? Wg : W;
  const int nb0 = cmap != nullptr ? n0 - c0 : n0, nb1 = cmap != nullptr ? c1 - c0 : c1;
  // The product's first k stage is requested before the tile's row and
  // column data, so the two loads' latencies overlap.
  Prefetch<C, true, true> pf;
  gemm_prefetch<C, true, true>(pf, X, D, m0, M, Bh, D, nb0, nb1, 0, D, vec_ok, vec_ok);
  // Row and column data of the tile.  The loads read clamped (in-bounds)
  // places and frames unconditionally and the values past the tile's ends
  // are masked afterwards, so that all of them are in flight together (a
  // load under a per-lane condition is waited for on the spot).
  for (int c = threadIdx.x; c < BN; c += C::THREADS) {
    const int v = n0 + c;
    const bool in = v < c1e;
    const int vc = in ? v : c1e - 1;
    const int rv = cmap != nullptr ? cmap[vc - c0] : vc;
    const int sl = col2sel[rv];
    const float bv = bias != nullptr ? Elem<T>::to_f32(bias[rv]) : 0.f;
    s_sel[c] = in ? sl : -1;
    s_bias[c] = in ? bv : 0.f;
    s_col[c] = rv - c0;
  }
  for (int rr = threadIdx.x; rr < BM; rr += C::THREADS) {
    const int mm = m0 + rr;
    const bool in = mm < M;
    const int mc = in ? mm : M - 1;
    const double gv = g[mc];
    const double guv = gu != nullptr ? gu[mc] : gv;
    const float lv = lamu != nullptr ? lamu[mc] : lamf[mc];
    s_g[rr] = in ? gv : 0.0;
    // unselected classes: dZ = rs * exp(z - shift); rs = grad g_m and shift =
    // lambda_m, or in the grouped form grad gu_m and the other column o_m
    s_rs[rr] = in ? (float)(grad * guv) : 0.f;
    s_lam2[rr] = in ? lv * LOG2E : 0.f;
  }
  lds_barrier();
  // A tile whose columns are all selected needs no recomputed logit (their
  // dZ comes from S, Gamma and g alone, the pages' reuse of S): its product
  // is skipped.  (Small vocabularies, where K is close to V, and the densely
  // selected low ids of Zipf-distributed labels.)
  bool any_unsel = false;
  for (int c = threadIdx.x; c < BN; c += C::THREADS) any_unsel |= n0 + c < c1e && s_sel[c] < 0;
  const bool need_product = __syncthreads_or(any_unsel) != 0;
  SelPre<C> pre;
  sel_prefetch<C>(pre, s_sel, n0, c1e, m0, M, S, Gam, ldS);
  f32x16 acc[C::FM][C::FN];
  if (need_product) {
    gemm_tile_run<C, true, true>(pf, X, D, m0, M, Bh, D, nb0, nb1, 0, D, vec_ok, vec_ok, acc,
                                 smem);
  } else {
#pragma unroll
    for (int fi = 0; fi < C::FM; ++fi)
#pragma unroll
      for (int fj = 0; fj < C::FN; ++fj) acc[fi][fj] = f32x16{};
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w / C::WGN;
  const bool rows_full = m0 + BM <= M;
  // Many selected columns in some wavefront: the whole work-group takes the
  // dense pass below.  (Also a barrier: every wavefront is done with the
  // operand stages, which that pass reuses.)
  const bool dense = __syncthreads_or(pre.n > SEL_DENSE) != 0;
  // Unselected classes on the accumulators, four rows at a time; selected
  // classes (role 2) and columns past the chunk (role 3) are skipped here.
  int csel[C::FN], crole[C::FN], ccol[C::FN];
  float cbv[C::FN], cs[C::FN];
#pragma unroll
  for (int fj = 0; fj < C::FN; ++fj) {
    const int col = acc_col<C>(fj);
    csel[fj] = s_sel[col];
    cbv[fj] = s_bias[col];
    ccol[fj] = s_col[col];
    crole[fj] = n0 + col < c1e ? (csel[fj] < 0 ? 0 : 2) : 3;
    cs[fj] = 0.f;
  }
#pragma unroll
  for (int fi = 0; fi < C::FM; ++fi) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row0 = acc_row<C>(fi, 4 * q);
      const f32x4 rs4 = *reinterpret_cast<const f32x4*>(s_rs + row0);
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(s_lam2 + row0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = row0 + e;
        const bool in = rows_full || m0 + row < M;
#pragma unroll
        for (int fj = 0; fj < C::FN; ++fj) {
          // the exponent is <= 0 for every class; the clamp also turns the
          // NaN logit of an excluded row (non-finite input) into rs = 0 times 1
          const float dz = rs4[e] * __builtin_amdgcn_exp2f(
                                        fminf(fmaf(acc[fi][fj][4 * q + e] + cbv[fj], LOG2E, -l4[e]), 0.f));
          if (in && crole[fj] == 0) {
            dZ[(long long)(m0 + row) * ldz + ccol[fj]] = Elem<T>::from_f32(dz);
            cs[fj] += dz;
          }
        }
      }
    }
  }
  // Selected classes: dZ needs no recomputed logit, only S, Gamma and g.
  // With few of them in each wavefront (the large-vocabulary case) each is
  // done by all 64 lanes of its wavefront in the pass further down.  With
  // many, the work-group forms them in batches in the free operand stages:
  // one thread per tile row reads a selected column's S and Gamma (class-
  // major, so these reads are contiguous), and each lane then takes its own
  // elements from there.
  if (dense) {
    // the selected tile columns in ascending order, and each one's place
    bool is_sel = false;
    int before = 0;
    if (threadIdx.x < BN) {
      is_sel = s_sel[threadIdx.x] >= 0;  // -1 past the chunk end
      const unsigned long long bal = __ballot(is_sel);
      before = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) s_cnt[w] = __popcll(bal);
    }
    lds_barrier();
    int n_sel = 0, base = 0;
#pragma unroll
    for (int q = 0; q < BN / 64; ++q) {
      base += q < w ? s_cnt[q] : 0;
      n_sel += s_cnt[q];
    }
    if (threadIdx.x < BN) {
      s_pos[threadIdx.x] = is_sel ? base + before : -1;
      if (is_sel) s_list[base + before] = threadIdx.x;
    }
    lds_barrier();
    float* tmp = reinterpret_cast<float*>(smem);
    constexpr int PADR = BM + 1;  // column stride: conflict-free both ways
    constexpr int CAP = C::STAGE_BYTES / (PADR * (int)sizeof(float));
    for (int k0 = 0; k0 < n_sel; k0 += CAP) {
      const int kn = min(CAP, n_sel - k0);
      const int total = kn * BM;
      // DENSE_ILP elements per thread at a time: their S and Gamma loads (of
      // clamped, in-bounds elements, masked afterwards) are all issued before
      // the first is used
      for (int base = threadIdx.x; base < total; base += DENSE_ILP * C::THREADS) {
        float sv[DENSE_ILP], gv[DENSE_ILP];
#pragma unroll
        for (int u = 0; u < DENSE_ILP; ++u) {
          const int idx = min(base + u * C::THREADS, total - 1);
          const int kk = idx / BM, row = idx - kk * BM;
          const long long o = (long long)s_sel[s_list[k0 + kk]] * ldS + min(m0 + row, M - 1);
          sv[u] = S[o];
          gv[u] = Gam[o];
        }
#pragma unroll
        for (int u = 0; u < DENSE_ILP; ++u) {
          const int idx = base + u * C::THREADS;
          if (idx < total) {
            const int kk = idx / BM, row = idx - kk * BM;
            // S <= 0 (a log-probability); rows past M give 0
            tmp[kk * PADR + row] =
                (rows_full || m0 + row < M)
                    ? (float)(grad * (s_g[row] * exp_nonpos((double)sv[u]) - (double)gv[u]))
                    : 0.f;
          }
        }
      }
      lds_barrier();
#pragma unroll
      for (int fj = 0; fj < C::FN; ++fj) {
        const int slot = s_pos[acc_col<C>(fj)] - k0;
        if (crole[fj] != 2 || slot < 0 || slot >= kn) continue;
#pragma unroll 1
        for (int fi = 0; fi < C::FM; ++fi)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = acc_row<C>(fi, r);
            if (rows_full || m0 + row < M) {
              const float dz = tmp[slot * PADR + row];
              dZ[(long long)(m0 + row) * ldz + ccol[fj]] = Elem<T>::from_f32(dz);
              cs[fj] += dz;
            }
          }
      }
      lds_barrier();
    }
  }
  // column sum: the two lane halves hold the same column, then the waves
  // stacked along M; both combined in a fixed order.
#pragma unroll
  for (int fj = 0; fj < C::FN; ++fj) {
    cs[fj] += __shfl_xor(cs[fj], 32, 64);
    if (lane < 32) s_db[wm][acc_col<C>(fj)] = cs[fj];
  }
  // Few selected classes: each prefetched column of this wavefront by all 64
  // lanes (WM / 64 of the wavefront's rows each).
  if (!dense) sel_finish<C, T>(pre, s_g, m0, M, s_col, grad, dZ, ldz, s_db[wm]);
  lds_barrier();
  for (int c = threadIdx.x; c < BN; c += C::THREADS) {
    const int v = n0 + c;
    if (v < c1e) {
      float t = s_db[0][c];
#pragma unroll
      for (int q = 1; q < C::WGM; ++q) t += s_db[q][c];
      dbpart[(long long)mt * ldz + s_col[c]] = t;
    }
  }
}

// dXacc[m][d] (+)= sum_{c in chunk} dZ[m][c] W[c0 + c][d].  With BKM the
// weight operand is the transposed chunk Wt[d][c] (leading dimension ldb),
// otherwise the chunk's rows W[c0 + c][d] (leading dimension D).
template <class C, bool BKM>
__global__ __launch_bounds__(C::THREADS, C::MINWG) void k_dx(
    const typename C::type* __restrict__ dZ, int ldz, const typename C::type* __restrict__ Wc,
    int ldb, int M, int D, int Cc, float* __restrict__ dXacc, int first, int mtiles, int a_vec,
    int b_vec) {
  __shared__ __attribute__((aligned(16))) char smem[C::STAGE_BYTES];
  // column tiles fastest: the work-groups sharing one block of dZ rows run
  // together
  const int ntiles = (D + C::BN - 1) / C::BN;
  const int lin = xcd_tile(blockIdx.x, gridDim.x);
  const int nt = lin % ntiles, mt = lin / ntiles;
  (void)mtiles;
  const int m0 = mt * C::BM, n0 = nt * C::BN;
  f32x16 acc[C::FM][C::FN];
  gemm_tile<C, true, BKM>(dZ, ldz, m0, M, Wc, ldb, n0, D, 0, Cc, a_vec, b_vec, acc, smem);
#pragma unroll
  for (int fi = 0; fi < C::FM; ++fi)
#pragma unroll
    for (int fj = 0; fj < C::FN; ++fj) {
      const int col = n0 + acc_col<C>(fj);
      float old[16];
      if (!first) {
        // the fragment's 16 accumulator values are loaded together (clamped,
        // in-bounds addresses; a load under a per-lane condition is waited
        // for on the spot), then updated
        const int cc = min(col, D - 1);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int row = min(m0 + acc_row<C>(fi, rr), M - 1);
          old[rr] = dXacc[(long long)row * D + cc];
        }
      } else {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) old[rr] = 0.f;
      }
      if (col >= D) continue;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int row = m0 + acc_row<C>(fi, rr);
        if (row < M) dXacc[(long long)row * D + col] = first ? acc[fi][fj][rr] : old[rr] + acc[fi][fj][rr];
      }
    }
}

// part[s][i][d] = sum_{m in split s} dZ[m][i] X[m][d]  (i = chunk column).
template <class C>
__global__ __launch_bounds__(C::THREADS, C::MINWG) void k_dw(
    const typename C::type* __restrict__ dZ, int ldz, const typename C::type* __restrict__ X,
    int M, int D, int Cc, float* __restrict__ part, int itiles, int ntiles, int kchunk, int a_vec,
    int b_vec) {
  __shared__ __attribute__((aligned(16))) char smem[C::STAGE_BYTES];
  // column tiles fastest: the work-groups sharing one block of dZ columns
  // run together
  const int lin = xcd_tile(blockIdx.x, gridDim.x);
  const int per = itiles * ntiles;
  const int s = lin / per, rem = lin % per;
  const int nt = rem % ntiles, it = rem / ntiles;
  const int i0 = it * C::BM, n0 = nt * C::BN;
  const int kb = s * kchunk, ke = min(M, kb + kchunk);
  f32x16 acc[C::FM][C::FN];
  gemm_tile<C, false, false>(dZ, ldz, i0, Cc, X, D, n0, D, kb, ke, a_vec, b_vec, acc, smem);
#pragma unroll
  for (int fi = 0; fi < C::FM; ++fi)
#pragma unroll
    for (int fj = 0; fj < C::FN; ++fj) {
      const int col = n0 + acc_col<C>(fj);
      if (col >= D) continue;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int row = i0 + acc_row<C>(fi, rr);
        if (row < Cc) part[((long long)s * Cc + row) * D + col] = acc[fi][fj][rr];
      }
    }
}
// dst[d][c] = src[c][d] for a rows x D block (64 x 64 tiles through LDS);
// columns c in [rows, rows_pad) of dst are written as zeros.
template <typename T>
__global__ void k_transpose(const T* __restrict__ src, int rows, int rows_pad, int D,
                            T* __restrict__ dst, int ldd) {
  __shared__ T t[64][65];
  const int r0 = blockIdx.y * 64, d0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int rr = r0 + r, dd = d0 + tx;
    t[r][tx] = (rr < rows && dd < D) ? src[(long long)rr * D + dd] : T(0);
  }
  lds_barrier();
  for (int d = ty; d < 64; d += 4) {
    const int dd = d0 + d, rr = r0 + tx;
    if (dd < D && rr < rows_pad) dst[(long long)dd * ldd + rr] = t[tx][d];
  }
}

// The same for 2-byte elements with 16-byte accesses on both sides (D and
// ldd multiples of 8, 16-byte aligned src and dst): eight consecutive
// elements of a source row are loaded and scattered into the LDS tile by
// column; eight consecutive elements of a destination row are gathered from
// it and stored.
template <typename T>
__global__ __launch_bounds__(256) void k_transpose16(const T* __restrict__ src, int rows,
                                                     int rows_pad, int D, T* __restrict__ dst,
                                                     int ldd) {
  static_assert(sizeof(T) == 2, "2-byte elements");
  __shared__ T t[64][66];  // t[d][c]
  const int r0 = blockIdx.y * 64, d0 = blockIdx.x * 64;
  for (int i = threadIdx.x; i < 512; i += 256) {
    const int r = i >> 3, v = i & 7;
    const int rr = r0 + r, dd = d0 + v * 8;
    uint4 x = {0u, 0u, 0u, 0u};
    if (rr < rows && dd < D) x = *reinterpret_cast<const uint4*>(src + (long long)rr * D + dd);
    const T* e = reinterpret_cast<const T*>(&x);
#pragma unroll
    for (int j = 0; j < 8; ++j) t[v * 8 + j][r] = e[j];
  }
  lds_barrier();
  for (int i = threadIdx.x; i < 512; i += 256) {
    const int d = i >> 3, v = i & 7;
    const int dd = d0 + d, rr = r0 + v * 8;
    if (dd >= D) continue;
    T* out = dst + (long long)dd * ldd + rr;
    if (rr + 8 <= rows_pad) {
      uint4 x;
      T* e = reinterpret_cast<T*>(&x);
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = t[d][v * 8 + j];
      *reinterpret_cast<uint4*>(out) = x;
    } else {
      for (int j = 0; j < 8 && rr + j < rows_pad; ++j) out[j] = t[d][v * 8 + j];
    }
  }
}

__global__ void k_cast_bf16(const float* __restrict__ src, bf16_t* __restrict__ dst, long long n) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x)
    dst[i] = f32_to_bf16(src[i]);
}

// ------------------------------------------------ bf16 core for 256 x 256 tiles
// A second GEMM core for bf16 heads whose reduction length is a multiple of
// 64 (the LLM head): a 256 x 256 work-group tile of eight wavefronts, WGM x
// WGN of them, both operands K-contiguous.  Each k stage holds BK values of
// all 256 rows of both operands; NBUF stages live in LDS (at most 128 KiB)
// and are filled NBUF - 1 stages ahead by 16-byte global->LDS loads that need
// no staging registers: one wave-wide load writes 1 KiB of LDS, lane l at
// byte 16 l.  A work-group barrier (after each wave's loads of the next
// stage have landed) separates the stages.
//
// LDS layout: row r at byte ROWB r (ROWB = 2 BK), its 16-byte chunk c (k
// values 8c..8c+7) at chunk position c ^ ((r / (256 / ROWB)) % (ROWB / 16)).
// A 16-byte fragment read is served for 16 lanes at a time over 64 four-byte
// banks; the 16 rows one such group reads share each 256-byte bank window
// 256 / ROWB at a time, and the permutation gives the rows sharing a window
// slot distinct chunk positions, so each group touches every bank once.  The
// loads write whole 1 KiB blocks, so they place row r's chunk c by choosing
// which global chunk each lane fetches.
//
// Within a stage, lane half h feeds the MFMA k values h BK/2 .. (h+1) BK/2 - 1,
// eight per v_mfma_f32_32x32x16_bf16 (the same relabelling of k for both
// operands).
template <int WGM_, int WGN_, int BK_, int NBUF_>
struct CfgBig {
  using type = bf16_t;
  static constexpr int BM = 256, BN = 256;
  static constexpr int WGM = WGM_, WGN = WGN_, WAVES = WGM * WGN, THREADS = 64 * WAVES;
  static constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
  static constexpr int BK = BK_, ROWB = 2 * BK, CH = ROWB / 16, KS = BK / 16;
  static constexpr int RPI = 1024 / ROWB;             // rows per 1 KiB load
  static constexpr int RPW = 256 / ROWB;              // rows per 256-byte bank window
  static constexpr int NBUF = NBUF_, DEPTH = NBUF - 1;
  static constexpr int TILEB = 256 * ROWB;            // one operand stage
  static constexpr int STAGEB = 2 * TILEB;            // both operands
  static constexpr int LDS_BYTES = NBUF * STAGEB;
  static constexpr int NLD = TILEB / 1024 / WAVES;    // 1 KiB loads per wave and operand
  static constexpr int INFLIGHT = (DEPTH - 1) * 2 * NLD;  // loads allowed past a barrier
  static constexpr int MINWG = 1;
  static_assert(TILEB % (1024 * WAVES) == 0 && WM % 32 == 0 && WN % 32 == 0, "big tile");
  static_assert((BK == 32 || BK == 64) && NBUF >= 2 && LDS_BYTES <= 128 * 1024, "big stages");
};
// The forward runs eight 64 x 128 wavefronts (4 x 2; ahead of 2 x 4 on the
// LLM head; its FP64 epilogue does not fit the registers of more).  The
// recompute and dX products run sixteen 64 x 64 wavefronts (4 x 4, four per
// SIMD; measured about 2% and 3% faster).
using CfgBigFwd = CfgBig<4, 2, 64, 2>;
using CfgBigRec = CfgBig<4, 4, 64, 2>;
using CfgBigDx = CfgBig<4, 4, 64, 2>;

#define PCX_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

template <class C>
__device__ __forceinline__ int big_swz(int r) { return (r / C::RPW) % C::CH; }

// Global->LDS loads of one operand stage: rows r0.. (clamped to rlim - 1;
// those rows only feed accumulator rows the callers discard), k0..k0+BK-1.
template <class C>
__device__ __forceinline__ void big_stage(const bf16_t* __restrict__ G, long long ld, int r0,
                                          int rlim, int k0, char* dst) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < C::NLD; ++q) {
    const int u = w * C::NLD + q;  // 1 KiB block: rows RPI u .. RPI u + RPI - 1
    const int row = u * C::RPI + l / C::CH;
    const int c = (l % C::CH) ^ big_swz<C>(row);
    const int gr = min(r0 + row, rlim - 1);
    __builtin_amdgcn_global_load_lds((const void*)(G + (long long)gr * ld + k0 + c * 8),
                                     PCX_LDS_PTR(dst + u * 1024), 16, 0, 0);
  }
}

// Two fp32 values rounded to nearest-even bf16 by the hardware conversion,
// packed low (lo) / high (hi).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b16x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b16x2));
}

// Value of lane l ^ 1 (DPP quad permutation 1,0,3,2) and of lane l ^ 2
// (2,3,0,1).
__device__ __forceinline__ uint32_t lane_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t lane_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);
}

// Barrier of the big core: this wave's LDS reads are complete and at most N
// of its global memory operations are in flight, then all waves meet.  (A
// release fence would also wait for every outstanding global->LDS load.)
template <int N>
__device__ __forceinline__ void big_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  // vmcnt(N) (bits 3:0 and 15:14), expcnt(7), lgkmcnt(0)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  asm volatile("s_barrier" ::: "memory");
}

template <class C>
__device__ __forceinline__ void big_frags(const char* buf, int j, int wm, int wn,
                                          bf16x8 (&a)[C::FM], bf16x8 (&b)[C::FN]) {
  const int lane = threadIdx.x & 63, i = lane & 31, h = lane >> 5;
  const int c = h * C::KS + j;
#pragma unroll
  for (int f = 0; f < C::FM; ++f) {
    const int r = wm * C::WM + f * 32 + i;
    a[f] = __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const uint4*>(buf + r * C::ROWB + ((c ^ big_swz<C>(r)) << 4)));
  }
#pragma unroll
  for (int f = 0; f < C::FN; ++f) {
    const int r = wn * C::WN + f * 32 + i;
    b[f] = __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const uint4*>(buf + C::TILEB + r * C::ROWB +
                                                ((c ^ big_swz<C>(r)) << 4)));
  }
}

// Pipeline state carried from one tile to the next by a work-group that
// walks several tiles: the LDS buffer that holds (or will hold) the tile's
// first k stage, and whether the loads of its first NBUF - 1 stages were
// already issued by the previous tile (cross-tile prefetch).
struct BigPipe {
  int buf0 = 0;
  bool staged = false;
};

// Operand rows of the next tile (its first stages are loaded during this
// tile's last stages).
struct BigNext {
  bool valid;
  int m0, m_lim, n0, n_lim;
};

// acc = A[m0:m0+256, k] . B[n0:n0+256, k]^T over k in [0, K); K % BK == 0,
// K > 0, lda and ldb multiples of 8, A and B 16-byte aligned, m_lim and
// n_lim >= 1.  With next.valid, the next tile's first stages (same A, B, lda,
// ldb, K) are loaded during this tile's last stages and `pipe` is updated for
// the next call; without, the call ends with no load in flight.  Every call
// starts with a barrier, so between two calls the waves may only touch LDS
// outside the operand buffers.
template <class C>
__device__ __forceinline__ void gemm_big(const bf16_t* __restrict__ A, long long lda, int m0,
                                         int m_lim, const bf16_t* __restrict__ B, long long ldb,
                                         int n0, int n_lim, int K, f32x16 (&acc)[C::FM][C::FN],
                                         char* smem, BigPipe& pipe, const BigNext& next) {
  const int w = threadIdx.x >> 6, wm = w / C::WGN, wn = w % C::WGN;
  const int nk = K / C::BK;
  const int b0 = pipe.buf0;
#pragma unroll
  for (int fi = 0; fi < C::FM; ++fi)
#pragma unroll
    for (int fj = 0; fj < C::FN; ++fj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[fi][fj][r] = 0.f;
  // Loads of pipeline stage g: this tile's stage g, past the end the next
  // tile's stage g - nk (clamped to its last stage), or (no next tile) a
  // harmless reload of the last stage into a buffer no longer read.
  auto issue = [&](int g) {
    const bool own = g < nk, nx = !own && next.valid;
    const int ra = nx ? next.m0 : m0, ra_lim = nx ? next.m_lim : m_lim;
    const int rb = nx ? next.n0 : n0, rb_lim = nx ? next.n_lim : n_lim;
    const int k = (own ? g : nx ? min(g - nk, nk - 1) : nk - 1) * C::BK;
    char* dst = smem + ((b0 + g) % C::NBUF) * C::STAGEB;
    big_stage<C>(A, lda, ra, ra_lim, k, dst);
    big_stage<C>(B, ldb, rb, rb_lim, k, dst + C::TILEB);
  };
  if (!pipe.staged) {
#pragma unroll
    for (int g = 0; g < C::DEPTH; ++g) issue(g);
  }
  big_barrier<C::INFLIGHT>();
  bf16x8 fa[2][C::FM], fb[2][C::FN];
  big_frags<C>(smem + b0 * C::STAGEB, 0, wm, wn, fa[0], fb[0]);
  for (int s = 0; s < nk; ++s) {
    const char* cur = smem + ((b0 + s) % C::NBUF) * C::STAGEB;
    const char* nxt = smem + ((b0 + s + 1) % C::NBUF) * C::STAGEB;
    issue(s + C::DEPTH);
#pragma unroll
    for (int j = 0; j < C::KS; ++j) {
      if (j + 1 < C::KS) {
        big_frags<C>(cur, j + 1, wm, wn, fa[(j + 1) & 1], fb[(j + 1) & 1]);
      } else {
        big_barrier<C::INFLIGHT>();
        big_frags<C>(nxt, 0, wm, wn, fa[(j + 1) & 1], fb[(j + 1) & 1]);
      }
#pragma unroll
      for (int fi = 0; fi < C::FM; ++fi)
#pragma unroll
        for (int fj = 0; fj < C::FN; ++fj)
          acc[fi][fj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[j & 1][fi], fb[j & 1][fj],
                                                                acc[fi][fj], 0, 0, 0);
      // one fragment read between consecutive MFMAs, so the reads of the
      // next k step overlap this step's matrix work
#pragma unroll
      for (int q = 0; q < C::FM + C::FN; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, C::FM * C::FN - C::FM - C::FN, 0);
    }
  }
  pipe.buf0 = (b0 + nk) % C::NBUF;
  pipe.staged = next.valid;
  if (!next.valid) big_barrier<0>();
}

// One tile, nothing carried over.
template <class C>
__device__ __forceinline__ void gemm_big1(const bf16_t* __restrict__ A, long long lda, int m0,
                                          int m_lim, const bf16_t* __restrict__ B, long long ldb,
                                          int n0, int n_lim, int K, f32x16 (&acc)[C::FM][C::FN],
                                          char* smem) {
  BigPipe pipe;
  const BigNext none{false, 0, 1, 0, 1};
  gemm_big<C>(A, lda, m0, m_lim, B, ldb, n0, n_lim, K, acc, smem, pipe, none);
}

// Forward on the big core, computed transposed: the tile is 256 vocabulary
// rows (operand A = W) by 256 frames (operand B = X), so every lane holds 64
// vocabulary values of each of its FN frames and the per-frame log-sum-exp
// of a tile needs no cross-lane step.  One work-group: 256 frames x one
// span-wide vocabulary span in 256-row tiles.  Per tile and frame, each
// lane folds max and FP64 sum of exp(z - max) over its 64 values into its
// running partial; at the end of the span the partials of the two lane
// halves and of the WGM wave rows are folded in a fixed order.  Selected
// vocabulary rows are gathered into Zsel (class-major, K x M), 32 frames per
// coalesced store.
template <class C, bool MASKED>
__global__ __launch_bounds__(C::THREADS, 1) void k_fwd_lse_big(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ W, const bf16_t* __restrict__ bias,
    int M, int D, int V, const int* __restrict__ col2sel, float* __restrict__ Zsel,
    double2* __restrict__ part, int nspan, int ftiles, int span) {
  // One LDS object for everything: with a second one, the compiler makes
  // every fragment read wait for all outstanding global->LDS loads.
  constexpr int O_SEL = C::LDS_BYTES, O_BIAS = O_SEL + 2 * C::BM * 4;
  constexpr int O_FM = O_BIAS + 2 * C::BM * 4, O_FS = O_FM + C::WGM * C::BN * 4;
  constexpr int O_EXP = O_FS + C::WGM * C::BN * 8;
  __shared__ __attribute__((aligned(16))) char smem[O_EXP + 64 * 8];
  int (*s_sel)[C::BM] = reinterpret_cast<int (*)[C::BM]>(smem + O_SEL);
  float (*s_bias)[C::BM] = reinterpret_cast<float (*)[C::BM]>(smem + O_BIAS);
  float (*f_m)[C::BN] = reinterpret_cast<float (*)[C::BN]>(smem + O_FM);
  double (*f_s)[C::BN] = reinterpret_cast<double (*)[C::BN]>(smem + O_FS);
  double* s_exp = reinterpret_cast<double*>(smem + O_EXP);  // 2^(j/64)
  if (threadIdx.x < 64) s_exp[threadIdx.x] = exp_tab_entry(threadIdx.x);
  int ft, sp;
  grouped_tile<8>(xcd_tile(blockIdx.x, gridDim.x), ftiles, nspan, ft, sp);
  const int f0 = ft * C::BN;
  const int c_begin = sp * span, c_end = min(V, c_begin + span);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w / C::WGN;
  float run_m[C::FN];
  double run_s[C::FN];
#pragma unroll
  for (int fj = 0; fj < C::FN; ++fj) {
    run_m[fj] = -INFINITY;
    run_s[fj] = 0.0;
  }
  // the first tile's row data; later tiles' are loaded during the tile before
  // (unconditional loads of a clamped id, masked afterwards: a load under a
  // per-lane condition is waited for on the spot)
  int nsel = -2;
  float nbias = 0.f;
  if (threadIdx.x < C::BM) {
    const int v = c_begin + threadIdx.x;
    const int vc = min(v, c_end - 1);
    const int sl = col2sel[vc];
    const float bv = bias != nullptr ? bf16_to_f32(bias[vc]) : 0.f;
    nsel = v < c_end ? sl : -2;  // -2: past the span
    nbias = v < c_end ? bv : 0.f;
  }
  BigPipe pipe;
  int par = 0;
  for (int v0 = c_begin; v0 < c_end; v0 += C::BM, par ^= 1) {
    // visible after the core's barriers; the buffer written here was last
    // read two tiles ago
    if (threadIdx.x < C::BM) {
      s_sel[par][threadIdx.x] = nsel;
      s_bias[par][threadIdx.x] = nbias;
    }
    const BigNext next{v0 + C::BM < c_end, v0 + C::BM, c_end, f0, M};
    // the next tile's row data is requested before this tile's product and
    // used after it, so its latency hides behind the product
    int psel = 0;
    float pbias = 0.f;
    const int vn = v0 + C::BM + (int)threadIdx.x;
    if (next.valid && threadIdx.x < C::BM) {
      const int vc = min(vn, c_end - 1);
      psel = col2sel[vc];
      pbias = bias != nullptr ? bf16_to_f32(bias[vc]) : 0.f;
    }
    f32x16 acc[C::FM][C::FN];
    gemm_big<C>(W, D, v0, c_end, X, D, f0, M, D, acc, smem, pipe, next);
    if (next.valid && threadIdx.x < C::BM) {
      nsel = vn < c_end ? psel : -2;
      nbias = vn < c_end ? pbias : 0.f;
    }
#pragma unroll
    for (int fj = 0; fj < C::FN; ++fj) {
      const int frame = f0 + acc_col<C>(fj);
      float mx = -INFINITY;
      float chk = 0.f;  // stays 0 unless a logit is NaN or infinite
#pragma unroll
      for (int fi = 0; fi < C::FM; ++fi)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r0 = acc_row<C>(fi, 4 * q);
          const int4 sel4 = *reinterpret_cast<const int4*>(&s_sel[par][r0]);
          const f32x4 b4 = *reinterpret_cast<const f32x4*>(&s_bias[par][r0]);
          const int sl[4] = {sel4.x, sel4.y, sel4.z, sel4.w};
          float z[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            z[e] = acc[fi][fj][4 * q + e] + b4[e];
            chk = fmaf(z[e], 0.f, chk);
          }
          // the gather, behind one test per group of four rows (selected
          // rows are rare in a large vocabulary: most groups skip it whole)
          if (max(max(sl[0], sl[1]), max(sl[2], sl[3])) >= 0 && frame < M) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (sl[e] >= 0) Zsel[(long long)sl[e] * M + frame] = z[e];
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // in the sum: every vocabulary row of the span, or (masked)
            // only the unselected ones
            acc[fi][fj][4 * q + e] = (MASKED ? sl[e] == -1 : sl[e] >= -1) ? z[e] : -INFINITY;
            mx = fmaxf(mx, acc[fi][fj][4 * q + e]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      double sum = 0.0;
      if (mx != -INFINITY) {
#pragma unroll
        for (int fi = 0; fi < C::FM; ++fi) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sum += exp_nonpos_tab((double)acc[fi][fj][r] - (double)mx, s_exp);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      nonfinite_partial(chk, mx, sum);
      lse_fold(run_m[fj], run_s[fj], mx, sum);
    }
  }
  // lane halves (lower half first), then wave rows in order
#pragma unroll
  for (int fj = 0; fj < C::FN; ++fj) {
    const float om = __shfl_xor(run_m[fj], 32, 64);
    const double os = __shfl_xor(run_s[fj], 32, 64);
    float m1 = lane < 32 ? run_m[fj] : om;
    double s1 = lane < 32 ? run_s[fj] : os;
    lse_fold(m1, s1, lane < 32 ? om : run_m[fj], lane < 32 ? os : run_s[fj]);
    if (lane < 32) {
      f_m[wm][acc_col<C>(fj)] = m1;
      f_s[wm][acc_col<C>(fj)] = s1;
    }
  }
  lds_barrier();
  for (int c = threadIdx.x; c < C::BN; c += C::THREADS) {
    const int frame = f0 + c;
    if (frame >= M) continue;
    float fm = f_m[0][c];
    double fs = f_s[0][c];
#pragma unroll
    for (int q = 1; q < C::WGM; ++q) lse_fold(fm, fs, f_m[q][c], f_s[q][c]);
    part[(long long)frame * nspan + sp] = make_double2((double)fm, fs);
  }
}

// Backward recompute on the big core (frames x vocabulary, as k_recompute):
// the same per-element formulas, stored four columns (8 bytes) per lane; in
// addition the chunk block's columns between the chunk end and the next
// multiple of 64 are written as zeros, because the dX product on the big
// core reduces over whole 64-column steps.
// dZ of a selected class on the bf16 core: grad (g p - Gamma) with p = exp(S)
// to fp32 precision (exp_split; far below the bf16 rounding of the result and
// the product's own error in S), combined in FP64 and rounded once.  The
// NaN score of an excluded row (non-finite input; g and Gamma are 0 there)
// is taken as -1e6, so its value is 0.
__device__ __forceinline__ float sel_dz(double grad, double g, float s, float gam) {
  int n;
  const float m = exp_split(fmaxf(s, -1e6f), n);
  return (float)(grad * fma(g, ldexp((double)m, n), -(double)gam));
}

template <class C>
__global__ __launch_bounds__(C::THREADS, 1) void k_recompute_big(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ W, const bf16_t* __restrict__ bias,
    int M, int D, int c0, int c1, const int* __restrict__ col2sel,
    const float* __restrict__ lamf, const double* __restrict__ g, const float* __restrict__ S,
    const float* __restrict__ Gam, double grad, bf16_t* __restrict__ dZ, int ldz,
    float* __restrict__ dbpart, int mtiles, const double* __restrict__ gu,
    const float* __restrict__ lamu, long long ldS) {
  constexpr int BM = C::BM, BN = C::BN;
  constexpr float LOG2E = 1.44269504088896340736f;
  // selected columns prefetched per wavefront: a fixed 24 KiB LDS region
  constexpr int SELP = SEL_PRE_BIG * 8 / C::WAVES;
  static_assert(SELP >= 1, "prefetch region");
  static_assert(C::WM == 64, "selected-class pass: one row per lane");
  // one LDS object (see k_fwd_lse_big): the operand stages, then the row and
  // column data, then per wavefront the S and Gamma values (64 rows each) of
  // up to SELP selected columns.  After the product the stage buffers
  // hold the selected-class values on their way to the accumulators (from
  // offset 0) and the column sums (from O_DB).
  constexpr int O_G = C::LDS_BYTES, O_SEL = O_G + BM * 8, O_BIAS = O_SEL + BN * 4;
  constexpr int O_LAM = O_BIAS + BN * 4, O_RS = O_LAM + BM * 4, O_PRE = O_RS + BM * 4;
  constexpr int O_DB = C::LDS_BYTES / 2;
  static_assert(C::WAVES * SELP * (C::WM + 1) * 4 <= O_DB &&
                    O_DB + C::WGM * BN * 4 <= C::LDS_BYTES, "post-product LDS use");
  __shared__ __attribute__((aligned(16))) char smem[O_PRE + C::WAVES * SELP * 512];
  double* s_g = reinterpret_cast<double*>(smem + O_G);
  int* s_sel = reinterpret_cast<int*>(smem + O_SEL);
  float* s_bias = reinterpret_cast<float*>(smem + O_BIAS);
  float* s_lam2 = reinterpret_cast<float*>(smem + O_LAM);
  float* s_rs = reinterpret_cast<float*>(smem + O_RS);
  float (*s_db)[BN] = reinterpret_cast<float (*)[BN]>(smem + O_DB);
  // groups of 4 row tiles (measured 1.2% ahead of 8 and 2 on the LLM head)
  int mt, nt;
  grouped_tile<4>(xcd_tile(blockIdx.x, gridDim.x), mtiles, (c1 - c0 + BN - 1) / BN, mt, nt);
  const int m0 = mt * BM, n0 = c0 + nt * BN;
  const int c_pad = c0 + ((c1 - c0 + 63) & ~63);
  // Row and column data: unconditional loads of clamped (in-bounds) entries,
  // masked afterwards, so that they are in flight together (a load under a
  // per-lane condition is waited for on the spot).
  for (int c = threadIdx.x; c < BN; c += C::THREADS) {
    const int v = n0 + c;
    const bool in = v < c1;
    const int vc = in ? v : c1 - 1;
    const int sl = col2sel[vc];
    const float bv = bias != nullptr ? bf16_to_f32(bias[vc]) : 0.f;
    s_sel[c] = in ? sl : -1;
    s_bias[c] = in ? bv : 0.f;
  }
  for (int rr = threadIdx.x; rr < BM; rr += C::THREADS) {
    const int mm = m0 + rr;
    const bool in = mm < M;
    const int mc = in ? mm : M - 1;
    const double gv = g[mc];
    const double guv = gu != nullptr ? gu[mc] : gv;
    const float lv = lamu != nullptr ? lamu[mc] : lamf[mc];
    s_g[rr] = in ? gv : 0.0;
    // unselected classes: dZ = rs * exp(z - shift); rs = grad g_m and shift =
    // lambda_m, or in the grouped form grad gu_m and the other column o_m
    s_rs[rr] = in ? (float)(grad * guv) : 0.f;
    s_lam2[rr] = in ? lv * LOG2E : 0.f;
  }
  lds_barrier();
  // the wavefront index as a uniform (scalar) value
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w / C::WGN;
  // Selected columns of this wavefront, in (fragment column, lane) order; with
  // at most SELP of them their S and Gamma values are loaded straight
  // into LDS now, behind the product (they do not depend on it).
  int pn, pcol[SELP];
  {
    unsigned long long mk[C::FN];
    int cs_[C::FN];
    pn = 0;
#pragma unroll
    for (int fj = 0; fj < C::FN; ++fj) {
      const int col = acc_col<C>(fj);
      cs_[fj] = s_sel[col];
      mk[fj] = __ballot(lane < 32 && n0 + col < c1 && cs_[fj] >= 0);
      pn += __popcll(mk[fj]);
    }
    const int grow = min(m0 + wm * C::WM + lane, M - 1);
#pragma unroll
    for (int k = 0; k < SELP; ++k) {
      int sel = 0, col = 0;
      bool found = false;
#pragma unroll
      for (int fj = 0; fj < C::FN; ++fj) {
        if (!found && mk[fj] != 0ull) {
          const int src = __ffsll((long long)mk[fj]) - 1;
          mk[fj] &= mk[fj] - 1;
          sel = __builtin_amdgcn_readlane(cs_[fj], src);
          col = (w % C::WGN) * C::WN + fj * 32 + src;
          found = true;
        }
      }
      pcol[k] = col;
      if (found && pn <= SELP) {
        char* dst = smem + O_PRE + (w * SELP + k) * 512;
        __builtin_amdgcn_global_load_lds((const void*)(S + sel * ldS + grow),
                                         PCX_LDS_PTR(dst), 4, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(Gam + sel * ldS + grow),
                                         PCX_LDS_PTR(dst + 256), 4, 0, 0);
      }
    }
  }
  f32x16 acc[C::FM][C::FN];
  gemm_big1<C>(X, D, m0, M, W, D, n0, c1, D, acc, smem);
  const bool rows_full = m0 + BM <= M;
  // Column roles: 0 = unselected class (formula below), 1 = padding up to
  // the next multiple of 64 (zero), 2 = selected class (its value from S and
  // Gamma, patched into the accumulators or stored by the dense pass) or past
  // the padding (not stored).
  int csel[C::FN], crole[C::FN];
  float cbv[C::FN], cs[C::FN];
#pragma unroll
  for (int fj = 0; fj < C::FN; ++fj) {
    const int col = acc_col<C>(fj);
    const int v = n0 + col;
    csel[fj] = s_sel[col];
    cbv[fj] = s_bias[col];
    crole[fj] = v < c1 ? (csel[fj] < 0 ? 0 : 2) : (v < c_pad ? 1 : 2);
    cs[fj] = 0.f;
  }
  // Few selected classes (at most SELP in this wavefront): each
  // column by all 64 lanes (one of the wavefront's rows each, sel_dz),
  // into LDS (one region per wavefront) with the column's sum
  // over the wavefront's rows (a fixed-order wave sum) ...
  const bool dense = pn > SELP;
  // this wavefront's share of the stage buffers (either pass below)
  float* tmp = reinterpret_cast<float*>(smem) + w * (O_DB / C::WAVES / 4);
  if (!dense && pn > 0) {
    const int row = wm * C::WM + lane;
#pragma unroll
    for (int k = 0; k < SELP; ++k) {
      if (k < pn) {
        const float* pv = reinterpret_cast<const float*>(smem + O_PRE +
                                                         (w * SELP + k) * 512);
        float sum = 0.f, dz = 0.f;
        if (m0 + row < M) {
          dz = sel_dz(grad, s_g[row], pv[lane], pv[64 + lane]);
          sum = dz;
        }
        tmp[k * C::WM + lane] = dz;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
        if (lane == 0) tmp[SELP * C::WM + k] = sum;
      }
    }
  }
  // Unselected classes, in place of the accumulators.  Padding columns get
  // the bias -inf, so their value is exp2(-inf) = 0.  The column sums take
  // every column; those of selected columns are replaced further down.
#pragma unroll
  for (int fj = 0; fj < C::FN; ++fj)
    if (crole[fj] == 1) cbv[fj] = -INFINITY;
#pragma unroll
  for (int fi = 0; fi < C::FM; ++fi) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row0 = acc_row<C>(fi, 4 * q);
      const f32x4 rs4 = *reinterpret_cast<const f32x4*>(s_rs + row0);
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(s_lam2 + row0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool in = rows_full || m0 + row0 + e < M;
#pragma unroll
        for (int fj = 0; fj < C::FN; ++fj) {
          // the exponent is <= 0 for every class; the clamp also turns the
          // NaN logit of an excluded row (non-finite input) into rs = 0 times 1
          const float dz = rs4[e] * __builtin_amdgcn_exp2f(
                                        fminf(fmaf(acc[fi][fj][4 * q + e] + cbv[fj], LOG2E, -l4[e]), 0.f));
          acc[fi][fj][4 * q + e] = dz;
          cs[fj] += in ? dz : 0.f;
        }
      }
    }
  }
  // Many selected classes (more than SELP in this wavefront): in batches of
  // up to SLOTS columns, each column by all 64 lanes (one row each) into an
  // LDS slot, then each lane that owns a selected column of the batch takes
  // its 32 rows from that column's slot into the accumulators, with their sum
  // as its part of the column sum.  The wavefront's selected ids are listed
  // in LDS (in the prefetch region, unused with this many) in (fragment
  // column, lane) order.
  if (dense) {
    constexpr int SLOT = C::WM + 4;  // 16-byte aligned slots, 4 banks apart
    constexpr int SLOTS = 8;  // (15 fit; 8 keeps the loads in registers)
    static_assert(C::WAVES * SLOTS * SLOT * 4 <= O_DB && SELP * 128 >= C::WN, "dense pass LDS use");
    float* buf = tmp;
    int* list = reinterpret_cast<int*>(smem + O_PRE) + w * (SELP * 128);
    const int h = lane >> 5;
    int rank[C::FN], tot = 0;
    bool mine[C::FN];
#pragma unroll
    for (int fj = 0; fj < C::FN; ++fj) {
      const unsigned long long mk = __ballot(lane < 32 && csel[fj] >= 0);
      const unsigned long long bit = 1ull << (lane & 31);
      mine[fj] = (mk & bit) != 0ull;
      rank[fj] = tot + __popcll(mk & (bit - 1ull));
      tot += __popcll(mk);
      if (lane < 32 && mine[fj]) list[rank[fj]] = csel[fj];
    }
    const int trow = wm * C::WM + lane;
    const int grow = min(m0 + trow, M - 1);
    const bool rin = m0 + trow < M;
    const double gr = s_g[trow];
    for (int b0 = 0; b0 < tot; b0 += SLOTS) {
      // every load of the batch in flight together (clamped to the last
      // listed column past the end)
      float sv[SLOTS], gv[SLOTS];
#pragma unroll
      for (int k = 0; k < SLOTS; ++k) {
        const long long base = (long long)list[min(b0 + k, tot - 1)] * ldS + grow;
        sv[k] = S[base];
        gv[k] = Gam[base];
      }
#pragma unroll
      for (int k = 0; k < SLOTS; ++k)
        if (b0 + k < tot) buf[k * SLOT + lane] = rin ? sel_dz(grad, gr, sv[k], gv[k]) : 0.f;
#pragma unroll
      for (int fj = 0; fj < C::FN; ++fj) {
        const int sl = rank[fj] - b0;
        const bool own = mine[fj] && sl >= 0 && sl < SLOTS;
        const float* src = buf + (own ? sl : 0) * SLOT + 4 * h;
        float sum = 0.f;
#pragma unroll
        for (int fi = 0; fi < C::FM; ++fi)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 v4 = *reinterpret_cast<const f32x4*>(src + fi * 32 + 8 * q);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[fi][fj][4 * q + e] = own ? v4[e] : acc[fi][fj][4 * q + e];
              sum += v4[e];
            }
          }
        if (own) cs[fj] = sum;
      }
    }
  }
#pragma unroll
  for (int fj = 0; fj < C::FN; ++fj) {
    cs[fj] += __shfl_xor(cs[fj], 32, 64);
    if (lane < 32) s_db[wm][acc_col<C>(fj)] = cs[fj];
  }
  // ... and into the accumulators of the lanes that own the selected columns;
  // their column sums overwrite the ones just written (later writes of this
  // wavefront to the same LDS word take effect after earlier ones).
  if (!dense && pn > 0) {
    const int h = lane >> 5;
#pragma unroll
    for (int k = 0; k < SELP; ++k) {
      if (k < pn) {
        const int cw = pcol[k] - (w % C::WGN) * C::WN;
        const bool own = (lane & 31) == (cw & 31);
#pragma unroll
        for (int fj = 0; fj < C::FN; ++fj) {
          if (fj != (cw >> 5)) continue;  // the same for the whole wavefront
#pragma unroll
          for (int fi = 0; fi < C::FM; ++fi)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x4 v4 =
                  *reinterpret_cast<const f32x4*>(tmp + k * C::WM + fi * 32 + 8 * q + 4 * h);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                acc[fi][fj][4 * q + e] = own ? v4[e] : acc[fi][fj][4 * q + e];
            }
        }
        if (lane == 0) s_db[wm][pcol[k]] = tmp[SELP * C::WM + k];
      }
    }
  }
  // Stores of four consecutive columns (8 bytes) per lane: a lane holds four
  // rows of one column, so lanes l, l ^ 1 and then l, l ^ 2 trade values until
  // lane l holds row (l & 3) of the group for columns (l & ~3) .. (l & ~3) + 3.
  {
    const int odd = lane & 1, b1 = (lane >> 1) & 1;
#pragma unroll
    for (int fi = 0; fi < C::FM; ++fi) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = acc_row<C>(fi, 4 * q) + (lane & 3);
        const bool rin = rows_full || m0 + row < M;
#pragma unroll
        for (int fj = 0; fj < C::FN; ++fj) {
          const float v[4] = {acc[fi][fj][4 * q], acc[fi][fj][4 * q + 1], acc[fi][fj][4 * q + 2],
                              acc[fi][fj][4 * q + 3]};
          const float r01 = __uint_as_float(lane_xor1(__float_as_uint(odd ? v[0] : v[1])));
          const float r23 = __uint_as_float(lane_xor1(__float_as_uint(odd ? v[2] : v[3])));
          // even lanes: rows 0 / 2 of columns (l, l + 1); odd: rows 1 / 3 of (l - 1, l)
          const uint32_t p0 = odd ? pack_bf16x2(r01, v[1]) : pack_bf16x2(v[0], r01);
          const uint32_t p1 = odd ? pack_bf16x2(r23, v[3]) : pack_bf16x2(v[2], r23);
          const uint32_t r = lane_xor2(b1 ? p0 : p1);
          const uint2 out = b1 ? make_uint2(r, p1) : make_uint2(p0, r);
          const int col = acc_col<C>(fj) & ~3;
          if (rin && n0 + col < c_pad)
            *reinterpret_cast<uint2*>(dZ + (long long)(m0 + row) * ldz + (n0 + col - c0)) = out;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  lds_barrier();
  for (int c = threadIdx.x; c < BN; c += C::THREADS) {
    const int v = n0 + c;
    if (v < c1) {
      float t = s_db[0][c];
#pragma unroll
      for (int q = 1; q < C::WGM; ++q) t += s_db[q][c];
      dbpart[(long long)mt * ldz + (v - c0)] = t;
    }
  }
}

// dXacc (+)= dZ_c . W_c on the big core: dZ_c (frames x Kp, leading
// dimension ldz) and the transposed chunk Wt (D x Kp, leading dimension ldz),
// both zero in the columns past the chunk end; Kp = chunk width rounded up to
// a multiple of 64.
template <class C>
__global__ __launch_bounds__(C::THREADS, 1) void k_dx_big(const bf16_t* __restrict__ dZ,
                                                          const bf16_t* __restrict__ Wt, int ldz,
                                                          int M, int D, int Kp,
                                                          float* __restrict__ dXacc, int first,
                                                          bf16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
  const int ntiles = (D + C::BN - 1) / C::BN;
  // tiles in groups of 4 row tiles: the 32 work-groups an XCD runs at once
  // cover 4 x 8 tiles, 12 operand panels (2 x 16, 18 panels, with column
  // tiles fastest; 4.5% slower on the LLM head)
  int nt, mt;
  grouped_tile<4>(xcd_tile(blockIdx.x, gridDim.x), (M + C::BM - 1) / C::BM, ntiles, mt, nt);
  const int m0 = mt * C::BM, n0 = nt * C::BN;
  f32x16 acc[C::FM][C::FN];
  gemm_big1<C>(dZ, ldz, m0, M, Wt, ldz, n0, D, Kp, acc, smem);
  // Read-modify-write of the fp32 accumulator with 16-byte accesses: a lane
  // holds four rows of one column, so lanes l, l ^ 1 and then l, l ^ 2 trade
  // values until lane l holds row (l & 3) of each four-row group for the
  // columns (l & ~3) .. (l & ~3) + 3; eight lanes then cover 128 contiguous
  // bytes of a row.  One 32 x 32 fragment at a time, its loads issued before
  // its stores.  With `out` (the last product into this accumulator) the sums
  // go to out as bf16 (round to nearest even, as the separate cast would)
  // instead of back to the accumulator.
  const int lane = threadIdx.x & 63, odd = lane & 1, b1 = (lane >> 1) & 1;
#pragma unroll
  for (int fi = 0; fi < C::FM; ++fi) {
#pragma unroll
    for (int fj = 0; fj < C::FN; ++fj) {
      f32x4 val[4], old[4];
      const f32x16& a = acc[fi][fj];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float r0 = __uint_as_float(lane_xor1(__float_as_uint(odd ? a[4 * q] : a[4 * q + 1])));
        const float r2 =
            __uint_as_float(lane_xor1(__float_as_uint(odd ? a[4 * q + 2] : a[4 * q + 3])));
        // row (odd) and row (2 + odd) of columns (l & ~1), (l & ~1) + 1
        const float p0 = odd ? r0 : a[4 * q], p1 = odd ? a[4 * q + 1] : r0;
        const float c0 = odd ? r2 : a[4 * q + 2], c1 = odd ? a[4 * q + 3] : r2;
        const float t0 = __uint_as_float(lane_xor2(__float_as_uint(b1 ? p0 : c0)));
        const float t1 = __uint_as_float(lane_xor2(__float_as_uint(b1 ? p1 : c1)));
        val[q] = b1 ? f32x4{t0, t1, c0, c1} : f32x4{p0, p1, t0, t1};
      }
      const int col = n0 + (acc_col<C>(fj) & ~3);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = m0 + acc_row<C>(fi, 4 * q) + (lane & 3);
        old[q] = (!first && row < M && col < D)
                     ? *reinterpret_cast<const f32x4*>(dXacc + (long long)row * D + col)
                     : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = m0 + acc_row<C>(fi, 4 * q) + (lane & 3);
        if (row < M && col < D) {
          const f32x4 sum = old[q] + val[q];
          if (out != nullptr) {
            const uint2 h = {(uint32_t)f32_to_bf16(sum[0]) | ((uint32_t)f32_to_bf16(sum[1]) << 16),
                             (uint32_t)f32_to_bf16(sum[2]) | ((uint32_t)f32_to_bf16(sum[3]) << 16)};
            *reinterpret_cast<uint2*>(out + (long long)row * D + col) = h;
          } else {
            *reinterpret_cast<f32x4*>(dXacc + (long long)row * D + col) = sum;
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

__global__ void k_widen_bf16(const bf16_t* __restrict__ src, float* __restrict__ dst, long long n) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x)
    dst[i] = bf16_to_f32(src[i]);
}

int grid_cap(long long n, int threads, int cap = 8192) {
  long long g = (n + threads - 1) / threads;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

}  // namespace

template <typename T>
hipError_t fwd_lse_t(hipStream_t st, const void* X, const void* W, const void* b, int M, int D,
                     int V, const int* col2sel, float* Zsel, double2* part, int nspan, int span0,
                     int part_ld, int masked, int span) {
  using C = typename Pick<T>::fwd;
  const int ftiles = ceil_div(M, C::BN);
  const int grid = ftiles * nspan;
  if (grid == 0) return hipSuccess;
  const int vec = (D % C::VEC == 0) && aligned16(X) && aligned16(W);
  if (masked)
    k_fwd_lse<C, true><<<grid, C::THREADS, 0, st>>>((const T*)X, (const T*)W, (const T*)b, M, D,
                                                    V, col2sel, Zsel, part, nspan, ftiles, vec,
                                                    span0, part_ld, span);
  else
    k_fwd_lse<C, false><<<grid, C::THREADS, 0, st>>>((const T*)X, (const T*)W, (const T*)b, M,
                                                     D, V, col2sel, Zsel, part, nspan, ftiles,
                                                     vec, span0, part_ld, span);
  return hipGetLastError();
}

hipError_t launch_fwd_lse(hipStream_t st, int dtype, const void* X, const void* W, const void* b,
                          int M, int D, int V, const int* col2sel, float* Zsel, double2* part,
                          int nspan, int big, int span0, int part_ld, int masked, int span) {
  if (dtype == 0)
    return fwd_lse_t<float>(st, X, W, b, M, D, V, col2sel, Zsel, part, nspan, span0, part_ld,
                            masked, span);
  if (span0 != 0 || part_ld != nspan) return hipErrorInvalidValue;  // bf16: whole vocabulary
  if (!big)
    return fwd_lse_t<bf16_t>(st, X, W, b, M, D, V, col2sel, Zsel, part, nspan, 0, nspan,
                             masked, span);
  using C = CfgBigFwd;
  const int ftiles = ceil_div(M, C::BN);
  const int grid = ftiles * nspan;
  if (grid == 0) return hipSuccess;
  if (masked)
    k_fwd_lse_big<C, true><<<grid, C::THREADS, 0, st>>>((const bf16_t*)X, (const bf16_t*)W,
                                                        (const bf16_t*)b, M, D, V, col2sel, Zsel,
                                                        part, nspan, ftiles, span);
  else
    k_fwd_lse_big<C, false><<<grid, C::THREADS, 0, st>>>((const bf16_t*)X, (const bf16_t*)W,
                                                         (const bf16_t*)b, M, D, V, col2sel,
                                                         Zsel, part, nspan, ftiles, span);
  return hipGetLastError();
}

int lse_span(int dtype, int big, int M, int V) {
  int bm, bn;
  if (dtype == 0 || dtype == 2) {
    bm = Pick<float>::fwd::BM;
    bn = Pick<float>::fwd::BN;
  } else if (big) {
    bm = CfgBigFwd::BM;
    bn = CfgBigFwd::BN;
  } else {
    bm = Pick<bf16_t>::fwd::BM;
    bn = Pick<bf16_t>::fwd::BN;
  }
  const long long ftiles = (M + bn - 1) / bn;
  long long span = (long long)V * ftiles / 2048;  // about 2048 work-groups or more
  span = span / bm * bm;
  if (span < bm) span = bm;
  if (span > LSE_SPAN_MAX) span = LSE_SPAN_MAX;
  return (int)span;
}

hipError_t launch_lambda(hipStream_t st, const double2* part, int M, int nspan, double* lam,
                         float* lamf) {
  if (M == 0) return hipSuccess;
  k_lambda<<<ceil_div((long long)M * LAM_LANES, 256), 256, 0, st>>>(part, M, nspan, lam, lamf);
  return hipGetLastError();
}

hipError_t launch_lambda_grouped(hipStream_t st, const float* Zsel, const double* other, int K,
                                 int M, double* lam, float* lamf) {
  if (M == 0) return hipSuccess;
  k_lambda_grouped<<<ceil_div(M, 256), 256, 0, st>>>(Zsel, other, K, M, lam, lamf);
  return hipGetLastError();
}

hipError_t launch_grouped_rowscale(hipStream_t st, const double* g, const double* other,
                                   const double* lam, int M, double* gu, float* ou) {
  if (M == 0) return hipSuccess;
  k_grouped_rowscale<<<ceil_div(M, 256), 256, 0, st>>>(g, other, lam, M, gu, ou);
  return hipGetLastError();
}

hipError_t launch_scores(hipStream_t st, float* S, const double* lam, int K, int M) {
  const long long n = (long long)K * M;
  if (n == 0) return hipSuccess;
  k_scores<<<grid_cap(n, 256), 256, 0, st>>>(S, lam, K, M);
  return hipGetLastError();
}

// Logit gradient of the recompute tiles whose places are all selected
// classes, in the unselected-first order (cmap, *nu): dZ = grad (g_m
// exp(S[j][m]) - Gamma[j][m]) from S, Gamma and g alone, the formula of the
// recompute's selected classes.  The tiles are the recompute's (BM frames x
// BN places; the ones holding an unselected place return at once, the
// recompute takes them), and each tile's column sums go to
// dbpart[mtile][column], summed over its frames in order.  Per block of 64
// places: each wavefront loads the class-major S and Gamma rows of 16 places
// (unconditional loads of clamped frames, all issued before the first is
// used), the values are transposed in LDS and written out as dZ rows.
template <typename T, int BM, int BN>
__global__ __launch_bounds__(256) void k_dz_sel(const int* __restrict__ col2sel, int c0, int c1,
                                                const int* __restrict__ cmap,
                                                const int* __restrict__ nu,
                                                const double* __restrict__ g,
                                                const float* __restrict__ S,
                                                const float* __restrict__ Gam, long long ldS,
                                                int M, double grad, T* __restrict__ dZ, int ldz,
                                                float* __restrict__ dbpart, int mtiles) {
  constexpr int CB = 64;       // places per block
  constexpr int PW = CB / 4;   // places per wavefront
  constexpr int RL = BM / 64;  // frames per lane
  static_assert(BM % 64 == 0, "whole frames per lane");
  __shared__ float s_dz[BM][CB + 1];
  __shared__ double s_g[BM];
  __shared__ int s_cls[CB], s_col[CB];
  const int mt = blockIdx.x % mtiles, nt = blockIdx.x / mtiles;
  const int p0 = nt * BN;
  const int m0 = mt * BM;
  const int np = min(BN, (c1 - c0) - p0);
  // the tile's selected places: all of them, or those past the unselected
  // ones in the tile that holds both (k_recompute forms the rest)
  const int pb = max(0, *nu - p0);
  if (pb >= np) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int r = threadIdx.x; r < BM; r += 256) s_g[r] = m0 + r < M ? g[m0 + r] : 0.0;
  for (int cb = pb; cb < np; cb += CB) {
    const int nc = min(CB, np - cb);
    if (threadIdx.x < CB) {
      const bool in = (int)threadIdx.x < nc;
      const int v = cmap[p0 + cb + (in ? (int)threadIdx.x : 0)];
      const int cls = col2sel[v];
      s_cls[threadIdx.x] = in ? cls : 0;
      s_col[threadIdx.x] = v - c0;
    }
    __syncthreads();
    float sv[PW][RL], gv[PW][RL];
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int c = w * PW + i;
      const long long base = (long long)s_cls[c] * ldS;  // class 0 past nc
#pragma unroll
      for (int h = 0; h < RL; ++h) {
        // clamped frames, loaded unconditionally (masked below)
        const long long o = base + min(m0 + lane + 64 * h, M - 1);
        sv[i][h] = S[o];
        gv[i][h] = Gam[o];
      }
    }
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int c = w * PW + i;
#pragma unroll
      for (int h = 0; h < RL; ++h) {
        const int r = lane + 64 * h;
        // S <= 0 (a log-probability); rows past M give g = S = Gamma = 0
        s_dz[r][c] = (c < nc && m0 + r < M)
                         ? (float)(grad * (s_g[r] * exp_nonpos((double)sv[i][h]) - (double)gv[i][h]))
                         : 0.f;
      }
    }
    __syncthreads();
    if (lane < nc)
      for (int r = w; r < BM; r += 4)
        if (m0 + r < M) dZ[(long long)(m0 + r) * ldz + s_col[lane]] = Elem<T>::from_f32(s_dz[r][lane]);
    if ((int)threadIdx.x < nc) {
      float t = 0.f;
      for (int r = 0; r < BM; ++r) t += s_dz[r][threadIdx.x];
      dbpart[(long long)mt * ldz + s_col[threadIdx.x]] = t;
    }
    __syncthreads();
  }
}

template <typename T>
hipError_t recompute_t(hipStream_t st, const void* X, const void* W, const void* b, int M, int D,
                       int c0, int c1, const int* col2sel, const float* lamf, const double* g,
                       const float* S, const float* Gam, double grad, void* dZ, int ldz,
                       float* dbpart, const double* gu, const float* lamu, long long ldS,
                       const int* cmap, const void* Wg, const int* nu, const ReduceJob* rj) {
  using C = typename Pick<T>::rec;
  const int mtiles = ceil_div(M, C::BM);
  const int grid = mtiles * ceil_div(c1 - c0, C::BN);
  const ReduceJob job = rj != nullptr ? *rj : ReduceJob{};
  if (grid + job.nb == 0) return hipSuccess;
  const int vec = (D % C::VEC == 0) && aligned16(X) && aligned16(cmap != nullptr ? Wg : W);
  k_recompute<C><<<grid + job.nb, C::THREADS, 0, st>>>(
      (const T*)X, (const T*)W, (const T*)b, M, D, c0, c1, col2sel, lamf, g, S, Gam, grad,
      (T*)dZ, ldz, dbpart, mtiles, vec, gu, lamu, ldS, cmap, (const T*)Wg, nu, job, grid);
  if (cmap != nullptr && grid > 0)
    k_dz_sel<T, C::BM, C::BN><<<grid, 256, 0, st>>>(col2sel, c0, c1, cmap, nu, g, S, Gam, ldS, M,
                                                     grad, (T*)dZ, ldz, dbpart, mtiles);
  return hipGetLastError();
}

// Column order of the chunk [c0, c1) for the recompute: its unselected
// columns (col2sel < 0) in ascending order, then its selected ones in
// ascending order; cmap[i] is the column at place i and *nu the number of
// unselected columns.  One work-group: a count pass, then a placement
// pass over blocks of 1024 columns (wavefront ballots for the ranks).
constexpr int PERM_THREADS = 1024;

__global__ __launch_bounds__(PERM_THREADS) void k_colperm(const int* __restrict__ col2sel, int c0,
                                                          int c1, int* __restrict__ cmap,
                                                          int* __restrict__ nu) {
  constexpr int NW = PERM_THREADS / 64;
  __shared__ int s_w[NW];
  __shared__ int s_total;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int cnt = 0;
  for (int v = c0 + (int)threadIdx.x; v < c1; v += PERM_THREADS) cnt += col2sel[v] < 0;
  for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
  if (lane == 0) s_w[w] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int q = 0; q < NW; ++q) t += s_w[q];
    s_total = t;
    *nu = t;
  }
  __syncthreads();
  const int total_u = s_total;
  int done_u = 0, done = 0;  // unselected / all columns of the blocks before
  for (int b0 = c0; b0 < c1; b0 += PERM_THREADS) {
    const int v = b0 + (int)threadIdx.x;
    const bool in = v < c1;
    const bool un = in && col2sel[v] < 0;
    const unsigned long long bu = __ballot(un), bi = __ballot(in);
    const unsigned long long below = (1ull << lane) - 1ull;
    __syncthreads();  // s_w of the previous block has been read
    if (lane == 0) s_w[w] = __popcll(bu);
    __syncthreads();
    int wu = 0, bu_all = 0;
    for (int q = 0; q < NW; ++q) {
      wu += q < w ? s_w[q] : 0;
      bu_all += s_w[q];
    }
    const int ru = done_u + wu + __popcll(bu & below);         // rank among unselected
    const int ri = done + w * 64 + __popcll(bi & below);       // rank among all
    if (in) cmap[un ? ru : total_u + (ri - ru)] = v;
    done_u += bu_all;
    done += min(PERM_THREADS, c1 - b0);
  }
}

// Wg[i][:] = W[cmap[i]][:] for the places i < round_up(*nu, tile)
// (the rows any product tile reads; the remaining places are selected
// columns of tiles without a product).  One work-group per place.
template <typename T>
__global__ __launch_bounds__(256) void k_gather_rows(const T* __restrict__ W, int D,
                                                     const int* __restrict__ cmap,
                                                     const int* __restrict__ nu, int tile,
                                                     T* __restrict__ Wg) {
  const int i = blockIdx.x;
  const int lim = (*nu + tile - 1) / tile * tile;
  if (i >= lim) return;
  const T* src = W + (long long)cmap[i] * D;
  T* dst = Wg + (long long)i * D;
  for (int d = threadIdx.x; d < D; d += 256) dst[d] = src[d];
}

hipError_t launch_colperm(hipStream_t st, int dtype, const int* col2sel, int c0, int c1,
                          const void* W, int D, int* cmap, int* nu, void* Wg) {
  const int n = c1 - c0;
  if (n <= 0) return hipSuccess;
  k_colperm<<<1, PERM_THREADS, 0, st>>>(col2sel, c0, c1, cmap, nu);
  if (dtype == 0)
    k_gather_rows<float><<<n, 256, 0, st>>>((const float*)W, D, cmap, nu,
                                            Pick<float>::rec::BN, (float*)Wg);
  else
    k_gather_rows<bf16_t><<<n, 256, 0, st>>>((const bf16_t*)W, D, cmap, nu,
                                             Pick<bf16_t>::rec::BN, (bf16_t*)Wg);
  return hipGetLastError();
}

int rec_tile_cols(int dtype) {
  return dtype == 0 ? Pick<float>::rec::BN : Pick<bf16_t>::rec::BN;
}

hipError_t launch_recompute(hipStream_t st, int dtype, const void* X, const void* W, const void* b,
                            int M, int D, int c0, int c1, const int* col2sel, const float* lamf,
                            const double* g, const float* S, const float* Gam, double grad,
                            void* dZ, int ldz, float* dbpart, int big, const double* gu,
                            const float* lamu, long long ldS, const int* cmap, const void* Wg,
                            const int* nu, const ReduceJob* rj) {
  if (ldS <= 0) ldS = M;
  if ((cmap == nullptr) != (nu == nullptr)) return hipErrorInvalidValue;
  if (dtype == 0)
    return recompute_t<float>(st, X, W, b, M, D, c0, c1, col2sel, lamf, g, S, Gam, grad, dZ, ldz,
                              dbpart, gu, lamu, ldS, cmap, Wg, nu, rj);
  if (!big)
    return recompute_t<bf16_t>(st, X, W, b, M, D, c0, c1, col2sel, lamf, g, S, Gam, grad, dZ,
                               ldz, dbpart, gu, lamu, ldS, cmap, Wg, nu, rj);
  if (cmap != nullptr) return hipErrorInvalidValue;  // the 256 x 256 core walks columns in order
  if (rj != nullptr && rj->nb > 0) return hipErrorInvalidValue;  // no appended reduction here
  using C = CfgBigRec;
  const int mtiles = ceil_div(M, C::BM);
  const int grid = mtiles * ceil_div(c1 - c0, C::BN);
  if (grid == 0) return hipSuccess;
  k_recompute_big<C><<<grid, C::THREADS, 0, st>>>((const bf16_t*)X, (const bf16_t*)W,
                                                   (const bf16_t*)b, M, D, c0, c1, col2sel, lamf,
                                                   g, S, Gam, grad, (bf16_t*)dZ, ldz, dbpart,
                                                   mtiles, gu, lamu, ldS);
  return hipGetLastError();
}

hipError_t launch_dx(hipStream_t st, int dtype, const void* dZ, int ldz, const void* W, int M,
                     int D, int c0, int c1, float* dXacc, int first, void* wt, int big,
                     int stage_wt, void* out_bf16) {
  if (out_bf16 != nullptr && !(dtype != 0 && big && aligned8(out_bf16)))
    return hipErrorInvalidValue;  // only the 256 x 256 core writes bf16 itself
  const int Cc = c1 - c0;
  if (dtype == 0) {
    using C = Pick<float>::dx;
    const int mtiles = ceil_div(M, C::BM);
    const int grid = mtiles * ceil_div(D, C::BN);
    if (grid == 0) return hipSuccess;
    const float* Wc = (const float*)W + (long long)c0 * D;
    const int av = (ldz % 4 == 0) && aligned16(dZ);
    const int bv = (D % 4 == 0) && aligned16(Wc);
    k_dx<C, false><<<grid, C::THREADS, 0, st>>>((const float*)dZ, ldz, Wc, D, M, D, Cc, dXacc,
                                                first, mtiles, av, bv);
  } else {
    // bf16: stage W_c^T (D x Cc, leading dimension ldz) so both operands are
    // K-contiguous; for the big core its rows up to the next multiple of 64
    // are zero.
    const bf16_t* Wc = (const bf16_t*)W + (long long)c0 * D;
    const int Kp = big ? (Cc + 63) & ~63 : Cc;
    // (stage_wt == 0: staged by an earlier call on the same columns)
    dim3 tg(ceil_div(D, 64), ceil_div(Kp, 64));
    if (stage_wt) {
      if (D % 8 == 0 && ldz % 8 == 0 && aligned16(Wc) && aligned16(wt))
        k_transpose16<bf16_t><<<tg, 256, 0, st>>>(Wc, Cc, Kp, D, (bf16_t*)wt, ldz);
      else
        k_transpose<bf16_t><<<tg, 256, 0, st>>>(Wc, Cc, Kp, D, (bf16_t*)wt, ldz);
    }
    if (big) {
      using C = CfgBigDx;
      const int grid = ceil_div(M, C::BM) * ceil_div(D, C::BN);
      if (grid == 0) return hipSuccess;
      k_dx_big<C><<<grid, C::THREADS, 0, st>>>((const bf16_t*)dZ, (const bf16_t*)wt, ldz, M, D,
                                                Kp, dXacc, first, (bf16_t*)out_bf16);
      return hipGetLastError();
    }
    using C = Pick<bf16_t>::dx;
    const int mtiles = ceil_div(M, C::BM);
    const int grid = mtiles * ceil_div(D, C::BN);
    if (grid == 0) return hipSuccess;
    const int av = (ldz % 8 == 0) && aligned16(dZ);
    const int bv = (ldz % 8 == 0) && aligned16(wt);
    k_dx<C, true><<<grid, C::THREADS, 0, st>>>((const bf16_t*)dZ, ldz, (const bf16_t*)wt, ldz, M,
                                               D, Cc, dXacc, first, mtiles, av, bv);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t dw_t(hipStream_t st, const void* dZ, int ldz, const void* X, int M, int D, int c0,
                int c1, float* part, int splitk) {
  using C = typename Pick<T>::dw;
  const int Cc = c1 - c0;
  const int itiles = ceil_div(Cc, C::BM), ntiles = ceil_div(D, C::BN);
  const int grid = itiles * ntiles * splitk;
  if (grid == 0) return hipSuccess;
  const int kchunk = ceil_div(ceil_div(M, splitk), 64) * 64;
  const int av = (ldz % C::VEC == 0) && aligned16(dZ);
  const int bv = (D % C::VEC == 0) && aligned16(X);
  k_dw<C><<<grid, C::THREADS, 0, st>>>((const T*)dZ, ldz, (const T*)X, M, D, Cc, part, itiles,
                                        ntiles, kchunk, av, bv);
  return hipGetLastError();
}

hipError_t launch_dw(hipStream_t st, int dtype, const void* dZ, int ldz, const void* X, int M,
                     int D, int c0, int c1, float* part, int splitk) {
  return dtype == 0 ? dw_t<float>(st, dZ, ldz, X, M, D, c0, c1, part, splitk)
                    : dw_t<bf16_t>(st, dZ, ldz, X, M, D, c0, c1, part, splitk);
}

int rec_tile_rows(int dtype, int big) {
  if (dtype == 0) return Pick<float>::rec::BM;
  return big ? CfgBigRec::BM : Pick<bf16_t>::rec::BM;
}

int use_big_fwd(int dtype, int D, const void* X, const void* W) {
  return dtype != 0 && D > 0 && D % 64 == 0 && aligned16(X) && aligned16(W);
}

int use_big_core(int dtype, int D, int chunk, const void* X, const void* W) {
  return use_big_fwd(dtype, D, X, W) && chunk % 64 == 0;
}

int dw_tiles(int dtype, int C, int D) {
  if (dtype == 0)
    return ceil_div(C, Pick<float>::dw::BM) * ceil_div(D, Pick<float>::dw::BN);
  return ceil_div(C, Pick<bf16_t>::dw::BM) * ceil_div(D, Pick<bf16_t>::dw::BN);
}

ReduceJob make_reduce_job(int dtype, const float* part, int splitk, int rows, int D, void* dW,
                          long long row_base, const float* dbpart, int mtiles, int cols, int ld,
                          void* db, long long col_base, int max_wg) {
  ReduceJob j;
  j.part = part;
  j.splitk = splitk;
  j.rows = dW ? rows : 0;
  j.D = D;
  j.dW = dW;
  j.row_base = row_base;
  j.dbpart = dbpart;
  j.mtiles = mtiles;
  j.cols = cols;
  j.ld = ld;
  j.db = db;
  j.col_base = col_base;
  j.out_bf16 = dtype != 0;
  const long long n = (long long)j.rows * D;
  // 16-byte partial loads when the rows' output starts on a four-element
  // boundary (the partials themselves are 16-byte aligned when n is a
  // multiple of four)
  const size_t esz = dtype == 0 ? 4 : 2;
  j.vec4 = n % 4 == 0 && ((uintptr_t)dW + (uintptr_t)(row_base * D) * esz) % (4 * esz) == 0;
  const int nb_dw = n ? grid_cap(j.vec4 ? n / 4 : n, 256, max_wg) : 0;
  j.nb_db = (db && cols > 0) ? ceil_div(cols, DB_COLS) : 0;
  j.nb = nb_dw + j.nb_db;
  return j;
}

hipError_t launch_grad_reduce(hipStream_t st, const ReduceJob& rj) {
  if (rj.nb == 0) return hipSuccess;
  if (rj.out_bf16)
    k_grad_reduce<bf16_t><<<rj.nb, 256, 0, st>>>(rj);
  else
    k_grad_reduce<float><<<rj.nb, 256, 0, st>>>(rj);
  return hipGetLastError();
}

hipError_t launch_widen(hipStream_t st, const void* src, float* dst, long long n) {
  if (n == 0) return hipSuccess;
  k_widen_bf16<<<grid_cap(n, 256), 256, 0, st>>>((const bf16_t*)src, dst, n);
  return hipGetLastError();
}

hipError_t launch_cast_out(hipStream_t st, int dtype, const float* src, void* dst, long long n) {
  if (n == 0 || dtype == 0) return hipSuccess;
  k_cast_bf16<<<grid_cap(n, 256), 256, 0, st>>>(src, (bf16_t*)dst, n);
  return hipGetLastError();
}

}  // namespace pcx

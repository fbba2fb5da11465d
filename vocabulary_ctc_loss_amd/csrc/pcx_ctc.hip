// CTC alignment dynamic program over the K selected classes, in FP64.
//
// "Pruned CTC for Memory-Efficient Large-Vocabulary ASR Training":
//  * Sec. 3.1, Eq. 2: the loss of utterance n is -log of the total
//    probability of the frame-level alignments that collapse to y_n; frames
//    are conditionally independent given the head inputs.
//  * Sec. 3.2: every valid alignment only visits blank and the labels of y_n,
//    so the recursion needs only the columns S[:, U] (Eq. 3); occupancies
//    gamma_v(m) are the posterior label probabilities per frame
//    (Proposition 1).
//  * App. B.1 / App. C.2: scores enter as FP32, the alignment log-likelihood
//    is accumulated in FP64; nonfinite per-utterance losses are replaced by
//    zero, unalignable utterances (|y| + r > T) contribute nothing.
//
// The recursion is the textbook one on the blank-interleaved label sequence
// (blank, y1, blank, ..., yL, blank): state s takes mass from s and s-1, and
// from s-2 when s is a label different from the label two states back.  One
// work-group owns one utterance; each thread owns up to SPT states and the
// previous frame's values live in LDS (double-buffered, one barrier per
// frame).  Emission scores for the next 8 frames (4 with two states per
// thread, 2 with four) are prefetched into registers while the current ones
// are processed.
#include <math.h>

#include "pcx_common.h"

namespace pcx {

namespace {

constexpr int PF = 8;  // frames per emission prefetch block

// The recursion is a serial chain of log-add-exps, so its FP64 exp and log
// are written for latency: the exp polynomial is evaluated by Estrin's
// scheme (tree of depth 4 instead of a 13-step Horner chain), and the log is
// specialised to arguments in [1, 4).

// exp(x), x <= 0: Cody-Waite reduction by ln2 (32-bit head, tail), degree-13
// Taylor polynomial of e^r, |r| <= ln2 / 2, scale by 2^n.
__device__ __forceinline__ double exp_nonpos_lat(double x) {
  x = fmax(x, -746.0);
  const double n = rint(x * 0x1.71547652b82fep+0);
  double r = fma(-n, 0x1.62e42ff000000p-1, x);
  r = fma(-n, -0x1.718432a1b0e26p-35, r);
  const double r2 = r * r, r4 = r2 * r2, r8 = r4 * r4;
  const double p01 = r + 1.0;
  const double p23 = fma(r, 0x1.5555555555555p-3, 0.5);                    // 1/3!, 1/2!
  const double p45 = fma(r, 0x1.1111111111111p-7, 0x1.5555555555555p-5);   // 1/5!, 1/4!
  const double p67 = fma(r, 0x1.a01a01a01a01ap-13, 0x1.6c16c16c16c17p-10); // 1/7!, 1/6!
  const double p89 = fma(r, 0x1.71de3a556c734p-19, 0x1.a01a01a01a01ap-16); // 1/9!, 1/8!
  const double pab = fma(r, 0x1.ae64567f544e4p-26, 0x1.27e4fb7789f5cp-22); // 1/11!, 1/10!
  const double pcd = fma(r, 0x1.6124613a86d09p-33, 0x1.1eed8eff8d898p-29); // 1/13!, 1/12!
  const double q0 = fma(r2, p23, p01), q1 = fma(r2, p67, p45), q2 = fma(r2, pab, p89);
  const double s0 = fma(r4, q1, q0), s1 = fma(r4, pcd, q2);
  return ldexp(fma(r8, s1, s0), (int)n);
}

// log(x), 1 <= x < 4: x = 2^e f with f in [sqrt(1/2), sqrt(2)), and
// log f = 2 atanh(u), u = (f - 1) / (f + 1), |u| <= 0.172, by its odd series
// through u^23 (truncation < 1e-18).
__device__ __forceinline__ double log_1to4(double x) {
  int e = 0;
  double f = frexp(x, &e);
  if (f < 0.70710678118654752440) {
    f *= 2.0;
    e -= 1;
  }
  // u = (f - 1) / (f + 1): hardware reciprocal refined by two Newton steps
  const double den = f + 1.0;
  double rc = __builtin_amdgcn_rcp(den);
  rc = fma(rc, fma(-den, rc, 1.0), rc);
  rc = fma(rc, fma(-den, rc, 1.0), rc);
  const double u = (f - 1.0) * rc;
  const double u2 = u * u, u4 = u2 * u2, u8 = u4 * u4;
  const double a = fma(u2, 1.0 / 5, 1.0 / 3), b = fma(u2, 1.0 / 9, 1.0 / 7);
  const double c = fma(u2, 1.0 / 13, 1.0 / 11), d = fma(u2, 1.0 / 17, 1.0 / 15);
  const double g = fma(u2, 1.0 / 21, 1.0 / 19);
  const double ab = fma(u4, b, a), cd = fma(u4, d, c), gh = fma(u4, 1.0 / 23, g);
  const double p = fma(u8, fma(u8, gh, cd), ab);
  const double lf = fma(2.0 * u * u2, p, 2.0 * u);
  return fma((double)e, 0x1.62e42fefa39efp-1, lf);  // + e ln2
}

// log(e^a + e^b + e^c) = m + log(1 + e^(x-m) + e^(y-m)), m the largest and
// x, y the other two (the max term contributes exactly 1).
__device__ __forceinline__ double lse3(double a, double b, double c) {
  const bool am = a >= b && a >= c;
  const bool bm = !am && b >= c;
  const double m = am ? a : (bm ? b : c);
  const double x = am ? b : a;
  const double y = (am || bm) ? c : b;
  if (m == -INFINITY) return -INFINITY;
  return m + log_1to4(1.0 + exp_nonpos_lat(x - m) + exp_nonpos_lat(y - m));
}

__device__ __forceinline__ double lse2(double a, double b) {
  const double m = fmax(a, b), x = fmin(a, b);
  if (m == -INFINITY) return -INFINITY;
  return m + log_1to4(1.0 + exp_nonpos_lat(x - m));
}

// What a recursion computes over the lattice of an utterance:
//   DP_SUM     the forward (backward) sums over every CTC transition: the
//              unpruned alpha (beta) of the loss, as scaled probabilities;
//   DP_PRUNED  the same over the arcs a finite alignment beam keeps (bit
//              masks from k_beam_mask, one byte per lattice node);
//   DP_MAX     best prefix scores vf (emission included) and best suffix
//              scores vb (emission of the node excluded) in FP64 max-plus
//              (log domain), and the best complete alignment's score per
//              utterance.
enum : int { DP_SUM = 0, DP_PRUNED = 1, DP_MAX = 2 };

// Scaled probabilities.  The sums of the recursions are kept in the
// probability domain as an FP64 mantissa and a separate int32 exponent,
// x = m 2^e, so that they neither underflow (an alignment sum of 1,100
// frames can lie far below 2^-1074) nor need an exp and a log per
// transition: a step is an exponent maximum, three exact rescalings, two
// additions and a multiplication by the emission, then one renormalisation.
// Rounding: one relative error of at most about 2^-52 per addition and
// multiplication, which in the log domain is an absolute error of the same
// size (the log-domain form also rounds its exp and log).  Zero is m = 0
// with the exponent ZERO_E, far below any reachable exponent, so that a
// rescaling by it gives exactly 0 without overflowing.
constexpr int ZERO_E = -(1 << 29);

struct Sc {
  double m;
  int e;
};

__device__ __forceinline__ Sc sc_make(double v, int e) {
  if (v == 0.0) return {0.0, ZERO_E};
  int ex = 0;
  const double mant = frexp(v, &ex);
  return {mant, e + ex};
}

// a + b + c of scaled values, exponent-aligned to the largest.
__device__ __forceinline__ double sc_sum3(const Sc& a, const Sc& b, const Sc& c, int& emax) {
  emax = max(a.e, max(b.e, c.e));
  return ldexp(a.m, a.e - emax) + ldexp(b.m, b.e - emax) + ldexp(c.m, c.e - emax);
}

// exp(S) of an fp32 log-probability S as a scaled value m 2^n, to fp32
// precision (exp_split).
__device__ __forceinline__ Sc sc_exp(float s) {
  int n;
  const float m = exp_split(s, n);
  return {(double)m, n};
}

// Stored form of a scaled value (the occupancy pass reads it): the mantissa
// rounded to fp32 beside its exponent, one 8-byte word per lattice node.
struct Sc32 {
  float m;
  int e;
};

// Buffers of the recursions, 8 bytes per lattice node.  Sum modes: am the
// forward values (emission of the node included), bm the backward values
// without the node's emission, both as Sc32, so that alpha * beta / P is the
// posterior of the node; utt_pm / utt_pe the total P.  DP_MAX: am the best
// prefix scores vf, bm the best suffix scores vb (FP64, log domain), best the
// best complete scores.
struct DpBufs {
  double* am;
  double* bm;
  double* utt_loss;
  double* utt_logp;
  double* utt_pm;
  int* utt_pe;
  int* utt_status;
  double* best;
};

// Arc bits of a lattice node (t, s): bits 0-2 the arcs into it from s
// (stay), s - 1 (advance) and s - 2 (skip); bits 3-5 the arcs out of it to
// s, s + 1 and s + 2.  At t = 0 bit 0 is the initial arc, at t = T - 1 bit 3
// the final arc.
constexpr int ARC_IN_STAY = 1, ARC_IN_ADV = 2, ARC_IN_SKIP = 4;
constexpr int ARC_OUT_STAY = 8, ARC_OUT_ADV = 16, ARC_OUT_SKIP = 32;

// Emission (and arc-mask byte) of a state at frame t for the first block of
// prefetch registers: a clamped, in-bounds frame and state are loaded
// unconditionally and the value is masked afterwards (a load under a
// per-lane condition is waited for on the spot, which had serialized these
// loads).  States past Sn read class 0's row of S.
template <bool MASK>
__device__ __forceinline__ void dp_fetch(const float* __restrict__ S, long long ebase,
                                         const uint8_t* __restrict__ mk, int t, int T, int s,
                                         int Sn, float& e, int& m) {
  const bool in = s < Sn && t >= 0 && t < T;
  const int tc = min(max(t, 0), T - 1);
  const float ev = S[ebase + tc];
  e = in ? ev : 0.f;
  if (MASK) {
    const int mv = mk[(long long)tc * Sn + min(s, Sn - 1)];
    m = in ? mv : 0;
  } else {
    m = 0;
  }
}

// The same for the prefetch inside the frame loop, as conditional loads:
// there they are issued a block of frames ahead and waited for only at the
// block's end (with unconditional loads the compiler placed their waits
// inside the frame steps, measured 15% slower).
template <bool MASK>
__device__ __forceinline__ void dp_fetch_next(const float* __restrict__ S, long long ebase,
                                              const uint8_t* __restrict__ mk, int t, int T, int s,
                                              int Sn, float& e, int& m) {
  const bool in = s < Sn && t >= 0 && t < T;
  e = in ? S[ebase + t] : 0.f;
  m = (MASK && in) ? mk[(long long)t * Sn + s] : 0;
}

__device__ __forceinline__ double max3(double a, double b, double c) {
  return fmax(a, fmax(b, c));
}

// Forward recursion of utterance n; alpha[t][s] (including the emission at
// t) is stored for the backward pass (not when alpha is NULL: the loss
// alone).  DP_MAX stores vf in alpha and the best complete score in best[n].
template <int SPT, int MODE>
__device__ __forceinline__ void alpha_utt(
    int n, double* sh, const float* __restrict__ S, int M, const int* __restrict__ row_off,
    const int* __restrict__ tgt_off, const int* __restrict__ tgt_rel,
    const uint8_t* __restrict__ flags, const long long* __restrict__ dp_off,
    const uint8_t* __restrict__ mask, double* __restrict__ alpha, double* __restrict__ utt_loss,
    double* __restrict__ utt_logp, int* __restrict__ utt_status, double* __restrict__ best) {
  // frames per prefetch block: fewer with more states per thread, so the
  // prefetch registers fit beside the states'
  constexpr int PFS = SPT >= 4 ? 2 : (SPT == 2 ? 4 : PF);
  const int row0 = row_off[n], T = row_off[n + 1] - row0;
  const int y0 = tgt_off[n], L = tgt_off[n + 1] - y0, Sn = 2 * L + 1;
  if (!flags[n]) {
    if (threadIdx.x == 0) {
      if (MODE == DP_MAX) {
        best[n] = -INFINITY;
      } else {
        utt_loss[n] = 0.0;
        utt_logp[n] = -INFINITY;
        utt_status[n] = UTT_UNALIGNABLE;
      }
    }
    return;
  }
  const int cap = SPT * blockDim.x;
  double* buf0 = sh;
  double* buf1 = sh + cap;
  double* out = alpha != nullptr ? alpha + dp_off[n] : nullptr;
  const uint8_t* mk = MODE == DP_PRUNED ? mask + dp_off[n] : nullptr;
  int sidx[SPT];
  long long ebase[SPT];
  bool skip[SPT];
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int s = threadIdx.x + j * blockDim.x;
    sidx[j] = s;
    int cls = 0;
    bool sk = false;
    if (s < Sn && (s & 1)) {
      cls = tgt_rel[y0 + (s >> 1)];
      sk = s >= 3 && cls != tgt_rel[y0 + (s >> 1) - 1];
    }
    skip[j] = sk;
    ebase[j] = (long long)cls * M + row0;
  }
  float ecur[SPT][PFS], enxt[SPT][PFS];
  int mcur[SPT][PFS], mnxt[SPT][PFS];
#pragma unroll
  for (int j = 0; j < SPT; ++j)
#pragma unroll
    for (int u = 0; u < PFS; ++u) {
      dp_fetch<MODE == DP_PRUNED>(S, ebase[j], mk, u, T, sidx[j], Sn, ecur[j][u], mcur[j][u]);
    }
  // frame 0: only the first blank and the first label can start (pruned:
  // if their initial arcs are kept).
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int s = sidx[j];
    if (s < Sn) {
      const bool start = s <= 1 && (MODE != DP_PRUNED || (mcur[j][0] & ARC_IN_STAY));
      const double a = start ? (double)ecur[j][0] : -INFINITY;
      buf0[s] = a;
      if (out) out[s] = a;
    }
  }
  lds_barrier();
  for (int tb = 0; tb < T; tb += PFS) {
    if (tb + PFS < T) {
#pragma unroll
      for (int j = 0; j < SPT; ++j)
#pragma unroll
        for (int u = 0; u < PFS; ++u) {
          const int t = tb + PFS + u;
          dp_fetch_next<MODE == DP_PRUNED>(S, ebase[j], mk, t, T, sidx[j], Sn, enxt[j][u], mnxt[j][u]);
        }
    }
#pragma unroll
    for (int u = 0; u < PFS; ++u) {
      const int t = tb + u;
      if (t >= T) break;
      if (t == 0) continue;
      const double* prev = (t & 1) ? buf0 : buf1;
      double* cur = (t & 1) ? buf1 : buf0;
#pragma unroll
      for (int j = 0; j < SPT; ++j) {
        const int s = sidx[j];
        if (s < Sn) {
          double a0 = prev[s];
          double a1 = s >= 1 ? prev[s - 1] : -INFINITY;
          double a2 = skip[j] ? prev[s - 2] : -INFINITY;
          if (MODE == DP_PRUNED) {
            const int m = mcur[j][u];
            a0 = (m & ARC_IN_STAY) ? a0 : -INFINITY;
            a1 = (m & ARC_IN_ADV) ? a1 : -INFINITY;
            a2 = (m & ARC_IN_SKIP) ? a2 : -INFINITY;
          }
          const double v =
              (MODE == DP_MAX ? max3(a0, a1, a2) : lse3(a0, a1, a2)) + (double)ecur[j][u];
          cur[s] = v;
          if (out) out[(long long)t * Sn + s] = v;
        }
      }
      lds_barrier();
    }
#pragma unroll
    for (int j = 0; j < SPT; ++j)
#pragma unroll
      for (int u = 0; u < PFS; ++u) {
        ecur[j][u] = enxt[j][u];
        mcur[j][u] = mnxt[j][u];
      }
  }
  if (threadIdx.x == 0) {
    const double* last = ((T - 1) & 1) ? buf1 : buf0;
    double e1 = last[Sn - 1], e2 = Sn > 1 ? last[Sn - 2] : -INFINITY;
    if (MODE == DP_MAX) {
      best[n] = fmax(e1, e2);
      return;
    }
    if (MODE == DP_PRUNED) {  // final arcs
      const uint8_t* lm = mk + (long long)(T - 1) * Sn;
      if (!(lm[Sn - 1] & ARC_OUT_STAY)) e1 = -INFINITY;
      if (Sn > 1 && !(lm[Sn - 2] & ARC_OUT_STAY)) e2 = -INFINITY;
    }
    const double logP = Sn > 1 ? lse2(e1, e2) : e1;
    utt_logp[n] = logP;
    if (isfinite(logP)) {
      utt_loss[n] = -logP;
      utt_status[n] = UTT_OK;
    } else {
      utt_loss[n] = 0.0;
      utt_status[n] = UTT_NONFINITE;
    }
  }
}

// Backward recursion of utterance n; beta[t][s] includes the emission at
// t.  Run for every structurally alignable utterance (an utterance whose
// loss turns out nonfinite gets no gradient: the occupancy pass skips it).
// DP_MAX stores vb, the best suffix score after the node (its own emission
// excluded), while the recursion carries vb + emission.
template <int SPT, int MODE>
__device__ __forceinline__ void beta_utt(
    int n, double* sh, const float* __restrict__ S, int M, const int* __restrict__ row_off,
    const int* __restrict__ tgt_off, const int* __restrict__ tgt_rel,
    const uint8_t* __restrict__ flags, const long long* __restrict__ dp_off,
    const uint8_t* __restrict__ mask, double* __restrict__ beta) {
  // frames per prefetch block: fewer with more states per thread, so the
  // prefetch registers fit beside the states'
  constexpr int PFS = SPT >= 4 ? 2 : (SPT == 2 ? 4 : PF);
  if (!flags[n]) return;
  const int row0 = row_off[n], T = row_off[n + 1] - row0;
  const int y0 = tgt_off[n], L = tgt_off[n + 1] - y0, Sn = 2 * L + 1;
  const int cap = SPT * blockDim.x;
  double* buf0 = sh;
  double* buf1 = sh + cap;
  double* out = beta + dp_off[n];
  const uint8_t* mk = MODE == DP_PRUNED ? mask + dp_off[n] : nullptr;
  int sidx[SPT];
  long long ebase[SPT];
  bool skip[SPT];
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int s = threadIdx.x + j * blockDim.x;
    sidx[j] = s;
    int cls = 0;
    bool sk = false;
    if (s < Sn && (s & 1)) {
      cls = tgt_rel[y0 + (s >> 1)];
      sk = s + 2 < Sn && cls != tgt_rel[y0 + (s >> 1) + 1];
    }
    skip[j] = sk;
    ebase[j] = (long long)cls * M + row0;
  }
  // Frames are visited downwards; block b covers frames T-1-b*PFS-u, u < PFS.
  float ecur[SPT][PFS], enxt[SPT][PFS];
  int mcur[SPT][PFS], mnxt[SPT][PFS];
#pragma unroll
  for (int j = 0; j < SPT; ++j)
#pragma unroll
    for (int u = 0; u < PFS; ++u) {
      const int t = T - 1 - u;
      dp_fetch<MODE == DP_PRUNED>(S, ebase[j], mk, t, T, sidx[j], Sn, ecur[j][u], mcur[j][u]);
    }
  const int tl = T - 1;
  double* lastbuf = (tl & 1) ? buf1 : buf0;
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int s = sidx[j];
    if (s < Sn) {
      const bool fin = s >= Sn - 2 && (MODE != DP_PRUNED || (mcur[j][0] & ARC_OUT_STAY));
      const double b = fin ? (double)ecur[j][0] : -INFINITY;  // DP_MAX: 0 + emission
      lastbuf[s] = b;
      out[(long long)tl * Sn + s] = MODE == DP_MAX ? (fin ? 0.0 : -INFINITY) : b;
    }
  }
  lds_barrier();
  for (int tb = 0; tb < T; tb += PFS) {
    if (tb + PFS < T) {
#pragma unroll
      for (int j = 0; j < SPT; ++j)
#pragma unroll
        for (int u = 0; u < PFS; ++u) {
          const int t = T - 1 - (tb + PFS + u);
          dp_fetch_next<MODE == DP_PRUNED>(S, ebase[j], mk, t, T, sidx[j], Sn, enxt[j][u], mnxt[j][u]);
        }
    }
#pragma unroll
    for (int u = 0; u < PFS; ++u) {
      const int t = T - 1 - (tb + u);
      if (t < 0) break;
      if (t == T - 1) continue;
      const double* nxt = ((t + 1) & 1) ? buf1 : buf0;
      double* cur = (t & 1) ? buf1 : buf0;
#pragma unroll
      for (int j = 0; j < SPT; ++j) {
        const int s = sidx[j];
        if (s < Sn) {
          double b0 = nxt[s];
          double b1 = s + 1 < Sn ? nxt[s + 1] : -INFINITY;
          double b2 = skip[j] ? nxt[s + 2] : -INFINITY;
          if (MODE == DP_PRUNED) {
            const int m = mcur[j][u];
            b0 = (m & ARC_OUT_STAY) ? b0 : -INFINITY;
            b1 = (m & ARC_OUT_ADV) ? b1 : -INFINITY;
            b2 = (m & ARC_OUT_SKIP) ? b2 : -INFINITY;
          }
          if (MODE == DP_MAX) {
            const double m = max3(b0, b1, b2);
            cur[s] = m + (double)ecur[j][u];
            out[(long long)t * Sn + s] = m;
          } else {
            const double v = lse3(b0, b1, b2) + (double)ecur[j][u];
            cur[s] = v;
            out[(long long)t * Sn + s] = v;
          }
        }
      }
      lds_barrier();
    }
#pragma unroll
    for (int j = 0; j < SPT; ++j)
#pragma unroll
      for (int u = 0; u < PFS; ++u) {
        ecur[j][u] = enxt[j][u];
        mcur[j][u] = mnxt[j][u];
      }
  }
}

// Forward sums of utterance n as scaled probabilities; the values (emission
// included) are stored for the occupancy pass unless am is NULL (the loss
// alone).  PRUNED: transitions masked by the kept-arc bits.
template <int SPT, bool PRUNED>
__device__ __forceinline__ void alpha_sum(
    int n, char* sh, const float* __restrict__ S, int M, const int* __restrict__ row_off,
    const int* __restrict__ tgt_off, const int* __restrict__ tgt_rel,
    const uint8_t* __restrict__ flags, const long long* __restrict__ dp_off,
    const uint8_t* __restrict__ mask, const DpBufs& b) {
  // frames per prefetch block: fewer with more states per thread, so the
  // prefetch registers fit beside the states'
  constexpr int PFS = SPT >= 4 ? 2 : (SPT == 2 ? 4 : PF);
  const int row0 = row_off[n], T = row_off[n + 1] - row0;
  const int y0 = tgt_off[n], L = tgt_off[n + 1] - y0, Sn = 2 * L + 1;
  if (!flags[n]) {
    if (threadIdx.x == 0) {
      b.utt_loss[n] = 0.0;
      b.utt_logp[n] = -INFINITY;
      b.utt_pm[n] = 0.0;
      b.utt_pe[n] = ZERO_E;
      b.utt_status[n] = UTT_UNALIGNABLE;
    }
    return;
  }
  const int cap = SPT * blockDim.x;
  double* mb0 = reinterpret_cast<double*>(sh);
  double* mb1 = mb0 + cap;
  int* eb0 = reinterpret_cast<int*>(mb1 + cap);
  int* eb1 = eb0 + cap;
  const long long o0 = dp_off[n];
  Sc32* om = b.am != nullptr ? reinterpret_cast<Sc32*>(b.am) + o0 : nullptr;
  const uint8_t* mk = PRUNED ? mask + o0 : nullptr;
  int sidx[SPT];
  long long ebase[SPT];
  bool skip[SPT];
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int s = threadIdx.x + j * blockDim.x;
    sidx[j] = s;
    int cls = 0;
    bool sk = false;
    if (s < Sn && (s & 1)) {
      cls = tgt_rel[y0 + (s >> 1)];
      sk = s >= 3 && cls != tgt_rel[y0 + (s >> 1) - 1];
    }
    skip[j] = sk;
    ebase[j] = (long long)cls * M + row0;
  }
  float ecur[SPT][PFS], enxt[SPT][PFS];
  int mcur[SPT][PFS], mnxt[SPT][PFS];
#pragma unroll
  for (int j = 0; j < SPT; ++j)
#pragma unroll
    for (int u = 0; u < PFS; ++u) {
      dp_fetch<PRUNED>(S, ebase[j], mk, u, T, sidx[j], Sn, ecur[j][u], mcur[j][u]);
    }
  // frame 0: only the first blank and the first label can start (pruned:
  // if their initial arcs are kept).
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int s = sidx[j];
    if (s < Sn) {
      const bool start = s <= 1 && (!PRUNED || (mcur[j][0] & ARC_IN_STAY));
      Sc a{0.0, ZERO_E};
      if (start) {
        const Sc p = sc_exp(ecur[j][0]);
        a = sc_make(p.m, p.e);
      }
      mb0[s] = a.m;
      eb0[s] = a.e;
      if (om) om[s] = Sc32{(float)a.m, a.e};
    }
  }
  lds_barrier();
  for (int tb = 0; tb < T; tb += PFS) {
    if (tb + PFS < T) {
#pragma unroll
      for (int j = 0; j < SPT; ++j)
#pragma unroll
        for (int u = 0; u < PFS; ++u) {
          const int t = tb + PFS + u;
          dp_fetch_next<PRUNED>(S, ebase[j], mk, t, T, sidx[j], Sn, enxt[j][u], mnxt[j][u]);
        }
    }
#pragma unroll
    for (int u = 0; u < PFS; ++u) {
      const int t = tb + u;
      if (t >= T) break;
      if (t == 0) continue;
      const double* pm = (t & 1) ? mb0 : mb1;
      const int* pe = (t & 1) ? eb0 : eb1;
      double* cm = (t & 1) ? mb1 : mb0;
      int* ce = (t & 1) ? eb1 : eb0;
#pragma unroll
      for (int j = 0; j < SPT; ++j) {
        const int s = sidx[j];
        if (s < Sn) {
          // the emission is ready before the chain needs it
          const Sc p = sc_exp(ecur[j][u]);
          const int m = mcur[j][u];
          const bool k0 = !PRUNED || (m & ARC_IN_STAY);
          const bool k1 = s >= 1 && (!PRUNED || (m & ARC_IN_ADV));
          const bool k2 = skip[j] && (!PRUNED || (m & ARC_IN_SKIP));
          const Sc a0 = k0 ? Sc{pm[s], pe[s]} : Sc{0.0, ZERO_E};
          const Sc a1 = k1 ? Sc{pm[s - 1], pe[s - 1]} : Sc{0.0, ZERO_E};
          const Sc a2 = k2 ? Sc{pm[s - 2], pe[s - 2]} : Sc{0.0, ZERO_E};
          int emax;
          const double sum = sc_sum3(a0, a1, a2, emax);
          const Sc v = sc_make(sum * p.m, emax + p.e);
          cm[s] = v.m;
          ce[s] = v.e;
          if (om) om[(long long)t * Sn + s] = Sc32{(float)v.m, v.e};
        }
      }
      lds_barrier();
    }
#pragma unroll
    for (int j = 0; j < SPT; ++j)
#pragma unroll
      for (int u = 0; u < PFS; ++u) {
        ecur[j][u] = enxt[j][u];
        mcur[j][u] = mnxt[j][u];
      }
  }
  if (threadIdx.x == 0) {
    const int l = (T - 1) & 1;
    const double* lm = l ? mb1 : mb0;
    const int* le = l ? eb1 : eb0;
    Sc f1{lm[Sn - 1], le[Sn - 1]};
    Sc f2 = Sn > 1 ? Sc{lm[Sn - 2], le[Sn - 2]} : Sc{0.0, ZERO_E};
    if (PRUNED) {  // final arcs
      const uint8_t* fm = mk + (long long)(T - 1) * Sn;
      if (!(fm[Sn - 1] & ARC_OUT_STAY)) f1 = Sc{0.0, ZERO_E};
      if (Sn > 1 && !(fm[Sn - 2] & ARC_OUT_STAY)) f2 = Sc{0.0, ZERO_E};
    }
    int emax;
    const double sum = sc_sum3(f1, f2, Sc{0.0, ZERO_E}, emax);
    const Sc P = sc_make(sum, emax);
    const double logP = P.m > 0.0 ? log(P.m) + (double)P.e * 0x1.62e42fefa39efp-1 : -INFINITY;
    b.utt_logp[n] = logP;
    b.utt_pm[n] = P.m;
    b.utt_pe[n] = P.e;
    if (isfinite(logP)) {
      b.utt_loss[n] = -logP;
      b.utt_status[n] = UTT_OK;
    } else {
      b.utt_loss[n] = 0.0;
      b.utt_status[n] = UTT_NONFINITE;
    }
  }
}

// Backward sums of utterance n as scaled probabilities.  The stored value of
// a node excludes its own emission (alpha * beta / P is then its posterior);
// the recursion carries the value with the emission.
template <int SPT, bool PRUNED>
__device__ __forceinline__ void beta_sum(
    int n, char* sh, const float* __restrict__ S, int M, const int* __restrict__ row_off,
    const int* __restrict__ tgt_off, const int* __restrict__ tgt_rel,
    const uint8_t* __restrict__ flags, const long long* __restrict__ dp_off,
    const uint8_t* __restrict__ mask, const DpBufs& b) {
  // frames per prefetch block: fewer with more states per thread, so the
  // prefetch registers fit beside the states'
  constexpr int PFS = SPT >= 4 ? 2 : (SPT == 2 ? 4 : PF);
  if (!flags[n]) return;
  const int row0 = row_off[n], T = row_off[n + 1] - row0;
  const int y0 = tgt_off[n], L = tgt_off[n + 1] - y0, Sn = 2 * L + 1;
  const int cap = SPT * blockDim.x;
  double* mb0 = reinterpret_cast<double*>(sh);
  double* mb1 = mb0 + cap;
  int* eb0 = reinterpret_cast<int*>(mb1 + cap);
  int* eb1 = eb0 + cap;
  const long long o0 = dp_off[n];
  Sc32* om = reinterpret_cast<Sc32*>(b.bm) + o0;
  const uint8_t* mk = PRUNED ? mask + o0 : nullptr;
  int sidx[SPT];
  long long ebase[SPT];
  bool skip[SPT];
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int s = threadIdx.x + j * blockDim.x;
    sidx[j] = s;
    int cls = 0;
    bool sk = false;
    if (s < Sn && (s & 1)) {
      cls = tgt_rel[y0 + (s >> 1)];
      sk = s + 2 < Sn && cls != tgt_rel[y0 + (s >> 1) + 1];
    }
    skip[j] = sk;
    ebase[j] = (long long)cls * M + row0;
  }
  // Frames are visited downwards; block b covers frames T-1-b*PFS-u, u < PFS.
  float ecur[SPT][PFS], enxt[SPT][PFS];
  int mcur[SPT][PFS], mnxt[SPT][PFS];
#pragma unroll
  for (int j = 0; j < SPT; ++j)
#pragma unroll
    for (int u = 0; u < PFS; ++u) {
      const int t = T - 1 - u;
      dp_fetch<PRUNED>(S, ebase[j], mk, t, T, sidx[j], Sn, ecur[j][u], mcur[j][u]);
    }
  const int tl = T - 1;
  double* lm = (tl & 1) ? mb1 : mb0;
  int* le = (tl & 1) ? eb1 : eb0;
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int s = sidx[j];
    if (s < Sn) {
      const bool fin = s >= Sn - 2 && (!PRUNED || (mcur[j][0] & ARC_OUT_STAY));
      // beta = 1 on the final states (0.5 * 2^1), times the emission
      const Sc p = sc_exp(ecur[j][0]);
      const Sc u = fin ? sc_make(p.m, p.e) : Sc{0.0, ZERO_E};
      lm[s] = u.m;
      le[s] = u.e;
      om[(long long)tl * Sn + s] = fin ? Sc32{0.5f, 1} : Sc32{0.f, ZERO_E};
    }
  }
  lds_barrier();
  for (int tb = 0; tb < T; tb += PFS) {
    if (tb + PFS < T) {
#pragma unroll
      for (int j = 0; j < SPT; ++j)
#pragma unroll
        for (int u = 0; u < PFS; ++u) {
          const int t = T - 1 - (tb + PFS + u);
          dp_fetch_next<PRUNED>(S, ebase[j], mk, t, T, sidx[j], Sn, enxt[j][u], mnxt[j][u]);
        }
    }
#pragma unroll
    for (int u = 0; u < PFS; ++u) {
      const int t = T - 1 - (tb + u);
      if (t < 0) break;
      if (t == T - 1) continue;
      const double* nm = ((t + 1) & 1) ? mb1 : mb0;
      const int* ne = ((t + 1) & 1) ? eb1 : eb0;
      double* cm = (t & 1) ? mb1 : mb0;
      int* ce = (t & 1) ? eb1 : eb0;
#pragma unroll
      for (int j = 0; j < SPT; ++j) {
        const int s = sidx[j];
        if (s < Sn) {
          const Sc p = sc_exp(ecur[j][u]);
          const int m = mcur[j][u];
          const bool k0 = !PRUNED || (m & ARC_OUT_STAY);
          const bool k1 = s + 1 < Sn && (!PRUNED || (m & ARC_OUT_ADV));
          const bool k2 = skip[j] && (!PRUNED || (m & ARC_OUT_SKIP));
          const Sc b0 = k0 ? Sc{nm[s], ne[s]} : Sc{0.0, ZERO_E};
          const Sc b1 = k1 ? Sc{nm[s + 1], ne[s + 1]} : Sc{0.0, ZERO_E};
          const Sc b2 = k2 ? Sc{nm[s + 2], ne[s + 2]} : Sc{0.0, ZERO_E};
          int emax;
          const double sum = sc_sum3(b0, b1, b2, emax);
          const Sc v = sc_make(sum * p.m, emax + p.e);
          cm[s] = v.m;
          ce[s] = v.e;
          // stored without the emission: the sum itself (not renormalised;
          // below 3 times a power of two)
          om[(long long)t * Sn + s] = Sc32{(float)sum, sum == 0.0 ? ZERO_E : emax};
        }
      }
      lds_barrier();
    }
#pragma unroll
    for (int j = 0; j < SPT; ++j)
#pragma unroll
      for (int u = 0; u < PFS; ++u) {
        ecur[j][u] = enxt[j][u];
        mcur[j][u] = mnxt[j][u];
      }
  }
}

// Both recursions in one launch: work-groups 0..N-1 run the forward
// recursion of utterance n, work-groups N..2N-1 (when launched) the backward
// recursion of utterance n - N.  The two only read S (and the arc masks), so
// they run side by side (the loss pass needs the forward ones only; the
// backward pass reads both).
template <int SPT, int MODE>
__global__ __launch_bounds__(1024) void k_alpha_beta(
    const float* __restrict__ S, int M, int N, const int* __restrict__ row_off,
    const int* __restrict__ tgt_off, const int* __restrict__ tgt_rel,
    const uint8_t* __restrict__ flags, const long long* __restrict__ dp_off,
    const uint8_t* __restrict__ mask, DpBufs bufs) {
  extern __shared__ double sh[];
  const int b = blockIdx.x;
  if (MODE == DP_MAX) {
    if (b < N)
      alpha_utt<SPT, DP_MAX>(b, sh, S, M, row_off, tgt_off, tgt_rel, flags, dp_off, mask,
                             bufs.am, nullptr, nullptr, nullptr, bufs.best);
    else
      beta_utt<SPT, DP_MAX>(b - N, sh, S, M, row_off, tgt_off, tgt_rel, flags, dp_off, mask,
                            bufs.bm);
  } else {
    char* shc = reinterpret_cast<char*>(sh);
    if (b < N)
      alpha_sum<SPT, MODE == DP_PRUNED>(b, shc, S, M, row_off, tgt_off, tgt_rel, flags, dp_off,
                                        mask, bufs);
    else
      beta_sum<SPT, MODE == DP_PRUNED>(b - N, shc, S, M, row_off, tgt_off, tgt_rel, flags,
                                       dp_off, mask, bufs);
  }
}

// Arc masks of a finite alignment beam.  An arc is kept when the best
// complete alignment through it scores at least B_n - beam, B_n the best
// alignment of utterance n ("Pruned CTC for Memory-Efficient Large-
// Vocabulary ASR Training", App. B.1 finite-beam computation; pruning
// relative to the best path, as a log-score output beam).  The score of the
// arc (t-1, s') -> (t, s) is (vf[t-1][s'] + e_t(s)) + vb[t][s] in FP64, in
// that association; the initial arc into (0, s) scores vf[0][s] + vb[0][s]
// and the final arc out of (T-1, s) scores vf[T-1][s].  Every node writes
// the bits of its incoming and of its outgoing arcs (the same decisions,
// read by the forward and by the backward recursion).
//
// Work-group (n, frame tile, state tile): MASK_TF frames x MASK_TS states of
// utterance n.  The emissions of the tile (and of the next frame and the
// next two states, for the outgoing arcs) are staged in LDS first, each
// state's frames read as one contiguous run of S (class-major); then thread
// j walks the tile's frames for state s0 + j, so that the best-score tables
// ([t][s], s contiguous) are read across the threads of a wavefront.
constexpr int MASK_TF = 16, MASK_TS = 256;

__global__ __launch_bounds__(MASK_TS) void k_beam_mask(
    const float* __restrict__ S, int M, const int* __restrict__ row_off,
    const int* __restrict__ tgt_off, const int* __restrict__ tgt_rel,
    const uint8_t* __restrict__ flags, const long long* __restrict__ dp_off,
    const double* __restrict__ vf, const double* __restrict__ vb,
    const double* __restrict__ best, double beam, uint8_t* __restrict__ mask) {
  constexpr int ET = MASK_TF + 1, ES = MASK_TS + 2;
  __shared__ float e_sh[ES][ET + 1];  // [state][frame], padded
  __shared__ int c_sh[ES];            // class of each state of the tile
  const int n = blockIdx.x;
  if (!flags[n]) return;
  const int row0 = row_off[n], T = row_off[n + 1] - row0;
  const int y0 = tgt_off[n], L = tgt_off[n + 1] - y0, Sn = 2 * L + 1;
  const int t0 = blockIdx.y * MASK_TF, s0 = blockIdx.z * MASK_TS;
  if (t0 >= T || s0 >= Sn) return;
  for (int k = threadIdx.x; k < ES; k += MASK_TS) {
    const int s = s0 + k;
    c_sh[k] = (s < Sn && (s & 1)) ? tgt_rel[y0 + (s >> 1)] : 0;
  }
  lds_barrier();
  for (int k = threadIdx.x; k < ES * ET; k += MASK_TS) {
    const int ss = k / ET, tt = k - ss * ET;
    const int s = s0 + ss, t = t0 + tt;
    e_sh[ss][tt] = (s < Sn && t < T) ? S[(long long)c_sh[ss] * M + row0 + t] : 0.f;
  }
  lds_barrier();
  const int j = threadIdx.x, s = s0 + j;
  if (s >= Sn) return;
  const long long base = dp_off[n];
  const double thr = best[n] - beam;
  const int cls = c_sh[j];
  const bool skip_in = (s & 1) && s >= 3 && cls != tgt_rel[y0 + (s >> 1) - 1];
  const bool skip_out = (s & 1) && s + 2 < Sn && c_sh[j + 2] != cls;
  const double* f = vf + base;
  const double* g = vb + base;
  const int t1 = min(T, t0 + MASK_TF);
  for (int t = t0; t < t1; ++t) {
    const int tt = t - t0;
    int bits = 0;
    if (t == 0) {
      if (s <= 1 && f[s] + g[s] >= thr) bits |= ARC_IN_STAY;  // initial arc
    } else {
      const double e = (double)e_sh[j][tt];
      const double* fp = f + (long long)(t - 1) * Sn;
      const double gs = g[(long long)t * Sn + s];
      if ((fp[s] + e) + gs >= thr) bits |= ARC_IN_STAY;
      if (s >= 1 && (fp[s - 1] + e) + gs >= thr) bits |= ARC_IN_ADV;
      if (skip_in && (fp[s - 2] + e) + gs >= thr) bits |= ARC_IN_SKIP;
    }
    const double fs = f[(long long)t * Sn + s];
    if (t == T - 1) {
      if (s >= Sn - 2 && fs >= thr) bits |= ARC_OUT_STAY;  // final arc
    } else {
      const double* gn = g + (long long)(t + 1) * Sn;
      if ((fs + (double)e_sh[j][tt + 1]) + gn[s] >= thr) bits |= ARC_OUT_STAY;
      if (s + 1 < Sn && (fs + (double)e_sh[j + 1][tt + 1]) + gn[s + 1] >= thr)
        bits |= ARC_OUT_ADV;
      if (skip_out && (fs + (double)e_sh[j + 2][tt + 1]) + gn[s + 2] >= thr)
        bits |= ARC_OUT_SKIP;
    }
    mask[base + (long long)t * Sn + s] = (uint8_t)bits;
  }
}

// Occupancies on the selected classes for OCC_FRAMES frames of one
// utterance: q(t, s) = alpha * beta / P per state (scaled probabilities;
// beta excludes the node's emission), gamma of a class = sum of q over its
// states (fixed order), g_m = sum_s q.  Rows of excluded utterances get
// g = 0 (Gamma was zero-filled).
//
// The frames are taken F at a time (F = 1, 2, 4 or 8, as many as the LDS
// holds for the longest utterance), so that the loads of F frames are in
// flight together and one pair of barriers serves F frames.  Work is split
// frame-fastest: thread k always handles frame k mod F of a round, and a
// class's Gamma stores for the F frames are contiguous.
constexpr int OCC_THREADS = 256;
// Frames per work-group (16 and 8 measured 8% faster than 32 at V = 500, 64
// 15% slower: more work-groups keep more loads in flight).
constexpr int OCC_FRAMES = 16;
constexpr int OCC_UNROLL = 8;  // states per thread whose loads are in flight together

template <int F>
__global__ __launch_bounds__(OCC_THREADS) void k_occupancy(
    int M, const int* __restrict__ row_off, const int* __restrict__ tgt_off,
    const int* __restrict__ tgt_rel, const int* __restrict__ utt_status,
    const double* __restrict__ utt_pm, const int* __restrict__ utt_pe,
    const long long* __restrict__ dp_off, const Sc32* __restrict__ am,
    const Sc32* __restrict__ bm, float* __restrict__ Gam, double* __restrict__ g, int Lcap) {
  static_assert(OCC_THREADS % F == 0 && 64 % F == 0, "frames per round");
  extern __shared__ double sh[];
  constexpr int NW = OCC_THREADS / 64;
  __shared__ double s_bl[NW][F], s_tot[NW][F];
  const int n = blockIdx.x;
  const int row0 = row_off[n], T = row_off[n + 1] - row0;
  const int t0 = blockIdx.y * OCC_FRAMES;
  if (t0 >= T) return;
  const int t1 = min(T, t0 + OCC_FRAMES);
  if (utt_status[n] != UTT_OK) {
    for (int t = t0 + threadIdx.x; t < t1; t += blockDim.x) g[row0 + t] = 0.0;
    return;
  }
  const int y0 = tgt_off[n], L = tgt_off[n + 1] - y0, Sn = 2 * L + 1;
  double* s_q = sh;                                            // [Sn][F] doubles
  int* s_y = reinterpret_cast<int*>(sh + F * (2 * Lcap + 1));  // L ints
  int* s_ord = s_y + Lcap;                                     // L ints
  int* s_seg = s_ord + Lcap;                                   // L ints
  for (int i = threadIdx.x; i < L; i += blockDim.x) s_y[i] = tgt_rel[y0 + i];
  lds_barrier();
  // Label positions sorted by (class, position): the occurrences of a class
  // form one segment, in position order.  The first occurrence of a class
  // (its lead) holds start << 16 | length of the segment; the others -1.
  for (int i = threadIdx.x; i < L; i += blockDim.x) {
    const int c = s_y[i];
    int less = 0, before = 0, same = 0;
    for (int j = 0; j < L; ++j) {
      const int cj = s_y[j];
      less += cj < c;
      same += cj == c;
      before += (cj == c) & (j < i);
    }
    s_ord[less + before] = i;
    s_seg[i] = before == 0 ? (less << 16) | same : -1;
  }
  lds_barrier();
  const double invP = 1.0 / utt_pm[n];
  const int Pe = utt_pe[n];
  const Sc32* Ab = am + dp_off[n];
  const Sc32* Bb = bm + dp_off[n];
  const int f = threadIdx.x % F;  // this thread's frame within a round
  for (int tb = t0; tb < t1; tb += F) {
    const int t = tb + f;
    const bool live = t < t1;
    // q of (state, frame) pairs, state-major / frame-fastest; OCC_UNROLL
    // states per thread at a time, their loads (of clamped, in-bounds nodes:
    // a load under a per-lane condition is waited for on the spot) issued
    // together
    double bl = 0.0, tot = 0.0;
    constexpr int SS = OCC_THREADS / F;  // state stride
    const long long ro = (long long)(live ? t : t1 - 1) * Sn;
    for (int s0 = threadIdx.x / F; s0 < Sn; s0 += OCC_UNROLL * SS) {
      Sc32 a[OCC_UNROLL], bb[OCC_UNROLL];
#pragma unroll
      for (int u = 0; u < OCC_UNROLL; ++u) {
        const long long o = ro + min(s0 + u * SS, Sn - 1);
        a[u] = Ab[o];
        bb[u] = Bb[o];
      }
#pragma unroll
      for (int u = 0; u < OCC_UNROLL; ++u) {
        const int s = s0 + u * SS;
        if (s < Sn) {
          const double q =
              live ? ldexp((double)a[u].m * (double)bb[u].m * invP, a[u].e + bb[u].e - Pe) : 0.0;
          s_q[s * F + f] = q;
          tot += q;
          if (!(s & 1)) bl += q;
        }
      }
    }
    // fixed-order sums per frame: a butterfly over the lanes of one frame
    // within each wavefront, then the wavefront sums in order
#pragma unroll
    for (int o = 32; o >= F; o >>= 1) {
      bl += __shfl_xor(bl, o, 64);
      tot += __shfl_xor(tot, o, 64);
    }
    if ((threadIdx.x & 63) < F) {
      s_bl[threadIdx.x >> 6][f] = bl;
      s_tot[threadIdx.x >> 6][f] = tot;
    }
    lds_barrier();
    for (int k = threadIdx.x; k < L * F; k += OCC_THREADS) {
      const int i = k / F, tk = tb + k % F;
      const int seg = s_seg[i];
      if (seg >= 0 && tk < t1) {
        const int* ord = s_ord + (seg >> 16);
        const int len = seg & 0xFFFF;
        double gm = 0.0;  // occurrences in position order
        for (int j = 0; j < len; ++j) gm += s_q[(2 * ord[j] + 1) * F + k % F];
        Gam[(long long)s_y[i] * M + row0 + tk] = (float)gm;
      }
    }
    if (threadIdx.x < F && tb + (int)threadIdx.x < t1) {
      const int fr = threadIdx.x;
      double b0 = s_bl[0][fr], t0s = s_tot[0][fr];
#pragma unroll
      for (int q = 1; q < NW; ++q) {
        b0 += s_bl[q][fr];
        t0s += s_tot[q][fr];
      }
      Gam[row0 + tb + fr] = (float)b0;  // blank is U[0]
      g[row0 + tb + fr] = t0s;
    }
    lds_barrier();
  }
}

// out = grad * sum_m (g_m exp(S[0][m]) - Gamma[0][m]): the blank is U[0], so
// this is the column sum of dZ at the blank (the gradient of a blank-logit
// offset).  FP64, strided per-thread sums then a fixed-order tree.
__global__ __launch_bounds__(256) void k_blank_grad(const float* __restrict__ S,
                                                    const float* __restrict__ Gam,
                                                    const double* __restrict__ g, int M,
                                                    double grad, double* __restrict__ out) {
  __shared__ double part[256];
  double s = 0.0;
  for (int m = threadIdx.x; m < M; m += 256)
    s += g[m] * exp_nonpos((double)S[m]) - (double)Gam[m];  // S <= 0
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = grad * part[0];
}

// Sum of the included utterances' losses and the counts of excluded ones.
// One work-group: thread i takes utterances i, i + 256, ... in order (both
// loads issued unconditionally), then a fixed-order tree over the threads,
// so the result does not depend on timing.
constexpr int LOSS_THREADS = 256;

__global__ __launch_bounds__(LOSS_THREADS) void k_loss_sum(int N,
                                                           const double* __restrict__ utt_loss,
                                                           const int* __restrict__ utt_status,
                                                           Meta* __restrict__ meta) {
  __shared__ double s_tot[LOSS_THREADS];
  __shared__ int s_nu[LOSS_THREADS], s_nf[LOSS_THREADS];
  double tot = 0.0;
  int nu = 0, nf = 0;
  for (int n = threadIdx.x; n < N; n += LOSS_THREADS) {
    const int st = utt_status[n];
    const double l = utt_loss[n];
    tot += st == UTT_OK ? l : 0.0;
    nu += st == UTT_UNALIGNABLE;
    nf += st != UTT_OK && st != UTT_UNALIGNABLE;
  }
  s_tot[threadIdx.x] = tot;
  s_nu[threadIdx.x] = nu;
  s_nf[threadIdx.x] = nf;
  __syncthreads();
  for (int w = LOSS_THREADS / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      s_tot[threadIdx.x] += s_tot[threadIdx.x + w];
      s_nu[threadIdx.x] += s_nu[threadIdx.x + w];
      s_nf[threadIdx.x] += s_nf[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    meta->loss = s_tot[0];
    meta->n_unalignable = s_nu[0];
    meta->n_nonfinite = s_nf[0];
  }
}

__global__ void k_fill_f32(float* __restrict__ p, long long n, float v) {
  const long long n4 = n / 4;
  f32x4 v4 = {v, v, v, v};
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n4;
       i += (long long)gridDim.x * blockDim.x)
    reinterpret_cast<f32x4*>(p)[i] = v4;
  for (long long i = n4 * 4 + blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void k_fill_zero_u16(uint16_t* __restrict__ p, long long n) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x)
    p[i] = 0;
}

void dp_shape(int max_L, int& threads, int& spt) {
  const int Smax = 2 * max_L + 1;
  threads = ((Smax + 63) / 64) * 64;
  if (threads > 1024) threads = 1024;
  spt = (Smax + threads - 1) / threads;
  if (spt == 3) spt = 4;
}

}  // namespace

hipError_t launch_alpha_beta(hipStream_t st, const float* S, int M, int N, int max_L,
                             const int* row_off, const int* tgt_off, const int* tgt_rel,
                             const uint8_t* flags, const long long* dp_off, double* am,
                             double* bm, double* utt_loss, double* utt_logp,
                             double* utt_pm, int* utt_pe, int* utt_status, int mode,
                             const uint8_t* mask, double* best, int fwd_only) {
  if (N == 0) return hipSuccess;
  int threads, spt;
  dp_shape(max_L, threads, spt);
  // two frames of values: FP64 (and, for the sums, an int32 exponent each)
  const size_t shm = 2 * (size_t)spt * threads * (sizeof(double) + (mode == 2 ? 0 : sizeof(int)));
  const int grid = fwd_only ? N : 2 * N;
  const DpBufs bufs{am, bm, utt_loss, utt_logp, utt_pm, utt_pe, utt_status, best};
#define PCX_AB(SPT_, MODE_)                                                                  \
  k_alpha_beta<SPT_, MODE_><<<grid, threads, shm, st>>>(S, M, N, row_off, tgt_off, tgt_rel,  \
                                                        flags, dp_off, mask, bufs)
#define PCX_AB_MODE(SPT_)                              \
  switch (mode) {                                      \
    case DP_SUM: PCX_AB(SPT_, DP_SUM); break;          \
    case DP_PRUNED: PCX_AB(SPT_, DP_PRUNED); break;    \
    case DP_MAX: PCX_AB(SPT_, DP_MAX); break;          \
    default: return hipErrorInvalidValue;              \
  }
  switch (spt) {
    case 1: PCX_AB_MODE(1); break;
    case 2: PCX_AB_MODE(2); break;
    case 4: PCX_AB_MODE(4); break;
    default:
      return hipErrorInvalidValue;
  }
#undef PCX_AB_MODE
#undef PCX_AB
  return hipGetLastError();
}

hipError_t launch_beam_mask(hipStream_t st, const float* S, int M, int N, long long dp_total,
                            int max_T, int max_L, const int* row_off, const int* tgt_off, const int* tgt_rel,
                            const uint8_t* flags, const long long* dp_off, const double* vf,
                            const double* vb, const double* best, double beam, uint8_t* mask) {
  if (N == 0 || dp_total == 0 || max_T <= 0) return hipSuccess;
  const dim3 grid(N, (max_T + MASK_TF - 1) / MASK_TF, (2 * max_L + 1 + MASK_TS - 1) / MASK_TS);
  k_beam_mask<<<grid, MASK_TS, 0, st>>>(S, M, row_off, tgt_off, tgt_rel, flags, dp_off, vf, vb,
                                        best, beam, mask);
  return hipGetLastError();
}

hipError_t launch_loss_sum(hipStream_t st, int N, const double* utt_loss, const int* utt_status,
                           Meta* meta) {
  k_loss_sum<<<1, LOSS_THREADS, 0, st>>>(N, utt_loss, utt_status, meta);
  return hipGetLastError();
}

hipError_t launch_occupancy(hipStream_t st, int M, int N, int max_T, int max_L,
                            const int* row_off, const int* tgt_off, const int* tgt_rel,
                            const int* utt_status, const double* utt_pm, const int* utt_pe,
                            const long long* dp_off, const double* am, const double* bm,
                            float* Gam, double* g) {
  if (N == 0 || max_T <= 0) return hipSuccess;
  const int Lcap = max_L > 0 ? max_L : 1;
  // frames per round: the most whose q block leaves room for four
  // work-groups per CU (one frame whatever the length)
  auto shm_of = [&](int F) {
    return (size_t)F * (2 * (size_t)Lcap + 1) * sizeof(double) + 3 * (size_t)Lcap * sizeof(int);
  };
  int F = 8;
  while (F > 1 && shm_of(F) > 40 * 1024) F >>= 1;
  const size_t shm = shm_of(F);
  dim3 grid(N, (max_T + OCC_FRAMES - 1) / OCC_FRAMES);
#define PCX_OCC(FR)                                                                          \
  k_occupancy<FR><<<grid, OCC_THREADS, shm, st>>>(M, row_off, tgt_off, tgt_rel, utt_status,    \
                                                  utt_pm, utt_pe, dp_off,                      \
                                                  reinterpret_cast<const Sc32*>(am),           \
                                                  reinterpret_cast<const Sc32*>(bm), Gam, g,   \
                                                  Lcap)
  switch (F) {
    case 8: PCX_OCC(8); break;
    case 4: PCX_OCC(4); break;
    case 2: PCX_OCC(2); break;
    default: PCX_OCC(1); break;
  }
#undef PCX_OCC
  return hipGetLastError();
}

hipError_t launch_blank_grad(hipStream_t st, const float* S, const float* Gam, const double* g,
                             int M, double grad, double* out) {
  k_blank_grad<<<1, 256, 0, st>>>(S, Gam, g, M, grad, out);
  return hipGetLastError();
}

hipError_t launch_fill_f32(hipStream_t st, float* p, long long n, float v) {
  if (n == 0) return hipSuccess;
  long long g = (n / 4 + 255) / 256;
  if (g < 1) g = 1;
  if (g > 8192) g = 8192;
  k_fill_f32<<<(int)g, 256, 0, st>>>(p, n, v);
  return hipGetLastError();
}

hipError_t launch_fill_zero(hipStream_t st, void* p, long long n, int esz) {
  if (n == 0) return hipSuccess;
  if (esz == 4) return launch_fill_f32(st, (float*)p, n, 0.f);
  if (esz != 2) return hipErrorInvalidValue;
  long long g = (n + 255) / 256;
  if (g > 8192) g = 8192;
  k_fill_zero_u16<<<(int)g, 256, 0, st>>>((uint16_t*)p, n);
  return hipGetLastError();
}

}  // namespace pcx

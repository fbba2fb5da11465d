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
// frame).  Emission scores for the next 8 frames are prefetched into
// registers while the current 8 are processed.
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
//   DP_SUM     log-sum of the forward (backward) scores over every CTC
//              transition: the unpruned alpha (beta) of the loss;
//   DP_PRUNED  the same over the arcs a finite alignment beam keeps (bit
//              masks from k_beam_mask, one byte per lattice node);
//   DP_MAX     best prefix scores vf (emission included) and best suffix
//              scores vb (emission of the node excluded) in FP64 max-plus,
//              and the best complete alignment's score per utterance.
enum : int { DP_SUM = 0, DP_PRUNED = 1, DP_MAX = 2 };

// Arc bits of a lattice node (t, s): bits 0-2 the arcs into it from s
// (stay), s - 1 (advance) and s - 2 (skip); bits 3-5 the arcs out of it to
// s, s + 1 and s + 2.  At t = 0 bit 0 is the initial arc, at t = T - 1 bit 3
// the final arc.
constexpr int ARC_IN_STAY = 1, ARC_IN_ADV = 2, ARC_IN_SKIP = 4;
constexpr int ARC_OUT_STAY = 8, ARC_OUT_ADV = 16, ARC_OUT_SKIP = 32;

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
  float ecur[SPT][PF], enxt[SPT][PF];
  int mcur[SPT][PF], mnxt[SPT][PF];
#pragma unroll
  for (int j = 0; j < SPT; ++j)
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const bool in = sidx[j] < Sn && u < T;
      ecur[j][u] = in ? S[ebase[j] + u] : 0.f;
      mcur[j][u] = (MODE == DP_PRUNED && in) ? mk[(long long)u * Sn + sidx[j]] : 0;
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
  for (int tb = 0; tb < T; tb += PF) {
    if (tb + PF < T) {
#pragma unroll
      for (int j = 0; j < SPT; ++j)
#pragma unroll
        for (int u = 0; u < PF; ++u) {
          const int t = tb + PF + u;
          const bool in = sidx[j] < Sn && t < T;
          enxt[j][u] = in ? S[ebase[j] + t] : 0.f;
          mnxt[j][u] = (MODE == DP_PRUNED && in) ? mk[(long long)t * Sn + sidx[j]] : 0;
        }
    }
#pragma unroll
    for (int u = 0; u < PF; ++u) {
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
      for (int u = 0; u < PF; ++u) {
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
  // Frames are visited downwards; block b covers frames T-1-b*PF-u, u < PF.
  float ecur[SPT][PF], enxt[SPT][PF];
  int mcur[SPT][PF], mnxt[SPT][PF];
#pragma unroll
  for (int j = 0; j < SPT; ++j)
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int t = T - 1 - u;
      const bool in = sidx[j] < Sn && t >= 0;
      ecur[j][u] = in ? S[ebase[j] + t] : 0.f;
      mcur[j][u] = (MODE == DP_PRUNED && in) ? mk[(long long)t * Sn + sidx[j]] : 0;
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
  for (int tb = 0; tb < T; tb += PF) {
    if (tb + PF < T) {
#pragma unroll
      for (int j = 0; j < SPT; ++j)
#pragma unroll
        for (int u = 0; u < PF; ++u) {
          const int t = T - 1 - (tb + PF + u);
          const bool in = sidx[j] < Sn && t >= 0;
          enxt[j][u] = in ? S[ebase[j] + t] : 0.f;
          mnxt[j][u] = (MODE == DP_PRUNED && in) ? mk[(long long)t * Sn + sidx[j]] : 0;
        }
    }
#pragma unroll
    for (int u = 0; u < PF; ++u) {
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
      for (int u = 0; u < PF; ++u) {
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
    const uint8_t* __restrict__ mask, double* __restrict__ alpha, double* __restrict__ beta,
    double* __restrict__ utt_loss, double* __restrict__ utt_logp, int* __restrict__ utt_status,
    double* __restrict__ best) {
  extern __shared__ double sh[];
  const int b = blockIdx.x;
  if (b < N)
    alpha_utt<SPT, MODE>(b, sh, S, M, row_off, tgt_off, tgt_rel, flags, dp_off, mask, alpha,
                         utt_loss, utt_logp, utt_status, best);
  else
    beta_utt<SPT, MODE>(b - N, sh, S, M, row_off, tgt_off, tgt_rel, flags, dp_off, mask, beta);
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
// read by the forward and by the backward recursion).  Work-group (n, k):
// nodes k, k + blockDim.x * gridDim.y, ... of utterance n.
__global__ __launch_bounds__(256) void k_beam_mask(
    const float* __restrict__ S, int M, const int* __restrict__ row_off,
    const int* __restrict__ tgt_off, const int* __restrict__ tgt_rel,
    const uint8_t* __restrict__ flags, const long long* __restrict__ dp_off,
    const double* __restrict__ vf, const double* __restrict__ vb,
    const double* __restrict__ best, double beam, uint8_t* __restrict__ mask) {
  const int n = blockIdx.x;
  if (!flags[n]) return;
  const int row0 = row_off[n], T = row_off[n + 1] - row0;
  const int y0 = tgt_off[n], L = tgt_off[n + 1] - y0, Sn = 2 * L + 1;
  const long long base = dp_off[n];
  const double thr = best[n] - beam;
  const long long nodes = (long long)T * Sn;
  for (long long i = blockIdx.y * (long long)blockDim.x + threadIdx.x; i < nodes;
       i += (long long)gridDim.y * blockDim.x) {
    const int t = (int)(i / Sn), s = (int)(i - (long long)t * Sn);
    const int cls = (s & 1) ? tgt_rel[y0 + (s >> 1)] : 0;
    const double* f = vf + base;
    const double* g = vb + base;
    int bits = 0;
    if (t == 0) {
      if (s <= 1 && f[s] + g[s] >= thr) bits |= ARC_IN_STAY;  // initial arc
    } else {
      const double e = (double)S[(long long)cls * M + row0 + t];
      const double* fp = f + (long long)(t - 1) * Sn;
      const double gs = g[(long long)t * Sn + s];
      if ((fp[s] + e) + gs >= thr) bits |= ARC_IN_STAY;
      if (s >= 1 && (fp[s - 1] + e) + gs >= thr) bits |= ARC_IN_ADV;
      if ((s & 1) && s >= 3 && cls != tgt_rel[y0 + (s >> 1) - 1] && (fp[s - 2] + e) + gs >= thr)
        bits |= ARC_IN_SKIP;
    }
    const double fs = f[(long long)t * Sn + s];
    if (t == T - 1) {
      if (s >= Sn - 2 && fs >= thr) bits |= ARC_OUT_STAY;  // final arc
    } else {
      const double* gn = g + (long long)(t + 1) * Sn;
      const long long r1 = row0 + t + 1;
      const double e0 = (double)S[(long long)cls * M + r1];
      if ((fs + e0) + gn[s] >= thr) bits |= ARC_OUT_STAY;
      if (s + 1 < Sn) {
        const int c1 = ((s + 1) & 1) ? tgt_rel[y0 + ((s + 1) >> 1)] : 0;
        if ((fs + (double)S[(long long)c1 * M + r1]) + gn[s + 1] >= thr) bits |= ARC_OUT_ADV;
      }
      if ((s & 1) && s + 2 < Sn) {
        const int c2 = tgt_rel[y0 + ((s + 2) >> 1)];
        if (c2 != cls && (fs + (double)S[(long long)c2 * M + r1]) + gn[s + 2] >= thr)
          bits |= ARC_OUT_SKIP;
      }
    }
    mask[base + i] = (uint8_t)bits;
  }
}

// Occupancies on the selected classes for OCC_FRAMES frames of one
// utterance: q(t, s) = exp(alpha + beta - emission - log P) per state,
// gamma of a class = sum of q over its states (fixed order), g_m = sum_s q.
// Rows of excluded utterances get g = 0 (Gamma was zero-filled).
//
// The frames are taken F at a time (F = 1, 2, 4 or 8, as many as the LDS
// holds for the longest utterance), so that the loads of F frames are in
// flight together and one pair of barriers serves F frames.  Work is split
// frame-fastest: thread k always handles frame k mod F of a round, and a
// class's Gamma stores for the F frames are contiguous.
constexpr int OCC_THREADS = 256;

template <int F>
__global__ __launch_bounds__(OCC_THREADS) void k_occupancy(
    const float* __restrict__ S, int M, const int* __restrict__ row_off,
    const int* __restrict__ tgt_off, const int* __restrict__ tgt_rel,
    const int* __restrict__ utt_status, const double* __restrict__ utt_logp,
    const long long* __restrict__ dp_off, const double* __restrict__ alpha,
    const double* __restrict__ beta, float* __restrict__ Gam, double* __restrict__ g,
    int Lcap) {
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
  const double logP = utt_logp[n];
  const double* A = alpha + dp_off[n];
  const double* B = beta + dp_off[n];
  const int f = threadIdx.x % F;  // this thread's frame within a round
  for (int tb = t0; tb < t1; tb += F) {
    const int t = tb + f;
    const bool live = t < t1;
    // q of (state, frame) pairs, state-major / frame-fastest
    double bl = 0.0, tot = 0.0;
#pragma unroll 4
    for (int s = threadIdx.x / F; s < Sn; s += OCC_THREADS / F) {
      double q = 0.0;
      if (live) {
        const int cls = (s & 1) ? s_y[s >> 1] : 0;
        const double e = (double)S[(long long)cls * M + row0 + t];
        const long long o = (long long)t * Sn + s;
        q = exp(A[o] + B[o] - e - logP);
      }
      s_q[s * F + f] = q;
      tot += q;
      if (!(s & 1)) bl += q;
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

__global__ void k_loss_sum(int N, const double* __restrict__ utt_loss,
                           const int* __restrict__ utt_status, Meta* __restrict__ meta) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  double tot = 0.0;
  int nu = 0, nf = 0;
  for (int n = 0; n < N; ++n) {
    const int st = utt_status[n];
    if (st == UTT_OK)
      tot += utt_loss[n];
    else if (st == UTT_UNALIGNABLE)
      ++nu;
    else
      ++nf;
  }
  meta->loss = tot;
  meta->n_unalignable = nu;
  meta->n_nonfinite = nf;
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
                             const uint8_t* flags, const long long* dp_off, double* alpha,
                             double* beta, double* utt_loss, double* utt_logp, int* utt_status,
                             int mode, const uint8_t* mask, double* best, int fwd_only) {
  if (N == 0) return hipSuccess;
  int threads, spt;
  dp_shape(max_L, threads, spt);
  const size_t shm = 2 * (size_t)spt * threads * sizeof(double);
  const int grid = fwd_only ? N : 2 * N;
#define PCX_AB(SPT_, MODE_)                                                                  \
  k_alpha_beta<SPT_, MODE_><<<grid, threads, shm, st>>>(S, M, N, row_off, tgt_off, tgt_rel,  \
                                                        flags, dp_off, mask, alpha, beta,    \
                                                        utt_loss, utt_logp, utt_status, best)
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
                            const int* row_off, const int* tgt_off, const int* tgt_rel,
                            const uint8_t* flags, const long long* dp_off, const double* vf,
                            const double* vb, const double* best, double beam, uint8_t* mask) {
  if (N == 0 || dp_total == 0) return hipSuccess;
  // about four nodes per thread on average, at least one work-group per
  // utterance, at most 64
  long long per = (dp_total / N + 1023) / 1024;
  if (per < 1) per = 1;
  if (per > 64) per = 64;
  k_beam_mask<<<dim3(N, (unsigned)per), 256, 0, st>>>(S, M, row_off, tgt_off, tgt_rel, flags,
                                                       dp_off, vf, vb, best, beam, mask);
  return hipGetLastError();
}

hipError_t launch_loss_sum(hipStream_t st, int N, const double* utt_loss, const int* utt_status,
                           Meta* meta) {
  k_loss_sum<<<1, 64, 0, st>>>(N, utt_loss, utt_status, meta);
  return hipGetLastError();
}

hipError_t launch_occupancy(hipStream_t st, const float* S, int M, int N, int max_T, int max_L,
                            const int* row_off, const int* tgt_off, const int* tgt_rel,
                            const int* utt_status, const double* utt_logp,
                            const long long* dp_off, const double* alpha, const double* beta,
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
  k_occupancy<FR><<<grid, OCC_THREADS, shm, st>>>(S, M, row_off, tgt_off, tgt_rel, utt_status, \
                                                  utt_logp, dp_off, alpha, beta, Gam, g, Lcap)
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

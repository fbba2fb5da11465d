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

__device__ __forceinline__ double lse3(double a, double b, double c) {
  const double m = fmax(a, fmax(b, c));
  if (m == -INFINITY) return -INFINITY;
  return m + log(exp_nonpos(a - m) + exp_nonpos(b - m) + exp_nonpos(c - m));
}

__device__ __forceinline__ double lse2(double a, double b) {
  const double m = fmax(a, b);
  if (m == -INFINITY) return -INFINITY;
  return m + log(exp_nonpos(a - m) + exp_nonpos(b - m));
}

// Forward recursion; alpha[t][s] (including the emission at t) is stored
// for the backward pass.
template <int SPT>
__global__ __launch_bounds__(1024) void k_alpha(
    const float* __restrict__ S, int M, const int* __restrict__ row_off,
    const int* __restrict__ tgt_off, const int* __restrict__ tgt_rel,
    const uint8_t* __restrict__ flags, const long long* __restrict__ dp_off,
    double* __restrict__ alpha, double* __restrict__ utt_loss, double* __restrict__ utt_logp,
    int* __restrict__ utt_status) {
  extern __shared__ double sh[];
  const int n = blockIdx.x;
  const int row0 = row_off[n], T = row_off[n + 1] - row0;
  const int y0 = tgt_off[n], L = tgt_off[n + 1] - y0, Sn = 2 * L + 1;
  if (!flags[n]) {
    if (threadIdx.x == 0) {
      utt_loss[n] = 0.0;
      utt_logp[n] = -INFINITY;
      utt_status[n] = UTT_UNALIGNABLE;
    }
    return;
  }
  const int cap = SPT * blockDim.x;
  double* buf0 = sh;
  double* buf1 = sh + cap;
  double* out = alpha + dp_off[n];
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
#pragma unroll
  for (int j = 0; j < SPT; ++j)
#pragma unroll
    for (int u = 0; u < PF; ++u) ecur[j][u] = (sidx[j] < Sn && u < T) ? S[ebase[j] + u] : 0.f;
  // frame 0: only the first blank and the first label can start.
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int s = sidx[j];
    if (s < Sn) {
      const double a = (s <= 1) ? (double)ecur[j][0] : -INFINITY;
      buf0[s] = a;
      out[s] = a;
    }
  }
  __syncthreads();
  for (int tb = 0; tb < T; tb += PF) {
    if (tb + PF < T) {
#pragma unroll
      for (int j = 0; j < SPT; ++j)
#pragma unroll
        for (int u = 0; u < PF; ++u) {
          const int t = tb + PF + u;
          enxt[j][u] = (sidx[j] < Sn && t < T) ? S[ebase[j] + t] : 0.f;
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
          const double a0 = prev[s];
          const double a1 = s >= 1 ? prev[s - 1] : -INFINITY;
          const double a2 = skip[j] ? prev[s - 2] : -INFINITY;
          const double v = lse3(a0, a1, a2) + (double)ecur[j][u];
          cur[s] = v;
          out[(long long)t * Sn + s] = v;
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < SPT; ++j)
#pragma unroll
      for (int u = 0; u < PF; ++u) ecur[j][u] = enxt[j][u];
  }
  if (threadIdx.x == 0) {
    const double* last = ((T - 1) & 1) ? buf1 : buf0;
    const double logP = Sn > 1 ? lse2(last[Sn - 1], last[Sn - 2]) : last[0];
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

// Backward recursion; beta[t][s] includes the emission at t.
template <int SPT>
__global__ __launch_bounds__(1024) void k_beta(
    const float* __restrict__ S, int M, const int* __restrict__ row_off,
    const int* __restrict__ tgt_off, const int* __restrict__ tgt_rel,
    const int* __restrict__ utt_status, const long long* __restrict__ dp_off,
    double* __restrict__ beta) {
  extern __shared__ double sh[];
  const int n = blockIdx.x;
  if (utt_status[n] != UTT_OK) return;
  const int row0 = row_off[n], T = row_off[n + 1] - row0;
  const int y0 = tgt_off[n], L = tgt_off[n + 1] - y0, Sn = 2 * L + 1;
  const int cap = SPT * blockDim.x;
  double* buf0 = sh;
  double* buf1 = sh + cap;
  double* out = beta + dp_off[n];
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
#pragma unroll
  for (int j = 0; j < SPT; ++j)
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int t = T - 1 - u;
      ecur[j][u] = (sidx[j] < Sn && t >= 0) ? S[ebase[j] + t] : 0.f;
    }
  const int tl = T - 1;
  double* lastbuf = (tl & 1) ? buf1 : buf0;
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int s = sidx[j];
    if (s < Sn) {
      const double b = (s >= Sn - 2) ? (double)ecur[j][0] : -INFINITY;
      lastbuf[s] = b;
      out[(long long)tl * Sn + s] = b;
    }
  }
  __syncthreads();
  for (int tb = 0; tb < T; tb += PF) {
    if (tb + PF < T) {
#pragma unroll
      for (int j = 0; j < SPT; ++j)
#pragma unroll
        for (int u = 0; u < PF; ++u) {
          const int t = T - 1 - (tb + PF + u);
          enxt[j][u] = (sidx[j] < Sn && t >= 0) ? S[ebase[j] + t] : 0.f;
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
          const double b0 = nxt[s];
          const double b1 = s + 1 < Sn ? nxt[s + 1] : -INFINITY;
          const double b2 = skip[j] ? nxt[s + 2] : -INFINITY;
          const double v = lse3(b0, b1, b2) + (double)ecur[j][u];
          cur[s] = v;
          out[(long long)t * Sn + s] = v;
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < SPT; ++j)
#pragma unroll
      for (int u = 0; u < PF; ++u) ecur[j][u] = enxt[j][u];
  }
}

// Occupancies on the selected classes for OCC_FRAMES frames of one
// utterance: q(t, s) = exp(alpha + beta - emission - log P) per state,
// gamma of a class = sum of q over its states (fixed order), g_m = sum_s q.
// Rows of excluded utterances get g = 0 (Gamma was zero-filled).
constexpr int OCC_THREADS = 256;

__global__ __launch_bounds__(OCC_THREADS) void k_occupancy(
    const float* __restrict__ S, int M, const int* __restrict__ row_off,
    const int* __restrict__ tgt_off, const int* __restrict__ tgt_rel,
    const int* __restrict__ utt_status, const double* __restrict__ utt_logp,
    const long long* __restrict__ dp_off, const double* __restrict__ alpha,
    const double* __restrict__ beta, float* __restrict__ Gam, double* __restrict__ g,
    int Lcap) {
  extern __shared__ double sh[];
  __shared__ double s_bl[OCC_THREADS], s_tot[OCC_THREADS];
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
  double* s_q = sh;                                       // Sn doubles
  int* s_y = reinterpret_cast<int*>(sh + (2 * Lcap + 1));  // L ints
  int* s_next = s_y + Lcap;                                // L ints
  int* s_lead = s_next + Lcap;                             // L ints
  for (int i = threadIdx.x; i < L; i += blockDim.x) s_y[i] = tgt_rel[y0 + i];
  __syncthreads();
  for (int i = threadIdx.x; i < L; i += blockDim.x) {
    const int c = s_y[i];
    int lead = 1;
    for (int j = 0; j < i; ++j)
      if (s_y[j] == c) {
        lead = 0;
        break;
      }
    int nx = -1;
    for (int j = i + 1; j < L; ++j)
      if (s_y[j] == c) {
        nx = j;
        break;
      }
    s_lead[i] = lead;
    s_next[i] = nx;
  }
  __syncthreads();
  const double logP = utt_logp[n];
  const double* A = alpha + dp_off[n];
  const double* B = beta + dp_off[n];
  for (int t = t0; t < t1; ++t) {
    const int row = row0 + t;
    double bl = 0.0, tot = 0.0;
    for (int s = threadIdx.x; s < Sn; s += blockDim.x) {
      const int cls = (s & 1) ? s_y[s >> 1] : 0;
      const double e = (double)S[(long long)cls * M + row];
      const long long o = (long long)t * Sn + s;
      const double q = exp(A[o] + B[o] - e - logP);
      s_q[s] = q;
      tot += q;
      if (!(s & 1)) bl += q;
    }
    s_bl[threadIdx.x] = bl;
    s_tot[threadIdx.x] = tot;
    __syncthreads();
    for (int stride = OCC_THREADS / 2; stride > 0; stride >>= 1) {
      if ((int)threadIdx.x < stride) {
        s_bl[threadIdx.x] += s_bl[threadIdx.x + stride];
        s_tot[threadIdx.x] += s_tot[threadIdx.x + stride];
      }
      __syncthreads();
    }
    for (int i = threadIdx.x; i < L; i += blockDim.x) {
      if (s_lead[i]) {
        double gm = 0.0;
        for (int k = i; k >= 0; k = s_next[k]) gm += s_q[2 * k + 1];
        Gam[(long long)s_y[i] * M + row] = (float)gm;
      }
    }
    if (threadIdx.x == 0) {
      Gam[row] = (float)s_bl[0];  // blank is U[0]
      g[row] = s_tot[0];
    }
    __syncthreads();
  }
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

void dp_shape(int max_L, int& threads, int& spt) {
  const int Smax = 2 * max_L + 1;
  threads = ((Smax + 63) / 64) * 64;
  if (threads > 1024) threads = 1024;
  spt = (Smax + threads - 1) / threads;
  if (spt == 3) spt = 4;
}

}  // namespace

hipError_t launch_alpha(hipStream_t st, const float* S, int M, int N, int max_L,
                        const int* row_off, const int* tgt_off, const int* tgt_rel,
                        const uint8_t* flags, const long long* dp_off, double* alpha,
                        double* utt_loss, double* utt_logp, int* utt_status) {
  if (N == 0) return hipSuccess;
  int threads, spt;
  dp_shape(max_L, threads, spt);
  const size_t shm = 2 * (size_t)spt * threads * sizeof(double);
  switch (spt) {
    case 1:
      k_alpha<1><<<N, threads, shm, st>>>(S, M, row_off, tgt_off, tgt_rel, flags, dp_off, alpha,
                                          utt_loss, utt_logp, utt_status);
      break;
    case 2:
      k_alpha<2><<<N, threads, shm, st>>>(S, M, row_off, tgt_off, tgt_rel, flags, dp_off, alpha,
                                          utt_loss, utt_logp, utt_status);
      break;
    case 4:
      k_alpha<4><<<N, threads, shm, st>>>(S, M, row_off, tgt_off, tgt_rel, flags, dp_off, alpha,
                                          utt_loss, utt_logp, utt_status);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_loss_sum(hipStream_t st, int N, const double* utt_loss, const int* utt_status,
                           Meta* meta) {
  k_loss_sum<<<1, 64, 0, st>>>(N, utt_loss, utt_status, meta);
  return hipGetLastError();
}

hipError_t launch_beta(hipStream_t st, const float* S, int M, int N, int max_L,
                       const int* row_off, const int* tgt_off, const int* tgt_rel,
                       const int* utt_status, const long long* dp_off, double* beta) {
  if (N == 0) return hipSuccess;
  int threads, spt;
  dp_shape(max_L, threads, spt);
  const size_t shm = 2 * (size_t)spt * threads * sizeof(double);
  switch (spt) {
    case 1:
      k_beta<1><<<N, threads, shm, st>>>(S, M, row_off, tgt_off, tgt_rel, utt_status, dp_off,
                                         beta);
      break;
    case 2:
      k_beta<2><<<N, threads, shm, st>>>(S, M, row_off, tgt_off, tgt_rel, utt_status, dp_off,
                                         beta);
      break;
    case 4:
      k_beta<4><<<N, threads, shm, st>>>(S, M, row_off, tgt_off, tgt_rel, utt_status, dp_off,
                                         beta);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_occupancy(hipStream_t st, const float* S, int M, int N, int max_T, int max_L,
                            const int* row_off, const int* tgt_off, const int* tgt_rel,
                            const int* utt_status, const double* utt_logp,
                            const long long* dp_off, const double* alpha, const double* beta,
                            float* Gam, double* g) {
  if (N == 0 || max_T <= 0) return hipSuccess;
  const int Lcap = max_L > 0 ? max_L : 1;
  const size_t shm = (2 * (size_t)Lcap + 1) * sizeof(double) + 3 * (size_t)Lcap * sizeof(int);
  dim3 grid(N, (max_T + OCC_FRAMES - 1) / OCC_FRAMES);
  k_occupancy<<<grid, OCC_THREADS, shm, st>>>(S, M, row_off, tgt_off, tgt_rel, utt_status,
                                              utt_logp, dp_off, alpha, beta, Gam, g, Lcap);
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

}  // namespace pcx

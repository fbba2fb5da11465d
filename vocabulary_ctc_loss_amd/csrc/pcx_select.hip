// Validation, structural alignability and selected-class construction.
//
// "Pruned CTC for Memory-Efficient Large-Vocabulary ASR Training":
//  * App. B.1: every repeated adjacent label pair forces one extra blank
//    frame, so an utterance is alignable when T_n >= |y_n| + r_n (r_n such
//    pairs in y_n).
//  * App. B.1 / Sec. 3.2: U holds the blank at index 0 and after it the
//    batch's distinct target labels in ascending order; each target label is
//    replaced by its index in U.
// Everything here is integer work; the results are unique and deterministic.
#include "pcx_common.h"

namespace pcx {

// Exclusive scan of one value per thread over a block of up to 1024 threads.
__device__ long long block_exclusive_scan(long long v, long long* total, long long* sm) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nw = (blockDim.x + 63) >> 6;
  long long x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    long long y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sm[wid] = x;
  __syncthreads();
  if (wid == 0) {
    long long s = lane < nw ? sm[lane] : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      long long y = __shfl_up(s, o, 64);
      if (lane >= o) s += y;
    }
    if (lane < nw) sm[lane] = s;
  }
  __syncthreads();
  const long long base = wid ? sm[wid - 1] : 0;
  *total = sm[nw - 1];
  __syncthreads();
  return base + x - v;
}

// Per-utterance checks, repeat pairs, flags and prefix sums (one block).
// The repeat pairs of one utterance are counted by one wavefront, its lanes
// reading consecutive labels.
__global__ __launch_bounds__(1024) void k_prepare_utts(
    int N, int M, long long L_tot, const int* __restrict__ tgt_off,
    const int* __restrict__ tgt, const int* __restrict__ frame_counts,
    int* __restrict__ row_off, uint8_t* __restrict__ flags,
    long long* __restrict__ dp_off, Meta* __restrict__ meta) {
  __shared__ long long sm[32];
  __shared__ int s_err, s_maxL, s_maxT;
  if (threadIdx.x == 0) {
    s_err = 0;
    s_maxL = 0;
    s_maxT = 0;
    if (tgt_off[0] != 0 || (long long)tgt_off[N] != L_tot) s_err |= ERRBIT_TARGET;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int n = wid; n < N; n += nw) {
    const int Tn = frame_counts[n];
    const int a = tgt_off[n], e = tgt_off[n + 1];
    const bool ok = a >= 0 && e >= a && (long long)e <= L_tot;
    int r = 0;
    if (ok)
      // four label pairs per lane at a time, loaded unconditionally from
      // clamped positions (a load under a per-lane condition is waited for on
      // the spot) and counted when in range
      for (int i0 = a; i0 + 1 < e; i0 += 4 * 64) {
        int x[4], y[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int ic = min(i0 + lane + 64 * u, e - 2);
          x[u] = tgt[ic];
          y[u] = tgt[ic + 1];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) r += (i0 + lane + 64 * u + 1 < e) && x[u] == y[u];
      }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) r += __shfl_xor(r, o, 64);
    if (lane == 0) {
      if (!ok) atomicOr(&s_err, ERRBIT_TARGET);
      if (Tn <= 0) atomicOr(&s_err, ERRBIT_LENGTHS);
      const int L = ok ? e - a : 0;
      flags[n] = (Tn > 0 && ok && L + r <= Tn) ? 1 : 0;
      atomicMax(&s_maxL, L);
      atomicMax(&s_maxT, Tn);
    }
  }
  __syncthreads();
  long long rows = 0, dps = 0;
  for (int base = 0; base < N; base += blockDim.x) {
    const int n = base + threadIdx.x;
    long long T = 0, dp = 0;
    if (n < N) {
      const int Tn = frame_counts[n];
      const int a = tgt_off[n], e = tgt_off[n + 1];
      const bool ok = a >= 0 && e >= a && (long long)e <= L_tot;
      const int L = ok ? e - a : 0;
      T = Tn > 0 ? Tn : 0;
      dp = T * (2LL * L + 1);
    }
    long long tot;
    const long long ex = block_exclusive_scan(T, &tot, sm);
    if (n < N) row_off[n] = (int)(rows + ex);
    rows += tot;
    const long long exd = block_exclusive_scan(dp, &tot, sm);
    if (n < N) dp_off[n] = dps + exd;
    dps += tot;
  }
  if (threadIdx.x == 0) {
    row_off[N] = (int)rows;
    dp_off[N] = dps;
    if (rows != (long long)M) s_err |= ERRBIT_LENGTHS;
    meta->err = s_err;
    meta->K = 0;
    meta->max_L = s_maxL;
    meta->max_T = s_maxT;
    meta->dp_total = dps;
    meta->loss = 0.0;
    meta->n_unalignable = 0;
    meta->n_nonfinite = 0;
  }
}

__global__ void k_fill_i32(int* __restrict__ p, int n, int v) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = v;
}

// Mark every label present in the batch (all writers store the same value).
__global__ void k_mark_labels(long long L_tot, const int* __restrict__ tgt, int V, int blank,
                              int* __restrict__ mark, Meta* __restrict__ meta) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < L_tot;
       i += (long long)gridDim.x * blockDim.x) {
    const int v = tgt[i];
    if (v < 0 || v >= V || v == blank)
      atomicOr(&meta->err, ERRBIT_TARGET);
    else
      mark[v] = 1;
  }
}

// Compaction of the marks into U (blank first, then ascending ids) and the
// column -> selected-index map (-1 for unselected columns).  One block; each
// wavefront owns a contiguous id range (a multiple of 64 ids) and walks it 64
// consecutive ids at a time, ranking the marked ones with a ballot, so the
// order is the id order.
__global__ __launch_bounds__(1024) void k_select(int V, int blank, int* __restrict__ col2sel,
                                                 int* __restrict__ U, Meta* __restrict__ meta) {
  __shared__ long long sm[32];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int per = ((V + nw - 1) / nw + 63) / 64 * 64;
  const int lo = min(V, wid * per), hi = min(V, lo + per);
  // SEL_BATCH blocks of 64 ids at a time: their marks are loaded together
  // (clamped ids, loaded unconditionally: a load under a per-lane condition is
  // waited for on the spot), then counted or placed in id order.
  constexpr int SEL_BATCH = 8;
  int cnt = 0;  // marked ids of this wavefront's range (wave-uniform)
  for (int v0 = lo; v0 < hi; v0 += SEL_BATCH * 64) {
    int mk[SEL_BATCH];
#pragma unroll
    for (int u = 0; u < SEL_BATCH; ++u) mk[u] = col2sel[min(v0 + 64 * u + lane, V - 1)];
#pragma unroll
    for (int u = 0; u < SEL_BATCH; ++u) {
      const int v = v0 + 64 * u + lane;
      cnt += __popcll(__ballot(v < hi && v != blank && mk[u] != 0));
    }
  }
  long long tot;
  // lane 0 carries the wavefront's count: its exclusive prefix is the number
  // of marked ids in the ranges of the lower wavefronts
  const long long ex = block_exclusive_scan(lane == 0 ? cnt : 0, &tot, sm);
  int idx = 1 + (int)__shfl(ex, 0, 64);
  for (int v0 = lo; v0 < hi; v0 += SEL_BATCH * 64) {
    int mk[SEL_BATCH];
#pragma unroll
    for (int u = 0; u < SEL_BATCH; ++u) mk[u] = col2sel[min(v0 + 64 * u + lane, V - 1)];
#pragma unroll
    for (int u = 0; u < SEL_BATCH; ++u) {
      const int v = v0 + 64 * u + lane;
      const bool in = v < hi;
      const bool sel = in && v != blank && mk[u] != 0;
      const unsigned long long bal = __ballot(sel);
      const int pos = idx + __popcll(bal & ((1ull << lane) - 1ull));
      if (in) {
        if (v == blank) {
          col2sel[v] = 0;
        } else if (sel) {
          col2sel[v] = pos;
          U[pos] = v;
        } else {
          col2sel[v] = -1;
        }
      }
      idx += __popcll(bal);
    }
  }
  if (threadIdx.x == 0) {
    U[0] = blank;
    meta->K = 1 + (int)tot;
  }
}

__global__ void k_relabel(long long L_tot, const int* __restrict__ tgt, int V,
                          const int* __restrict__ col2sel, int* __restrict__ tgt_rel) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < L_tot;
       i += (long long)gridDim.x * blockDim.x) {
    const int v = tgt[i];
    tgt_rel[i] = (v >= 0 && v < V) ? col2sel[v] : 0;
  }
}

static int grid_for(long long n, int threads, int cap = 4096) {
  long long g = (n + threads - 1) / threads;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

hipError_t launch_prepare(hipStream_t st, int N, int M, int V, int blank, long long L_tot,
                          const int* tgt_off, const int* tgt, const int* frame_counts,
                          int* row_off, uint8_t* flags, long long* dp_off, int* col2sel,
                          int* U, int* tgt_rel, Meta* meta) {
  k_prepare_utts<<<1, 1024, 0, st>>>(N, M, L_tot, tgt_off, tgt, frame_counts, row_off, flags,
                                     dp_off, meta);
  k_fill_i32<<<grid_for(V, 256), 256, 0, st>>>(col2sel, V, 0);
  if (L_tot > 0)
    k_mark_labels<<<grid_for(L_tot, 256), 256, 0, st>>>(L_tot, tgt, V, blank, col2sel, meta);
  k_select<<<1, 1024, 0, st>>>(V, blank, col2sel, U, meta);
  if (L_tot > 0)
    k_relabel<<<grid_for(L_tot, 256), 256, 0, st>>>(L_tot, tgt, V, col2sel, tgt_rel);
  return hipGetLastError();
}

}  // namespace pcx

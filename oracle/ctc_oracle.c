/*
 * CPU FP64 oracle for the vocabulary-head + CTC loss path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or helper with the HIP
 * implementation.
 *
 * What it computes is the plain definition, written out, of full-vocabulary
 * CTC through an affine head (source: "Pruned CTC for Memory-Efficient
 * Large-Vocabulary ASR Training", Sec. 3.1 problem statement, Eq. 1 and 2;
 * Sec. 3.2 Proposition 1 and the logit gradient of Eq. 5):
 *
 *   Z = X W^T + 1 b^T                         (every vocabulary column)
 *   lambda_m = log sum_v exp Z[m][v]          (Eq. 1, the normalizer)
 *   logp[m][v] = Z[m][v] - lambda_m
 *   loss_n = -log sum over alignments pi with B(pi) = y_n of
 *            prod_t p_{pi_t}(frame t)         (Eq. 2, textbook CTC forward
 *                                              recursion on the
 *                                              blank-interleaved labels)
 *   dZ[m][v] = grad * (p_v(m) - gamma_v(m))   (Eq. 5, gamma = occupancy)
 *   dX = dZ W,  dW = dZ^T X,  db = column sums of dZ.
 *
 * Everything is IEEE FP64 with natural-order loops.  The selected-class set
 * and the chunk width of the reduced method play no part in the numerics.
 * Utterances whose target cannot be aligned (|y| + r > T, r = number of
 * adjacent equal label pairs; App. B.1 of the same paper) and utterances
 * whose loss comes out nonfinite contribute zero loss and zero gradient
 * (App. B.1; PrunedCTC README, return value).
 *
 * With a finite alignment beam (oracle_ctc_beam, oracle_pcx_beam) the same
 * quantities are formed over the alignments that survive log-score lattice
 * pruning relative to the best alignment (the pages' finite-beam objective
 * L_beta, App. B.1; the reading is stated at oracle_ctc_beam).
 *
 * Parity pins for every function here live in tests/test_oracle_pins.py
 * (brute-force alignment enumeration, closed forms, finite differences,
 * the reduced-vocabulary identity of Proposition 1, and invariants).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_TARGET 2
#define ORACLE_ERR_LENGTHS 3
#define ORACLE_ERR_NOMEM 4

/* log(exp(a) + exp(b)) with -inf handled. */
static double log_add(double a, double b) {
  if (a == -INFINITY) return b;
  if (b == -INFINITY) return a;
  double hi = a > b ? a : b;
  double lo = a > b ? b : a;
  return hi + log1p(exp(lo - hi));
}

/* Number of adjacent equal label pairs r_n (App. B.1). */
static int repeat_pairs(const int32_t* y, int L) {
  int r = 0;
  for (int i = 0; i + 1 < L; ++i)
    if (y[i] == y[i + 1]) ++r;
  return r;
}

/*
 * Structural alignability and the selected-class set.
 *
 * flags[n] = 1 iff |y_n| + r_n <= T_n (App. B.1).  U = blank first, then
 * the distinct target labels of the whole batch in ascending id order;
 * tgt_rel[i] = position of tgt[i] in U (App. B.1 and Sec. 3.2).
 * Returns the number K of selected classes, or a negative error code.
 */
int oracle_select(int N, int V, int blank, const int32_t* frame_counts,
                  const int32_t* tgt_off, const int32_t* tgt, int32_t* U,
                  int32_t* tgt_rel, uint8_t* flags) {
  if (N < 0 || V <= 0 || blank < 0 || blank >= V) return -ORACLE_ERR_ARG;
  if (tgt_off[0] != 0) return -ORACLE_ERR_TARGET;
  for (int n = 0; n < N; ++n) {
    if (tgt_off[n + 1] < tgt_off[n]) return -ORACLE_ERR_TARGET;
    if (frame_counts[n] <= 0) return -ORACLE_ERR_LENGTHS;
  }
  int Ltot = tgt_off[N];
  unsigned char* present = (unsigned char*)calloc((size_t)V, 1);
  if (!present) return -ORACLE_ERR_NOMEM;
  for (int i = 0; i < Ltot; ++i) {
    if (tgt[i] < 0 || tgt[i] >= V || tgt[i] == blank) {
      free(present);
      return -ORACLE_ERR_TARGET;
    }
    present[tgt[i]] = 1;
  }
  int K = 0;
  U[K++] = blank;
  for (int v = 0; v < V; ++v)
    if (present[v] && v != blank) U[K++] = v;
  for (int i = 0; i < Ltot; ++i) {
    int lo = 1, hi = K - 1; /* U[1..K-1] is ascending */
    while (lo < hi) {
      int mid = (lo + hi) / 2;
      if (U[mid] < tgt[i]) lo = mid + 1; else hi = mid;
    }
    tgt_rel[i] = lo;
  }
  for (int n = 0; n < N; ++n) {
    int L = tgt_off[n + 1] - tgt_off[n];
    int r = repeat_pairs(tgt + tgt_off[n], L);
    flags[n] = (L + r <= frame_counts[n]) ? 1 : 0;
  }
  free(present);
  return K;
}

/*
 * CTC for one utterance from raw logits Z (T x V, row-major).
 *
 * Computes lambda (Eq. 1), the log-likelihood by the forward recursion on
 * the extended label sequence (blank, y1, blank, y2, ..., yL, blank), the
 * backward recursion, the occupancies gamma and the logit gradient of Eq. 5:
 *   dZ[t][v] = grad * (p_v(t) - gamma_v(t)).
 * status: 0 = finite loss; 1 = not structurally alignable; 2 = nonfinite.
 * For status != 0 the loss is 0 and dZ / gamma are all zero.
 * Any of lambda_out, dZ, gamma may be NULL.
 */
int oracle_ctc_logits(int T, int V, int blank, const double* Z,
                      const int32_t* y, int L, double grad,
                      double* loss_out, int* status_out, double* lambda_out,
                      double* dZ, double* gamma) {
  if (T <= 0 || V <= 0 || L < 0 || blank < 0 || blank >= V)
    return ORACLE_ERR_ARG;
  for (int i = 0; i < L; ++i)
    if (y[i] < 0 || y[i] >= V || y[i] == blank) return ORACLE_ERR_TARGET;
  const int S = 2 * L + 1;
  double* logp = (double*)malloc(sizeof(double) * (size_t)T * V);
  double* alpha = (double*)malloc(sizeof(double) * (size_t)T * S);
  double* beta = (double*)malloc(sizeof(double) * (size_t)T * S);
  int32_t* ext = (int32_t*)malloc(sizeof(int32_t) * (size_t)S);
  if (!logp || !alpha || !beta || !ext) {
    free(logp); free(alpha); free(beta); free(ext);
    return ORACLE_ERR_NOMEM;
  }
  /* Eq. 1: log-softmax over the whole vocabulary, one row at a time. */
  for (int t = 0; t < T; ++t) {
    const double* z = Z + (size_t)t * V;
    double mx = -INFINITY;
    for (int v = 0; v < V; ++v) if (z[v] > mx) mx = z[v];
    double s = 0.0;
    for (int v = 0; v < V; ++v) s += exp(z[v] - mx);
    double lam = mx + log(s);
    if (lambda_out) lambda_out[t] = lam;
    for (int v = 0; v < V; ++v) logp[(size_t)t * V + v] = z[v] - lam;
  }
  for (int s = 0; s < S; ++s) ext[s] = (s % 2 == 0) ? blank : y[s / 2];

  int r = repeat_pairs(y, L);
  int status = 0;
  double loss = 0.0;
  if (L + r > T) {
    status = 1;
  } else {
    /* Forward recursion (alpha includes the emission at frame t). */
    for (int s = 0; s < S; ++s) alpha[s] = -INFINITY;
    alpha[0] = logp[ext[0]];
    if (S > 1) alpha[1] = logp[ext[1]];
    for (int t = 1; t < T; ++t) {
      const double* lp = logp + (size_t)t * V;
      const double* prev = alpha + (size_t)(t - 1) * S;
      double* cur = alpha + (size_t)t * S;
      for (int s = 0; s < S; ++s) {
        double a = prev[s];
        if (s >= 1) a = log_add(a, prev[s - 1]);
        if (s >= 2 && ext[s] != blank && ext[s] != ext[s - 2])
          a = log_add(a, prev[s - 2]);
        cur[s] = a + lp[ext[s]];
      }
    }
    const double* last = alpha + (size_t)(T - 1) * S;
    double logP = last[S - 1];
    if (S > 1) logP = log_add(logP, last[S - 2]);
    /* Backward recursion (beta also includes the emission at frame t). */
    for (int s = 0; s < S; ++s) beta[(size_t)(T - 1) * S + s] = -INFINITY;
    beta[(size_t)(T - 1) * S + S - 1] = logp[(size_t)(T - 1) * V + ext[S - 1]];
    if (S > 1)
      beta[(size_t)(T - 1) * S + S - 2] =
          logp[(size_t)(T - 1) * V + ext[S - 2]];
    for (int t = T - 2; t >= 0; --t) {
      const double* lp = logp + (size_t)t * V;
      const double* nxt = beta + (size_t)(t + 1) * S;
      double* cur = beta + (size_t)t * S;
      for (int s = 0; s < S; ++s) {
        double b = nxt[s];
        if (s + 1 < S) b = log_add(b, nxt[s + 1]);
        if (s + 2 < S && ext[s] != blank && ext[s] != ext[s + 2])
          b = log_add(b, nxt[s + 2]);
        cur[s] = b + lp[ext[s]];
      }
    }
    if (!isfinite(logP)) {
      status = 2;
    } else {
      loss = -logP;
    }
    if (status == 0 && (dZ || gamma)) {
      double* gam_row = (double*)malloc(sizeof(double) * (size_t)V);
      if (!gam_row) {
        free(logp); free(alpha); free(beta); free(ext);
        return ORACLE_ERR_NOMEM;
      }
      for (int t = 0; t < T; ++t) {
        memset(gam_row, 0, sizeof(double) * (size_t)V);
        const double* lp = logp + (size_t)t * V;
        for (int s = 0; s < S; ++s) {
          double lg = alpha[(size_t)t * S + s] + beta[(size_t)t * S + s] -
                      lp[ext[s]] - logP;
          gam_row[ext[s]] += exp(lg);
        }
        for (int v = 0; v < V; ++v) {
          if (gamma) gamma[(size_t)t * V + v] = gam_row[v];
          if (dZ) dZ[(size_t)t * V + v] = grad * (exp(lp[v]) - gam_row[v]);
        }
      }
      free(gam_row);
    }
  }
  if (status != 0) {
    if (dZ) memset(dZ, 0, sizeof(double) * (size_t)T * V);
    if (gamma) memset(gamma, 0, sizeof(double) * (size_t)T * V);
  }
  *loss_out = loss;
  *status_out = status;
  free(logp); free(alpha); free(beta); free(ext);
  return ORACLE_OK;
}

/*
 * Finite-beam CTC for one utterance from raw logits Z (T x V): the pages'
 * pruned objective L_beta ("Pruned CTC for Memory-Efficient
 * Large-Vocabulary ASR Training", App. B.1 finite-beam computation, the
 * finite-beam gap analysis of App. B, and the PrunedCTC README's
 * "alignment pruning" with a log-score beam, output_beam).
 *
 * The body of the objective's equation is missing from the pages; the
 * reading taken here is lattice pruning relative to the best alignment:
 *   * the lattice of utterance n has a node (t, s) per frame t and state s of
 *     the blank-interleaved labels, an initial arc into (0, 0) and (0, 1), an
 *     arc (t-1, s') -> (t, s) for every CTC transition (stay, advance, skip a
 *     blank between different labels), and a final arc out of (T-1, S-1) and
 *     (T-1, S-2); entering (t, s) scores the log-probability logp[t][l'_s];
 *   * the score of an arc is that of the best complete alignment through it:
 *     (vf[t-1][s'] + logp[t][l'_s]) + vb[t][s], with vf the best score of a
 *     prefix ending in a node (its emission included) and vb the best score
 *     of the suffix after it (its emission excluded); the initial arc into
 *     (0, s) scores vf[0][s] + vb[0][s], the final arc out of (T-1, s)
 *     scores vf[T-1][s];
 *   * an arc is kept when its score is at least B - beam, B the best
 *     alignment's score (evaluated in IEEE FP64 in exactly the association
 *     written above); an alignment is retained when all of its arcs are;
 *   * L_beta = -log of the summed probability of the retained alignments,
 *     by the forward / backward recursions restricted to kept arcs; with
 *     the retained lattice held fixed, the logit gradient is
 *     grad * (p_v(m) - gamma^beta_v(m)), gamma^beta the occupancy over the
 *     retained alignments (App. B.1: "with the retained lattice locally
 *     fixed").
 * beam = INFINITY keeps every arc.  A nonfinite L_beta (an empty retained
 * lattice, or nonfinite scores) is replaced by zero loss and zero gradient
 * (App. B.1), status 2; unalignable utterances give status 1.
 *
 * Outputs besides those of oracle_ctc_logits:
 *   full_loss_out  the unpruned loss L_n of the same utterance (NaN when the
 *                  unpruned loss is excluded)
 *   margin_out     the smallest |arc score - (B - beam)| over arcs with a
 *                  finite score (INFINITY for an infinite beam or without
 *                  arcs): how far the pruning decision is from a tie.
 */
int oracle_ctc_beam(int T, int V, int blank, const double* Z, const int32_t* y,
                    int L, double beam, double grad, double* loss_out,
                    int* status_out, double* full_loss_out, double* lambda_out,
                    double* dZ, double* gamma, double* margin_out) {
  if (T <= 0 || V <= 0 || L < 0 || blank < 0 || blank >= V || !(beam >= 0.0))
    return ORACLE_ERR_ARG;
  /* normalizer and unpruned loss from the full-vocabulary routine above */
  double* lam = (double*)malloc(sizeof(double) * (size_t)T);
  if (!lam) return ORACLE_ERR_NOMEM;
  double full = 0.0;
  int full_status = 0;
  int rc = oracle_ctc_logits(T, V, blank, Z, y, L, grad, &full, &full_status,
                             lam, NULL, NULL);
  if (rc != ORACLE_OK) {
    free(lam);
    return rc;
  }
  if (lambda_out) memcpy(lambda_out, lam, sizeof(double) * (size_t)T);
  if (full_loss_out) *full_loss_out = full_status == 0 ? full : NAN;
  if (margin_out) *margin_out = INFINITY;
  *loss_out = 0.0;
  *status_out = full_status;
  if (dZ) memset(dZ, 0, sizeof(double) * (size_t)T * V);
  if (gamma) memset(gamma, 0, sizeof(double) * (size_t)T * V);
  if (full_status == 1) { /* not structurally alignable: nothing to prune */
    free(lam);
    return ORACLE_OK;
  }

  const int S = 2 * L + 1;
  /* per node: label, and its incoming arcs (predecessor states) */
  int32_t* lab = (int32_t*)malloc(sizeof(int32_t) * (size_t)S);
  int32_t* npred = (int32_t*)malloc(sizeof(int32_t) * (size_t)S);
  int32_t* pred = (int32_t*)malloc(sizeof(int32_t) * 3 * (size_t)S);
  double* em = (double*)malloc(sizeof(double) * (size_t)T * S);   /* logp at nodes */
  double* vf = (double*)malloc(sizeof(double) * (size_t)T * S);
  double* vb = (double*)malloc(sizeof(double) * (size_t)T * S);
  double* fa = (double*)malloc(sizeof(double) * (size_t)T * S);   /* pruned alpha */
  double* fb = (double*)malloc(sizeof(double) * (size_t)T * S);   /* pruned beta */
  unsigned char* keep = (unsigned char*)malloc((size_t)T * S * 3); /* kept in-arcs */
  unsigned char* kinit = (unsigned char*)calloc((size_t)S, 1);
  unsigned char* kfin = (unsigned char*)calloc((size_t)S, 1);
  if (!lab || !npred || !pred || !em || !vf || !vb || !fa || !fb || !keep || !kinit ||
      !kfin) {
    free(lam); free(lab); free(npred); free(pred); free(em); free(vf); free(vb);
    free(fa); free(fb); free(keep); free(kinit); free(kfin);
    return ORACLE_ERR_NOMEM;
  }
  for (int s = 0; s < S; ++s) {
    lab[s] = (s & 1) ? y[s / 2] : blank;
    int k = 0;
    pred[3 * s + k++] = s;                          /* stay */
    if (s >= 1) pred[3 * s + k++] = s - 1;          /* advance */
    /* skip over a blank, only into a label that differs from the one before */
    if (s >= 2 && lab[s] != blank && y[s / 2 - 1] != lab[s]) pred[3 * s + k++] = s - 2;
    npred[s] = k;
  }
  for (int t = 0; t < T; ++t)
    for (int s = 0; s < S; ++s)
      em[(size_t)t * S + s] = Z[(size_t)t * V + lab[s]] - lam[t];
  const int first_final = S >= 2 ? S - 2 : 0;

  /* best prefix scores (emission included) */
  for (int s = 0; s < S; ++s) vf[s] = s <= 1 ? em[s] : -INFINITY;
  for (int t = 1; t < T; ++t)
    for (int s = 0; s < S; ++s) {
      double m = -INFINITY;
      for (int k = 0; k < npred[s]; ++k) {
        const double c = vf[(size_t)(t - 1) * S + pred[3 * s + k]];
        if (c > m) m = c;
      }
      vf[(size_t)t * S + s] = m + em[(size_t)t * S + s];
    }
  /* best suffix scores (emission of the node itself excluded) */
  for (int s = 0; s < S; ++s) vb[(size_t)(T - 1) * S + s] = s >= first_final ? 0.0 : -INFINITY;
  for (int t = T - 2; t >= 0; --t) {
    for (int s = 0; s < S; ++s) vb[(size_t)t * S + s] = -INFINITY;
    for (int s2 = 0; s2 < S; ++s2)
      for (int k = 0; k < npred[s2]; ++k) {
        const int s = pred[3 * s2 + k];
        const double c = em[(size_t)(t + 1) * S + s2] + vb[(size_t)(t + 1) * S + s2];
        if (c > vb[(size_t)t * S + s]) vb[(size_t)t * S + s] = c;
      }
  }
  double best = -INFINITY;
  for (int s = first_final; s < S; ++s)
    if (vf[(size_t)(T - 1) * S + s] > best) best = vf[(size_t)(T - 1) * S + s];
  const double thr = best - beam;

  /* which arcs are kept */
  double margin = INFINITY;
#define ORACLE_KEEP(score, flag)                                   \
  do {                                                             \
    const double sc_ = (score);                                    \
    (flag) = sc_ >= thr;                                           \
    if (isfinite(sc_) && isfinite(thr) && fabs(sc_ - thr) < margin) \
      margin = fabs(sc_ - thr);                                    \
  } while (0)
  for (int s = 0; s <= 1 && s < S; ++s) ORACLE_KEEP(vf[s] + vb[s], kinit[s]);
  for (int s = first_final; s < S; ++s) ORACLE_KEEP(vf[(size_t)(T - 1) * S + s], kfin[s]);
  for (int t = 1; t < T; ++t)
    for (int s = 0; s < S; ++s)
      for (int k = 0; k < npred[s]; ++k) {
        const double sc = (vf[(size_t)(t - 1) * S + pred[3 * s + k]] + em[(size_t)t * S + s]) +
                          vb[(size_t)t * S + s];
        ORACLE_KEEP(sc, keep[((size_t)t * S + s) * 3 + k]);
      }
#undef ORACLE_KEEP
  if (margin_out) *margin_out = margin;

  /* forward recursion over kept arcs */
  for (int s = 0; s < S; ++s) fa[s] = (s <= 1 && kinit[s]) ? em[s] : -INFINITY;
  for (int t = 1; t < T; ++t)
    for (int s = 0; s < S; ++s) {
      double a = -INFINITY;
      for (int k = 0; k < npred[s]; ++k)
        if (keep[((size_t)t * S + s) * 3 + k])
          a = log_add(a, fa[(size_t)(t - 1) * S + pred[3 * s + k]]);
      fa[(size_t)t * S + s] = a + em[(size_t)t * S + s];
    }
  double logP = -INFINITY;
  for (int s = first_final; s < S; ++s)
    if (kfin[s]) logP = log_add(logP, fa[(size_t)(T - 1) * S + s]);
  /* backward recursion over the same arcs (emission of the node included) */
  for (int s = 0; s < S; ++s)
    fb[(size_t)(T - 1) * S + s] =
        (s >= first_final && kfin[s]) ? em[(size_t)(T - 1) * S + s] : -INFINITY;
  for (int t = T - 2; t >= 0; --t) {
    for (int s = 0; s < S; ++s) fb[(size_t)t * S + s] = -INFINITY;
    for (int s2 = 0; s2 < S; ++s2)
      for (int k = 0; k < npred[s2]; ++k)
        if (keep[((size_t)(t + 1) * S + s2) * 3 + k]) {
          const int s = pred[3 * s2 + k];
          fb[(size_t)t * S + s] = log_add(fb[(size_t)t * S + s], fb[(size_t)(t + 1) * S + s2]);
        }
    for (int s = 0; s < S; ++s) fb[(size_t)t * S + s] += em[(size_t)t * S + s];
  }

  if (!isfinite(logP)) {
    *status_out = 2;
  } else {
    *status_out = 0;
    *loss_out = -logP;
    if (dZ || gamma) {
      double* occ = (double*)calloc((size_t)V, sizeof(double));
      if (!occ) {
        free(lam); free(lab); free(npred); free(pred); free(em); free(vf); free(vb);
        free(fa); free(fb); free(keep); free(kinit); free(kfin);
        return ORACLE_ERR_NOMEM;
      }
      for (int t = 0; t < T; ++t) {
        for (int v = 0; v < V; ++v) occ[v] = 0.0;
        for (int s = 0; s < S; ++s) {
          const size_t o = (size_t)t * S + s;
          occ[lab[s]] += exp(fa[o] + fb[o] - em[o] - logP);
        }
        for (int v = 0; v < V; ++v) {
          const double pv = exp(Z[(size_t)t * V + v] - lam[t]);
          if (gamma) gamma[(size_t)t * V + v] = occ[v];
          if (dZ) dZ[(size_t)t * V + v] = grad * (pv - occ[v]);
        }
      }
      free(occ);
    }
  }
  free(lam); free(lab); free(npred); free(pred); free(em); free(vf); free(vb);
  free(fa); free(fb); free(keep); free(kinit); free(kfin);
  return ORACLE_OK;
}

/*
 * The whole path: head projection, CTC loss and gradients for a batch of N
 * utterances stacked without padding into X (M x D, row-major; utterance n
 * owns rows [o_n, o_n + T_n) with o_n = T_0 + ... + T_{n-1}).  W is V x D
 * row-major, b has V entries (NULL = zero bias).  Targets are given in CSR
 * form (tgt_off has N+1 entries).  grad is the scalar upstream gradient of
 * the summed loss.
 *
 * Outputs (any pointer except loss_out may be NULL):
 *   loss_out      summed loss over utterances with a finite loss
 *   utt_loss[N]   per-utterance loss (0 for excluded utterances)
 *   status[N]     0 finite, 1 unalignable, 2 nonfinite
 *   lambda[M]     normalizer per frame (Eq. 1)
 *   logp_cols     M x ncols log-probabilities at the columns cols[]
 *   gamma_cols    M x ncols occupancies at the columns cols[]
 *   dX[M*D], dW[V*D], db[V]   gradients (dW and db are overwritten)
 * Utterances are processed one at a time; within one, the T_n x V logit
 * block is materialised in FP64 (the dense reference groups whole
 * utterances, App. B "accuracy" paragraph).
 */
static int pcx_batch(int N, int M, int D, int V, int blank, const double* X,
                     const double* W, const double* b, const int32_t* frame_counts,
                     const int32_t* tgt_off, const int32_t* tgt, double beam, double grad,
                     double* loss_out, double* utt_loss, int32_t* status, double* delta,
                     double* margin, double* lambda, int ncols, const int32_t* cols,
                     double* logp_cols, double* gamma_cols, double* dX, double* dW,
                     double* db) {
  if (N < 0 || M < 0 || D <= 0 || V <= 0 || blank < 0 || blank >= V)
    return ORACLE_ERR_ARG;
  long long sumT = 0;
  for (int n = 0; n < N; ++n) {
    if (frame_counts[n] <= 0) return ORACLE_ERR_LENGTHS;
    sumT += frame_counts[n];
  }
  if (sumT != M) return ORACLE_ERR_LENGTHS;
  if (tgt_off[0] != 0) return ORACLE_ERR_TARGET;
  for (int n = 0; n < N; ++n)
    if (tgt_off[n + 1] < tgt_off[n]) return ORACLE_ERR_TARGET;
  for (int i = 0; i < tgt_off[N]; ++i)
    if (tgt[i] < 0 || tgt[i] >= V || tgt[i] == blank) return ORACLE_ERR_TARGET;
  for (int c = 0; c < ncols; ++c)
    if (cols[c] < 0 || cols[c] >= V) return ORACLE_ERR_ARG;

  if (dW) memset(dW, 0, sizeof(double) * (size_t)V * D);
  if (db) memset(db, 0, sizeof(double) * (size_t)V);
  const int want_grad = (dX || dW || db || gamma_cols) ? 1 : 0;
  double total = 0.0;
  int row0 = 0;
  for (int n = 0; n < N; ++n) {
    const int T = frame_counts[n];
    const int L = tgt_off[n + 1] - tgt_off[n];
    const double* Xn = X + (size_t)row0 * D;
    double* Zn = (double*)malloc(sizeof(double) * (size_t)T * V);
    double* lam = (double*)malloc(sizeof(double) * (size_t)T);
    double* dZn = want_grad ? (double*)malloc(sizeof(double) * (size_t)T * V) : NULL;
    double* gam = gamma_cols ? (double*)malloc(sizeof(double) * (size_t)T * V) : NULL;
    if (!Zn || !lam || (want_grad && !dZn) || (gamma_cols && !gam)) {
      free(Zn); free(lam); free(dZn); free(gam);
      return ORACLE_ERR_NOMEM;
    }
    /* Z_n = X_n W^T + b, natural-order dot products (Sec. 3.1). */
#pragma omp parallel for collapse(2) schedule(static)
    for (int t = 0; t < T; ++t) {
      for (int v = 0; v < V; ++v) {
        const double* x = Xn + (size_t)t * D;
        const double* w = W + (size_t)v * D;
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += x[d] * w[d];
        Zn[(size_t)t * V + v] = acc + (b ? b[v] : 0.0);
      }
    }
    double loss_n = 0.0, full_n = 0.0, margin_n = INFINITY;
    int st = 0;
    int rc = beam == INFINITY
                 ? oracle_ctc_logits(T, V, blank, Zn, tgt + tgt_off[n], L, grad,
                                     &loss_n, &st, lam, dZn, gam)
                 : oracle_ctc_beam(T, V, blank, Zn, tgt + tgt_off[n], L, beam, grad,
                                   &loss_n, &st, &full_n, lam, dZn, gam, &margin_n);
    if (beam == INFINITY) full_n = st == 0 ? loss_n : NAN;
    if (rc != ORACLE_OK) {
      free(Zn); free(lam); free(dZn); free(gam);
      return rc;
    }
    if (utt_loss) utt_loss[n] = loss_n;
    if (status) status[n] = st;
    /* posterior mass of the discarded alignments, 1 - exp(-(L_beta - L)) */
    if (delta) delta[n] = st == 0 ? -expm1(-(loss_n - full_n)) : NAN;
    if (margin) margin[n] = margin_n;
    if (st == 0) total += loss_n;
    if (lambda) memcpy(lambda + row0, lam, sizeof(double) * (size_t)T);
    for (int t = 0; t < T; ++t) {
      for (int c = 0; c < ncols; ++c) {
        if (logp_cols)
          logp_cols[(size_t)(row0 + t) * ncols + c] =
              Zn[(size_t)t * V + cols[c]] - lam[t];
        if (gamma_cols)
          gamma_cols[(size_t)(row0 + t) * ncols + c] = gam[(size_t)t * V + cols[c]];
      }
    }
    /* dX_n = dZ_n W */
    if (dX) {
#pragma omp parallel for schedule(static)
      for (int t = 0; t < T; ++t) {
        double* dx = dX + (size_t)(row0 + t) * D;
        for (int d = 0; d < D; ++d) dx[d] = 0.0;
        for (int v = 0; v < V; ++v) {
          const double g = dZn[(size_t)t * V + v];
          const double* w = W + (size_t)v * D;
          for (int d = 0; d < D; ++d) dx[d] += g * w[d];
        }
      }
    }
    /* dW += dZ_n^T X_n,  db += column sums of dZ_n */
    if (dW || db) {
#pragma omp parallel for schedule(static)
      for (int v = 0; v < V; ++v) {
        for (int t = 0; t < T; ++t) {
          const double g = dZn[(size_t)t * V + v];
          if (db) db[v] += g;
          if (dW) {
            double* dw = dW + (size_t)v * D;
            const double* x = Xn + (size_t)t * D;
            for (int d = 0; d < D; ++d) dw[d] += g * x[d];
          }
        }
      }
    }
    free(Zn); free(lam); free(dZn); free(gam);
    row0 += T;
  }
  *loss_out = total;
  return ORACLE_OK;
}

int oracle_pcx(int N, int M, int D, int V, int blank, const double* X,
               const double* W, const double* b, const int32_t* frame_counts,
               const int32_t* tgt_off, const int32_t* tgt, double grad,
               double* loss_out, double* utt_loss, int32_t* status,
               double* lambda, int ncols, const int32_t* cols,
               double* logp_cols, double* gamma_cols, double* dX, double* dW,
               double* db) {
  return pcx_batch(N, M, D, V, blank, X, W, b, frame_counts, tgt_off, tgt, INFINITY, grad,
                   loss_out, utt_loss, status, NULL, NULL, lambda, ncols, cols, logp_cols,
                   gamma_cols, dX, dW, db);
}

/*
 * The whole path with the finite-beam objective L_beta (oracle_ctc_beam per
 * utterance; beam = INFINITY gives oracle_pcx).  Extra outputs (may be NULL):
 *   delta[N]   1 - exp(-(L_beta,n - L_n)), the posterior mass of the
 *              alignments the pruning discards (the pages' delta_n); NaN for
 *              excluded utterances
 *   margin[N]  per utterance, the distance of the nearest arc score from the
 *              pruning threshold (see oracle_ctc_beam)
 */
int oracle_pcx_beam(int N, int M, int D, int V, int blank, const double* X,
                    const double* W, const double* b, const int32_t* frame_counts,
                    const int32_t* tgt_off, const int32_t* tgt, double beam, double grad,
                    double* loss_out, double* utt_loss, int32_t* status, double* delta,
                    double* margin, double* lambda, int ncols, const int32_t* cols,
                    double* logp_cols, double* gamma_cols, double* dX, double* dW,
                    double* db) {
  if (!(beam >= 0.0)) return ORACLE_ERR_ARG;
  return pcx_batch(N, M, D, V, blank, X, W, b, frame_counts, tgt_off, tgt, beam, grad,
                   loss_out, utt_loss, status, delta, margin, lambda, ncols, cols, logp_cols,
                   gamma_cols, dX, dW, db);
}

/* Number of threads OpenMP will use for the parallel loops above. */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

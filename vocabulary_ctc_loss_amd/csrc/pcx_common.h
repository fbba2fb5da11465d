// Shared device helpers and kernel launchers of the pcx library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pcx {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// bf16 values travel as their 16-bit patterns.
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (NaNs stay NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// exp(s) of an fp32 log-probability s as m 2^n, to fp32 precision (the
// precision of s itself, an fp32 score): x = s log2(e) is formed as hi + lo
// (hi the fp32 product, lo its rounding error by a fused multiply-add plus
// s times the tail of log2(e)), n = rint(hi), and m = 2^((hi - n) + lo) by
// the hardware exp2 (hi - n is exact and |(hi - n) + lo| <= 1/2 + 2^-20, so
// m lies in [0.7, 1.42]); about 2^-22 relative error in all.  s below -1e6
// is taken as -1e6; a NaN stays NaN.
__device__ __forceinline__ float exp_split(float s, int& n) {
  constexpr float L2E_HI = 0x1.715476p+0f;   // fp32 log2(e)
  constexpr float L2E_LO = 0x1.4ae0c0p-26f;  // log2(e) - L2E_HI, rounded
  const float x = s < -1e6f ? -1e6f : s;
  const float hi = x * L2E_HI;
  const float lo = fmaf(x, L2E_HI, -hi) + x * L2E_LO;
  const float nf = rintf(hi);
  n = (int)nf;
  return __builtin_amdgcn_exp2f((hi - nf) + lo);
}

// exp(x) for x <= 0 in IEEE double (0 below the double range; branch-free).
// Cody-Waite reduction x = n ln2 + r with ln2 split into a 32-bit head (so
// n * head is exact) and a tail, |r| <= ln2 / 2, then the degree-13 Taylor
// polynomial of e^r (truncation < 1e-17 relative) and a scale by 2^n.
__device__ __forceinline__ double exp_nonpos(double x) {
  x = fmax(x, -746.0);  // -inf -> 0 through the underflowing scale below
  const double n = rint(x * 0x1.71547652b82fep+0);  // x / ln2
  double r = fma(-n, 0x1.62e42ff000000p-1, x);      // ln2 head
  r = fma(-n, -0x1.718432a1b0e26p-35, r);           // ln2 tail
  double p = 0x1.6124613a86d09p-33;                 // 1/13!
  p = fma(p, r, 0x1.1eed8eff8d898p-29);             // 1/12!
  p = fma(p, r, 0x1.ae64567f544e4p-26);             // 1/11!
  p = fma(p, r, 0x1.27e4fb7789f5cp-22);             // 1/10!
  p = fma(p, r, 0x1.71de3a556c734p-19);             // 1/9!
  p = fma(p, r, 0x1.a01a01a01a01ap-16);             // 1/8!
  p = fma(p, r, 0x1.a01a01a01a01ap-13);             // 1/7!
  p = fma(p, r, 0x1.6c16c16c16c17p-10);             // 1/6!
  p = fma(p, r, 0x1.1111111111111p-7);              // 1/5!
  p = fma(p, r, 0x1.5555555555555p-5);              // 1/4!
  p = fma(p, r, 0x1.5555555555555p-3);              // 1/3!
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  return ldexp(p, (int)n);
}

// Table entry j of exp_nonpos_tab: 2^(j/64) = 2 exp((j - 64) ln2 / 64),
// j = 0..63 (within one ulp).
__device__ __forceinline__ double exp_tab_entry(int j) {
  return 2.0 * exp_nonpos((double)(j - 64) * 0x1.62e42fefa39efp-7);
}

// exp(x) for x <= 0 in IEEE double with a 64-entry table of 2^(j/64):
// x = (64 q + j) ln2 / 64 + r with |r| <= ln2 / 128 (Cody-Waite, ln2 / 64
// split into head and tail), exp(x) = 2^q 2^(j/64) e^r, e^r by its degree-5
// Taylor polynomial (truncation < 4e-17 relative).  Within about 2 ulp over
// the normal range; 0 below it.  About half the double-precision operations
// of exp_nonpos.
__device__ __forceinline__ double exp_nonpos_tab(double x, const double* __restrict__ tab) {
  x = fmax(x, -746.0);
  const double kd = rint(x * 0x1.71547652b82fep+6);  // x * 64 / ln2
  double r = fma(-kd, 0x1.62e42ff000000p-7, x);      // ln2/64 head
  r = fma(-kd, -0x1.718432a1b0e26p-41, r);           // ln2/64 tail
  const int k = (int)kd;
  double p = 0x1.1111111111111p-7;                   // 1/5!
  p = fma(p, r, 0x1.5555555555555p-5);               // 1/4!
  p = fma(p, r, 0x1.5555555555555p-3);               // 1/3!
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  return ldexp(tab[k & 63] * p, k >> 6);
}

// Work-group barrier that orders LDS accesses only: the waves' outstanding
// global loads and stores are not waited for (a plain __syncthreads also
// drains them, which would expose prefetch and store latency).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int VEC = 4;  // elements per 16-byte vector
  __device__ static float to_f32(float x) { return x; }
  __device__ static float from_f32(float x) { return x; }
};
template <> struct Elem<bf16_t> {
  static constexpr int VEC = 8;
  __device__ static float to_f32(bf16_t x) { return bf16_to_f32(x); }
  __device__ static bf16_t from_f32(float x) { return f32_to_bf16(x); }
};

// Error bits raised by the validation kernels.
enum : int {
  ERRBIT_TARGET = 1,   // label out of range / blank in target / bad offsets
  ERRBIT_LENGTHS = 2,  // frame count <= 0 or sum != M
};

// Small device-resident summary read back by the host after selection and
// after the loss reduction.
struct Meta {
  int err;
  int K;
  int max_L;
  int max_T;
  long long dp_total;   // sum_n T_n * (2 L_n + 1)
  double loss;
  int n_unalignable;
  int n_nonfinite;
  int pad[2];
};

// Utterance status codes.
enum : int { UTT_OK = 0, UTT_UNALIGNABLE = 1, UTT_NONFINITE = 2 };

// Largest vocabulary span folded into one normalizer partial by the forward
// kernel (one work-group walks one span of one frame tile).
constexpr int LSE_SPAN_MAX = 2048;
// Most parts the frames are split into for a backward that wants dX alone
// (chunks are then taken in groups of as many).
constexpr int DX_PARTS = 2;

// ---------------------------------------------------------------- launchers
// Selection / validation (pcx_select.hip).
hipError_t launch_prepare(hipStream_t st, int N, int M, int V, int blank, long long L_tot,
                          const int* tgt_off, const int* tgt, const int* frame_counts,
                          int* row_off, uint8_t* flags, long long* dp_off,
                          int* col2sel, int* U, int* tgt_rel, Meta* meta);

// Whether a bf16 head runs on the 256 x 256 GEMM core: the forward needs a
// head dimension that is a multiple of 64 and 16-byte aligned X and W (so it
// does not depend on the chunk width); the backward products also need a
// chunk width that is a multiple of 64.
int use_big_fwd(int dtype, int D, const void* X, const void* W);
int use_big_core(int dtype, int D, int chunk, const void* X, const void* W);

// Forward head (pcx_gemm.hip).
// span0 / part_ld: the launch covers the 2048-class spans span0.. of a
// partial array with part_ld spans per frame (fp32 only; bf16: 0 / nspan).
// masked: the log-sum-exp partials cover the unselected classes only (the
// grouped form's other column); Zsel is written either way.
hipError_t launch_fwd_lse(hipStream_t st, int dtype, const void* X, const void* W,
                          const void* b, int M, int D, int V, const int* col2sel,
                          float* Zsel, double2* part, int nspan, int big, int span0,
                          int part_ld, int masked, int span);
// Span width of the forward for a head: the largest multiple of the kernel's
// tile rows, at most LSE_SPAN_MAX, that still gives about 2048 work-groups or
// more (small vocabularies get narrow spans, so the launch fills the chip).
// A function of the dtype, the core, M and V only.
int lse_span(int dtype, int big, int M, int V);
hipError_t launch_lambda(hipStream_t st, const double2* part, int M, int nspan,
                         double* lam, float* lamf);
// Grouped form: lambda from the K gathered logits and the other column.
hipError_t launch_lambda_grouped(hipStream_t st, const float* Zsel, const double* other, int K,
                                 int M, double* lam, float* lamf);
// Grouped backward: gu_m = g_m exp(o_m - lambda_m) and the fp32 shift
// ou_m = o_m (0 where the complement is empty).
hipError_t launch_grouped_rowscale(hipStream_t st, const double* g, const double* other,
                                   const double* lam, int M, double* gu, float* ou);
hipError_t launch_scores(hipStream_t st, float* S, const double* lam, int K, int M);

// Backward head (pcx_gemm.hip).
// The gradient reduction of one chunk: dW rows [row_base, row_base + rows)
// from the splitk split partials and db columns [col_base, col_base + cols)
// from the per-row-tile partials (leading dimension ld); either output may
// be NULL.  nb work-groups of 256 threads do it (the first nb_db the db
// columns); out_bf16: the outputs are bf16, else fp32.
struct ReduceJob {
  const float* part = nullptr;
  int splitk = 0, rows = 0, D = 0;
  void* dW = nullptr;
  long long row_base = 0;
  const float* dbpart = nullptr;
  int mtiles = 0, cols = 0, ld = 0;
  void* db = nullptr;
  long long col_base = 0;
  int nb_db = 0, nb = 0, vec4 = 0, out_bf16 = 0;
};
// max_wg: most work-groups for the dW part.
ReduceJob make_reduce_job(int dtype, const float* part, int splitk, int rows, int D, void* dW,
                          long long row_base, const float* dbpart, int mtiles, int cols, int ld,
                          void* db, long long col_base, int max_wg = 8192);
// rj (optional, fp32 and bf16 128-row cores only): a reduction appended to
// the launch as rj->nb extra work-groups after the tiles.  It must not touch
// what the recompute writes (the dZ block, dbpart).
hipError_t launch_recompute(hipStream_t st, int dtype, const void* X, const void* W,
                            const void* b, int M, int D, int c0, int c1,
                            const int* col2sel, const float* lamf, const double* g,
                            const float* S, const float* Gam, double grad,
                            void* dZ, int ldz, float* dbpart, int big,
                            const double* gu = nullptr, const float* ou = nullptr,
                            long long ldS = 0,  // S / Gamma leading dimension (0: M)
                            const int* cmap = nullptr, const void* Wg = nullptr,
                            const int* nu = nullptr, const ReduceJob* rj = nullptr);
// Unselected-first column order of the chunk [c0, c1) into cmap[0 ..] and
// *nu, and the head rows the recompute products read, gathered into Wg
// (the recompute's cmap / Wg; not for the 256 x 256 bf16 core).
hipError_t launch_colperm(hipStream_t st, int dtype, const int* col2sel, int c0, int c1,
                          const void* W, int D, int* cmap, int* nu, void* Wg);
// Columns of the recompute tile (of the cores that take a column order).
int rec_tile_cols(int dtype);
// wt: D x ldz scratch for the transposed weight chunk (bf16 only); with
// stage_wt == 0 it already holds these columns (an earlier call staged them).
// Rows of the recompute tile (one bias-gradient partial per row tile) and
// the number of output tiles of one dW product.
int rec_tile_rows(int dtype, int big);
int dw_tiles(int dtype, int C, int D);
// out_bf16 (256 x 256 core only, 8-byte aligned): the last product into
// these rows of the accumulator writes the bf16 result there instead.
hipError_t launch_dx(hipStream_t st, int dtype, const void* dZ, int ldz, const void* W,
                     int M, int D, int c0, int c1, float* dXacc, int first, void* wt, int big,
                     int stage_wt = 1, void* out_bf16 = nullptr);
hipError_t launch_dw(hipStream_t st, int dtype, const void* dZ, int ldz, const void* X,
                     int M, int D, int c0, int c1, float* part, int splitk);
// A gradient reduction as a launch of its own.
hipError_t launch_grad_reduce(hipStream_t st, const ReduceJob& rj);
hipError_t launch_cast_out(hipStream_t st, int dtype, const float* src, void* dst,
                           long long n);
// dst[i] = fp32(src[i]) for n bf16 values.
hipError_t launch_widen(hipStream_t st, const void* src, float* dst, long long n);

// Alignment DP (pcx_ctc.hip).
// Forward and backward recursions of every utterance in one launch.
// mode 0: sums over every transition, as scaled probabilities (am, ae: the
// forward values, emission included; bm, be: the backward values without
// the node's emission; utt_pm, utt_pe: the total per utterance);
// mode 1: the same over the arcs kept by a finite beam (mask: one byte per
// lattice node, from launch_beam_mask);
// mode 2: max-plus in the log domain (am <- best prefix scores, bm <- best
// suffix scores without the node's emission, best[n] <- best alignment
// score; ae, be, utt_* unused).
// fwd_only: the forward recursion alone (am may then be NULL: losses only).
hipError_t launch_alpha_beta(hipStream_t st, const float* S, int M, int N, int max_L,
                             const int* row_off, const int* tgt_off, const int* tgt_rel,
                             const uint8_t* flags, const long long* dp_off, double* am,
                             double* bm, double* utt_loss, double* utt_logp,
                             double* utt_pm, int* utt_pe, int* utt_status, int mode,
                             const uint8_t* mask, double* best, int fwd_only);
// Arc masks of a finite alignment beam from the max-plus scores.
hipError_t launch_beam_mask(hipStream_t st, const float* S, int M, int N, long long dp_total,
                            int max_T, int max_L, const int* row_off, const int* tgt_off, const int* tgt_rel,
                            const uint8_t* flags, const long long* dp_off, const double* vf,
                            const double* vb, const double* best, double beam, uint8_t* mask);
hipError_t launch_loss_sum(hipStream_t st, int N, const double* utt_loss,
                           const int* utt_status, Meta* meta);
hipError_t launch_occupancy(hipStream_t st, int M, int N, int max_T, int max_L,
                            const int* row_off, const int* tgt_off, const int* tgt_rel,
                            const int* utt_status, const double* utt_pm, const int* utt_pe,
                            const long long* dp_off, const double* am, const double* bm,
                            float* Gam, double* g);
// d_eta (device double) = grad * sum_m (g_m exp(S[0][m]) - Gamma[0][m]).
hipError_t launch_blank_grad(hipStream_t st, const float* S, const float* Gam, const double* g,
                             int M, double grad, double* out);
hipError_t launch_fill_f32(hipStream_t st, float* p, long long n, float v);
// Zero n elements of esz bytes each (esz 2 or 4; p aligned to esz).
hipError_t launch_fill_zero(hipStream_t st, void* p, long long n, int esz);

}  // namespace pcx

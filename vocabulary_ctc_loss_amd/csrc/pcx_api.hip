// C ABI of the pcx library: argument checks, the per-context workspace, the
// launch sequence of the forward and backward passes, optional per-kernel
// event timing, and the inspection getters.  Declarations: include/pcx.h.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/pcx.h"
#include "pcx_common.h"

using namespace pcx;

namespace {

thread_local std::string g_last_error;

pcx_status fail(pcx_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

#define PCX_HIP(call)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (call);                                                             \
    if (e_ != hipSuccess)                                                               \
      return fail(PCX_ERR_HIP, "%s failed: %s", #call, hipGetErrorString(e_));          \
  } while (0)

// A grow-only device buffer, with the stream it was allocated on (for a
// stream-ordered release through the caller's allocator).
struct DevBuf {
  void* p = nullptr;
  size_t cap = 0;
  hipStream_t st = nullptr;
};

// Kernel families timed by the optional event profiler.
enum Kid {
  K_PREPARE, K_FWD_LSE, K_LAMBDA, K_SCORES, K_ALPHA_BETA, K_LOSS, K_FILL, K_OCC,
  K_RECOMPUTE, K_DX, K_DW, K_REDUCE, K_CAST, K_BLANK, K_WIDEN, K_ROWSCALE, K_VITERBI,
  K_BEAM_MASK, K_COUNT
};
const char* kKidNames[K_COUNT] = {
    "prepare_select", "fwd_gemm_lse", "lambda", "scores", "ctc_alpha_beta", "loss_sum",
    "fill", "occupancy", "bwd_recompute_dz", "dx_gemm", "dw_gemm",
    "grad_reduce", "cast", "blank_offset_grad", "widen_head", "grouped_rowscale",
    "ctc_viterbi", "beam_mask"};

struct Pending {
  int kid;
  hipEvent_t a, b;
};

}  // namespace

struct pcx_ctx {
  // workspace
  DevBuf meta, row_off, flags, dp_off, col2sel, U, tgt_rel, tgt_off;
  DevBuf part, lam, lamf, S, alpha, beta, utt_loss, utt_logp, utt_status;
  DevBuf Gam, g, dZ, dXacc, dwpart, dbpart, wt, eta, w32, b32, other, gu, ou;
  DevBuf cmap, wg;  // selected-first column order of the recompute
  DevBuf arcmask, ubest, loss_full, logp_full, status_full;  // finite beam
  DevBuf utt_pm, utt_pe, pm_full, pe_full;   // scaled totals (mantissa, exponent)
  Meta* host_meta = nullptr;  // pinned
  // caller's allocator (both NULL: hipMalloc / hipFree)
  pcx_alloc_fn alloc = nullptr;
  pcx_free_fn release = nullptr;
  void* user = nullptr;
  // fixed workspace (the static-scratch entry point): buffers are carved in
  // order from [fixed_base, fixed_base + fixed_cap) and never released
  bool fixed = false;
  char* fixed_base = nullptr;
  size_t fixed_cap = 0, fixed_used = 0;
  // forward state kept for backward / getters
  bool fwd_ok = false;
  bool bwd_done = false;
  hipStream_t stream = nullptr;  // stream of the latest call
  bool stream_set = false;
  hipEvent_t handoff = nullptr;  // orders a call after the previous one's stream
  const void* X = nullptr;
  const void* W = nullptr;
  const void* b = nullptr;
  int dtype = 0;
  int form = PCX_FORM_DIRECT;      // for the next forward
  int fwd_form = PCX_FORM_DIRECT;  // of the last forward
  double beam = INFINITY;          // alignment beam of the next forward
  double fwd_beam = INFINITY;      // of the last forward
  int M = 0, D = 0, V = 0, N = 0, blank = 0, chunk = 1, K = 0, max_L = 0, max_T = 0;
  long long L_tot = 0, dp_total = 0;
  int nspan = 0;
  // profiling
  bool prof = false;
  uint32_t prof_mask = 0xFFFFFFFFu;  // bit i: kernel family i is timed
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;
  double prof_ms[K_COUNT] = {0};
  long long prof_n[K_COUNT] = {0};
};

namespace {

// Calls on one context run in call order even when they come on different
// streams: a call on another stream than the previous call's first makes its
// stream wait for everything issued so far on that one.  (Not while the new
// stream is being captured into a graph: a capture may not wait on work
// recorded outside it, and whoever captures orders the capture stream.)
pcx_status follow_last_call(pcx_ctx* c, hipStream_t st) {
  if (c->stream_set && c->stream != st) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    PCX_HIP(hipStreamIsCapturing(st, &cs));
    if (cs == hipStreamCaptureStatusNone) {
      if (!c->handoff) PCX_HIP(hipEventCreateWithFlags(&c->handoff, hipEventDisableTiming));
      PCX_HIP(hipEventRecord(c->handoff, c->stream));
      PCX_HIP(hipStreamWaitEvent(st, c->handoff, 0));
    }
  }
  c->stream = st;
  c->stream_set = true;
  return PCX_OK;
}

}  // namespace

namespace {

size_t total_bytes(const pcx_ctx* c) {
  const DevBuf* bufs[] = {&c->meta, &c->row_off, &c->flags, &c->dp_off, &c->col2sel, &c->U,
                          &c->tgt_rel, &c->tgt_off, &c->part, &c->lam, &c->lamf, &c->S, &c->alpha,
                          &c->beta, &c->utt_loss, &c->utt_logp, &c->utt_status, &c->Gam,
                          &c->g, &c->dZ, &c->dXacc, &c->dwpart, &c->dbpart, &c->wt, &c->eta,
                          &c->w32, &c->b32, &c->other, &c->gu, &c->ou, &c->arcmask, &c->ubest,
                          &c->loss_full, &c->logp_full, &c->status_full,
                          &c->utt_pm, &c->utt_pe, &c->pm_full, &c->pe_full,
                          &c->cmap, &c->wg};
  size_t t = 0;
  for (const DevBuf* b : bufs) t += b->cap;
  return t;
}

pcx_status ensure(pcx_ctx* c, DevBuf& b, size_t bytes, hipStream_t st) {
  if (bytes == 0) bytes = 16;
  if (b.cap >= bytes) return PCX_OK;
  if (c->fixed) {
    bytes = (bytes + 255) & ~size_t(255);
    if (bytes > c->fixed_cap - c->fixed_used)
      return fail(PCX_ERR_WORKSPACE,
                  "the call needs more workspace than the %zu-byte static scratch (%zu in use, "
                  "%zu more asked for); use pcx_forward / pcx_backward",
                  c->fixed_cap, c->fixed_used, bytes);
    b.p = c->fixed_base + c->fixed_used;
    b.cap = bytes;
    b.st = st;
    c->fixed_used += bytes;
    return PCX_OK;
  }
  {
    // a graph must not record an allocation or a release
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    PCX_HIP(hipStreamIsCapturing(st, &cs));
    if (cs != hipStreamCaptureStatusNone)
      return fail(PCX_ERR_WORKSPACE,
                  "the workspace would grow (%zu > %zu bytes) while the stream is being "
                  "captured; run one call of the same shapes before the capture",
                  bytes, b.cap);
  }
  if (b.p) {
    if (c->release) {
      // Every earlier call of this context is ordered before the work
      // already issued to st (the stream hand-off); released on its own
      // allocation stream, the buffer is then safe for that stream's later
      // work.  Released from another stream's call, wait for st first.
      if (b.st != st) PCX_HIP(hipStreamSynchronize(st));
      c->release(b.p, b.cap, c->user, (void*)b.st);
    } else {
      // the old buffer may still be read by work of an earlier call, possibly
      // on another stream: wait for the whole device before freeing it
      // (growth is rare; a sized workspace never gets here)
      PCX_HIP(hipDeviceSynchronize());
      PCX_HIP(hipFree(b.p));
    }
    b.p = nullptr;
    b.cap = 0;
  }
  bytes = (bytes + 255) & ~size_t(255);
  if (c->alloc) {
    b.p = c->alloc(bytes, c->user, (void*)st);
    if (!b.p) return fail(PCX_ERR_WORKSPACE, "the allocation callback returned NULL for %zu bytes", bytes);
  } else {
    hipError_t e = hipMalloc(&b.p, bytes);
    if (e != hipSuccess) {
      b.p = nullptr;
      return fail(PCX_ERR_HIP, "hipMalloc(%zu) failed: %s", bytes, hipGetErrorString(e));
    }
  }
  b.cap = bytes;
  b.st = st;
  return PCX_OK;
}

hipEvent_t take_event(pcx_ctx* c) {
  if (!c->pool.empty()) {
    hipEvent_t e = c->pool.back();
    c->pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Pending timing pairs past which a forward folds them into the totals.
constexpr size_t kMaxPendingTimed = 4096;

// Collect finished event pairs into the per-kernel totals.
void prof_drain(pcx_ctx* c) {
  for (Pending& p : c->pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
      c->prof_ms[p.kid] += ms;
      c->prof_n[p.kid] += 1;
    }
    c->pool.push_back(p.a);
    c->pool.push_back(p.b);
  }
  c->pending.clear();
}

// RAII bracket of one kernel launch with events on the launch stream.
struct Timed {
  pcx_ctx* c;
  int kid;
  hipStream_t st;
  hipEvent_t a = nullptr;
  Timed(pcx_ctx* c_, int kid_, hipStream_t st_) : c(c_), kid(kid_), st(st_) {
    if (c->prof && ((c->prof_mask >> kid) & 1u)) {
      a = take_event(c);
      if (a) (void)hipEventRecord(a, st);
    }
  }
  ~Timed() {
    if (c->prof && a) {
      hipEvent_t b = take_event(c);
      if (b) {
        (void)hipEventRecord(b, st);
        c->pending.push_back({kid, a, b});
      } else {
        c->pool.push_back(a);
      }
    }
  }
};

#define LAUNCH(kid, call)                                                          \
  do {                                                                             \
    hipError_t e_;                                                                 \
    {                                                                              \
      Timed t_(ctx, kid, st);                                                      \
      e_ = (call);                                                                 \
    }                                                                              \
    if (e_ != hipSuccess)                                                          \
      return fail(PCX_ERR_HIP, "%s launch failed: %s", kKidNames[kid],             \
                  hipGetErrorString(e_));                                          \
  } while (0)

#define ENSURE(buf, bytes)                                      \
  do {                                                          \
    pcx_status s_ = ensure(ctx, ctx->buf, (size_t)(bytes), st); \
    if (s_ != PCX_OK) return s_;                                \
  } while (0)

}  // namespace

// Static scratch of pcx_loss_grad_static: one copy per GPU, held until the
// process ends.  Host code uses the address hipGetSymbolAddress returns for
// the current device, never the symbol itself.
__device__ __align__(256) unsigned char scratch[PCX_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
Meta g_static_meta[kMaxDevices];  // host copy of the device summary, per GPU
}  // namespace

extern "C" {

const char* pcx_last_error(void) { return g_last_error.c_str(); }

pcx_status pcx_create(pcx_ctx** out_ctx, pcx_alloc_fn alloc, pcx_free_fn release, void* user) {
  g_last_error.clear();
  if (!out_ctx) return fail(PCX_ERR_ARG, "out_ctx is NULL");
  if ((alloc == nullptr) != (release == nullptr))
    return fail(PCX_ERR_ARG, "alloc and release callbacks must both be set or both be NULL");
  // No HIP call here: device and pinned memory are taken on first use.
  pcx_ctx* c = new (std::nothrow) pcx_ctx();
  if (!c) return fail(PCX_ERR_ARG, "out of host memory");
  c->alloc = alloc;
  c->release = release;
  c->user = user;
  *out_ctx = c;
  return PCX_OK;
}

void pcx_destroy(pcx_ctx* c) {
  if (!c) return;
  DevBuf* bufs[] = {&c->meta, &c->row_off, &c->flags, &c->dp_off, &c->col2sel, &c->U,
                    &c->tgt_rel, &c->tgt_off, &c->part, &c->lam, &c->lamf, &c->S, &c->alpha, &c->beta,
                    &c->utt_loss, &c->utt_logp, &c->utt_status, &c->Gam, &c->g, &c->dZ,
                    &c->dXacc, &c->dwpart, &c->dbpart, &c->wt, &c->eta, &c->w32, &c->b32,
                    &c->other, &c->gu, &c->ou, &c->arcmask, &c->ubest, &c->loss_full,
                    &c->logp_full, &c->status_full, &c->utt_pm, &c->utt_pe, &c->pm_full,
                    &c->pe_full, &c->cmap, &c->wg};
  if (c->release) {
    // every call of the context is ordered before the last call's stream
    // tail: once that has finished, nothing of ours touches the workspace
    if (c->stream_set) (void)hipStreamSynchronize(c->stream);
    for (DevBuf* b : bufs)
      if (b->p) c->release(b->p, b->cap, c->user, (void*)b->st);
  } else {
    if (c->host_meta || c->meta.p) (void)hipDeviceSynchronize();
    for (DevBuf* b : bufs)
      if (b->p) (void)hipFree(b->p);
  }
  for (Pending& p : c->pending) {
    (void)hipEventDestroy(p.a);
    (void)hipEventDestroy(p.b);
  }
  for (hipEvent_t e : c->pool) (void)hipEventDestroy(e);
  if (c->handoff) (void)hipEventDestroy(c->handoff);
  if (c->host_meta) (void)hipHostFree(c->host_meta);
  delete c;
}

pcx_status pcx_forward(pcx_ctx* ctx, const void* X, const void* W, const void* b, int32_t dtype,
                       int64_t M, int64_t D, int64_t V, int32_t N, const int32_t* tgt_off,
                       const int32_t* tgt, int64_t L_tot, const int32_t* frame_counts,
                       int32_t blank, int32_t chunk, void* stream, double* loss,
                       pcx_fwd_info* info) {
  g_last_error.clear();
  if (!ctx) return fail(PCX_ERR_ARG, "ctx is NULL");
  ctx->fwd_ok = false;
  ctx->bwd_done = false;
  if (dtype != PCX_F32 && dtype != PCX_BF16 && dtype != PCX_F32_BF16W)
    return fail(PCX_ERR_DTYPE, "dtype %d is not supported (fp32, bf16 or fp32 with a bf16 head)",
                (int)dtype);
  if (M < 0 || D < 1 || V < 1 || N < 0 || L_tot < 0)
    return fail(PCX_ERR_ARG, "bad sizes M=%lld D=%lld V=%lld N=%d L_tot=%lld", (long long)M,
                (long long)D, (long long)V, (int)N, (long long)L_tot);
  if (M > INT_MAX / 2 || D > INT_MAX / 2 || V > INT_MAX / 2 || L_tot > INT_MAX / 2)
    return fail(PCX_ERR_ARG, "sizes exceed the 32-bit index range");
  if (blank < 0 || blank >= V) return fail(PCX_ERR_ARG, "blank %d outside [0, V)", (int)blank);
  if (chunk < 1) return fail(PCX_ERR_ARG, "chunk must be >= 1");
  if (!tgt_off) return fail(PCX_ERR_ARG, "tgt_off is NULL");
  if (N > 0 && !frame_counts) return fail(PCX_ERR_ARG, "frame_counts is NULL");
  if (L_tot > 0 && !tgt) return fail(PCX_ERR_ARG, "tgt is NULL");
  if (M > 0 && (!X || !W)) return fail(PCX_ERR_ARG, "X / W is NULL");
  hipStream_t st = (hipStream_t)stream;
  {
    const pcx_status s_ = follow_last_call(ctx, st);
    if (s_ != PCX_OK) return s_;
  }
  const int iM = (int)M, iD = (int)D, iV = (int)V;
  if (!ctx->host_meta) {
    hipError_t e = hipHostMalloc((void**)&ctx->host_meta, sizeof(Meta), hipHostMallocDefault);
    if (e != hipSuccess) {
      ctx->host_meta = nullptr;
      return fail(PCX_ERR_HIP, "hipHostMalloc failed: %s", hipGetErrorString(e));
    }
  }

  ENSURE(meta, sizeof(Meta));
  ENSURE(row_off, (N + 1) * sizeof(int));
  ENSURE(flags, (N + 1) * sizeof(uint8_t));
  ENSURE(dp_off, (N + 1) * sizeof(long long));
  ENSURE(col2sel, (size_t)V * sizeof(int));
  const long long Ucap = (L_tot + 1 < V) ? L_tot + 1 : V;
  ENSURE(U, Ucap * sizeof(int));
  ENSURE(tgt_rel, (L_tot + 1) * sizeof(int));
  ENSURE(tgt_off, (N + 1) * sizeof(int));
  Meta* dmeta = (Meta*)ctx->meta.p;
  // The context keeps its own copy of the offsets for the backward pass.
  PCX_HIP(hipMemcpyAsync(ctx->tgt_off.p, tgt_off, (N + 1) * sizeof(int), hipMemcpyDeviceToDevice,
                         st));

  LAUNCH(K_PREPARE, launch_prepare(st, N, iM, iV, blank, L_tot, tgt_off, tgt, frame_counts,
                                   (int*)ctx->row_off.p, (uint8_t*)ctx->flags.p,
                                   (long long*)ctx->dp_off.p, (int*)ctx->col2sel.p,
                                   (int*)ctx->U.p, (int*)ctx->tgt_rel.p, dmeta));
  PCX_HIP(hipMemcpyAsync(ctx->host_meta, dmeta, sizeof(Meta), hipMemcpyDeviceToHost, st));
  PCX_HIP(hipStreamSynchronize(st));
  // everything recorded so far on this stream has finished: past a few
  // thousand pending timing events (nobody is reading them), fold them into
  // the totals here, so that they stay bounded
  if (ctx->pending.size() > kMaxPendingTimed) prof_drain(ctx);
  const Meta hm = *ctx->host_meta;
  if (hm.err & ERRBIT_LENGTHS)
    return fail(PCX_ERR_LENGTHS, "frame counts must be positive and sum to M=%d", iM);
  if (hm.err & ERRBIT_TARGET)
    return fail(PCX_ERR_TARGET,
                "targets invalid: labels must lie in [0, V) without blank and offsets must be "
                "monotone from 0 to L_tot");
  if (hm.max_L > PCX_MAX_TARGET_LEN)
    return fail(PCX_ERR_LIMIT, "target of %d labels exceeds the supported %d", hm.max_L,
                PCX_MAX_TARGET_LEN);
  const int K = hm.K;
  ctx->K = K;
  ctx->max_L = hm.max_L;
  ctx->max_T = hm.max_T;
  ctx->dp_total = hm.dp_total;

  const int big = (M > 0 && dtype != PCX_F32_BF16W) ? use_big_fwd(dtype, iD, X, W) : 0;
  const int span = lse_span(dtype, big, iM, iV);
  const int nspan = (iV + span - 1) / span;
  ctx->nspan = nspan;
  // Grouped form: the projection's log-sum-exp covers the unselected classes
  // only, giving the other column o; lambda then comes from [Z[:, U], o].
  const int grouped = ctx->form == PCX_FORM_GROUPED;
  if (grouped) ENSURE(other, (size_t)M * sizeof(double));
  ENSURE(part, (size_t)M * nspan * sizeof(double2));
  ENSURE(lam, (size_t)M * sizeof(double));
  ENSURE(lamf, (size_t)M * sizeof(float));
  ENSURE(S, (size_t)K * M * sizeof(float));
  // 8 bytes per lattice node each: FP64 max-plus scores (finite beam), then
  // the sums as fp32 mantissa + int32 exponent
  ENSURE(alpha, (size_t)hm.dp_total * sizeof(double));
  ENSURE(beta, (size_t)hm.dp_total * sizeof(double));
  ENSURE(utt_pm, (size_t)(N + 1) * sizeof(double));
  ENSURE(utt_pe, (size_t)(N + 1) * sizeof(int));
  ENSURE(utt_loss, (size_t)(N + 1) * sizeof(double));
  ENSURE(utt_logp, (size_t)(N + 1) * sizeof(double));
  ENSURE(utt_status, (size_t)(N + 1) * sizeof(int));

  if (M > 0 && dtype == PCX_F32_BF16W) {
    // fp32 projection of a bf16 head: whole spans of W (about C rows)
    // widened to fp32 at a time.
    const int eff_chunk = chunk < iV ? chunk : iV;
    const int fspans = eff_chunk / span > 1 ? eff_chunk / span : 1;
    const int Cf = fspans * span;
    ENSURE(w32, (size_t)Cf * D * sizeof(float));
    if (b) ENSURE(b32, (size_t)Cf * sizeof(float));
    for (int c0 = 0; c0 < iV; c0 += Cf) {
      const int c1 = (c0 + Cf < iV) ? c0 + Cf : iV;
      LAUNCH(K_WIDEN, launch_widen(st, (const uint16_t*)W + (long long)c0 * D, (float*)ctx->w32.p,
                                   (long long)(c1 - c0) * D));
      if (b)
        LAUNCH(K_WIDEN, launch_widen(st, (const uint16_t*)b + c0, (float*)ctx->b32.p, c1 - c0));
      LAUNCH(K_FWD_LSE, launch_fwd_lse(st, PCX_F32, X, ctx->w32.p, b ? ctx->b32.p : nullptr, iM,
                                       iD, c1 - c0, (const int*)ctx->col2sel.p + c0,
                                       (float*)ctx->S.p, (double2*)ctx->part.p,
                                       (c1 - c0 + span - 1) / span, 0, c0 / span, nspan,
                                       grouped, span));
    }
  } else if (M > 0) {
    LAUNCH(K_FWD_LSE, launch_fwd_lse(st, dtype, X, W, b, iM, iD, iV, (const int*)ctx->col2sel.p,
                                     (float*)ctx->S.p, (double2*)ctx->part.p, nspan, big, 0,
                                     nspan, grouped, span));
  }
  if (M > 0) {
    LAUNCH(K_LAMBDA, launch_lambda(st, (const double2*)ctx->part.p, iM, nspan,
                                   grouped ? (double*)ctx->other.p : (double*)ctx->lam.p,
                                   (float*)ctx->lamf.p));
    if (grouped)
      LAUNCH(K_LAMBDA, launch_lambda_grouped(st, (const float*)ctx->S.p,
                                             (const double*)ctx->other.p, K, iM,
                                             (double*)ctx->lam.p, (float*)ctx->lamf.p));
    LAUNCH(K_SCORES, launch_scores(st, (float*)ctx->S.p, (const double*)ctx->lam.p, K, iM));
  }
  // A finite alignment beam: best prefix / suffix scores (max-plus, into
  // the alpha / beta buffers), then the kept-arc masks; the recursions
  // below then run over the kept arcs only.
  const bool pruned = !isinf(ctx->beam);
  if (pruned) {
    ENSURE(arcmask, (size_t)hm.dp_total);
    ENSURE(ubest, (size_t)(N + 1) * sizeof(double));
    LAUNCH(K_VITERBI,
           launch_alpha_beta(st, (const float*)ctx->S.p, iM, N, hm.max_L,
                             (const int*)ctx->row_off.p, (const int*)ctx->tgt_off.p,
                             (const int*)ctx->tgt_rel.p, (const uint8_t*)ctx->flags.p,
                             (const long long*)ctx->dp_off.p, (double*)ctx->alpha.p,
                             (double*)ctx->beta.p, nullptr, nullptr, nullptr, nullptr,
                             nullptr, 2, nullptr, (double*)ctx->ubest.p, 0));
    LAUNCH(K_BEAM_MASK,
           launch_beam_mask(st, (const float*)ctx->S.p, iM, N, hm.dp_total, hm.max_T, hm.max_L,
                            (const int*)ctx->row_off.p, (const int*)ctx->tgt_off.p,
                            (const int*)ctx->tgt_rel.p, (const uint8_t*)ctx->flags.p,
                            (const long long*)ctx->dp_off.p, (const double*)ctx->alpha.p,
                            (const double*)ctx->beta.p, (const double*)ctx->ubest.p,
                            ctx->beam, (uint8_t*)ctx->arcmask.p));
  }
  // The backward recursion runs here too, beside the forward one (it only
  // reads S): on the otherwise idle compute units it costs no extra time.
  LAUNCH(K_ALPHA_BETA,
         launch_alpha_beta(st, (const float*)ctx->S.p, iM, N, hm.max_L,
                           (const int*)ctx->row_off.p, (const int*)ctx->tgt_off.p,
                           (const int*)ctx->tgt_rel.p, (const uint8_t*)ctx->flags.p,
                           (const long long*)ctx->dp_off.p, (double*)ctx->alpha.p,
                           (double*)ctx->beta.p, (double*)ctx->utt_loss.p,
                           (double*)ctx->utt_logp.p,
                           (double*)ctx->utt_pm.p, (int*)ctx->utt_pe.p,
                           (int*)ctx->utt_status.p, pruned ? 1 : 0,
                           pruned ? (const uint8_t*)ctx->arcmask.p : nullptr, nullptr, 0));
  LAUNCH(K_LOSS, launch_loss_sum(st, N, (const double*)ctx->utt_loss.p,
                                 (const int*)ctx->utt_status.p, dmeta));
  PCX_HIP(hipMemcpyAsync(ctx->host_meta, dmeta, sizeof(Meta), hipMemcpyDeviceToHost, st));
  PCX_HIP(hipStreamSynchronize(st));
  const Meta fm = *ctx->host_meta;

  ctx->X = X;
  ctx->W = W;
  ctx->b = b;
  ctx->dtype = dtype;
  ctx->fwd_form = grouped ? PCX_FORM_GROUPED : PCX_FORM_DIRECT;
  ctx->fwd_beam = ctx->beam;
  ctx->M = iM;
  ctx->D = iD;
  ctx->V = iV;
  ctx->N = N;
  ctx->blank = blank;
  ctx->chunk = chunk < iV ? chunk : iV;
  ctx->L_tot = L_tot;
  ctx->fwd_ok = true;
  if (loss) *loss = fm.loss;
  if (info) {
    info->K = K;
    info->n_unalignable = fm.n_unalignable;
    info->n_nonfinite = fm.n_nonfinite;
    info->max_target_len = hm.max_L;
    info->workspace_bytes = total_bytes(ctx);
    info->lse_spans = nspan;
  }
  return PCX_OK;
}

// Occupancies Gamma on U and their row sums g for the last forward pass
// (they need the backward recursion, run during the forward call).
static pcx_status run_occupancy(pcx_ctx* ctx, hipStream_t st) {
  const int M = ctx->M, N = ctx->N, K = ctx->K;
  ENSURE(Gam, (size_t)K * M * sizeof(float));
  ENSURE(g, (size_t)M * sizeof(double));
  LAUNCH(K_FILL, launch_fill_f32(st, (float*)ctx->Gam.p, (long long)K * M, 0.f));
  LAUNCH(K_OCC, launch_occupancy(st, M, N, ctx->max_T, ctx->max_L, (const int*)ctx->row_off.p,
                                 (const int*)ctx->tgt_off.p, (const int*)ctx->tgt_rel.p,
                                 (const int*)ctx->utt_status.p, (const double*)ctx->utt_pm.p,
                                 (const int*)ctx->utt_pe.p, (const long long*)ctx->dp_off.p,
                                 (const double*)ctx->alpha.p, (const double*)ctx->beta.p,
                                 (float*)ctx->Gam.p, (double*)ctx->g.p));
  return PCX_OK;
}

pcx_status pcx_blank_offset_grad(pcx_ctx* ctx, double grad_loss, double* d_eta, void* stream) {
  g_last_error.clear();
  if (!ctx) return fail(PCX_ERR_ARG, "ctx is NULL");
  if (!d_eta) return fail(PCX_ERR_ARG, "d_eta is NULL");
  if (!ctx->fwd_ok) return fail(PCX_ERR_STATE, "pcx_blank_offset_grad needs a successful pcx_forward");
  hipStream_t st = (hipStream_t)stream;
  {
    const pcx_status s_ = follow_last_call(ctx, st);
    if (s_ != PCX_OK) return s_;
  }
  if (ctx->M == 0) {
    *d_eta = 0.0;
    return PCX_OK;
  }
  {
    const pcx_status s_ = run_occupancy(ctx, st);
    if (s_ != PCX_OK) return s_;
  }
  ENSURE(eta, sizeof(double));
  LAUNCH(K_BLANK, launch_blank_grad(st, (const float*)ctx->S.p, (const float*)ctx->Gam.p,
                                    (const double*)ctx->g.p, ctx->M, grad_loss,
                                    (double*)ctx->eta.p));
  PCX_HIP(hipStreamSynchronize(st));
  PCX_HIP(hipMemcpy(d_eta, ctx->eta.p, sizeof(double), hipMemcpyDeviceToHost));
  return PCX_OK;
}

pcx_status pcx_backward(pcx_ctx* ctx, double grad_loss, void* dX, void* dW, void* db,
                        void* stream) {
  g_last_error.clear();
  if (!ctx) return fail(PCX_ERR_ARG, "ctx is NULL");
  if (!ctx->fwd_ok) return fail(PCX_ERR_STATE, "pcx_backward needs a successful pcx_forward");
  hipStream_t st = (hipStream_t)stream;
  {
    const pcx_status s_ = follow_last_call(ctx, st);
    if (s_ != PCX_OK) return s_;
  }
  const int M = ctx->M, D = ctx->D, V = ctx->V, dt = ctx->dtype;
  const int C = ctx->chunk;
  // compute dtype of the products, and dtype of the head-shaped outputs
  const bool widen = dt == PCX_F32_BF16W;
  const int cdt = widen ? PCX_F32 : dt;
  const int wdt = widen ? PCX_BF16 : dt;
  const size_t esz = cdt == PCX_F32 ? 4 : 2;
  const size_t wesz = wdt == PCX_F32 ? 4 : 2;
  if (!dX && !dW && !db) return PCX_OK;
  if (M == 0) {
    // No frames: every head gradient is zero (a fill kernel, not a memset
    // node, so that the call can be captured into a graph).
    if (dW) LAUNCH(K_FILL, launch_fill_zero(st, dW, (long long)V * D, (int)wesz));
    if (db) LAUNCH(K_FILL, launch_fill_zero(st, db, V, (int)wesz));
    return PCX_OK;
  }
  const float* S = (const float*)ctx->S.p;

  {
    const pcx_status s_ = run_occupancy(ctx, st);
    if (s_ != PCX_OK) return s_;
  }

  // Grouped form: the unselected classes take the other column's gradient
  // through the log-sum-exp that formed it.
  const double* gu = nullptr;
  const float* ou = nullptr;
  if (ctx->fwd_form == PCX_FORM_GROUPED) {
    ENSURE(gu, (size_t)M * sizeof(double));
    ENSURE(ou, (size_t)M * sizeof(float));
    LAUNCH(K_ROWSCALE, launch_grouped_rowscale(st, (const double*)ctx->g.p,
                                               (const double*)ctx->other.p,
                                               (const double*)ctx->lam.p, M,
                                               (double*)ctx->gu.p, (float*)ctx->ou.p));
    gu = (const double*)ctx->gu.p;
    ou = (const float*)ctx->ou.p;
  }

  const int big = use_big_core(cdt, D, C, ctx->X, ctx->W);
  const int rtile = rec_tile_rows(cdt, big);
  const int nchunks = (V + C - 1) / C;
  // dX only: the frames are taken in G parts and the chunks in groups of G.
  // A part's dZ block is (part rows) x G C, the same M x C elements, and each
  // dX product reduces over G C columns, so the fp32 dX accumulator is read
  // and written once per group of chunks instead of once per chunk.  (dW
  // and db need every frame of a chunk in one block.)
  int G = 1;
  if (dX && !dW && !db)
    while (G < DX_PARTS && nchunks >= 2 * G && M >= 2 * G * rtile) G *= 2;
  const int CG = G * C;  // columns per group
  // Width (and leading dimension) of the group blocks: the group's columns,
  // or the whole vocabulary rounded up to 64 when that is narrower (a small
  // vocabulary in one wide chunk); the 256 x 256 core's zero padding of a
  // group to a multiple of 64 columns still fits.
  const int V64 = (V + 63) / 64 * 64;
  const int LZ = CG < V64 ? CG : V64;
  // rows per part: whole row tiles, so that every part starts on a tile
  const int Mh = G == 1 ? M : ((M + G - 1) / G + rtile - 1) / rtile * rtile;
  const int mtiles = (Mh + rtile - 1) / rtile;  // row tiles of the largest part
  // The gradient reduction of a chunk runs inside the next chunk's recompute
  // launch, as work-groups appended after its tiles (the launch's last,
  // partial wave of tiles leaves CUs free for them); the last chunk's runs as
  // a launch of its own.  The bias partials then alternate between two
  // halves of dbpart, so that a recompute never writes the half its appended
  // reduction reads.  (The 256 x 256 core keeps a launch per reduction.)
  const bool fuse = !big && (dW || db) && G == 1;
  const size_t dbhalf = (size_t)mtiles * LZ;
  ENSURE(dZ, (size_t)Mh * LZ * esz);
  ENSURE(dbpart, (fuse ? 2 : 1) * dbhalf * sizeof(float));
  float* dxacc = nullptr;
  if (dX) {
    if (cdt == PCX_F32) {
      dxacc = (float*)dX;
    } else {
      ENSURE(dXacc, (size_t)M * D * sizeof(float));
      ENSURE(wt, (size_t)D * LZ * esz);
      dxacc = (float*)ctx->dXacc.p;
    }
  }
  if (widen) {
    ENSURE(w32, (size_t)LZ * D * sizeof(float));
    if (ctx->b) ENSURE(b32, (size_t)LZ * sizeof(float));
  }
  // Split of the frame reduction of dW: enough work-groups to fill the chip,
  // at least 1024 frames per split; fixed for a given shape.  (512 frames
  // per split, 64 instead of 48 splits at V = 500, measured no faster.)
  const int Cw = C < V ? C : V;  // widest chunk
  const int wtiles = dw_tiles(cdt, Cw, D);
  int splitk = (1024 + wtiles - 1) / wtiles;
  const int maxsplit = (M + 1023) / 1024;
  if (splitk > maxsplit) splitk = maxsplit;
  if (splitk < 1) splitk = 1;
  if (dW) ENSURE(dwpart, (size_t)splitk * Cw * D * sizeof(float));

  // Where a chunk group can be expected to hold a tile's worth of selected
  // classes or more and at least a quarter of the classes are selected (K
  // close to V: small vocabularies), the recompute walks each group's columns
  // unselected-first, so that the selected classes fill whole tiles whose
  // product is skipped; its products then read the head rows they need
  // gathered into wg (which costs a copy of the unselected rows, hence the
  // quarter).  (Not on the 256 x 256 bf16 core.)
  const int Cg = CG < V ? CG : V;
  const bool order = !big && (long long)ctx->K * Cg >= (long long)V * rec_tile_cols(cdt) &&
                     4LL * ctx->K >= (long long)V;
  if (order) {
    ENSURE(cmap, ((size_t)LZ + 1) * sizeof(int));
    ENSURE(wg, (size_t)LZ * D * esz);
  }
  int* cmap = order ? (int*)ctx->cmap.p : nullptr;

  const int ngroups = (V + CG - 1) / CG;
  // bf16 dX on the 256 x 256 core: the last product into each row's
  // accumulator writes the bf16 result itself (no separate cast pass)
  const bool cast_in_dx = dX && cdt != PCX_F32 && big && ((uintptr_t)dX & 7u) == 0;
  ReduceJob pend;  // a chunk's reduction still to run (nb == 0: none)
  for (int gi = 0; gi < ngroups; ++gi) {
    float* dbp = (float*)ctx->dbpart.p + (fuse ? (size_t)(gi & 1) * dbhalf : 0);
    const int c0 = gi * CG, c1 = (c0 + CG < V) ? c0 + CG : V, Cc = c1 - c0;
    // The products see the group's head rows as rows [w0, w0 + Cc) of Wk
    // (the head itself, or its fp32 copy for a bf16-stored head).
    const void* Wk = ctx->W;
    const void* bk = ctx->b;
    const int* sel = (const int*)ctx->col2sel.p;
    int w0 = c0;
    if (widen) {
      LAUNCH(K_WIDEN, launch_widen(st, (const uint16_t*)ctx->W + (long long)c0 * D,
                                   (float*)ctx->w32.p, (long long)Cc * D));
      if (ctx->b)
        LAUNCH(K_WIDEN, launch_widen(st, (const uint16_t*)ctx->b + c0, (float*)ctx->b32.p, Cc));
      Wk = ctx->w32.p;
      bk = ctx->b ? ctx->b32.p : nullptr;
      sel += c0;
      w0 = 0;
    }
    if (order)
      LAUNCH(K_RECOMPUTE, launch_colperm(st, cdt, sel, w0, w0 + Cc, Wk, D, cmap, cmap + LZ,
                                         ctx->wg.p));
    for (int part = 0; part < G; ++part) {
      // frames [r0, r0 + Mp); S and Gamma keep their leading dimension M
      const int r0 = part * Mh;
      const int Mp = (r0 + Mh < M ? r0 + Mh : M) - r0;
      if (Mp <= 0) continue;
      LAUNCH(K_RECOMPUTE,
             launch_recompute(st, cdt, (const char*)ctx->X + (size_t)r0 * D * esz, Wk, bk, Mp,
                              D, w0, w0 + Cc, sel, (const float*)ctx->lamf.p + r0,
                              (const double*)ctx->g.p + r0, S + r0,
                              (const float*)ctx->Gam.p + r0, grad_loss, ctx->dZ.p, LZ, dbp,
                              big, gu ? gu + r0 : nullptr, ou ? ou + r0 : nullptr, M, cmap,
                              order ? ctx->wg.p : nullptr, order ? cmap + LZ : nullptr,
                              fuse ? &pend : nullptr));
      pend = ReduceJob{};
      if (dX)
        LAUNCH(K_DX, launch_dx(st, cdt, ctx->dZ.p, LZ, Wk, Mp, D, w0, w0 + Cc,
                               dxacc + (size_t)r0 * D, gi == 0, ctx->wt.p, big, part == 0,
                               cast_in_dx && gi == ngroups - 1
                                   ? (void*)((char*)dX + (size_t)r0 * D * esz)
                                   : nullptr));
      // dW and db are only wanted with G == 1: this part is all M frames
      if (dW)
        LAUNCH(K_DW, launch_dw(st, cdt, ctx->dZ.p, LZ, ctx->X, M, D, w0, w0 + Cc,
                               (float*)ctx->dwpart.p, splitk));
      if (dW || db) {
        // Appended to a recompute launch, its work-groups reserve the
        // recompute's LDS and registers (three per CU), so the dW part takes
        // 256 of them, each thread summing several elements (measured against
        // 128, 512 and 2304: 128 and 256 best).
        const ReduceJob rj = make_reduce_job(wdt, (const float*)ctx->dwpart.p, splitk, Cc, D, dW,
                                             c0, dbp, mtiles, Cc, LZ, db, c0,
                                             fuse ? 256 : 8192);
        if (fuse)
          pend = rj;
        else
          LAUNCH(K_REDUCE, launch_grad_reduce(st, rj));
      }
    }
  }
  if (pend.nb > 0) LAUNCH(K_REDUCE, launch_grad_reduce(st, pend));
  if (dX && cdt != PCX_F32 && !cast_in_dx)
    LAUNCH(K_CAST, launch_cast_out(st, cdt, dxacc, dX, (long long)M * D));
  ctx->bwd_done = true;
  return PCX_OK;
}

pcx_status pcx_loss_grad_static(const void* X, const void* W, const void* b, int32_t dtype,
                                int64_t M, int64_t D, int64_t V, int32_t N,
                                const int32_t* tgt_off, const int32_t* tgt, int64_t L_tot,
                                const int32_t* frame_counts, int32_t blank, int32_t chunk,
                                double grad_loss, void* dX, void* dW, void* db, void* stream,
                                double* loss, pcx_fwd_info* info) {
  g_last_error.clear();
  int dev = 0;
  PCX_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(PCX_ERR_ARG, "device %d out of range", dev);
  void* base = nullptr;
  {
    // once per device, with that device current: the device address of its
    // copy of the scratch array
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr)
        return fail(PCX_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
      g_scratch_ptr[dev] = p;
    }
    base = g_scratch_ptr[dev];
  }
  // A context on the stack whose workspace is carved from the scratch; its
  // host summary lives in static host memory.  It owns no allocation, so it
  // is simply dropped at the end.
  pcx_ctx c;
  c.fixed = true;
  c.fixed_base = (char*)base;
  c.fixed_cap = PCX_STATIC_SCRATCH_BYTES;
  c.host_meta = &g_static_meta[dev];
  pcx_status s = pcx_forward(&c, X, W, b, dtype, M, D, V, N, tgt_off, tgt, L_tot, frame_counts,
                             blank, chunk, stream, loss, info);
  if (s == PCX_OK) s = pcx_backward(&c, grad_loss, dX, dW, db, stream);
  if (s == PCX_OK && info) info->workspace_bytes = c.fixed_used;
  c.host_meta = nullptr;
  return s;
}

pcx_status pcx_set_beam(pcx_ctx* ctx, double beam) {
  g_last_error.clear();
  if (!ctx) return fail(PCX_ERR_ARG, "ctx is NULL");
  if (!(beam >= 0.0)) return fail(PCX_ERR_ARG, "the alignment beam must be >= 0 (or +inf)");
  ctx->beam = beam;
  return PCX_OK;
}

pcx_status pcx_get_discarded_mass(pcx_ctx* ctx, double* out, int64_t capacity) {
  g_last_error.clear();
  if (!ctx) return fail(PCX_ERR_ARG, "ctx is NULL");
  if (!ctx->fwd_ok) return fail(PCX_ERR_STATE, "no completed forward pass");
  const int N = ctx->N;
  if (!out || capacity < N)
    return fail(PCX_ERR_ARG, "output buffer too small (%lld < %d)", (long long)capacity, N);
  if (N == 0) return PCX_OK;
  hipStream_t st = ctx->stream;
  std::vector<double> lb(N), lf(N, 0.0);
  std::vector<int> sb(N), sf(N, UTT_OK);
  if (!isinf(ctx->fwd_beam)) {
    // the unpruned losses of the same scores: the forward recursion alone,
    // nothing stored but the losses
    ENSURE(loss_full, (size_t)(N + 1) * sizeof(double));
    ENSURE(logp_full, (size_t)(N + 1) * sizeof(double));
    ENSURE(status_full, (size_t)(N + 1) * sizeof(int));
    ENSURE(pm_full, (size_t)(N + 1) * sizeof(double));
    ENSURE(pe_full, (size_t)(N + 1) * sizeof(int));
    LAUNCH(K_ALPHA_BETA,
           launch_alpha_beta(st, (const float*)ctx->S.p, ctx->M, N, ctx->max_L,
                             (const int*)ctx->row_off.p, (const int*)ctx->tgt_off.p,
                             (const int*)ctx->tgt_rel.p, (const uint8_t*)ctx->flags.p,
                             (const long long*)ctx->dp_off.p, nullptr, nullptr,
                             (double*)ctx->loss_full.p, (double*)ctx->logp_full.p,
                             (double*)ctx->pm_full.p, (int*)ctx->pe_full.p,
                             (int*)ctx->status_full.p, 0, nullptr, nullptr, 1));
  }
  PCX_HIP(hipStreamSynchronize(st));
  PCX_HIP(hipMemcpy(lb.data(), ctx->utt_loss.p, N * sizeof(double), hipMemcpyDeviceToHost));
  PCX_HIP(hipMemcpy(sb.data(), ctx->utt_status.p, N * sizeof(int), hipMemcpyDeviceToHost));
  if (!isinf(ctx->fwd_beam)) {
    PCX_HIP(hipMemcpy(lf.data(), ctx->loss_full.p, N * sizeof(double), hipMemcpyDeviceToHost));
    PCX_HIP(hipMemcpy(sf.data(), ctx->status_full.p, N * sizeof(int), hipMemcpyDeviceToHost));
  } else {
    lf = lb;
  }
  for (int n = 0; n < N; ++n)
    out[n] = (sb[n] == UTT_OK && sf[n] == UTT_OK) ? -expm1(-(lb[n] - lf[n])) : NAN;
  return PCX_OK;
}

pcx_status pcx_set_formulation(pcx_ctx* ctx, int32_t form) {
  g_last_error.clear();
  if (!ctx) return fail(PCX_ERR_ARG, "ctx is NULL");
  if (form != PCX_FORM_DIRECT && form != PCX_FORM_GROUPED)
    return fail(PCX_ERR_ARG, "formulation %d is not supported (direct or grouped)", (int)form);
  ctx->form = form;
  return PCX_OK;
}

// ------------------------------------------------------------- profiling
pcx_status pcx_profile_enable(pcx_ctx* ctx, int32_t on) {
  if (!ctx) return fail(PCX_ERR_ARG, "ctx is NULL");
  ctx->prof = on != 0;
  return PCX_OK;
}

pcx_status pcx_profile_mask(pcx_ctx* ctx, uint32_t mask) {
  if (!ctx) return fail(PCX_ERR_ARG, "ctx is NULL");
  ctx->prof_mask = mask;
  return PCX_OK;
}

pcx_status pcx_profile_reset(pcx_ctx* ctx) {
  if (!ctx) return fail(PCX_ERR_ARG, "ctx is NULL");
  prof_drain(ctx);
  for (int i = 0; i < K_COUNT; ++i) {
    ctx->prof_ms[i] = 0.0;
    ctx->prof_n[i] = 0;
  }
  return PCX_OK;
}

int32_t pcx_profile_count(void) { return K_COUNT; }

pcx_status pcx_profile_read(pcx_ctx* ctx, int32_t i, const char** name, double* total_ms,
                            int64_t* launches) {
  if (!ctx) return fail(PCX_ERR_ARG, "ctx is NULL");
  if (i < 0 || i >= K_COUNT) return fail(PCX_ERR_ARG, "kernel index %d out of range", (int)i);
  prof_drain(ctx);
  if (name) *name = kKidNames[i];
  if (total_ms) *total_ms = ctx->prof_ms[i];
  if (launches) *launches = ctx->prof_n[i];
  return PCX_OK;
}

// ------------------------------------------------------------- getters
static pcx_status get_copy(pcx_ctx* ctx, const DevBuf& b, size_t n, size_t esz, void* out,
                           int64_t capacity, bool need_bwd) {
  if (!ctx) return fail(PCX_ERR_ARG, "ctx is NULL");
  if (!ctx->fwd_ok) return fail(PCX_ERR_STATE, "no completed forward pass");
  if (need_bwd && !ctx->bwd_done) return fail(PCX_ERR_STATE, "no completed backward pass");
  if (!out || capacity < (int64_t)n) return fail(PCX_ERR_ARG, "output buffer too small (%lld < %zu)",
                                                  (long long)capacity, n);
  if (n == 0) return PCX_OK;
  PCX_HIP(hipStreamSynchronize(ctx->stream));
  PCX_HIP(hipMemcpy(out, b.p, n * esz, hipMemcpyDeviceToHost));
  return PCX_OK;
}

pcx_status pcx_get_selected(pcx_ctx* ctx, int32_t* out, int64_t capacity) {
  return get_copy(ctx, ctx ? ctx->U : DevBuf(), ctx ? ctx->K : 0, 4, out, capacity, false);
}
pcx_status pcx_get_relabeled(pcx_ctx* ctx, int32_t* out, int64_t capacity) {
  return get_copy(ctx, ctx ? ctx->tgt_rel : DevBuf(), ctx ? ctx->L_tot : 0, 4, out, capacity,
                  false);
}
pcx_status pcx_get_alignable(pcx_ctx* ctx, uint8_t* out, int64_t capacity) {
  return get_copy(ctx, ctx ? ctx->flags : DevBuf(), ctx ? ctx->N : 0, 1, out, capacity, false);
}
pcx_status pcx_get_utt_losses(pcx_ctx* ctx, double* out, int64_t capacity) {
  return get_copy(ctx, ctx ? ctx->utt_loss : DevBuf(), ctx ? ctx->N : 0, 8, out, capacity, false);
}
pcx_status pcx_get_utt_status(pcx_ctx* ctx, int32_t* out, int64_t capacity) {
  return get_copy(ctx, ctx ? ctx->utt_status : DevBuf(), ctx ? ctx->N : 0, 4, out, capacity,
                  false);
}
pcx_status pcx_get_normalizer(pcx_ctx* ctx, double* out, int64_t capacity) {
  return get_copy(ctx, ctx ? ctx->lam : DevBuf(), ctx ? ctx->M : 0, 8, out, capacity, false);
}
pcx_status pcx_get_other(pcx_ctx* ctx, double* out, int64_t capacity) {
  if (ctx && ctx->fwd_ok && ctx->fwd_form != PCX_FORM_GROUPED)
    return fail(PCX_ERR_STATE, "the last forward pass did not use the grouped formulation");
  return get_copy(ctx, ctx ? ctx->other : DevBuf(), ctx ? ctx->M : 0, 8, out, capacity, false);
}
pcx_status pcx_get_scores(pcx_ctx* ctx, float* out, int64_t capacity) {
  return get_copy(ctx, ctx ? ctx->S : DevBuf(), ctx ? (size_t)ctx->K * ctx->M : 0, 4, out,
                  capacity, false);
}
pcx_status pcx_get_occupancy(pcx_ctx* ctx, float* out, int64_t capacity) {
  return get_copy(ctx, ctx ? ctx->Gam : DevBuf(), ctx ? (size_t)ctx->K * ctx->M : 0, 4, out,
                  capacity, true);
}

}  // extern "C"

/*
 * pcx: vocabulary-head projection fused with the exact reduced-class CTC loss
 * and its gradients, for AMD Instinct MI355X (gfx950).
 *
 * The operation follows "Pruned CTC for Memory-Efficient Large-Vocabulary
 * ASR Training" (Sec. 3.1 problem statement, Eq. 1-2; Sec. 3.2 selected
 * classes and Proposition 1; Sec. 3.3 / App. B.1 chunked projection, FP64
 * normalizer and backward recomputation) with an unbounded alignment beam,
 * i.e. the pages' "unpruned reduced CTC", by default, and with the pages'
 * finite-beam objective L_beta (App. B.1) after pcx_set_beam.  The calls
 * mirror the interface of
 * the PrunedCTC README (pruned_ctc_loss: encoder states, head weight and
 * bias, ragged targets, frame counts, chunk size, blank id; the return value
 * is the plain sum of per-utterance losses; fp32 or bf16 inputs, gradients
 * in the input dtype; only first-order gradients).
 *
 * Plain C ABI: no C++ or framework types.  Every device pointer is memory on
 * the current HIP device; every "stream" is a hipStream_t passed as void*
 * (NULL = the default stream).  All work is ordered on that stream.  No call
 * throws; each returns a pcx_status and, on failure, pcx_last_error() gives a
 * message (thread-local, valid until the next pcx call on that thread).
 */
#ifndef PCX_H
#define PCX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type shared by X, W and b (and the gradients written back). */
typedef enum {
  PCX_F32 = 0,  /* IEEE binary32 */
  PCX_BF16 = 1, /* bfloat16; float16 is not supported (README constraints) */
  PCX_F32_BF16W = 2 /* X fp32; W and b stored bf16 and widened to fp32 one
                       chunk at a time for an fp32 projection (the pages'
                       frozen-LLM-head setting, App. C.3) */
} pcx_dtype;

typedef enum {
  PCX_OK = 0,
  PCX_ERR_ARG = 1,     /* null pointer, negative or inconsistent size      */
  PCX_ERR_DTYPE = 2,   /* dtype other than the three of pcx_dtype           */
  PCX_ERR_TARGET = 3,  /* label outside [0, V), blank inside a target,     */
                       /* target offsets not monotone or not ending at L   */
  PCX_ERR_LENGTHS = 4, /* a frame count <= 0, or the counts do not sum to M */
  PCX_ERR_STATE = 5,   /* backward without a successful forward            */
  PCX_ERR_HIP = 6,     /* HIP runtime failure (allocation, launch, copy)   */
  PCX_ERR_LIMIT = 7,   /* a target longer than PCX_MAX_TARGET_LEN labels   */
  PCX_ERR_WORKSPACE = 8 /* the allocation callback returned NULL, or the    */
                        /* workspace would have to grow while the stream is */
                        /* being captured into a graph                      */
} pcx_status;

/* How the normalizer and the gradient of the unselected classes are formed
 * ("Pruned CTC for Memory-Efficient Large-Vocabulary ASR Training", Sec. 3.2
 * Eq. 4 and App. B.1 Eq. 11).  Both give the same loss and gradients in exact
 * arithmetic (Proposition 1); they differ only in rounding.
 *   DIRECT   lambda_m is the online log-sum-exp over the whole vocabulary;
 *            an unselected class v gets grad g_m exp(z_mv - lambda_m).
 *   GROUPED  the projection's log-sum-exp covers the unselected classes only,
 *            giving the "other" column o_m; lambda_m is the log-sum-exp of
 *            the grouped logits R_m = [Z[m][U], o_m] (o_m left out when every
 *            class is selected); the other column's gradient
 *            grad g_m exp(o_m - lambda_m) reaches class v with the weight
 *            exp(z_mv - o_m).  A cross-check of the direct path, at the same
 *            cost up to two small per-frame passes. */
typedef enum {
  PCX_FORM_DIRECT = 0,
  PCX_FORM_GROUPED = 1
} pcx_formulation;

/* Longest target (in labels) the alignment kernels accept. */
#define PCX_MAX_TARGET_LEN 2047

/* Opaque per-call-site context: holds the device workspace and what the
 * forward pass leaves for the backward pass (selected classes, relabelled
 * targets, flags, normalizers, selected-class scores S, DP tables). */
typedef struct pcx_ctx pcx_ctx;

/* Filled by pcx_forward. */
typedef struct {
  int32_t K;               /* number of selected classes |U|               */
  int32_t n_unalignable;   /* utterances with |y| + r > T (zero loss/grad)  */
  int32_t n_nonfinite;     /* alignable utterances whose loss was not finite */
  int32_t max_target_len;  /* longest target in the batch                   */
  uint64_t workspace_bytes;/* device bytes the context holds after the call */
  int32_t lse_spans;       /* vocabulary spans of the forward normalizer fold */
} pcx_fwd_info;

/* Device-memory callbacks for a context's workspace, so that it can live in
 * the caller's allocator and show in its memory accounting (the pages
 * measure head-and-loss memory with the framework's allocated-memory
 * counters, App. C.1; the PrunedCTC README keeps every tensor of a call on
 * one device).
 *   alloc(bytes, user, stream)  returns at least `bytes` bytes of device
 *       memory on the current HIP device, for use by work ordered on
 *       `stream` (a hipStream_t as void*, NULL = default stream), or NULL on
 *       failure (the call then fails with PCX_ERR_WORKSPACE).
 *   release(ptr, bytes, user, stream)  gives back a pointer alloc returned;
 *       `stream` is the stream it was allocated on and `bytes` the size
 *       asked for.  Every piece of library work that touches ptr is either
 *       finished or ordered before the work already issued to `stream`, so
 *       the memory may go to any work issued to that stream afterwards (the
 *       contract of a stream-ordered caching allocator).
 * Neither callback may call back into the library. */
typedef void* (*pcx_alloc_fn)(size_t bytes, void* user, void* stream);
typedef void (*pcx_free_fn)(void* ptr, size_t bytes, void* user, void* stream);

/* Create / destroy a context.  The context owns its device workspace, which
 * grows on demand and is released by pcx_destroy.
 *   alloc, release  both NULL: the library allocates with hipMalloc, and
 *                   growth waits for the whole device before hipFree;
 *                   both set: the workspace comes from these callbacks, and
 *                   growth waits for nothing when the buffer is released on
 *                   the stream of the current call (otherwise the current
 *                   stream is synchronised first).  One NULL and one set is
 *                   PCX_ERR_ARG.
 *   user            passed through to the callbacks.
 * No HIP call is made here.  A context may be used by one thread at a time.
 * Its calls run in call order even when they name different streams: a call
 * on another stream than the previous call's makes its stream wait for the
 * previous one (except while that stream is being captured into a graph,
 * whose capture the caller orders).  pcx_destroy waits for the last call's
 * stream before it releases the workspace. */
pcx_status pcx_create(pcx_ctx** out_ctx, pcx_alloc_fn alloc, pcx_free_fn release, void* user);
void pcx_destroy(pcx_ctx* ctx);

/*
 * Forward pass: selected classes, chunked projection with the FP64 online
 * normalizer, S = Z[:, U] - lambda rounded once to FP32, the FP64 CTC
 * forward recursion over the K selected columns, and the summed loss.
 *
 *   X             device, M x D row-major: the head inputs of all utterances
 *                 stacked without padding, utterance n owning the T_n rows
 *                 after those of utterances 0..n-1 (Sec. 3.1).
 *   W             device, V x D row-major (nn.Linear weight layout).
 *   b             device, V entries, or NULL for a zero bias.
 *                 X, W and b must be finite (PrunedCTC README constraints).
 *                 An utterance whose rows of X are not finite comes out
 *                 nonfinite: it is excluded (zero loss, zero dX rows,
 *                 counted), but dW and db, which mix all rows, are then
 *                 undefined.
 *   dtype         PCX_F32 or PCX_BF16 (the element type of X, W and b), or
 *                 PCX_F32_BF16W (X fp32, W and b bf16; the projections run in
 *                 fp32 on W widened chunk by chunk, C rows at a time in the
 *                 backward pass and whole normalizer spans in the forward).
 *   M, D, V, N    frames, head width, vocabulary size, utterances (N >= 0,
 *                 M >= 0, D >= 1, V >= 1).
 *   tgt_off       device int32, N + 1 monotone offsets into tgt, tgt_off[0]
 *                 = 0 and tgt_off[N] = L_tot (CSR form of the ragged,
 *                 blank-free targets).
 *   tgt           device int32, L_tot labels in [0, V) \ {blank}.
 *   L_tot         number of labels in tgt.
 *   frame_counts  device int32, N positive frame counts summing to M (may be
 *                 NULL when N = 0).
 *   blank         blank class id in [0, V).
 *   chunk         vocabulary chunk width C >= 1 used by the backward pass for
 *                 its one M x C gradient block (App. B.1); results do not
 *                 depend on it beyond rounding.  (A backward that wants dX
 *                 alone fills the block as half the frames by 2C columns,
 *                 the half rounded up to whole row tiles.)
 *   stream        hipStream_t (void*), NULL for the default stream.
 *   loss          host out, may be NULL: sum of the finite per-utterance
 *                 losses (unalignable / nonfinite ones contribute 0; the
 *                 README's "excluded with a warning" case is reported in
 *                 info instead of printed).
 *   info          host out, may be NULL.
 *
 * X, W and b must stay alive and unchanged until the matching pcx_backward.
 * The call synchronises the stream twice (to size the workspace once K is
 * known, and to read the loss back).  Errors in the device-resident targets
 * and lengths are detected on the device and reported after the first sync.
 */
pcx_status pcx_forward(pcx_ctx* ctx, const void* X, const void* W,
                       const void* b, int32_t dtype, int64_t M, int64_t D,
                       int64_t V, int32_t N, const int32_t* tgt_off,
                       const int32_t* tgt, int64_t L_tot,
                       const int32_t* frame_counts, int32_t blank,
                       int32_t chunk, void* stream, double* loss,
                       pcx_fwd_info* info);

/*
 * Backward pass for the last successful pcx_forward on ctx: the FP64 CTC
 * backward recursion, occupancies gamma on the selected classes, and, one
 * vocabulary chunk at a time, the recomputed logits, the logit gradient
 *   dZ[m][v] = grad_loss * (g_m p_v(m) - gamma_v(m))   (Eq. 5 / Eq. 7)
 * and the products dX = dZ W, dW = dZ^T X, db = column sums of dZ.
 *
 *   grad_loss  upstream gradient of the summed loss (any scaling, e.g. a
 *              division by the target-token count, goes here).
 *   dX         device, M x D in the dtype of X, or NULL to skip.
 *   dW         device, V x D in the dtype of W, or NULL to skip.
 *   db         device, V in the dtype of b (that of W), or NULL to skip.
 * Outputs are overwritten, not accumulated.  Rows of excluded utterances get
 * exact zeros.  May be called more than once per forward.  No host sync; once
 * a first call on ctx has sized its workspace for these shapes, a call makes
 * no allocation either (kernel launches on `stream` only, no memset nodes),
 * so it can be captured in a HIP graph and replayed.  A captured backward is
 * valid only for the pcx_forward that preceded the capture: the graph holds
 * that forward's workspace addresses, sizes (M, K) and X / W pointers, and
 * the next pcx_forward on ctx may move or resize the workspace or change
 * them, after which the graph must not be replayed.  Growth of the
 * workspace during a capture fails with PCX_ERR_WORKSPACE.
 */
pcx_status pcx_backward(pcx_ctx* ctx, double grad_loss, void* dX, void* dW,
                        void* db, void* stream);

/*
 * Gradient of the summed loss with respect to a scalar offset eta added to
 * the blank logit of every frame, b = b_pre + eta e_blank ("Pruned CTC for
 * Memory-Efficient Large-Vocabulary ASR Training", Sec. 4: the frozen LLM
 * head keeps its weights and learns only this blank offset):
 *   d_eta = grad_loss * sum_m (g_m p_blank(m) - gamma_blank(m)),
 * i.e. db[blank] without the V-wide db output or any GEMM.  Computed in FP64
 * from S and the occupancies (a fixed-order sum); runs the occupancy pass
 * itself, so it needs only a successful pcx_forward.
 *   grad_loss  as for pcx_backward.
 *   d_eta      host out.
 * Synchronises the stream once.
 */
pcx_status pcx_blank_offset_grad(pcx_ctx* ctx, double grad_loss, double* d_eta,
                                 void* stream);

/*
 * pcx_forward followed by pcx_backward in one call that allocates nothing,
 * for callers that cannot allocate device memory (code being captured into
 * a graph, tight serving loops, harnesses that forbid hipMalloc).  The
 * workspace is a static device array of PCX_STATIC_SCRATCH_BYTES bytes, one
 * copy per GPU the library runs on, held until the process ends; no context
 * is involved and no hipMalloc, hipFree or allocation callback is called.
 *   Arguments as pcx_forward (X ... chunk, stream, loss, info) and
 *   pcx_backward (grad_loss, dX, dW, db), with the same layouts, dtypes,
 *   ownership and results: the same kernels run with the same launch shapes.
 *   info->workspace_bytes reports the part of the scratch the call used.
 * A call whose workspace would exceed the scratch fails with
 * PCX_ERR_WORKSPACE without writing dX, dW or db (the loss and info of its
 * forward part may have been written).  The call synchronises the
 * stream twice, as pcx_forward does.  Every call on one GPU uses that GPU's
 * one scratch array: calls that overlap on a GPU (from two host threads, or
 * on two streams without ordering between them) race and give wrong
 * results; calls in order on one stream do not.
 */
#define PCX_STATIC_SCRATCH_BYTES (64u << 20)
pcx_status pcx_loss_grad_static(const void* X, const void* W, const void* b, int32_t dtype,
                                int64_t M, int64_t D, int64_t V, int32_t N,
                                const int32_t* tgt_off, const int32_t* tgt, int64_t L_tot,
                                const int32_t* frame_counts, int32_t blank, int32_t chunk,
                                double grad_loss, void* dX, void* dW, void* db, void* stream,
                                double* loss, pcx_fwd_info* info);

/*
 * Alignment beam of the following pcx_forward calls of this context (the
 * PrunedCTC README's output_beam; "Pruned CTC for Memory-Efficient
 * Large-Vocabulary ASR Training", App. B.1 finite-beam computation and the
 * finite-beam gap analysis).  beam = +inf (the default) keeps every
 * alignment: the exact loss.  A finite beam >= 0 prunes the alignment
 * lattice of each utterance relative to its best alignment: the arc
 * (t-1, s') -> (t, s) between states of the blank-interleaved labels is kept
 * when the best complete alignment through it scores at least B_n - beam
 * (scores are sums of the FP32 log-probabilities S in FP64; the arc's score
 * is (best prefix score at (t-1, s') + S_t(s)) + best suffix score after
 * (t, s), evaluated in that order), B_n being the best alignment's score;
 * the initial and final arcs likewise.  The loss of an utterance is then
 * -log of the summed probability of the alignments all of whose arcs are
 * kept, and pcx_backward differentiates it with the kept arcs held fixed
 * (gamma is the occupancy over the retained alignments).  An utterance
 * whose retained lattice comes out empty, or whose loss is not finite,
 * contributes zero loss and gradient and is counted in n_nonfinite.  Costs
 * two extra passes over the lattice in the forward call (best scores, arc
 * masks: one byte per lattice node of workspace).  PCX_ERR_ARG for a
 * negative or NaN beam.
 */
pcx_status pcx_set_beam(pcx_ctx* ctx, double beam);

/*
 * Posterior mass of the alignments the beam of the last pcx_forward
 * discarded, per utterance: delta_n = 1 - exp(-(L_beta,n - L_n)), with L_n
 * the unpruned loss on the same scores S (the pages' delta_n estimate; both
 * losses in FP64).  0 for every included utterance after an unbounded beam;
 * NaN for excluded utterances (unalignable, or a nonfinite pruned or
 * unpruned loss).  Runs the unpruned forward recursion (losses only; the
 * workspace of the pruned backward is untouched) and synchronises the
 * context's stream.  out: N doubles (capacity >= N).
 */
pcx_status pcx_get_discarded_mass(pcx_ctx* ctx, double* out, int64_t capacity);

/*
 * Formulation used by the following pcx_forward calls of this context
 * (PCX_FORM_DIRECT by default); pcx_backward follows the formulation of the
 * forward pass it differentiates.  PCX_ERR_ARG for any other value.
 */
pcx_status pcx_set_formulation(pcx_ctx* ctx, int32_t form);

/* Message for the last failing call on this thread ("" if none). */
const char* pcx_last_error(void);

/*
 * Inspection getters (synchronous device-to-host copies after the context's
 * stream has finished), used by parity tests.  Each copies at most
 * `capacity` elements into the host buffer and fails with PCX_ERR_ARG if the
 * buffer is too small, PCX_ERR_STATE if no forward has completed.
 *   selected    K int32: U, blank first then ascending distinct labels.
 *   relabeled   L_tot int32: index of each target label in U.
 *   alignable   N uint8: 1 iff |y_n| + r_n <= T_n.
 *   utt_losses  N double: per-utterance loss (0 when excluded).
 *   utt_status  N int32: 0 finite, 1 unalignable, 2 nonfinite.
 *   normalizer  M double: lambda_m (Eq. 1).
 *   scores      K x M float, class-major: S[j][m] = fp32(Z[m][U[j]] - lambda_m).
 *   occupancy   K x M float, class-major: gamma_{U[j]}(m) (after a backward).
 *   other       M double: the other column o_m = log sum over the unselected
 *               classes of exp z_mv (-inf when every class is selected);
 *               PCX_ERR_STATE unless the last forward was PCX_FORM_GROUPED.
 */
pcx_status pcx_get_selected(pcx_ctx* ctx, int32_t* out, int64_t capacity);
pcx_status pcx_get_relabeled(pcx_ctx* ctx, int32_t* out, int64_t capacity);
pcx_status pcx_get_alignable(pcx_ctx* ctx, uint8_t* out, int64_t capacity);
pcx_status pcx_get_utt_losses(pcx_ctx* ctx, double* out, int64_t capacity);
pcx_status pcx_get_utt_status(pcx_ctx* ctx, int32_t* out, int64_t capacity);
pcx_status pcx_get_normalizer(pcx_ctx* ctx, double* out, int64_t capacity);
pcx_status pcx_get_scores(pcx_ctx* ctx, float* out, int64_t capacity);
pcx_status pcx_get_occupancy(pcx_ctx* ctx, float* out, int64_t capacity);
pcx_status pcx_get_other(pcx_ctx* ctx, double* out, int64_t capacity);

/*
 * Optional per-kernel timing.  While enabled, every kernel the context
 * launches is bracketed by two hipEvents recorded on the launch stream;
 * pcx_profile_read waits for the recorded events and returns, for kernel
 * family i in [0, pcx_profile_count()), its name, the summed event-measured
 * duration in milliseconds and the number of launches since the last reset.
 * Off by default; enabling adds two event records per launch.  When more
 * than 4096 pairs are pending, pcx_forward folds them into the totals at its
 * first synchronisation, so they stay bounded when nothing reads them.
 */
pcx_status pcx_profile_enable(pcx_ctx* ctx, int32_t on);
/* Restrict the timing to the kernel families whose bit is set in `mask`
 * (bit i: family i; all families by default).  Each timed launch adds two
 * event records to the stream, so timing one family perturbs a run far less
 * than timing all of them. */
pcx_status pcx_profile_mask(pcx_ctx* ctx, uint32_t mask);
pcx_status pcx_profile_reset(pcx_ctx* ctx);
int32_t pcx_profile_count(void);
pcx_status pcx_profile_read(pcx_ctx* ctx, int32_t i, const char** name,
                            double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* PCX_H */

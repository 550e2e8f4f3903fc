/*
 * kd_topk_kl.h - C ABI of the fused chunked top-K KL distillation loss for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (offline distillation against a cached teacher top-K):
 *   for each position t with student hidden state h_t (row of hidden[S,H]) and
 *   cached teacher entries (id_tk, l_tk), k = 0..K-1:
 *     z_t    = h_t W^T                       student logits over the vocabulary V
 *     p_tk   = softmax_k(l_tk / T)           teacher top-K softmax, renormalised
 *                                            over the K cached entries
 *     KL_t   = sum_k p_tk (log p_tk - log softmax(z_t/T)[id_tk])
 *   loss = (sum over valid t of KL_t) / N,  N = number of valid positions.
 * The [S,V] logit grid is never stored: rows are projected tile by tile, the
 * log-normaliser of z/T is reduced online and the teacher ids are gathered as
 * the tiles pass; the backward pass projects each chunk of rows again.
 *
 * Sources (web pages; cited by title and section):
 *  - "Making Knowledge Distillation Cheap Enough to Run at Scale" (aibase.it
 *    write-up "Knowledge Distillation 비용 줄이기"): section "offline top-K
 *    logits" (per-position top-100 ids and logits, cached once with the
 *    temperature), section "what chunked KL loss does" (dense KL as the
 *    correctness baseline; fused chunked KL folds the output projection into
 *    the loss, projects one sequence chunk at a time, discards it, and
 *    recomputes it in the backward pass), section "operations" (cache
 *    validation: id range, missing positions, sort order, logit dtype).
 *  - "Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and a
 *    Fused Chunked KL Loss" (paper review), section 1 (fused chunked KL loss:
 *    no full-vocabulary logit tensor) and section 3 (memory linear in S).
 *  - "LLM Primer, Chapter 6 - Pruning and Distillation", section 6.2 (KL of
 *    temperature-softened teacher and student distributions).
 *  - "Rethinking Selective Knowledge Distillation" (summary), Method
 *    section 2 (SE-KD: top-k% positions by student entropy H(q_t)) and
 *    section 3 (selective LM head; chunked entropy computation).
 *
 * Conventions for every entry point:
 *  - Pointers marked [device] are device memory owned by the caller; the
 *    library never allocates or frees device memory. Pointers marked [host]
 *    are host memory. All arrays are dense row-major.
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *    on it in order; no entry point synchronises the host unless it says so.
 *  - `ws` / `ws_bytes`: caller-provided device workspace of at least
 *    kd_topk_kl_workspace_bytes(problem) bytes, 256-byte aligned. Its contents on
 *    entry are ignored and on exit are unspecified. Calls that overlap in time
 *    must use distinct workspaces.
 *  - Argument errors are detected on the host before anything is enqueued and
 *    returned as a kd_status; a failed launch returns KD_ERR_HIP. Data errors
 *    (ids outside [0,V), rows whose K logits are all -inf) are not errors of
 *    fwd/bwd: out-of-range ids are skipped (never dereferenced) and treated as
 *    absent entries, and all -inf rows are excluded like masked rows;
 *    kd_validate_topk reports them.
 */
#ifndef KD_TOPK_KL_H
#define KD_TOPK_KL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KD_ABI_VERSION 7

typedef enum kd_status {
  KD_OK = 0,
  KD_ERR_NULL = 1,         /* a required pointer is NULL                          */
  KD_ERR_SHAPE = 2,        /* S<0, H/V/K<=0, K>V, H not a multiple of 8, sizes too large */
  KD_ERR_DTYPE = 3,        /* dtype code not one of kd_dtype                      */
  KD_ERR_TEMPERATURE = 4,  /* T <= 0 or not finite                                */
  KD_ERR_CHUNK = 5,        /* chunk <= 0                                          */
  KD_ERR_WORKSPACE = 6,    /* ws NULL, misaligned, or smaller than kd_topk_kl_workspace_bytes */
  KD_ERR_BAD_ID = 7,       /* reserved: reported counts come from kd_validate_topk */
  KD_ERR_HIP = 8,          /* a HIP runtime call or kernel launch failed          */
  KD_ERR_ARCH = 9,         /* current device is not gfx950                        */
  KD_ERR_ARG = 10          /* other invalid argument (fraction, accumulate flag, tl_kind) */
} kd_status;

typedef enum kd_dtype { KD_BF16 = 0, KD_F32 = 1 } kd_dtype;

/* What topk_logits holds.
 *   KD_TEACHER_LOGITS  cached teacher logits: p_tk = softmax_k(l_tk / T), the
 *                      softmax taken over the row's K entries ("offline top-K
 *                      logits").
 *   KD_TEACHER_PROBS   teacher probabilities at the K ids, e.g. sampled sparse
 *                      targets ("Rethinking Selective Knowledge Distillation",
 *                      Method section 2, SE-KD3X class axis): p_tk = v_tk over
 *                      the sum of the row's usable values (id in [0, V),
 *                      value > 0); T then softens the student side only. A row
 *                      with a negative or non-finite value, or no positive
 *                      value, takes no part (like a masked row).              */
typedef enum kd_teacher_kind { KD_TEACHER_LOGITS = 0, KD_TEACHER_PROBS = 1 } kd_teacher_kind;

/* Problem description shared by all entry points.
 *   S      positions (rows of hidden); S = 0 is allowed (empty problem)
 *   H      hidden size; multiple of 8
 *   V      vocabulary size (rows of W)
 *   K      teacher entries per position, 1 <= K <= min(V, 4096)
 *   chunk  rows per backward chunk. The backward holds the gradient tiles
 *          of a group of consecutive chunks (about max(chunk, 8192) rows x V
 *          in hw_dtype; fp32 also keeps a transposed copy): with W^T, the
 *          only workspace terms that grow with V
 * Size limits (KD_ERR_SHAPE otherwise): S < 2^30, H <= 2^20, V <= 2^30, and
 * 256 rows of the padded gradient-tile pitch (about V elements of hw_dtype)
 * and of the transposed chunk pitch (about 8192 or chunk elements) each below
 * 2^31 bytes: V up to about 4.19M for bf16 (2.09M for fp32). 
 *   temperature  T > 0, applied to teacher and student logits alike (to the
 *                student only when tl_kind is KD_TEACHER_PROBS)
 *   hw_dtype     storage type of hidden and W (both the same)
 *   tl_dtype     storage type of topk_logits
 *   tl_kind      kd_teacher_kind: what topk_logits holds                     */
typedef struct kd_problem {
  int64_t S, H, V, K, chunk;
  float temperature;
  int32_t hw_dtype;
  int32_t tl_dtype;
  int32_t tl_kind;
} kd_problem;

/* ABI version of the loaded library (KD_ABI_VERSION). */
int kd_abi_version(void);

/* Static, NUL-terminated description of a status code. Never NULL. */
const char* kd_status_str(int status);

/* Workspace bytes needed by every entry point below for this problem (the
 * maximum over them). Returns 0 if the problem itself is invalid. The size is
 * linear in S (per-row teacher tables and partials) plus a part that does
 * not grow with S (the gradient tiles of a group of chunks, W^T and the
 * split-K partials of dHidden). */
size_t kd_topk_kl_workspace_bytes(const kd_problem* problem);

/* Forward pass ("what chunked KL loss does": project, fold into the loss,
 * discard; the online log-normaliser of z/T over V and the gather of z at the
 * teacher ids run inside the projection's epilogue).
 *   hidden      [device] [S,H] hw_dtype
 *   W           [device] [V,H] hw_dtype (output projection, nn.Linear layout)
 *   topk_ids    [device] [S,K] int32 teacher ids, any order, duplicates add
 *   topk_logits [device] [S,K] tl_dtype teacher logits (-inf = absent entry)
 *   mask        [device] [S] uint8, nonzero = position takes part; NULL = all
 *   loss        [device] [1] float32: sum of KL_t over valid rows / N (0 if N=0)
 *   lse         [device] [S] float32: log sum_v exp(z_tv / T) for valid rows,
 *               0 for rows not taking part; needed by kd_topk_kl_bwd
 *   kl_rows     [device] [S] float32 or NULL: KL_t for valid rows, 0 otherwise
 *   z_topk      [device] [S,K] float32 or NULL: z_t[id_tk] / T for valid rows
 *               and in-range ids (same order as topk_ids), NaN elsewhere      */
int kd_topk_kl_fwd(const kd_problem* problem, const void* hidden, const void* W,
                   const int32_t* topk_ids, const void* topk_logits, const uint8_t* mask,
                   float* loss, float* lse, float* kl_rows, float* z_topk,
                   void* ws, size_t ws_bytes, void* stream);

/* The forward pass for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation, outputs and argument rules as
 * kd_topk_kl_fwd, without the workspace argument. Its scratch is a fixed
 * device array of KD_NOALLOC_SCRATCH_BYTES inside the library, one copy per
 * GPU, held until the process ends. A problem whose forward scratch is larger
 * returns KD_ERR_WORKSPACE before any launch: the scratch is about
 * S*(16*K + 13) bytes plus 8 bytes per row and vocabulary range of the sweep,
 * so S up to about 40000 at K = 100. It calls no hipMalloc or hipFree and
 * records no profiling events. Every call on one GPU uses that GPU's array:
 * calls that overlap in time on one GPU (other streams, other threads) race
 * and give wrong results, so such callers must serialise them. Nothing in the
 * array needs clearing between calls: every value a call reads, it wrote.   */
#define KD_NOALLOC_SCRATCH_BYTES 67108864
int kd_topk_kl_fwd_noalloc(const kd_problem* problem, const void* hidden, const void* W,
                           const int32_t* topk_ids, const void* topk_logits,
                           const uint8_t* mask, float* loss, float* lse, float* kl_rows,
                           float* z_topk, void* stream);

/* Backward pass: rows are projected again chunk by chunk ("backward
 * recomputes the chunk"); the logit gradient
 *   G_tv = g/N * (softmax(z_t/T)_v - p_t(v)) / T,   g = *grad_loss,
 * with p_t(v) the teacher probability scattered to its id, is formed in the
 * projection's epilogue as a [chunk,V] tile in hw_dtype and contracted twice:
 *   dhidden[t] = G_t W  (rows not taking part are set to 0),
 *   dW        (+)= G^T hidden_chunk, accumulated over chunks in fp32.
 *   lse         [device] [S] float32 from kd_topk_kl_fwd with the same inputs
 *   grad_loss   [device] [1] float32 upstream gradient of loss
 *   dhidden     [device] [S,H] float32 output
 *   dW          [device] [V,H] float32 output; accumulate_dW = 1 adds to its
 *               contents (tied weights), 0 overwrites                          */
int kd_topk_kl_bwd(const kd_problem* problem, const void* hidden, const void* W,
                   const int32_t* topk_ids, const void* topk_logits, const uint8_t* mask,
                   const float* lse, const float* grad_loss,
                   float* dhidden, float* dW, int accumulate_dW,
                   void* ws, size_t ws_bytes, void* stream);

/* Forward and backward in one call, for callers that know the upstream
 * gradient before the forward (training steps: g = 1, or a loss scale). The
 * fused chunked loss of "what chunked KL loss does", with the chunk's
 * gradient taken without projecting the chunk a second time: per chunk, one
 * projection sweep forms the partial log-normalisers and the logits at the
 * teacher ids (as kd_topk_kl_fwd) and keeps the chunk's fp32 logits
 * [chunk,V] in the workspace; once the chunk's lse is known, the logit
 * gradient G (as kd_topk_kl_bwd) is formed from them, then dhidden and dW.
 * This trades the recompute that the "operations" section charges to the
 * fused loss at short context for one chunk of fp32 logits (4*chunk*V bytes,
 * not growing with S). Outputs are those of kd_topk_kl_fwd followed by
 * kd_topk_kl_bwd with the same arguments, within fp32 rounding: lse is
 * merged over the vocabulary ranges of a chunk's sweep rather than of one
 * sweep over all rows, so it may differ in the last bits, and G with it.
 *   grad_loss   [device] [1] float32 upstream gradient g of loss
 *   loss, lse, kl_rows, z_topk   as kd_topk_kl_fwd
 *   dhidden, dW, accumulate_dW   as kd_topk_kl_bwd
 *   ws          kd_topk_kl_fwd_bwd_workspace_bytes(problem) bytes, 256-aligned
 * Errors as kd_topk_kl_fwd and kd_topk_kl_bwd. Does not sync.                */
size_t kd_topk_kl_fwd_bwd_workspace_bytes(const kd_problem* problem);
int kd_topk_kl_fwd_bwd(const kd_problem* problem, const void* hidden, const void* W,
                       const int32_t* topk_ids, const void* topk_logits, const uint8_t* mask,
                       const float* grad_loss, float* loss, float* lse, float* kl_rows,
                       float* z_topk, float* dhidden, float* dW, int accumulate_dW,
                       void* ws, size_t ws_bytes, void* stream);

/* x[i] *= *g for i < n (x, g: device float32). With kd_topk_kl_fwd_bwd run
 * at g = 1 in a forward pass, this applies the upstream gradient that an
 * autograd backward receives later to dhidden and dW: the chunked loss's
 * gradient is linear in g. Errors: KD_ERR_SHAPE for n < 0, KD_ERR_NULL for a
 * NULL pointer with n > 0. Does not sync.                                   */
int kd_scale_f32(float* x, int64_t n, const float* g, void* stream);

/* Comparator forms of the loss ("what chunked KL loss does" sets the fused
 * chunked loss beside two others, and the "operations" section says the
 * fused one is slower than the forward-chunked one at short context, since
 * its backward projects again). Same loss, same gradients, different memory:
 *   KD_FORM_DENSE            the cached top-K expanded into a dense teacher
 *                            probability grid P [S,V] (fp32), the student's
 *                            log-probabilities logQ [S,V] (fp32) from the
 *                            logits Z [S,V] (bf16) of one projection over all
 *                            rows; KL per row from the grids; the backward
 *                            takes the logit gradient from P and logQ.
 *   KD_FORM_FORWARD_CHUNKED  the teacher stays sparse and rows are projected
 *                            chunk by chunk, but the logits Z [S,V] (bf16) of
 *                            every row are kept; the backward takes the logit
 *                            gradient from Z instead of projecting again.
 * KD_FORM_FUSED names kd_topk_kl_fwd / kd_topk_kl_bwd, which keep no grid.  */
typedef enum kd_loss_form {
  KD_FORM_FUSED = 0,
  KD_FORM_DENSE = 1,
  KD_FORM_FORWARD_CHUNKED = 2
} kd_loss_form;

/* Workspace bytes of a comparator form (0 for an invalid problem or form).
 * It holds the stored grids: about S*Vp*2 bytes (forward-chunked) or
 * S*Vp*10 bytes (dense), Vp = V rounded up to 8, on top of
 * kd_topk_kl_workspace_bytes. */
size_t kd_kl_comparator_workspace_bytes(const kd_problem* problem, int form);

/* Forward of a comparator form: the same arguments and outputs as
 * kd_topk_kl_fwd (z_topk is not offered), with form = KD_FORM_DENSE or
 * KD_FORM_FORWARD_CHUNKED (KD_ERR_ARG otherwise). hw_dtype must be KD_BF16
 * (KD_ERR_DTYPE otherwise). The grids it stores stay in ws for
 * kd_kl_comparator_bwd. Does not synchronise the host.                      */
int kd_kl_comparator_fwd(const kd_problem* problem, int form, const void* hidden, const void* W,
                         const int32_t* topk_ids, const void* topk_logits, const uint8_t* mask,
                         float* loss, float* lse, float* kl_rows, void* ws, size_t ws_bytes,
                         void* stream);

/* Backward of a comparator form: the same arguments and outputs as
 * kd_topk_kl_bwd. It reads the grids that kd_kl_comparator_fwd of the same
 * form left in ws: call it with the same problem, inputs, mask and ws, with no
 * other call on that ws in between.                                         */
int kd_kl_comparator_bwd(const kd_problem* problem, int form, const void* hidden, const void* W,
                         const int32_t* topk_ids, const void* topk_logits, const uint8_t* mask,
                         const float* lse, const float* grad_loss, float* dhidden, float* dW,
                         int accumulate_dW, void* ws, size_t ws_bytes, void* stream);

/* Per-position student entropy H(q_t) = -sum_v q_tv ln q_tv in nats, with
 * q_t = softmax(z_t) over the full vocabulary at temperature 1 ("Rethinking
 * Selective Knowledge Distillation", Method 2-3: student entropy as the
 * position signal, computed chunk-wise without storing logits). The
 * temperature field of the problem is not used.
 *   entropy     [device] [S] float64 output                                   */
int kd_student_entropy(const kd_problem* problem, const void* hidden, const void* W,
                       double* entropy, void* ws, size_t ws_bytes, void* stream);

/* Keep the floor(num*S/den) positions of highest entropy, lower index first
 * on ties (SE-KD top-k% selection, Method section 2). Entropies within a band
 * around the cut are recomputed in fp64 from hidden and W before the decision
 * (the whole band, in pieces, whatever its size), so the kept set is the one
 * an fp64 evaluation gives. The band is +-2 eps around the k-th largest
 * entropy, where eps bounds |entropy - fp64 entropy|: 2e-5 nats (which
 * kd_student_entropy's fp32-path values meet for logits |z| of order 10 or
 * less at H of a few thousand), or four times the largest such error measured
 * on the positions the call recomputes in fp64 if that is larger: its band
 * (taken first with 2e-5 nats) and 16 positions spread evenly over [0, S),
 * refined together; a call whose measured bound exceeds 2e-5 nats is redone
 * once with the wider band. Entropies less accurate than 2e-5 nats thus widen
 * the band instead of deciding the cut. The tests check the kept
 * set against the fp64 one for unit-variance logits, logits of standard
 * deviation 4, and entropies given with errors of up to 1e-4 nats.
 *   entropy     [device] [S] float64 from kd_student_entropy (not modified)
 *   mask_out    [device] [S] uint8: 1 = kept
 *   idx_out     [device] [S] int32 or NULL: kept positions in ascending order
 *               in the first count entries
 *   count_out   [host] number kept. Synchronises the host with the stream.  */
int kd_select_top_fraction(const kd_problem* problem, const void* hidden, const void* W,
                           const double* entropy, int64_t num, int64_t den,
                           uint8_t* mask_out, int32_t* idx_out, int64_t* count_out,
                           void* ws, size_t ws_bytes, void* stream);

/* Keep floor(num*B/den) of B training samples by the mean entropy of their
 * positions, highest first, lower sample index on ties ("Rethinking Selective
 * Knowledge Distillation", Method section 2, SE-KD3X sample axis: the top l% of
 * samples by mean student entropy from a frozen student's forward pass).
 * Sample b is positions [offsets[b], offsets[b+1]); an empty sample has mean
 * -inf. Samples whose mean lies within 2 eps of the cut (eps the entropy error
 * bound of kd_select_top_fraction, measured the same way) have
 * their positions' entropies recomputed in fp64 from hidden and W before the
 * decision (each such position once, in pieces, whatever their number), so
 * the kept set is the one fp64 entropies give.
 *   entropy     [device] [S] float64 from kd_student_entropy (not modified)
 *   offsets     [device] [B+1] int64, non-decreasing within [0, S]
 *               (KD_ERR_ARG otherwise); B <= max(S, 1)
 *   mask_out    [device] [B] uint8: 1 = kept
 *   idx_out     [device] [B] int32 or NULL: kept samples in ascending order in
 *               the first count entries
 *   count_out   [host] number kept. Synchronises the host with the stream.  */
int kd_select_samples(const kd_problem* problem, const void* hidden, const void* W,
                      const double* entropy, const int64_t* offsets, int64_t B, int64_t num,
                      int64_t den, uint8_t* mask_out, int32_t* idx_out, int64_t* count_out,
                      void* ws, size_t ws_bytes, void* stream);

/* Position importance signals ("Rethinking Selective Knowledge Distillation",
 * Method section 1: student cross-entropy, teacher uncertainty 1 - p_t(y_t),
 * student entropy; the teacher-student KL per position is kd_topk_kl_fwd's
 * kl_rows). Each output may be NULL; the others are still computed.
 *   entropy      [device] [S] float64: H(softmax(z_t)) at T = 1, as
 *                kd_student_entropy (needs hidden, W)
 *   ce           [device] [S] float64: log sum_v exp(z_tv) - z_{t,y_t} at T = 1,
 *                the student's cross-entropy on the label (needs hidden, W,
 *                labels); NaN where the label is outside [0, V)
 *   teacher_unc  [device] [S] float64: 1 - p_t(y_t), p_t the row's KD target
 *                (renormalised top-K softmax at the problem's temperature, or
 *                the given probabilities for KD_TEACHER_PROBS), entries sharing
 *                the label's id adding; 1 when the label is not among the ids;
 *                NaN where the label is outside [0, V) or the teacher row takes
 *                no part (needs topk_ids, topk_logits, labels)
 *   labels       [device] [S] int32 next-token ids
 * Entropy and ce share one projection sweep over the vocabulary; ce adds an
 * fp64 dot product per position and teacher_unc an fp64 pass over the K
 * entries. Does not synchronise the host.                                    */
int kd_position_signals(const kd_problem* problem, const void* hidden, const void* W,
                        const int32_t* topk_ids, const void* topk_logits, const int32_t* labels,
                        double* entropy, double* ce, double* teacher_unc, void* ws,
                        size_t ws_bytes, void* stream);

/* Top-k% positions by a signal, per segment ("Rethinking Selective Knowledge
 * Distillation", Method section 1: top-k% selection; per sequence when a batch
 * of sequences is given as segments). Segment b is positions
 * [offsets[b], offsets[b+1]); it keeps floor(num*len_b/den) positions, highest
 * signal first, lower index first among equal values (-0 equals +0). NaN
 * signals are never kept, so a segment with fewer non-NaN positions keeps
 * fewer. Positions outside every segment are not kept. The decision is exact
 * on the given values.
 *   signal          [device] [S] float64 (not modified)
 *   offsets         [device] [B+1] int64, non-decreasing within [0, S]
 *                   (KD_ERR_ARG otherwise), or NULL: one segment [0, S) (B is
 *                   then taken as 1)
 *   num, den        0 <= num <= den, 0 < den < 2^31 (KD_ERR_ARG otherwise)
 *   mask_out        [device] [S] uint8: 1 = kept
 *   idx_out         [device] [S] int32 or NULL: kept positions in ascending
 *                   order in the first count entries
 *   thresholds_out  [device] [B] float64 or NULL: per segment, the smallest
 *                   kept value (NaN when none is kept): a global threshold for
 *                   kd_select_above when computed over a pooled set of signals
 *   count_out       [host] number kept. Synchronises the host with the stream. */
int kd_select_by_signal(const kd_problem* problem, const double* signal, const int64_t* offsets,
                        int64_t B, int64_t num, int64_t den, uint8_t* mask_out,
                        int32_t* idx_out, double* thresholds_out, int64_t* count_out, void* ws,
                        size_t ws_bytes, void* stream);

/* Per-sequence top-k% by student entropy (SE-KD, "Rethinking Selective
 * Knowledge Distillation", Method section 2, applied within each sequence of a
 * batch): segment b = positions [offsets[b], offsets[b+1]) keeps
 * floor(num*len_b/den) positions of highest entropy, lower index first on ties.
 * As in kd_select_top_fraction, the entries within 2 eps of a segment's cut
 * (eps the same measured entropy error bound) are recomputed in fp64 from hidden and W before the
 * decision (every such entry, in pieces, whatever their number), so the kept
 * set is the one fp64 entropies give.
 *   entropy     [device] [S] float64 from kd_student_entropy (not modified)
 *   offsets     [device] [B+1] int64, non-decreasing within [0, S] (KD_ERR_ARG
 *               otherwise); positions outside every segment are not kept
 *   num, den    0 <= num <= den, 0 < den < 2^31
 *   mask_out, idx_out, count_out as for kd_select_top_fraction.            */
int kd_select_top_fraction_segments(const kd_problem* problem, const void* hidden,
                                    const void* W, const double* entropy,
                                    const int64_t* offsets, int64_t B, int64_t num, int64_t den,
                                    uint8_t* mask_out, int32_t* idx_out, int64_t* count_out,
                                    void* ws, size_t ws_bytes, void* stream);

/* Global threshold policy (GLS, "Rethinking Selective Knowledge
 * Distillation", Method section 1, named there without a definition; read
 * here as one threshold shared by all positions): keep signal >= tau. NaN is
 * never kept; tau must not be NaN (KD_ERR_ARG).
 *   mask_out, idx_out, count_out as for kd_select_by_signal.                 */
int kd_select_above(const kd_problem* problem, const double* signal, double tau,
                    uint8_t* mask_out, int32_t* idx_out, int64_t* count_out, void* ws,
                    size_t ws_bytes, void* stream);

/* Cache validation ("operations": id range and missing positions).
 *   n_bad_id     [host] ids outside [0, V)
 *   n_empty_row  [host] rows whose K logits are all -inf
 *   n_bad_logit  [host] logits that are NaN or +inf
 * Synchronises the host with the stream.                                     */
int kd_validate_topk(const kd_problem* problem, const int32_t* topk_ids, const void* topk_logits,
                     int64_t* n_bad_id, int64_t* n_empty_row, int64_t* n_bad_logit,
                     void* ws, size_t ws_bytes, void* stream);

/* Cache validation, the top-K order ("operations": the cache checks include
 * the top-K sorting):
 *   n_unsorted_row   [host] rows whose K values (logits, or probabilities) are
 *                    not non-increasing: some value smaller than the next (NaN
 *                    compares with nothing and is counted by kd_validate_topk)
 *   n_duplicate_row  [host] rows holding an id more than once
 * One wave per row, O(K^2) id comparisons per row. Synchronises the host.    */
int kd_validate_topk_order(const kd_problem* problem, const int32_t* topk_ids,
                           const void* topk_logits, int64_t* n_unsorted_row,
                           int64_t* n_duplicate_row, void* ws, size_t ws_bytes, void* stream);

/* Teacher top-K cache writer ("offline top-K logits": the teacher's output
 * is computed once and only each position's K most likely tokens are kept;
 * "operations": the cache stores token ids and logits per position, in top-K
 * order). For every position t: the K entries of largest teacher logit
 * z_tv = h_t . w_v, ordered by logit descending, the lower id first among
 * equal logits. The choice is exact: logits near the K-th largest are
 * recomputed in fp64 from the inputs before the decision, so the entries are
 * the ones an fp64 evaluation selects, and every logit written is that fp64
 * value rounded to fp32 (then to bf16 for a bf16 cache). The [S,V] logit grid
 * is never stored: problem->chunk positions are processed at a time.
 *   hidden      [device] [S,H] hw_dtype: the teacher's final hidden states
 *   W           [device] [V,H] hw_dtype: the teacher's output projection
 *   topk_ids    [device] [S,K] int32 output
 *   topk_logits [device] [S,K] tl_dtype output (raw logits: the temperature
 *               is stored with the cache by the caller and not used here)
 *   ws          at least kd_teacher_topk_workspace_bytes(problem) bytes (this
 *               entry point does not use kd_topk_kl_workspace_bytes).
 * Inputs must be finite. Logits that are equal to within the fp32 rounding
 * bound take longer (a slower ranking path), not a different result.       */
size_t kd_teacher_topk_workspace_bytes(const kd_problem* problem);
int kd_teacher_topk(const kd_problem* problem, const void* hidden, const void* W,
                    int32_t* topk_ids, void* topk_logits, void* ws, size_t ws_bytes,
                    void* stream);

/* Sampled sparse teacher targets ("Rethinking Selective Knowledge
 * Distillation", Method section 2: RS-KD, the class axis of SE-KD3X, where a
 * position's target is a few ids sampled from the teacher's distribution).
 * For every position t and draw n (N = problem->K draws, 1 <= N <= min(V,
 * 4096)), with u = uniforms[t,n]: the smallest vocabulary id v such that the
 * cumulative teacher probability F_t(v) = sum over ids w <= v of
 * softmax(z_t / T)_w exceeds u (inverse transform in vocabulary order),
 * z_tv = h_t . w_v and T = problem->temperature. The target of position t is
 * then the N ids with weight 1/N each (give it to kd_topk_kl_* as a
 * probability cache: tl_kind KD_TEACHER_PROBS, equal values; repeated ids
 * add up). The [S,V] grid is never stored: per chunk of problem->chunk
 * positions one sweep stores the mass of every 128 consecutive ids (each in
 * the scale of its own largest logit), and a second pass resolves each draw
 * inside its 128 ids, recomputing only the tiles of 256 ids that positions
 * of the chunk draw in, for those positions.
 *   hidden    [device] [S,H] hw_dtype: the teacher's final hidden states
 *   W         [device] [V,H] hw_dtype: the teacher's output projection
 *   uniforms  [device] [S,N] double in [0, 1), each row non-decreasing (sort
 *             the caller's draws per row; the ids come out in that order).
 *             Checked first: KD_ERR_ARG, with nothing written, otherwise
 *             (this check synchronises the host).
 *   ids_out   [device] [S,N] int32 output
 *   ws        at least kd_teacher_sample_workspace_bytes(problem) bytes (this
 *             entry point does not use kd_topk_kl_workspace_bytes).
 * Precision: the weights are formed in fp32 from the fp32-accumulated
 * logits, relative to the largest logit of their 128 ids, summed in fp32 per
 * 4 and 128 ids and in fp64 above, so F_t is met to about 1e-5 absolute; a u that close to a step of F_t may
 * get the neighbouring id. A u within rounding of 1 gives the largest id of
 * positive computed probability. A position with non-finite logits gets -1
 * for every draw. problem->K is N here; problem->tl_* are not used.          */
size_t kd_teacher_sample_workspace_bytes(const kd_problem* problem);
int kd_teacher_sample(const kd_problem* problem, const void* hidden, const void* W,
                      const double* uniforms, int32_t* ids_out, void* ws, size_t ws_bytes,
                      void* stream);

/* Kernel timing (off by default). When on, every kernel the library enqueues
 * is bracketed by HIP events on the same stream. kd_profile_read synchronises
 * those events and reports, per kernel name, the number of launches and the
 * summed duration in milliseconds; it returns the number of names written (at
 * most max_entries). kd_profile_reset discards the records. The records and
 * the on/off flag are process-wide (shared by every thread and device, guarded
 * by a lock that is taken only while profiling is on); they never change a
 * result. The no-alloc forward records no events.                          */
typedef struct kd_kernel_stat {
  char name[48];
  int64_t launches;
  double total_ms;
} kd_kernel_stat;
int kd_profile_enable(int on);
int kd_profile_read(kd_kernel_stat* out, int max_entries);
int kd_profile_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* KD_TOPK_KL_H */

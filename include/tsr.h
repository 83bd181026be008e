/*
 * tsr.h - C ABI of the batched logits-to-token sampler for AMD Instinct MI355X
 * (gfx950): temperature, softmax, top-k, top-p, min-p, renormalisation and a
 * Philox draw per row, and the speculative-decoding verify step.
 *
 * Pages this interface implements:
 *  [P1] fareedkhan-dev.github.io "Inference: Sampling, the KV Cache,
 *       Speculative Decoding and int8" - "Picking the next token" (the knobs
 *       and their order, the min-p rule), "Speculative decoding".
 *  [P2] gowda.ai "Chapter 39 Decoding & Speculative Sampling" - 39.1 (greedy),
 *       39.2 (filters as transforms, eq. 39.2, Listing 39.2), 39.3 (an empty
 *       allowed set is an invalid state), 39.4 (eqs. 39.3-39.4, Listing 39.4).
 *  [P3] brentwoodlivery.com "Speculative decoding - Hinglish notes" - "The
 *       Algorithm (Step-by-Step)", "Batching Speculation", "Temperature and
 *       Sampling".
 *  [P4] scratchllm.com "Efficient Inference & Compression" - "Speculative
 *       decoding".
 *  [P5] legost.in "Choosing the next word" - "Temperature", "Cutting off the
 *       tail: top-k and top-p", "Where the randomness comes from".
 *
 * Conventions shared by every call
 *  - All tensors are caller-owned DEVICE memory on the handle's device. The
 *    library never allocates, frees or retains them.
 *  - Calls enqueue work on `hip_stream` (a hipStream_t; NULL = the default
 *    stream) and return without waiting. Outputs are valid once the stream
 *    has reached that point.
 *  - Argument errors are returned synchronously and nothing is enqueued.
 *    Per-row data errors (NaN/+inf logits, an all -inf row, a draft token out
 *    of range) are reported per row through a status array, with token -1.
 *    A failed launch returns TSR_EDEVICE. No C++ exception crosses this ABI.
 *  - Logits are float32 or bfloat16, row-major; each row holds `vocab`
 *    elements. Pointers must be aligned to the element size. Rows may start
 *    at any element boundary (a contiguous batch of an odd vocab too): they
 *    are read in 16-byte loads at whatever alignment they have, under the
 *    unaligned access mode the HSA runtime sets, and no byte outside a row
 *    is read.
 *  - A handle is not thread-safe. Two calls on one handle may run on different
 *    streams only if they are not verify calls (verify uses per-handle
 *    workspace).
 */
#ifndef TSR_H_
#define TSR_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tsr_ctx* tsr_handle;

/* Return codes. */
enum {
  TSR_OK = 0,
  TSR_EINVAL = 1,        /* bad argument: null pointer, size or parameter out of range */
  TSR_ENOMEM = 2,        /* workspace allocation failed in sampler_init */
  TSR_EDEVICE = 3,       /* HIP runtime error (device selection, launch) */
  TSR_EUNSUPPORTED = 4   /* a size this build has no kernel for */
};

/* Element types of the logits. */
enum { TSR_F32 = 0, TSR_BF16 = 1 };

/* How top-p combines with top-k [P2 Listing 39.2 vs P5's generation loop].
 * JOINT: every filter reads the same post-temperature p; the kept set is the
 *   intersection of the filters' sets and is renormalised once (eq. 39.2).
 * SEQUENTIAL: top-p measures mass relative to the tokens top-k kept. */
enum { TSR_JOINT = 0, TSR_SEQUENTIAL = 1 };

/* Per-row status. */
enum {
  TSR_ROW_OK = 0,
  TSR_ROW_NONFINITE = 1, /* the row holds NaN or +inf */
  TSR_ROW_EMPTY = 2,     /* every logit is -inf: the kept set is empty [P2 39.3] */
  TSR_ROW_BADTOKEN = 3,  /* verify only: a draft token outside [0, vocab) */
  TSR_ROW_BADPARAM = 4   /* the row's own parameters (tsr_constraints.row_params) are invalid */
};

/* Sampling parameters, one set per call [P1 "Picking the next token"].
 *  temperature: 0 = greedy (the lowest token id among the maximal logits);
 *               otherwise >= 1e-30, and p = softmax(logits / temperature).
 *               Not clamped. Negative or non-finite values are TSR_EINVAL.
 *  top_k:       keep every token with fewer than top_k strictly larger
 *               logits (ties with the k-th value stay); <= 0 or >= vocab: off.
 *  top_p:       keep the tie groups, in descending logit order, whose mass
 *               strictly above them is below top_p (times the top-k kept mass
 *               in SEQUENTIAL mode); the top group always stays. >= 1: off;
 *               < 0 or non-finite: TSR_EINVAL.
 *  min_p:       keep p_i >= min_p * max_j p_j; active iff 0 < min_p < 1.
 *  filter_mode: TSR_JOINT or TSR_SEQUENTIAL.
 * The kept set S always has the form {i : logit_i >= tau} and excludes -inf
 * logits; the draw renormalises over S (eq. 39.2). */
typedef struct {
  double temperature;
  int32_t top_k;
  double top_p;
  double min_p;
  int32_t filter_mode;
} tsr_params;

/* Optional per-row diagnostics for sample_rows; every pointer may be NULL.
 *  status      [rows]        TSR_ROW_* per row.
 *  kept_count  [rows]        |S| (0 on bad rows).
 *  threshold   [rows]        the smallest kept logit (as float32).
 *  kept_mass   [rows]        sum over S of softmax(logits / T), in (0, 1].
 *  probs       [rows][vocab] the renormalised distribution p~ (eq. 39.2),
 *                            0 outside S (all 0 on bad rows). Written by an
 *                            extra pass: meant for validation, not for the
 *                            timed hot path.
 * A greedy row (temperature 0) reports p~ as the point mass at its token:
 * kept_count 1, threshold the row's largest logit, kept_mass 1, probs one-hot. */
typedef struct {
  int32_t* status;
  int32_t* kept_count;
  float* threshold;
  double* kept_mass;
  float* probs;
} tsr_diag;

/* Create a handle on `device` and allocate its workspace once.
 *  max_rows, max_vocab, max_k bound later calls (max_k: the largest draft
 *  length K of spec_verify). The Philox4x32-10 key is `seed` (low word first);
 *  the counter of each draw is (row, position | domain << 16, step low, step
 *  high), so a token depends only on (seed, row, position, step) and the
 *  parameters [P5 "Where the randomness comes from"].
 *  Returns TSR_OK and writes *out, or an error code with *out = NULL. */
int sampler_init(tsr_handle* out, int device, int max_rows, int max_vocab, int max_k,
                 uint64_t seed);

/* Free the handle and its workspace. NULL is accepted. Waits for the device. */
int sampler_destroy(tsr_handle h);

/* Greedy decoding [P2 39.1]: out_tokens[r] = the lowest id among the maximal
 * logits of row r. logits[r] starts at logits + r * row_stride elements.
 * out_status (nullable, [rows]) gets TSR_ROW_*; bad rows get token -1. */
int greedy_argmax(tsr_handle h, const void* logits, int dtype, int rows, int vocab,
                  int64_t row_stride, int32_t* out_tokens, int32_t* out_status,
                  void* hip_stream);

/* The sampler [P1 "Picking the next token"; P2 39.2; P5]. For each row r:
 * z = logits[r] / T, p = softmax(z), the kept set S by top-k, top-p and
 * min-p (see tsr_params), p~ = p 1{S} / sum_S p (eq. 39.2), then one draw by
 * inverse CDF: u = w0 * 2^-32 with w0 the first Philox word of counter
 * (r, 0, step), and the token is the first kept id, in ascending id order,
 * whose running total of p~ exceeds u. temperature 0 gives greedy_argmax.
 * logits[r] starts at logits + r * row_stride elements (row_stride >= vocab).
 * diag may be NULL. */
int sample_rows(tsr_handle h, const void* logits, int dtype, int rows, int vocab,
                int64_t row_stride, const tsr_params* params, uint64_t step,
                int32_t* out_tokens, const tsr_diag* diag, void* hip_stream);

/* The sampler restricted to an allowed-token set (constrained decoding)
 * [P2 39.3: the disallowed logits become -inf before the softmax, every step;
 * an empty allowed set is an invalid state], with the log-probability of each
 * drawn token [P1 "Picking the next token": generation can return it].
 *  allowed [rows][allowed_stride] uint32 words (nullable: every token is
 *      allowed, and the call equals sample_rows): token i of row r is allowed
 *      iff bit (i % 32) of allowed[r * allowed_stride + i / 32] is set; bits
 *      of ids >= vocab are ignored. allowed_stride >= ceil(vocab / 32); the
 *      pointer is 4-byte aligned. Disallowed logits are replaced by -inf
 *      before any other step, so a NaN or +inf there does not make the row
 *      TSR_ROW_NONFINITE, and a row with no allowed finite logit is
 *      TSR_ROW_EMPTY (token -1).
 *  out_logprob [rows] float32 (nullable): log p~(token) of eq. 39.2 over the
 *      masked and filtered distribution, i.e. (z_tok - M) / T minus the log
 *      of sum over S of exp((z - M) / T); 0 for greedy rows (temperature 0)
 *      and NaN for rows whose status is not TSR_ROW_OK.
 * Every other argument, and the draw itself (the same uniform of counter
 * (r, 0, step)), is as in sample_rows: the call computes what sample_rows
 * computes for logits whose disallowed entries are -inf. */
int sample_rows_masked(tsr_handle h, const void* logits, int dtype, int rows, int vocab,
                       int64_t row_stride, const uint32_t* allowed, int64_t allowed_stride,
                       const tsr_params* params, uint64_t step, int32_t* out_tokens,
                       float* out_logprob, const tsr_diag* diag, void* hip_stream);

/* Per-row inputs applied to the logits before temperature and the filters
 * (device memory; every pointer may be NULL, a NULL struct means none).
 *  allowed, allowed_stride: the allowed-token bitmask, laid out and applied
 *      as in sample_rows_masked [P2 39.3].
 *  history [rows][history_stride] int32: the look-back window of each row,
 *      its last history_len token ids (0 <= history_len <= 64,
 *      history_stride >= history_len); ids outside [0, vocab) are padding.
 *  repetition_penalty: r, finite and >= 1 (TSR_EINVAL otherwise when a
 *      window is given). Every distinct id of the window has its logit
 *      rescaled once, z / r if z > 0, z * r otherwise, before anything else
 *      [P5 "The repetition penalty"]; the rescaled logit is rounded to the
 *      logits' element type (float32; bf16 to nearest even from that float32).
 *      r = 1 or history_len 0: no penalty. history NULL with history_len > 0
      is TSR_EINVAL.
 *  row_params [rows] tsr_params (device memory): each row's own sampling
 *      parameters in place of the call's `params` (which may then be NULL);
 *      a row whose parameters tsr_params would reject gets
 *      TSR_ROW_BADPARAM and token -1 (checked on the device, per row). */
typedef struct {
  const uint32_t* allowed;
  int64_t allowed_stride;
  const int32_t* history;
  int32_t history_len;
  int64_t history_stride;
  double repetition_penalty;
  const tsr_params* row_params;
} tsr_constraints;

/* sample_rows with the per-row inputs of `cons` (nullable) and log p~ of each
 * drawn token (out_logprob, nullable, as in sample_rows_masked). The penalty
 * applies first, then the mask; everything after is sample_rows.
 * sample_rows_masked(..., allowed, allowed_stride, ...) is this call with a
 * constraint holding the mask only. */
int sample_rows_ex(tsr_handle h, const void* logits, int dtype, int rows, int vocab,
                   int64_t row_stride, const tsr_constraints* cons, const tsr_params* params,
                   uint64_t step, int32_t* out_tokens, float* out_logprob,
                   const tsr_diag* diag, void* hip_stream);

/* The speculative verify step [P3 "The Algorithm"; P1, P4 "Speculative
 * decoding"; P2 39.4] for `rows` sequences with K drafted tokens each.
 *  target_logits [rows][K+1][vocab]: the target's logits at the K draft
 *      positions and at the position after them.
 *  draft_logits  [rows][K][vocab]:   the draft's logits (not read when the
 *      temperature is 0).
 *  draft_tokens  [rows][K] int32:    the drafted ids.
 * Both distributions go through the same chain (temperature and filters),
 * p~ and q~. For j = 0..K-1 in order, with (w0, w1) the Philox words of
 * counter (row, j | 1 << 16, step): keep x_j iff w0 * 2^-32 <
 * min(1, p~(x_j) / max(q~(x_j), 1e-300)) (eq. 39.3); at the first rejection
 * emit a draw from max(0, p~ - q~) / Z with w1 (eq. 39.4) and stop; if every
 * draft is kept emit a bonus draw from the target's row K with w0 of
 * position K. Greedy (temperature 0): keep x_j iff it is the target's argmax,
 * emit the argmax at the first mismatch, the bonus is row K's argmax.
 *  out_tokens   [rows][K+1]: emitted ids, -1 after the last one.
 *  out_accepted [rows]:      number of drafts kept (0..K).
 *  out_status   [rows] (nullable): TSR_ROW_*; a bad sequence gets all -1 and 0.
 * 1 <= K <= max_k (set by sampler_init) and K <= 32. vocab <= 155,648 bf16
 * or 77,824 float32 logits (TSR_EUNSUPPORTED beyond). Up to 65,536 bf16 or
 * 32,768 float32 logits each position's two rows are held in one workgroup's
 * registers; wider rows take one workgroup per row, then one per sequence,
 * which re-reads the rejecting position's rows for the residual draw. */
int spec_verify(tsr_handle h, const void* target_logits, const void* draft_logits,
                int dtype, const int32_t* draft_tokens, int rows, int K, int vocab,
                const tsr_params* params, uint64_t step, int32_t* out_tokens,
                int32_t* out_accepted, int32_t* out_status, void* hip_stream);

/* spec_verify for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * No handle: the Philox key is `seed` (as sampler_init's), and the call runs
 * on `device` (made current for the call, the caller's restored after). The
 * verify workspace is a static device array in the library, 1 MiB, one
 * copy per device, held until the process ends; the call allocates nothing
 * and calls no allocating routine. Limits of that array: rows <= 16384 and
 * rows * (K + 1) <= 65536 (TSR_EINVAL beyond); 1 <= K <= 32; vocab <= 65,536
 * bf16 or 32,768 float32 logits (TSR_EUNSUPPORTED beyond: the array holds no
 * per-row records for spec_verify's wider-row path). Every call on a device shares that device's array: calls that overlap on
 * one device (on different streams, or from several threads) race and give
 * undefined results. Arguments, outputs and results are spec_verify's. */
int spec_verify_noalloc(int device, uint64_t seed, const void* target_logits,
                        const void* draft_logits, int dtype, const int32_t* draft_tokens,
                        int rows, int K, int vocab, const tsr_params* params, uint64_t step,
                        int32_t* out_tokens, int32_t* out_accepted, int32_t* out_status,
                        void* hip_stream);

/* Tree (multi-candidate) verify [P3 "Extensions and Variants": the draft
 * proposes a tree of candidates with several branches and the target
 * verifies every path; P2 39.4 for the rule at one candidate] for `rows`
 * sequences of `nodes` tree nodes each (1 <= nodes <= 32 and <= max_k + 1).
 *  parent [rows][nodes] int32: node 0 is the current context (parent -1);
 *      node n > 0 extends node parent[n] < n (else the sequence gets status 5).
 *  tokens [rows][nodes] int32: the token node n appends (tokens[0] unused).
 *  target_logits, draft_logits [rows][nodes][vocab]: the target's and the
 *      draft's logits for the token after node n's path (the draft's only read
 *      for nodes with children, and not at all at temperature 0).
 * The children of a node (in node order) are its candidates, taken as
 * independent draws from the draft's distribution q~ there. From the root:
 * child c of the current node v is kept iff w0 * 2^-32 < min(1, p_c(x) /
 * q~(x)), p_1 = p~_v and p_{c+1} = max(0, p_c - q~) normalised after each
 * rejection (w0 of the Philox counter (row, v * 32 + c | 2 << 16, step)); a
 * kept child becomes v; when every child of v is rejected, or v has none, one
 * token is drawn from the current p with w1 of (row, v * 32 | 2 << 16, step)
 * and the step ends. Temperature and filters shape p~ and q~ as in
 * spec_verify. Greedy (temperature 0): the first child holding the target's
 * argmax is kept, else the argmax is emitted.
 *  out_tokens [rows][nodes]: the kept children's tokens then the drawn one,
 *      -1 after; out_path [rows][nodes]: the kept nodes, -1 after;
 *  out_accepted [rows]: how many nodes were kept; out_status [rows]
 *      (nullable): TSR_ROW_* (NONFINITE/EMPTY for a bad target row or a bad
 *      draft row of a node with children, BADTOKEN for a token outside
 *      [0, vocab), 5 for a parent that is not an earlier node).
 * vocab limits as spec_verify's (above 65,536 bf16 or 32,768 float32 logits,
 * one workgroup per row, then one per sequence that follows the tree and
 * streams the rows of the nodes where candidates were rejected).
 * Shares the verify workspace: not concurrent with spec_verify on the handle. */
int tree_verify(tsr_handle h, const void* target_logits, const void* draft_logits, int dtype,
                const int32_t* parent, const int32_t* tokens, int rows, int nodes, int vocab,
                const tsr_params* params, uint64_t step, int32_t* out_tokens, int32_t* out_path,
                int32_t* out_accepted, int32_t* out_status, void* hip_stream);

/* One beam-search step [P2 39.1: eq. 39.1, Listing 39.1; P4 "Beam search"]
 * for `groups` independent searches of `beam` beams each (no length penalty
 * or end token, as in the listing).
 *  logits [groups * beam][vocab]: row g * beam + b holds beam b of group g,
 *      row_stride elements apart (vocab beyond 155,648 bf16 or 77,824
 *      float32 logits: TSR_EUNSUPPORTED).
 *  beam_scores [groups * beam] double: each beam's running score s_b, the sum
 *      of its tokens' log-probabilities (eq. 39.1); -inf marks a dead beam.
 * Every candidate (b, i) scores s_b + log softmax(logits_b)_i (temperature
 * 1, the row's own normalisation, so a row without a finite logit adds
 * nothing); the `beam` best of the group's beam * vocab candidates are kept,
 * best first, equal scores in the order (b, then i) ascending.
 *  out_parent [groups * beam] int32: the beam (0..beam-1) each kept candidate
 *      extends; out_token the token; out_score (double) its score. Positions
 *      past the group's finite candidates hold -1, -1, -inf.
 *  out_status [groups] (nullable): TSR_ROW_OK; TSR_ROW_NONFINITE when a NaN or
 *      +inf logit or score is in the group (outputs -1, -1, NaN);
 *      TSR_ROW_EMPTY when no candidate is finite.
 * 1 <= beam <= 16 and groups * beam <= max_rows (TSR_EINVAL otherwise). Uses
 * per-handle workspace: not concurrent with another beam_step on the handle. */
int beam_step(tsr_handle h, const void* logits, int dtype, int groups, int beam, int vocab,
              int64_t row_stride, const double* beam_scores, int32_t* out_parent,
              int32_t* out_token, double* out_score, int32_t* out_status, void* hip_stream);

/* Test hook: out_words[i][0..3] = Philox4x32-10(counters[i][0..3], key = the
 * handle's seed) for i < n, computed on the device by the same function the
 * sampler uses. counters and out_words are device memory. */
int sampler_philox(tsr_handle h, const uint32_t* counters, int n, uint32_t* out_words,
                   void* hip_stream);

/* Static description of a return code. */
const char* sampler_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* TSR_H_ */

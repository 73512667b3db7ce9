/*
 * tsel.h -- C ABI of libtsel.so: batched token selection over the logits of
 * one decode step, one step of beam search, and verification of assistant
 * drafts, on AMD Instinct MI355X (gfx950).
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" point to GPU memory; everything else is host.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued asynchronously on it; results are valid after the
 *    caller synchronizes the stream.
 *  - The caller allocates and frees every buffer (logits, history, masks,
 *    outputs, workspace).  The library keeps no allocation between calls and
 *    no state that changes a result (it only remembers, per device, that a
 *    kernel's LDS limit is raised), so independent calls may run
 *    concurrently on different streams.  (The pages' generation loop
 *    likewise frees only the tensors it made and never the caller's:
 *    "Transmuter.Generation", section "Device memory".)
 *  - Return value: TSEL_OK, or a negative tsel_status that is decided on the
 *    host before anything is enqueued (invalid or unsupported arguments), or
 *    TSEL_ERR_LAUNCH when the runtime refuses a launch.  Faults inside a
 *    kernel surface at the caller's stream synchronization.  No entry point
 *    prints, throws or exits.
 *  - Inputs and outputs must not alias.
 */
#ifndef TSEL_H
#define TSEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t tsel_status;
#define TSEL_OK 0
#define TSEL_ERR_INVALID_ARG (-1)  /* an argument is out of its documented range */
#define TSEL_ERR_UNSUPPORTED (-2)  /* valid, but outside what this build handles */
#define TSEL_ERR_LAUNCH (-3)       /* the HIP runtime refused a launch */
#define TSEL_ERR_WORKSPACE (-4)    /* workspace missing or too small */

/* Element type of the logits. */
#define TSEL_F32 0
#define TSEL_BF16 1

/* Initial number of draft tokens of assisted generation ("Assisted
 * Generation: a new direction toward low-latency text generation", section
 * "Greedy decoding with assisted generation", step 1). */
#define TSEL_INITIAL_K 5

/* Largest number of eos ids a call carries. */
#define TSEL_MAX_EOS 8

/*
 * Generation settings of one call, named as in generation_config.json.  Read
 * on the host at call time (the struct may be reused or freed after the call
 * returns).  Section references are to "Transmuter.Generation (transmuter
 * v2.0.0)": the module doc fixes the processor order, "Lengths" the length
 * rules, "Processors" the static masks.
 */
typedef struct tsel_params {
  int32_t batch;                /* B >= 0 rows; B == 0 is a no-op */
  int32_t vocab;                /* V >= 1 */
  int64_t logits_row_stride;    /* elements between consecutive logits rows */
  int32_t dtype;                /* TSEL_F32 or TSEL_BF16 */
  int32_t hist_stride;          /* int32 elements between history rows, >= every len */

  float repetition_penalty;     /* > 0; 1 = off.  Seen id: score < 0 -> score * p,
                                   else score / p (module doc, first processor) */
  int32_t no_repeat_ngram_size; /* >= 0; 0 = off ("Lengths") */
  const uint32_t *bad_words_mask;      /* device bitmask of single-token bad words, or NULL */
  const uint32_t *suppress_mask;       /* device bitmask of suppress_tokens, or NULL */
  const uint32_t *begin_suppress_mask; /* device bitmask of begin_suppress_tokens, or NULL */
  int32_t min_length;           /* >= 0; 0 = off */
  int32_t min_new_tokens;       /* >= 0; 0 = off; when > 0 it replaces min_length */
  int32_t n_eos;                /* 0 .. TSEL_MAX_EOS */
  int32_t eos_ids[TSEL_MAX_EOS];/* the eos set removed by min_length / min_new_tokens */
  int32_t forced_bos_token_id;  /* < 0 = off */
  int32_t forced_eos_token_id;  /* < 0 = off */

  int32_t do_sample;            /* 0 = greedy argmax (the warpers below are ignored) */
  float temperature;            /* > 0 when sampling; 1 = off */
  int32_t top_k;                /* >= 0; 0 = off */
  float top_p;                  /* in (0, 1]; 1 = off */

  int32_t renormalize_logits;   /* nonzero: the log-softmax of the row after the
                                   processors, before temperature (module doc) */
  int32_t output_logprobs;      /* nonzero: out_logprobs is given ("Log-probabilities") */
} tsel_params;

/*
 * tsel_process_select -- one decode step of token selection for B rows.
 *
 * Applies, per row and in this order, the processors of "Transmuter.
 * Generation" (module doc; "Lengths"): repetition_penalty,
 * no_repeat_ngram_size, single-token bad words, min_length /
 * min_new_tokens, forced_bos_token_id, forced_eos_token_id, suppress_tokens,
 * begin_suppress_tokens, renormalize_logits when set; then, when sampling,
 * temperature, top_k and top_p;
 * then selects the token: the argmax (lowest id among equal scores) when
 * greedy, else the inverse CDF of uniforms[b] over the kept ids taken in
 * (score descending, id ascending) order.  Removed ids score -inf; a forced
 * id scores 0; the penalty acts once per distinct history id; a row whose
 * every id is removed selects id 0.
 *
 *  logits      device, B rows of V elements of params->dtype, row b at
 *              logits + b * logits_row_stride, 16-byte aligned.  Any stride
 *              >= V: when logits_row_stride * element size is not a multiple
 *              of 16 the rows are first copied into the workspace at the
 *              smallest stride that is (one more read and write of the
 *              logits).  Not modified.
 *  history     device int32 [B, hist_stride]: the prompt then the new tokens
 *              of each row, oldest first; row b uses its first lens[b] ids.
 *              Ids outside [0, V) are ignored by every processor.
 *  lens        device int32 [3 * B]: lens[b] = prompt + new tokens (0 marks a
 *              padding row: token -1, nothing else computed);
 *              lens[B + b] = prompt length; lens[2B + b] = max_length
 *              (prompt length + max_new_tokens).  ("Lengths"; "Batches")
 *  uniforms    device float [B] in [0, 1), one per row; required iff sampling.
 *  out_tokens  device int32 [B]: the selected id, or -1 for a padding row.
 *  out_processed  device float [B, V] or NULL: the final scores the token is
 *              chosen from (after top_p when sampling).  A debugging and
 *              parity aid: it costs one extra pass over each row.
 *  out_logprobs   device float [B], given iff params->output_logprobs: the
 *              log-softmax of those final scores at the selected token, in
 *              binary64 rounded to binary32; the quiet NaN with sign bit 0
 *              for a padding row, and NaN for a row whose scores are all
 *              -inf ("Transmuter.Generation", "Log-probabilities", and the
 *              function doc of generate/5).  It costs a write and a read of
 *              the final scores (into the workspace when out_processed is
 *              NULL).
 *  workspace, workspace_bytes  device scratch of at least
 *              tsel_process_select_workspace_size(params) bytes, 256-byte
 *              aligned (NULL/0 when that is 0): the copied rows when the
 *              stride needs them, fp32 rows of the renormalized scores when
 *              renormalize_logits is set, and of the final scores when
 *              output_logprobs is.
 *
 * Errors: TSEL_ERR_INVALID_ARG for B < 0, V < 1, a stride below V, a
 * hist_stride below 0, penalty <= 0, n < 0, min lengths < 0, n_eos outside
 * [0, TSEL_MAX_EOS], an unknown dtype, temperature <= 0 / top_k < 0 / top_p
 * outside (0, 1] when sampling, a NULL required pointer, or out_logprobs
 * given without output_logprobs (or the reverse); TSEL_ERR_WORKSPACE when
 * the workspace is missing or too small;
 * TSEL_ERR_UNSUPPORTED for logits not 16-byte aligned or a vocabulary too
 * large for the on-chip masks (V > 524,288).
 */
tsel_status tsel_process_select(const void *logits, const int32_t *history,
                                const int32_t *lens, const tsel_params *params,
                                const float *uniforms, int32_t *out_tokens,
                                float *out_processed, float *out_logprobs, void *workspace,
                                size_t workspace_bytes, void *stream);

/* Workspace bytes tsel_process_select needs for these params (0 if none). */
size_t tsel_process_select_workspace_size(const tsel_params *params);

/*
 * tsel_validate_params -- the host-side argument checks of
 * tsel_process_select on the params alone (no pointers are dereferenced and
 * no GPU call is made).  Returns what tsel_process_select would return for
 * them.
 */
tsel_status tsel_validate_params(const tsel_params *params, int32_t sampling_uniforms_given);

/*
 * tsel_mask_build -- the static mask of a list of single token ids ("the
 * bad words of one token" and suppress_tokens, made once per group of rows:
 * "Transmuter.Generation", section "Processors").
 *
 *  ids       device int32 [n_ids]; ids outside [0, vocab) are ignored.
 *  out_mask  device uint32 [ceil(vocab / 32)]: bit (v % 32) of word v / 32
 *            is set iff v is listed.  Fully overwritten.
 * Errors: TSEL_ERR_INVALID_ARG for vocab < 1, n_ids < 0, NULL out_mask, or
 * NULL ids with n_ids > 0.
 */
tsel_status tsel_mask_build(int32_t vocab, const int32_t *ids, int32_t n_ids,
                            uint32_t *out_mask, void *stream);

/*
 * tsel_verify -- greedy verification of k assistant drafts per row
 * ("Assisted Generation: a new direction toward low-latency text
 * generation", section "Greedy decoding with assisted generation", steps
 * 3-6).  For row b and position j = 0..k, next[j] is the argmax of the raw
 * logits at that position (lowest id among equal maxima).  n_match is the
 * length of the common prefix of candidates[b] and next (comparison stops at
 * the first mismatch); the kept tokens are next[0..n_match] (the matches and
 * the first divergent token, or the extra token when all k match); the next
 * draft count is k + 2 when all k match, else max(1, k - 1).
 *
 *  logits       device [B, k+1, V] of dtype, position (b, j) at
 *               logits + (b * (k+1) + j) * row_stride; 16-byte aligned rows.
 *  candidates   device int32 [B, k] (may be NULL when k == 0).
 *  out_n_match  device int32 [B]
 *  out_tokens   device int32 [B, k+1]: kept tokens, then -1.
 *  out_next     device int32 [B]: next[n_match].
 *  out_k        device int32 [B]: the next draft count.
 *  workspace    device, 8-byte aligned, >= tsel_verify_workspace_size(B, k,
 *               V) bytes: the argmax of every chunk of every position row.
 *               Its contents before a call do not matter (each call writes
 *               what it reads); two calls in flight at once need two.
 * Errors: TSEL_ERR_INVALID_ARG for B < 0, k < 0, V < 1, a stride below V,
 * an unknown dtype, or NULL required pointers; TSEL_ERR_WORKSPACE when the
 * workspace is missing or too small; TSEL_ERR_UNSUPPORTED for misaligned
 * rows or workspace, k > 1023 or B * (k+1) > 65535.
 */
tsel_status tsel_verify(const void *logits, int32_t dtype, int32_t batch, int32_t k,
                        int32_t vocab, int64_t row_stride, const int32_t *candidates,
                        int32_t *out_n_match, int32_t *out_tokens, int32_t *out_next,
                        int32_t *out_k, void *workspace, size_t workspace_bytes,
                        void *stream);

/* Workspace bytes tsel_verify needs. */
size_t tsel_verify_workspace_size(int32_t batch, int32_t k, int32_t vocab);

/*
 * tsel_verify_noalloc -- tsel_verify for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops that forbid
 * allocation).  Same arguments, results and checks as tsel_verify, without
 * the workspace: its partial maxima live in a file-scope device array of
 * TSEL_NOALLOC_SCRATCH_BYTES that each GPU holds from its first call until
 * the process ends.  The first call on a device (device ids below 64) takes
 * the array's address; no call allocates or frees memory, and nothing in the
 * array needs to start at zero.  Every call on one
 * GPU shares that GPU's array, so calls that overlap in time on one GPU race
 * and give wrong results: the caller orders them (e.g. one stream).
 * Errors: as tsel_verify; TSEL_ERR_UNSUPPORTED when
 * tsel_verify_workspace_size(batch, k, vocab) exceeds
 * TSEL_NOALLOC_SCRATCH_BYTES; TSEL_ERR_LAUNCH also for a device id of 64 or
 * more.
 */
#define TSEL_NOALLOC_SCRATCH_BYTES (1u << 20)
tsel_status tsel_verify_noalloc(const void *logits, int32_t dtype, int32_t batch, int32_t k,
                                int32_t vocab, int64_t row_stride, const int32_t *candidates,
                                int32_t *out_n_match, int32_t *out_tokens, int32_t *out_next,
                                int32_t *out_k, void *stream);

/*
 * tsel_verify_select -- verification of k assistant drafts per row with the
 * token selection method of the step ("Assisted Generation: a new direction
 * toward low-latency text generation", "Greedy decoding with assisted
 * generation", step 3: ".argmax() for greedy search or .multinomial() for
 * sampling"; "Sample with assisted generation").  Position j of row b was
 * computed after the row's history and the drafts 0..j-1; its token is
 * tsel_process_select's selection of that position row, whose history is
 * the row's history followed by candidates[b][0..j-1] and whose length is
 * lens[b] + j (prompt length and max_length unchanged; a padding row stays
 * one), drawing with uniforms[b * (k+1) + j] when sampling.  The matches,
 * kept tokens, next token and next draft count then follow as in
 * tsel_verify: drafts are accepted left to right while they equal the
 * selected token.
 *
 *  logits      device [B, k+1, params->logits_row_stride] of params->dtype
 *              (16-byte aligned; any stride >= V, as tsel_process_select);
 *              params->batch is B.
 *  history, lens  as tsel_process_select (history [B, params->hist_stride],
 *              lens [3 * B]).
 *  params      the selection settings (processors, warpers,
 *              renormalize_logits); output_logprobs must be 0.
 *  candidates  device int32 [B, k] (NULL when k == 0).
 *  uniforms    device float [B * (k+1)], required iff sampling.
 *  out_n_match, out_tokens [B, k+1], out_next, out_k  as tsel_verify.
 *  workspace   device, 256-byte aligned, at least
 *              tsel_verify_select_workspace_size(params, k) bytes: the
 *              position rows' histories, lengths and tokens (and what the
 *              selection itself needs, the copied rows among it).
 * Errors: those of tsel_process_select for the settings; TSEL_ERR_INVALID_ARG
 * for k < 0, output_logprobs set, or NULL required pointers;
 * TSEL_ERR_WORKSPACE for a missing or small workspace; TSEL_ERR_UNSUPPORTED
 * for k > 1023 or rows the selection's on-chip layout cannot hold.
 */
tsel_status tsel_verify_select(const void *logits, const int32_t *history, const int32_t *lens,
                               const tsel_params *params, int32_t k, const int32_t *candidates,
                               const float *uniforms, int32_t *out_n_match, int32_t *out_tokens,
                               int32_t *out_next, int32_t *out_k, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Workspace bytes tsel_verify_select needs. */
size_t tsel_verify_select_workspace_size(const tsel_params *params, int32_t k);

/*
 * tsel_beam_step -- one step of beam search ("Transmuter.Generation
 * (transmuter v2.0.0)", the beam paragraph under "Log-probabilities").  The
 * batch holds P prompts of num_beams rows each (row p * num_beams + j is
 * beam j of prompt p).  Each beam row takes the log-softmax of its logits
 * ((x - m) - ls in binary32, m the row's largest logit, ls =
 * log(sum exp(x - m)) from binary64; -inf stays -inf), then the processors
 * of tsel_process_select in their order with removed ids at -FLT_MAX (the
 * smallest finite value) instead of -inf and a forced id at 0, then adds the
 * beam's score; a candidate's score is raised to -FLT_MAX when below it.
 * Candidate (beam j, id v) has the flattened index j * V + v.  Of each
 * prompt's candidates the best K = tsel_beam_width(num_beams, n_eos) are
 * kept, by score descending and, among equal scores, by flattened index
 * ascending.  On the first step only beam 0 of a prompt gives candidates
 * (its beams are all alike); a padding beam row (lens[r] == 0) gives none.
 * Slots past a prompt's candidates hold score -inf, beam -1, id -1.
 *
 *  logits       device, params->batch = P * num_beams rows as in
 *               tsel_process_select (16-byte aligned; any stride >= V).
 *  history, lens  as tsel_process_select, one row per beam.
 *  params       the processors' settings; the warpers are not used
 *               (do_sample must be 0), nor are renormalize_logits and
 *               output_logprobs (both 0).
 *  num_beams    beams per prompt, 1 .. 64; params->batch a multiple of it.
 *  beam_scores  device float [P * num_beams]: each beam's running score
 *               (-inf for a dead beam).
 *  first_step   nonzero on the first step of the search.
 *  out_scores   device float [P, K]; out_beams, out_tokens device int32
 *               [P, K]: the kept candidates, best first.
 *  workspace    device, 256-byte aligned, at least
 *               tsel_beam_step_workspace_size(params, num_beams) bytes: the
 *               copied rows when the stride needs them, then each beam row's
 *               best K candidates.
 * Errors: those of tsel_process_select for the params; TSEL_ERR_INVALID_ARG
 * for do_sample, renormalize_logits or output_logprobs set, num_beams < 1,
 * a batch that is not a multiple of num_beams, or NULL required pointers;
 * TSEL_ERR_WORKSPACE for a missing or small workspace; TSEL_ERR_UNSUPPORTED
 * for num_beams > 64, num_beams * V >= 2^32, or V beyond the on-chip masks
 * and lists of this path (V > 344,064).
 */
tsel_status tsel_beam_step(const void *logits, const int32_t *history, const int32_t *lens,
                           const tsel_params *params, int32_t num_beams,
                           const float *beam_scores, int32_t first_step, float *out_scores,
                           int32_t *out_beams, int32_t *out_tokens, void *workspace,
                           size_t workspace_bytes, void *stream);

/* K, the candidates a prompt keeps per beam step: max(2, 1 + n_eos) *
 * num_beams (0 for num_beams < 1 or n_eos < 0). */
int32_t tsel_beam_width(int32_t num_beams, int32_t n_eos);

/* Workspace bytes tsel_beam_step needs. */
size_t tsel_beam_step_workspace_size(const tsel_params *params, int32_t num_beams);

/*
 * tsel_finish_step -- the end of one decode step for every row, on the
 * device, so that a decode loop needs no host read per step
 * ("Transmuter.Generation (transmuter v2.0.0)", function doc of generate/5:
 * a row with no new token reports -1, a finished row has no more tokens and
 * the eos token is not returned; mlxcel inference pipeline, decode loop,
 * EOS detection and stopping: a sampled id in the merged stop set ends the
 * row unemitted, and the loop also ends at the maximum length).  For row b
 * with selected token t = tokens[b]:
 *   finished[b] != 0, or t < 0:   out_tokens[b] = -1, finished[b] = 1;
 *   t one of eos_ids:             out_tokens[b] = -1, finished[b] = 1;
 *   otherwise:                    out_tokens[b] = t,
 *                                 finished[b] = (lens[b] + 1 >= max_lengths[b]).
 *
 *  tokens       device int32 [B]: the step's tokens (tsel_process_select's
 *               out_tokens, -1 for none).
 *  lens         device int32 [B]: each row's length before this token
 *               (prompt + tokens so far), as in tsel_process_select.
 *  max_lengths  device int32 [B]: each row's maximum length.
 *  eos_ids      device int32 [n_eos], the merged stop set (NULL when
 *               n_eos == 0; duplicates allowed).
 *  finished     device uint8 [B], 0 or 1: read, then overwritten with the
 *               flag after this step.
 *  out_tokens   device int32 [B]; may be the tokens buffer itself.
 * The call owns no memory; it is asynchronous on `stream`.
 * Errors: TSEL_ERR_INVALID_ARG for B < 0, n_eos < 0, or NULL required
 * pointers; TSEL_ERR_UNSUPPORTED for n_eos > 256.  B == 0 does nothing.
 */
tsel_status tsel_finish_step(int32_t batch, const int32_t *tokens, const int32_t *lens,
                             const int32_t *max_lengths, const int32_t *eos_ids, int32_t n_eos,
                             uint8_t *finished, int32_t *out_tokens, void *stream);

/* Static text for a status code. */
const char *tsel_status_string(tsel_status s);

#ifdef __cplusplus
}
#endif

#endif /* TSEL_H */

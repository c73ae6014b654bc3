/*
 * h2o.h - C ABI of the H2O (Heavy-Hitter Oracle) KV-cache hot path on MI355X (gfx950).
 *
 * What the calls compute follows the H2O pages: the summary "H2O: Heavy-Hitter
 * Oracle for Efficient Generative Inference" (sections "The mechanism" with its
 * Definition 4.3, and "Algorithm / figure walkthrough", steps 1-5) and the
 * paper's abstract.  Per (batch, head) unit the cache holds at most
 * k = recent + heavy key/value rows:
 *
 *   - the token being decoded attends over the cached rows and itself;
 *   - every softmax weight is added into that row's accumulated score, and the
 *     new token starts with its own weight;
 *   - the new token is admitted; when that makes k + 1 members, the member with
 *     the lowest score among those outside the protected window of the
 *     `recent` newest positions (the current one included) is evicted, the
 *     older position first on equal scores; so at most one membership change
 *     happens per step (Definition 4.3).
 *
 * The prefill seeds the scores with the column sums of the prompt's exact causal
 * attention and keeps the newest `recent` prompt positions plus the `heavy`
 * best-scoring older ones (ties keep the newer position); a prompt no longer
 * than k is kept whole.
 *
 * Slot layout (caller-owned state, row-major, contiguous):
 *   k_slots, v_slots : [batch, heads, k, head_dim] in kv_dtype
 *   score            : [batch, heads, k] float32, accumulated attention
 *   pos              : [batch, heads, k] int32, absolute position, -1 = empty
 *   slots [0, recent)  form a ring: position p lives in slot p % recent;
 *   slots [recent, k)  hold heavy hitters, filled from slot `recent` upward.
 *   An eviction overwrites at most two rows in place; nothing is moved.
 *   With recent = 0 (no protected window) every slot is a heavy slot and the
 *   decoded token is itself a candidate for eviction.
 *
 * Conventions
 *   - Pointers to tensors are HIP device pointers, 16-byte aligned (evicted_pos:
 *     4-byte aligned), else H2O_ERR_INVALID; config/state structs and the ctx
 *     are host memory.  `stream` is a hipStream_t (NULL = default
 *     stream).  Every call that touches device memory only enqueues work on
 *     `stream` and returns without synchronising.
 *   - All arguments are validated before any HIP call; on an error return the
 *     state buffers and the ctx counters are unchanged, except when a launch
 *     of h2o_decode_steps' per-step path fails after earlier steps were
 *     enqueued: the counters then count those steps (h2o_query).
 *   - A ctx is not thread-safe; calls on one ctx must be serialised by the
 *     caller, and consecutive calls must go to the same stream (or be ordered
 *     by the caller) because each step reads what the previous one wrote.
 *   - A ctx belongs to the device that is current at h2o_create (its scratch
 *     lives there): later calls must run with that device current, and their
 *     buffers and stream must be on it.
 *   - Device faults are reported by the caller's next synchronisation.
 */
#ifndef H2O_H
#define H2O_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct h2o_ctx h2o_ctx; /* opaque, library-owned */

typedef enum {
  H2O_OK = 0,
  H2O_ERR_INVALID = 1,     /* null pointer, size or range out of bounds */
  H2O_ERR_UNSUPPORTED = 2, /* head_dim not in {64, 96, 128}, k above the kernel limit */
  H2O_ERR_STATE = 3,       /* call order: decode before any prefill/adopted state, position overflow */
  H2O_ERR_OOM = 4,         /* scratch allocation failed */
  H2O_ERR_HIP = 5,         /* a HIP runtime call or launch failed */
  H2O_ERR_TOO_LARGE = 6    /* h2o_prefill_no_alloc: needs more than H2O_NO_ALLOC_SCRATCH_BYTES */
} h2o_status;

typedef enum { H2O_F32 = 0, H2O_BF16 = 1 } h2o_dtype;

/* How the cache stores K/V rows.  H2O_CACHE_INPUT: in kv_dtype, exact copies of
 * the input rows.  H2O_CACHE_E4M3 (kv_dtype must be H2O_BF16): OCP E4M3 codes
 * (bias 7, largest 448, round to nearest even) of x * (448 / amax) with the
 * row scale amax / 448 in float32, amax = max |x| over the row (both
 * quotients correctly rounded in float32; a zero row has zero codes and scale
 * 0).  This composes the cache with quantization (summary, "What to notice
 * when reading": H2O composes with quantization).  The prefill scores and the
 * decoded token's own attention use the exact bf16 rows. */
typedef enum { H2O_CACHE_INPUT = 0, H2O_CACHE_E4M3 = 1 } h2o_cache_dtype;

/* Eviction policy: H2O, or one of the ablations the pages contrast it with
 * (summary, "Prior limits": static Top-K without heavy-hitter dynamics;
 * "Limitations": naive Top-K each step is a different algorithm).  All three
 * attend, admit while the cache is filling, and keep the protected window the
 * same way.
 *   H2O_POLICY_H2O:    scores accumulate; the victim is the lowest (score,
 *                      position) outside the window.
 *   H2O_POLICY_STATIC: the heavy set is chosen once by the prefill scores; once
 *                      the cache is full the victim is always the position that
 *                      leaves the window (t - recent), so the heavy rows never
 *                      change and the rest is a sliding window.  Scores still
 *                      accumulate but decide nothing.
 *   H2O_POLICY_NAIVE:  a member's score is the weight of the current step only
 *                      (no accumulation); the prefill ranks prompt positions by
 *                      the attention of the last prompt token; the victim is the
 *                      lowest (score, position) outside the window.
 * The heavy-only ablation is recent = 0 under H2O_POLICY_H2O. */
typedef enum { H2O_POLICY_H2O = 0, H2O_POLICY_STATIC = 1, H2O_POLICY_NAIVE = 2 } h2o_policy;

/* How h2o_decode_steps launches its n steps.  H2O_STEPS_PERSISTENT: one
 * launch carries every (batch, head) unit through all n steps, keeping its
 * scores and positions in LDS between steps and streaming its K/V rows from
 * memory at every step; it pays off when a step moves little data (launch and
 * tail latency dominate) and loses to per-step launches with single-wavefront
 * units on large batches.  H2O_STEPS_RESIDENT: one launch that also keeps
 * each unit's K/V rows (and E4M3 row scales) in LDS across the steps, so a
 * step reads only its new token from memory (the long-stream case: summary,
 * "Algorithm / figure walkthrough", step 5, memory stays O(k)); it needs a
 * compute unit per (batch, head) unit and 2k rows plus 3k + 1 words of LDS
 * within the device's per-workgroup limit (k = 256 at d = 128 in bf16 on
 * MI355X), else one launch per step is used.  H2O_STEPS_PER_STEP: one launch
 * per step.  H2O_STEPS_AUTO: resident when it fits and n_steps > 1; else
 * persistent when every unit's workgroup fits on the device at once (the
 * runtime's occupancy for the kernel) and either the decode runs several
 * wavefronts per unit or the cached K/V rows of one step total at most 64 MiB;
 * else per step.  Persistent and resident launches also need decode_split = 1
 * and the unit's 3k + 1 words of LDS beside the kernel's own; otherwise one
 * launch per step is used.  Results are bit-identical in every mode. */
typedef enum {
  H2O_STEPS_AUTO = 0,
  H2O_STEPS_PER_STEP = 1,
  H2O_STEPS_PERSISTENT = 2,
  H2O_STEPS_RESIDENT = 3
} h2o_steps_mode;

/* Longest prompt a ctx can be created for (max_prompt). */
#define H2O_MAX_PROMPT (1 << 28)

/* Largest budget k = recent + heavy the decode kernel accepts (its per-row
 * logits live in LDS). */
#define H2O_MAX_K 8192

typedef struct {
  int32_t batch;       /* >= 1 */
  int32_t heads;       /* >= 1 */
  int32_t head_dim;    /* 64, 96 or 128 */
  int32_t recent;      /* r >= 0: size of the protected window (includes the decoded token) */
  int32_t heavy;       /* h >= 0: heavy-hitter slots; 1 <= k = r + h <= H2O_MAX_K */
  int32_t max_prompt;  /* 0 <= max_prompt <= H2O_MAX_PROMPT: longest prompt h2o_prefill will accept
                          (sizes the scratch) */
  int32_t kv_dtype;    /* h2o_dtype of q, k, v inputs and of the K/V slots */
  float scale;         /* softmax scale; 0 selects 1/sqrt(head_dim) */
  int32_t start_pos;   /* adopt an existing state: position of the next token to decode */
  int32_t start_live;  /* adopt an existing state: number of live slots (0 = no state yet) */
  int32_t decode_waves;/* wavefronts per decode workgroup: 0 = automatic, else 1, 2, 4 or 8 */
  int32_t decode_split;/* decode workgroups per (batch, head) unit: 0 = automatic, 1 = one,
                          2..64 = that many (each streams a share of the rows).  Automatic
                          splits only when the units are fewer than the device's compute
                          units, the workgroups have 8 wavefronts, k >= 768 and every
                          share keeps at least 256 rows (long contexts at small
                          batch) */
  int32_t cache_dtype; /* h2o_cache_dtype */
  int32_t policy;      /* h2o_policy */
  int32_t steps_mode;  /* h2o_steps_mode */
} h2o_config;

typedef struct {
  void* k_slots;       /* [B, H, k, d] kv_dtype, or uint8 E4M3 codes; device */
  void* v_slots;       /* [B, H, k, d] likewise */
  float* score;        /* [B, H, k] float32, device */
  int32_t* pos;        /* [B, H, k] int32, device */
  float* k_scale;      /* [B, H, k] float32 row scales, device (E4M3 cache; else may be NULL) */
  float* v_scale;      /* [B, H, k] float32 row scales, device (E4M3 cache; else may be NULL) */
} h2o_state;

/* Create a context bound to a caller-owned state.  Allocates the prefill
 * scratch (row statistics and column sums, 2 * B * H * max_prompt floats,
 * max_prompt rounded up to 16) and, when the decode is split over S > 1
 * workgroups per unit, the split scratch (B * H * (S * (d + 2) + k + 1)
 * floats and B * H arrival counters, zeroed here) with
 * hipMalloc on the current device; the state buffers are neither allocated nor
 * touched.  With start_live > 0 the ctx adopts the state already in the
 * buffers: it must satisfy min(start_pos, recent) <= start_live <= min(start_pos, k),
 * start_live == start_pos when start_pos < recent, and the slot layout above.
 * On success *out receives the ctx; on error *out is left unchanged. */
h2o_status h2o_create(const h2o_config* cfg, const h2o_state* state, h2o_ctx** out);

/* Prefill from a prompt of prompt_len tokens (summary, "Algorithm / figure
 * walkthrough", step 1).  q, k, v: [B, H, prompt_len, d] kv_dtype, device,
 * read only.  Overwrites the whole state: scores become the causal-attention
 * column sums of the kept positions, K/V rows are copied into their slots,
 * unused slots get pos = -1 and score = 0 (their K/V rows and E4M3 scales are
 * left as they were and are never read).  Afterwards the next decoded
 * position is prompt_len.  1 <= prompt_len <= max_prompt, else
 * H2O_ERR_INVALID.  Three kernels on `stream`. */
h2o_status h2o_prefill(h2o_ctx* ctx, const void* q, const void* k, const void* v,
                       int32_t prompt_len, void* stream);

/* h2o_prefill that also returns the attention output of every prompt position
 * (summary, "Algorithm / figure walkthrough", step 1: the prompt is processed
 * with full causal attention over its own prefix before any eviction):
 * out[b, h, i, :] = sum_{j <= i} softmax_j(scale * q_i . k_j) v_j.  out:
 * [B, H, prompt_len, d] float32, device, 16-byte aligned, written whole.  The
 * cache state afterwards is the one h2o_prefill leaves.  For bf16 inputs the
 * probabilities enter the value product rounded to bf16 (relative error at most
 * 2^-8 per weight); the row statistics and sums stay float32.  out == NULL is
 * h2o_prefill.  Same errors as h2o_prefill, plus H2O_ERR_INVALID for a
 * misaligned out.  Three kernels on `stream`. */
h2o_status h2o_prefill_with_output(h2o_ctx* ctx, const void* q, const void* k, const void* v,
                                   int32_t prompt_len, float* out, void* stream);

/* One decode step for every unit (summary, "Algorithm / figure walkthrough",
 * steps 2-4; "The mechanism", H2O eviction).  q, k_new, v_new: [B, H, d]
 * kv_dtype, device, the token at the current position t.  out: [B, H, d]
 * float32, device, receives the attention output.  evicted_pos: [B, H] int32,
 * device, receives the evicted absolute position or -1; may be NULL.  Updates
 * score/pos/K/V in place and advances t by one.  One kernel on `stream`;
 * allocates nothing.  H2O_ERR_STATE before any prefill or adopted state, or
 * when t would exceed INT32_MAX - 1. */
h2o_status h2o_decode_step(h2o_ctx* ctx, const void* q, const void* k_new, const void* v_new,
                           float* out, int32_t* evicted_pos, void* stream);

/* n_steps consecutive decode steps over tokens known in advance, as when a
 * long stream is fed through the cache (summary, "Algorithm / figure
 * walkthrough", step 5; "Results and evidence", long streams).  Identical in
 * effect to n_steps calls of h2o_decode_step with the step-s slices
 * q[s], k_new[s], v_new[s] -> out[s], evicted_pos[s], without a host round
 * trip per step.  q, k_new, v_new: [n_steps, B, H, d] kv_dtype; out:
 * [n_steps, B, H, d] float32; evicted_pos: [n_steps, B, H] int32 or NULL.
 * n_steps >= 1 and t + n_steps must stay below INT32_MAX - 1, else
 * H2O_ERR_INVALID / H2O_ERR_STATE before anything is enqueued.  n_steps
 * kernels on `stream`; allocates nothing.  On a launch error the counters
 * reflect the steps that were enqueued. */
h2o_status h2o_decode_steps(h2o_ctx* ctx, int32_t n_steps, const void* q, const void* k_new,
                            const void* v_new, float* out, int32_t* evicted_pos, void* stream);

/* How h2o_decode_steps would launch n_steps steps on this ctx now:
 * *mode = H2O_STEPS_RESIDENT or H2O_STEPS_PERSISTENT (one launch, with or
 * without the rows held in LDS) or H2O_STEPS_PER_STEP (one launch per step),
 * after the steps_mode of the config and the device checks it implies.  May
 * ask the runtime for device attributes (once per ctx); enqueues nothing. */
h2o_status h2o_steps_launch(h2o_ctx* ctx, int32_t n_steps, int32_t* mode);

/* Host-side counters: position of the next token to decode and number of live
 * slots per unit (the same for every unit).  Either pointer may be NULL. */
h2o_status h2o_query(const h2o_ctx* ctx, int32_t* next_pos, int32_t* n_live);

/* Decode launch shape chosen at h2o_create: wavefronts per workgroup and
 * workgroups per (batch, head) unit (1 = no split), after the automatic
 * choices and the LDS check.  Either pointer may be NULL. */
h2o_status h2o_launch_shape(const h2o_ctx* ctx, int32_t* decode_waves, int32_t* decode_split);

/* Scratch bytes h2o_prefill_no_alloc may use on a device (32 MiB). */
#define H2O_NO_ALLOC_SCRATCH_BYTES (32u << 20)

/* h2o_prefill_with_output for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops that must not call hipMalloc, and
 * harnesses that forbid it.  It allocates nothing (no hipMalloc, hipFree or
 * allocating library routine): the row statistics and column sums go to a
 * fixed array of H2O_NO_ALLOC_SCRATCH_BYTES in the library's code object,
 * which every device the library runs on holds until the process ends, instead
 * of the ctx's scratch.  The ctx may therefore be created with max_prompt = 0
 * (then h2o_create allocates no device memory either, unless the decode is
 * split).  Same kernels and same results as h2o_prefill_with_output; out ==
 * NULL is h2o_prefill.  Needs 2 * batch * heads * round_up(prompt_len, 16) * 4
 * bytes of that array: a larger call returns H2O_ERR_TOO_LARGE before anything
 * is enqueued, as do the errors of h2o_prefill_with_output except that
 * prompt_len is not bounded by max_prompt (1 <= prompt_len <= H2O_MAX_PROMPT).
 * All calls on one device share its array and leave their contents in it:
 * calls that overlap on one device (other streams, threads or contexts) race,
 * so the caller must order them.  The first call on a device asks the runtime
 * for the array's address on that device (H2O_ERR_HIP if that fails). */
h2o_status h2o_prefill_no_alloc(h2o_ctx* ctx, const void* q, const void* k, const void* v,
                                int32_t prompt_len, float* out, void* stream);

/* Free the scratch and the ctx.  NULL-safe.  Never frees caller buffers.  The
 * caller must make sure no enqueued work still uses the ctx's scratch. */
h2o_status h2o_destroy(h2o_ctx* ctx);

/* Static description of a status code. */
const char* h2o_status_string(h2o_status status);

#ifdef __cplusplus
}
#endif

#endif /* H2O_H */

/*
 * dlm.h -- C ABI of the MI355X (gfx950) denoising-step engine for masked
 * diffusion language models with converged-token locking.
 *
 * Method: SureLock, as explained on the page "Stopping Computation for
 * Converged Tokens in Masked Diffusion-LM Decoding" (gist.science explainer,
 * §1 Problem statement, §2 Methodology).  A denoising iteration recomputes
 * only the M positions that are still active; locked positions keep their
 * per-layer K and V in a cache that every active query still attends to, so
 * the per-step cost is O(M N d) + O(M d^2) instead of O(N^2 d).  Positions
 * are unmasked by confidence-ranked top-k inside semi-autoregressive blocks
 * (page "Accelerating Diffusion LLMs with SlowFast Sampling", §1 and §2).
 *
 * Conventions
 *  - Every call returns an int status: DLM_OK or a negative DLM_E_* code.
 *    No call throws, exits or prints.
 *  - Argument errors are detected on the host before any launch and leave
 *    the state untouched.
 *  - Device-side numeric errors (a non-finite log-normaliser) are latched in
 *    a device word and reported as DLM_E_NUMERIC by the next dlm_step.
 *  - All launches go on the stream given to dlm_step_init.  Calls are
 *    asynchronous except where stated.  A handle is driven by one thread.
 *  - The library never allocates device memory.  Weights and prompts are
 *    caller-owned device memory, borrowed (not copied) and must outlive the
 *    handle.  All mutable state lives in the caller's state_mem block of
 *    dlm_state_bytes() bytes (256-byte aligned).
 *  - Linear maps y = x W^T store W as [out_features][in_features], row-major
 *    and contiguous.  Element type is float (DLM_FP32) or bfloat16 stored as
 *    uint16 (DLM_BF16) for every weight, norm gain and the embedding.
 */
#ifndef DLM_H
#define DLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DLM_OK = 0,
  DLM_E_INVALID = -1,     /* bad argument or descriptor */
  DLM_E_SIZE = -2,        /* state_mem too small */
  DLM_E_HIP = -3,         /* a HIP runtime call failed */
  DLM_E_STATE = -4,       /* call out of order (step twice, update before step, t >= steps) */
  DLM_E_UNSUPPORTED = -5, /* shape outside what the kernels support */
  DLM_E_NUMERIC = -6      /* device latched a non-finite posterior */
};

enum { DLM_FP32 = 0, DLM_BF16 = 1 };
enum { DLM_LOCK_NONE = 0, DLM_LOCK_TEST = 1 };
enum { DLM_SAMPLER_SEMI_AR = 0, DLM_SAMPLER_SLOWFAST = 1 };

/* Model shape.  Pre-RMSNorm bidirectional transformer, SwiGLU FFN, untied LM
 * head, no biases, rotary embedding with half-split pairs (component j with
 * j + head_dim/2, angle pos * rope_base^(-2j/head_dim)).  Query head h reads
 * K/V head h * n_kv_heads / n_heads.  The mask token's logit is forced to
 * -inf, so it is never decoded.  Requires n_heads % n_kv_heads == 0, even
 * head_dim <= 256, 0 <= mask_id < vocab. */
typedef struct {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ff, vocab, mask_id;
  float rope_base; /* <= 0: no rotary embedding */
  float rms_eps;
  int32_t dtype;   /* DLM_FP32 | DLM_BF16 */
} dlm_model_desc;

/* Device pointers, element type per dlm_model_desc.dtype.  Per-layer arrays
 * are host arrays of n_layers device pointers (read during dlm_step_init and
 * copied into the handle). */
typedef struct {
  const void* tok_emb;           /* [vocab][d_model] */
  const void* final_norm;        /* [d_model] */
  const void* lm_head;           /* [vocab][d_model] */
  const void* const* attn_norm;  /* L x [d_model] */
  const void* const* w_qkv;      /* L x [(n_heads + 2 n_kv_heads) head_dim][d_model]: q heads, k heads, v heads */
  const void* const* w_o;        /* L x [d_model][n_heads head_dim] */
  const void* const* ffn_norm;   /* L x [d_model] */
  const void* const* w_gate;     /* L x [d_ff][d_model] */
  const void* const* w_up;       /* L x [d_ff][d_model] */
  const void* const* w_down;     /* L x [d_model][d_ff] */
} dlm_weights;

/* One decoding run.  Positions [0, prompt_len) hold the prompt, the rest
 * start as mask_id.  The generated span is split into blocks of block_len;
 * the steps are split over the blocks as T_b = floor(T(b+1)/n_blk) -
 * floor(T b/n_blk), and the s-th step of block b unmasks
 * floor(G_b(s+1)/T_b) - floor(G_b s/T_b) positions (requires steps >= n_blk).
 * Lock test (policy DLM_LOCK_TEST), for every active position whose input
 * token this step was real: pass = KL defined && KL <= kl_eps && conf >=
 * conf_tau; a counter of consecutive passes locks the position at n_consec.
 * KL is KL(p_t || p_{t-1}) (kl_dir 0) or KL(p_{t-1} || p_t) (kl_dir 1).  With
 * lock_prompt_after_first_step, every prompt position locks after step 0.
 *
 * sampler DLM_SAMPLER_SLOWFAST replaces the block schedule by SlowFast's
 * two-stage cycle (SlowFast page, §2 two-stage pipeline; the page's §4
 * ablation settles on sf_kmax 8, sf_whist 2, sf_var 1.0), per sequence.
 * Candidates are the step's active positions still holding the mask; the
 * frontier s is the first.  Exploratory step: the end point (largest
 * candidate position with conf >= sf_tau_conv; none if no candidate reaches
 * it) is recorded; the stage ends when sf_whist (1..8) end points are
 * recorded and their population variance is below sf_var, or after sf_kmax
 * exploratory steps, fixing the span [s, max(last end point, s)]; otherwise
 * the sf_k most confident candidates of [s, s + block_len) commit.
 * Accelerated step (also the step that fixed the span): every in-span
 * candidate with conf > sf_tau_high commits when at least sf_k do, else the
 * sf_k most confident in-span candidates; while in-span masks remain, the
 * masked positions beyond the span leave the active set (frozen: their K/V
 * and last prediction stand), and once the span is decoded they return
 * without a previous posterior (no KL on their first step back) and a new
 * cycle starts.  The other sf_ fields are ignored for the semi-AR sampler.
 *
 * refresh_budget > 0 turns on the drift-aware refresh of locked positions
 * (Polestar page, "Polestar: Drift-Aware Cache Calibration and Token
 * Commitment ...", section "Polestar: The Smart Painter", Polestar-Cache:
 * recompute only the cached positions whose distribution drifts most, the
 * drift measured by a KL divergence).  A position's drift is the KL (kl_dir's
 * direction) between its two most recent posteriors, +inf while undefined.
 * At the start of every step, the refresh_budget locked positions of each
 * sequence with the largest drift (ties: smaller position) rejoin the active
 * set: their K/V are recomputed and their drift measured against the
 * posterior they had when last computed.  At the lock update a recomputed
 * position stays locked if that drift is at most refresh_eps and is unlocked
 * (counter cleared) otherwise; the lock test does not apply to it.  Requires
 * the semi-AR sampler and refresh_budget <= seq_len; 0 turns it off. */
typedef struct {
  int32_t batch, seq_len, prompt_len, steps, block_len;
  float kl_eps, conf_tau;
  int32_t n_consec, kl_dir, lock_prompt_after_first_step, lock_policy;
  int32_t sampler, sf_k, sf_kmax, sf_whist;
  float sf_tau_conv, sf_tau_high, sf_var;
  int32_t refresh_budget;
  float refresh_eps;
} dlm_run_desc;

/* Replay override for dlm_lock_update (host pointers).  n_commit >= 0 replaces
 * the top-k choice by the listed (seq, pos, tok) commits (with the SlowFast
 * sampler the cycle state and frozen set are then left as they were); lock_bits non-null
 * replaces the lock test: bits |= lock_bits ([batch][ceil(seq_len/64)]) and
 * the counters are set from counters ([batch][seq_len]) when non-null, else
 * kept.  With the refresh on, lock_bits also decides the positions the step
 * recomputed while locked: such a position stays locked iff its bit is set. */
typedef struct {
  const int32_t* commit_seq;
  const int32_t* commit_pos;
  const int32_t* commit_tok;
  int32_t n_commit; /* < 0: no commit override */
  const uint64_t* lock_bits;
  const int32_t* counters;
} dlm_override;

typedef struct dlm_handle dlm_handle;

/* Bytes of state_mem needed for this model and run; 0 if the descriptors are
 * invalid.  The block holds everything the method keeps between steps: the
 * per-layer K/V cache of every position (SureLock page, §2 Methodology, core
 * mechanism: locked positions keep their cached K and V), the previous
 * step's posterior of every position (§2 locking condition: the KL test
 * compares p_t with p_{t-1}), tokens, lock bits and counters, plus the
 * activations of at most batch*seq_len active rows and kernel workspace. */
size_t dlm_state_bytes(const dlm_model_desc* model, const dlm_run_desc* run);

/* Starts a decoding run (SureLock page, §1 Problem Statement: a masked
 * diffusion LM denoises the whole sequence over T steps; §2 Methodology:
 * every position starts active, the active set A_0 is all of them).
 * Validates the descriptors, carves state_mem, zeroes the lock bits, counters
 * and flags, writes tokens (prompt then mask_id) and builds the rotary table.
 * model, weights, run: host structs, read during the call (the weight
 * pointers are kept).  prompt_tokens: device int32 [batch][prompt_len]
 * (may be NULL when prompt_len == 0).  state_mem: caller-owned device memory
 * of at least dlm_state_bytes() bytes, 256-byte aligned; its contents need
 * not be initialised and it must outlive the handle.  hip_stream: a
 * hipStream_t (NULL: the default stream).  Enqueued on the stream; *out
 * receives a host-allocated handle freed by dlm_destroy.  Errors:
 * DLM_E_INVALID (bad descriptor, null or misaligned pointer), DLM_E_SIZE
 * (state_bytes too small), DLM_E_HIP (a launch failed; no handle). */
int dlm_step_init(const dlm_model_desc* model, const dlm_weights* weights,
                  const dlm_run_desc* run, const int32_t* prompt_tokens, void* state_mem,
                  size_t state_bytes, void* hip_stream, dlm_handle** out);

/* One denoising iteration over the active positions (SureLock page, §2
 * Methodology: permanent deactivation -- locked positions get no query
 * projection and no FFN; continued attention -- the active queries attend
 * to every position through the cached K/V, fresh Q/K/V only for the active
 * subset; algorithmic complexity -- attention O(M_t N d), FFN O(M_t d^2)):
 * compaction of the active set from the lock bitmask, then per layer
 * RMSNorm, QKV projection, rotary embedding and K/V scatter into the cache,
 * attention of the active queries over all seq_len cached positions,
 * out-projection, SwiGLU FFN; then final norm, LM head and the vocabulary
 * statistics the locking condition needs (log-normaliser, argmax,
 * max-probability confidence, KL against the previous step's posterior).
 * Synchronises the stream once (to read the active count).  *m_tot_out (if
 * non-null) receives the number of active rows.  Errors: DLM_E_STATE if a
 * step is pending its dlm_lock_update or all steps were taken; DLM_E_NUMERIC
 * if the previous step latched a non-finite posterior (nothing launched);
 * DLM_E_HIP if a launch failed (the state is then undefined). */
int dlm_step(dlm_handle* h, int32_t* m_tot_out);

/* State transition after dlm_step.  Commit: the top-k most confident masked
 * positions of the current semi-autoregressive block take their argmax
 * (SlowFast page, "Accelerating Diffusion LLMs with SlowFast Sampling", §1
 * confidence-based selection in semi-autoregressive blocks, §2 top-k; or
 * SlowFast's two-stage cycle, §2 two-stage pipeline, with sampler
 * DLM_SAMPLER_SLOWFAST).  Lock: the KL test with the confidence gate and the
 * monotone bitmask update (SureLock page, §2 Methodology: locking condition
 * KL(p_t || p_{t-1}) <= eps with an optional confidence gate; permanent
 * deactivation); with the refresh on, a recomputed locked position is kept
 * or unlocked by its drift against refresh_eps (Polestar page, "The Smart
 * Painter", Polestar-Cache) and every row's drift is recorded.  ov
 * (nullable, host memory) replays given decisions in
 * place of the rule (see dlm_override).  If the step latched a non-finite
 * posterior, neither commits nor locks happen (the error is returned by the
 * next dlm_step).  Asynchronous except for the copy of override arrays.
 * Errors: DLM_E_STATE without a pending step; DLM_E_INVALID for an
 * out-of-range override entry (checked before any launch). */
int dlm_lock_update(dlm_handle* h, const dlm_override* ov);

/* Device pointer and element count of a state array (aliases state_mem;
 * valid until the next dlm_step or dlm_lock_update; read-only for the
 * caller except through the documented replay path).  The arrays are the
 * method's per-step quantities (SureLock page, §2 Methodology): tokens, the
 * lock bitmask and counters, the active set A_t (row sequence / position),
 * the posterior statistics of the locking condition (argmax, confidence,
 * KL, log-normaliser, logits) and the per-layer K/V cache.  Errors:
 * DLM_E_INVALID for an unknown `what` or null outputs. */
enum {
  DLM_GET_TOKENS = 0,    /* int32  [batch][seq_len] */
  DLM_GET_LOCK_BITS = 1, /* uint64 [batch][ceil(seq_len/64)] */
  DLM_GET_COUNTERS = 2,  /* int32  [batch][seq_len] */
  DLM_GET_ROW_SEQ = 3,   /* int32  [M] sequence of each active row (this step) */
  DLM_GET_ROW_POS = 4,   /* int32  [M] position of each active row */
  DLM_GET_ARGMAX = 5,    /* int32  [M] */
  DLM_GET_CONF = 6,      /* float  [M] */
  DLM_GET_KL = 7,        /* float  [M] (NaN where undefined) */
  DLM_GET_HAS_KL = 8,    /* int32  [M] */
  DLM_GET_LSE = 9,       /* float  [M] */
  DLM_GET_LOGITS = 10,   /* float  [batch][seq_len][vocab]; rows of this step's active positions */
  DLM_GET_ROW_REAL = 11, /* int32  [M] input token was not the mask */
  DLM_GET_KCACHE = 12,   /* dtype  [L][batch][n_kv_heads][seq_len][head_dim] */
  DLM_GET_VCACHE = 13,   /* dtype  [L][batch][n_kv_heads][head_dim][seq_len] (transposed) */
  DLM_GET_FROZEN = 14,   /* uint64 [batch][ceil(seq_len/64)] SlowFast out-of-span positions */
  DLM_GET_SF_STATE = 15, /* int32  [batch][16] SlowFast cycle: phase (0 exploratory, 1
                            accelerated), span lo, span hi (exclusive), exploratory steps,
                            recorded end points n, the last n end points (up to 8), 3 unused */
  DLM_GET_HAS_PREV = 16, /* int32  [batch][seq_len] a previous-step posterior is stored */
  DLM_GET_DRIFT = 17,    /* float  [batch][seq_len] KL between the two latest posteriors
                            (+inf while undefined; kept only with the refresh on) */
  DLM_GET_REFRESH = 18   /* uint64 [batch][ceil(seq_len/64)] locked positions this step
                            recomputed (refresh on) */
};
int dlm_get(dlm_handle* h, int32_t what, const void** dev_ptr, int64_t* n);

/* Host-side counters of the last dlm_step: its step index, active count and
 * algorithmic FLOPs, the sum over the GEMM and attention launches it made
 * (SureLock page, §2 algorithmic complexity: projections and FFN on M_t
 * rows, attention of M_t queries over N keys, plus the LM head). */
int dlm_last_step_info(const dlm_handle* h, int32_t* step, int32_t* m_tot, double* flops);

/* Debug aid: fills every state array that a step writes before it reads
 * (the per-layer K/V cache, both logit buffers and log-normalisers, the
 * per-row statistics, the activations and the workspace) with a quiet NaN
 * pattern, so that a read of a value no step wrote shows up as a NaN in a
 * logit or statistic.  Tokens, lock bits, counters and flags keep what
 * dlm_step_init wrote.  Only before the first dlm_step (DLM_E_STATE
 * otherwise); enqueued on the handle's stream. */
int dlm_debug_poison(dlm_handle* h);

/* Checkpoint of a run at a step boundary, for resuming it or replaying it
 * from a chosen step.  The pages define no checkpoint; the image holds the
 * state a later step reads (SureLock page, §2 Methodology): the tokens, the
 * lock bitmask and consecutive-pass counters, the previous-posterior flags,
 * log-normalisers and logits that the next step's KL reads, the per-layer
 * K/V cache that locked positions keep attending to, the SlowFast cycle
 * state and frozen set, the last step's per-row arrays and the device's
 * latched numeric flag, plus the host counters (step index, last active count
 * and FLOPs) and a copy of the model and run descriptors.  The layout is
 * private to this library and version.
 *
 * dlm_checkpoint_bytes: size of the image for this handle (0 for null).
 * dlm_checkpoint_save: writes the image to dst, host or device memory of at
 *   least that size (owned by the caller); returns once the copy is complete.
 * dlm_checkpoint_load: restores an image into a handle made with the same
 *   model and run descriptors (byte for byte), at any step; the weights are
 *   the handle's own.  After it the handle continues exactly as the saved
 *   one would have (same kernels, same order: the steps that follow are
 *   bitwise those of the uninterrupted run).
 * Errors: DLM_E_INVALID (null pointer; on load a bad header or descriptors
 * that differ), DLM_E_STATE (a step is pending its dlm_lock_update),
 * DLM_E_SIZE (buffer smaller than dlm_checkpoint_bytes), DLM_E_HIP (a copy
 * failed; after a failed load the state is undefined). */
size_t dlm_checkpoint_bytes(const dlm_handle* h);
int dlm_checkpoint_save(dlm_handle* h, void* dst, size_t dst_bytes);
int dlm_checkpoint_load(dlm_handle* h, const void* src, size_t src_bytes);

/* Frees the handle (not state_mem).  Waits for the stream. */
int dlm_destroy(dlm_handle* h);

const char* dlm_error_string(int status);

/* Per-kernel-class timing with HIP events recorded on the handle's stream
 * around each launch (off by default).  Classes: */
enum {
  DLM_K_COMPACT = 0, DLM_K_EMBED_NORM, DLM_K_RMSNORM, DLM_K_GEMM_QKV, DLM_K_ROPE_KV,
  DLM_K_ATTENTION, DLM_K_GEMM_O, DLM_K_GEMM_GATE_UP, DLM_K_GEMM_DOWN, DLM_K_GEMM_LM_HEAD,
  DLM_K_VOCAB_STATS, DLM_K_COMMIT_LOCK, DLM_K_NUM_CLASSES
};
/* on != 0 starts timing (and clears the accumulators). */
int dlm_set_timing(dlm_handle* h, int32_t on);
/* Synchronises, then returns the summed event time (ms), launch count and
 * summed algorithmic bytes and FLOPs of a class since timing was switched on. */
int dlm_read_timing(dlm_handle* h, int32_t kclass, double* total_ms, int64_t* launches,
                    double* bytes, double* flops);

#ifdef __cplusplus
}
#endif
#endif /* DLM_H */

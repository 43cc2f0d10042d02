/*
 * dlm_ops.h -- op-level C ABI: each call launches one stage of the denoising
 * step (the same kernels and launch plans dlm_step uses) on caller buffers.
 * Used for kernel-level parity and for timing one layer in isolation.
 *
 * Conventions as in dlm.h: int status, host-side validation before any
 * launch, no allocation, all pointers are device memory unless stated,
 * launches on `stream` (a hipStream_t; NULL = default stream), asynchronous.
 * dtype is DLM_FP32 or DLM_BF16 (bf16 as uint16); "dtype" arrays below use
 * that element type.  Workspace sizes come from the *_ws_bytes queries; a
 * call given at least that much uses the same launch plan as dlm_step.
 */
#ifndef DLM_OPS_H
#define DLM_OPS_H

#include <stddef.h>
#include <stdint.h>

#include "dlm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Active-set compaction (SureLock page, §2 core mechanism: a locked position
 * leaves the active set A_t for good).  bits: uint64 [batch][ceil(seq_len/64)],
 * bit (pos % 64) of word pos/64 set = locked.  Writes the active rows in
 * ascending (seq, pos) order: row_seq, row_pos int32 [<= batch*seq_len];
 * m_b int32 [batch] (rows per sequence); row_start int32 [batch+1] (prefix
 * of m_b); ctl int32 [4]: ctl[0] = total rows M (ctl[1..3] untouched). */
int dlm_op_compact(const uint64_t* bits, int32_t batch, int32_t seq_len, int32_t* row_seq,
                   int32_t* row_pos, int32_t* m_b, int32_t* row_start, int32_t* ctl,
                   void* stream);

/* Embedding gather + RMSNorm for the active rows (SureLock page, §2: locked
 * positions get no compute at all).  tokens int32 [batch][seq_len]; emb
 * dtype [vocab][d]; g dtype [d].  Writes h float [M][d] = emb[token],
 * y dtype [M][d] = h / sqrt(mean(h^2) + eps) * g, row_real int32 [M] =
 * (token != mask_id). */
int dlm_op_embed_rmsnorm(int32_t dtype, int32_t M, int32_t d, int32_t seq_len, float eps,
                         int32_t mask_id, const int32_t* tokens, const int32_t* row_seq,
                         const int32_t* row_pos, const void* emb, const void* g, float* h,
                         void* y, int32_t* row_real, void* stream);

/* y dtype [M][d] = x / sqrt(mean(x^2) + eps) * g; x float [M][d]. */
int dlm_op_rmsnorm(int32_t dtype, int32_t M, int32_t d, float eps, const float* x,
                   const void* g, void* y, void* stream);

/* GEMM epilogues. */
enum {
  DLM_EPI_STORE_F32 = 0, /* C float [M][N] = A W^T */
  DLM_EPI_RESID_ADD = 1, /* C float [M][N] += A W^T (the residual stream) */
  DLM_EPI_SWIGLU = 2,    /* C dtype [M][N] = silu(A W^T) * (A W2^T), silu(x) = x/(1+e^-x) */
  DLM_EPI_LOGITS = 3     /* C float, row r stored at (row_seq[r]*seq_len + row_pos[r])*N;
                            column mask_id set to -inf */
};
/* Active-row GEMM on ragged M (SureLock page, §2: query projection and FFN
 * only for active rows; FFN cost O(M d^2)).  A dtype [M][K] row-major, W (and
 * W2 for SWIGLU) dtype [N][K], all 16-byte aligned.  Requires M >= 0, N > 0,
 * K > 0 (bf16 fast path: K % 64 == 0; other shapes take the generic kernel).
 * When the plan splits K (dlm_op_gemm_ws_bytes > 0), fp32 partials go to ws
 * and a second kernel sums them in split order.  Calls that share a
 * workspace must not overlap. */
size_t dlm_op_gemm_ws_bytes(int32_t dtype, int32_t epi, int32_t M, int32_t N, int32_t K);
int dlm_op_gemm(int32_t dtype, int32_t epi, int32_t M, int32_t N, int32_t K, const void* A,
                const void* W, const void* W2, void* C, const int32_t* row_seq,
                const int32_t* row_pos, int32_t seq_len, int32_t mask_id, void* ws,
                size_t ws_bytes, void* stream);

/* dlm_op_gemm without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, kernels and launch
 * plan as dlm_op_gemm given dlm_op_gemm_ws_bytes() of workspace; the split-K
 * partial sums go to a file-scope device array of
 * dlm_op_gemm_noalloc_max_bytes() bytes (8 MiB) that each GPU the library
 * runs on holds until the process ends.  The call allocates nothing.
 * Returns DLM_E_SIZE, before any launch, when the plan's partials
 * (dlm_op_gemm_ws_bytes(dtype, epi, M, N, K)) exceed that size.  Every call
 * on one GPU shares that GPU's array and the partials need no initial
 * contents (each split writes all of its own); calls that overlap on one
 * GPU (different streams, or threads) race on it and must be serialised by
 * the caller.  The stream (NULL: the current device's null stream) selects
 * the GPU. */
size_t dlm_op_gemm_noalloc_max_bytes(void);
int dlm_op_gemm_noalloc(int32_t dtype, int32_t epi, int32_t M, int32_t N, int32_t K,
                        const void* A, const void* W, const void* W2, void* C,
                        const int32_t* row_seq, const int32_t* row_pos, int32_t seq_len,
                        int32_t mask_id, void* stream);

/* The same GEMM with a forced launch configuration, for tuning and for
 * testing every configuration the plan can choose: cfg indexes the bf16 MFMA
 * tile table (dlm_op_gemm_num_configs() entries; < 0 = the default plan),
 * splits > 0 forces the split-K factor.  Needs ws of at least
 * splits*M*N*4 bytes (2x for SWIGLU) when splits > 1. */
int dlm_op_gemm_num_configs(void);
int dlm_op_gemm_config(int32_t dtype, int32_t epi, int32_t M, int32_t N, int32_t K,
                       const void* A, const void* W, const void* W2, void* C,
                       const int32_t* row_seq, const int32_t* row_pos, int32_t seq_len,
                       int32_t mask_id, int32_t cfg, int32_t splits, void* ws, size_t ws_bytes,
                       void* stream);

/* Rotary table float [seq_len][head_dim/2][2] = (cos, sin) of
 * pos * base^(-2j/head_dim), computed in double on the device. */
int dlm_op_rope_table(int32_t seq_len, int32_t head_dim, float base, float* table,
                      void* stream);

/* Rotary embedding of q and k at each row's position, then K/V scatter into
 * the cache (SureLock page, §2: K and V of positions are cached; fresh
 * Q/K/V exist only for the active subset).  qkv float [M][(nq+2nkv)hd];
 * table from dlm_op_rope_table or NULL (no rotation).  Writes q dtype
 * [M][nq hd] and, for each row, kcache dtype [batch][nkv][seq_len][hd] at
 * (row_seq, kv head, row_pos) and vcache dtype [batch][nkv][hd][seq_len]
 * (transposed) at (row_seq, kv head, :, row_pos); other cache entries are
 * untouched. */
int dlm_op_rope_scatter(int32_t dtype, int32_t M, int32_t nq, int32_t nkv, int32_t hd,
                        int32_t seq_len, const float* qkv, const int32_t* row_seq,
                        const int32_t* row_pos, const float* table, void* q, void* kcache,
                        void* vcache, void* stream);

/* Attention of the active queries over every cached position of their
 * sequence, non-causal (SureLock page, §2 continued attention; cost
 * O(M N d)): o[r][h] = sum_j softmax_j(q[r][h].k[j] / sqrt(hd)) v[j] over
 * j < seq_len, K/V head h*nkv/nq.  q dtype [M][nq hd]; kcache [batch][nkv]
 * [seq_len][hd], vcache [batch][nkv][hd][seq_len]; rows of sequence b are
 * rows [row_start[b], row_start[b+1]) (row_start int32 [batch+1], as written
 * by dlm_op_compact); o dtype [M][nq hd]. */
size_t dlm_op_attention_ws_bytes(int32_t dtype, int32_t M, int32_t batch, int32_t seq_len,
                                 int32_t nq, int32_t nkv, int32_t hd);
int dlm_op_attention(int32_t dtype, int32_t M, int32_t batch, int32_t seq_len, int32_t nq,
                     int32_t nkv, int32_t hd, const void* q, const int32_t* row_start,
                     const void* kcache, const void* vcache, void* o, void* ws,
                     size_t ws_bytes, void* stream);
/* The same attention with a forced split of the keys (splits > 0: that many
 * key ranges, partial results merged by log-sum-exp in a second pass; 0:
 * the default plan), LDS ring depth (stages 2 or 4; 0: the plan's), number
 * of key groups (key_halves 1, 2 or 4: waves sharing each block of 16
 * queries, each over its share of every key tile, merged by log-sum-exp; 0:
 * the plan's), 16-query blocks per wave (qblocks 1 or 2; 0: the plan's) and
 * keys per LDS tile (key_tile 64 or 128; 0: the plan's, which takes 128
 * only together with four key groups of its own choosing; a tile that does
 * not divide seq_len falls back to 64; 128-key tiles always run a 2-stage
 * ring),
 * for tuning sweeps; the layouts built are (key groups, query blocks) =
 * (1, 1), (2, 1), (4, 1), (2, 2), (4, 2), any other pair runs (2, 1).  ws
 * must hold dlm_op_attention_config_ws_bytes() bytes; DLM_E_SIZE otherwise. */
size_t dlm_op_attention_config_ws_bytes(int32_t dtype, int32_t M, int32_t batch, int32_t seq_len,
                                        int32_t nq, int32_t nkv, int32_t hd, int32_t splits);
int dlm_op_attention_config(int32_t dtype, int32_t M, int32_t batch, int32_t seq_len, int32_t nq,
                            int32_t nkv, int32_t hd, const void* q, const int32_t* row_start,
                            const void* kcache, const void* vcache, void* o, int32_t splits,
                            int32_t stages, int32_t key_halves, int32_t qblocks,
                            int32_t key_tile, void* ws, size_t ws_bytes, void* stream);

/* The same attention on the 32x32-MFMA kernel (bf16, head_dim 64 or 128,
 * seq_len a multiple of the layout's key tile; else DLM_E_UNSUPPORTED) with
 * a forced wave layout and key split, for tuning sweeps and for testing
 * every layout the plan may choose.  layout indexes the kernel's layout
 * table (dlm_op_attention_num_layouts() entries: keys per LDS tile, ring
 * depth, query waves, key groups, 32-query blocks per wave; -1: the plan's
 * layout); splits > 0 forces that many key ranges (clamped to the number of
 * key tiles; partial results merged by log-sum-exp in a second pass), 0 the
 * plan's count.  ws must hold dlm_op_attention_layout_ws_bytes() bytes;
 * DLM_E_SIZE otherwise. */
int dlm_op_attention_num_layouts(void);
size_t dlm_op_attention_layout_ws_bytes(int32_t dtype, int32_t M, int32_t batch, int32_t seq_len,
                                        int32_t nq, int32_t nkv, int32_t hd, int32_t splits,
                                        int32_t layout);
int dlm_op_attention_layout(int32_t dtype, int32_t M, int32_t batch, int32_t seq_len, int32_t nq,
                            int32_t nkv, int32_t hd, const void* q, const int32_t* row_start,
                            const void* kcache, const void* vcache, void* o, int32_t splits,
                            int32_t layout, void* ws, size_t ws_bytes, void* stream);

/* QKV projection with the rotary embedding and the K/V cache scatter in the
 * GEMM epilogue (SureLock page, §2: fresh Q/K/V only for the active rows,
 * K/V of every position kept in the cache), as dlm_step runs it for bf16
 * models with head_dim 128: A bf16 [M][K] (K % 64 == 0, else
 * DLM_E_UNSUPPORTED), W bf16 [(nq + 2 nkv) 128][K] (q heads, k heads, v
 * heads).  Row r (sequence row_seq[r], position row_pos[r]) writes q bf16
 * [M][nq 128] rotated, K cache bf16 [batch][nkv][seq_len][128] rotated and
 * the transposed V cache bf16 [batch][nkv][128][seq_len]; rope_table as
 * dlm_op_rope_table writes it (null: no rotation).  cfg: -1 for the default
 * tile plan, else a tile configuration whose tile stages at least one wave
 * row of fp32 results in its LDS ring (else DLM_E_UNSUPPORTED). */
int dlm_op_gemm_qkv(int32_t M, int32_t K, int32_t nq, int32_t nkv, int32_t seq_len,
                    const void* A, const void* W, const int32_t* row_seq, const int32_t* row_pos,
                    const float* rope_table, void* q, void* kcache, void* vcache, int32_t cfg,
                    void* stream);

/* Vocabulary statistics of the active rows (SureLock page, §2 locking
 * condition: KL between the current and previous posterior, confidence
 * gate).  Logits live per position: z_cur/z_prev float [batch][seq_len][V],
 * row r at (row_seq[r], row_pos[r]).  For each row, over v != mask_id:
 * lse = log sum e^z; argmax = smallest v with the largest z; conf =
 * e^{z_argmax - lse}; if has_prev[pos]: kl = KL(p_t||p_{t-1}) (kl_dir 0) or
 * KL(p_{t-1}||p_t) (kl_dir 1), where log p_{t-1} = z_prev - lse_prev[pos].
 * Writes per row argmax, conf, kl (NaN without previous), has_kl, lse_row;
 * per position lse_cur[pos] = lse and has_prev[pos] = 1.  A non-finite lse
 * sets *err = 1. */
size_t dlm_op_vocab_ws_bytes(int32_t M, int32_t V);
int dlm_op_vocab_stats(int32_t M, int32_t V, int32_t mask_id, int32_t kl_dir, int32_t seq_len,
                       const int32_t* row_seq, const int32_t* row_pos, const float* z_cur,
                       const float* z_prev, const float* lse_prev, int32_t* has_prev,
                       float* lse_cur, int32_t* argmax, float* conf, float* kl,
                       int32_t* has_kl, float* lse_row, int32_t* err, void* ws,
                       size_t ws_bytes, void* stream);

/* LM head with the vocabulary statistics fused into its epilogue (bf16
 * operands, K % 64 == 0; else DLM_E_UNSUPPORTED).  Computes, on the M
 * compacted rows, z = A W^T (A bf16 [M][K], W bf16 [V][K]) stored as
 * dlm_op_gemm's DLM_EPI_LOGITS stores it (row r at (row_seq[r], row_pos[r])
 * of z_cur [batch][seq_len][V], mask column -inf), and the same per-row and
 * per-position outputs as dlm_op_vocab_stats (SureLock page, §2 locking
 * condition) without re-reading z_cur: each output tile folds its logits and
 * the row's previous logits into online partial sums (maximum, sum of
 * e^{z-max}, and the sum the requested KL direction needs: e^{z-max}(z -
 * z_prev) for kl_dir 0, q(z_prev - z) for kl_dir 1), one partial per row and
 * column tile in ws, which a second kernel merges per row.  ws: at least dlm_op_lm_head_stats_ws_bytes(M, V, K, cfg) bytes of
 * device memory (no initial contents needed).  cfg: -1 for the default tile
 * plan, else a tile configuration index (tuning; DLM_E_UNSUPPORTED for a
 * configuration the fused epilogue is not built for). */
size_t dlm_op_lm_head_stats_ws_bytes(int32_t M, int32_t V, int32_t K, int32_t cfg);
int dlm_op_lm_head_stats(int32_t M, int32_t V, int32_t K, const void* A, const void* W,
                         float* z_cur, const int32_t* row_seq, const int32_t* row_pos,
                         int32_t seq_len, int32_t mask_id, int32_t kl_dir, const float* z_prev,
                         const float* lse_prev, int32_t* has_prev, float* lse_cur,
                         int32_t* argmax, float* conf, float* kl, int32_t* has_kl,
                         float* lse_row, int32_t* err, int32_t cfg, void* ws, size_t ws_bytes,
                         void* stream);

/* Commit + lock transition of one step (SlowFast page §1/§2: confidence-
 * ranked top-k unmasking in semi-autoregressive blocks; SureLock page §2:
 * KL lock test with confidence gate, permanent deactivation).  Per sequence:
 * among its rows whose token is mask_id and whose position is in
 * [blk_lo, blk_hi), the k with the largest conf (ties: smaller position)
 * take their argmax (if do_commit).  If do_lock and policy == DLM_LOCK_TEST:
 * each row passes iff row_real && has_kl && kl <= kl_eps && conf >= conf_tau;
 * counter = pass ? counter + 1 : 0; lock bit set when counter >= n_consec.
 * lock_prompt != 0 additionally locks positions [0, prompt_len). */
int dlm_op_commit_lock(int32_t batch, int32_t seq_len, int32_t prompt_len, int32_t mask_id,
                       int32_t blk_lo, int32_t blk_hi, int32_t k, int32_t do_commit,
                       int32_t do_lock, int32_t policy, float kl_eps, float conf_tau,
                       int32_t n_consec, int32_t lock_prompt, const int32_t* row_seq,
                       const int32_t* row_pos, const int32_t* row_start,
                       const int32_t* row_real, const int32_t* argmax, const float* conf,
                       const float* kl, const int32_t* has_kl, int32_t* tokens,
                       uint64_t* bits, int32_t* counters, void* stream);

/* One SlowFast commit decision per sequence (SlowFast page, §2 two-stage
 * pipeline; the rule dlm_run_desc documents for DLM_SAMPLER_SLOWFAST, with
 * window = the exploratory window, block_len there), as dlm_lock_update runs
 * it, without the lock test.  Device arrays: the step's rows (row_pos,
 * argmax, conf [M], sequences delimited by row_start [batch+1]); tokens
 * [batch][seq_len] (commits written), frozen bits uint64
 * [batch][ceil(seq_len/64)], has_prev int32 [batch][seq_len] (cleared for
 * the positions a finished cycle unfreezes) and the cycle state int32
 * [batch][16] (phase, lo, hi, exploratory steps, end points recorded, end
 * points[8], unused[3]; all zero at the start) are updated in place.
 * seq_len <= 4096 (the candidates are staged in LDS), else DLM_E_INVALID. */
int dlm_op_slowfast_commit(int32_t batch, int32_t seq_len, int32_t mask_id, int32_t window,
                           int32_t sf_k, int32_t sf_kmax, int32_t sf_whist, float sf_tau_conv,
                           float sf_tau_high, float sf_var, const int32_t* row_pos,
                           const int32_t* row_start, const int32_t* argmax, const float* conf,
                           int32_t* tokens, uint64_t* frozen, int32_t* has_prev,
                           int32_t* sf_state, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DLM_OPS_H */

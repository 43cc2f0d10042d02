// Host-side launchers of the engine's kernels (one per stage of the step).
// Each takes device pointers and a stream, validates nothing (the C ABI
// layer does) and returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dlm {

enum Dtype { kF32 = 0, kBF16 = 1 };
enum Epi {
  kEpiStoreF32 = 0, kEpiResidAdd = 1, kEpiSwiglu = 2, kEpiLogits = 3, kEpiQKV = 4,
  kEpiLogitsStats = 5  // logits as kEpiLogits plus per-(row, column tile) posterior partials
};

// ---- compaction -------------------------------------------------------------
// frozen (nullable): positions also out of the active set; refresh
// (nullable): locked positions that are active this step; last_step
// (nullable): [B][N] set to t for every active position
hipError_t launch_compact(const uint64_t* bits, const uint64_t* frozen, int B, int N,
                          int32_t* row_seq, int32_t* row_pos, int32_t* m_b, int32_t* row_start,
                          int32_t* ctl, hipStream_t s, const uint64_t* refresh = nullptr,
                          int32_t* last_step = nullptr, int t = 0);
// Drift-aware refresh (Polestar page, "The Smart Painter", Polestar-Cache):
// per sequence, the `budget` locked positions with the largest drift (ties:
// smaller position) into refresh [B][ceil(N/64)] (rewritten) and rlist
// [B][budget] (position by rank, -1 past the candidates).  N <= 4096.
hipError_t launch_refresh_select(int B, int N, int budget, const uint64_t* bits,
                                 const float* drift, uint64_t* refresh, int32_t* rlist,
                                 hipStream_t s);
// Puts each listed position's last posterior (logits row and log-normaliser,
// in the buffer of the step that last computed it, last_step & 1) into the
// buffer that step t reads as the previous one ((t - 1) & 1).
hipError_t launch_refresh_copy(int B, int N, int V, int budget, int t, const int32_t* rlist,
                               const int32_t* last_step, float* z0, float* z1, float* lse0,
                               float* lse1, hipStream_t s);

// ---- norms / embedding / rotary ----------------------------------------------
hipError_t launch_embed_rmsnorm(int dtype, int M, int d, int N, float eps, int mask_id,
                                const int32_t* tokens, const int32_t* row_seq,
                                const int32_t* row_pos, const void* emb, const void* g, float* h,
                                void* y, int32_t* row_real, hipStream_t s);
hipError_t launch_rmsnorm(int dtype, int M, int d, float eps, const float* x, const void* g,
                          void* y, hipStream_t s);
// RMSNorm of the residual after it absorbs split-K partials [splits][M][d].
hipError_t launch_rmsnorm_resid(int dtype, int M, int d, float eps, float* h,
                                const float* partial, int splits, const void* g, void* y,
                                hipStream_t s);
hipError_t launch_rope_table(int N, int hd, float base, float* table, hipStream_t s);
hipError_t launch_rope_scatter(int dtype, int M, int nq, int nkv, int hd, int N, const float* qkv,
                               const int32_t* row_seq, const int32_t* row_pos,
                               const float* table, void* q, void* kc, void* vc, hipStream_t s);
// Same, with the QKV values given as split-K partials [splits][M][width].
hipError_t launch_rope_scatter_split(int dtype, int M, int nq, int nkv, int hd, int N,
                                     const float* qkv, const float* partial, int splits,
                                     const int32_t* row_seq, const int32_t* row_pos,
                                     const float* table, void* q, void* kc, void* vc,
                                     hipStream_t s);

// ---- GEMM ---------------------------------------------------------------------
struct GemmArgs {
  int dtype, epi, M, N, K;
  const void* A;
  const void* W;
  const void* W2;
  void* C;
  const int32_t* row_seq;
  const int32_t* row_pos;
  int seq_len, mask_id;
  // kEpiQKV only: rotary table [seq_len][hd/2][2] (or null), q out [M][nq hd],
  // K cache [B][nkv][seq_len][hd], V cache transposed [B][nkv][hd][seq_len];
  // hd must be 128.
  const float* rope;
  void* q;
  void* kc;
  void* vc;
  int nq, nkv;
  // kEpiLogitsStats only: previous-step logits [B][seq_len][N] and
  // log-normaliser [B][seq_len], has_prev [B][seq_len] (read only), the
  // partials out [M][gemm_logits_stats_parts()] (VocabPart; S1 accumulated
  // for kl_dir 0, T1 for kl_dir 1: the sums that direction's KL needs).
  const float* zprev;
  const float* lse_prev;
  const int32_t* has_prev;
  void* parts;
  int kl_dir = 0;
};
size_t gemm_ws_bytes(int dtype, int epi, int M, int N, int K);
hipError_t launch_gemm(const GemmArgs& a, void* ws, size_t ws_bytes, hipStream_t s);
// For the float-store and residual-add epilogues: when the plan splits K, run
// only the GEMM (partials [splits][M][N] in ws) and report the split count,
// leaving the reduction to the consumer kernel; otherwise as launch_gemm with
// *splits_out = 0.
hipError_t launch_gemm_deferred(const GemmArgs& a, void* ws, size_t ws_bytes, hipStream_t s,
                                int* splits_out);
int gemm_num_configs();
// QKV projection with rotary embedding and K/V cache scatter fused into the
// epilogue (bf16, head_dim 128, K % 64 == 0); false if the shape is not
// supported (then use kEpiStoreF32 + launch_rope_scatter_split).
bool gemm_qkv_fusable(int dtype, int M, int hd, int K);
hipError_t launch_gemm_cfg(const GemmArgs& a, int cfg, int splits, void* ws, size_t ws_bytes,
                           hipStream_t s);
// LM head with the posterior statistics in its epilogue (kEpiLogitsStats):
// supported for bf16 with K % 64 == 0.  Partials per row (one per column
// tile of the plan) and their bytes; the launch never splits K and does not
// use ws.  cfg >= 0 forces a tile configuration (sweeps).
constexpr size_t kVocabPartBytes = 20;  // one partial: m, s0, s1, t1 (float), argmax (int32)
bool gemm_logits_stats_fusable(int dtype, int K);
// Whether the fused form is the faster one at this M (else the LM head with
// kEpiLogits followed by launch_vocab_stats).
bool gemm_logits_stats_preferred(int M, int N);
int gemm_logits_stats_parts(int M, int N, int K, int cfg);
size_t gemm_logits_stats_bytes(int dtype, int M, int N, int K);
hipError_t launch_gemm_logits_stats(const GemmArgs& a, int cfg, hipStream_t s);

// ---- attention -----------------------------------------------------------------
size_t attention_ws_bytes(int dtype, int M, int B, int N, int nq, int nkv, int hd);
hipError_t launch_attention(int dtype, int M, int B, int N, int nq, int nkv, int hd,
                            const void* q, const int32_t* row_start, const void* kc,
                            const void* vc, void* o, void* ws, size_t ws_bytes, hipStream_t s);
// Same with a forced split-KV count, LDS stage count and number of waves per
// 16-query block (0: the plan's).
size_t attention_cfg_ws_bytes(int dtype, int M, int B, int N, int nq, int nkv, int hd, int splits);
hipError_t launch_attention_cfg(int dtype, int M, int B, int N, int nq, int nkv, int hd,
                                const void* q, const int32_t* row_start, const void* kc,
                                const void* vc, void* o, void* ws, size_t ws_bytes, int splits,
                                int stages, int key_halves, int qblocks, int key_tile,
                                hipStream_t s);

// 32x32 MFMA attention with a forced layout (index into its layout table)
// and split count (0: the plan's); false / invalid when the layout does not
// apply (dtype, head dim, N not a multiple of its key tile).
int attention_num_layouts();
bool attention_layout_supported(int dtype, int N, int hd, int layout);
size_t attention_layout_ws_bytes(int dtype, int M, int B, int N, int nq, int nkv, int hd,
                                 int splits, int layout);
hipError_t launch_attention_layout(int dtype, int M, int B, int N, int nq, int nkv, int hd,
                                   const void* q, const int32_t* row_start, const void* kc,
                                   const void* vc, void* o, void* ws, size_t ws_bytes, int splits,
                                   int layout, hipStream_t s);

// ---- vocabulary statistics ----------------------------------------------------------
size_t vocab_ws_bytes(int M, int V);
hipError_t launch_vocab_stats(int M, int V, int mask_id, int kl_dir, int N,
                              const int32_t* row_seq, const int32_t* row_pos,
                              const float* z_cur, const float* z_prev, const float* lse_prev,
                              int32_t* has_prev, float* lse_cur, int32_t* argmax, float* conf,
                              float* kl, int32_t* has_kl, float* lse_row, int32_t* err,
                              void* ws, size_t ws_bytes, hipStream_t s);

// Merges partials [M][nparts] (from kEpiLogitsStats) and finishes the rows
// as launch_vocab_stats does.
hipError_t launch_vocab_merge_parts(int M, int nparts, int N, int kl_dir, const int32_t* row_seq,
                                    const int32_t* row_pos, const float* lse_prev,
                                    int32_t* has_prev, float* lse_cur, const void* parts,
                                    int32_t* argmax, float* conf, float* kl, int32_t* has_kl,
                                    float* lse_row, int32_t* err, hipStream_t s);

// ---- commit + lock -------------------------------------------------------------------
struct LockArgs {
  int B, N, P, mask_id, blk_lo, blk_hi, k, do_commit, do_lock, policy;
  float kl_eps, conf_tau;
  int n_consec, lock_prompt;
  const int32_t *row_seq, *row_pos, *row_start, *row_real, *argmax;
  const float *conf, *kl;
  const int32_t* has_kl;
  int32_t* tokens;
  uint64_t* bits;
  int32_t* counters;
  // SlowFast sampler (sampler 1): exploratory window, k, stage limits and
  // thresholds; per-sequence frozen bits [B][ceil(N/64)], previous-posterior
  // flags [B][N] and cycle state [B][kSfStateInts]
  int sampler, sf_window, sf_k, sf_kmax, sf_whist;
  float sf_tau_conv, sf_tau_high, sf_var;
  uint64_t* frozen;
  int32_t* has_prev;
  int32_t* sf_state;
  // nullable: the device word the statistics latch on a non-finite
  // log-normaliser; while it is set the kernel commits and locks nothing
  const int32_t* err;
  // drift-aware refresh (nullable when off): the locked positions this step
  // recomputed [B][ceil(N/64)], the drift above which one is unlocked, and
  // every position's drift [B][N] (written for each row of the step)
  const uint64_t* refresh;
  float refresh_eps;
  float* drift;
};
constexpr int kSfStateInts = 16;  // phase, lo, hi, slow_n, hist_n, hist[8], 3 unused
hipError_t launch_commit_lock(const LockArgs& a, hipStream_t s);
// refresh (nullable): positions whose lock bit the override sets outright
// (bits = bits & ~refresh | bits_or) rather than ORs
hipError_t launch_apply_override(int B, int N, int n_commit, const int32_t* cseq,
                                 const int32_t* cpos, const int32_t* ctok, const uint64_t* bits_or,
                                 const int32_t* counters, int32_t* tokens, uint64_t* bits,
                                 int32_t* cnt, hipStream_t s, const uint64_t* refresh = nullptr);
// Fills bytes / 4 words at p with the pattern v.
hipError_t launch_fill_u32(void* p, size_t bytes, uint32_t v, hipStream_t s);
hipError_t launch_init_state(int B, int N, int P, int mask_id, const int32_t* prompts,
                             int32_t* tokens, uint64_t* bits, int32_t* counters,
                             int32_t* has_prev, int32_t* ctl, uint64_t* frozen,
                             int32_t* sf_state, hipStream_t s);

}  // namespace dlm

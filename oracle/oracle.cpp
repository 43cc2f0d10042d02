// CPU oracle for one denoising iteration of a masked diffusion LM with
// converged-token locking.  TEST INFRASTRUCTURE ONLY: nothing on the product
// path may link, load or call this file; only the tests, the smoke check and
// the benchmark's CPU-baseline leg do.  It shares no code, header or table
// with the GPU engine.
//
// Sources (web explainers of the two papers):
//   [SL] "Stopping Computation for Converged Tokens in Masked Diffusion-LM
//        Decoding" (SureLock), gist.science explainer, Hindi and Arabic
//        versions with identical sections.
//   [SF] "Accelerating Diffusion LLMs with SlowFast Sampling: The Three
//        Golden Principles", gist.science explainer.
//
// What is computed, with the reading adopted where the pages are silent:
//  * Vanilla masked-diffusion decoding runs T denoising steps, each a full
//    bidirectional transformer forward over all N positions ([SL] §1 Problem
//    statement).  With locking off this file computes exactly that.
//  * SureLock keeps an active set A_t; a position leaves it for good once its
//    step-wise KL(p_t || p_{t-1}) is at most eps, optionally gated by high
//    confidence ([SL] §2 Methodology, core mechanism: locking condition and
//    permanent deactivation).  Locked positions get no query projection and no
//    FFN; their K and V stay cached, and active queries still attend to all N
//    positions through that cache ([SL] §2, continued attention).  Cost per
//    step becomes O(M_t N d) + O(M_t d^2) ([SL] §2, algorithmic complexity).
//  * The base sampler that unmasks tokens is confidence-ranked top-k inside
//    semi-autoregressive blocks ([SF] §1 Problem statement names both; [SF]
//    §2 two-stage pipeline uses top-k by confidence).
//  * The alternative sampler is SlowFast's two-stage cycle ([SF] §2, the
//    exploratory and accelerated stages): slow steps commit the top-k of a
//    window while the convergence end point (the farthest still-masked
//    position whose confidence reaches a threshold) is recorded; once the
//    variance of its last few values falls below a threshold (or after a
//    maximum number of slow steps) the span from the decoding frontier to
//    that end point is fixed, fast steps commit every in-span position above
//    a high confidence threshold (top-k when too few qualify), and the masked
//    positions beyond the span keep their last prediction and cached K/V
//    (they leave the active set) until the span is decoded.
//
//  * Optional drift-aware partial refresh of locked positions, the
//    Polestar-Cache idea on the Polestar page ("Polestar: Drift-Aware Cache
//    Calibration and Token Commitment ...", section "Polestar: The Smart
//    Painter"): instead of keeping every cached position frozen forever, go
//    back and recompute only the positions whose understanding drifts most,
//    drift measured as a KL divergence between the position's successive
//    distributions.  A locked position's drift can only be observed when it
//    is recomputed, so the reading here is: a position's drift is the KL (in
//    the run's direction) between its two most recent posteriors, kept as a
//    float32 number and +inf while undefined; at every step the
//    refresh_budget locked positions of each sequence with the largest drift
//    (ties: smaller position) join the active set, their K/V are recomputed
//    and their new drift measured against the posterior they had when last
//    computed; one whose new drift exceeds refresh_eps is unlocked (it stays
//    active until it passes the lock test again), the others stay locked.
//
// Arithmetic is fp64.  In bf16-storage mode the values the GPU engine keeps
// in bf16 are rounded to bf16 at exactly those points (the normalised GEMM
// inputs, q, the K/V cache, the attention output and the SwiGLU product);
// everything else stays fp64.  Model details the pages leave open (RMSNorm,
// half-split RoPE, SwiGLU, untied LM head, no biases) are stated where used.
//
// Every function here has a pin in tests/test_oracle_pins.py except the
// Theorem 1 error bound, whose constant the pages never give (parity unpinned,
// reported only as a diagnostic).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

extern "C" {

typedef struct {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ff, vocab, mask_id;
  double rope_base;  // <= 0: no rotary embedding
  double rms_eps;
  int32_t bf16_storage;  // 1: round the bf16-stored intermediates
} orc_model;

typedef struct {
  int32_t batch, seq_len, prompt_len, steps, block_len;
  double kl_eps, conf_tau;
  int32_t n_consec;
  int32_t kl_dir;  // 0: KL(p_t || p_{t-1}); 1: KL(p_{t-1} || p_t)
  int32_t lock_prompt_after_first_step;
  int32_t policy;  // 0: never lock; 1: lock test
  // sampler 0: semi-autoregressive top-k; 1: SlowFast ([SF] §2), with k per
  // exploratory step (also the accelerated stage's fallback), the most
  // exploratory steps per cycle, the end points in the variance window
  // (1..8), the convergence and in-span thresholds and sigma^2_stable; the
  // exploratory window is block_len positions from the decoding frontier
  int32_t sampler;
  int32_t sf_k, sf_kmax, sf_whist;
  double sf_tau_conv, sf_tau_high, sf_var;
  // drift-aware refresh of locked positions (semi-AR sampler only): locked
  // positions recomputed per sequence per step (0: off) and the drift above
  // which a recomputed position is unlocked
  int32_t refresh_budget;
  double refresh_eps;
} orc_run;

typedef struct {
  const float* tok_emb;     // [V][d]
  const float* final_norm;  // [d]
  const float* lm_head;     // [V][d]
  const float* const* attn_norm;  // L x [d]
  const float* const* w_qkv;      // L x [(nq+2nkv)hd][d]
  const float* const* w_o;        // L x [d][nq hd]
  const float* const* ffn_norm;   // L x [d]
  const float* const* w_gate;     // L x [dff][d]
  const float* const* w_up;       // L x [dff][d]
  const float* const* w_down;     // L x [d][dff]
} orc_weights;

}  // extern "C"

namespace {

const double kNegInf = -std::numeric_limits<double>::infinity();

// Nearest bfloat16 (8 significant bits, ties to even) of a double, rounded
// once.  Subnormal bf16 values are not needed by any workload here.
double bf16_round(double x) {
  if (!std::isfinite(x) || x == 0.0) return x;
  int e;
  std::frexp(x, &e);  // x = m 2^e, 0.5 <= |m| < 1
  const double scale = std::ldexp(1.0, e - 8);
  double q = std::nearbyint(x / scale) * scale;  // default mode: ties to even
  if (std::fabs(q) > 3.3895313892515355e38) q = std::copysign(INFINITY, x);
  return q;
}

inline double store(const orc_model& m, double x) {
  return m.bf16_storage ? bf16_round(x) : x;
}

// RMSNorm with gain: y = x / sqrt(mean(x^2) + eps) * g.
void rmsnorm(const double* x, const float* g, int d, double eps, double* y) {
  double ss = 0.0;
  for (int k = 0; k < d; ++k) ss += x[k] * x[k];
  const double inv = 1.0 / std::sqrt(ss / d + eps);
  for (int k = 0; k < d; ++k) y[k] = x[k] * inv * (double)g[k];
}

// Rotary position embedding, half-split pairing: component j is rotated
// with component j + hd/2 by angle pos * base^(-2j/hd).
void rope(double* u, int hd, int pos, double base) {
  if (base <= 0.0) return;
  const int half = hd / 2;
  for (int j = 0; j < half; ++j) {
    const double theta = std::pow(base, -2.0 * j / hd);
    const double a = pos * theta;
    const double c = std::cos(a), s = std::sin(a);
    const double x0 = u[j], x1 = u[j + half];
    u[j] = x0 * c - x1 * s;
    u[j + half] = x0 * s + x1 * c;
  }
}

// y[M][N] = x[M][K] W^T, with W stored [N][K].
void linear(const double* x, const float* W, int M, int N, int K, double* y) {
#pragma omp parallel for schedule(dynamic, 8)
  for (int n = 0; n < N; ++n) {
    const float* w = W + (size_t)n * K;
    for (int i = 0; i < M; ++i) {
      const double* xi = x + (size_t)i * K;
      double acc = 0.0;
      for (int k = 0; k < K; ++k) acc += xi[k] * (double)w[k];
      y[(size_t)i * N + n] = acc;
    }
  }
}

double silu(double v) { return v / (1.0 + std::exp(-v)); }

// Attention of one query head over keys 0..n-1 of one K/V head:
// o = sum_j softmax_j(q.k_j / sqrt(hd)) v_j, non-causal.
void attend(const double* q, const double* K, const double* V, int n, int hd,
            double* o, double* scratch) {
  const double scale = 1.0 / std::sqrt((double)hd);
  double mx = kNegInf;
  for (int j = 0; j < n; ++j) {
    double s = 0.0;
    for (int c = 0; c < hd; ++c) s += q[c] * K[(size_t)j * hd + c];
    s *= scale;
    scratch[j] = s;
    mx = std::max(mx, s);
  }
  double den = 0.0;
  for (int c = 0; c < hd; ++c) o[c] = 0.0;
  for (int j = 0; j < n; ++j) {
    const double p = std::exp(scratch[j] - mx);
    den += p;
    for (int c = 0; c < hd; ++c) o[c] += p * V[(size_t)j * hd + c];
  }
  for (int c = 0; c < hd; ++c) o[c] /= den;
}

// Per-row posterior statistics over the vocabulary ([SL] §2 locking
// condition).  The mask column is excluded (its probability is 0).
//   lse = log sum_v e^{z_v}; logp = z - lse;
//   argmax = smallest v with the largest z; conf = e^{z_argmax - lse};
//   KL (dir 0) = sum_v p_v (logp_v - prev_v); (dir 1) = sum_v q_v (prev_v - logp_v)
//   where q = e^{prev}; terms whose weight is 0 contribute 0.
void vocab_stats(const double* z, const double* prev, int V, int mask_id, int kl_dir,
                 double* lse_out, int32_t* argmax_out, double* conf_out, double* kl_out,
                 double* logp_out) {
  double mx = kNegInf;
  int am = -1;
  for (int v = 0; v < V; ++v) {
    if (v == mask_id) continue;
    if (z[v] > mx) { mx = z[v]; am = v; }
  }
  double s = 0.0;
  for (int v = 0; v < V; ++v) {
    if (v == mask_id) continue;
    s += std::exp(z[v] - mx);
  }
  const double lse = mx + std::log(s);
  *lse_out = lse;
  *argmax_out = am;
  *conf_out = std::exp(mx - lse);
  for (int v = 0; v < V; ++v) logp_out[v] = (v == mask_id) ? kNegInf : z[v] - lse;
  if (prev) {
    double kl = 0.0;
    for (int v = 0; v < V; ++v) {
      if (v == mask_id) continue;
      const double lp = logp_out[v], lq = prev[v];
      if (kl_dir == 0) {
        const double p = std::exp(lp);
        if (p > 0.0) kl += p * (lp - lq);
      } else {
        const double q = std::exp(lq);
        if (q > 0.0) kl += q * (lq - lp);
      }
    }
    *kl_out = kl;
  } else {
    *kl_out = std::numeric_limits<double>::quiet_NaN();
  }
}

// Semi-autoregressive block schedule.  The G = N - P generated positions
// split into blocks of block_len; the T steps split over the n_blk blocks as
// T_b = floor(T(b+1)/n_blk) - floor(T b/n_blk); inside block b at its s-th step
// k = floor(G_b (s+1)/T_b) - floor(G_b s/T_b) positions are unmasked, which
// unmasks the whole block by its last step.
struct Sched { int beta, lo, hi, k; };

Sched schedule(const orc_run& r, int t) {
  const int G = r.seq_len - r.prompt_len;
  const int nblk = (G + r.block_len - 1) / r.block_len;
  Sched out{-1, 0, 0, 0};
  if (G <= 0 || t < 0 || t >= r.steps) return out;
  for (int b = 0; b < nblk; ++b) {
    const long t0 = (long)r.steps * b / nblk, t1 = (long)r.steps * (b + 1) / nblk;
    if (t >= t0 && t < t1) {
      const int Tb = (int)(t1 - t0), s = (int)(t - t0);
      const int lo = r.prompt_len + b * r.block_len;
      const int hi = std::min(r.seq_len, lo + r.block_len);
      const long Gb = hi - lo;
      out.beta = b;
      out.lo = lo;
      out.hi = hi;
      out.k = (int)(Gb * (s + 1) / Tb - Gb * s / Tb);
      return out;
    }
  }
  return out;
}

// SlowFast cycle state of one sequence.
struct SfSeq {
  int32_t phase = 0;       // 0: exploratory (slow), 1: accelerated (fast)
  int32_t lo = 0, hi = 0;  // accelerated stage: the stable span [lo, hi)
  int32_t slow_n = 0;      // exploratory steps taken in this cycle
  int32_t hist_n = 0;      // end points recorded in this cycle (at most sf_whist kept)
  int32_t hist[8] = {0, 0, 0, 0, 0, 0, 0, 0};  // the kept end points, oldest first
};

// One SlowFast commit decision for one sequence ([SF] §2 two-stage pipeline).
// Rows: this step's computed positions of the sequence (ascending), with
// their argmax and confidence; x, frozen and has_prev are the sequence's
// [N] arrays.  The readings where the page leaves a step open:
//  - candidates are the computed rows still holding the mask; the decoding
//    frontier s is the first of them;
//  - exploratory step: the end point e = the largest candidate position
//    whose confidence is >= sf_tau_conv is recorded (nothing is recorded
//    when no candidate reaches it), and the stage ends when sf_whist end
//    points are recorded and their population variance is below sf_var
//    (compared in integers: W sum e^2 - (sum e)^2 < W^2 sf_var), or after
//    sf_kmax exploratory steps; the span is then [s, max(e', s)] with e' the
//    last recorded end point (s if none), and the same step already commits
//    by the accelerated rule;
//  - otherwise the exploratory step commits the sf_k most confident
//    candidates in the window [s, s + block_len) (ties: smaller position);
//  - accelerated step: every in-span candidate with confidence > sf_tau_high
//    commits if there are at least sf_k of them, else the sf_k most
//    confident in-span candidates do;
//  - while in-span masks remain, masked positions at or beyond the span's
//    end leave the active set (frozen: their last prediction and K/V stand);
//    when the span is decoded the cycle ends, frozen positions return and,
//    having no posterior from the step before, start without a previous
//    posterior (no KL on their first step back).
void slowfast_commit(const orc_run& r, int mask_id, int N, int n, const int32_t* pos,
                     const int32_t* argmax, const double* conf, int32_t* x, uint8_t* frozen,
                     uint8_t* has_prev, SfSeq& st, std::vector<int32_t>* cpos,
                     std::vector<int32_t>* ctok) {
  std::vector<int> cand;
  for (int i = 0; i < n; ++i)
    if (x[pos[i]] == mask_id) cand.push_back(i);
  if (cand.empty()) return;
  const int s = pos[cand[0]];
  auto ahead = [&](int a, int c) {
    if (conf[a] != conf[c]) return conf[a] > conf[c];
    return pos[a] < pos[c];
  };
  auto commit = [&](int i) {
    x[pos[i]] = argmax[i];
    if (cpos) { cpos->push_back(pos[i]); ctok->push_back(argmax[i]); }
  };
  auto top_k = [&](std::vector<int> c) {
    std::stable_sort(c.begin(), c.end(), ahead);
    const int take = std::min<int>(r.sf_k, (int)c.size());
    for (int j = 0; j < take; ++j) commit(c[j]);
  };
  const int W = r.sf_whist;
  if (st.phase == 0) {
    int e = -1;
    for (int i : cand)
      if (conf[i] >= r.sf_tau_conv) e = std::max(e, (int)pos[i]);
    if (e >= 0) {
      if (st.hist_n < W) {
        st.hist[st.hist_n++] = e;
      } else {
        for (int j = 1; j < W; ++j) st.hist[j - 1] = st.hist[j];
        st.hist[W - 1] = e;
      }
    }
    st.slow_n += 1;
    bool stable = false;
    if (st.hist_n == W) {
      long long s1 = 0, s2 = 0;
      for (int j = 0; j < W; ++j) {
        s1 += st.hist[j];
        s2 += (long long)st.hist[j] * st.hist[j];
      }
      stable = (double)(W * s2 - s1 * s1) < (double)W * W * r.sf_var;
    }
    if (stable || st.slow_n >= r.sf_kmax) {
      st.phase = 1;
      st.lo = s;
      st.hi = std::max(st.hist_n > 0 ? st.hist[st.hist_n - 1] : s, s) + 1;
    } else {
      std::vector<int> win;
      for (int i : cand)
        if (pos[i] < s + r.block_len) win.push_back(i);
      top_k(win);
      return;
    }
  }
  std::vector<int> in, high;
  for (int i : cand)
    if (pos[i] >= st.lo && pos[i] < st.hi) in.push_back(i);
  for (int i : in)
    if (conf[i] > r.sf_tau_high) high.push_back(i);
  if ((int)high.size() >= r.sf_k) {
    for (int i : high) commit(i);
  } else {
    top_k(in);
  }
  bool left = false;
  for (int p = st.lo; p < st.hi; ++p) left = left || x[p] == mask_id;
  if (left) {
    for (int i : cand)
      if (pos[i] >= st.hi) frozen[pos[i]] = 1;
  } else {
    st = SfSeq{};
    for (int p = 0; p < N; ++p)
      if (frozen[p]) {
        frozen[p] = 0;
        has_prev[p] = 0;
      }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// State machine: init / step / lock_update, one sequence batch.
// ---------------------------------------------------------------------------
struct orc_state {
  orc_model m;
  orc_run r;
  const float* tok_emb;
  const float* final_norm;
  const float* lm_head;
  std::vector<const float*> attn_norm, w_qkv, w_o, ffn_norm, w_gate, w_up, w_down;

  int t = 0;
  std::vector<int32_t> x;          // [B][N] tokens
  std::vector<uint8_t> locked;     // [B][N]
  std::vector<int32_t> cnt;        // [B][N] consecutive passes
  std::vector<uint8_t> has_prev;   // [B][N]
  std::vector<double> kc, vc;      // [L][B][nkv][N][hd]
  std::vector<double> prevlogp;    // [B][N][V]
  std::vector<uint8_t> frozen;     // [B][N] out of the active set during an accelerated stage
  std::vector<SfSeq> sf;           // [B] SlowFast cycle state
  std::vector<float> drift;        // [B][N] KL between the two latest posteriors (+inf: none)
  std::vector<uint8_t> refresh;    // [B][N] locked positions recomputed by the last step

  // results of the last step (rows in (b, pos) ascending order)
  bool stepped = false, partial = false;
  int M = 0;
  std::vector<int32_t> row_seq, row_pos;
  std::vector<uint8_t> row_real, row_has_kl;
  std::vector<int32_t> row_argmax;
  std::vector<double> row_conf, row_kl, row_lse;
  std::vector<int32_t> logit_rows;  // which rows have logits (all, or a sample)
  std::vector<double> logits;       // [logit_rows][V]
  double flops = 0.0;
  // results of the last lock update
  std::vector<int32_t> commit_seq, commit_pos, commit_tok;
};

namespace {

size_t kv_index(const orc_state& s, int l, int b, int g, int pos) {
  const orc_model& m = s.m;
  const orc_run& r = s.r;
  return ((((size_t)l * r.batch + b) * m.n_kv_heads + g) * r.seq_len + pos) * m.head_dim;
}

// Refresh set of one step (Polestar page, "The Smart Painter", Polestar-Cache:
// recompute only where the drift is largest): per sequence, the
// refresh_budget locked positions with the largest drift, ties to the
// smaller position; refresh [B][N] is rewritten.
void refresh_select(const orc_run& r, const uint8_t* locked, const float* drift,
                    uint8_t* refresh) {
  const int N = r.seq_len;
  std::fill(refresh, refresh + (size_t)r.batch * N, 0);
  if (r.refresh_budget <= 0) return;
  for (int b = 0; b < r.batch; ++b) {
    std::vector<int> cand;
    for (int i = 0; i < N; ++i)
      if (locked[(size_t)b * N + i]) cand.push_back(i);
    const float* dr = drift + (size_t)b * N;
    std::stable_sort(cand.begin(), cand.end(), [&](int a, int c) {
      if (dr[a] != dr[c]) return dr[a] > dr[c];
      return a < c;
    });
    const int take = std::min<int>(r.refresh_budget, (int)cand.size());
    for (int j = 0; j < take; ++j) refresh[(size_t)b * N + cand[j]] = 1;
  }
}

// The lock state transition for one step: commit, then lock test.
// Inputs are the rows of the step (ascending (b, pos)) and their statistics.
void lock_transition(const orc_model& m, const orc_run& r, int t, int M,
                     const int32_t* row_seq, const int32_t* row_pos, const uint8_t* row_real,
                     const int32_t* argmax, const double* conf, const double* kl,
                     const uint8_t* has_kl, int32_t* x, uint8_t* locked, int32_t* cnt,
                     std::vector<int32_t>* cseq, std::vector<int32_t>* cpos,
                     std::vector<int32_t>* ctok, bool do_commit = true, bool do_lock = true,
                     SfSeq* sf = nullptr, uint8_t* frozen = nullptr,
                     uint8_t* has_prev = nullptr, const uint8_t* refresh = nullptr,
                     float* drift = nullptr) {
  const int N = r.seq_len;
  const bool slowfast = r.sampler == 1;
  const Sched sc = do_commit && !slowfast ? schedule(r, t) : Sched{-1, 0, 0, 0};
  if (do_commit && slowfast && sf) {
    // rows are in ascending (sequence, position) order: one contiguous run
    // per sequence
    int i0 = 0;
    for (int b = 0; b < r.batch; ++b) {
      int i1 = i0;
      while (i1 < M && row_seq[i1] == b) ++i1;
      std::vector<int32_t> bp, bt;
      slowfast_commit(r, m.mask_id, N, i1 - i0, row_pos + i0, argmax + i0, conf + i0,
                      x + (size_t)b * N, frozen + (size_t)b * N, has_prev + (size_t)b * N, sf[b],
                      &bp, &bt);
      for (size_t j = 0; j < bp.size(); ++j)
        if (cseq) { cseq->push_back(b); cpos->push_back(bp[j]); ctok->push_back(bt[j]); }
      i0 = i1;
    }
  }
  // Commit: among this step's rows whose token is still the mask and which
  // lie in the current block, the k most confident take their argmax
  // (ties: smaller position first).
  if (sc.beta >= 0) {
    for (int b = 0; b < r.batch; ++b) {
      std::vector<int> cand;
      for (int i = 0; i < M; ++i)
        if (row_seq[i] == b && x[(size_t)b * N + row_pos[i]] == m.mask_id &&
            row_pos[i] >= sc.lo && row_pos[i] < sc.hi)
          cand.push_back(i);
      std::stable_sort(cand.begin(), cand.end(), [&](int a, int c) {
        if (conf[a] != conf[c]) return conf[a] > conf[c];
        return row_pos[a] < row_pos[c];
      });
      const int take = std::min<int>(sc.k, (int)cand.size());
      for (int j = 0; j < take; ++j) {
        const int i = cand[j];
        x[(size_t)b * N + row_pos[i]] = argmax[i];
        if (cseq) { cseq->push_back(b); cpos->push_back(row_pos[i]); ctok->push_back(argmax[i]); }
      }
    }
  }
  // Drift of every recomputed position: its KL between this posterior and
  // the one before (a statistic, kept whatever decides the lock state).
  if (drift)
    for (int i = 0; i < M; ++i)
      drift[(size_t)row_seq[i] * N + row_pos[i]] =
          has_kl[i] ? (float)kl[i] : std::numeric_limits<float>::infinity();
  // Lock test: a row with a real input token passes when its KL is defined,
  // at most eps, and its confidence is at least tau; n_consec consecutive
  // passes lock it.  A locked position recomputed by the refresh instead
  // stays locked while its drift is defined and at most refresh_eps, and is
  // unlocked (counter cleared) otherwise.
  if (do_lock && r.policy == 1) {
    for (int i = 0; i < M; ++i) {
      const size_t p = (size_t)row_seq[i] * N + row_pos[i];
      if (refresh && refresh[p]) {
        if (!(has_kl[i] && kl[i] <= r.refresh_eps)) {
          locked[p] = 0;
          cnt[p] = 0;
        }
        continue;
      }
      const bool pass = row_real[i] && has_kl[i] && kl[i] <= r.kl_eps && conf[i] >= r.conf_tau;
      cnt[p] = pass ? cnt[p] + 1 : 0;
      if (cnt[p] >= r.n_consec) locked[p] = 1;
    }
    if (t == 0 && r.lock_prompt_after_first_step)
      for (int b = 0; b < r.batch; ++b)
        for (int i = 0; i < r.prompt_len; ++i) locked[(size_t)b * N + i] = 1;
  }
}

}  // namespace

extern "C" {

double orc_bf16_round(double x) { return bf16_round(x); }

orc_state* orc_create(const orc_model* m, const orc_weights* w, const orc_run* r,
                      const int32_t* prompts /* [B][P] */) {
  if (!m || !w || !r || !prompts) return nullptr;
  if (r->batch <= 0 || r->seq_len <= 0 || r->prompt_len < 0 || r->prompt_len > r->seq_len ||
      r->steps <= 0 || r->block_len <= 0 || m->n_heads % m->n_kv_heads != 0 ||
      m->head_dim % 2 != 0 || (r->sampler != 0 && r->sampler != 1) ||
      (r->sampler == 1 && (r->sf_k < 1 || r->sf_kmax < 1 || r->sf_whist < 1 || r->sf_whist > 8)) ||
      r->refresh_budget < 0 || r->refresh_budget > r->seq_len ||
      (r->refresh_budget > 0 && r->sampler != 0) || std::isnan(r->refresh_eps))
    return nullptr;
  orc_state* s = new orc_state();
  s->m = *m;
  s->r = *r;
  s->tok_emb = w->tok_emb;
  s->final_norm = w->final_norm;
  s->lm_head = w->lm_head;
  const int L = m->n_layers;
  s->attn_norm.assign(w->attn_norm, w->attn_norm + L);
  s->w_qkv.assign(w->w_qkv, w->w_qkv + L);
  s->w_o.assign(w->w_o, w->w_o + L);
  s->ffn_norm.assign(w->ffn_norm, w->ffn_norm + L);
  s->w_gate.assign(w->w_gate, w->w_gate + L);
  s->w_up.assign(w->w_up, w->w_up + L);
  s->w_down.assign(w->w_down, w->w_down + L);
  const size_t BN = (size_t)r->batch * r->seq_len;
  s->x.assign(BN, m->mask_id);
  for (int b = 0; b < r->batch; ++b)
    for (int i = 0; i < r->prompt_len; ++i)
      s->x[(size_t)b * r->seq_len + i] = prompts[(size_t)b * r->prompt_len + i];
  s->locked.assign(BN, 0);
  s->cnt.assign(BN, 0);
  s->has_prev.assign(BN, 0);
  s->frozen.assign(BN, 0);
  s->sf.assign(r->batch, SfSeq{});
  s->drift.assign(BN, std::numeric_limits<float>::infinity());
  s->refresh.assign(BN, 0);
  const size_t kvn = (size_t)L * BN * m->n_kv_heads * m->head_dim;
  s->kc.assign(kvn, 0.0);
  s->vc.assign(kvn, 0.0);
  s->prevlogp.assign(BN * (size_t)m->vocab, 0.0);
  return s;
}

void orc_destroy(orc_state* s) { delete s; }

// One denoising iteration over the active rows ([SL] §2): forward pass of the
// unlocked positions against the cached K/V of every position, then the
// posterior statistics.  If n_sample >= 0, logits and statistics are computed
// only for the listed rows (indices into the step's row list); such a step
// cannot be followed by a lock update.
int orc_step_sample(orc_state* s, const int32_t* sample_rows, int n_sample) {
  const orc_model& m = s->m;
  const orc_run& r = s->r;
  if (s->stepped) return -4;
  const int N = r.seq_len, d = m.d_model, hd = m.head_dim, nq = m.n_heads, nkv = m.n_kv_heads;
  const int dff = m.d_ff, V = m.vocab, qo = nq * hd, qkv_out = (nq + 2 * nkv) * hd;

  // Active set: every unlocked position, ascending ([SL] §2 permanent
  // deactivation), less the positions a SlowFast accelerated stage froze,
  // plus the locked positions the drift-aware refresh recomputes.
  s->row_seq.clear();
  s->row_pos.clear();
  s->row_real.clear();
  refresh_select(r, s->locked.data(), s->drift.data(), s->refresh.data());
  for (int b = 0; b < r.batch; ++b)
    for (int i = 0; i < N; ++i)
      if ((!s->locked[(size_t)b * N + i] || s->refresh[(size_t)b * N + i]) &&
          !s->frozen[(size_t)b * N + i]) {
        s->row_seq.push_back(b);
        s->row_pos.push_back(i);
        s->row_real.push_back(s->x[(size_t)b * N + i] != m.mask_id);
      }
  const int M = (int)s->row_seq.size();
  s->M = M;
  s->flops = 0.0;
  s->stepped = true;
  s->partial = n_sample >= 0;
  s->logit_rows.clear();
  s->logits.clear();
  s->row_argmax.assign(M, -1);
  s->row_conf.assign(M, NAN);
  s->row_kl.assign(M, NAN);
  s->row_lse.assign(M, NAN);
  s->row_has_kl.assign(M, 0);
  if (M == 0) return 0;

  std::vector<double> h((size_t)M * d), a((size_t)M * std::max(d, dff));
  std::vector<double> qkv((size_t)M * qkv_out), q((size_t)M * qo), o((size_t)M * qo);
  std::vector<double> g((size_t)M * dff), u((size_t)M * dff), tmp((size_t)M * d);

  for (int i = 0; i < M; ++i) {
    const float* e = s->tok_emb + (size_t)s->x[(size_t)s->row_seq[i] * N + s->row_pos[i]] * d;
    for (int k = 0; k < d; ++k) h[(size_t)i * d + k] = e[k];
  }

  for (int l = 0; l < m.n_layers; ++l) {
    // attention sublayer on the active rows only
    for (int i = 0; i < M; ++i) {
      rmsnorm(&h[(size_t)i * d], s->attn_norm[l], d, m.rms_eps, &a[(size_t)i * d]);
      for (int k = 0; k < d; ++k) a[(size_t)i * d + k] = store(m, a[(size_t)i * d + k]);
    }
    linear(a.data(), s->w_qkv[l], M, qkv_out, d, qkv.data());
    s->flops += 2.0 * M * qkv_out * d;
    for (int i = 0; i < M; ++i) {
      double* row = &qkv[(size_t)i * qkv_out];
      const int b = s->row_seq[i], pos = s->row_pos[i];
      for (int hh = 0; hh < nq + nkv; ++hh) rope(row + (size_t)hh * hd, hd, pos, m.rope_base);
      for (int c = 0; c < qo; ++c) q[(size_t)i * qo + c] = store(m, row[c]);
      // fresh K/V of an active position replace its cache entry
      for (int gk = 0; gk < nkv; ++gk) {
        const size_t base = kv_index(*s, l, b, gk, pos);
        for (int c = 0; c < hd; ++c) {
          s->kc[base + c] = store(m, row[qo + gk * hd + c]);
          s->vc[base + c] = store(m, row[qo + nkv * hd + gk * hd + c]);
        }
      }
    }
    // every active query attends to all N cached positions of its sequence
#pragma omp parallel
    {
      std::vector<double> sc(N);
#pragma omp for collapse(2) schedule(static)
      for (int i = 0; i < M; ++i)
        for (int hh = 0; hh < nq; ++hh) {
          const int gk = hh * nkv / nq;
          const size_t base = kv_index(*s, l, s->row_seq[i], gk, 0);
          attend(&q[(size_t)i * qo + (size_t)hh * hd], &s->kc[base], &s->vc[base], N, hd,
                 &o[(size_t)i * qo + (size_t)hh * hd], sc.data());
        }
    }
    s->flops += 4.0 * M * (double)N * qo;
    for (size_t c = 0; c < o.size(); ++c) o[c] = store(m, o[c]);
    linear(o.data(), s->w_o[l], M, d, qo, tmp.data());
    s->flops += 2.0 * M * d * qo;
    for (size_t c = 0; c < h.size(); ++c) h[c] += tmp[c];

    // SwiGLU FFN sublayer
    for (int i = 0; i < M; ++i) {
      rmsnorm(&h[(size_t)i * d], s->ffn_norm[l], d, m.rms_eps, &a[(size_t)i * d]);
      for (int k = 0; k < d; ++k) a[(size_t)i * d + k] = store(m, a[(size_t)i * d + k]);
    }
    linear(a.data(), s->w_gate[l], M, dff, d, g.data());
    linear(a.data(), s->w_up[l], M, dff, d, u.data());
    s->flops += 4.0 * M * dff * (double)d;
    for (size_t c = 0; c < g.size(); ++c) g[c] = store(m, silu(g[c]) * u[c]);
    linear(g.data(), s->w_down[l], M, d, dff, tmp.data());
    s->flops += 2.0 * M * d * (double)dff;
    for (size_t c = 0; c < h.size(); ++c) h[c] += tmp[c];
  }

  // final norm + LM head on the rows whose posterior is wanted
  std::vector<int32_t> rows;
  if (n_sample < 0) {
    for (int i = 0; i < M; ++i) rows.push_back(i);
  } else {
    for (int j = 0; j < n_sample; ++j)
      if (sample_rows[j] >= 0 && sample_rows[j] < M) rows.push_back(sample_rows[j]);
  }
  const int R = (int)rows.size();
  std::vector<double> af((size_t)R * d);
  for (int j = 0; j < R; ++j) {
    rmsnorm(&h[(size_t)rows[j] * d], s->final_norm, d, m.rms_eps, &af[(size_t)j * d]);
    for (int k = 0; k < d; ++k) af[(size_t)j * d + k] = store(m, af[(size_t)j * d + k]);
  }
  s->logit_rows = rows;
  s->logits.assign((size_t)R * V, 0.0);
  linear(af.data(), s->lm_head, R, V, d, s->logits.data());
  s->flops += 2.0 * M * d * (double)V;  // the step's LM-head work is for all M rows
  for (int j = 0; j < R; ++j) s->logits[(size_t)j * V + m.mask_id] = kNegInf;

  std::vector<double> logp((size_t)R * V);
#pragma omp parallel for schedule(dynamic, 1)
  for (int j = 0; j < R; ++j) {
    const int i = rows[j];
    const size_t p = (size_t)s->row_seq[i] * N + s->row_pos[i];
    const double* prev = s->has_prev[p] ? &s->prevlogp[p * V] : nullptr;
    vocab_stats(&s->logits[(size_t)j * V], prev, V, m.mask_id, r.kl_dir, &s->row_lse[i],
                &s->row_argmax[i], &s->row_conf[i], &s->row_kl[i], &logp[(size_t)j * V]);
    s->row_has_kl[i] = prev != nullptr;
  }
  if (n_sample < 0) {
    for (int j = 0; j < R; ++j) {
      const int i = rows[j];
      const size_t p = (size_t)s->row_seq[i] * N + s->row_pos[i];
      std::memcpy(&s->prevlogp[p * V], &logp[(size_t)j * V], sizeof(double) * V);
      s->has_prev[p] = 1;
    }
  }
  return 0;
}

int orc_step(orc_state* s) { return orc_step_sample(s, nullptr, -1); }

// State transition after a step: commit + lock test.  An override replaces
// a decision instead of the rule: given commits replace the top-k choice;
// given lock bits replace the lock test (locked |= bits, counters set from
// ov_cnt when given, else kept).  Used to replay near-tie decisions.
int orc_lock_update(orc_state* s, const int32_t* ov_commit_seq, const int32_t* ov_commit_pos,
                    const int32_t* ov_commit_tok, int32_t n_ov_commit,
                    const uint8_t* ov_locked /* [B][N] or null */,
                    const int32_t* ov_cnt /* [B][N] or null */) {
  // after a sampled step only a fully overridden transition is defined (the
  // rule would read statistics that exist for the sampled rows only)
  if (!s->stepped || (s->partial && !(n_ov_commit >= 0 && ov_locked != nullptr))) return -4;
  const orc_run& r = s->r;
  s->commit_seq.clear();
  s->commit_pos.clear();
  s->commit_tok.clear();
  const bool ov_commit = n_ov_commit >= 0, ov_lock = ov_locked != nullptr;
  lock_transition(s->m, r, s->t, s->M, s->row_seq.data(), s->row_pos.data(), s->row_real.data(),
                  s->row_argmax.data(), s->row_conf.data(), s->row_kl.data(),
                  s->row_has_kl.data(), s->x.data(), s->locked.data(), s->cnt.data(),
                  &s->commit_seq, &s->commit_pos, &s->commit_tok, !ov_commit, !ov_lock,
                  s->sf.data(), s->frozen.data(), s->has_prev.data(), s->refresh.data(),
                  s->drift.data());
  if (ov_commit) {
    s->commit_seq.assign(ov_commit_seq, ov_commit_seq + n_ov_commit);
    s->commit_pos.assign(ov_commit_pos, ov_commit_pos + n_ov_commit);
    s->commit_tok.assign(ov_commit_tok, ov_commit_tok + n_ov_commit);
    for (int j = 0; j < n_ov_commit; ++j)
      s->x[(size_t)ov_commit_seq[j] * r.seq_len + ov_commit_pos[j]] = ov_commit_tok[j];
  }
  const size_t BN = (size_t)r.batch * r.seq_len;
  if (ov_lock) {
    // the override also decides the refreshed positions: locked iff given
    for (size_t p = 0; p < BN; ++p)
      s->locked[p] = (s->refresh[p] ? 0 : s->locked[p]) | (ov_locked[p] ? 1 : 0);
    if (ov_cnt) std::memcpy(s->cnt.data(), ov_cnt, sizeof(int32_t) * BN);
  }
  s->t += 1;
  s->stepped = false;
  return 0;
}

// --- accessors --------------------------------------------------------------
int orc_t(const orc_state* s) { return s->t; }
int orc_m(const orc_state* s) { return s->M; }
double orc_flops(const orc_state* s) { return s->flops; }
void orc_get_tokens(const orc_state* s, int32_t* out) { std::copy(s->x.begin(), s->x.end(), out); }
void orc_get_locked(const orc_state* s, uint8_t* out) { std::copy(s->locked.begin(), s->locked.end(), out); }
void orc_get_cnt(const orc_state* s, int32_t* out) { std::copy(s->cnt.begin(), s->cnt.end(), out); }
void orc_get_has_prev(const orc_state* s, uint8_t* out) {
  std::copy(s->has_prev.begin(), s->has_prev.end(), out);
}
void orc_get_drift(const orc_state* s, float* out) {
  std::copy(s->drift.begin(), s->drift.end(), out);
}
void orc_get_refresh(const orc_state* s, uint8_t* out) {
  std::copy(s->refresh.begin(), s->refresh.end(), out);
}
void orc_get_frozen(const orc_state* s, uint8_t* out) {
  std::copy(s->frozen.begin(), s->frozen.end(), out);
}
// SlowFast state per sequence: phase, lo, hi, slow_n, hist_n, hist[8]
void orc_get_sf(const orc_state* s, int32_t* out /* [B][13] */) {
  for (size_t b = 0; b < s->sf.size(); ++b) {
    const SfSeq& q = s->sf[b];
    int32_t* o = out + b * 13;
    o[0] = q.phase; o[1] = q.lo; o[2] = q.hi; o[3] = q.slow_n; o[4] = q.hist_n;
    for (int j = 0; j < 8; ++j) o[5 + j] = q.hist[j];
  }
}
void orc_get_rows(const orc_state* s, int32_t* seq, int32_t* pos, uint8_t* real) {
  std::copy(s->row_seq.begin(), s->row_seq.end(), seq);
  std::copy(s->row_pos.begin(), s->row_pos.end(), pos);
  std::copy(s->row_real.begin(), s->row_real.end(), real);
}
void orc_get_stats(const orc_state* s, int32_t* argmax, double* conf, double* kl, double* lse,
                   uint8_t* has_kl) {
  std::copy(s->row_argmax.begin(), s->row_argmax.end(), argmax);
  std::copy(s->row_conf.begin(), s->row_conf.end(), conf);
  std::copy(s->row_kl.begin(), s->row_kl.end(), kl);
  std::copy(s->row_lse.begin(), s->row_lse.end(), lse);
  std::copy(s->row_has_kl.begin(), s->row_has_kl.end(), has_kl);
}
int orc_n_logit_rows(const orc_state* s) { return (int)s->logit_rows.size(); }
void orc_get_logits(const orc_state* s, int32_t* rows, double* z) {
  std::copy(s->logit_rows.begin(), s->logit_rows.end(), rows);
  std::copy(s->logits.begin(), s->logits.end(), z);
}
int orc_n_commits(const orc_state* s) { return (int)s->commit_pos.size(); }
void orc_get_commits(const orc_state* s, int32_t* seq, int32_t* pos, int32_t* tok) {
  std::copy(s->commit_seq.begin(), s->commit_seq.end(), seq);
  std::copy(s->commit_pos.begin(), s->commit_pos.end(), pos);
  std::copy(s->commit_tok.begin(), s->commit_tok.end(), tok);
}
// K/V cache of one layer, [B][nkv][N][hd]
void orc_get_kv(const orc_state* s, int layer, double* k, double* v) {
  const size_t n = (size_t)s->r.batch * s->m.n_kv_heads * s->r.seq_len * s->m.head_dim;
  const size_t off = (size_t)layer * n;
  std::copy(s->kc.begin() + off, s->kc.begin() + off + n, k);
  std::copy(s->vc.begin() + off, s->vc.begin() + off + n, v);
}

// --- the individual steps, for pins and kernel-level parity ------------------
void orc_unit_rmsnorm(const double* x, const float* g, int M, int d, double eps, double* y) {
  for (int i = 0; i < M; ++i) rmsnorm(x + (size_t)i * d, g, d, eps, y + (size_t)i * d);
}
// u: [M][nh][hd] rotated in place at positions pos[M]
void orc_unit_rope(double* u, const int32_t* pos, int M, int nh, int hd, double base) {
  for (int i = 0; i < M; ++i)
    for (int h = 0; h < nh; ++h) rope(u + ((size_t)i * nh + h) * hd, hd, pos[i], base);
}
void orc_unit_linear(const double* x, const float* W, int M, int N, int K, double* y) {
  linear(x, W, M, N, K, y);
}
// q [M][nq][hd], row_seq [M], kc/vc [B][nkv][N][hd] -> o [M][nq][hd]
void orc_unit_attention(const double* q, const int32_t* row_seq, const double* kc,
                        const double* vc, int M, int B, int N, int nq, int nkv, int hd,
                        double* o) {
  (void)B;
#pragma omp parallel
  {
    std::vector<double> sc(std::max(N, 1));
#pragma omp for collapse(2) schedule(static)
    for (int i = 0; i < M; ++i)
      for (int h = 0; h < nq; ++h) {
        const int g = h * nkv / nq;
        const size_t base = (((size_t)row_seq[i] * nkv + g) * N) * hd;
        attend(q + ((size_t)i * nq + h) * hd, kc + base, vc + base, N, hd,
               o + ((size_t)i * nq + h) * hd, sc.data());
      }
  }
}
// z [M][V]; prev [M][V] log-probabilities (row used iff has_prev[i])
void orc_unit_vocab_stats(const double* z, const double* prev, const uint8_t* has_prev, int M,
                          int V, int mask_id, int kl_dir, double* lse, int32_t* argmax,
                          double* conf, double* kl, double* logp) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < M; ++i) {
    const double* pv = (prev && has_prev && has_prev[i]) ? prev + (size_t)i * V : nullptr;
    vocab_stats(z + (size_t)i * V, pv, V, mask_id, kl_dir, &lse[i], &argmax[i], &conf[i], &kl[i],
                logp + (size_t)i * V);
  }
}
void orc_unit_schedule(const orc_run* r, int t, int32_t* out4 /* beta, lo, hi, k */) {
  const Sched s = schedule(*r, t);
  out4[0] = s.beta;
  out4[1] = s.lo;
  out4[2] = s.hi;
  out4[3] = s.k;
}
// The commit + lock transition on given statistics; x, locked, cnt updated in place.
int orc_unit_lock_transition(const orc_model* m, const orc_run* r, int t, int M,
                             const int32_t* row_seq, const int32_t* row_pos,
                             const uint8_t* row_real, const int32_t* argmax, const double* conf,
                             const double* kl, const uint8_t* has_kl, int32_t* x,
                             uint8_t* locked, int32_t* cnt, const uint8_t* refresh,
                             float* drift) {
  lock_transition(*m, *r, t, M, row_seq, row_pos, row_real, argmax, conf, kl, has_kl, x, locked,
                  cnt, nullptr, nullptr, nullptr, true, true, nullptr, nullptr, nullptr, refresh,
                  drift);
  return 0;
}
// Refresh set from the lock state and drift ([B][N] each); refresh rewritten.
void orc_unit_refresh_select(const orc_run* r, const uint8_t* locked, const float* drift,
                             uint8_t* refresh) {
  refresh_select(*r, locked, drift, refresh);
}
// One SlowFast commit decision for one sequence on given rows; state
// [13] = phase, lo, hi, slow_n, hist_n, hist[8] in and out; commits (at most
// n) written to commit_pos / commit_tok, their count returned.
int orc_unit_slowfast(const orc_run* r, int mask_id, int N, int n, const int32_t* pos,
                      const int32_t* argmax, const double* conf, int32_t* x, uint8_t* frozen,
                      uint8_t* has_prev, int32_t* state, int32_t* commit_pos,
                      int32_t* commit_tok) {
  SfSeq st;
  st.phase = state[0]; st.lo = state[1]; st.hi = state[2]; st.slow_n = state[3];
  st.hist_n = state[4];
  for (int j = 0; j < 8; ++j) st.hist[j] = state[5 + j];
  std::vector<int32_t> cp, ct;
  slowfast_commit(*r, mask_id, N, n, pos, argmax, conf, x, frozen, has_prev, st, &cp, &ct);
  state[0] = st.phase; state[1] = st.lo; state[2] = st.hi; state[3] = st.slow_n;
  state[4] = st.hist_n;
  for (int j = 0; j < 8; ++j) state[5 + j] = st.hist[j];
  std::copy(cp.begin(), cp.end(), commit_pos);
  std::copy(ct.begin(), ct.end(), commit_tok);
  return (int)cp.size();
}
// Active set from a bitmask: rows (b, pos) with bit clear, ascending.
int orc_unit_compact(const uint64_t* bits, int B, int N, int32_t* row_seq, int32_t* row_pos,
                     int32_t* m_b) {
  const int W = (N + 63) / 64;
  int M = 0;
  for (int b = 0; b < B; ++b) {
    m_b[b] = 0;
    for (int i = 0; i < N; ++i) {
      const bool lk = (bits[(size_t)b * W + i / 64] >> (i % 64)) & 1u;
      if (!lk) {
        row_seq[M] = b;
        row_pos[M] = i;
        ++M;
        ++m_b[b];
      }
    }
  }
  return M;
}
int orc_num_threads() {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

}  // extern "C"

// C ABI of the denoising-step engine (declared in include/dlm.h and
// include/dlm_ops.h): descriptor validation, carving of the caller's state
// block, the launch sequence of one step, the lock update, accessors and
// per-kernel timing.
//
// The step follows the SureLock page ("Stopping Computation for Converged
// Tokens in Masked Diffusion-LM Decoding"), §2 Methodology: compute only the
// active (unlocked) positions, keep every position's K/V in a per-layer cache
// that active queries attend to, lock a position once KL(p_t || p_{t-1}) <=
// eps (optionally gated by confidence), never unlock.  Unmasking uses the
// confidence-ranked top-k inside semi-autoregressive blocks named on the
// SlowFast page ("Accelerating Diffusion LLMs with SlowFast Sampling"), §1.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "dlm.h"
#include "dlm_ops.h"
#include "internal.h"

using namespace dlm;

namespace {

constexpr size_t kAlign = 256;
inline size_t al(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// Offsets of every array inside state_mem.
struct Layout {
  size_t tokens, bits, counters, has_prev, row_seq, row_pos, m_b, row_start, ctl, row_real;
  size_t frozen, sf_state, drift, last_step, refresh, rlist;
  size_t argmax, conf, kl, has_kl, lse_row, lse[2], z[2], kc, vc, rope, h, a, qkv, q, o, u;
  size_t ws, ws_bytes, ov_cseq, ov_cpos, ov_ctok, ov_bits, ov_cnt, total;
};

bool valid_model(const dlm_model_desc* m) {
  if (!m) return false;
  if (m->n_layers < 1 || m->d_model < 1 || m->n_heads < 1 || m->n_kv_heads < 1 ||
      m->head_dim < 2 || m->head_dim > 256 || (m->head_dim & 1) || m->d_ff < 1 ||
      m->vocab < 2 || m->mask_id < 0 || m->mask_id >= m->vocab)
    return false;
  if (m->n_heads % m->n_kv_heads) return false;
  if (m->dtype != DLM_FP32 && m->dtype != DLM_BF16) return false;
  if (!(m->rms_eps >= 0.f) || !std::isfinite(m->rms_eps)) return false;
  return true;
}

int n_blocks(const dlm_run_desc* r) {
  const int G = r->seq_len - r->prompt_len;
  return G > 0 ? (G + r->block_len - 1) / r->block_len : 0;
}

bool valid_run(const dlm_run_desc* r) {
  if (!r) return false;
  if (r->batch < 1 || r->batch > 1024 || r->seq_len < 1 || r->seq_len > 65536 ||
      r->prompt_len < 0 || r->prompt_len > r->seq_len || r->steps < 1 || r->block_len < 1 ||
      r->block_len > 4096 || r->n_consec < 1 || (r->kl_dir != 0 && r->kl_dir != 1) ||
      (r->lock_policy != DLM_LOCK_NONE && r->lock_policy != DLM_LOCK_TEST))
    return false;
  if ((int64_t)r->batch * r->seq_len > (1 << 24)) return false;
  if (n_blocks(r) > r->steps) return false;
  if (std::isnan(r->kl_eps) || std::isnan(r->conf_tau)) return false;
  if (r->sampler != DLM_SAMPLER_SEMI_AR && r->sampler != DLM_SAMPLER_SLOWFAST) return false;
  if (r->sampler == DLM_SAMPLER_SLOWFAST &&
      (r->seq_len > 4096 || r->sf_k < 1 || r->sf_kmax < 1 || r->sf_whist < 1 || r->sf_whist > 8 ||
       std::isnan(r->sf_tau_conv) || std::isnan(r->sf_tau_high) || std::isnan(r->sf_var)))
    return false;
  // drift-aware refresh: semi-AR sampler, one sequence's keys in 32 KB of LDS
  if (r->refresh_budget < 0 || r->refresh_budget > r->seq_len || std::isnan(r->refresh_eps))
    return false;
  if (r->refresh_budget > 0 && (r->sampler != DLM_SAMPLER_SEMI_AR || r->seq_len > 4096))
    return false;
  return true;
}

size_t max_ws(const dlm_model_desc& m, const dlm_run_desc& r) {
  const int BN = r.batch * r.seq_len;
  const int qo = m.n_heads * m.head_dim, qkv = (m.n_heads + 2 * m.n_kv_heads) * m.head_dim;
  size_t w = 0;
  for (int M = 1; M <= BN; ++M) {
    w = std::max(w, gemm_ws_bytes(m.dtype, kEpiStoreF32, M, qkv, m.d_model));
    w = std::max(w, gemm_ws_bytes(m.dtype, kEpiResidAdd, M, m.d_model, qo));
    w = std::max(w, gemm_ws_bytes(m.dtype, kEpiSwiglu, M, m.d_ff, m.d_model));
    w = std::max(w, gemm_ws_bytes(m.dtype, kEpiResidAdd, M, m.d_model, m.d_ff));
    w = std::max(w, gemm_ws_bytes(m.dtype, kEpiLogits, M, m.vocab, m.d_model));
    w = std::max(w, attention_ws_bytes(m.dtype, M, r.batch, r.seq_len, m.n_heads,
                                       m.n_kv_heads, m.head_dim));
    w = std::max(w, vocab_ws_bytes(M, m.vocab));
    w = std::max(w, gemm_logits_stats_bytes(m.dtype, M, m.vocab, m.d_model));
  }
  return w;
}

Layout make_layout(const dlm_model_desc& m, const dlm_run_desc& r) {
  Layout L{};
  const size_t B = r.batch, N = r.seq_len, BN = B * N, W = (N + 63) / 64;
  const size_t es = m.dtype == DLM_BF16 ? 2 : 4;
  const size_t d = m.d_model, qo = (size_t)m.n_heads * m.head_dim;
  const size_t qkv = (size_t)(m.n_heads + 2 * m.n_kv_heads) * m.head_dim;
  const size_t kvn = (size_t)m.n_layers * B * m.n_kv_heads * N * m.head_dim;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += al(bytes);
    return at;
  };
  L.tokens = take(BN * 4);
  L.bits = take(B * W * 8);
  L.frozen = take(B * W * 8);
  L.sf_state = take(B * kSfStateInts * 4);
  L.drift = take(BN * 4);
  L.last_step = take(BN * 4);
  L.refresh = take(B * W * 8);
  L.rlist = take(B * std::max<size_t>(1, (size_t)r.refresh_budget) * 4);
  L.counters = take(BN * 4);
  L.has_prev = take(BN * 4);
  L.row_seq = take(BN * 4);
  L.row_pos = take(BN * 4);
  L.m_b = take(B * 4);
  L.row_start = take((B + 1) * 4);
  L.ctl = take(16);
  L.row_real = take(BN * 4);
  L.argmax = take(BN * 4);
  L.conf = take(BN * 4);
  L.kl = take(BN * 4);
  L.has_kl = take(BN * 4);
  L.lse_row = take(BN * 4);
  L.lse[0] = take(BN * 4);
  L.lse[1] = take(BN * 4);
  L.z[0] = take(BN * m.vocab * 4);
  L.z[1] = take(BN * m.vocab * 4);
  L.kc = take(kvn * es);
  L.vc = take(kvn * es);
  L.rope = take(N * (m.head_dim / 2) * 2 * 4);
  L.h = take(BN * d * 4);
  L.a = take(BN * d * es);
  L.qkv = take(BN * qkv * 4);
  L.q = take(BN * qo * es);
  L.o = take(BN * qo * es);
  L.u = take(BN * (size_t)m.d_ff * es);
  L.ws_bytes = std::max<size_t>(max_ws(m, r), 256);
  L.ws = take(L.ws_bytes);
  L.ov_cseq = take(BN * 4);
  L.ov_cpos = take(BN * 4);
  L.ov_ctok = take(BN * 4);
  L.ov_bits = take(B * W * 8);
  L.ov_cnt = take(BN * 4);
  L.total = o;
  return L;
}

struct Sched { int beta, lo, hi, k; };

// Block schedule: G generated positions in blocks of block_len; the steps
// split over blocks as T_b = floor(T(b+1)/n) - floor(Tb/n); the s-th step of
// block b unmasks floor(G_b(s+1)/T_b) - floor(G_b s/T_b) positions.
Sched schedule(const dlm_run_desc& r, int t) {
  Sched s{-1, 0, 0, 0};
  const int nb = n_blocks(&r);
  for (int b = 0; b < nb; ++b) {
    const long t0 = (long)r.steps * b / nb, t1 = (long)r.steps * (b + 1) / nb;
    if (t >= t0 && t < t1) {
      const long Tb = t1 - t0, si = t - t0;
      s.beta = b;
      s.lo = r.prompt_len + b * r.block_len;
      s.hi = std::min(r.seq_len, s.lo + r.block_len);
      const long Gb = s.hi - s.lo;
      s.k = (int)(Gb * (si + 1) / Tb - Gb * si / Tb);
      break;
    }
  }
  return s;
}

struct Timed {
  int cls;
  hipEvent_t e0, e1;
  double bytes, flops;
};

}  // namespace

struct dlm_handle {
  dlm_model_desc m;
  dlm_run_desc r;
  Layout lay;
  unsigned char* base;
  hipStream_t stream;
  const void *emb, *fnorm, *lm;
  std::vector<const void*> attn_norm, w_qkv, w_o, ffn_norm, w_gate, w_up, w_down;
  int t = 0, last_t = -1, M = 0;
  bool stepped = false;
  double flops = 0.0;
  // timing
  bool timing = false;
  std::vector<hipEvent_t> pool;
  std::vector<Timed> pending;
  double t_ms[DLM_K_NUM_CLASSES] = {}, t_bytes[DLM_K_NUM_CLASSES] = {},
         t_flops[DLM_K_NUM_CLASSES] = {};
  int64_t t_n[DLM_K_NUM_CLASSES] = {};

  template <typename T> T* at(size_t off) const { return reinterpret_cast<T*>(base + off); }
};

namespace {

int hip_status(hipError_t e) { return e == hipSuccess ? DLM_OK : DLM_E_HIP; }

hipError_t harvest(dlm_handle* h) {
  hipError_t e = hipStreamSynchronize(h->stream);
  if (e != hipSuccess) return e;
  for (const Timed& x : h->pending) {
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, x.e0, x.e1);
    if (e != hipSuccess) return e;
    h->t_ms[x.cls] += ms;
    h->t_bytes[x.cls] += x.bytes;
    h->t_flops[x.cls] += x.flops;
    h->t_n[x.cls] += 1;
    h->pool.push_back(x.e0);
    h->pool.push_back(x.e1);
  }
  h->pending.clear();
  return hipSuccess;
}

template <typename F>
hipError_t timed(dlm_handle* h, int cls, double bytes, double flops, F&& launch) {
  if (!h->timing) return launch();
  if (h->pool.size() < 2) {
    hipError_t e = harvest(h);
    if (e != hipSuccess) return e;
    while (h->pool.size() < 64) {
      hipEvent_t ev;
      e = hipEventCreate(&ev);
      if (e != hipSuccess) return e;
      h->pool.push_back(ev);
    }
  }
  hipEvent_t e1 = h->pool.back();
  h->pool.pop_back();
  hipEvent_t e0 = h->pool.back();
  h->pool.pop_back();
  hipError_t e = hipEventRecord(e0, h->stream);
  if (e == hipSuccess) e = launch();
  if (e == hipSuccess) e = hipEventRecord(e1, h->stream);
  if (e != hipSuccess) return e;
  h->pending.push_back(Timed{cls, e0, e1, bytes, flops});
  return hipSuccess;
}

#define TRY(x)                              \
  do {                                      \
    hipError_t _e = (x);                    \
    if (_e != hipSuccess) return DLM_E_HIP; \
  } while (0)

}  // namespace

// Workspace of dlm_op_gemm_noalloc: split-K partial sums in a file-scope
// device array, so that the call needs no allocation (one copy per GPU the
// library runs on, held until the process ends).  Host code never uses the
// array's name as an address: the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
namespace {
constexpr size_t kGemmScratchBytes = size_t(8) << 20;
}  // namespace
static __device__ __align__(256) unsigned char scratch[kGemmScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch array on the device that owns `stream` (the
// current device for the null stream).
int gemm_scratch_for(hipStream_t stream, void** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return DLM_E_HIP;
  int dev = cur;
  if (stream) {
    hipDevice_t sd = 0;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return DLM_E_HIP;
    dev = (int)sd;
  }
  if (dev < 0 || dev >= kMaxDevices) return DLM_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return DLM_E_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return DLM_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DLM_OK;
}
}  // namespace

extern "C" {

const char* dlm_error_string(int status) {
  switch (status) {
    case DLM_OK: return "ok";
    case DLM_E_INVALID: return "invalid argument";
    case DLM_E_SIZE: return "state buffer too small";
    case DLM_E_HIP: return "HIP runtime error";
    case DLM_E_STATE: return "call out of order";
    case DLM_E_UNSUPPORTED: return "unsupported shape";
    case DLM_E_NUMERIC: return "non-finite posterior detected on the device";
    default: return "unknown status";
  }
}

size_t dlm_state_bytes(const dlm_model_desc* model, const dlm_run_desc* run) {
  if (!valid_model(model) || !valid_run(run)) return 0;
  return make_layout(*model, *run).total;
}

int dlm_step_init(const dlm_model_desc* model, const dlm_weights* w, const dlm_run_desc* run,
                  const int32_t* prompt_tokens, void* state_mem, size_t state_bytes,
                  void* hip_stream, dlm_handle** out) {
  if (!out) return DLM_E_INVALID;
  *out = nullptr;
  if (!valid_model(model) || !valid_run(run) || !w || !state_mem) return DLM_E_INVALID;
  if (run->prompt_len > 0 && !prompt_tokens) return DLM_E_INVALID;
  if ((uintptr_t)state_mem % kAlign) return DLM_E_INVALID;
  const int L = model->n_layers;
  if (!w->tok_emb || !w->final_norm || !w->lm_head || !w->attn_norm || !w->w_qkv || !w->w_o ||
      !w->ffn_norm || !w->w_gate || !w->w_up || !w->w_down)
    return DLM_E_INVALID;
  auto aligned = [](const void* p) { return p && ((uintptr_t)p % 16) == 0; };
  if (!aligned(w->tok_emb) || !aligned(w->final_norm) || !aligned(w->lm_head))
    return DLM_E_INVALID;
  for (int l = 0; l < L; ++l)
    if (!aligned(w->attn_norm[l]) || !aligned(w->w_qkv[l]) || !aligned(w->w_o[l]) ||
        !aligned(w->ffn_norm[l]) || !aligned(w->w_gate[l]) || !aligned(w->w_up[l]) ||
        !aligned(w->w_down[l]))
      return DLM_E_INVALID;
  const Layout lay = make_layout(*model, *run);
  if (state_bytes < lay.total) return DLM_E_SIZE;

  dlm_handle* h = new (std::nothrow) dlm_handle();
  if (!h) return DLM_E_INVALID;
  h->m = *model;
  h->r = *run;
  h->lay = lay;
  h->base = (unsigned char*)state_mem;
  h->stream = (hipStream_t)hip_stream;
  h->emb = w->tok_emb;
  h->fnorm = w->final_norm;
  h->lm = w->lm_head;
  h->attn_norm.assign(w->attn_norm, w->attn_norm + L);
  h->w_qkv.assign(w->w_qkv, w->w_qkv + L);
  h->w_o.assign(w->w_o, w->w_o + L);
  h->ffn_norm.assign(w->ffn_norm, w->ffn_norm + L);
  h->w_gate.assign(w->w_gate, w->w_gate + L);
  h->w_up.assign(w->w_up, w->w_up + L);
  h->w_down.assign(w->w_down, w->w_down + L);

  const int B = run->batch, N = run->seq_len;
  hipError_t e = launch_init_state(B, N, run->prompt_len, model->mask_id, prompt_tokens,
                                   h->at<int32_t>(lay.tokens), h->at<uint64_t>(lay.bits),
                                   h->at<int32_t>(lay.counters), h->at<int32_t>(lay.has_prev),
                                   h->at<int32_t>(lay.ctl), h->at<uint64_t>(lay.frozen),
                                   h->at<int32_t>(lay.sf_state), h->stream);
  // drift +inf (undefined), last computed at no step (-1), nothing refreshed
  if (e == hipSuccess)
    e = launch_fill_u32(h->base + lay.drift, (size_t)B * N * 4, 0x7f800000u, h->stream);
  if (e == hipSuccess)
    e = launch_fill_u32(h->base + lay.last_step, (size_t)B * N * 4, 0xffffffffu, h->stream);
  if (e == hipSuccess)
    e = launch_fill_u32(h->base + lay.refresh, (size_t)B * ((N + 63) / 64) * 8, 0u, h->stream);
  if (e == hipSuccess && model->rope_base > 0.f)
    e = launch_rope_table(N, model->head_dim, model->rope_base, h->at<float>(lay.rope), h->stream);
  if (e != hipSuccess) {
    delete h;
    return DLM_E_HIP;
  }
  *out = h;
  return DLM_OK;
}

int dlm_step(dlm_handle* h, int32_t* m_tot_out) {
  if (!h) return DLM_E_INVALID;
  if (h->stepped || h->t >= h->r.steps) return DLM_E_STATE;
  const dlm_model_desc& m = h->m;
  const dlm_run_desc& r = h->r;
  const Layout& y = h->lay;
  hipStream_t s = h->stream;
  const int B = r.batch, N = r.seq_len, d = m.d_model, nq = m.n_heads, nkv = m.n_kv_heads,
            hd = m.head_dim, dff = m.d_ff, V = m.vocab, dt = m.dtype;
  const int qo = nq * hd, qkv_out = (nq + 2 * nkv) * hd;
  const double es = dt == DLM_BF16 ? 2.0 : 4.0;

  int32_t* row_seq = h->at<int32_t>(y.row_seq);
  int32_t* row_pos = h->at<int32_t>(y.row_pos);
  int32_t* row_start = h->at<int32_t>(y.row_start);
  int32_t* ctl = h->at<int32_t>(y.ctl);
  const bool refresh = r.refresh_budget > 0;
  if (refresh) {
    // drift-aware refresh (Polestar page, "The Smart Painter", Polestar-Cache):
    // choose the locked positions to recompute, and put each one's last
    // posterior where this step reads the previous one
    TRY(timed(h, DLM_K_COMPACT, 0.0, 0.0, [&] {
      return launch_refresh_select(B, N, r.refresh_budget, h->at<uint64_t>(y.bits),
                                   h->at<float>(y.drift), h->at<uint64_t>(y.refresh),
                                   h->at<int32_t>(y.rlist), s);
    }));
    TRY(timed(h, DLM_K_COMPACT, 0.0, 0.0, [&] {
      return launch_refresh_copy(B, N, V, r.refresh_budget, h->t, h->at<int32_t>(y.rlist),
                                 h->at<int32_t>(y.last_step), h->at<float>(y.z[0]),
                                 h->at<float>(y.z[1]), h->at<float>(y.lse[0]),
                                 h->at<float>(y.lse[1]), s);
    }));
  }
  TRY(timed(h, DLM_K_COMPACT, B * ((N + 63) / 64) * 8.0, 0.0, [&] {
    return launch_compact(h->at<uint64_t>(y.bits),
                          r.sampler == DLM_SAMPLER_SLOWFAST ? h->at<uint64_t>(y.frozen) : nullptr,
                          B, N, row_seq, row_pos, h->at<int32_t>(y.m_b), row_start, ctl, s,
                          refresh ? h->at<uint64_t>(y.refresh) : nullptr,
                          refresh ? h->at<int32_t>(y.last_step) : nullptr, h->t);
  }));
  int32_t hctl[2] = {0, 0};
  TRY(hipMemcpyAsync(hctl, ctl, sizeof(hctl), hipMemcpyDeviceToHost, s));
  TRY(hipStreamSynchronize(s));
  if (hctl[1] != 0) return DLM_E_NUMERIC;
  const int M = hctl[0];
  h->M = M;
  h->flops = 0.0;
  h->last_t = h->t;
  h->stepped = true;
  if (m_tot_out) *m_tot_out = M;
  if (M == 0) return DLM_OK;

  const int cur = h->t & 1, prv = cur ^ 1;
  float* hres = h->at<float>(y.h);
  void* a = h->base + y.a;
  float* qkv = h->at<float>(y.qkv);
  void* q = h->base + y.q;
  void* o = h->base + y.o;
  void* u = h->base + y.u;
  void* ws = h->base + y.ws;
  const size_t kv_layer = (size_t)B * nkv * N * hd * (size_t)es;

  TRY(timed(h, DLM_K_EMBED_NORM, M * (double)d * (4 + es), 0.0, [&] {
    return launch_embed_rmsnorm(dt, M, d, N, m.rms_eps, m.mask_id, h->at<int32_t>(y.tokens),
                                row_seq, row_pos, h->emb, h->attn_norm[0], hres, a,
                                h->at<int32_t>(y.row_real), s);
  }));
  // GEMM launch with its algorithmic work; `deferred` (float-store and
  // residual epilogues) leaves split-K partials in ws for the next kernel
  // and returns the split count through *splits.
  auto gemm = [&](int cls, int epi, int Nn, int K, const void* A, const void* W, const void* W2,
                  void* C, int* splits) {
    GemmArgs g{dt, epi, M, Nn, K, A, W, W2, C, row_seq, row_pos, N, m.mask_id,
               nullptr, nullptr, nullptr, nullptr, 0, 0};
    const double mats = epi == kEpiSwiglu ? 2.0 : 1.0;
    const double fl = 2.0 * M * (double)Nn * K * mats;
    const double out_b = epi == kEpiSwiglu ? es : (epi == kEpiResidAdd ? 8.0 : 4.0);
    const double by = mats * Nn * (double)K * es + M * (double)K * es + M * (double)Nn * out_b;
    h->flops += fl;
    return timed(h, cls, by, fl, [&] {
      if (splits) return launch_gemm_deferred(g, ws, y.ws_bytes, s, splits);
      return launch_gemm(g, ws, y.ws_bytes, s);
    });
  };
  const float* part = (const float*)ws;
  int sp_res = 0;  // split-K partials of the last residual update, pending
  for (int l = 0; l < m.n_layers; ++l) {
    // residual norm: read h and the pending split-K partials, write h and y
    if (l > 0)
      TRY(timed(h, DLM_K_RMSNORM, M * (double)d * (4.0 * (2 + sp_res) + es), 0.0, [&] {
        return launch_rmsnorm_resid(dt, M, d, m.rms_eps, hres, part, sp_res, h->attn_norm[l], a,
                                    s);
      }));
    unsigned char* kcl = h->base + y.kc + l * kv_layer;
    unsigned char* vcl = h->base + y.vc + l * kv_layer;
    const float* rope = m.rope_base > 0.f ? h->at<float>(y.rope) : nullptr;
    if (gemm_qkv_fusable(dt, M, hd, d)) {
      // QKV projection with rotary embedding and cache scatter in its epilogue
      GemmArgs g{dt, kEpiQKV, M, qkv_out, d, a, h->w_qkv[l], nullptr, nullptr, row_seq, row_pos,
                 N, m.mask_id, rope, q, kcl, vcl, nq, nkv};
      const double fl = 2.0 * M * (double)qkv_out * d;
      const double by = qkv_out * (double)d * es + M * (double)d * es + M * (double)qkv_out * es;
      h->flops += fl;
      TRY(timed(h, DLM_K_GEMM_QKV, by, fl, [&] { return launch_gemm(g, ws, y.ws_bytes, s); }));
    } else {
      int sp_qkv = 0;
      TRY(gemm(DLM_K_GEMM_QKV, kEpiStoreF32, qkv_out, d, a, h->w_qkv[l], nullptr, qkv, &sp_qkv));
      TRY(timed(h, DLM_K_ROPE_KV, M * (double)qkv_out * (4 + es), 0.0, [&] {
        return launch_rope_scatter_split(dt, M, nq, nkv, hd, N, qkv, part, sp_qkv, row_seq,
                                         row_pos, rope, q, kcl, vcl, s);
      }));
    }
    {
      const double fl = 4.0 * M * (double)N * qo;
      const double by = 2.0 * kv_layer + 2.0 * M * (double)qo * es;
      h->flops += fl;
      TRY(timed(h, DLM_K_ATTENTION, by, fl, [&] {
        return launch_attention(dt, M, B, N, nq, nkv, hd, q, row_start, kcl, vcl, o, ws,
                                y.ws_bytes, s);
      }));
    }
    TRY(gemm(DLM_K_GEMM_O, kEpiResidAdd, d, qo, o, h->w_o[l], nullptr, hres, &sp_res));
    TRY(timed(h, DLM_K_RMSNORM, M * (double)d * (4.0 * (2 + sp_res) + es), 0.0, [&] {
      return launch_rmsnorm_resid(dt, M, d, m.rms_eps, hres, part, sp_res, h->ffn_norm[l], a, s);
    }));
    TRY(gemm(DLM_K_GEMM_GATE_UP, kEpiSwiglu, dff, d, a, h->w_gate[l], h->w_up[l], u, nullptr));
    TRY(gemm(DLM_K_GEMM_DOWN, kEpiResidAdd, d, dff, u, h->w_down[l], nullptr, hres, &sp_res));
  }
  TRY(timed(h, DLM_K_RMSNORM, M * (double)d * (4.0 * (2 + sp_res) + es), 0.0, [&] {
    return launch_rmsnorm_resid(dt, M, d, m.rms_eps, hres, part, sp_res, h->fnorm, a, s);
  }));
  float* zc = h->at<float>(y.z[cur]);
  if (gemm_logits_stats_fusable(dt, d) && gemm_logits_stats_preferred(M, V)) {
    // LM head whose epilogue also folds the posterior statistics (with the
    // previous step's logits) into one partial per row and column tile; a
    // small pass merges them per row.
    GemmArgs g{dt, kEpiLogitsStats, M, V, d, a, h->lm, nullptr, zc, row_seq, row_pos, N,
               m.mask_id, nullptr, nullptr, nullptr, nullptr, 0, 0, h->at<float>(y.z[prv]),
               h->at<float>(y.lse[prv]), h->at<int32_t>(y.has_prev), ws, r.kl_dir};
    const double fl = 2.0 * M * (double)V * d;
    const double by = V * (double)d * es + M * (double)d * es + M * (double)V * 8.0;
    h->flops += fl;
    TRY(timed(h, DLM_K_GEMM_LM_HEAD, by, fl, [&] { return launch_gemm_logits_stats(g, -1, s); }));
    const int nparts = gemm_logits_stats_parts(M, V, d, -1);
    TRY(timed(h, DLM_K_VOCAB_STATS, M * (double)nparts * kVocabPartBytes, 0.0, [&] {
      return launch_vocab_merge_parts(M, nparts, N, r.kl_dir, row_seq, row_pos,
                                      h->at<float>(y.lse[prv]), h->at<int32_t>(y.has_prev),
                                      h->at<float>(y.lse[cur]), ws, h->at<int32_t>(y.argmax),
                                      h->at<float>(y.conf), h->at<float>(y.kl),
                                      h->at<int32_t>(y.has_kl), h->at<float>(y.lse_row), ctl + 1,
                                      s);
    }));
    return DLM_OK;
  }
  TRY(gemm(DLM_K_GEMM_LM_HEAD, kEpiLogits, V, d, a, h->lm, nullptr, zc, nullptr));
  TRY(timed(h, DLM_K_VOCAB_STATS, M * (double)V * 8.0, 0.0, [&] {
    return launch_vocab_stats(M, V, m.mask_id, r.kl_dir, N, row_seq, row_pos, zc,
                              h->at<float>(y.z[prv]), h->at<float>(y.lse[prv]),
                              h->at<int32_t>(y.has_prev), h->at<float>(y.lse[cur]),
                              h->at<int32_t>(y.argmax), h->at<float>(y.conf),
                              h->at<float>(y.kl), h->at<int32_t>(y.has_kl),
                              h->at<float>(y.lse_row), ctl + 1, ws, y.ws_bytes, s);
  }));
  return DLM_OK;
}

int dlm_lock_update(dlm_handle* h, const dlm_override* ov) {
  if (!h) return DLM_E_INVALID;
  if (!h->stepped) return DLM_E_STATE;
  const dlm_run_desc& r = h->r;
  const Layout& y = h->lay;
  const int B = r.batch, N = r.seq_len, W = (N + 63) / 64;
  const bool ov_commit = ov && ov->n_commit >= 0;
  const bool ov_lock = ov && ov->lock_bits;
  if (ov) {
    if (ov->n_commit > B * N) return DLM_E_INVALID;
    if (ov_commit && ov->n_commit > 0) {
      if (!ov->commit_seq || !ov->commit_pos || !ov->commit_tok) return DLM_E_INVALID;
      for (int i = 0; i < ov->n_commit; ++i)
        if (ov->commit_seq[i] < 0 || ov->commit_seq[i] >= B || ov->commit_pos[i] < 0 ||
            ov->commit_pos[i] >= N || ov->commit_tok[i] < 0 || ov->commit_tok[i] >= h->m.vocab)
          return DLM_E_INVALID;
    }
    if (!ov_lock && ov->counters) return DLM_E_INVALID;
  }
  const Sched sc = schedule(r, h->t);
  LockArgs la{};
  la.B = B;
  la.N = N;
  la.P = r.prompt_len;
  la.mask_id = h->m.mask_id;
  la.blk_lo = sc.lo;
  la.blk_hi = sc.hi;
  la.k = sc.beta >= 0 ? sc.k : 0;
  la.do_commit = !ov_commit;
  la.do_lock = !ov_lock;
  la.policy = r.lock_policy;
  la.kl_eps = r.kl_eps;
  la.conf_tau = r.conf_tau;
  la.n_consec = r.n_consec;
  la.lock_prompt = (h->t == 0 && r.lock_prompt_after_first_step) ? 1 : 0;
  la.row_seq = h->at<int32_t>(y.row_seq);
  la.row_pos = h->at<int32_t>(y.row_pos);
  la.row_start = h->at<int32_t>(y.row_start);
  la.row_real = h->at<int32_t>(y.row_real);
  la.argmax = h->at<int32_t>(y.argmax);
  la.conf = h->at<float>(y.conf);
  la.kl = h->at<float>(y.kl);
  la.has_kl = h->at<int32_t>(y.has_kl);
  la.tokens = h->at<int32_t>(y.tokens);
  la.bits = h->at<uint64_t>(y.bits);
  la.counters = h->at<int32_t>(y.counters);
  la.sampler = r.sampler;
  la.sf_window = r.block_len;
  la.sf_k = r.sf_k;
  la.sf_kmax = r.sf_kmax;
  la.sf_whist = r.sf_whist;
  la.sf_tau_conv = r.sf_tau_conv;
  la.sf_tau_high = r.sf_tau_high;
  la.sf_var = r.sf_var;
  la.frozen = h->at<uint64_t>(y.frozen);
  la.has_prev = h->at<int32_t>(y.has_prev);
  la.sf_state = h->at<int32_t>(y.sf_state);
  la.err = h->at<int32_t>(y.ctl) + 1;
  const bool refresh = r.refresh_budget > 0;
  la.refresh = refresh ? h->at<uint64_t>(y.refresh) : nullptr;
  la.refresh_eps = r.refresh_eps;
  la.drift = refresh ? h->at<float>(y.drift) : nullptr;
  if (la.do_commit || la.do_lock || la.drift)
    TRY(timed(h, DLM_K_COMMIT_LOCK, 0.0, 0.0, [&] { return launch_commit_lock(la, h->stream); }));
  if (ov && (ov_commit || ov_lock)) {
    const int nc = ov_commit ? ov->n_commit : 0;
    if (nc > 0) {
      TRY(hipMemcpyAsync(h->at<int32_t>(y.ov_cseq), ov->commit_seq, nc * 4,
                         hipMemcpyHostToDevice, h->stream));
      TRY(hipMemcpyAsync(h->at<int32_t>(y.ov_cpos), ov->commit_pos, nc * 4,
                         hipMemcpyHostToDevice, h->stream));
      TRY(hipMemcpyAsync(h->at<int32_t>(y.ov_ctok), ov->commit_tok, nc * 4,
                         hipMemcpyHostToDevice, h->stream));
    }
    if (ov_lock) {
      TRY(hipMemcpyAsync(h->at<uint64_t>(y.ov_bits), ov->lock_bits, (size_t)B * W * 8,
                         hipMemcpyHostToDevice, h->stream));
      if (ov->counters)
        TRY(hipMemcpyAsync(h->at<int32_t>(y.ov_cnt), ov->counters, (size_t)B * N * 4,
                           hipMemcpyHostToDevice, h->stream));
    }
    TRY(launch_apply_override(B, N, nc, h->at<int32_t>(y.ov_cseq), h->at<int32_t>(y.ov_cpos),
                              h->at<int32_t>(y.ov_ctok),
                              ov_lock ? h->at<uint64_t>(y.ov_bits) : nullptr,
                              (ov_lock && ov->counters) ? h->at<int32_t>(y.ov_cnt) : nullptr,
                              h->at<int32_t>(y.tokens), h->at<uint64_t>(y.bits),
                              h->at<int32_t>(y.counters), h->stream,
                              refresh ? h->at<uint64_t>(y.refresh) : nullptr));
    // the host arrays may be released as soon as this call returns
    TRY(hipStreamSynchronize(h->stream));
  }
  h->t += 1;
  h->stepped = false;
  return DLM_OK;
}

int dlm_get(dlm_handle* h, int32_t what, const void** dev_ptr, int64_t* n) {
  if (!h || !dev_ptr || !n) return DLM_E_INVALID;
  const Layout& y = h->lay;
  const int64_t B = h->r.batch, N = h->r.seq_len, BN = B * N, M = h->M;
  const int slot = (h->last_t >= 0 ? h->last_t : 0) & 1;
  const int64_t kvn =
      (int64_t)h->m.n_layers * B * h->m.n_kv_heads * N * h->m.head_dim;
  size_t off;
  int64_t cnt;
  switch (what) {
    case DLM_GET_TOKENS: off = y.tokens; cnt = BN; break;
    case DLM_GET_LOCK_BITS: off = y.bits; cnt = B * ((N + 63) / 64); break;
    case DLM_GET_COUNTERS: off = y.counters; cnt = BN; break;
    case DLM_GET_ROW_SEQ: off = y.row_seq; cnt = M; break;
    case DLM_GET_ROW_POS: off = y.row_pos; cnt = M; break;
    case DLM_GET_ARGMAX: off = y.argmax; cnt = M; break;
    case DLM_GET_CONF: off = y.conf; cnt = M; break;
    case DLM_GET_KL: off = y.kl; cnt = M; break;
    case DLM_GET_HAS_KL: off = y.has_kl; cnt = M; break;
    case DLM_GET_LSE: off = y.lse_row; cnt = M; break;
    case DLM_GET_LOGITS: off = y.z[slot]; cnt = BN * h->m.vocab; break;
    case DLM_GET_ROW_REAL: off = y.row_real; cnt = M; break;
    case DLM_GET_KCACHE: off = y.kc; cnt = kvn; break;
    case DLM_GET_VCACHE: off = y.vc; cnt = kvn; break;
    case DLM_GET_FROZEN: off = y.frozen; cnt = B * ((N + 63) / 64); break;
    case DLM_GET_SF_STATE: off = y.sf_state; cnt = B * kSfStateInts; break;
    case DLM_GET_HAS_PREV: off = y.has_prev; cnt = BN; break;
    case DLM_GET_DRIFT: off = y.drift; cnt = BN; break;
    case DLM_GET_REFRESH: off = y.refresh; cnt = B * ((N + 63) / 64); break;
    default: return DLM_E_INVALID;
  }
  *dev_ptr = h->base + off;
  *n = cnt;
  return DLM_OK;
}

int dlm_debug_poison(dlm_handle* h) {
  if (!h) return DLM_E_INVALID;
  if (h->t != 0 || h->stepped) return DLM_E_STATE;
  const Layout& y = h->lay;
  const dlm_model_desc& m = h->m;
  const size_t B = h->r.batch, N = h->r.seq_len, BN = B * N;
  const size_t es = m.dtype == DLM_BF16 ? 2 : 4;
  const size_t d = m.d_model, qo = (size_t)m.n_heads * m.head_dim;
  const size_t qkv = (size_t)(m.n_heads + 2 * m.n_kv_heads) * m.head_dim;
  const size_t kvn = (size_t)m.n_layers * B * m.n_kv_heads * N * m.head_dim;
  // 0x7FC07FC0 is a quiet NaN as one float and as each of two bfloat16s
  const uint32_t nan2 = 0x7FC07FC0u;
  const struct { size_t off, bytes; } regions[] = {
      {y.z[0], BN * m.vocab * 4}, {y.z[1], BN * m.vocab * 4}, {y.lse[0], BN * 4},
      {y.lse[1], BN * 4},         {y.kc, kvn * es},           {y.vc, kvn * es},
      {y.h, BN * d * 4},          {y.a, BN * d * es},         {y.qkv, BN * qkv * 4},
      {y.q, BN * qo * es},        {y.o, BN * qo * es},        {y.u, BN * m.d_ff * es},
      {y.ws, y.ws_bytes},         {y.argmax, BN * 4},         {y.conf, BN * 4},
      {y.kl, BN * 4},             {y.has_kl, BN * 4},         {y.lse_row, BN * 4},
      {y.row_real, BN * 4}};
  for (const auto& r : regions)
    TRY(launch_fill_u32(h->base + r.off, r.bytes, nan2, h->stream));
  return DLM_OK;
}

}  // extern "C"

namespace {
// Checkpoint image: a 256-byte header, then three byte ranges of the state
// copied as they lie: the per-position and per-row arrays (tokens through
// the two log-normaliser buffers, contiguous in the layout), the logits
// buffer the next step reads as the previous posterior (with the refresh on,
// then also the other one: a locked position's last posterior may lie in
// either), and the K and V caches (contiguous).
constexpr char kCkptMagic[8] = {'D', 'L', 'M', 'C', 'K', 'P', 'T', '1'};
constexpr uint32_t kCkptVersion = 1;
constexpr size_t kCkptHeaderBytes = 256;
static_assert(sizeof(dlm_model_desc) == 11 * 4, "model descriptor without padding");
static_assert(sizeof(dlm_run_desc) == 20 * 4, "run descriptor without padding");

struct CkptHeader {
  char magic[8];
  uint32_t version, header_bytes;
  dlm_model_desc m;
  dlm_run_desc r;
  int32_t t, last_t, M, reserved;
  double flops;
  uint64_t small_bytes, z_bytes, kv_bytes, total;
};
static_assert(sizeof(CkptHeader) <= kCkptHeaderBytes, "checkpoint header");

struct CkptParts {
  size_t small_off, small_bytes, z_bytes, kv_off, kv_bytes, total;
};

CkptParts ckpt_parts(const dlm_handle* h) {
  const Layout& y = h->lay;
  CkptParts c;
  c.small_off = y.tokens;
  c.small_bytes = y.z[0] - y.tokens;
  c.z_bytes = (size_t)h->r.batch * h->r.seq_len * h->m.vocab * 4 * (h->r.refresh_budget > 0 ? 2 : 1);
  c.kv_off = y.kc;
  c.kv_bytes = y.rope - y.kc;
  c.total = kCkptHeaderBytes + c.small_bytes + c.z_bytes + c.kv_bytes;
  return c;
}

// logits buffer that the handle's next step reads as the previous posterior
size_t ckpt_prev_z(const dlm_handle* h) { return h->lay.z[(h->t & 1) ^ 1]; }
// the other logits buffer
size_t ckpt_cur_z(const dlm_handle* h) { return h->lay.z[h->t & 1]; }
}  // namespace

extern "C" {

size_t dlm_checkpoint_bytes(const dlm_handle* h) { return h ? ckpt_parts(h).total : 0; }

int dlm_checkpoint_save(dlm_handle* h, void* dst, size_t dst_bytes) {
  if (!h || !dst) return DLM_E_INVALID;
  if (h->stepped) return DLM_E_STATE;
  const CkptParts c = ckpt_parts(h);
  if (dst_bytes < c.total) return DLM_E_SIZE;
  unsigned char hd_bytes[kCkptHeaderBytes] = {};
  CkptHeader hd{};
  std::memcpy(hd.magic, kCkptMagic, sizeof(kCkptMagic));
  hd.version = kCkptVersion;
  hd.header_bytes = (uint32_t)kCkptHeaderBytes;
  hd.m = h->m;
  hd.r = h->r;
  hd.t = h->t;
  hd.last_t = h->last_t;
  hd.M = h->M;
  hd.flops = h->flops;
  hd.small_bytes = c.small_bytes;
  hd.z_bytes = c.z_bytes;
  hd.kv_bytes = c.kv_bytes;
  hd.total = c.total;
  std::memcpy(hd_bytes, &hd, sizeof(hd));
  unsigned char* d = static_cast<unsigned char*>(dst);
  TRY(hipMemcpyAsync(d, hd_bytes, kCkptHeaderBytes, hipMemcpyDefault, h->stream));
  d += kCkptHeaderBytes;
  TRY(hipMemcpyAsync(d, h->base + c.small_off, c.small_bytes, hipMemcpyDefault, h->stream));
  d += c.small_bytes;
  {
    const size_t zb = (size_t)h->r.batch * h->r.seq_len * h->m.vocab * 4;
    TRY(hipMemcpyAsync(d, h->base + ckpt_prev_z(h), zb, hipMemcpyDefault, h->stream));
    if (c.z_bytes > zb)
      TRY(hipMemcpyAsync(d + zb, h->base + ckpt_cur_z(h), zb, hipMemcpyDefault, h->stream));
  }
  d += c.z_bytes;
  TRY(hipMemcpyAsync(d, h->base + c.kv_off, c.kv_bytes, hipMemcpyDefault, h->stream));
  TRY(hipStreamSynchronize(h->stream));  // hd_bytes lives on this stack frame
  return DLM_OK;
}

int dlm_checkpoint_load(dlm_handle* h, const void* src, size_t src_bytes) {
  if (!h || !src) return DLM_E_INVALID;
  if (h->stepped) return DLM_E_STATE;
  const CkptParts c = ckpt_parts(h);
  if (src_bytes < c.total) return DLM_E_SIZE;
  CkptHeader hd{};
  TRY(hipMemcpyAsync(&hd, src, sizeof(hd), hipMemcpyDefault, h->stream));
  TRY(hipStreamSynchronize(h->stream));
  const int64_t BN = (int64_t)h->r.batch * h->r.seq_len;
  const bool ok =
      std::memcmp(hd.magic, kCkptMagic, sizeof(kCkptMagic)) == 0 &&
      hd.version == kCkptVersion && hd.header_bytes == kCkptHeaderBytes &&
      std::memcmp(&hd.m, &h->m, sizeof(dlm_model_desc)) == 0 &&
      std::memcmp(&hd.r, &h->r, sizeof(dlm_run_desc)) == 0 && hd.small_bytes == c.small_bytes &&
      hd.z_bytes == c.z_bytes && hd.kv_bytes == c.kv_bytes && hd.total == c.total &&
      hd.t >= 0 && hd.t <= h->r.steps && hd.last_t == hd.t - 1 && hd.M >= 0 && hd.M <= BN;
  if (!ok) return DLM_E_INVALID;
  h->t = hd.t;  // fixes which logits buffer the next step reads as the previous one
  const unsigned char* s = static_cast<const unsigned char*>(src) + kCkptHeaderBytes;
  TRY(hipMemcpyAsync(h->base + c.small_off, s, c.small_bytes, hipMemcpyDefault, h->stream));
  s += c.small_bytes;
  {
    const size_t zb = (size_t)h->r.batch * h->r.seq_len * h->m.vocab * 4;
    TRY(hipMemcpyAsync(h->base + ckpt_prev_z(h), s, zb, hipMemcpyDefault, h->stream));
    if (c.z_bytes > zb)
      TRY(hipMemcpyAsync(h->base + ckpt_cur_z(h), s + zb, zb, hipMemcpyDefault, h->stream));
  }
  s += c.z_bytes;
  TRY(hipMemcpyAsync(h->base + c.kv_off, s, c.kv_bytes, hipMemcpyDefault, h->stream));
  TRY(hipStreamSynchronize(h->stream));
  h->last_t = hd.last_t;
  h->M = hd.M;
  h->flops = hd.flops;
  h->stepped = false;
  return DLM_OK;
}

int dlm_last_step_info(const dlm_handle* h, int32_t* step, int32_t* m_tot, double* flops) {
  if (!h) return DLM_E_INVALID;
  if (step) *step = h->last_t;
  if (m_tot) *m_tot = h->M;
  if (flops) *flops = h->flops;
  return DLM_OK;
}

int dlm_destroy(dlm_handle* h) {
  if (!h) return DLM_E_INVALID;
  hipError_t e = hipStreamSynchronize(h->stream);
  for (const Timed& x : h->pending) {
    hipEventDestroy(x.e0);
    hipEventDestroy(x.e1);
  }
  for (hipEvent_t ev : h->pool) hipEventDestroy(ev);
  delete h;
  return hip_status(e);
}

int dlm_set_timing(dlm_handle* h, int32_t on) {
  if (!h) return DLM_E_INVALID;
  if (harvest(h) != hipSuccess) return DLM_E_HIP;
  h->timing = on != 0;
  for (int c = 0; c < DLM_K_NUM_CLASSES; ++c) {
    h->t_ms[c] = h->t_bytes[c] = h->t_flops[c] = 0.0;
    h->t_n[c] = 0;
  }
  return DLM_OK;
}

int dlm_read_timing(dlm_handle* h, int32_t kclass, double* total_ms, int64_t* launches,
                    double* bytes, double* flops) {
  if (!h || kclass < 0 || kclass >= DLM_K_NUM_CLASSES) return DLM_E_INVALID;
  if (harvest(h) != hipSuccess) return DLM_E_HIP;
  if (total_ms) *total_ms = h->t_ms[kclass];
  if (launches) *launches = h->t_n[kclass];
  if (bytes) *bytes = h->t_bytes[kclass];
  if (flops) *flops = h->t_flops[kclass];
  return DLM_OK;
}

// ---------------------------------------------------------------------------
// op-level ABI
// ---------------------------------------------------------------------------
static bool dt_ok(int32_t dt) { return dt == DLM_FP32 || dt == DLM_BF16; }

int dlm_op_compact(const uint64_t* bits, int32_t batch, int32_t seq_len, int32_t* row_seq,
                   int32_t* row_pos, int32_t* m_b, int32_t* row_start, int32_t* ctl,
                   void* stream) {
  if (!bits || !row_seq || !row_pos || !m_b || !row_start || !ctl) return DLM_E_INVALID;
  if (batch < 1 || batch > 1024 || seq_len < 1 || (int64_t)batch * seq_len > (1 << 24))
    return DLM_E_INVALID;
  return hip_status(launch_compact(bits, nullptr, batch, seq_len, row_seq, row_pos, m_b,
                                   row_start, ctl, (hipStream_t)stream));
}

int dlm_op_embed_rmsnorm(int32_t dtype, int32_t M, int32_t d, int32_t seq_len, float eps,
                         int32_t mask_id, const int32_t* tokens, const int32_t* row_seq,
                         const int32_t* row_pos, const void* emb, const void* g, float* h,
                         void* y, int32_t* row_real, void* stream) {
  if (!dt_ok(dtype) || M < 0 || d < 1 || seq_len < 1) return DLM_E_INVALID;
  if (M > 0 && (!tokens || !row_seq || !row_pos || !emb || !g || !h || !y || !row_real))
    return DLM_E_INVALID;
  return hip_status(launch_embed_rmsnorm(dtype, M, d, seq_len, eps, mask_id, tokens, row_seq,
                                         row_pos, emb, g, h, y, row_real, (hipStream_t)stream));
}

int dlm_op_rmsnorm(int32_t dtype, int32_t M, int32_t d, float eps, const float* x, const void* g,
                   void* y, void* stream) {
  if (!dt_ok(dtype) || M < 0 || d < 1) return DLM_E_INVALID;
  if (M > 0 && (!x || !g || !y)) return DLM_E_INVALID;
  return hip_status(launch_rmsnorm(dtype, M, d, eps, x, g, y, (hipStream_t)stream));
}

size_t dlm_op_gemm_ws_bytes(int32_t dtype, int32_t epi, int32_t M, int32_t N, int32_t K) {
  if (!dt_ok(dtype) || epi < 0 || epi > 3 || M < 0 || N < 1 || K < 1) return 0;
  return gemm_ws_bytes(dtype, epi, M, N, K);
}

int dlm_op_gemm(int32_t dtype, int32_t epi, int32_t M, int32_t N, int32_t K, const void* A,
                const void* W, const void* W2, void* C, const int32_t* row_seq,
                const int32_t* row_pos, int32_t seq_len, int32_t mask_id, void* ws,
                size_t ws_bytes, void* stream) {
  if (!dt_ok(dtype) || epi < 0 || epi > 3 || M < 0 || N < 1 || K < 1) return DLM_E_INVALID;
  if (M == 0) return DLM_OK;
  if (!A || !W || !C || (epi == kEpiSwiglu && !W2)) return DLM_E_INVALID;
  if (epi == kEpiLogits && (!row_seq || !row_pos || seq_len < 1)) return DLM_E_INVALID;
  auto al16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  if (!al16(A) || !al16(W) || (W2 && !al16(W2))) return DLM_E_INVALID;
  GemmArgs g{dtype, epi, M, N, K, A, W, W2, C, row_seq, row_pos, seq_len, mask_id,
             nullptr, nullptr, nullptr, nullptr, 0, 0};
  return hip_status(launch_gemm(g, ws, ws ? ws_bytes : 0, (hipStream_t)stream));
}

int dlm_op_gemm_num_configs(void) { return gemm_num_configs(); }

size_t dlm_op_gemm_noalloc_max_bytes(void) { return kGemmScratchBytes; }

int dlm_op_gemm_noalloc(int32_t dtype, int32_t epi, int32_t M, int32_t N, int32_t K,
                        const void* A, const void* W, const void* W2, void* C,
                        const int32_t* row_seq, const int32_t* row_pos, int32_t seq_len,
                        int32_t mask_id, void* stream) {
  if (!dt_ok(dtype) || epi < 0 || epi > 3 || M < 0 || N < 1 || K < 1) return DLM_E_INVALID;
  if (M == 0) return DLM_OK;
  if (!A || !W || !C || (epi == kEpiSwiglu && !W2)) return DLM_E_INVALID;
  if (epi == kEpiLogits && (!row_seq || !row_pos || seq_len < 1)) return DLM_E_INVALID;
  auto al16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  if (!al16(A) || !al16(W) || (W2 && !al16(W2))) return DLM_E_INVALID;
  // the plan dlm_op_gemm takes with enough workspace; its split-K partials
  // must fit the scratch array
  if (gemm_ws_bytes(dtype, epi, M, N, K) > kGemmScratchBytes) return DLM_E_SIZE;
  void* ws = nullptr;
  const int st = gemm_scratch_for((hipStream_t)stream, &ws);
  if (st != DLM_OK) return st;
  GemmArgs g{dtype, epi, M, N, K, A, W, W2, C, row_seq, row_pos, seq_len, mask_id,
             nullptr, nullptr, nullptr, nullptr, 0, 0};
  return hip_status(launch_gemm(g, ws, kGemmScratchBytes, (hipStream_t)stream));
}

int dlm_op_gemm_config(int32_t dtype, int32_t epi, int32_t M, int32_t N, int32_t K,
                       const void* A, const void* W, const void* W2, void* C,
                       const int32_t* row_seq, const int32_t* row_pos, int32_t seq_len,
                       int32_t mask_id, int32_t cfg, int32_t splits, void* ws, size_t ws_bytes,
                       void* stream) {
  if (!dt_ok(dtype) || epi < 0 || epi > 3 || M < 0 || N < 1 || K < 1 || splits < 0 ||
      cfg >= gemm_num_configs())
    return DLM_E_INVALID;
  if (M == 0) return DLM_OK;
  if (!A || !W || !C || (epi == kEpiSwiglu && !W2)) return DLM_E_INVALID;
  if (epi == kEpiLogits && (!row_seq || !row_pos || seq_len < 1)) return DLM_E_INVALID;
  auto al16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  if (!al16(A) || !al16(W) || (W2 && !al16(W2))) return DLM_E_INVALID;
  if (splits > 1 && (size_t)splits * M * N * (epi == kEpiSwiglu ? 8 : 4) > ws_bytes)
    return DLM_E_SIZE;
  GemmArgs g{dtype, epi, M, N, K, A, W, W2, C, row_seq, row_pos, seq_len, mask_id,
             nullptr, nullptr, nullptr, nullptr, 0, 0};
  return hip_status(launch_gemm_cfg(g, cfg, splits, ws, ws ? ws_bytes : 0, (hipStream_t)stream));
}

int dlm_op_gemm_qkv(int32_t M, int32_t K, int32_t nq, int32_t nkv, int32_t seq_len,
                    const void* A, const void* W, const int32_t* row_seq, const int32_t* row_pos,
                    const float* rope_table, void* q, void* kcache, void* vcache, int32_t cfg,
                    void* stream) {
  if (M < 0 || K < 1 || nq < 1 || nkv < 1 || nq % nkv || seq_len < 1 ||
      cfg >= gemm_num_configs())
    return DLM_E_INVALID;
  if (K % 64 != 0) return DLM_E_UNSUPPORTED;
  if (M == 0) return DLM_OK;
  if (!A || !W || !row_seq || !row_pos || !q || !kcache || !vcache) return DLM_E_INVALID;
  auto al16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  if (!al16(A) || !al16(W) || ((uintptr_t)q & 3) || ((uintptr_t)kcache & 3) ||
      ((uintptr_t)vcache & 7) || (rope_table && !al16(rope_table)))
    return DLM_E_INVALID;
  GemmArgs g{kBF16, kEpiQKV, M, (nq + 2 * nkv) * 128, K, A, W, nullptr, nullptr, row_seq, row_pos,
             seq_len, 0, rope_table, q, kcache, vcache, nq, nkv};
  const hipError_t e = launch_gemm_cfg(g, cfg, 1, nullptr, 0, (hipStream_t)stream);
  if (e == hipErrorInvalidValue) return DLM_E_UNSUPPORTED;
  return hip_status(e);
}

int dlm_op_rope_table(int32_t seq_len, int32_t head_dim, float base, float* table,
                      void* stream) {
  if (seq_len < 1 || head_dim < 2 || (head_dim & 1) || !table || !(base > 0.f))
    return DLM_E_INVALID;
  return hip_status(launch_rope_table(seq_len, head_dim, base, table, (hipStream_t)stream));
}

int dlm_op_rope_scatter(int32_t dtype, int32_t M, int32_t nq, int32_t nkv, int32_t hd,
                        int32_t seq_len, const float* qkv, const int32_t* row_seq,
                        const int32_t* row_pos, const float* table, void* q, void* kcache,
                        void* vcache, void* stream) {
  if (!dt_ok(dtype) || M < 0 || nq < 1 || nkv < 1 || hd < 2 || (hd & 1) || seq_len < 1)
    return DLM_E_INVALID;
  if (M > 0 && (!qkv || !row_seq || !row_pos || !q || !kcache || !vcache)) return DLM_E_INVALID;
  return hip_status(launch_rope_scatter(dtype, M, nq, nkv, hd, seq_len, qkv, row_seq, row_pos,
                                        table, q, kcache, vcache, (hipStream_t)stream));
}

size_t dlm_op_attention_ws_bytes(int32_t dtype, int32_t M, int32_t batch, int32_t seq_len,
                                 int32_t nq, int32_t nkv, int32_t hd) {
  if (!dt_ok(dtype) || M < 0 || batch < 1 || seq_len < 1 || nq < 1 || nkv < 1 || nq % nkv)
    return 0;
  return attention_ws_bytes(dtype, M, batch, seq_len, nq, nkv, hd);
}

int dlm_op_attention(int32_t dtype, int32_t M, int32_t batch, int32_t seq_len, int32_t nq,
                     int32_t nkv, int32_t hd, const void* q, const int32_t* row_start,
                     const void* kcache, const void* vcache, void* o, void* ws,
                     size_t ws_bytes, void* stream) {
  if (!dt_ok(dtype) || M < 0 || batch < 1 || seq_len < 1 || nq < 1 || nkv < 1 || nq % nkv ||
      hd < 2 || hd > 256 || (hd & 1))
    return DLM_E_INVALID;
  if (M == 0) return DLM_OK;
  if (!q || !row_start || !kcache || !vcache || !o) return DLM_E_INVALID;
  return hip_status(launch_attention(dtype, M, batch, seq_len, nq, nkv, hd, q, row_start, kcache,
                                     vcache, o, ws, ws ? ws_bytes : 0, (hipStream_t)stream));
}

size_t dlm_op_attention_config_ws_bytes(int32_t dtype, int32_t M, int32_t batch, int32_t seq_len,
                                        int32_t nq, int32_t nkv, int32_t hd, int32_t splits) {
  if (!dt_ok(dtype) || M < 0 || batch < 1 || seq_len < 1 || nq < 1 || nkv < 1 || nq % nkv ||
      splits < 0)
    return 0;
  return attention_cfg_ws_bytes(dtype, M, batch, seq_len, nq, nkv, hd, splits);
}

int dlm_op_attention_config(int32_t dtype, int32_t M, int32_t batch, int32_t seq_len, int32_t nq,
                            int32_t nkv, int32_t hd, const void* q, const int32_t* row_start,
                            const void* kcache, const void* vcache, void* o, int32_t splits,
                            int32_t stages, int32_t key_halves, int32_t qblocks,
                            int32_t key_tile, void* ws, size_t ws_bytes, void* stream) {
  if (!dt_ok(dtype) || M < 0 || batch < 1 || seq_len < 1 || nq < 1 || nkv < 1 || nq % nkv ||
      hd < 2 || hd > 256 || (hd & 1) || splits < 0 || (stages != 0 && stages != 2 && stages != 4) ||
      (key_halves != 0 && key_halves != 1 && key_halves != 2 && key_halves != 4) ||
      qblocks < 0 || qblocks > 2 || (key_tile != 0 && key_tile != 64 && key_tile != 128))
    return DLM_E_INVALID;
  if (M == 0) return DLM_OK;
  if (!q || !row_start || !kcache || !vcache || !o) return DLM_E_INVALID;
  if (attention_cfg_ws_bytes(dtype, M, batch, seq_len, nq, nkv, hd, splits) > (ws ? ws_bytes : 0))
    return DLM_E_SIZE;
  return hip_status(launch_attention_cfg(dtype, M, batch, seq_len, nq, nkv, hd, q, row_start,
                                         kcache, vcache, o, ws, ws ? ws_bytes : 0, splits, stages,
                                         key_halves, qblocks, key_tile, (hipStream_t)stream));
}

int dlm_op_attention_num_layouts(void) { return attention_num_layouts(); }

size_t dlm_op_attention_layout_ws_bytes(int32_t dtype, int32_t M, int32_t batch, int32_t seq_len,
                                        int32_t nq, int32_t nkv, int32_t hd, int32_t splits,
                                        int32_t layout) {
  if (!dt_ok(dtype) || M < 0 || batch < 1 || seq_len < 1 || nq < 1 || nkv < 1 || nq % nkv ||
      splits < 0)
    return 0;
  return attention_layout_ws_bytes(dtype, M, batch, seq_len, nq, nkv, hd, splits, layout);
}

int dlm_op_attention_layout(int32_t dtype, int32_t M, int32_t batch, int32_t seq_len, int32_t nq,
                            int32_t nkv, int32_t hd, const void* q, const int32_t* row_start,
                            const void* kcache, const void* vcache, void* o, int32_t splits,
                            int32_t layout, void* ws, size_t ws_bytes, void* stream) {
  if (!dt_ok(dtype) || M < 0 || batch < 1 || seq_len < 1 || nq < 1 || nkv < 1 || nq % nkv ||
      splits < 0 || layout < -1 || layout >= attention_num_layouts())
    return DLM_E_INVALID;
  if (M == 0) return DLM_OK;
  if (!q || !row_start || !kcache || !vcache || !o) return DLM_E_INVALID;
  if (layout >= 0 && !attention_layout_supported(dtype, seq_len, hd, layout))
    return DLM_E_UNSUPPORTED;
  if (layout < 0 && attention_layout_ws_bytes(dtype, M, batch, seq_len, nq, nkv, hd, 0, -1) == 0 &&
      !(dtype == DLM_BF16 && (hd == 64 || hd == 128) && seq_len % 64 == 0))
    return DLM_E_UNSUPPORTED;
  if (attention_layout_ws_bytes(dtype, M, batch, seq_len, nq, nkv, hd, splits, layout) >
      (ws ? ws_bytes : 0))
    return DLM_E_SIZE;
  const hipError_t e = launch_attention_layout(dtype, M, batch, seq_len, nq, nkv, hd, q,
                                               row_start, kcache, vcache, o, ws,
                                               ws ? ws_bytes : 0, splits, layout,
                                               (hipStream_t)stream);
  return e == hipErrorInvalidValue ? DLM_E_UNSUPPORTED : hip_status(e);
}

size_t dlm_op_vocab_ws_bytes(int32_t M, int32_t V) {
  if (M < 0 || V < 1) return 0;
  return vocab_ws_bytes(M, V);
}

int dlm_op_vocab_stats(int32_t M, int32_t V, int32_t mask_id, int32_t kl_dir, int32_t seq_len,
                       const int32_t* row_seq, const int32_t* row_pos, const float* z_cur,
                       const float* z_prev, const float* lse_prev, int32_t* has_prev,
                       float* lse_cur, int32_t* argmax, float* conf, float* kl,
                       int32_t* has_kl, float* lse_row, int32_t* err, void* ws,
                       size_t ws_bytes, void* stream) {
  if (M < 0 || V < 2 || (kl_dir != 0 && kl_dir != 1) || seq_len < 1) return DLM_E_INVALID;
  if (M == 0) return DLM_OK;
  if (!row_seq || !row_pos || !z_cur || !z_prev || !lse_prev || !has_prev || !lse_cur ||
      !argmax || !conf || !kl || !has_kl || !lse_row || !err || !ws)
    return DLM_E_INVALID;
  if (vocab_ws_bytes(M, V) > ws_bytes) return DLM_E_SIZE;
  return hip_status(launch_vocab_stats(M, V, mask_id, kl_dir, seq_len, row_seq, row_pos, z_cur,
                                       z_prev, lse_prev, has_prev, lse_cur, argmax, conf, kl,
                                       has_kl, lse_row, err, ws, ws_bytes, (hipStream_t)stream));
}

size_t dlm_op_lm_head_stats_ws_bytes(int32_t M, int32_t V, int32_t K, int32_t cfg) {
  if (M < 0 || V < 2 || K < 1 || cfg >= gemm_num_configs()) return 0;
  if (!gemm_logits_stats_fusable(kBF16, K) || M == 0) return 0;
  return (size_t)M * gemm_logits_stats_parts(M, V, K, cfg) * kVocabPartBytes;
}

int dlm_op_lm_head_stats(int32_t M, int32_t V, int32_t K, const void* A, const void* W,
                         float* z_cur, const int32_t* row_seq, const int32_t* row_pos,
                         int32_t seq_len, int32_t mask_id, int32_t kl_dir, const float* z_prev,
                         const float* lse_prev, int32_t* has_prev, float* lse_cur,
                         int32_t* argmax, float* conf, float* kl, int32_t* has_kl,
                         float* lse_row, int32_t* err, int32_t cfg, void* ws, size_t ws_bytes,
                         void* stream) {
  if (M < 0 || V < 2 || K < 1 || (kl_dir != 0 && kl_dir != 1) || seq_len < 1 ||
      mask_id < 0 || mask_id >= V || cfg >= gemm_num_configs())
    return DLM_E_INVALID;
  if (!gemm_logits_stats_fusable(kBF16, K)) return DLM_E_UNSUPPORTED;
  if (M == 0) return DLM_OK;
  if (!A || !W || !z_cur || !row_seq || !row_pos || !z_prev || !lse_prev || !has_prev ||
      !lse_cur || !argmax || !conf || !kl || !has_kl || !lse_row || !err || !ws)
    return DLM_E_INVALID;
  auto al16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  if (!al16(A) || !al16(W)) return DLM_E_INVALID;
  const int nparts = gemm_logits_stats_parts(M, V, K, cfg);
  if ((size_t)M * nparts * kVocabPartBytes > ws_bytes) return DLM_E_SIZE;
  hipStream_t s = (hipStream_t)stream;
  GemmArgs g{kBF16, kEpiLogitsStats, M, V, K, A, W, nullptr, z_cur, row_seq, row_pos, seq_len,
             mask_id, nullptr, nullptr, nullptr, nullptr, 0, 0, z_prev, lse_prev, has_prev, ws,
             kl_dir};
  const hipError_t e = launch_gemm_logits_stats(g, cfg, s);
  if (e != hipSuccess) return e == hipErrorInvalidValue ? DLM_E_UNSUPPORTED : DLM_E_HIP;
  return hip_status(launch_vocab_merge_parts(M, nparts, seq_len, kl_dir, row_seq, row_pos,
                                             lse_prev, has_prev, lse_cur, ws, argmax, conf, kl,
                                             has_kl, lse_row, err, s));
}

int dlm_op_commit_lock(int32_t batch, int32_t seq_len, int32_t prompt_len, int32_t mask_id,
                       int32_t blk_lo, int32_t blk_hi, int32_t k, int32_t do_commit,
                       int32_t do_lock, int32_t policy, float kl_eps, float conf_tau,
                       int32_t n_consec, int32_t lock_prompt, const int32_t* row_seq,
                       const int32_t* row_pos, const int32_t* row_start,
                       const int32_t* row_real, const int32_t* argmax, const float* conf,
                       const float* kl, const int32_t* has_kl, int32_t* tokens,
                       uint64_t* bits, int32_t* counters, void* stream) {
  if (batch < 1 || batch > 1024 || seq_len < 1 || prompt_len < 0 || prompt_len > seq_len ||
      blk_lo < 0 || blk_hi < blk_lo || blk_hi > seq_len || blk_hi - blk_lo > 4096 || k < 0 ||
      n_consec < 1)
    return DLM_E_INVALID;
  if (!row_pos || !row_start || !row_real || !argmax || !conf || !kl || !has_kl || !tokens ||
      !bits || !counters)
    return DLM_E_INVALID;
  LockArgs la{batch, seq_len, prompt_len, mask_id, blk_lo, blk_hi, k, do_commit, do_lock,
              policy, kl_eps, conf_tau, n_consec, lock_prompt, row_seq, row_pos, row_start,
              row_real, argmax, conf, kl, has_kl, tokens, bits, counters};
  return hip_status(launch_commit_lock(la, (hipStream_t)stream));
}

int dlm_op_slowfast_commit(int32_t batch, int32_t seq_len, int32_t mask_id, int32_t window,
                           int32_t sf_k, int32_t sf_kmax, int32_t sf_whist, float sf_tau_conv,
                           float sf_tau_high, float sf_var, const int32_t* row_pos,
                           const int32_t* row_start, const int32_t* argmax, const float* conf,
                           int32_t* tokens, uint64_t* frozen, int32_t* has_prev,
                           int32_t* sf_state, void* stream) {
  if (batch < 1 || batch > 1024 || seq_len < 1 || seq_len > 4096 || window < 1 || sf_k < 1 ||
      sf_kmax < 1 || sf_whist < 1 || sf_whist > 8 || std::isnan(sf_tau_conv) ||
      std::isnan(sf_tau_high) || std::isnan(sf_var))
    return DLM_E_INVALID;
  if (!row_pos || !row_start || !argmax || !conf || !tokens || !frozen || !has_prev || !sf_state)
    return DLM_E_INVALID;
  LockArgs la{};
  la.B = batch;
  la.N = seq_len;
  la.mask_id = mask_id;
  la.do_commit = 1;
  la.do_lock = 0;
  la.row_pos = row_pos;
  la.row_start = row_start;
  la.argmax = argmax;
  la.conf = conf;
  la.tokens = tokens;
  la.sampler = DLM_SAMPLER_SLOWFAST;
  la.sf_window = window;
  la.sf_k = sf_k;
  la.sf_kmax = sf_kmax;
  la.sf_whist = sf_whist;
  la.sf_tau_conv = sf_tau_conv;
  la.sf_tau_high = sf_tau_high;
  la.sf_var = sf_var;
  la.frozen = frozen;
  la.has_prev = has_prev;
  la.sf_state = sf_state;
  return hip_status(launch_commit_lock(la, (hipStream_t)stream));
}

}  // extern "C"

// Lock-state kernels: state init, active-set compaction, commit + lock
// transition, replay override.
//
// SureLock page ("Stopping Computation for Converged Tokens in Masked
// Diffusion-LM Decoding"), §2 Methodology, core mechanism: a position whose
// step-wise KL(p_t || p_{t-1}) is at most eps (with an optional confidence
// gate) is locked and leaves the active set A_t for all later steps; the
// active count M_t is therefore non-increasing (§2 algorithmic complexity).
// SlowFast page ("Accelerating Diffusion LLMs with SlowFast Sampling"), §1
// and §2: positions are unmasked by confidence-ranked top-k inside
// semi-autoregressive blocks, or by SlowFast's two-stage cycle (exploratory
// top-k while the convergence end point settles, then every high-confidence
// position of the stable span at once, positions beyond the span kept out of
// the active set until the span is decoded).
#include "common.h"
#include "internal.h"

namespace dlm {

// ---------------------------------------------------------------------------
__global__ void init_state_kernel(int B, int N, int P, int mask_id, const int32_t* prompts,
                                  int32_t* tokens, uint64_t* bits, int32_t* counters,
                                  int32_t* has_prev, int32_t* ctl, uint64_t* frozen,
                                  int32_t* sf_state) {
  const int W = (N + 63) >> 6;
  const size_t total = (size_t)B * N;
  for (size_t f = blockIdx.x * (size_t)blockDim.x + threadIdx.x; f < total;
       f += (size_t)gridDim.x * blockDim.x) {
    if (f < (size_t)B * N) {
      const int b = (int)(f / N), i = (int)(f - (size_t)b * N);
      tokens[f] = i < P ? prompts[(size_t)b * P + i] : mask_id;
      counters[f] = 0;
      has_prev[f] = 0;
    }
    if (f < (size_t)B * W) {
      bits[f] = 0ull;
      frozen[f] = 0ull;
    }
    if (f < (size_t)B * kSfStateInts) sf_state[f] = 0;
    if (f < 4) ctl[f] = 0;
  }
}

hipError_t launch_init_state(int B, int N, int P, int mask_id, const int32_t* prompts,
                             int32_t* tokens, uint64_t* bits, int32_t* counters,
                             int32_t* has_prev, int32_t* ctl, uint64_t* frozen,
                             int32_t* sf_state, hipStream_t s) {
  const size_t total = std::max<size_t>((size_t)B * N, (size_t)B * kSfStateInts);
  const int grid = (int)std::min<size_t>((total + 255) / 256, 4096);
  init_state_kernel<<<grid, 256, 0, s>>>(B, N, P, mask_id, prompts, tokens, bits, counters,
                                         has_prev, ctl, frozen, sf_state);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Compaction: one workgroup of 1024 threads scans the B*N positions in
// (seq, pos) order, 1024 at a time.  Each wave ballots its 64 "active"
// predicates; the lane's rank is the popcount of the ballot below it, the
// wave's base is the prefix over the wave counts of this chunk.
constexpr int kCompactThreads = 1024;

// A position is active when its lock bit and (if given) its frozen bit are
// both clear.
__global__ __launch_bounds__(kCompactThreads) void compact_kernel(
    const uint64_t* __restrict__ bits, const uint64_t* __restrict__ frozen, int B, int N,
    int32_t* __restrict__ row_seq,
    int32_t* __restrict__ row_pos, int32_t* __restrict__ m_b, int32_t* __restrict__ row_start,
    int32_t* __restrict__ ctl) {
  __shared__ int wave_cnt[kCompactThreads / 64];
  __shared__ int base_s;
  __shared__ int mb_s[1024];
  const int W = (N + 63) >> 6;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int total = B * N;
  if (tid == 0) base_s = 0;
  __syncthreads();
  for (int c0 = 0; c0 < total; c0 += kCompactThreads) {
    const int f = c0 + tid;
    bool act = false;
    int b = 0, i = 0;
    if (f < total) {
      b = f / N;
      i = f - b * N;
      uint64_t word = bits[(size_t)b * W + (i >> 6)];
      if (frozen) word |= frozen[(size_t)b * W + (i >> 6)];
      act = !((word >> (i & 63)) & 1ull);
    }
    const uint64_t ballot = __ballot(act);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(ballot >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)ballot, 0u));
    if (lane == 0) wave_cnt[w] = __popcll(ballot);
    __syncthreads();
    int off = base_s;
    for (int j = 0; j < w; ++j) off += wave_cnt[j];
    if (act) {
      row_seq[off + below] = b;
      row_pos[off + below] = i;
    }
    __syncthreads();
    if (tid == 0) {
      int t = 0;
      for (int j = 0; j < kCompactThreads / 64; ++j) t += wave_cnt[j];
      base_s += t;
    }
    __syncthreads();
  }
  // rows per sequence: popcount of the cleared bits below seq_len
  for (int b = tid; b < B; b += kCompactThreads) {
    int cnt = 0;
    for (int wd = 0; wd < W; ++wd) {
      uint64_t v = ~(bits[(size_t)b * W + wd] | (frozen ? frozen[(size_t)b * W + wd] : 0ull));
      const int valid = N - wd * 64;
      if (valid < 64) v &= (1ull << valid) - 1ull;
      cnt += __popcll(v);
    }
    mb_s[b] = cnt;
    m_b[b] = cnt;
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int b = 0; b < B; ++b) {
      row_start[b] = acc;
      acc += mb_s[b];
    }
    row_start[B] = acc;
    ctl[0] = base_s;
  }
}

hipError_t launch_compact(const uint64_t* bits, const uint64_t* frozen, int B, int N,
                          int32_t* row_seq, int32_t* row_pos, int32_t* m_b, int32_t* row_start,
                          int32_t* ctl, hipStream_t s) {
  compact_kernel<<<1, kCompactThreads, 0, s>>>(bits, frozen, B, N, row_seq, row_pos, m_b,
                                               row_start, ctl);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Commit + lock, one workgroup per sequence.
// Candidates (masked rows of the current block) are gathered in LDS; each
// candidate's rank is the number of candidates strictly ahead of it in the
// order (conf descending, position ascending); ranks below k commit.
constexpr int kLockThreads = 1024;

// SlowFast commit for sequence b ([SF] §2 two-stage pipeline), the rule of
// the CPU reference in the same words: candidates are this step's rows still
// holding the mask, the frontier s is the first of them.  Exploratory step:
// record the end point (largest candidate position with conf >= tau_conv,
// none if no candidate reaches it); the stage ends when sf_whist end points
// are recorded with population variance below sf_var (W sum e^2 - (sum e)^2 <
// W^2 sf_var, in integers) or after sf_kmax exploratory steps, with span
// [s, max(last end point, s)]; otherwise commit the sf_k most confident
// candidates of [s, s + window).  Accelerated step: commit every in-span
// candidate with conf > tau_high if at least sf_k do, else the sf_k most
// confident in-span candidates; while in-span masks remain, freeze the
// candidates at or beyond the span's end; when none remain, end the cycle:
// unfreeze, clear those positions' previous-posterior flag, reset the state.
// State per sequence (kSfStateInts ints): phase, lo, hi, slow_n, hist_n,
// hist[8].
__device__ void slowfast_commit(const LockArgs& a, int b, int C, const float* cconf,
                                const int* cpos, const int* crow, int s_front, int e_max) {
  __shared__ int sh_fast, sh_lo, sh_hi, sh_nhigh, sh_left;
  const int tid = threadIdx.x, N = a.N, W = (N + 63) >> 6;
  int32_t* st = a.sf_state + (size_t)b * kSfStateInts;
  int32_t* tok = a.tokens + (size_t)b * N;
  if (tid == 0) {
    int phase = st[0], lo = st[1], hi = st[2];
    if (phase == 0) {
      const int Wh = a.sf_whist;
      int hn = st[4];
      if (e_max >= 0) {
        if (hn < Wh) {
          st[5 + hn] = e_max;
          hn += 1;
        } else {
          for (int j = 1; j < Wh; ++j) st[5 + j - 1] = st[5 + j];
          st[5 + Wh - 1] = e_max;
        }
        st[4] = hn;
      }
      const int slow_n = st[3] + 1;
      st[3] = slow_n;
      bool stable = false;
      if (hn == Wh) {
        long long s1 = 0, s2 = 0;
        for (int j = 0; j < Wh; ++j) {
          s1 += st[5 + j];
          s2 += (long long)st[5 + j] * st[5 + j];
        }
        stable = (double)(Wh * s2 - s1 * s1) < (double)Wh * Wh * (double)a.sf_var;
      }
      if (stable || slow_n >= a.sf_kmax) {
        phase = 1;
        lo = s_front;
        hi = max(hn > 0 ? st[5 + hn - 1] : s_front, s_front) + 1;
        st[0] = phase;
        st[1] = lo;
        st[2] = hi;
      }
    }
    sh_fast = phase;
    sh_lo = lo;
    sh_hi = hi;
    sh_nhigh = 0;
    sh_left = 0;
  }
  __syncthreads();
  const int fast = sh_fast, lo = sh_lo, hi = sh_hi;
  // the candidate set of this step's commit rule
  auto eligible = [&](int c) {
    return fast ? (cpos[c] >= lo && cpos[c] < hi) : (cpos[c] < s_front + a.sf_window);
  };
  if (fast) {
    int nh = 0;
    for (int c = tid; c < C; c += kLockThreads)
      nh += eligible(c) && cconf[c] > a.sf_tau_high;
    if (nh) atomicAdd(&sh_nhigh, nh);
    __syncthreads();
  }
  const bool by_threshold = fast && sh_nhigh >= a.sf_k;
  for (int c = tid; c < C; c += kLockThreads) {
    if (!eligible(c)) continue;
    bool take;
    if (by_threshold) {
      take = cconf[c] > a.sf_tau_high;
    } else {
      const float cf = cconf[c];
      const int cp = cpos[c];
      int rank = 0;
      for (int j = 0; j < C; ++j) {
        if (!eligible(j)) continue;
        const float f = cconf[j];
        rank += (f > cf) || (f == cf && cpos[j] < cp);
      }
      take = rank < a.sf_k;
    }
    if (take) tok[cpos[c]] = a.argmax[crow[c]];
    else if (fast) sh_left = 1;  // benign race: every writer stores 1
  }
  if (!fast) return;
  __syncthreads();
  uint64_t* fz = a.frozen + (size_t)b * W;
  if (sh_left) {
    for (int c = tid; c < C; c += kLockThreads)
      if (cpos[c] >= hi) atomicOr((unsigned long long*)&fz[cpos[c] >> 6], 1ull << (cpos[c] & 63));
  } else {
    if (tid == 0)
      for (int j = 0; j < kSfStateInts; ++j) st[j] = 0;
    int32_t* hp = a.has_prev + (size_t)b * N;
    for (int w = tid; w < W; w += kLockThreads) {
      uint64_t v = fz[w];
      while (v) {
        const int bit = __builtin_ctzll(v);
        hp[w * 64 + bit] = 0;
        v &= v - 1;
      }
      fz[w] = 0ull;
    }
  }
}

__global__ __launch_bounds__(kLockThreads) void commit_lock_kernel(LockArgs a) {
  extern __shared__ unsigned char smem[];
  const int cap = a.sampler == 1 ? a.N : a.blk_hi - a.blk_lo;
  float* cconf = reinterpret_cast<float*>(smem);
  int* cpos = reinterpret_cast<int*>(cconf + (cap > 0 ? cap : 1));
  int* crow = cpos + (cap > 0 ? cap : 1);
  __shared__ int ncand;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int N = a.N, W = (N + 63) >> 6;
  const int r0 = a.row_start[b], r1 = a.row_start[b + 1];
  int32_t* tok = a.tokens + (size_t)b * N;

  if (a.do_commit && a.sampler == 1) {
    __shared__ int s_front, e_max;
    if (tid == 0) {
      ncand = 0;
      s_front = 0x7fffffff;
      e_max = -1;
    }
    __syncthreads();
    for (int r = r0 + tid; r < r1; r += kLockThreads) {
      const int pos = a.row_pos[r];
      if (tok[pos] == a.mask_id) {
        const int slot = atomicAdd(&ncand, 1);
        const float cf = a.conf[r];
        cconf[slot] = cf;
        cpos[slot] = pos;
        crow[slot] = r;
        atomicMin(&s_front, pos);
        if (cf >= a.sf_tau_conv) atomicMax(&e_max, pos);
      }
    }
    __syncthreads();
    if (ncand > 0) slowfast_commit(a, b, ncand, cconf, cpos, crow, s_front, e_max);
    __syncthreads();
  } else if (a.do_commit && a.k > 0 && cap > 0) {
    if (tid == 0) ncand = 0;
    __syncthreads();
    for (int r = r0 + tid; r < r1; r += kLockThreads) {
      const int pos = a.row_pos[r];
      if (pos >= a.blk_lo && pos < a.blk_hi && tok[pos] == a.mask_id) {
        const int slot = atomicAdd(&ncand, 1);
        cconf[slot] = a.conf[r];
        cpos[slot] = pos;
        crow[slot] = r;
      }
    }
    __syncthreads();
    const int C = ncand;
    for (int c = tid; c < C; c += kLockThreads) {
      const float cf = cconf[c];
      const int cp = cpos[c];
      int rank = 0;
#pragma unroll 8
      for (int j = 0; j < C; ++j) {
        const float f = cconf[j];
        rank += (f > cf) || (f == cf && cpos[j] < cp);
      }
      if (rank < a.k) tok[cp] = a.argmax[crow[c]];
    }
  }
  if (a.do_lock && a.policy == 1) {
    uint64_t* bw = a.bits + (size_t)b * W;
    for (int r = r0 + tid; r < r1; r += kLockThreads) {
      const int pos = a.row_pos[r];
      const bool pass = a.row_real[r] && a.has_kl[r] && (a.kl[r] <= a.kl_eps) &&
                        (a.conf[r] >= a.conf_tau);
      int32_t* cnt = a.counters + (size_t)b * N + pos;
      const int c = pass ? *cnt + 1 : 0;
      *cnt = c;
      if (c >= a.n_consec) atomicOr((unsigned long long*)&bw[pos >> 6], 1ull << (pos & 63));
    }
    if (a.lock_prompt) {
      for (int wd = tid; wd * 64 < a.P; wd += kLockThreads) {
        const int n = min(64, a.P - wd * 64);
        const uint64_t m = n == 64 ? ~0ull : ((1ull << n) - 1ull);
        atomicOr((unsigned long long*)&bw[wd], m);
      }
    }
  }
}

hipError_t launch_commit_lock(const LockArgs& a, hipStream_t s) {
  const int cap = std::max(1, a.sampler == 1 ? a.N : a.blk_hi - a.blk_lo);
  const size_t lds = (size_t)cap * (sizeof(float) + 2 * sizeof(int));
  commit_lock_kernel<<<a.B, kLockThreads, lds, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
__global__ void apply_override_kernel(int B, int N, int n_commit, const int32_t* cseq,
                                      const int32_t* cpos, const int32_t* ctok,
                                      const uint64_t* bits_or, const int32_t* counters,
                                      int32_t* tokens, uint64_t* bits, int32_t* cnt) {
  const int W = (N + 63) >> 6;
  const size_t bn = (size_t)B * N;
  const size_t nc = n_commit > 0 ? (size_t)n_commit : 0;
  const size_t total = bn > nc ? bn : nc;
  for (size_t f = blockIdx.x * (size_t)blockDim.x + threadIdx.x; f < total;
       f += (size_t)gridDim.x * blockDim.x) {
    if (f < nc) tokens[(size_t)cseq[f] * N + cpos[f]] = ctok[f];
    if (bits_or && f < (size_t)B * W) bits[f] |= bits_or[f];
    if (counters && f < (size_t)B * N) cnt[f] = counters[f];
  }
}

hipError_t launch_apply_override(int B, int N, int n_commit, const int32_t* cseq,
                                 const int32_t* cpos, const int32_t* ctok, const uint64_t* bits_or,
                                 const int32_t* counters, int32_t* tokens, uint64_t* bits,
                                 int32_t* cnt, hipStream_t s) {
  const size_t total = std::max<size_t>((size_t)B * N, (size_t)std::max(n_commit, 0));
  const int grid = (int)std::min<size_t>((total + 255) / 256, 4096);
  apply_override_kernel<<<grid, 256, 0, s>>>(B, N, n_commit, cseq, cpos, ctok, bits_or, counters,
                                             tokens, bits, cnt);
  return hipGetLastError();
}

}  // namespace dlm

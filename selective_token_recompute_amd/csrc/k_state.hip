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
// Polestar page ("Polestar: Drift-Aware Cache Calibration and Token
// Commitment ..."), section "Polestar: The Smart Painter", Polestar-Cache:
// optionally, the locked positions whose distribution drifted most (KL
// between a position's two latest posteriors) are recomputed, and unlocked
// when the drift measured then exceeds a threshold.
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
// Fill of a buffer with a 32-bit pattern (a kernel, not a memset, so that it
// may sit in a captured graph).
__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_u32(void* p, size_t bytes, uint32_t v, hipStream_t s) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  const int grid = (int)std::min<size_t>((n + 255) / 256, 8192);
  fill_u32_kernel<<<grid, 256, 0, s>>>((uint32_t*)p, n, v);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Compaction: one workgroup of 1024 threads scans the B*N positions in
// (seq, pos) order, 1024 at a time.  Each wave ballots its 64 "active"
// predicates; the lane's rank is the popcount of the ballot below it, the
// wave's base is the prefix over the wave counts of this chunk.
constexpr int kCompactThreads = 1024;

// A position is active when its lock bit (unless the refresh recomputes it)
// and its frozen bit (if given) are both clear; with last_step given, every
// active position records the step t.
__device__ __forceinline__ uint64_t inactive_word(const uint64_t* bits, const uint64_t* frozen,
                                                  const uint64_t* refresh, size_t w) {
  uint64_t word = bits[w];
  if (refresh) word &= ~refresh[w];
  if (frozen) word |= frozen[w];
  return word;
}

__global__ __launch_bounds__(kCompactThreads) void compact_kernel(
    const uint64_t* __restrict__ bits, const uint64_t* __restrict__ frozen, int B, int N,
    int32_t* __restrict__ row_seq,
    int32_t* __restrict__ row_pos, int32_t* __restrict__ m_b, int32_t* __restrict__ row_start,
    int32_t* __restrict__ ctl, const uint64_t* __restrict__ refresh,
    int32_t* __restrict__ last_step, int t) {
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
      const uint64_t word = inactive_word(bits, frozen, refresh, (size_t)b * W + (i >> 6));
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
      if (last_step) last_step[f] = t;
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
      uint64_t v = ~inactive_word(bits, frozen, refresh, (size_t)b * W + wd);
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
                          int32_t* ctl, hipStream_t s, const uint64_t* refresh,
                          int32_t* last_step, int t) {
  compact_kernel<<<1, kCompactThreads, 0, s>>>(bits, frozen, B, N, row_seq, row_pos, m_b,
                                               row_start, ctl, refresh, last_step, t);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Commit + lock, one workgroup per sequence.
// Candidates (masked rows of the current block) are gathered in LDS in row
// order; each candidate's rank is the number of candidates strictly ahead of
// it in the order (conf descending, position ascending); ranks below k
// commit.
constexpr int kLockThreads = 1024;
constexpr int kLockWaves = kLockThreads / 64;

// Key whose unsigned order is the commit order: confidence descending, then
// position ascending.  The confidence's bits are mapped to an unsigned
// integer of the same order (-0 taken as +0, so the two tie as floats do);
// the low half is INT_MAX - pos.  Every key is above 0, the padding key.
// (Confidences are maxima of a softmax: never NaN on a step that decides.)
__device__ __forceinline__ uint64_t rank_key(float conf, int pos) {
  uint32_t u = __float_as_uint(conf + 0.0f);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(0x7fffffff - pos);
}
__device__ __forceinline__ int key_pos(uint64_t key) {
  return 0x7fffffff - (int)(uint32_t)key;
}

// Gathers the rows r0 .. r1-1 for which take(pos) holds into (cconf, cpos,
// crow), in row order: a wave ballot gives each lane its slot among its
// wave's candidates and per-wave counts give the waves' offsets (a shared
// counter bumped by every candidate would serialise them).  Returns the
// number gathered, at most cap (the positions a candidate can hold, distinct
// for distinct rows), with each candidate's rank key, and pads the arrays to
// the next multiple of 16 (their length; padding keys are 0, behind every
// candidate); every thread of the workgroup calls it.
template <typename Take>
__device__ int gather_candidates(const LockArgs& a, int r0, int r1, Take take, int cap,
                                 uint64_t* ckey, float* cconf, int* cpos, int* crow) {
  __shared__ int wcnt[kLockWaves];
  __shared__ int s_base;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) s_base = 0;
  __syncthreads();
  for (int c0 = r0; c0 < r1; c0 += kLockThreads) {
    const int r = c0 + tid;
    int pos = 0;
    float cf = 0.f;
    bool t = false;
    if (r < r1) {
      pos = a.row_pos[r];
      cf = a.conf[r];
      t = take(pos);
    }
    const uint64_t bal = __ballot(t);
    if (lane == 0) wcnt[wv] = __popcll(bal);
    __syncthreads();
    int off = s_base;
    for (int w = 0; w < wv; ++w) off += wcnt[w];
    const int slot = off + __popcll(bal & ((1ull << lane) - 1ull));
    if (t && slot < cap) {
      ckey[slot] = rank_key(cf, pos);
      cconf[slot] = cf;
      cpos[slot] = pos;
      crow[slot] = r;
    }
    __syncthreads();
    if (tid == 0) {
      int n = s_base;
      for (int w = 0; w < kLockWaves; ++w) n += wcnt[w];
      s_base = n;
    }
    __syncthreads();
  }
  const int C = min(s_base, cap);
  // pad to a multiple of 16 with entries that rank behind every candidate
  if (tid < ((C + 15) & ~15) - C) {
    ckey[C + tid] = 0ull;
    cconf[C + tid] = -INFINITY;
    cpos[C + tid] = 0x7fffffff;
  }
  __syncthreads();
  return C;
}

// bits[pos / 64] |= 1 << (pos % 64) for the lanes with `set`: one atomic OR
// per distinct word per wave (lanes whose positions share a word OR their
// bits together first).  Every lane of the wave calls it.
__device__ void or_position_bits(uint64_t* bits, bool set, int pos) {
  const int lane = threadIdx.x & 63;
  bool pending = set;
  for (uint64_t pend = __ballot(pending); pend; pend = __ballot(pending)) {
    const int leader = __ffsll((unsigned long long)pend) - 1;
    const int w0 = __shfl(pos >> 6, leader);
    const bool mine = pending && (pos >> 6) == w0;
    unsigned long long v = mine ? (1ull << (pos & 63)) : 0ull;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o);
    if (lane == leader) atomicOr((unsigned long long*)&bits[w0], v);
    pending = pending && !mine;
  }
}

// bits[pos / 64] &= ~(1 << (pos % 64)) for the lanes with `clear`, one
// atomic AND per distinct word per wave.  Every lane of the wave calls it.
__device__ void clear_position_bits(uint64_t* bits, bool clear, int pos) {
  const int lane = threadIdx.x & 63;
  bool pending = clear;
  for (uint64_t pend = __ballot(pending); pend; pend = __ballot(pending)) {
    const int leader = __ffsll((unsigned long long)pend) - 1;
    const int w0 = __shfl(pos >> 6, leader);
    const bool mine = pending && (pos >> 6) == w0;
    unsigned long long v = mine ? (1ull << (pos & 63)) : 0ull;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o);
    if (lane == leader) atomicAnd((unsigned long long*)&bits[w0], ~v);
    pending = pending && !mine;
  }
}

// Rank of candidate c among the candidates whose position p has ok(p): the
// number whose key is above c's, counted only up to `cap` (a candidate with
// k candidates ahead of it is out of any top k).  16 keys per pass, read as
// 16-byte LDS broadcasts; branch-free (the keys are the same for every lane,
// and tests on them would otherwise compile to scalar branches).
template <typename Ok>
__device__ int rank_upto(int c, int C, const uint64_t* ckey, int cap, Ok ok) {
  const uint64_t kc = ckey[c];
  const int Cp = (C + 15) & ~15;
  int rank = 0;
  for (int j0 = 0; j0 < Cp && rank < cap; j0 += 16) {
    ulonglong2 k2[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) k2[q] = *reinterpret_cast<const ulonglong2*>(ckey + j0 + 2 * q);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      rank += (int)((k2[q].x > kc) & (bool)ok(key_pos(k2[q].x))) +
              (int)((k2[q].y > kc) & (bool)ok(key_pos(k2[q].y)));
  }
  return rank;
}

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
__device__ void slowfast_commit(const LockArgs& a, int b, int C, const uint64_t* ckey,
                                const float* cconf, const int* cpos, const int* crow,
                                int s_front, int e_max) {
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
  const int e_lo = fast ? lo : 0, e_hi = fast ? hi : s_front + a.sf_window;
  auto eligible_pos = [&](int p) { return (p >= e_lo) & (p < e_hi); };
  auto eligible = [&](int c) { return eligible_pos(cpos[c]); };
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
      take = rank_upto(c, C, ckey, a.sf_k, eligible_pos) < a.sf_k;
    }
    if (take) tok[cpos[c]] = a.argmax[crow[c]];
    else if (fast) sh_left = 1;  // benign race: every writer stores 1
  }
  if (!fast) return;
  __syncthreads();
  uint64_t* fz = a.frozen + (size_t)b * W;
  if (sh_left) {
    for (int c0 = 0; c0 < C; c0 += kLockThreads) {
      const int c = c0 + tid;
      const int p = c < C ? cpos[c] : 0;
      or_position_bits(fz, c < C && p >= hi, p);
    }
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
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int cap = a.sampler == 1 ? a.N : a.blk_hi - a.blk_lo;
  const int cap16 = ((cap > 0 ? cap : 1) + 15) & ~15;  // arrays padded to 16
  uint64_t* ckey = reinterpret_cast<uint64_t*>(smem);
  float* cconf = reinterpret_cast<float*>(ckey + cap16);
  int* cpos = reinterpret_cast<int*>(cconf + cap16);
  int* crow = cpos + cap16;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int N = a.N, W = (N + 63) >> 6;
  const int r0 = a.row_start[b], r1 = a.row_start[b + 1];
  int32_t* tok = a.tokens + (size_t)b * N;
  // a step whose posterior was non-finite decides nothing: its argmax and
  // statistics are not meaningful (the error is reported by the next step)
  if (a.err && *a.err) return;

  if (a.do_commit && a.sampler == 1) {
    __shared__ int s_front, e_max;
    const int C = gather_candidates(
        a, r0, r1, [&](int pos) { return tok[pos] == a.mask_id; }, cap, ckey, cconf, cpos,
        crow);
    // frontier (smallest candidate position) and end point (largest
    // candidate position with conf >= tau_conv, -1 if none): wave
    // reductions, then one shared update per wave
    if (tid == 0) {
      s_front = 0x7fffffff;
      e_max = -1;
    }
    __syncthreads();
    int lo = 0x7fffffff, hi = -1;
    for (int c = tid; c < C; c += kLockThreads) {
      lo = min(lo, cpos[c]);
      if (cconf[c] >= a.sf_tau_conv) hi = max(hi, cpos[c]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      lo = min(lo, __shfl_xor(lo, o));
      hi = max(hi, __shfl_xor(hi, o));
    }
    if ((tid & 63) == 0) {
      atomicMin(&s_front, lo);
      atomicMax(&e_max, hi);
    }
    __syncthreads();
    if (C > 0) slowfast_commit(a, b, C, ckey, cconf, cpos, crow, s_front, e_max);
    __syncthreads();
  } else if (a.do_commit && a.k > 0 && cap > 0) {
    const int C = gather_candidates(
        a, r0, r1,
        [&](int pos) { return pos >= a.blk_lo && pos < a.blk_hi && tok[pos] == a.mask_id; },
        cap, ckey, cconf, cpos, crow);
    for (int c = tid; c < C; c += kLockThreads)
      if (rank_upto(c, C, ckey, a.k, [](int) { return true; }) < a.k)
        tok[cpos[c]] = a.argmax[crow[c]];
  }
  // every recomputed position's drift: its KL between this posterior and the
  // one before (+inf while undefined), whatever decides the lock state
  if (a.drift)
    for (int r = r0 + tid; r < r1; r += kLockThreads)
      a.drift[(size_t)b * N + a.row_pos[r]] = a.has_kl[r] ? a.kl[r] : INFINITY;
  if (a.do_lock && a.policy == 1) {
    uint64_t* bw = a.bits + (size_t)b * W;
    const uint64_t* rw = a.refresh ? a.refresh + (size_t)b * W : nullptr;
    for (int c0 = r0; c0 < r1; c0 += kLockThreads) {
      const int r = c0 + tid;
      int pos = 0;
      bool lock = false, unlock = false;
      if (r < r1) {
        pos = a.row_pos[r];
        int32_t* cnt = a.counters + (size_t)b * N + pos;
        if (rw && ((rw[pos >> 6] >> (pos & 63)) & 1ull)) {
          // recomputed while locked: kept while the drift is defined and at
          // most refresh_eps, unlocked (counter cleared) otherwise
          unlock = !(a.has_kl[r] && a.kl[r] <= a.refresh_eps);
          if (unlock) *cnt = 0;
        } else {
          const bool pass = a.row_real[r] && a.has_kl[r] && (a.kl[r] <= a.kl_eps) &&
                            (a.conf[r] >= a.conf_tau);
          const int c = pass ? *cnt + 1 : 0;
          *cnt = c;
          lock = c >= a.n_consec;
        }
      }
      or_position_bits(bw, lock, pos);
      if (rw) clear_position_bits(bw, unlock, pos);
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
  const size_t lds =
      (size_t)((cap + 15) & ~15) * (sizeof(uint64_t) + sizeof(float) + 2 * sizeof(int));
  if (lds > 64 * 1024)
    (void)hipFuncSetAttribute((const void*)commit_lock_kernel,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  commit_lock_kernel<<<a.B, kLockThreads, lds, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
__global__ void apply_override_kernel(int B, int N, int n_commit, const int32_t* cseq,
                                      const int32_t* cpos, const int32_t* ctok,
                                      const uint64_t* bits_or, const int32_t* counters,
                                      int32_t* tokens, uint64_t* bits, int32_t* cnt,
                                      const uint64_t* refresh) {
  const int W = (N + 63) >> 6;
  const size_t bn = (size_t)B * N;
  const size_t nc = n_commit > 0 ? (size_t)n_commit : 0;
  const size_t total = bn > nc ? bn : nc;
  for (size_t f = blockIdx.x * (size_t)blockDim.x + threadIdx.x; f < total;
       f += (size_t)gridDim.x * blockDim.x) {
    if (f < nc) tokens[(size_t)cseq[f] * N + cpos[f]] = ctok[f];
    if (bits_or && f < (size_t)B * W)
      bits[f] = (refresh ? bits[f] & ~refresh[f] : bits[f]) | bits_or[f];
    if (counters && f < (size_t)B * N) cnt[f] = counters[f];
  }
}

hipError_t launch_apply_override(int B, int N, int n_commit, const int32_t* cseq,
                                 const int32_t* cpos, const int32_t* ctok, const uint64_t* bits_or,
                                 const int32_t* counters, int32_t* tokens, uint64_t* bits,
                                 int32_t* cnt, hipStream_t s, const uint64_t* refresh) {
  const size_t total = std::max<size_t>((size_t)B * N, (size_t)std::max(n_commit, 0));
  const int grid = (int)std::min<size_t>((total + 255) / 256, 4096);
  apply_override_kernel<<<grid, 256, 0, s>>>(B, N, n_commit, cseq, cpos, ctok, bits_or, counters,
                                             tokens, bits, cnt, refresh);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Refresh selection, one workgroup per sequence: the locked positions are
// gathered into LDS in position order by a wave ballot, each with the key of
// rank_key (drift in place of confidence: larger drift first, then smaller
// position); a candidate whose rank (keys above it, counted up to the budget)
// is below the budget is selected, sets its refresh bit and takes list slot
// `rank` (ranks are distinct: the keys are).
constexpr int kRefreshMaxN = 4096;  // keys of one sequence fit 32 KB of LDS

__global__ __launch_bounds__(kLockThreads) void refresh_select_kernel(
    int N, int budget, const uint64_t* __restrict__ bits, const float* __restrict__ drift,
    uint64_t* __restrict__ refresh, int32_t* __restrict__ rlist) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint64_t* ckey = reinterpret_cast<uint64_t*>(smem);
  __shared__ int wcnt[kLockWaves];
  __shared__ int s_base;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int W = (N + 63) >> 6;
  const uint64_t* bw = bits + (size_t)b * W;
  uint64_t* rw = refresh + (size_t)b * W;
  const float* dr = drift + (size_t)b * N;
  for (int w = tid; w < W; w += kLockThreads) rw[w] = 0ull;
  for (int j = tid; j < budget; j += kLockThreads) rlist[(size_t)b * budget + j] = -1;
  if (tid == 0) s_base = 0;
  __syncthreads();
  for (int p0 = 0; p0 < N; p0 += kLockThreads) {
    const int p = p0 + tid;
    const bool t = p < N && ((bw[p >> 6] >> (p & 63)) & 1ull);
    const uint64_t bal = __ballot(t);
    if (lane == 0) wcnt[wv] = __popcll(bal);
    __syncthreads();
    int off = s_base;
    for (int w = 0; w < wv; ++w) off += wcnt[w];
    if (t) ckey[off + __popcll(bal & ((1ull << lane) - 1ull))] = rank_key(dr[p], p);
    __syncthreads();
    if (tid == 0) {
      int n = s_base;
      for (int w = 0; w < kLockWaves; ++w) n += wcnt[w];
      s_base = n;
    }
    __syncthreads();
  }
  const int C = s_base;
  if (tid < ((C + 15) & ~15) - C) ckey[C + tid] = 0ull;  // padding ranks behind all
  __syncthreads();
  for (int c0 = 0; c0 < C; c0 += kLockThreads) {
    const int c = c0 + tid;
    int pos = 0, rank = budget;
    if (c < C) {
      pos = key_pos(ckey[c]);
      rank = rank_upto(c, C, ckey, budget, [](int) { return true; });
      if (rank < budget) rlist[(size_t)b * budget + rank] = pos;
    }
    or_position_bits(rw, rank < budget, pos);
  }
}

hipError_t launch_refresh_select(int B, int N, int budget, const uint64_t* bits,
                                 const float* drift, uint64_t* refresh, int32_t* rlist,
                                 hipStream_t s) {
  if (N > kRefreshMaxN || budget < 1) return hipErrorInvalidValue;
  const size_t lds = (size_t)((N + 15) & ~15) * sizeof(uint64_t);
  refresh_select_kernel<<<B, kLockThreads, lds, s>>>(N, budget, bits, drift, refresh, rlist);
  return hipGetLastError();
}

// Copy of a refreshed position's last posterior into the previous-step
// buffer: grid (B * budget list entries, vocabulary chunks of 4096).
constexpr int kCopyChunk = 4096;

__global__ __launch_bounds__(256) void refresh_copy_kernel(int N, int V, int budget, int t,
                                                           const int32_t* __restrict__ rlist,
                                                           const int32_t* __restrict__ last_step,
                                                           float* z0, float* z1, float* lse0,
                                                           float* lse1) {
  const int e = blockIdx.x, b = e / budget;
  const int pos = rlist[e];
  if (pos < 0) return;
  const size_t slot = (size_t)b * N + pos;
  const int ls = last_step[slot];
  const int src = ls & 1, dst = (t - 1) & 1;
  if (ls < 0 || src == dst) return;  // already where step t reads it
  const float* zs = (src ? z1 : z0) + slot * V;
  float* zd = (dst ? z1 : z0) + slot * V;
  const int c0 = blockIdx.y * kCopyChunk;
  const int c1 = min(V, c0 + kCopyChunk);
  for (int c = c0 + threadIdx.x; c < c1; c += 256) zd[c] = zs[c];
  if (blockIdx.y == 0 && threadIdx.x == 0) (dst ? lse1 : lse0)[slot] = (src ? lse1 : lse0)[slot];
}

hipError_t launch_refresh_copy(int B, int N, int V, int budget, int t, const int32_t* rlist,
                               const int32_t* last_step, float* z0, float* z1, float* lse0,
                               float* lse1, hipStream_t s) {
  if (budget < 1 || t < 1) return hipSuccess;
  const dim3 grid(B * budget, (V + kCopyChunk - 1) / kCopyChunk);
  refresh_copy_kernel<<<grid, 256, 0, s>>>(N, V, budget, t, rlist, last_step, z0, z1, lse0,
                                           lse1);
  return hipGetLastError();
}

}  // namespace dlm

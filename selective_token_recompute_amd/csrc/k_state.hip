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
// semi-autoregressive blocks.
#include "common.h"
#include "internal.h"

namespace dlm {

// ---------------------------------------------------------------------------
__global__ void init_state_kernel(int B, int N, int P, int mask_id, const int32_t* prompts,
                                  int32_t* tokens, uint64_t* bits, int32_t* counters,
                                  int32_t* has_prev, int32_t* ctl) {
  const int W = (N + 63) >> 6;
  const size_t total = (size_t)B * N;
  for (size_t f = blockIdx.x * (size_t)blockDim.x + threadIdx.x; f < total;
       f += (size_t)gridDim.x * blockDim.x) {
    const int b = (int)(f / N), i = (int)(f - (size_t)b * N);
    tokens[f] = i < P ? prompts[(size_t)b * P + i] : mask_id;
    counters[f] = 0;
    has_prev[f] = 0;
    if (f < (size_t)B * W) bits[f] = 0ull;
    if (f < 4) ctl[f] = 0;
  }
}

hipError_t launch_init_state(int B, int N, int P, int mask_id, const int32_t* prompts,
                             int32_t* tokens, uint64_t* bits, int32_t* counters,
                             int32_t* has_prev, int32_t* ctl, hipStream_t s) {
  const size_t total = (size_t)B * N;
  const int grid = (int)std::min<size_t>((total + 255) / 256, 4096);
  init_state_kernel<<<grid, 256, 0, s>>>(B, N, P, mask_id, prompts, tokens, bits, counters,
                                         has_prev, ctl);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Compaction: one workgroup of 1024 threads scans the B*N positions in
// (seq, pos) order, 1024 at a time.  Each wave ballots its 64 "active"
// predicates; the lane's rank is the popcount of the ballot below it, the
// wave's base is the prefix over the wave counts of this chunk.
constexpr int kCompactThreads = 1024;

__global__ __launch_bounds__(kCompactThreads) void compact_kernel(
    const uint64_t* __restrict__ bits, int B, int N, int32_t* __restrict__ row_seq,
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
      act = !((bits[(size_t)b * W + (i >> 6)] >> (i & 63)) & 1ull);
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
      uint64_t v = ~bits[(size_t)b * W + wd];
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

hipError_t launch_compact(const uint64_t* bits, int B, int N, int32_t* row_seq, int32_t* row_pos,
                          int32_t* m_b, int32_t* row_start, int32_t* ctl, hipStream_t s) {
  compact_kernel<<<1, kCompactThreads, 0, s>>>(bits, B, N, row_seq, row_pos, m_b, row_start, ctl);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Commit + lock, one workgroup per sequence.
// Candidates (masked rows of the current block) are gathered in LDS; each
// candidate's rank is the number of candidates strictly ahead of it in the
// order (conf descending, position ascending); ranks below k commit.
constexpr int kLockThreads = 1024;

__global__ __launch_bounds__(kLockThreads) void commit_lock_kernel(LockArgs a) {
  extern __shared__ unsigned char smem[];
  const int cap = a.blk_hi - a.blk_lo;
  float* cconf = reinterpret_cast<float*>(smem);
  int* cpos = reinterpret_cast<int*>(cconf + (cap > 0 ? cap : 1));
  int* crow = cpos + (cap > 0 ? cap : 1);
  __shared__ int ncand;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int N = a.N, W = (N + 63) >> 6;
  const int r0 = a.row_start[b], r1 = a.row_start[b + 1];
  int32_t* tok = a.tokens + (size_t)b * N;

  if (a.do_commit && a.k > 0 && cap > 0) {
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
  const int cap = std::max(1, a.blk_hi - a.blk_lo);
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

// Posterior statistics of the active rows over the vocabulary.
//
// SureLock page ("Stopping Computation for Converged Tokens in Masked
// Diffusion-LM Decoding"), §2 Methodology, locking condition: the primary
// criterion is the step-wise divergence D = KL(p_t || p_{t-1}) between the
// current and previous posterior of a position, with an optional gate that
// the token is also highly confident.  Confidence here is the max
// probability; the argmax is the token a commit would write.
//
// One pass reads the current logits z and, where a previous posterior
// exists, the previous logits z' (the engine keeps each position's logits of
// the last step, double-buffered by step parity, plus that step's
// log-normaliser lse') and folds them into the partial statistics of
// vocab_part.h.  Rows are split over several workgroups (chunks of the
// vocabulary); a second pass merges the chunk partials per row.  The LM-head
// GEMM can instead produce the partials in its epilogue (one per row and
// column tile); vocab_merge_parts_kernel merges those.
#include "common.h"
#include "internal.h"
#include "vocab_part.h"

namespace dlm {

typedef VocabPart VPart;

constexpr int kVThreads = 256;

template <int KLDIR>
__global__ __launch_bounds__(kVThreads) void vocab_partial_kernel(
    int V, int mask_id, int N, int chunk, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_pos, const float* __restrict__ z_cur,
    const float* __restrict__ z_prev, const float* __restrict__ lse_prev,
    const int32_t* __restrict__ has_prev, VPart* __restrict__ part) {
  __shared__ VPart red[kVThreads / 64];
  const int r = blockIdx.y, c = blockIdx.x, nchunks = gridDim.x;
  const size_t slot = (size_t)row_seq[r] * N + row_pos[r];
  const float* z = z_cur + slot * V;
  const float* zp = z_prev + slot * V;
  const bool hp = has_prev[slot] != 0;
  const float lsep = hp ? lse_prev[slot] : 0.f;
  const int v0 = c * chunk, v1 = min(V, v0 + chunk);

  VPart acc = vpart_empty();
  auto visit = [&](int v, float zv, float zpv) {
    vpart_visit<KLDIR>(acc, v, zv, zpv, hp, lsep, mask_id);
  };
  // each thread visits its elements in increasing v, so a strict '>' keeps
  // the smallest index among equal maxima
  const bool vec = ((V & 3) == 0) && ((v0 & 3) == 0);
  if (vec) {
    const int n4 = (v1 - v0) >> 2;
    const float4* z4 = (const float4*)(z + v0);
    const float4* zp4 = (const float4*)(zp + v0);
    // U float4 of z (and of z') loaded before any is folded, so that the
    // loads of a thread are in flight together
    constexpr int U = 4;
    const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
    int i = threadIdx.x;
    for (; i + (U - 1) * kVThreads < n4; i += U * kVThreads) {
      float4 a[U], p[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        a[u] = z4[i + u * kVThreads];
        p[u] = hp ? zp4[i + u * kVThreads] : zero;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + 4 * (i + u * kVThreads);
        visit(v, a[u].x, p[u].x);
        visit(v + 1, a[u].y, p[u].y);
        visit(v + 2, a[u].z, p[u].z);
        visit(v + 3, a[u].w, p[u].w);
      }
    }
    for (; i < n4; i += kVThreads) {
      const float4 a = z4[i];
      const float4 p = hp ? zp4[i] : zero;
      const int v = v0 + 4 * i;
      visit(v, a.x, p.x);
      visit(v + 1, a.y, p.y);
      visit(v + 2, a.z, p.z);
      visit(v + 3, a.w, p.w);
    }
    for (int v = v0 + 4 * n4 + threadIdx.x; v < v1; v += kVThreads)
      visit(v, z[v], hp ? zp[v] : 0.f);
  } else {
    for (int v = v0 + threadIdx.x; v < v1; v += kVThreads) visit(v, z[v], hp ? zp[v] : 0.f);
  }
  // wave merge then cross-wave merge
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc = vmerge(acc, vpart_shfl_xor(acc, o));
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    VPart t = red[0];
    for (int i = 1; i < kVThreads / 64; ++i) t = vmerge(t, red[i]);
    part[(size_t)r * nchunks + c] = t;
  }
}

// Finishes row r from its merged partial: statistics, lse recorded for the
// next step, has_prev set, non-finite lse latched.
__device__ __forceinline__ void finish_row(int r, const VPart& t, int N, int kl_dir,
                                           const int32_t* __restrict__ row_seq,
                                           const int32_t* __restrict__ row_pos,
                                           const float* __restrict__ lse_prev,
                                           int32_t* __restrict__ has_prev,
                                           float* __restrict__ lse_cur,
                                           int32_t* __restrict__ argmax, float* __restrict__ conf,
                                           float* __restrict__ kl, int32_t* __restrict__ has_kl,
                                           float* __restrict__ lse_row, int32_t* __restrict__ err) {
  const size_t slot = (size_t)row_seq[r] * N + row_pos[r];
  const float lse = t.m + logf(t.s0);
  const bool hp = has_prev[slot] != 0;
  argmax[r] = t.am;
  conf[r] = 1.f / t.s0;
  lse_row[r] = lse;
  if (hp) {
    const float dl = lse - lse_prev[slot];
    kl[r] = kl_dir == 0 ? (t.s1 / t.s0 - dl) : (t.t1 + dl);
    has_kl[r] = 1;
  } else {
    kl[r] = __int_as_float(0x7fc00000);
    has_kl[r] = 0;
  }
  lse_cur[slot] = lse;
  has_prev[slot] = 1;
  if (!isfinite(lse)) atomicExch(err, 1);
}

// One wave per row over many partials [M][nparts]: lane l merges partials
// l, l+64, ... in order, then the lanes merge by xor shuffles.
__global__ __launch_bounds__(256) void vocab_merge_parts_kernel(
    int M, int nparts, int N, int kl_dir, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_pos, const float* __restrict__ lse_prev,
    int32_t* __restrict__ has_prev, float* __restrict__ lse_cur, const VPart* __restrict__ part,
    int32_t* __restrict__ argmax, float* __restrict__ conf, float* __restrict__ kl,
    int32_t* __restrict__ has_kl, float* __restrict__ lse_row, int32_t* __restrict__ err) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= M) return;  // wave-uniform
  VPart t = vpart_empty();
  const VPart* p = part + (size_t)r * nparts;
  // four partials loaded before any is merged, so that a lane's loads are in
  // flight together (the merges form one dependent chain)
  constexpr int U = 4;
  int c = lane;
  for (; c + (U - 1) * 64 < nparts; c += U * 64) {
    VPart q[U];
#pragma unroll
    for (int u = 0; u < U; ++u) q[u] = p[c + u * 64];
#pragma unroll
    for (int u = 0; u < U; ++u) t = vmerge(t, q[u]);
  }
  for (; c < nparts; c += 64) t = vmerge(t, p[c]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) t = vmerge(t, vpart_shfl_xor(t, o));
  if (lane == 0)
    finish_row(r, t, N, kl_dir, row_seq, row_pos, lse_prev, has_prev, lse_cur, argmax, conf, kl,
               has_kl, lse_row, err);
}

namespace {
struct VPlan { int chunks, chunk; };
VPlan make_vplan(int M, int V) {
  // aim for ~2048 workgroups, chunks of >= 1024 elements, <= 256 chunks
  int chunks = std::max(1, (2048 + M - 1) / std::max(M, 1));
  chunks = std::min(chunks, std::max(1, V / 1024));
  chunks = std::min(chunks, 256);
  int chunk = (V + chunks - 1) / chunks;
  chunk = (chunk + 3) & ~3;
  chunks = (V + chunk - 1) / chunk;
  return VPlan{chunks, chunk};
}
}  // namespace

size_t vocab_ws_bytes(int M, int V) {
  if (M <= 0) return 0;
  const VPlan p = make_vplan(M, V);
  return (size_t)M * p.chunks * sizeof(VPart);
}

hipError_t launch_vocab_stats(int M, int V, int mask_id, int kl_dir, int N,
                              const int32_t* row_seq, const int32_t* row_pos,
                              const float* z_cur, const float* z_prev, const float* lse_prev,
                              int32_t* has_prev, float* lse_cur, int32_t* argmax, float* conf,
                              float* kl, int32_t* has_kl, float* lse_row, int32_t* err,
                              void* ws, size_t ws_bytes, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const VPlan p = make_vplan(M, V);
  if ((size_t)M * p.chunks * sizeof(VPart) > ws_bytes) return hipErrorInvalidValue;
  VPart* part = (VPart*)ws;
  dim3 grid(p.chunks, M);
  if (kl_dir == 0)
    vocab_partial_kernel<0><<<grid, kVThreads, 0, s>>>(V, mask_id, N, p.chunk, row_seq, row_pos,
                                                       z_cur, z_prev, lse_prev, has_prev, part);
  else
    vocab_partial_kernel<1><<<grid, kVThreads, 0, s>>>(V, mask_id, N, p.chunk, row_seq, row_pos,
                                                       z_cur, z_prev, lse_prev, has_prev, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // one wave per row: the chunk partials of a row are loaded in parallel
  // (a thread per row walking them in order waits one load latency per chunk)
  vocab_merge_parts_kernel<<<(M + 3) / 4, 256, 0, s>>>(M, p.chunks, N, kl_dir, row_seq, row_pos,
                                                      lse_prev, has_prev, lse_cur, part, argmax,
                                                      conf, kl, has_kl, lse_row, err);
  return hipGetLastError();
}

hipError_t launch_vocab_merge_parts(int M, int nparts, int N, int kl_dir, const int32_t* row_seq,
                                    const int32_t* row_pos, const float* lse_prev,
                                    int32_t* has_prev, float* lse_cur, const void* parts,
                                    int32_t* argmax, float* conf, float* kl, int32_t* has_kl,
                                    float* lse_row, int32_t* err, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  vocab_merge_parts_kernel<<<(M + 3) / 4, 256, 0, s>>>(M, nparts, N, kl_dir, row_seq, row_pos,
                                                      lse_prev, has_prev, lse_cur,
                                                      (const VPart*)parts, argmax, conf, kl,
                                                      has_kl, lse_row, err);
  return hipGetLastError();
}

}  // namespace dlm

// Row-wise kernels of the active-row forward pass: embedding gather + RMSNorm,
// RMSNorm, the rotary table, and rotary embedding + K/V cache scatter.
//
// SureLock page ("Stopping Computation for Converged Tokens in Masked
// Diffusion-LM Decoding"), §2 Methodology, core mechanism: locked positions
// get no computation; the K and V of every position are kept in a cache, and
// fresh Q/K/V are produced only for the active subset, overwriting that
// subset's cache entries.  The model details (pre-RMSNorm, half-split rotary
// embedding) are not on the pages; they follow the LLaDA-style architecture
// the experiments use.
#include "common.h"
#include "internal.h"

namespace dlm {

constexpr int kNormThreads = 256;

// One workgroup per active row.  h (float) is the residual stream; y is the
// normalised row in the storage type (the next GEMM's A operand).
template <typename T, bool kGather>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(
    int d, int N, float eps, int mask_id, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_pos,
    const T* __restrict__ emb, const T* __restrict__ g, float* __restrict__ h,
    T* __restrict__ y, int32_t* __restrict__ row_real) {
  __shared__ float red[16];
  const int r = blockIdx.x, tid = threadIdx.x;
  float* hr = h + (size_t)r * d;
  const float* src = hr;
  if (kGather) {
    const int tok = tokens[(size_t)row_seq[r] * N + row_pos[r]];
    if (tid == 0) row_real[r] = tok != mask_id;
    const T* e = emb + (size_t)tok * d;
    for (int c = tid; c < d; c += kNormThreads) hr[c] = ld(e, c);
    __syncthreads();  // each thread re-reads only its own columns, but keep it simple
  }
  float ss = 0.f;
  for (int c = tid; c < d; c += kNormThreads) {
    const float v = src[c];
    ss += v * v;
  }
  ss = block_sum(ss, red);
  const float inv = rsqrtf(ss / (float)d + eps);
  T* yr = y + (size_t)r * d;
  for (int c = tid; c < d; c += kNormThreads) st(yr, c, src[c] * inv * ld(g, c));
}

hipError_t launch_embed_rmsnorm(int dtype, int M, int d, int N, float eps, int mask_id,
                                const int32_t* tokens, const int32_t* row_seq,
                                const int32_t* row_pos, const void* emb, const void* g, float* h,
                                void* y, int32_t* row_real, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (dtype == kBF16)
    rmsnorm_kernel<bf16_t, true><<<M, kNormThreads, 0, s>>>(
        d, N, eps, mask_id, tokens, row_seq, row_pos, (const bf16_t*)emb, (const bf16_t*)g, h,
        (bf16_t*)y, row_real);
  else
    rmsnorm_kernel<float, true><<<M, kNormThreads, 0, s>>>(
        d, N, eps, mask_id, tokens, row_seq, row_pos, (const float*)emb, (const float*)g, h,
        (float*)y, row_real);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int dtype, int M, int d, float eps, const float* x, const void* g,
                          void* y, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (dtype == kBF16)
    rmsnorm_kernel<bf16_t, false><<<M, kNormThreads, 0, s>>>(
        d, 0, eps, 0, nullptr, nullptr, nullptr, nullptr, (const bf16_t*)g, (float*)x,
        (bf16_t*)y, nullptr);
  else
    rmsnorm_kernel<float, false><<<M, kNormThreads, 0, s>>>(
        d, 0, eps, 0, nullptr, nullptr, nullptr, nullptr, (const float*)g, (float*)x, (float*)y,
        nullptr);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Rotary table: (cos, sin) of pos * base^(-2j/hd), evaluated in double.
__global__ void rope_table_kernel(int N, int hd, double base, float* table) {
  const int half = hd / 2;
  const size_t total = (size_t)N * half;
  for (size_t f = blockIdx.x * (size_t)blockDim.x + threadIdx.x; f < total;
       f += (size_t)gridDim.x * blockDim.x) {
    const int pos = (int)(f / half), j = (int)(f % half);
    const double ang = (double)pos * pow(base, -2.0 * j / (double)hd);
    table[2 * f] = (float)cos(ang);
    table[2 * f + 1] = (float)sin(ang);
  }
}

hipError_t launch_rope_table(int N, int hd, float base, float* table, hipStream_t s) {
  const size_t total = (size_t)N * (hd / 2);
  const int grid = (int)std::min<size_t>((total + 255) / 256, 4096);
  rope_table_kernel<<<grid, 256, 0, s>>>(N, hd, (double)base, table);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Rotary embedding + scatter.  One workgroup per active row; work items are
// the (head, pair) rotations of q and k plus the v copies.
template <typename T>
__global__ __launch_bounds__(256) void rope_scatter_kernel(
    int nq, int nkv, int hd, int N, const float* __restrict__ qkv,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_pos,
    const float* __restrict__ table, T* __restrict__ q, T* __restrict__ kc, T* __restrict__ vc) {
  const int r = blockIdx.x;
  const int half = hd / 2;
  const int width = (nq + 2 * nkv) * hd;
  const float* x = qkv + (size_t)r * width;
  const int b = row_seq[r], pos = row_pos[r];
  const float* tb = table ? table + (size_t)pos * hd : nullptr;
  const int n_rot = (nq + nkv) * half;
  const int n_all = n_rot + nkv * hd;
  for (int it = threadIdx.x; it < n_all; it += blockDim.x) {
    if (it < n_rot) {
      const int head = it / half, j = it - head * half;
      const float* u = x + (size_t)head * hd;
      float a0 = u[j], a1 = u[j + half];
      if (tb) {
        const float c = tb[2 * j], sn = tb[2 * j + 1];
        const float r0 = a0 * c - a1 * sn, r1 = a0 * sn + a1 * c;
        a0 = r0;
        a1 = r1;
      }
      if (head < nq) {
        T* qo = q + (size_t)r * nq * hd + (size_t)head * hd;
        st(qo, j, a0);
        st(qo, j + half, a1);
      } else {
        const int g = head - nq;
        T* ko = kc + (((size_t)b * nkv + g) * N + pos) * hd;
        st(ko, j, a0);
        st(ko, j + half, a1);
      }
    } else {
      const int v = it - n_rot, g = v / hd, c = v - g * hd;
      T* vo = vc + (((size_t)b * nkv + g) * N + pos) * hd;
      st(vo, c, x[(size_t)(nq + nkv) * hd + v]);
    }
  }
}

hipError_t launch_rope_scatter(int dtype, int M, int nq, int nkv, int hd, int N, const float* qkv,
                               const int32_t* row_seq, const int32_t* row_pos,
                               const float* table, void* q, void* kc, void* vc, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (dtype == kBF16)
    rope_scatter_kernel<bf16_t><<<M, 256, 0, s>>>(nq, nkv, hd, N, qkv, row_seq, row_pos, table,
                                                  (bf16_t*)q, (bf16_t*)kc, (bf16_t*)vc);
  else
    rope_scatter_kernel<float><<<M, 256, 0, s>>>(nq, nkv, hd, N, qkv, row_seq, row_pos, table,
                                                 (float*)q, (float*)kc, (float*)vc);
  return hipGetLastError();
}

}  // namespace dlm

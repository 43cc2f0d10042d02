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
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace dlm {

constexpr int kNormThreads = 256;

// One workgroup per active row.  h (float) is the residual stream; y is the
// normalised row in the storage type (the next GEMM's A operand).  With
// kGather the row is first gathered from the embedding; with splits > 0 the
// row first absorbs the split-K partial sums of the GEMM that produced its
// residual update (h += sum_s partial[s][row], in split order).
// Vector path: d % 4 == 0 and d <= 4 * 4 * kNormThreads, the row lives in
// registers (one read of h, one write of h and y).
template <typename T>
__device__ __forceinline__ void st4(T* p, size_t i, float4 v);
template <>
__device__ __forceinline__ void st4<float>(float* p, size_t i, float4 v) {
  *(float4*)(p + i) = v;
}
template <>
__device__ __forceinline__ void st4<bf16_t>(bf16_t* p, size_t i, float4 v) {
  ushort4 w;
  w.x = f2bf(v.x);
  w.y = f2bf(v.y);
  w.z = f2bf(v.z);
  w.w = f2bf(v.w);
  *(ushort4*)(p + i) = w;
}
template <typename T>
__device__ __forceinline__ float4 ld4(const T* p, size_t i);
template <>
__device__ __forceinline__ float4 ld4<float>(const float* p, size_t i) {
  return *(const float4*)(p + i);
}
template <>
__device__ __forceinline__ float4 ld4<bf16_t>(const bf16_t* p, size_t i) {
  const ushort4 w = *(const ushort4*)(p + i);
  return make_float4(bf2f(w.x), bf2f(w.y), bf2f(w.z), bf2f(w.w));
}

template <typename T, bool kGather, int SP>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_vec_kernel(
    int M, int d, int N, float eps, int mask_id, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_pos,
    const T* __restrict__ emb, const T* __restrict__ g, float* __restrict__ h,
    const float* __restrict__ partial, int splits, T* __restrict__ y,
    int32_t* __restrict__ row_real) {
  // SP: compile-time bound on the split-K partials (splits <= SP), so that
  // every load of a row is independent and in flight at once
  constexpr int MAXV = 4;
  __shared__ float red[16];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int d4 = d >> 2;
  float* hr = h + (size_t)r * d;
  const T* src = nullptr;
  if (kGather) {
    const int tok = tokens[(size_t)row_seq[r] * N + row_pos[r]];
    if (tid == 0) row_real[r] = tok != mask_id;
    src = emb + (size_t)tok * d;
  }
  float4 v[MAXV], gg[MAXV];
  float4 pp[SP > 0 ? SP : 1][MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c4 = tid + i * kNormThreads;
    v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c4 < d4) {
      // the gain is read with the row, not after the reduction (one memory
      // round trip less on the row's critical path)
      gg[i] = ld4(g, (size_t)c4 * 4);
      if (kGather) {
        v[i] = ld4(src, (size_t)c4 * 4);
      } else {
        v[i] = *(const float4*)(hr + (size_t)c4 * 4);
#pragma unroll
        for (int sp = 0; sp < SP; ++sp)
          pp[sp][i] = sp < splits ? *(const float4*)(partial + ((size_t)sp * M + r) * d +
                                                     (size_t)c4 * 4)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c4 = tid + i * kNormThreads;
    if (c4 < d4) {
      if (!kGather) {
        // partials summed in split order, as the split-K reduction does
#pragma unroll
        for (int sp = 0; sp < SP; ++sp) {
          v[i].x += pp[sp][i].x;
          v[i].y += pp[sp][i].y;
          v[i].z += pp[sp][i].z;
          v[i].w += pp[sp][i].w;
        }
      }
      if (kGather || splits > 0) *(float4*)(hr + (size_t)c4 * 4) = v[i];
      ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
    }
  }
  ss = block_sum(ss, red);
  const float inv = rsqrtf(ss / (float)d + eps);
  T* yr = y + (size_t)r * d;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c4 = tid + i * kNormThreads;
    if (c4 < d4) {
      st4(yr, (size_t)c4 * 4,
          make_float4(v[i].x * inv * gg[i].x, v[i].y * inv * gg[i].y, v[i].z * inv * gg[i].z,
                      v[i].w * inv * gg[i].w));
    }
  }
}

// Generic path (any d).
template <typename T, bool kGather>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(
    int M, int d, int N, float eps, int mask_id, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_pos,
    const T* __restrict__ emb, const T* __restrict__ g, float* __restrict__ h,
    const float* __restrict__ partial, int splits, T* __restrict__ y,
    int32_t* __restrict__ row_real) {
  __shared__ float red[16];
  const int r = blockIdx.x, tid = threadIdx.x;
  float* hr = h + (size_t)r * d;
  if (kGather) {
    const int tok = tokens[(size_t)row_seq[r] * N + row_pos[r]];
    if (tid == 0) row_real[r] = tok != mask_id;
    const T* e = emb + (size_t)tok * d;
    for (int c = tid; c < d; c += kNormThreads) hr[c] = ld(e, c);
  } else if (splits > 0) {
    for (int c = tid; c < d; c += kNormThreads) {
      float v = hr[c];
      for (int sp = 0; sp < splits; ++sp) v += partial[((size_t)sp * M + r) * d + c];
      hr[c] = v;
    }
  }
  float ss = 0.f;
  for (int c = tid; c < d; c += kNormThreads) {
    const float v = hr[c];
    ss += v * v;
  }
  ss = block_sum(ss, red);
  const float inv = rsqrtf(ss / (float)d + eps);
  T* yr = y + (size_t)r * d;
  for (int c = tid; c < d; c += kNormThreads) st(yr, c, hr[c] * inv * ld(g, c));
}

template <typename T, bool kGather>
hipError_t run_norm(int M, int d, int N, float eps, int mask_id, const int32_t* tokens,
                    const int32_t* row_seq, const int32_t* row_pos, const void* emb,
                    const void* g, float* h, const float* partial, int splits, void* y,
                    int32_t* row_real, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (d % 4 == 0 && d <= 16 * kNormThreads && splits <= 8) {
    auto go = [&](auto sp_tag) {
      constexpr int SP = decltype(sp_tag)::value;
      rmsnorm_vec_kernel<T, kGather, SP><<<M, kNormThreads, 0, s>>>(
          M, d, N, eps, mask_id, tokens, row_seq, row_pos, (const T*)emb, (const T*)g, h,
          partial, splits, (T*)y, row_real);
    };
    if (kGather || splits == 0) go(std::integral_constant<int, 0>{});
    else if (splits == 1) go(std::integral_constant<int, 1>{});
    else if (splits == 2) go(std::integral_constant<int, 2>{});
    else if (splits <= 4) go(std::integral_constant<int, 4>{});
    else go(std::integral_constant<int, 8>{});
  } else
    rmsnorm_kernel<T, kGather><<<M, kNormThreads, 0, s>>>(
        M, d, N, eps, mask_id, tokens, row_seq, row_pos, (const T*)emb, (const T*)g, h, partial,
        splits, (T*)y, row_real);
  return hipGetLastError();
}

hipError_t launch_embed_rmsnorm(int dtype, int M, int d, int N, float eps, int mask_id,
                                const int32_t* tokens, const int32_t* row_seq,
                                const int32_t* row_pos, const void* emb, const void* g, float* h,
                                void* y, int32_t* row_real, hipStream_t s) {
  if (dtype == kBF16)
    return run_norm<bf16_t, true>(M, d, N, eps, mask_id, tokens, row_seq, row_pos, emb, g, h,
                                  nullptr, 0, y, row_real, s);
  return run_norm<float, true>(M, d, N, eps, mask_id, tokens, row_seq, row_pos, emb, g, h,
                               nullptr, 0, y, row_real, s);
}

hipError_t launch_rmsnorm(int dtype, int M, int d, float eps, const float* x, const void* g,
                          void* y, hipStream_t s) {
  return launch_rmsnorm_resid(dtype, M, d, eps, (float*)x, nullptr, 0, g, y, s);
}

hipError_t launch_rmsnorm_resid(int dtype, int M, int d, float eps, float* h,
                                const float* partial, int splits, const void* g, void* y,
                                hipStream_t s) {
  if (dtype == kBF16)
    return run_norm<bf16_t, false>(M, d, 0, eps, 0, nullptr, nullptr, nullptr, nullptr, g, h,
                                   partial, splits, y, nullptr, s);
  return run_norm<float, false>(M, d, 0, eps, 0, nullptr, nullptr, nullptr, nullptr, g, h,
                                partial, splits, y, nullptr, s);
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
// Rotary embedding + scatter.  K is cached [seq][kv head][N][hd], V
// transposed [seq][kv head][hd][N] (the layout attention streams).
// With splits > 0 the QKV values are the sum of the GEMM's split-K partials
// [splits][M][width] (split order).
__device__ __forceinline__ float qkv_val(const float* qkv, const float* partial, int splits,
                                         int M, int width, int r, int c) {
  if (splits == 0) return qkv[(size_t)r * width + c];
  float v = 0.f;
  for (int sp = 0; sp < splits; ++sp) v += partial[((size_t)sp * M + r) * width + c];
  return v;
}

// q and k heads: workgroup (row, 4 heads), one wave per head; lane j rotates
// the pairs (j, j + hd/2).
template <typename T>
__global__ __launch_bounds__(256) void rope_qk_kernel(
    int M, int nq, int nkv, int hd, int N, const float* __restrict__ qkv,
    const float* __restrict__ partial, int splits, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_pos, const float* __restrict__ table, T* __restrict__ q,
    T* __restrict__ kc) {
  const int r = blockIdx.x;
  const int head = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (head >= nq + nkv) return;
  const int half = hd >> 1;
  const int width = (nq + 2 * nkv) * hd;
  const int b = row_seq[r], pos = row_pos[r];
  T* dst = head < nq ? q + (size_t)r * nq * hd + (size_t)head * hd
                     : kc + (((size_t)b * nkv + (head - nq)) * N + pos) * hd;
  for (int j = lane; j < half; j += 64) {
    float a0 = qkv_val(qkv, partial, splits, M, width, r, head * hd + j);
    float a1 = qkv_val(qkv, partial, splits, M, width, r, head * hd + j + half);
    if (table) {
      const float c = table[((size_t)pos * half + j) * 2];
      const float sn = table[((size_t)pos * half + j) * 2 + 1];
      const float r0 = a0 * c - a1 * sn, r1 = a0 * sn + a1 * c;
      a0 = r0;
      a1 = r1;
    }
    st(dst, j, a0);
    st(dst, j + half, a1);
  }
}

// v heads: workgroup (64 rows, one kv head); the 64 x hd block is transposed
// through LDS so that consecutive lanes write consecutive positions of a V^T
// row.
constexpr int kVRows = 64;
template <typename T>
__global__ __launch_bounds__(256) void scatter_vt_kernel(
    int M, int nq, int nkv, int hd, int N, const float* __restrict__ qkv,
    const float* __restrict__ partial, int splits, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_pos, T* __restrict__ vc) {
  extern __shared__ float tile[];  // [hd][kVRows + 1]
  const int r0 = blockIdx.x * kVRows, g = blockIdx.y;
  const int rows = min(kVRows, M - r0);
  const int width = (nq + 2 * nkv) * hd;
  const int col0 = (nq + nkv + g) * hd;
  for (int e = threadIdx.x; e < rows * hd; e += blockDim.x) {
    const int rr = e / hd, c = e % hd;
    tile[c * (kVRows + 1) + rr] = qkv_val(qkv, partial, splits, M, width, r0 + rr, col0 + c);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < rows * hd; e += blockDim.x) {
    const int c = e / rows, rr = e % rows;
    const int r = r0 + rr;
    T* vt = vc + (((size_t)row_seq[r] * nkv + g) * hd + c) * N + row_pos[r];
    st(vt, 0, tile[c * (kVRows + 1) + rr]);
  }
}

hipError_t launch_rope_scatter(int dtype, int M, int nq, int nkv, int hd, int N, const float* qkv,
                               const int32_t* row_seq, const int32_t* row_pos,
                               const float* table, void* q, void* kc, void* vc, hipStream_t s) {
  return launch_rope_scatter_split(dtype, M, nq, nkv, hd, N, qkv, nullptr, 0, row_seq, row_pos,
                                   table, q, kc, vc, s);
}

template <typename T>
hipError_t run_rope_scatter(int M, int nq, int nkv, int hd, int N, const float* qkv,
                            const float* partial, int splits, const int32_t* row_seq,
                            const int32_t* row_pos, const float* table, void* q, void* kc,
                            void* vc, hipStream_t s) {
  dim3 g1(M, (nq + nkv + 3) / 4);
  rope_qk_kernel<T><<<g1, 256, 0, s>>>(M, nq, nkv, hd, N, qkv, partial, splits, row_seq,
                                       row_pos, table, (T*)q, (T*)kc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2((M + kVRows - 1) / kVRows, nkv);
  const size_t lds = (size_t)hd * (kVRows + 1) * sizeof(float);
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&scatter_vt_kernel<T>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 256 * (kVRows + 1) * 4);
    attr = true;
  }
  scatter_vt_kernel<T><<<g2, 256, lds, s>>>(M, nq, nkv, hd, N, qkv, partial, splits, row_seq,
                                            row_pos, (T*)vc);
  return hipGetLastError();
}

hipError_t launch_rope_scatter_split(int dtype, int M, int nq, int nkv, int hd, int N,
                                     const float* qkv, const float* partial, int splits,
                                     const int32_t* row_seq, const int32_t* row_pos,
                                     const float* table, void* q, void* kc, void* vc,
                                     hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (dtype == kBF16)
    return run_rope_scatter<bf16_t>(M, nq, nkv, hd, N, qkv, partial, splits, row_seq, row_pos,
                                    table, q, kc, vc, s);
  return run_rope_scatter<float>(M, nq, nkv, hd, N, qkv, partial, splits, row_seq, row_pos,
                                 table, q, kc, vc, s);
}

}  // namespace dlm

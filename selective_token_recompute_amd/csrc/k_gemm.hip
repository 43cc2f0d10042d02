// Active-row GEMMs: Y = A W^T on the M compacted rows, with fused epilogues.
//
// SureLock page ("Stopping Computation for Converged Tokens in Masked
// Diffusion-LM Decoding"), §2 Methodology: locked positions skip the query
// projection and the FFN; only the active subset gets fresh Q/K/V; FFN cost
// falls to O(M_t d^2) (§2 algorithmic complexity).  M shrinks from step to
// step, so the launch plan depends on M: large M is MFMA-bound (bf16
// 16x16x32 MFMA, LDS double buffering), small M is bound by streaming the
// weights once (narrow row tile, split-K across workgroups, deterministic
// two-pass reduction).
//
// Epilogues: plain float store (QKV, before the rotary step), residual add
// into the float residual stream (out-projection, down-projection), SwiGLU
// over a gate/up pair of weight matrices (silu(A Wg^T) * (A Wu^T), stored in
// the storage type), and logits scattered to each row's (seq, pos) slot with
// the mask token's column forced to -inf.
#include "common.h"
#include "internal.h"

namespace dlm {

// ---------------------------------------------------------------------------
// Epilogue of one output element (row, col) given the accumulator(s).
struct EpiParams {
  void* C;
  int M, N;  // N: output columns (features for SwiGLU)
  const int32_t* row_seq;
  const int32_t* row_pos;
  int seq_len, mask_id;
};

template <int EPI, typename T>
__device__ __forceinline__ void epi_store(const EpiParams& p, int row, int col, float v,
                                          float v_up) {
  if (EPI == kEpiStoreF32) {
    ((float*)p.C)[(size_t)row * p.N + col] = v;
  } else if (EPI == kEpiResidAdd) {
    float* c = (float*)p.C + (size_t)row * p.N + col;
    *c += v;
  } else if (EPI == kEpiSwiglu) {
    st((T*)p.C, (size_t)row * p.N + col, silu(v) * v_up);
  } else {  // logits
    const size_t slot = (size_t)p.row_seq[row] * p.seq_len + p.row_pos[row];
    ((float*)p.C)[slot * p.N + col] = (col == p.mask_id) ? -INFINITY : v;
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel.
//   Tile BM x BN x BK, WAVES_M x WAVES_N waves, each wave (BM/WAVES_M) x
//   (BN/WAVES_N) made of 16x16 MFMA tiles.  For SwiGLU (DUAL) the BN tile
//   rows are [BN/2 gate rows | BN/2 up rows] of the same BN/2 features, and
//   each wave owns matching gate/up column tiles so the epilogue pairs them
//   in registers.
//   v_mfma_f32_16x16x32_bf16: lane l supplies A[row l%16][k-group l/16] and
//   B[k-group l/16][col l%16] (8 consecutive k each; the same k mapping on
//   both sides) and receives C[4*(l/16)+i][l%16], i = 0..3.
//   Split-K (gridDim.z > 1) writes fp32 partials [split][M][NC] instead of
//   the epilogue, NC = N (2N for DUAL: gate at f, up at N+f).
template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int EPI, bool SPLIT>
__global__ __launch_bounds__(64 * WAVES_M* WAVES_N) void gemm_bf16_mfma_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ W, const bf16_t* __restrict__ W2,
    EpiParams ep, int K, int k_per_split, int tiles_m, int tiles_n, float* __restrict__ partial) {
  constexpr bool DUAL = EPI == kEpiSwiglu;
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int LDSK = BK + 8;  // padded row pitch (elements)
  constexpr int KC = BK / 8;    // 16-byte chunks per tile row
  constexpr int A_CH = BM * KC, B_CH = BN * KC;
  constexpr int A_PT = (A_CH + NT - 1) / NT, B_PT = (B_CH + NT - 1) / NT;
  static_assert(!DUAL || (TN % 2 == 0), "dual tiles need an even number of column tiles");
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * LDSK];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * LDSK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int M = ep.M, N = ep.N;

  // XCD-aware tile order: workgroup i runs on XCD i % 8; give consecutive
  // workgroups of one XCD the row tiles of one column tile.
  const int ntiles = tiles_m * tiles_n;
  int lin = blockIdx.x;
  if ((ntiles & 7) == 0) lin = (lin & 7) * (ntiles >> 3) + (lin >> 3);
  const int mt = lin % tiles_m, nt = lin / tiles_m;
  const int m0 = mt * BM;
  const int n0 = DUAL ? nt * (BN / 2) : nt * BN;  // first output feature / column

  const int kbeg = blockIdx.y * k_per_split;
  const int kend = min(K, kbeg + k_per_split);
  const int KT = kend > kbeg ? (kend - kbeg) / BK : 0;

  // global source row pointers of this thread's chunks
  const bf16_t* a_src[A_PT];
  bool a_ok[A_PT];
  int a_dst[A_PT];
#pragma unroll
  for (int i = 0; i < A_PT; ++i) {
    const int c = tid + i * NT;
    const int row = c / KC, kc = (c % KC) * 8;
    a_ok[i] = c < A_CH && (m0 + row) < M;
    a_src[i] = A + (size_t)(a_ok[i] ? m0 + row : 0) * K + kbeg + kc;
    a_dst[i] = row * LDSK + kc;
  }
  const bf16_t* b_src[B_PT];
  bool b_ok[B_PT];
  int b_dst[B_PT];
#pragma unroll
  for (int i = 0; i < B_PT; ++i) {
    const int c = tid + i * NT;
    const int row = c / KC, kc = (c % KC) * 8;
    int grow;
    const bf16_t* base;
    if (DUAL) {
      const bool up = row >= BN / 2;
      grow = n0 + (up ? row - BN / 2 : row);
      base = up ? W2 : W;
    } else {
      grow = n0 + row;
      base = W;
    }
    b_ok[i] = c < B_CH && grow < N;
    b_src[i] = base + (size_t)(b_ok[i] ? grow : 0) * K + kbeg + kc;
    b_dst[i] = row * LDSK + kc;
  }

  uint4 ra[A_PT], rb[B_PT];
  auto gload = [&](int kt) {
    const int ko = kt * BK;
#pragma unroll
    for (int i = 0; i < A_PT; ++i)
      ra[i] = a_ok[i] ? *(const uint4*)(a_src[i] + ko) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < B_PT; ++i)
      rb[i] = b_ok[i] ? *(const uint4*)(b_src[i] + ko) : make_uint4(0, 0, 0, 0);
  };
  auto sstore = [&](int stg) {
#pragma unroll
    for (int i = 0; i < A_PT; ++i)
      if (tid + i * NT < A_CH) *(uint4*)&sA[stg][a_dst[i]] = ra[i];
#pragma unroll
    for (int i = 0; i < B_PT; ++i)
      if (tid + i * NT < B_CH) *(uint4*)&sB[stg][b_dst[i]] = rb[i];
  };

  // tile-local B row of this wave's j-th 16-column tile
  auto brow = [&](int j) {
    if (DUAL) {
      return j < TN / 2 ? wn * (WN / 2) + j * 16 : BN / 2 + wn * (WN / 2) + (j - TN / 2) * 16;
    }
    return wn * WN + j * 16;
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (KT > 0) {
    gload(0);
    sstore(0);
    __syncthreads();
  }
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  for (int kt = 0; kt < KT; ++kt) {
    const int stg = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *(const bf16x8*)&sA[stg][(wm * WM + i * 16 + lr) * LDSK + ks * 32 + lk];
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *(const bf16x8*)&sB[stg][(brow(j) + lr) * LDSK + ks * 32 + lk];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(stg ^ 1);
    __syncthreads();
  }

  // epilogue
  const int rq = (lane >> 4) * 4, cl = lane & 15;
  if (SPLIT) {
    const int NC = DUAL ? 2 * N : N;
    float* part = partial + (size_t)blockIdx.y * M * NC;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        int col;
        if (DUAL) {
          const int br = brow(j);
          col = br < BN / 2 ? n0 + br + cl : N + n0 + (br - BN / 2) + cl;
          if (n0 + (br < BN / 2 ? br : br - BN / 2) + cl >= N) continue;
        } else {
          col = n0 + brow(j) + cl;
          if (col >= N) continue;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = m0 + wm * WM + i * 16 + rq + q;
          if (row < M) part[(size_t)row * NC + col] = acc[i][j][q];
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (DUAL) {
#pragma unroll
        for (int j = 0; j < TN / 2; ++j) {
          const int col = n0 + brow(j) + cl;
          if (col >= N) continue;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = m0 + wm * WM + i * 16 + rq + q;
            if (row < M) epi_store<EPI, bf16_t>(ep, row, col, acc[i][j][q], acc[i][j + TN / 2][q]);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = n0 + brow(j) + cl;
          if (col >= N) continue;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = m0 + wm * WM + i * 16 + rq + q;
            if (row < M) epi_store<EPI, bf16_t>(ep, row, col, acc[i][j][q], 0.f);
          }
        }
      }
    }
  }
}

// Split-K reduction: sums the partials in split order, then the epilogue.
template <int EPI, typename T>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial,
                                                            int splits, EpiParams ep) {
  constexpr bool DUAL = EPI == kEpiSwiglu;
  const int NC = DUAL ? 2 * ep.N : ep.N;
  const size_t total = (size_t)ep.M * ep.N;
  const size_t stride = (size_t)ep.M * NC;
  for (size_t f = blockIdx.x * (size_t)blockDim.x + threadIdx.x; f < total;
       f += (size_t)gridDim.x * blockDim.x) {
    const int row = (int)(f / ep.N), col = (int)(f % ep.N);
    float v = 0.f, u = 0.f;
    for (int s = 0; s < splits; ++s) {
      v += partial[s * stride + (size_t)row * NC + col];
      if (DUAL) u += partial[s * stride + (size_t)row * NC + ep.N + col];
    }
    epi_store<EPI, T>(ep, row, col, v, u);
  }
}

// ---------------------------------------------------------------------------
// Generic kernel (any shape, float or bf16 storage): 64x64 tile, 16x16
// threads, 4x4 outputs per thread, fp32 FMA.  DUAL keeps gate and up
// accumulators side by side.
template <typename T, int EPI>
__global__ __launch_bounds__(256) void gemm_generic_kernel(const T* __restrict__ A,
                                                           const T* __restrict__ W,
                                                           const T* __restrict__ W2, EpiParams ep,
                                                           int K) {
  constexpr bool DUAL = EPI == kEpiSwiglu;
  constexpr int TB = 64, TK = 16;
  __shared__ float sA[TK][TB + 1];
  __shared__ float sB[TK][TB + 1];
  __shared__ float sB2[DUAL ? TK : 1][TB + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * TB, n0 = blockIdx.x * TB;
  const int M = ep.M, N = ep.N;
  float acc[4][4] = {}, acc2[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += TK) {
    for (int e = threadIdx.x; e < TB * TK; e += 256) {
      const int r = e / TK, kk = e % TK;
      const int gk = k0 + kk;
      sA[kk][r] = (m0 + r < M && gk < K) ? ld(A, (size_t)(m0 + r) * K + gk) : 0.f;
      sB[kk][r] = (n0 + r < N && gk < K) ? ld(W, (size_t)(n0 + r) * K + gk) : 0.f;
      if (DUAL) sB2[kk][r] = (n0 + r < N && gk < K) ? ld(W2, (size_t)(n0 + r) * K + gk) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[4], b2[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b[j] = sB[kk][tx * 4 + j];
        if (DUAL) b2[j] = sB2[kk][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] += a[i] * b[j];
          if (DUAL) acc2[i][j] += a[i] * b2[j];
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = m0 + ty * 4 + i, col = n0 + tx * 4 + j;
      if (row < M && col < N) epi_store<EPI, T>(ep, row, col, acc[i][j], acc2[i][j]);
    }
}

// ---------------------------------------------------------------------------
// Launch plans.
namespace {

enum TileCfg { kTileS = 0, kTileM = 1, kTileL = 2 };
struct TileDims { int bm, bn; };
constexpr TileDims kTiles[3] = {{32, 128}, {64, 128}, {128, 128}};
constexpr int kBK = 64;
constexpr size_t kSplitCapBytes = 64ull << 20;  // split-K partials never exceed this

struct Plan {
  bool mfma;
  int tile, tiles_m, tiles_n, splits, k_per_split;
  size_t ws;
};

Plan make_plan(int dtype, int epi, int M, int N, int K) {
  Plan p{};
  p.mfma = dtype == kBF16 && K % kBK == 0 && K >= kBK;
  p.splits = 1;
  p.ws = 0;
  if (!p.mfma || M <= 0) return p;
  p.tile = M <= 32 ? kTileS : (M <= 64 ? kTileM : kTileL);
  const TileDims td = kTiles[p.tile];
  const bool dual = epi == kEpiSwiglu;
  const int cols = dual ? 2 * N : N;
  p.tiles_m = (M + td.bm - 1) / td.bm;
  p.tiles_n = (cols + td.bn - 1) / td.bn;
  const int tiles = p.tiles_m * p.tiles_n;
  // split K while the grid is short of two workgroups per CU and every split
  // keeps at least 4 K-steps
  int splits = 1;
  const int ksteps = K / kBK;
  while (tiles * splits < 512 && ksteps / (splits * 2) >= 4 &&
         (size_t)(splits * 2) * M * cols * sizeof(float) <= kSplitCapBytes)
    splits *= 2;
  p.splits = splits;
  p.k_per_split = ((ksteps + splits - 1) / splits) * kBK;
  p.ws = splits > 1 ? (size_t)splits * M * cols * sizeof(float) : 0;
  return p;
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int EPI>
hipError_t run_mfma(const GemmArgs& a, const Plan& p, EpiParams ep, float* ws, hipStream_t s) {
  dim3 grid(p.tiles_m * p.tiles_n, p.splits, 1);
  const int threads = 64 * WAVES_M * WAVES_N;
  if (p.splits > 1) {
    gemm_bf16_mfma_kernel<BM, BN, kBK, WAVES_M, WAVES_N, EPI, true><<<grid, threads, 0, s>>>(
        (const bf16_t*)a.A, (const bf16_t*)a.W, (const bf16_t*)a.W2, ep, a.K, p.k_per_split,
        p.tiles_m, p.tiles_n, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t total = (size_t)a.M * a.N;
    const int g = (int)std::min<size_t>((total + 255) / 256, 8192);
    splitk_reduce_kernel<EPI, bf16_t><<<g, 256, 0, s>>>(ws, p.splits, ep);
  } else {
    gemm_bf16_mfma_kernel<BM, BN, kBK, WAVES_M, WAVES_N, EPI, false><<<grid, threads, 0, s>>>(
        (const bf16_t*)a.A, (const bf16_t*)a.W, (const bf16_t*)a.W2, ep, a.K, p.k_per_split,
        p.tiles_m, p.tiles_n, nullptr);
  }
  return hipGetLastError();
}

template <int EPI>
hipError_t dispatch_mfma(const GemmArgs& a, const Plan& p, EpiParams ep, float* ws,
                         hipStream_t s) {
  switch (p.tile) {
    case kTileS: return run_mfma<32, 128, 1, 4, EPI>(a, p, ep, ws, s);
    case kTileM: return run_mfma<64, 128, 2, 2, EPI>(a, p, ep, ws, s);
    default: return run_mfma<128, 128, 2, 2, EPI>(a, p, ep, ws, s);
  }
}

template <typename T, int EPI>
hipError_t run_generic(const GemmArgs& a, EpiParams ep, hipStream_t s) {
  dim3 grid((a.N + 63) / 64, (a.M + 63) / 64);
  gemm_generic_kernel<T, EPI><<<grid, 256, 0, s>>>((const T*)a.A, (const T*)a.W,
                                                   (const T*)a.W2, ep, a.K);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_generic(const GemmArgs& a, EpiParams ep, hipStream_t s) {
  switch (a.epi) {
    case kEpiStoreF32: return run_generic<T, kEpiStoreF32>(a, ep, s);
    case kEpiResidAdd: return run_generic<T, kEpiResidAdd>(a, ep, s);
    case kEpiSwiglu: return run_generic<T, kEpiSwiglu>(a, ep, s);
    default: return run_generic<T, kEpiLogits>(a, ep, s);
  }
}

}  // namespace

size_t gemm_ws_bytes(int dtype, int epi, int M, int N, int K) {
  return make_plan(dtype, epi, M, N, K).ws;
}

hipError_t launch_gemm(const GemmArgs& a, void* ws, size_t ws_bytes, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  EpiParams ep{a.C, a.M, a.N, a.row_seq, a.row_pos, a.seq_len, a.mask_id};
  Plan p = make_plan(a.dtype, a.epi, a.M, a.N, a.K);
  if (p.mfma && p.ws > ws_bytes) {  // not enough workspace: no split
    p.splits = 1;
    p.k_per_split = a.K;
  }
  if (p.mfma) {
    switch (a.epi) {
      case kEpiStoreF32: return dispatch_mfma<kEpiStoreF32>(a, p, ep, (float*)ws, s);
      case kEpiResidAdd: return dispatch_mfma<kEpiResidAdd>(a, p, ep, (float*)ws, s);
      case kEpiSwiglu: return dispatch_mfma<kEpiSwiglu>(a, p, ep, (float*)ws, s);
      default: return dispatch_mfma<kEpiLogits>(a, p, ep, (float*)ws, s);
    }
  }
  if (a.dtype == kBF16) return dispatch_generic<bf16_t>(a, ep, s);
  return dispatch_generic<float>(a, ep, s);
}

}  // namespace dlm

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
  const float* rope;
  bf16_t* q;
  bf16_t* kc;
  bf16_t* vc;
  int nq, nkv;
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
//   Tile BM x BN x 64, WAVES_M x WAVES_N waves, each wave (BM/WAVES_M) x
//   (BN/WAVES_N) made of 16x16 MFMA tiles.  For SwiGLU (DUAL) the BN tile
//   rows are [BN/2 gate rows | BN/2 up rows] of the same BN/2 features, and
//   each wave owns matching gate/up column tiles so the epilogue pairs them
//   in registers.
//   Operands go straight from global memory into an LDS ring of STAGES
//   stages with global_load_lds_dwordx4: one wave instruction fills 1 KB =
//   8 tile rows of 128 B; lane i writes row i/8, 16-byte slot i%8, and loads
//   the global chunk slot ^ (row & 7), so that the fragment reads below are
//   free of bank conflicts.  The loads of stage kt+STAGES-1 are issued before stage kt is
//   consumed; an explicit vmcnt wait (counting this wave's instructions of
//   the later stages still in flight) plus a workgroup barrier publish a
//   stage.
//   v_mfma_f32_16x16x32_bf16: lane l supplies A[row l%16][k-group l/16] and
//   B[k-group l/16][col l%16] (8 consecutive k each; the same k mapping on
//   both sides) and receives C[4*(l/16)+i][l%16], i = 0..3.
//   Split-K (gridDim.y > 1) writes fp32 partials [split][M][NC] instead of
//   the epilogue, NC = N (2N for DUAL: gate at f, up at N+f).
typedef __attribute__((address_space(3))) void lds_void;

// 16-byte slot XOR for 128-byte tile rows.  Measured on gfx950 with
// SQ_LDS_BANK_CONFLICT: the fragment reads below (lane l: row l%16, chunk
// l/16) are conflict-free with r & 7 and two-way conflicted with padded rows
// or with (r & 7) ^ ((r >> 3) & 1).
__device__ __forceinline__ int swz(int r) { return r & 7; }

// One 16-byte-per-lane direct load from global memory into LDS; the LDS
// destination (wave-uniform) receives lane i's 16 bytes at offset 16 i.
__device__ __forceinline__ void dma16(const void* g, unsigned char* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] at bits 3:0 and vmcnt[5:4] at bits 15:14; expcnt and lgkmcnt at
// their maxima, i.e. not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int EPI, bool SPLIT>
__global__ __launch_bounds__(64 * WAVES_M* WAVES_N) void gemm_bf16_mfma_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ W, const bf16_t* __restrict__ W2,
    EpiParams ep, int K, int k_per_split, int tiles_m, int tiles_n, float* __restrict__ partial) {
  constexpr bool DUAL = EPI == kEpiSwiglu;
  constexpr int BK = 64;
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int ROWS = BM + BN;                // tile rows per stage (A then B)
  constexpr int INSTR = ROWS / 8;              // 1 KB load instructions per stage
  constexpr int IPW = INSTR / NW;              // per wave
  constexpr int STAGE_BYTES = ROWS * 128;
  static_assert(INSTR % NW == 0, "load instructions must split evenly over the waves");
  static_assert(!DUAL || (TN % 2 == 0), "dual tiles need an even number of column tiles");
  static_assert(STAGES >= 2 && STAGES <= 4, "stages");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

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

  // this lane's source pointer for each of its load instructions
  const bf16_t* src[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int j = wave + i * NW;             // instruction index within the stage
    const int r = j * 8 + (lane >> 3);       // tile row (A rows then B rows)
    const int chunk = (lane & 7) ^ swz(r);   // global 16-byte chunk for slot lane&7
    const bf16_t* base;
    if (r < BM) {
      const int gr = min(m0 + r, M - 1);     // rows past M load a valid row; discarded
      base = A + (size_t)gr * K;
    } else {
      const int br = r - BM;
      int grow;
      const bf16_t* wb;
      if (DUAL) {
        const bool up = br >= BN / 2;
        grow = n0 + (up ? br - BN / 2 : br);
        wb = up ? W2 : W;
      } else {
        grow = n0 + br;
        wb = W;
      }
      base = wb + (size_t)min(grow, N - 1) * K;
    }
    src[i] = base + kbeg + chunk * 8;
  }
  auto issue = [&](int kt) {
    unsigned char* st = smem + (kt % STAGES) * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int j = wave + i * NW;
      dma16(src[i] + kt * BK, st + j * 1024);
    }
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

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < KT) issue(s);

  const int lr = lane & 15, lk = lane >> 4;
  for (int kt = 0; kt < KT; ++kt) {
    // wait for this wave's loads of stage kt (the later stages issued so far
    // may stay in flight), then publish the stage to the workgroup
    const int ahead = min(STAGES - 2, KT - 1 - kt);
    if (STAGES >= 4 && ahead >= 2) wait_vmcnt<2 * IPW>();
    else if (STAGES >= 3 && ahead >= 1) wait_vmcnt<IPW>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    // every wave has finished iteration kt-1, so its stage can be refilled
    if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1);
    const unsigned char* st = smem + (kt % STAGES) * STAGE_BYTES;
    bf16x8 af[BK / 32][TM], bfr[BK / 32][TN];
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WM + i * 16 + lr;
        af[ks][i] = *(const bf16x8*)(st + r * 128 + (((ks * 4 + lk) ^ swz(r)) << 4));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = BM + brow(j) + lr;
        bfr[ks][j] = *(const bf16x8*)(st + r * 128 + (((ks * 4 + lk) ^ swz(r)) << 4));
      }
    }
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks][i], bfr[ks][j], acc[i][j], 0, 0, 0);
  }

  // epilogue
  const int rq = (lane >> 4) * 4, cl = lane & 15;
  if constexpr (EPI == kEpiQKV) {
    // The tile is one head (BN = hd = 128) and each wave holds all of its
    // columns, so lane l has both halves (c, c + 64) of each rotary pair.
    static_assert(BN == 128 && WAVES_N == 1, "fused QKV epilogue needs one head per wave");
    const int hix = n0 / 128;  // head in the q | k | v list
    const int nq = ep.nq, nkv = ep.nkv, Nseq = ep.seq_len;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      int rows[4], seqs[4], poss[4];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        rows[qq] = m0 + wm * WM + i * 16 + rq + qq;
        const int rr = min(rows[qq], M - 1);
        seqs[qq] = ep.row_seq[rr];
        poss[qq] = ep.row_pos[rr];
      }
      if (hix < nq + nkv) {
        // all rotary factors of this row block first (independent loads in
        // flight together), then the rotations and stores
        float cs[4][4], sn[4][4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const float2 t2 = ep.rope ? *(const float2*)(ep.rope +
                                                         ((size_t)poss[qq] * 64 + jt * 16 + cl) * 2)
                                      : make_float2(1.f, 0.f);
            cs[jt][qq] = t2.x;
            sn[jt][qq] = t2.y;
          }
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const int c = jt * 16 + cl;  // rotary pair (c, c + 64)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            if (rows[qq] >= M) continue;
            const float a0 = acc[i][jt][qq], a1 = acc[i][jt + 4][qq];
            const float r0 = a0 * cs[jt][qq] - a1 * sn[jt][qq];
            const float r1 = a0 * sn[jt][qq] + a1 * cs[jt][qq];
            bf16_t* dst = hix < nq
                              ? ep.q + (size_t)rows[qq] * nq * 128 + (size_t)hix * 128
                              : ep.kc + (((size_t)seqs[qq] * nkv + (hix - nq)) * Nseq + poss[qq]) * 128;
            dst[c] = f2bf(r0);
            dst[c + 64] = f2bf(r1);
          }
        }
      } else {
        const int g = hix - nq - nkv;
        const bool packed = rows[3] < M && seqs[3] == seqs[0] && poss[3] == poss[0] + 3 &&
                            seqs[1] == seqs[0] && poss[1] == poss[0] + 1 &&
                            seqs[2] == seqs[0] && poss[2] == poss[0] + 2 && (poss[0] & 3) == 0;
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) {
          const int c = jt * 16 + cl;
          if (packed) {
            ushort4 w;
            w.x = f2bf(acc[i][jt][0]);
            w.y = f2bf(acc[i][jt][1]);
            w.z = f2bf(acc[i][jt][2]);
            w.w = f2bf(acc[i][jt][3]);
            *(ushort4*)(ep.vc + (((size_t)seqs[0] * nkv + g) * 128 + c) * Nseq + poss[0]) = w;
          } else {
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
              if (rows[qq] < M)
                ep.vc[(((size_t)seqs[qq] * nkv + g) * 128 + c) * Nseq + poss[qq]] =
                    f2bf(acc[i][jt][qq]);
          }
        }
      }
    }
  } else if (SPLIT) {
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
//
// Tile configurations (rows x cols, waves, LDS stages).  The plan picks the
// configuration by M (the ragged active-row count) and splits K while the
// grid would leave CUs idle.
namespace {

struct TileCfg {
  int bm, bn, wm, wn, stages;
};
constexpr TileCfg kCfgs[] = {
    {32, 128, 1, 4, 4},   // 0: weight streaming
    {64, 128, 2, 2, 4},   // 1: weight streaming
    {128, 128, 2, 2, 3},  // 2
    {128, 256, 2, 2, 3},  // 3
    {256, 128, 2, 2, 3},  // 4
    {192, 128, 2, 2, 3},  // 5
    {96, 128, 1, 4, 3},   // 6
    {32, 64, 1, 4, 4},    // 7: narrow column tiles (not for SwiGLU)
    {128, 128, 2, 4, 3},  // 8: 8 waves
    {256, 128, 4, 2, 3},  // 9: 8 waves
    {128, 256, 2, 4, 3},  // 10: 8 waves
    {128, 128, 2, 2, 2},  // 11: two workgroups per CU
    {192, 128, 2, 2, 2},  // 12: two workgroups per CU
    {256, 256, 2, 4, 2},  // 13: 8 waves, 128x64 per wave
    {64, 64, 2, 2, 4},    // 14
    {192, 128, 4, 1, 2},  // 15: one head per wave (fused QKV epilogue)
    {128, 128, 4, 1, 3},  // 16: one head per wave
    {256, 128, 4, 1, 2},  // 17: one head per wave
    {64, 128, 4, 1, 4},   // 18: one head per wave
};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);
constexpr int kBK = 64;
constexpr size_t kSplitCapBytes = 64ull << 20;  // split-K partials never exceed this
constexpr int kCUs = 256;

inline size_t cfg_lds(const TileCfg& c) { return (size_t)c.stages * (c.bm + c.bn) * 128; }

struct Plan {
  bool mfma;
  int cfg, tiles_m, tiles_n, splits, k_per_split;
  size_t ws;
  bool defer_reduce;  // split-K partials are left for the consumer kernel
};

// Default configuration by GEMM class and M bucket, from a sweep of every
// configuration on MI355X at the LLaDA-8B shapes (QKV 4096->12288, O
// 4096->4096, gate/up 4096->2x12288, down 12288->4096, LM head
// 4096->126464): small M favours narrow row tiles that stream the weights
// with many workgroups; large M favours 2-stage tiles with two workgroups per
// CU or 256x256 tiles with 8 waves.
int pick_cfg(int M, int N, bool dual) {
  static const int kBucket[] = {16, 32, 64, 128, 192, 256, 320, 384, 512};
  static const int kNarrow[] = {7, 7, 1, 1, 6, 8, 5, 5, 8, 13};
  static const int kMedium[] = {7, 7, 14, 1, 6, 8, 5, 5, 9, 13};
  static const int kDual[] = {1, 1, 1, 8, 5, 9, 12, 12, 13, 13};
  static const int kWide[] = {7, 7, 14, 10, 12, 13, 12, 12, 13, 13};
  int b = 0;
  while (b < 9 && M > kBucket[b]) ++b;
  if (dual) return kDual[b];
  if (N <= 8192) return kNarrow[b];
  if (N <= 32768) return kMedium[b];
  return kWide[b];
}

Plan make_plan_cfg(int dtype, int epi, int M, int N, int K, int cfg) {
  Plan p{};
  p.mfma = dtype == kBF16 && K % kBK == 0 && K >= kBK;
  p.splits = 1;
  p.ws = 0;
  p.cfg = cfg;
  if (!p.mfma || M <= 0) return p;
  const TileCfg td = kCfgs[cfg];
  const bool dual = epi == kEpiSwiglu;
  const int cols = dual ? 2 * N : N;
  p.tiles_m = (M + td.bm - 1) / td.bm;
  p.tiles_n = (cols + td.bn - 1) / td.bn;
  const int tiles = p.tiles_m * p.tiles_n;
  const int per_cu = cfg_lds(td) <= 80 * 1024 ? 2 : 1;  // resident workgroups per CU
  // split K while the grid covers less than the resident slots and every
  // split keeps at least 4 K-steps
  int splits = 1;
  const int ksteps = K / kBK;
  while (tiles * splits * 2 <= kCUs * per_cu && ksteps / (splits * 2) >= 4 &&
         (size_t)(splits * 2) * M * cols * sizeof(float) <= kSplitCapBytes)
    splits *= 2;
  p.splits = splits;
  p.k_per_split = ((ksteps + splits - 1) / splits) * kBK;
  p.ws = splits > 1 ? (size_t)splits * M * cols * sizeof(float) : 0;
  return p;
}

Plan make_plan(int dtype, int epi, int M, int N, int K) {
  return make_plan_cfg(dtype, epi, M, N, K, pick_cfg(M, N, epi == kEpiSwiglu));
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int EPI>
hipError_t run_mfma(const GemmArgs& a, const Plan& p, EpiParams ep, void* ws, hipStream_t s) {
  constexpr bool DUAL = EPI == kEpiSwiglu;
  if constexpr (DUAL && ((BN / WAVES_N / 16) % 2 != 0)) {
    return hipErrorInvalidValue;  // a dual tile needs matching gate/up column tiles per wave
  } else if constexpr (EPI == kEpiQKV && !(BN == 128 && WAVES_N == 1)) {
    return hipErrorInvalidValue;  // the fused QKV epilogue needs one head per wave
  } else {
    dim3 grid(p.tiles_m * p.tiles_n, p.splits, 1);
    const int threads = 64 * WAVES_M * WAVES_N;
    const size_t lds = (size_t)STAGES * (BM + BN) * 128;
    float* partial = (float*)ws;
    if (p.splits > 1) {
      static bool attr = false;
      if (!attr) {
        (void)hipFuncSetAttribute(
            reinterpret_cast<const void*>(
                &gemm_bf16_mfma_kernel<BM, BN, WAVES_M, WAVES_N, STAGES, EPI, true>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        attr = true;
      }
      gemm_bf16_mfma_kernel<BM, BN, WAVES_M, WAVES_N, STAGES, EPI, true>
          <<<grid, threads, lds, s>>>((const bf16_t*)a.A, (const bf16_t*)a.W,
                                      (const bf16_t*)a.W2, ep, a.K, p.k_per_split, p.tiles_m,
                                      p.tiles_n, partial);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const size_t total = (size_t)a.M * a.N;
      const int g = (int)std::min<size_t>((total + 255) / 256, 8192);
      if (!p.defer_reduce) splitk_reduce_kernel<EPI, bf16_t><<<g, 256, 0, s>>>(partial, p.splits, ep);
    } else {
      static bool attr = false;
      if (!attr) {
        (void)hipFuncSetAttribute(
            reinterpret_cast<const void*>(
                &gemm_bf16_mfma_kernel<BM, BN, WAVES_M, WAVES_N, STAGES, EPI, false>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        attr = true;
      }
      gemm_bf16_mfma_kernel<BM, BN, WAVES_M, WAVES_N, STAGES, EPI, false>
          <<<grid, threads, lds, s>>>((const bf16_t*)a.A, (const bf16_t*)a.W,
                                      (const bf16_t*)a.W2, ep, a.K, p.k_per_split, p.tiles_m,
                                      p.tiles_n, nullptr);
    }
    return hipGetLastError();
  }
}

template <int EPI>
hipError_t dispatch_mfma(const GemmArgs& a, const Plan& p, EpiParams ep, void* ws,
                         hipStream_t s) {
  switch (p.cfg) {
    case 0: return run_mfma<32, 128, 1, 4, 4, EPI>(a, p, ep, ws, s);
    case 1: return run_mfma<64, 128, 2, 2, 4, EPI>(a, p, ep, ws, s);
    case 2: return run_mfma<128, 128, 2, 2, 3, EPI>(a, p, ep, ws, s);
    case 3: return run_mfma<128, 256, 2, 2, 3, EPI>(a, p, ep, ws, s);
    case 4: return run_mfma<256, 128, 2, 2, 3, EPI>(a, p, ep, ws, s);
    case 5: return run_mfma<192, 128, 2, 2, 3, EPI>(a, p, ep, ws, s);
    case 6: return run_mfma<96, 128, 1, 4, 3, EPI>(a, p, ep, ws, s);
    case 7: return run_mfma<32, 64, 1, 4, 4, EPI>(a, p, ep, ws, s);
    case 8: return run_mfma<128, 128, 2, 4, 3, EPI>(a, p, ep, ws, s);
    case 9: return run_mfma<256, 128, 4, 2, 3, EPI>(a, p, ep, ws, s);
    case 10: return run_mfma<128, 256, 2, 4, 3, EPI>(a, p, ep, ws, s);
    case 11: return run_mfma<128, 128, 2, 2, 2, EPI>(a, p, ep, ws, s);
    case 12: return run_mfma<192, 128, 2, 2, 2, EPI>(a, p, ep, ws, s);
    case 13: return run_mfma<256, 256, 2, 4, 2, EPI>(a, p, ep, ws, s);
    case 14: return run_mfma<64, 64, 2, 2, 4, EPI>(a, p, ep, ws, s);
    case 15: return run_mfma<192, 128, 4, 1, 2, EPI>(a, p, ep, ws, s);
    case 16: return run_mfma<128, 128, 4, 1, 3, EPI>(a, p, ep, ws, s);
    case 17: return run_mfma<256, 128, 4, 1, 2, EPI>(a, p, ep, ws, s);
    default: return run_mfma<64, 128, 4, 1, 4, EPI>(a, p, ep, ws, s);
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

hipError_t launch_plan(const GemmArgs& a, Plan p, void* ws, size_t ws_bytes, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  EpiParams ep{a.C, a.M, a.N, a.row_seq, a.row_pos, a.seq_len, a.mask_id, a.rope,
               (bf16_t*)a.q, (bf16_t*)a.kc, (bf16_t*)a.vc, a.nq, a.nkv};
  if (a.epi == kEpiQKV) {
    p.splits = 1;  // the fused epilogue needs complete sums
    p.k_per_split = a.K;
    return dispatch_mfma<kEpiQKV>(a, p, ep, ws, s);
  }
  if (p.mfma && p.ws > ws_bytes) {  // not enough workspace: no split
    p.splits = 1;
    p.k_per_split = a.K;
  }
  if (p.mfma) {
    switch (a.epi) {
      case kEpiStoreF32: return dispatch_mfma<kEpiStoreF32>(a, p, ep, ws, s);
      case kEpiResidAdd: return dispatch_mfma<kEpiResidAdd>(a, p, ep, ws, s);
      case kEpiSwiglu: return dispatch_mfma<kEpiSwiglu>(a, p, ep, ws, s);
      default: return dispatch_mfma<kEpiLogits>(a, p, ep, ws, s);
    }
  }
  if (a.dtype == kBF16) return dispatch_generic<bf16_t>(a, ep, s);
  return dispatch_generic<float>(a, ep, s);
}

}  // namespace

size_t gemm_ws_bytes(int dtype, int epi, int M, int N, int K) {
  return make_plan(dtype, epi, M, N, K).ws;
}

bool gemm_qkv_fusable(int dtype, int M, int hd, int K) {
  return dtype == kBF16 && hd == 128 && K % kBK == 0 && M >= 96;
}

// Tile for the fused QKV epilogue by M.
int pick_qkv_cfg(int M) {
  if (M <= 128) return 16;
  if (M <= 192) return 15;
  if (M <= 256) return 16;
  if (M <= 384) return 15;
  return 17;
}

hipError_t launch_gemm(const GemmArgs& a, void* ws, size_t ws_bytes, hipStream_t s) {
  if (a.epi == kEpiQKV)
    return launch_plan(a, make_plan_cfg(a.dtype, a.epi, a.M, a.N, a.K, pick_qkv_cfg(a.M)), ws,
                       ws_bytes, s);
  return launch_plan(a, make_plan(a.dtype, a.epi, a.M, a.N, a.K), ws, ws_bytes, s);
}

hipError_t launch_gemm_deferred(const GemmArgs& a, void* ws, size_t ws_bytes, hipStream_t s,
                                int* splits_out) {
  Plan p = make_plan(a.dtype, a.epi, a.M, a.N, a.K);
  *splits_out = 0;
  if (p.mfma && p.splits > 1 && p.ws <= ws_bytes &&
      (a.epi == kEpiStoreF32 || a.epi == kEpiResidAdd)) {
    p.defer_reduce = true;
    *splits_out = p.splits;
  }
  return launch_plan(a, p, ws, ws_bytes, s);
}

int gemm_num_configs() { return kNumCfgs; }

// Same GEMM with a forced tile configuration (for tuning sweeps); cfg < 0
// uses the default plan.
hipError_t launch_gemm_cfg(const GemmArgs& a, int cfg, int splits, void* ws, size_t ws_bytes,
                           hipStream_t s) {
  if (cfg < 0 || cfg >= kNumCfgs) return launch_gemm(a, ws, ws_bytes, s);
  Plan p = make_plan_cfg(a.dtype, a.epi, a.M, a.N, a.K, cfg);
  if (p.mfma && splits > 0) {
    const int ksteps = a.K / kBK;
    p.splits = splits;
    p.k_per_split = ((ksteps + splits - 1) / splits) * kBK;
    p.ws = splits > 1 ? (size_t)splits * a.M * (a.epi == kEpiSwiglu ? 2 : 1) * a.N * 4 : 0;
  }
  return launch_plan(a, p, ws, ws_bytes, s);
}

}  // namespace dlm

// Active-row GEMMs: Y = A W^T on the M compacted rows, with fused epilogues.
//
// SureLock page ("Stopping Computation for Converged Tokens in Masked
// Diffusion-LM Decoding"), §2 Methodology: locked positions skip the query
// projection and the FFN; only the active subset gets fresh Q/K/V; FFN cost
// falls to O(M_t d^2) (§2 algorithmic complexity).  M shrinks from step to
// step, so the launch plan depends on M: large M is MFMA-bound (bf16
// 16x16x32 MFMA fed from an LDS ring of k-slices, with fragment prefetch on
// the 8-wave tiles), small M is bound by streaming the weights once (narrow
// row tiles, split-K across workgroups whose partial sums are added in split
// order, by a reduction kernel or by the next residual RMSNorm).
//
// Epilogues: plain float store, residual add into the float residual stream
// (out-projection, down-projection), SwiGLU over a gate/up pair of weight
// matrices (silu(A Wg^T) * (A Wu^T), stored in the storage type), QKV with
// the rotary embedding and the K / V^T cache scatter, and logits scattered to
// each row's (seq, pos) slot with the mask token's column forced to -inf; the
// last optionally also folds each row's logits, with the row's previous-step
// logits, into the partial posterior statistics (log-normaliser, argmax,
// confidence, KL) of its column tile, so that no separate pass re-reads the
// current logits.
#include <utility>

#include "common.h"
#include "internal.h"
#include "vocab_part.h"

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
  const float* zprev;
  const float* lse_prev;
  const int32_t* has_prev;
  VocabPart* parts;
  int kl_dir;
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
//   Tile BM x BN, K consumed in slices of BK (32 or 64), WAVES_M x WAVES_N
//   waves, each wave (BM/WAVES_M) x (BN/WAVES_N) made of 16x16 MFMA tiles.
//   For SwiGLU (DUAL) the BN tile rows are [BN/2 gate rows | BN/2 up rows]
//   of the same BN/2 features, and each wave owns matching gate/up column
//   tiles so the epilogue pairs them in registers.
//   Operands go straight from global memory into an LDS ring of STAGES
//   k-slices with global_load_lds_dwordx4: one wave instruction fills 1 KB
//   of consecutive tile rows of 2 BK bytes; lane i writes row i/CH, 16-byte
//   slot i%CH (CH = BK/8 slots per row) and loads the global chunk
//   slot ^ x(row), where x is the slot XOR that keeps the fragment reads
//   below free of bank conflicts.  Slices kt+1 .. kt+STAGES-1 are in flight
//   while slice kt is multiplied; an explicit vmcnt wait (counting this
//   wave's load instructions of the later slices) plus a workgroup barrier
//   publish a slice, and the slot of slice kt-1 is refilled right after that
//   barrier (every wave has finished slice kt-1 by then).
//   v_mfma_f32_16x16x32_bf16: lane l supplies A[row l%16][k-group l/16] and
//   B[k-group l/16][col l%16] (8 consecutive k each; the same k mapping on
//   both sides) and receives C[4*(l/16)+i][l%16], i = 0..3.
//   Split-K (gridDim.y > 1) writes fp32 partials [split][M][NC] instead of
//   the epilogue, NC = N (2N for DUAL: gate at f, up at N+f).
typedef __attribute__((address_space(3))) void lds_void;

// 16-byte slot XOR by tile row, measured conflict-free on gfx950
// (SQ_LDS_BANK_CONFLICT) for the fragment reads (lane l: row l%16, slot l/16):
// 128-byte rows (8 slots): r & 7; 64-byte rows (4 slots): (r >> 1) & 2.  (For
// 64-byte rows, (r >> 2) & 3 is two-way conflicted.)
template <int CH>
__device__ __forceinline__ int slot_xor(int r) {
  if constexpr (CH == 8) return r & 7;
  else return (r >> 1) & 2;
}

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

// Waits until at most n (0 <= n < S) k-slices of IPW load instructions each
// are still in flight for this wave.
template <int IPW, int S>
__device__ __forceinline__ void wait_slices(int n) {
  if constexpr (S <= 1) {
    wait_vmcnt<0>();
  } else {
    if (n >= S - 1) wait_vmcnt<(S - 1) * IPW>();
    else wait_slices<IPW, S - 1>(n);
  }
}

// s_waitcnt lgkmcnt(0) only (vmcnt and expcnt at their maxima).
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

// Workgroup barrier without the vmcnt(0) that __syncthreads() implies; the
// empty asm statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Largest divisor k of waves_m such that k wave rows of wm tile rows, of
// row_bytes each, fit in ring bytes (0 if none does).
constexpr int qkv_wave_rows_per_pass(int waves_m, int wm, int row_bytes, int ring) {
  for (int k = waves_m; k >= 1; --k)
    if (waves_m % k == 0 && (long long)k * wm * row_bytes <= ring) return k;
  return 0;
}

// QKV column order inside each 128-wide head: the tile's column v holds the
// weight row (output feature) with bits 5 and 6 of v swapped, an involution
// that puts the rotary partners j and j + 64 of a half-split head into the
// same 64-column chunk (chunk hb of a head holds j = 32 hb + w and
// j + 64, w < 32), so a QKV tile may be any multiple of 64 columns wide.
__host__ __device__ constexpr int qkv_col_swap(int v) {
  return (v & ~0x60) | ((v & 0x20) << 1) | ((v & 0x40) >> 1);
}

template <bool B, typename T>
__device__ __forceinline__ T& pick(T& a, T& b) {
  if constexpr (B) return b;
  else return a;
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>), in order.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// The 4-wave prefetch tiles are bounded to 256 registers (two waves per
// SIMD): without the bound the compiler spreads the loop-carried
// accumulators over AGPRs and VGPRs and copies them between the two files
// every iteration; with it, they stay in VGPRs (252 on the 96x192 tile, no
// spills).
// Two waves per SIMD (at most 256 registers each) for the 4-wave prefetch
// tiles, and for the 4-wave statistics tiles whose LDS ring lets two
// workgroups share a CU (one's epilogue then overlaps the other's main loop).
template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int BK, int EPI, bool PF>
constexpr int gemm_waves_per_simd() {
  return (WAVES_M * WAVES_N == 4 &&
          (PF || (EPI == kEpiLogitsStats && STAGES * (BM + BN) * BK * 2 <= 80 * 1024)))
             ? 2
             : 1;
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int BK, int EPI, bool SPLIT,
          bool PF = false>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N,
                             (gemm_waves_per_simd<BM, BN, WAVES_M, WAVES_N, STAGES, BK, EPI,
                                                  PF>())) void gemm_bf16_mfma_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ W, const bf16_t* __restrict__ W2,
    EpiParams ep, int K, int k_per_split, int tiles_m, int tiles_n, float* __restrict__ partial) {
  constexpr bool DUAL = EPI == kEpiSwiglu;
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int KS = BK / 32;                  // MFMA k-steps per slice
  constexpr int CH = BK / 8;                   // 16-byte slots per tile row
  constexpr int RB = BK * 2;                   // bytes per tile row
  constexpr int RPI = 64 / CH;                 // tile rows per 1 KB load instruction
  constexpr int ROWS = BM + BN;                // tile rows per slice (A then B)
  constexpr int INSTR = ROWS / RPI;            // load instructions per slice
  // Instruction j of a slice is issued by wave j % NW: the first INSTR % NW
  // waves issue IPW per slice, the others IPW_LO.  Every wave waits as if it
  // issued IPW_LO, which is exact for the latter and, since a wave's loads
  // complete in order, only waits for a few more of the newest loads in the
  // former.
  constexpr int IPW_LO = INSTR / NW;
  constexpr int IPW = (INSTR + NW - 1) / NW;
  constexpr bool EVEN = IPW == IPW_LO;
  constexpr int STAGE_BYTES = ROWS * RB;
  static_assert(BK == 32 || BK == 64, "k-slice");
  static_assert(ROWS % RPI == 0 && IPW_LO >= 1,
                "every wave issues at least one load instruction per slice");
  static_assert((STAGES - 1) * IPW < 64, "in-flight loads must fit the vmcnt counter");
  static_assert(!DUAL || (TN % 2 == 0), "dual tiles need an even number of column tiles");
  static_assert(STAGES >= 2 && STAGES <= 8, "stages");
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
    // instruction index within the slice (a wave's missing last one, never
    // issued, points at the slice's last row)
    const int j = min(wave + i * NW, INSTR - 1);
    const int r = j * RPI + lane / CH;             // tile row (A rows then B rows)
    const int chunk = (lane % CH) ^ slot_xor<CH>(r);  // global chunk for this slot
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
        if constexpr (EPI == kEpiQKV) grow = qkv_col_swap(grow);
        wb = W;
      }
      base = wb + (size_t)min(grow, N - 1) * K;
    }
    src[i] = base + kbeg + chunk * 8;
  }
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // The gate/up, fused-QKV and LM-head GEMMs walk their k-slices in a
  // rotated order, so that the workgroups of an XCD request different
  // k-offsets of their weight rows at a time (rows 8 KB apart all share one
  // offset modulo the row size otherwise): gate/up by the workgroup's place
  // in the grid, QKV and the LM head by the column tile, which keeps the row
  // tiles of a weight block in step (four and two of them share it in L2;
  // each order measured the faster for its class).  Each tile's sums then
  // run in a different order, which only rounding sees (and which is the
  // same for the logits and the logits-with-statistics epilogues of one
  // tile); the split-K projections keep the plain order (measured slower).
  constexpr bool ROT = !SPLIT && (EPI == kEpiSwiglu || EPI == kEpiQKV || EPI == kEpiLogits ||
                                  EPI == kEpiLogitsStats);
  const int krot = !ROT || KT <= 0 ? 0 : (EPI == kEpiSwiglu ? lin : nt) % KT;
  auto issue = [&](int kt) {
    unsigned char* st = smem + (kt % STAGES) * STAGE_BYTES;
    const int kp = kt + krot < KT ? kt + krot : kt + krot - KT;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int j = wave_u + i * NW;
      if (EVEN || i < IPW_LO || j < INSTR) dma16(src[i] + kp * BK, st + j * 1024);
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

  struct Frags {
    bf16x8 a[KS][TM], b[KS][TN];
  };
  const int lr = lane & 15, lk = lane >> 4;
  auto read_frags = [&](int slice, Frags& F) {
    const unsigned char* st = smem + (slice % STAGES) * STAGE_BYTES;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WM + i * 16 + lr;
        F.a[ks][i] = *(const bf16x8*)(st + r * RB + (((ks * 4 + lk) ^ slot_xor<CH>(r)) << 4));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = BM + brow(j) + lr;
        F.b[ks][j] = *(const bf16x8*)(st + r * RB + (((ks * 4 + lk) ^ slot_xor<CH>(r)) << 4));
      }
    }
  };
  auto mma = [&](const Frags& F) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(F.a[ks][i], F.b[ks][j], acc[i][j], 0, 0, 0);
  };
  if constexpr (!PF) {
    // slice kt: publish it, refill the slot of slice kt-1 (every wave has
    // passed this barrier, so it finished slice kt-1), then read and multiply
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < KT) issue(s);
    for (int kt = 0; kt < KT; ++kt) {
      wait_slices<IPW_LO, STAGES - 1>(min(STAGES - 2, KT - 1 - kt));
      lds_barrier();
      if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1);
      Frags f;
      read_frags(kt, f);
      mma(f);
      {
        // issue order within the slice: the first k-step's fragment reads,
        // then its MFMAs interleaved with the next k-step's reads, then the
        // remaining MFMAs (the compiler's own order waited for most reads
        // before the first MFMA; measured 1-6% faster)
        constexpr int R = TM + TN, MM = TM * TN;
        constexpr int PER = MM / R > 0 ? MM / R : 1;
        __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
#pragma unroll
        for (int ks = 1; ks < KS; ++ks) {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
        }
        __builtin_amdgcn_sched_group_barrier(0x008, KS * MM - (KS - 1) * R * PER, 0);
      }
    }
  } else {
    // Fragment prefetch over a 3-slot ring: while the MFMAs of slice kt run
    // on fragments already in registers, the fragments of slice kt+1 are
    // read from LDS, and slice kt+3 is loaded into the slot slice kt left
    // (every wave read it before this step's barrier).  Two slices of loads
    // are in flight behind the one being read.
    static_assert(STAGES == 3, "fragment prefetch runs a 3-slot ring");
    static_assert(2 * IPW < 64, "in-flight loads must fit the vmcnt counter");
    constexpr int RT = (TM + TN) * KS, MT = TM * TN * KS;
    constexpr int PER = MT / RT > 0 ? MT / RT : 1;
    Frags f0, f1;
#pragma unroll
    for (int s = 0; s < 3; ++s)
      if (s < KT) issue(s);
    if (KT > 0) {
      wait_slices<IPW_LO, 3>(min(2, KT - 1));
      lds_barrier();
      read_frags(0, f0);
      wait_lgkm0();
    }
    // step kt: slice kt+1 lands (the last step re-reads slice kt, which no
    // load overwrites any more, so that the reads and the MFMAs stay in one
    // block), slice kt+3 is issued while kt + 3 < KT
    auto step = [&](int kt, Frags& cur, Frags& nxt) __attribute__((always_inline)) {
      wait_slices<IPW_LO, 3>(min(1, max(0, KT - 2 - kt)));
      lds_barrier();
      if (kt + 3 < KT) issue(kt + 3);
      read_frags(min(kt + 1, KT - 1), nxt);
      mma(cur);
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, MT - RT * PER, 0);
      wait_lgkm0();  // this wave's reads are done before the next barrier
    };
    for (int kt = 0; kt < KT; kt += 2) {
      step(kt, f0, f1);
      if (kt + 1 < KT) step(kt + 1, f1, f0);
    }
  }

  // epilogue
  const int rq = (lane >> 4) * 4, cl = lane & 15;
  if constexpr (EPI == kEpiQKV) {
    // The tile is BN/64 chunks of 64 columns in the swapped order of
    // qkv_col_swap: chunk g of the q | k | v list is half hb = g & 1 of head
    // g >> 1, with columns w < 32 holding head dimension 32 hb + w and
    // columns 32 + w holding its rotary partner 64 + 32 hb + w.  The fp32
    // tile is staged in LDS (the operand ring is free by now), with each
    // row's (sequence, position), in passes of whole wave rows when it does
    // not fit at once, so that any thread can pair a column with its partner
    // for the rotary embedding and the stores coalesce: q and K rows as
    // packed bf16 pairs along the head dimension, V transposed with 4
    // consecutive positions per 8-byte store.  The item loops have
    // compile-time trip counts and are unrolled so that their loads are all
    // in flight together.
    static_assert(BN % 64 == 0, "the fused QKV epilogue works on 64-column chunks");
    constexpr int LDW = BN + 4;  // padded LDS row stride (floats)
    constexpr int NT = 64 * NW;
    constexpr int WMP = qkv_wave_rows_per_pass(WAVES_M, WM, LDW * 4 + 8, STAGES * STAGE_BYTES);
    static_assert(WMP >= 1, "one wave row of the tile must fit the LDS ring");
    constexpr int PR = WMP * WM;  // tile rows per pass
    static_assert(PR % 4 == 0, "row quads");
    float* T = (float*)smem;
    int2* meta = (int2*)(smem + (size_t)PR * LDW * 4);  // (sequence, position) per row
    const int nq = ep.nq, nkv = ep.nkv, Nseq = ep.seq_len;
    const int nheads = nq + 2 * nkv;
    auto pass = [&](auto P) __attribute__((always_inline)) {
      constexpr int p = decltype(P)::value;
      const int r0 = m0 + p * PR;  // first row of this pass
      __syncthreads();  // operand ring, or the previous pass's rows, no longer read
      if (wm / WMP == p) {
        const int rb = (wm % WMP) * WM;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              T[(rb + i * 16 + rq + q) * LDW + wn * WN + j * 16 + cl] = acc[i][j][q];
      }
      for (int r = tid; r < PR; r += NT) {
        const int rr = min(r0 + r, M - 1);
        meta[r] = make_int2(ep.row_seq[rr], ep.row_pos[rr]);
      }
      __syncthreads();
#pragma unroll
      for (int ch = 0; ch < BN / 64; ++ch) {
        const int g = n0 / 64 + ch;
        const int hix = g >> 1, hb = g & 1;  // head in the q | k | v list, its half
        const float* Tc = T + ch * 64;
        if (hix >= nheads) {
          // columns past N: nothing to store
        } else if (hix < nq + nkv) {
          // q or K head: item = (row, two consecutive rotary pairs w, w + 1)
          constexpr int ITEMS = PR * 16, ITER = (ITEMS + NT - 1) / NT;
#pragma unroll
          for (int k = 0; k < ITER; ++k) {
            const int it = tid + k * NT;
            const int r = it >> 4, w = (it & 15) * 2;
            const int row = r0 + r;
            if (it < ITEMS && row < M) {
              const int2 sp = meta[r];
              const int jp = hb * 32 + w;  // head dimension of the first pair
              const float2 lo = *(const float2*)(Tc + r * LDW + w);
              const float2 hi = *(const float2*)(Tc + r * LDW + 32 + w);
              const float4 cs = ep.rope
                                    ? *(const float4*)(ep.rope + ((size_t)sp.y * 64 + jp) * 2)
                                    : make_float4(1.f, 0.f, 1.f, 0.f);
              bf16_t* dst = hix < nq ? ep.q + (size_t)row * nq * 128 + (size_t)hix * 128
                                     : ep.kc + (((size_t)sp.x * nkv + (hix - nq)) * Nseq + sp.y) *
                                                   128;
              *(uint32_t*)(dst + jp) =
                  f2bf2(lo.x * cs.x - hi.x * cs.y, lo.y * cs.z - hi.y * cs.w);
              *(uint32_t*)(dst + 64 + jp) =
                  f2bf2(lo.x * cs.y + hi.x * cs.x, lo.y * cs.w + hi.y * cs.z);
            }
          }
        } else {
          // V head, stored transposed: item = (row quad, chunk column w),
          // row quads fastest so that a wave's stores go to consecutive
          // positions of one V^T row (one head-dimension column)
          const int gv = hix - nq - nkv;
          constexpr int QN = PR / 4;  // row quads per pass
          constexpr int ITEMS = QN * 64, ITER = (ITEMS + NT - 1) / NT;
#pragma unroll
          for (int k = 0; k < ITER; ++k) {
            const int it = tid + k * NT;
            const int w = it / QN, r4 = (it - w * QN) * 4;
            const int c = (w & 32) * 2 + hb * 32 + (w & 31);  // head dimension
            const int row = r0 + r4;
            if (it < ITEMS && row < M) {
              int2 sp[4];
              float v[4];
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                sp[t] = meta[r4 + t];
                v[t] = Tc[(r4 + t) * LDW + w];
              }
              const bool packed = row + 3 < M && (Nseq & 3) == 0 && (sp[0].y & 3) == 0 &&
                                  sp[3].x == sp[0].x && sp[3].y == sp[0].y + 3 &&
                                  sp[1].x == sp[0].x && sp[1].y == sp[0].y + 1 &&
                                  sp[2].x == sp[0].x && sp[2].y == sp[0].y + 2;
              if (packed) {
                uint2 u;
                u.x = f2bf2(v[0], v[1]);
                u.y = f2bf2(v[2], v[3]);
                *(uint2*)(ep.vc + (((size_t)sp[0].x * nkv + gv) * 128 + c) * Nseq + sp[0].y) = u;
              } else {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                  if (row + t < M)
                    ep.vc[(((size_t)sp[t].x * nkv + gv) * 128 + c) * Nseq + sp[t].y] =
                        f2bf(v[t]);
              }
            }
          }
        }
      }
    };
    static_for<WAVES_M / WMP>(pass);
  } else if constexpr (EPI == kEpiLogitsStats) {
    // Logits stored as for kEpiLogits.  Per row: the lane folds its TN
    // columns (increasing column order) into a partial, the 16 lanes that
    // hold the row merge by xor shuffles, the WAVES_N waves of a tile row
    // merge through LDS (in wave order); one partial per (row, column tile).
    // The rows' (slot, has_prev, lse_prev) are staged in LDS once per tile,
    // and the previous logits of row block i+1 are loaded while block i is
    // folded.
    struct RowMeta {
      long long slot;
      int hp;
      float lsep;
    };
    static_assert(!SPLIT, "the statistics epilogue needs complete sums");
    constexpr size_t kRedBytes = (size_t)BM * WAVES_N * sizeof(VocabPart);
    static_assert(kRedBytes % 16 == 0, "row metadata alignment");
    static_assert(kRedBytes + BM * sizeof(RowMeta) <= (size_t)STAGES * STAGE_BYTES,
                  "statistics staging must fit the operand ring");
    __syncthreads();  // every wave is done with the operand ring
    VocabPart* red = (VocabPart*)smem;                // [BM][WAVES_N]
    RowMeta* meta = (RowMeta*)(smem + kRedBytes);     // [BM]
    for (int t = tid; t < BM; t += 64 * NW) {
      const int rr = min(m0 + t, M - 1);
      const size_t slot = (size_t)ep.row_seq[rr] * ep.seq_len + ep.row_pos[rr];
      const int hp = ep.has_prev[slot];
      meta[t] = RowMeta{(long long)slot, hp, hp ? ep.lse_prev[slot] : 0.f};
    }
    __syncthreads();
    // previous logits of row block i (read whether or not the row has a
    // previous posterior: every slot is valid memory, unused values ignored)
    auto load_block = [&](auto I, float(&zp)[4][TN]) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float* prow = ep.zprev + (size_t)meta[wm * WM + i * 16 + rq + q].slot * N;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          // unconditional (a column past N reads the row's last entry and is
          // never folded): loads in a branch left the compiler unable to
          // count them, and it then waited for all of them at every use
          zp[q][j] = prow[min(n0 + brow(j) + cl, N - 1)];
        }
      }
    };
    float zpa[4][TN], zpb[4][TN];
    load_block(std::integral_constant<int, 0>{}, zpa);
    // one row block (16 rows) of the wave per call, expanded at compile time
    // (a plain unrolled loop over the row blocks exceeds the unroller's size
    // limit for the largest tiles, which would leave acc in scratch)
    auto row_block = [&](auto I, auto D) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      constexpr int kd = decltype(D)::value;  // KL direction whose sums are folded
      float(&cur)[4][TN] = pick<(i & 1) != 0>(zpa, zpb);
      float(&nxt)[4][TN] = pick<(i & 1) == 0>(zpa, zpb);
      if constexpr (i + 1 < TM) load_block(std::integral_constant<int, i + 1>{}, nxt);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rl = wm * WM + i * 16 + rq + q;
        const RowMeta mt = meta[rl];
        const bool hp = mt.hp != 0;
        VocabPart a = vpart_empty();
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = n0 + brow(j) + cl;
          if (col < N) {
            const float zv = (col == ep.mask_id) ? -INFINITY : acc[i][j][q];
            vpart_visit<kd>(a, col, zv, cur[q][j], hp, mt.lsep, ep.mask_id);
          }
        }
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) a = vmerge(a, vpart_shfl_xor(a, o));
        if (cl == 0) red[rl * WAVES_N + wn] = a;
      }
      // keep loads of later row blocks from being hoisted above this point
      // (register pressure of the large tiles)
      asm volatile("" ::: "memory");
    };
    // one instance per KL direction: the reverse direction's extra
    // exponential per logit is spent only when it is asked for
    auto rows_fwd = [&](auto I) __attribute__((always_inline)) {
      row_block(I, std::integral_constant<int, 0>{});
    };
    auto rows_rev = [&](auto I) __attribute__((always_inline)) {
      row_block(I, std::integral_constant<int, 1>{});
    };
    if (ep.kl_dir == 0)
      static_for<TM>(rows_fwd);
    else
      static_for<TM>(rows_rev);
    // The logits are stored only now, after every row block is folded:
    // loads and stores share the vector-memory counter, so a store issued
    // between the previous-logit loads made every later wait for a load
    // also wait for that store to complete (one round trip per row block).
    // (row blocks expanded at compile time, as above)
    auto store_rows = [&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rl = wm * WM + i * 16 + rq + q;
        if (m0 + rl < M) {
          float* zrow = (float*)ep.C + (size_t)meta[rl].slot * N;
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int col = n0 + brow(j) + cl;
            if (col < N) zrow[col] = (col == ep.mask_id) ? -INFINITY : acc[i][j][q];
          }
        }
      }
    };
    static_for<TM>(store_rows);
    __syncthreads();
    for (int t = tid; t < BM; t += 64 * NW) {
      const int row = m0 + t;
      if (row < M) {
        VocabPart a = red[t * WAVES_N];
#pragma unroll
        for (int w = 1; w < WAVES_N; ++w) a = vmerge(a, red[t * WAVES_N + w]);
        ep.parts[(size_t)row * tiles_n + nt] = a;
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
      } else if constexpr (EPI == kEpiResidAdd) {
        // h += acc: the row block's loads first, then the adds and stores
        // (element by element, every load would wait for the store before
        // it, which may alias as far as the compiler can tell)
        float* C = (float*)ep.C;
        float hv[TN][4];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = n0 + brow(j) + cl;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = m0 + wm * WM + i * 16 + rq + q;
            hv[j][q] = (col < N && row < M) ? C[(size_t)row * N + col] : 0.f;
          }
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = n0 + brow(j) + cl;
          if (col >= N) continue;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = m0 + wm * WM + i * 16 + rq + q;
            if (row < M) C[(size_t)row * N + col] = hv[j][q] + acc[i][j][q];
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
// Tile configurations (rows x cols, waves, k-slices in the LDS ring, k-slice
// width).  The plan picks the configuration by M (the ragged active-row
// count) and splits K while the grid would leave CUs idle.
namespace {

struct TileCfg {
  int bm, bn, wm, wn, stages, bk;
  bool pf = false;  // fragment prefetch over a 3-slot ring
};
constexpr TileCfg kCfgs[] = {
    {32, 128, 1, 4, 4, 64},   // 0: weight streaming
    {64, 128, 2, 2, 4, 64},   // 1: weight streaming
    {128, 128, 2, 2, 3, 64},  // 2
    {128, 256, 2, 2, 3, 64},  // 3
    {256, 128, 2, 2, 3, 64},  // 4
    {192, 128, 2, 2, 3, 64},  // 5
    {96, 128, 1, 4, 3, 64},   // 6
    {32, 64, 1, 4, 4, 64},    // 7: narrow column tiles (not for SwiGLU)
    {128, 128, 2, 4, 3, 64},  // 8: 8 waves
    {256, 128, 4, 2, 3, 64},  // 9: 8 waves
    {128, 256, 2, 4, 3, 64},  // 10: 8 waves
    {128, 128, 2, 2, 2, 64},  // 11: two workgroups per CU
    {192, 128, 2, 2, 2, 64},  // 12: two workgroups per CU
    {256, 256, 2, 4, 2, 64},  // 13: 8 waves, 128x64 per wave
    {64, 64, 2, 2, 4, 64},    // 14
    {192, 128, 4, 1, 2, 64},  // 15: one head per wave
    {128, 128, 4, 1, 3, 64},  // 16: one head per wave
    {256, 128, 4, 1, 2, 64},  // 17: one head per wave
    {64, 128, 4, 1, 4, 64},   // 18: one head per wave
    {64, 128, 2, 2, 8, 32},   // 19: weight streaming, 7 slices in flight
    {64, 64, 2, 2, 8, 32},    // 20: weight streaming, 7 slices in flight
    {64, 128, 4, 1, 8, 32},   // 21: one head per wave, 7 slices in flight
    {384, 128, 4, 2, 5, 32},  // 22: 8 waves
    {192, 128, 2, 2, 4, 64},  // 23
    {192, 256, 2, 4, 2, 64},  // 24: 8 waves, 96x64 per wave
    {384, 128, 4, 2, 2, 64},  // 25: 8 waves, 96x64 per wave
    {128, 256, 2, 4, 2, 64},  // 26: 8 waves, 64x64 per wave
    {192, 192, 2, 4, 2, 64},  // 27: 8 waves, 96x48 per wave (not for SwiGLU)
    {192, 128, 2, 4, 3, 64},  // 28: 8 waves, 2 slices in flight
    {192, 128, 2, 4, 4, 64},  // 29: 8 waves, 3 slices in flight
    {192, 128, 4, 1, 3, 64},  // 30: one head per wave, 2 slices in flight
    {192, 128, 4, 1, 4, 64},  // 31: one head per wave, 3 slices in flight
    {128, 128, 4, 1, 2, 64},  // 32: one head per wave, two workgroups per CU
    {192, 192, 4, 2, 2, 64},  // 33: 8 waves, 48x96 per wave
    {192, 192, 2, 2, 2, 64},  // 34: 96x96 per wave
    {192, 192, 4, 2, 3, 64, true},  // 35: 33 with fragment prefetch
    {192, 128, 2, 4, 3, 64, true},  // 36: 28 with fragment prefetch
    {256, 128, 4, 2, 3, 64, true},  // 37: 9 with fragment prefetch
    {128, 128, 2, 4, 3, 64, true},  // 38: 8 with fragment prefetch
    {128, 256, 2, 4, 3, 64, true},  // 39: 10 with fragment prefetch
    {96, 192, 2, 2, 3, 64, true},   // 40: 48x96 per wave, fragment prefetch
    {64, 192, 2, 2, 3, 64, true},   // 41: 32x96 per wave, fragment prefetch
    {128, 192, 2, 4, 3, 64, true},  // 42: 8 waves, 64x48 per wave, fragment prefetch
    {128, 192, 4, 2, 3, 64, true},  // 43: 8 waves, 32x96 per wave, fragment prefetch
    {96, 192, 2, 2, 3, 64},         // 44: 40 without fragment prefetch
    {96, 192, 2, 6, 3, 64, true},   // 45: 12 waves, 48x32 per wave, fragment prefetch
    {192, 192, 4, 3, 3, 64},        // 46: 12 waves, 48x64 per wave
    {192, 128, 3, 4, 3, 64, true},  // 47: 12 waves, 64x32 per wave, fragment prefetch
    {192, 128, 6, 2, 3, 64, true},  // 48: 12 waves, 32x64 per wave, fragment prefetch
    {128, 192, 4, 3, 3, 64, true},  // 49: 12 waves, 32x64 per wave, fragment prefetch
    {256, 192, 4, 3, 2, 64},        // 50: 12 waves, 64x64 per wave
};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);
constexpr bool cfgs_fit_lds() {
  for (const TileCfg& c : kCfgs)
    if ((size_t)c.stages * (c.bm + c.bn) * c.bk * 2 > 160 * 1024) return false;
  return true;
}
static_assert(cfgs_fit_lds(), "every tile configuration must fit the 160 KB of LDS of a CU");
constexpr int kBK = 64;  // K granularity every configuration accepts
constexpr size_t kSplitCapBytes = 64ull << 20;  // split-K partials never exceed this
constexpr int kCUs = 256;

inline size_t cfg_lds(const TileCfg& c) { return (size_t)c.stages * (c.bm + c.bn) * c.bk * 2; }

struct Plan {
  bool mfma;
  int cfg, tiles_m, tiles_n, splits, k_per_split;
  size_t ws;
  bool defer_reduce;  // split-K partials are left for the consumer kernel
};

// Default configuration by GEMM class and M bucket, from sweeps of the
// configurations on MI355X at the LLaDA-8B shapes (QKV 4096->12288, O
// 4096->4096, gate/up 4096->2x12288, down 12288->4096, LM head
// 4096->126464) with the weights streamed from HBM: small M favours narrow
// row tiles that stream the weights with many workgroups; from M ~ 192 to
// 512, 8-wave tiles with fragment prefetch that give every CU one workgroup
// (gate/up 192x192 at M = 384: 2 x 128 tiles; 128x192 at 128 < M <= 256:
// 2 x 128 tiles, 4-13% ahead of the 192x128 and 256x128 tiles there); large M
// favours 256x256 tiles with 8 waves.  The loop is bound by latency more than
// by LDS bandwidth, so three waves per SIMD pay where the registers allow:
// gate/up at 256 < M <= 384 runs the 12-wave 192x192 tile without prefetch
// (4-5% ahead of the 8-wave prefetch tile at M = 288-320, 3% in the engine at
// M = 384), gate/up at 128 < M <= 256 the 12-wave 128x192 prefetch tile (2-5%
// ahead of 8 waves), O at 256 < M <= 384 and down at 256 < M <= 320 the
// 12-wave 192x128 prefetch tile (1-4% ahead; level for down at M = 384), and
// gate/up at 384 < M <= 1536 the 12-wave 256x192 tile (one workgroup per CU
// at M = 512; 10-16% ahead of 256x256, which wins again from M = 2048).
int pick_cfg(int M, int N, int K, bool dual) {
  static const int kBucket[] = {16, 32, 64, 128, 192, 256, 320, 384, 512, 1536};
  static const int kNarrow[] = {7, 7, 1, 1, 6, 8, 47, 47, 8, 13, 13};
  static const int kNarrowDeep[] = {7, 7, 1, 1, 6, 8, 47, 36, 37, 13, 13};  // K >= 8192
  static const int kMedium[] = {7, 7, 14, 1, 6, 8, 5, 5, 37, 13, 13};
  static const int kDual[] = {1, 1, 1, 8, 49, 49, 46, 46, 50, 50, 13};
  static const int kWide[] = {7, 7, 14, 10, 12, 13, 25, 25, 13, 13, 13};
  int b = 0;
  while (b < 10 && M > kBucket[b]) ++b;
  if (dual) return kDual[b];
  if (N <= 8192) return K >= 8192 ? kNarrowDeep[b] : kNarrow[b];
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

// Large-M plans of the single-output GEMMs pick the 8-wave 256x256 tile,
// one workgroup per CU.  When that grid does not split K and its last round
// of workgroups leaves many CUs idle (the Dream-7B projections, N = 3584:
// 14 column tiles, so 336 workgroups at M = 6144, 1.31 rounds), the 12-wave
// 256x192 tile is taken instead if it scores higher on fill (workgroups over
// the CU slots of the rounds they need) per byte pulled per FLOP (1/bm +
// 1/bn).  Measured there with the weights cold: O 228.8 -> 181.6 us, down
// 980 -> 864 us at M = 6144; at M = 3792 (210 workgroups, one round) the
// 256x256 tile stays ahead and is kept.
int tile_grid(int c, int M, int N) {
  return ((M + kCfgs[c].bm - 1) / kCfgs[c].bm) * ((N + kCfgs[c].bn - 1) / kCfgs[c].bn);
}

// Fill of the rounds a grid of tile c needs (its workgroups over the
// resident slots of those rounds) per byte pulled into the CUs per FLOP
// (1/bm + 1/bn): larger is better.
double fill_score(int c, int M, int N) {
  const int slots = kCUs * (cfg_lds(kCfgs[c]) <= 80 * 1024 ? 2 : 1);
  const int w = tile_grid(c, M, N);
  const double fill = (double)w / (((w + slots - 1) / slots) * slots);
  return fill / (1.0 / kCfgs[c].bm + 1.0 / kCfgs[c].bn);
}

int refine_wide_cfg(int cfg, int M, int N) {
  constexpr int kWideTile = 13, kWideAlt = 50;
  if (cfg != kWideTile) return cfg;
  if (tile_grid(kWideTile, M, N) * 2 <= kCUs) return cfg;  // the plan splits K to fill the CUs
  return fill_score(kWideAlt, M, N) > fill_score(kWideTile, M, N) ? kWideAlt : kWideTile;
}

// gate/up + SwiGLU above M = 384: the tile with the best fill_score over
// the 2 d_ff output columns among 256x192, 256x256 and the 12-wave 192x192
// (the first on ties).  Swept with the weights cold it picked the fastest
// tile at every point at the LLaDA-8B width (M = 512 .. 4096; M = 768: 130
// against 172 us for 256x192) and the Dream-7B width (M = 700 .. 6144;
// M = 700: 185 against 233 us).  At M <= 384 the table from the engine A/Bs
// stands.
int pick_dual_cfg(int cfg, int M, int N) {
  if (M <= 384) return cfg;
  static const int kCand[] = {50, 13, 46};
  int best = kCand[0];
  for (int c : kCand)
    if (fill_score(c, M, 2 * N) > fill_score(best, M, 2 * N)) best = c;
  return best;
}

Plan make_plan(int dtype, int epi, int M, int N, int K) {
  const bool dual = epi == kEpiSwiglu;
  int cfg = pick_cfg(M, N, K, dual);
  cfg = dual ? pick_dual_cfg(cfg, M, N) : refine_wide_cfg(cfg, M, N);
  return make_plan_cfg(dtype, epi, M, N, K, cfg);
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int BK, int EPI, bool PF = false>
hipError_t run_mfma(const GemmArgs& a, const Plan& p, EpiParams ep, void* ws, hipStream_t s) {
  constexpr bool DUAL = EPI == kEpiSwiglu;
  if constexpr (DUAL && ((BN / WAVES_N / 16) % 2 != 0)) {
    return hipErrorInvalidValue;  // a dual tile needs matching gate/up column tiles per wave
  } else if constexpr (EPI == kEpiQKV &&
                       (BN % 64 != 0 ||
                        qkv_wave_rows_per_pass(WAVES_M, BM / WAVES_M, (BN + 4) * 4 + 8,
                                               STAGES * (BM + BN) * BK * 2) == 0)) {
    // the fused QKV epilogue works on 64-column chunks and stages at least
    // one wave row of the tile in the LDS ring
    return hipErrorInvalidValue;
  } else {
    dim3 grid(p.tiles_m * p.tiles_n, p.splits, 1);
    const int threads = 64 * WAVES_M * WAVES_N;
    const size_t lds = (size_t)STAGES * (BM + BN) * BK * 2;
    float* partial = (float*)ws;
    if constexpr (EPI == kEpiLogitsStats) {
      if (p.splits > 1) return hipErrorInvalidValue;  // the epilogue needs complete sums
    }
    if (p.splits > 1) {
      if constexpr (EPI != kEpiLogitsStats) {
        static bool attr = false;
        if (!attr) {
          (void)hipFuncSetAttribute(
              reinterpret_cast<const void*>(
                  &gemm_bf16_mfma_kernel<BM, BN, WAVES_M, WAVES_N, STAGES, BK, EPI, true, PF>),
              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
          attr = true;
        }
        gemm_bf16_mfma_kernel<BM, BN, WAVES_M, WAVES_N, STAGES, BK, EPI, true, PF>
            <<<grid, threads, lds, s>>>((const bf16_t*)a.A, (const bf16_t*)a.W,
                                        (const bf16_t*)a.W2, ep, a.K, p.k_per_split, p.tiles_m,
                                        p.tiles_n, partial);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const size_t total = (size_t)a.M * a.N;
        const int g = (int)std::min<size_t>((total + 255) / 256, 8192);
        if (!p.defer_reduce)
          splitk_reduce_kernel<EPI, bf16_t><<<g, 256, 0, s>>>(partial, p.splits, ep);
      }
    } else {
      static bool attr = false;
      if (!attr) {
        (void)hipFuncSetAttribute(
            reinterpret_cast<const void*>(
                &gemm_bf16_mfma_kernel<BM, BN, WAVES_M, WAVES_N, STAGES, BK, EPI, false, PF>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        attr = true;
      }
      gemm_bf16_mfma_kernel<BM, BN, WAVES_M, WAVES_N, STAGES, BK, EPI, false, PF>
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
    case 0: return run_mfma<32, 128, 1, 4, 4, 64, EPI>(a, p, ep, ws, s);
    case 1: return run_mfma<64, 128, 2, 2, 4, 64, EPI>(a, p, ep, ws, s);
    case 2: return run_mfma<128, 128, 2, 2, 3, 64, EPI>(a, p, ep, ws, s);
    case 3: return run_mfma<128, 256, 2, 2, 3, 64, EPI>(a, p, ep, ws, s);
    case 4: return run_mfma<256, 128, 2, 2, 3, 64, EPI>(a, p, ep, ws, s);
    case 5: return run_mfma<192, 128, 2, 2, 3, 64, EPI>(a, p, ep, ws, s);
    case 6: return run_mfma<96, 128, 1, 4, 3, 64, EPI>(a, p, ep, ws, s);
    case 7: return run_mfma<32, 64, 1, 4, 4, 64, EPI>(a, p, ep, ws, s);
    case 8: return run_mfma<128, 128, 2, 4, 3, 64, EPI>(a, p, ep, ws, s);
    case 9: return run_mfma<256, 128, 4, 2, 3, 64, EPI>(a, p, ep, ws, s);
    case 10: return run_mfma<128, 256, 2, 4, 3, 64, EPI>(a, p, ep, ws, s);
    case 11: return run_mfma<128, 128, 2, 2, 2, 64, EPI>(a, p, ep, ws, s);
    case 12: return run_mfma<192, 128, 2, 2, 2, 64, EPI>(a, p, ep, ws, s);
    case 13: return run_mfma<256, 256, 2, 4, 2, 64, EPI>(a, p, ep, ws, s);
    case 14: return run_mfma<64, 64, 2, 2, 4, 64, EPI>(a, p, ep, ws, s);
    case 15: return run_mfma<192, 128, 4, 1, 2, 64, EPI>(a, p, ep, ws, s);
    case 16: return run_mfma<128, 128, 4, 1, 3, 64, EPI>(a, p, ep, ws, s);
    case 17: return run_mfma<256, 128, 4, 1, 2, 64, EPI>(a, p, ep, ws, s);
    case 18: return run_mfma<64, 128, 4, 1, 4, 64, EPI>(a, p, ep, ws, s);
    case 19: return run_mfma<64, 128, 2, 2, 8, 32, EPI>(a, p, ep, ws, s);
    case 20: return run_mfma<64, 64, 2, 2, 8, 32, EPI>(a, p, ep, ws, s);
    case 21: return run_mfma<64, 128, 4, 1, 8, 32, EPI>(a, p, ep, ws, s);
    case 22: return run_mfma<384, 128, 4, 2, 5, 32, EPI>(a, p, ep, ws, s);
    case 23: return run_mfma<192, 128, 2, 2, 4, 64, EPI>(a, p, ep, ws, s);
    case 24: return run_mfma<192, 256, 2, 4, 2, 64, EPI>(a, p, ep, ws, s);
    case 25: return run_mfma<384, 128, 4, 2, 2, 64, EPI>(a, p, ep, ws, s);
    case 26: return run_mfma<128, 256, 2, 4, 2, 64, EPI>(a, p, ep, ws, s);
    case 27: return run_mfma<192, 192, 2, 4, 2, 64, EPI>(a, p, ep, ws, s);
    case 28: return run_mfma<192, 128, 2, 4, 3, 64, EPI>(a, p, ep, ws, s);
    case 29: return run_mfma<192, 128, 2, 4, 4, 64, EPI>(a, p, ep, ws, s);
    case 30: return run_mfma<192, 128, 4, 1, 3, 64, EPI>(a, p, ep, ws, s);
    case 31: return run_mfma<192, 128, 4, 1, 4, 64, EPI>(a, p, ep, ws, s);
    case 32: return run_mfma<128, 128, 4, 1, 2, 64, EPI>(a, p, ep, ws, s);
    case 33: return run_mfma<192, 192, 4, 2, 2, 64, EPI>(a, p, ep, ws, s);
    case 34: return run_mfma<192, 192, 2, 2, 2, 64, EPI>(a, p, ep, ws, s);
    case 35: return run_mfma<192, 192, 4, 2, 3, 64, EPI, true>(a, p, ep, ws, s);
    case 36: return run_mfma<192, 128, 2, 4, 3, 64, EPI, true>(a, p, ep, ws, s);
    case 37: return run_mfma<256, 128, 4, 2, 3, 64, EPI, true>(a, p, ep, ws, s);
    case 38: return run_mfma<128, 128, 2, 4, 3, 64, EPI, true>(a, p, ep, ws, s);
    case 39: return run_mfma<128, 256, 2, 4, 3, 64, EPI, true>(a, p, ep, ws, s);
    case 40: return run_mfma<96, 192, 2, 2, 3, 64, EPI, true>(a, p, ep, ws, s);
    case 41: return run_mfma<64, 192, 2, 2, 3, 64, EPI, true>(a, p, ep, ws, s);
    case 42: return run_mfma<128, 192, 2, 4, 3, 64, EPI, true>(a, p, ep, ws, s);
    case 43: return run_mfma<128, 192, 4, 2, 3, 64, EPI, true>(a, p, ep, ws, s);
    case 45: return run_mfma<96, 192, 2, 6, 3, 64, EPI, true>(a, p, ep, ws, s);
    case 46: return run_mfma<192, 192, 4, 3, 3, 64, EPI>(a, p, ep, ws, s);
    case 47: return run_mfma<192, 128, 3, 4, 3, 64, EPI, true>(a, p, ep, ws, s);
    case 48: return run_mfma<192, 128, 6, 2, 3, 64, EPI, true>(a, p, ep, ws, s);
    case 49: return run_mfma<128, 192, 4, 3, 3, 64, EPI, true>(a, p, ep, ws, s);
    case 50: return run_mfma<256, 192, 4, 3, 2, 64, EPI>(a, p, ep, ws, s);
    default: return run_mfma<96, 192, 2, 2, 3, 64, EPI>(a, p, ep, ws, s);
  }
}

// The statistics epilogue is instantiated for every configuration pick_cfg
// returns for a non-dual GEMM, plus tile 24 for sweeps.
hipError_t dispatch_logits_stats(const GemmArgs& a, const Plan& p, EpiParams ep, hipStream_t s) {
  constexpr int E = kEpiLogitsStats;
  switch (p.cfg) {
    case 1: return run_mfma<64, 128, 2, 2, 4, 64, E>(a, p, ep, nullptr, s);
    case 5: return run_mfma<192, 128, 2, 2, 3, 64, E>(a, p, ep, nullptr, s);
    case 6: return run_mfma<96, 128, 1, 4, 3, 64, E>(a, p, ep, nullptr, s);
    case 7: return run_mfma<32, 64, 1, 4, 4, 64, E>(a, p, ep, nullptr, s);
    case 8: return run_mfma<128, 128, 2, 4, 3, 64, E>(a, p, ep, nullptr, s);
    case 9: return run_mfma<256, 128, 4, 2, 3, 64, E>(a, p, ep, nullptr, s);
    case 10: return run_mfma<128, 256, 2, 4, 3, 64, E>(a, p, ep, nullptr, s);
    case 12: return run_mfma<192, 128, 2, 2, 2, 64, E>(a, p, ep, nullptr, s);
    case 13: return run_mfma<256, 256, 2, 4, 2, 64, E>(a, p, ep, nullptr, s);
    case 14: return run_mfma<64, 64, 2, 2, 4, 64, E>(a, p, ep, nullptr, s);
    case 24: return run_mfma<192, 256, 2, 4, 2, 64, E>(a, p, ep, nullptr, s);
    case 25: return run_mfma<384, 128, 4, 2, 2, 64, E>(a, p, ep, nullptr, s);
    case 28: return run_mfma<192, 128, 2, 4, 3, 64, E>(a, p, ep, nullptr, s);
    default: return hipErrorInvalidValue;
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

EpiParams epi_params(const GemmArgs& a) {
  return EpiParams{a.C,  a.M,   a.N,  a.row_seq, a.row_pos, a.seq_len,  a.mask_id,
                   a.rope, (bf16_t*)a.q, (bf16_t*)a.kc, (bf16_t*)a.vc, a.nq, a.nkv,
                   a.zprev, a.lse_prev, a.has_prev, (VocabPart*)a.parts, a.kl_dir};
}

hipError_t launch_plan(const GemmArgs& a, Plan p, void* ws, size_t ws_bytes, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  EpiParams ep = epi_params(a);
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
  return dtype == kBF16 && hd == 128 && K % kBK == 0 && M >= 1;
}

// Tile for the fused QKV epilogue by M, from a sweep of the configurations
// at the LLaDA-8B shape (d 4096 -> 12288); at every M it beat the plain GEMM
// followed by the separate rotary / scatter kernels.  The 192-column tiles
// give 4 x 64 = 256 workgroups at M = 384 and 512 where 128-column tiles give
// 192, but run each tile less efficiently (4 waves, or 48-column wave tiles),
// so they gain only 2-9%; 64-column (half-head) tiles stream the weights with
// twice the workgroups at M <= 64 (13-22% faster there).
int pick_qkv_cfg(int M, int N) {
  if (M <= 32) return 7;    // 32x64, 4 waves: weight streaming, 192 half-head column tiles
  if (M <= 64) return 14;   // 64x64
  if (M <= 128) return 1;   // 64x128
  if (M <= 192) return 6;   // 96x128
  if (M <= 256) return 8;   // 128x128, 8 waves
  if (M <= 384) return 45;  // 96x192, 12 waves, prefetch: 8-12% ahead of 4 waves
  if (M <= 512) return 42;  // 128x192, 8 waves, fragment prefetch
  // Larger M: the tile with the best fill per byte (fill_score) among the
  // 128x192, 96x192, 12-wave 192x192, 12-wave 256x192 and 128x128 tiles (the
  // first on ties).  Against the weights cold, that rule picked the fastest
  // tile, or one within 2% of it, at every point measured: the LLaDA-8B
  // width (12288 columns) at M = 768 .. 12288 and the Dream-7B width (4608)
  // at M = 700 .. 6144, where the 128x192 tile alone ran up to 1.4x slower
  // (Dream-7B at M = 1392: 85.7 against 59.9 us).
  static const int kCand[] = {42, 45, 46, 50, 8};
  int best = kCand[0];
  for (int c : kCand)
    if (fill_score(c, M, N) > fill_score(best, M, N)) best = c;
  return best;
}

hipError_t launch_gemm(const GemmArgs& a, void* ws, size_t ws_bytes, hipStream_t s) {
  if (a.epi == kEpiQKV)
    return launch_plan(a, make_plan_cfg(a.dtype, a.epi, a.M, a.N, a.K, pick_qkv_cfg(a.M, a.N)), ws,
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

bool gemm_logits_stats_fusable(int dtype, int K) {
  return dtype == kBF16 && K % kBK == 0 && K >= kBK;
}

namespace {
// Tile of the fused LM head by M: the 4-wave 192x128 tile (two workgroups per
// CU, so one workgroup's epilogue overlaps the other's main loop) for
// 256 < M <= 384, else the plain LM-head choice.
int pick_logits_stats_cfg(int M, int N, int K) {
  if (M > 256 && M <= 384) return 12;
  const int c = pick_cfg(M, N, K, false);
  // the statistics epilogue is not built for the fragment-prefetch tiles:
  // their plain twins
  switch (c) {
    case 35: return 13;
    case 36: return 28;
    case 37: return 9;
    case 38: return 8;
    case 39: return 10;
    default: return c;
  }
}

Plan logits_stats_plan(int M, int N, int K, int cfg) {
  Plan p = make_plan_cfg(kBF16, kEpiLogitsStats, M, N, K,
                         cfg >= 0 ? cfg : pick_logits_stats_cfg(M, N, K));
  p.splits = 1;  // the epilogue needs complete sums
  p.k_per_split = K;
  p.ws = 0;
  return p;
}
}  // namespace

// Measured at V = 126464, d = 4096 against the LM head followed by the
// separate statistics kernel: in the fused form every workgroup reads the
// previous logits in its epilogue at about the same time, with the MFMA units
// idle, so it is ahead only where the GEMM is short of tiles or runs two
// workgroups per CU: M <= 64 and 256 < M <= 384.
bool gemm_logits_stats_preferred(int M, int N) {
  (void)N;
  return M <= 64 || (M > 256 && M <= 384);
}

int gemm_logits_stats_parts(int M, int N, int K, int cfg) {
  if (M <= 0 || (cfg >= kNumCfgs)) return 0;
  return logits_stats_plan(M, N, K, cfg).tiles_n;
}

size_t gemm_logits_stats_bytes(int dtype, int M, int N, int K) {
  if (!gemm_logits_stats_fusable(dtype, K) || M <= 0) return 0;
  return (size_t)M * gemm_logits_stats_parts(M, N, K, -1) * sizeof(VocabPart);
}

hipError_t launch_gemm_logits_stats(const GemmArgs& a, int cfg, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (!gemm_logits_stats_fusable(a.dtype, a.K) || cfg >= kNumCfgs) return hipErrorInvalidValue;
  return dispatch_logits_stats(a, logits_stats_plan(a.M, a.N, a.K, cfg), epi_params(a), s);
}

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

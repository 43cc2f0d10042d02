// Attention of the M active queries over all N cached positions.
//
// SureLock page ("Stopping Computation for Converged Tokens in Masked
// Diffusion-LM Decoding"), §2 Methodology, continued attention: active
// (unlocked) tokens still attend to the locked ones through their cached K/V
// while fresh Q/K/V exist only for the active subset; attention cost is
// O(M_t N d) (§2 algorithmic complexity).  Non-causal: every query sees every
// position of its sequence.  §5 names fused kernels and a contiguous cache
// layout as the way to turn the FLOP saving into wall-clock; the cache here
// is head-major: K as [seq][kv head][pos][hd] and V transposed as
// [seq][kv head][hd][pos], so one (seq, kv head) is two contiguous N x hd
// slabs that a workgroup streams through LDS with plain 16-byte loads.
//
// MFMA kernel (bf16, hd in {64, 128}): a workgroup owns 64 query vectors of
// one (seq, kv head) -- (row, query head) pairs, so GQA groups share the K/V
// stream -- 16 per wave, and walks the keys in tiles of 64:
//   S^T = K Q^T   with v_mfma_f32_16x16x32_bf16 (K from LDS, Q in registers);
//                 lane l then holds S[key 4(l/16)+i][query l%16];
//   online softmax per query column (exp2 domain, max/sum over the 4 lanes
//                 sharing l%16);
//   O^T += V^T P^T with v_mfma_f32_16x16x16_bf16: the S^T registers are
//                 already the B operand; V^T rows (keys contiguous) come
//                 straight from the transposed cache.
// Split-KV (gridDim.z > 1) writes unnormalised partials (o, max, sum) that a
// combine pass merges by log-sum-exp.
#include "common.h"
#include "internal.h"

namespace dlm {

constexpr int kAttnQ = 64;     // query vectors per workgroup
constexpr int kAttnKeys = 64;  // keys per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyMax = 8.f;  // log2 headroom before the running maximum is raised
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int HD, bool SPLIT>
__global__ __launch_bounds__(256) void attn_mfma_kernel(
    const bf16_t* __restrict__ q, const int32_t* __restrict__ row_start,
    const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc, bf16_t* __restrict__ o, int N,
    int nq, int nkv, int keys_per_split, int M, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  constexpr int KP = HD + 8;          // K tile pitch (elements)
  constexpr int VP = kAttnKeys + 8;   // V^T tile pitch (elements; rows 16-byte aligned)
  constexpr int NKC = HD / 32;        // 32-wide hd chunks for S
  constexpr int NCB = HD / 16;        // 16-wide hd blocks for O
  __shared__ __attribute__((aligned(16))) bf16_t sK[kAttnKeys * KP];
  __shared__ __attribute__((aligned(16))) bf16_t sVt[HD * VP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bg = blockIdx.y;
  const int b = bg / nkv, g = bg % nkv;
  const int G = nq / nkv;
  const int r0 = row_start[b], Mb = row_start[b + 1] - r0;
  const int Qn = Mb * G;
  const int qbase = blockIdx.x * kAttnQ;
  if (qbase >= Qn) return;

  // this lane's query vector (column l%16 of the wave's 16)
  const int qv = qbase + wave * 16 + (lane & 15);
  const bool qok = qv < Qn;
  const int row = r0 + (qok ? qv / G : 0);
  const int head = g * G + (qok ? qv % G : 0);
  bf16x8 qf[NKC];
  {
    const bf16_t* qp = q + (size_t)row * nq * HD + (size_t)head * HD + (lane >> 4) * 8;
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      if (qok) {
        qf[c] = *(const bf16x8*)(qp + c * 32);
      } else {
        const uint4 z = make_uint4(0, 0, 0, 0);
        qf[c] = *(const bf16x8*)&z;
      }
    }
  }

  const size_t slab = ((size_t)b * nkv + g) * N * HD;
  const bf16_t* kslab = kc + slab;   // [N][HD]
  const bf16_t* vslab = vc + slab;   // [HD][N]
  const int key0 = blockIdx.z * keys_per_split;
  const int key1 = min(N, key0 + keys_per_split);
  const float scale = kLog2e / sqrtf((float)HD);
  const bool vec_v = (N % 8) == 0;   // V^T rows 16-byte aligned

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 oacc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) oacc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int CH = kAttnKeys * HD / 8;  // 16-byte chunks per tile (K or V^T)
  for (int t0 = key0; t0 < key1; t0 += kAttnKeys) {
    __syncthreads();  // previous tile fully consumed
    for (int c = tid; c < CH; c += 256) {
      // K tile: 64 keys x HD
      const int kr = c / (HD / 8), cc = (c % (HD / 8)) * 8;
      uint4 kv = make_uint4(0, 0, 0, 0);
      if (t0 + kr < key1) kv = *(const uint4*)(kslab + (size_t)(t0 + kr) * HD + cc);
      *(uint4*)&sK[kr * KP + cc] = kv;
      // V^T tile: HD rows x 64 keys
      const int vr = c / (kAttnKeys / 8), vk = (c % (kAttnKeys / 8)) * 8;
      const bf16_t* vsrc = vslab + (size_t)vr * N + t0 + vk;
      uint4 vv = make_uint4(0, 0, 0, 0);
      if (vec_v && t0 + vk + 8 <= key1) {
        vv = *(const uint4*)vsrc;
      } else {
        bf16_t* ve = (bf16_t*)&vv;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (t0 + vk + j < key1) ve[j] = vsrc[j];
      }
      *(uint4*)&sVt[vr * VP + vk] = vv;
    }
    __syncthreads();

    // S^T for the 4 key blocks of this tile
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NKC; ++c) {
        const bf16x8 a =
            *(const bf16x8*)&sK[(kb * 16 + (lane & 15)) * KP + c * 32 + (lane >> 4) * 8];
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[c], s[kb], 0, 0, 0);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = t0 + kb * 16 + (lane >> 4) * 4 + i;
        const float v = key < key1 ? s[kb][i] * scale : -INFINITY;
        s[kb][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
    float psum = 0.f;
    s16x4 pb[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = (m_new == -INFINITY) ? 0.f : exp2f(s[kb][i] - m_new);
        psum += p;
        pb[kb][i] = (short)f2bf(p);
      }
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      oacc[cb] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const s16x4 va =
            *(const s16x4*)&sVt[(cb * 16 + (lane & 15)) * VP + kb * 16 + (lane >> 4) * 4];
        oacc[cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb[kb], oacc[cb], 0, 0, 0);
      }
    }
  }

  if (!qok) return;
  const int gq = row * nq + head;  // global query-vector id
  if (SPLIT) {
    const size_t base = (size_t)blockIdx.z * M * nq + gq;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        part_o[base * HD + cb * 16 + (lane >> 4) * 4 + i] = oacc[cb][i];
    if ((lane >> 4) == 0) {
      part_ml[base * 2] = m_run;
      part_ml[base * 2 + 1] = l_run;
    }
  } else {
    const float inv = 1.f / l_run;
    bf16_t* op = o + (size_t)row * nq * HD + (size_t)head * HD;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int c = cb * 16 + (lane >> 4) * 4;
      ushort4 w;
      w.x = f2bf(oacc[cb][0] * inv);
      w.y = f2bf(oacc[cb][1] * inv);
      w.z = f2bf(oacc[cb][2] * inv);
      w.w = f2bf(oacc[cb][3] * inv);
      *(ushort4*)(op + c) = w;
    }
  }
}

// DMA variant (N a multiple of the key tile KT = 64 or 128): K and V^T tiles
// go straight from global memory into a STAGES-deep LDS ring with
// global_load_lds_dwordx4, the next tiles in flight while the current one is
// consumed.  K tile rows (one key, HD elements) and V^T tile rows (one hd
// column, KT keys = 128 or 256 B) are stored with their 16-byte chunks
// XOR-swizzled by the row index so that the fragment reads hit distinct
// banks.
typedef __attribute__((address_space(3))) void attn_lds_void;
__device__ __forceinline__ void attn_dma16(const void* g, unsigned char* lds) {
  __builtin_amdgcn_global_load_lds(g, (attn_lds_void*)lds, 16, 0, 0);
}
// Slot XORs measured conflict-free on gfx950 (SQ_LDS_BANK_CONFLICT): 16-byte
// reads of 16 consecutive K rows at one chunk -> r & 15 (256-byte rows) or
// r & 7 (128-byte rows); 8-byte reads of 16 consecutive V^T rows ->
// (r & 7) ^ ((r >> 3) & 1).  (The compiler pairs V^T reads whose addresses
// differ by a multiple of 512 bytes into ds_read2st64_b64, whose two halves
// share banks; that pairing, not the XOR, leaves two-way conflicts there.)
__device__ __forceinline__ int kswz(int r, int chunks) { return chunks == 16 ? (r & 15) : (r & 7); }
__device__ __forceinline__ int vswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
// 256-byte V^T rows (128-key tiles): the 16 rows a fragment read touches get
// 16 distinct 16-byte slots of one chunk
__device__ __forceinline__ int vswz16(int r) { return r & 15; }
// Reductions over the lanes l, l^16, l^32, l^48 with the gfx950 lane-swap
// instructions: permlane16_swap(v, v) returns v from lanes l and l^16 in its
// two outputs, permlane32_swap(v, v) from lanes l and l^32.
__device__ __forceinline__ float xor16_max(float v) {
  const auto r =
      __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r =
      __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r =
      __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r =
      __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int N>
__device__ __forceinline__ void attn_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Waits until at most n (0 <= n < S) tiles of IPW load instructions each are
// still in flight for this wave.
template <int IPW, int S>
__device__ __forceinline__ void attn_wait_tiles(int n) {
  if constexpr (S <= 1) {
    attn_wait_vmcnt<0>();
  } else {
    if (n >= S - 1) attn_wait_vmcnt<(S - 1) * IPW>();
    else attn_wait_tiles<IPW, S - 1>(n);
  }
}
// Workgroup barrier without the vmcnt(0) of __syncthreads(); the empty asm
// statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void attn_lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wave layout: QW = 4 / QB query waves of 16 QB queries each, times KH key
// groups.  Wave (kh, qw) takes keys [kh * 64 / KH, (kh + 1) * 64 / KH) of
// every 64-key tile with its own online-softmax state per 16-query block; the
// KH states of a query block are merged through LDS at the end, in pairs.
// With QB = 2 every K and V^T fragment read from LDS feeds the MFMAs of two
// query blocks, which halves the LDS reads per query (the loop over key tiles
// is bound by LDS bandwidth and latency, not by HBM).
template <int HD, int KH, int QB>
constexpr size_t attn_merge_bytes() {
  return KH == 1 ? 0
                 : (size_t)(KH / 2) * (4 / QB) * (QB * (HD / 16) * 64 * 16 + QB * 64 * 8);
}

template <int HD, bool SPLIT, int STAGES, int KH, int QB, int KT>
__global__ __launch_bounds__(64 * (4 / QB) * KH) void attn_mfma_dma_kernel(
    const bf16_t* __restrict__ q, const int32_t* __restrict__ row_start,
    const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc, bf16_t* __restrict__ o, int N,
    int nq, int nkv, int keys_per_split, int M, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  static_assert(KH == 1 || KH == 2 || KH == 4, "key groups");
  static_assert(QB == 1 || QB == 2, "query blocks per wave");
  static_assert(KT == 64 || KT == 128, "key tile");
  constexpr int QW = 4 / QB;                        // query waves
  constexpr int NWV = QW * KH;                      // waves
  constexpr int NKB = KT / (16 * KH);               // 16-key blocks per wave per tile
  constexpr int NKC = HD / 32, NCB = HD / 16;
  constexpr int KCH = HD / 8;                       // 16-byte chunks per K row
  constexpr int VRB = KT * 2, VCH = VRB / 16;       // V^T row bytes, 16-byte chunks per row
  constexpr int K_BYTES = KT * HD * 2, V_BYTES = HD * KT * 2;
  constexpr int STAGE = K_BYTES + V_BYTES;
  constexpr int K_INSTR = K_BYTES / 1024, V_INSTR = V_BYTES / 1024;
  constexpr int IPW = (K_INSTR + V_INSTR) / NWV;    // per wave
  static_assert((K_INSTR + V_INSTR) % NWV == 0, "instructions per wave");
  static_assert((STAGES - 1) * IPW < 64, "in-flight loads must fit the vmcnt counter");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qw = wave % QW, kh = wave / QW;
  // XCD-aware order: workgroup i (x fastest) runs on XCD i % 8; give
  // consecutive workgroups of one XCD the query tiles of one (sequence,
  // kv head), which then read its K/V slab through that XCD's L2.
  const int nx = gridDim.x, ny = gridDim.y;
  const int total = nx * ny * gridDim.z;
  int lin = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  if ((total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);
  const int bx = lin % nx, by = (lin / nx) % ny, bz = lin / (nx * ny);
  const int bg = by;
  const int b = bg / nkv, g = bg % nkv;
  const int G = nq / nkv;
  const int r0 = row_start[b], Mb = row_start[b + 1] - r0;
  const int Qn = Mb * G;
  const int qbase = bx * kAttnQ;
  if (qbase >= Qn) return;  // uniform over the workgroup

  bool qok[QB];
  int row[QB], head[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qv = qbase + (qw * QB + qb) * 16 + (lane & 15);
    qok[qb] = qv < Qn;
    row[qb] = r0 + (qok[qb] ? qv / G : 0);
    head[qb] = g * G + (qok[qb] ? qv % G : 0);
  }
  const bool wave_live = qbase + qw * QB * 16 < Qn;  // wave-uniform
  const size_t slab = ((size_t)b * nkv + g) * N * HD;
  const bf16_t* kslab = kc + slab;  // [N][HD]
  const bf16_t* vslab = vc + slab;  // [HD][N]
  const int key0 = bz * keys_per_split;
  const int key1 = min(N, key0 + keys_per_split);
  const int ntiles = key1 > key0 ? (key1 - key0) / KT : 0;
  const float scale = kLog2e / sqrtf((float)HD);

  // this lane's global source for each of its DMA instructions (tile 0)
  const bf16_t* src[IPW];
  int dst[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int j = wave + i * NWV;
    if (j < K_INSTR) {
      const int kr = j * (1024 / (HD * 2)) + lane / KCH;       // key row in the tile
      const int lc = (lane % KCH) ^ kswz(kr, KCH);
      src[i] = kslab + (size_t)(key0 + kr) * HD + lc * 8;
      dst[i] = j * 1024;
    } else {
      const int jv = j - K_INSTR;
      const int vr = jv * (1024 / VRB) + lane / VCH;           // hd row of V^T
      const int lc = (lane % VCH) ^ (VCH == 16 ? vswz16(vr) : vswz(vr));
      src[i] = vslab + (size_t)vr * N + key0 + lc * 8;
      dst[i] = K_BYTES + jv * 1024;
    }
  }
  auto issue = [&](int t) {
    unsigned char* st = smem + (t % STAGES) * STAGE;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int j = wave + i * NWV;
      const size_t adv = j < K_INSTR ? (size_t)t * KT * HD : (size_t)t * KT;
      attn_dma16(src[i] + adv, st + dst[i]);
    }
  };

  float m_run[QB], l_run[QB];
  f32x4 oacc[QB][NCB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) oacc[qb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

#pragma unroll
  for (int t = 0; t < STAGES - 1; ++t)
    if (t < ntiles) issue(t);
  // the query fragments load while the first tiles are in flight
  bf16x8 qf[QB][NKC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const bf16_t* qp =
        q + (size_t)row[qb] * nq * HD + (size_t)head[qb] * HD + (lane >> 4) * 8;
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      if (qok[qb]) {
        qf[qb][c] = *(const bf16x8*)(qp + c * 32);
      } else {
        const uint4 z = make_uint4(0, 0, 0, 0);
        qf[qb][c] = *(const bf16x8*)&z;
      }
    }
  }

  const int kofs = kh * (KT / KH);  // first key of this wave in a tile
  for (int t = 0; t < ntiles; ++t) {
    // this wave's loads of tile t (later tiles may stay in flight), then
    // everyone's; every wave is done with tile t-1 after the barrier
    attn_wait_tiles<IPW, STAGES - 1>(min(STAGES - 2, ntiles - 1 - t));
    attn_lds_barrier();
    if (t + STAGES - 1 < ntiles) issue(t + STAGES - 1);
    if (!wave_live) continue;  // no query of this wave is valid: loads only
    const unsigned char* st = smem + (t % STAGES) * STAGE;
    f32x4 s[QB][NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = kofs + kb * 16 + (lane & 15);
#pragma unroll
      for (int c = 0; c < NKC; ++c) {
        const int lc = c * 4 + (lane >> 4);
        const bf16x8 a =
            *(const bf16x8*)(st + r * (HD * 2) + ((lc ^ kswz(r, KCH)) << 4));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[qb][c], s[qb][kb], 0, 0, 0);
      }
    }
    // Online softmax in base 2 on the scaled scores.  The running maximum of
    // a query is raised (and its accumulators rescaled) only when the tile
    // maximum exceeds it by more than kLazyMax; otherwise the exponentials
    // are taken against the stale maximum and stay below 2^kLazyMax.  The
    // normalised result is the same either way.
    s16x4 pb[QB][NKB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[qb][kb][i]);
      mx = xor16_max(mx);
      mx = xor32_max(mx);
      mx *= scale;
      if (__any(mx > m_run[qb] + kLazyMax)) {  // wave-uniform branch
        const float m_new = fmaxf(m_run[qb], mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);  // -inf -> 0
        l_run[qb] *= alpha;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) oacc[qb][cb] *= alpha;
        m_run[qb] = m_new;
      }
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][i], scale, -m_run[qb]));
          psum += p[i];
        }
        const u32x2 w = {f2bf2(p[0], p[1]), f2bf2(p[2], p[3])};
        pb[qb][kb] = __builtin_bit_cast(s16x4, w);
      }
      psum = xor32_sum(xor16_sum(psum));
      l_run[qb] += psum;
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int vr = cb * 16 + (lane & 15);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int u = (kofs + kb * 16) / 4 + (lane >> 4);  // 8-byte unit: 4 keys
        const int vx = VCH == 16 ? vswz16(vr) : vswz(vr);
        const s16x4 va = *(const s16x4*)(st + K_BYTES + vr * VRB + (((u >> 1) ^ vx) << 4) +
                                          ((u & 1) << 3));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          oacc[qb][cb] =
              __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb[qb][kb], oacc[qb][cb], 0, 0, 0);
      }
    }
  }

  if constexpr (KH > 1) {
    // merge the key groups in pairs, (m, l, o) of disjoint key sets by the
    // log-sum-exp rule: in the round of width h the groups [h, 2h) hand
    // their state to the groups [0, h) through LDS; every wave takes part in
    // every barrier
    constexpr int REG = QB * NCB * 64 * 16 + QB * 64 * 8;  // o fragments + (m, l)
    attn_lds_barrier();  // every wave is done with the tiles in LDS
#pragma unroll
    for (int h = KH / 2; h >= 1; h /= 2) {
      if (kh >= h && kh < 2 * h) {
        unsigned char* mine = smem + ((kh - h) * QW + qw) * REG;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            ((f32x4*)mine)[(qb * NCB + cb) * 64 + lane] = oacc[qb][cb];
          ((float2*)(mine + QB * NCB * 64 * 16))[qb * 64 + lane] =
              make_float2(m_run[qb], l_run[qb]);
        }
      }
      attn_lds_barrier();
      if (kh < h) {
        const unsigned char* other = smem + (kh * QW + qw) * REG;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float2 ml = ((const float2*)(other + QB * NCB * 64 * 16))[qb * 64 + lane];
          const float m = fmaxf(m_run[qb], ml.x);
          const float a0 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[qb] - m);
          const float a1 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml.x - m);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            oacc[qb][cb] =
                oacc[qb][cb] * a0 + ((const f32x4*)other)[(qb * NCB + cb) * 64 + lane] * a1;
          l_run[qb] = l_run[qb] * a0 + ml.y * a1;
          m_run[qb] = m;
        }
      }
      attn_lds_barrier();  // the slots are read before the next round writes
    }
    if (kh != 0) return;
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (!qok[qb]) continue;
    const int gq = row[qb] * nq + head[qb];
    if (SPLIT) {
      const size_t base = (size_t)bz * M * nq + gq;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        *(f32x4*)(part_o + base * HD + cb * 16 + (lane >> 4) * 4) = oacc[qb][cb];
      if ((lane >> 4) == 0) {
        part_ml[base * 2] = m_run[qb];
        part_ml[base * 2 + 1] = l_run[qb];
      }
    } else {
      const float inv = 1.f / l_run[qb];
      bf16_t* op = o + (size_t)row[qb] * nq * HD + (size_t)head[qb] * HD;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int c = cb * 16 + (lane >> 4) * 4;
        ushort4 w;
        w.x = f2bf(oacc[qb][cb][0] * inv);
        w.y = f2bf(oacc[qb][cb][1] * inv);
        w.z = f2bf(oacc[qb][cb][2] * inv);
        w.w = f2bf(oacc[qb][cb][3] * inv);
        *(ushort4*)(op + c) = w;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 32x32 MFMA kernel (bf16, hd 64 or 128; N a multiple of the key tile KT).
//
// A workgroup owns QT = QW * QB * 32 query vectors of one (sequence, kv head)
// and one key range, and streams the range's K and V^T tiles through an
// STAGES-deep LDS ring with direct global->LDS loads.  Wave (qw, kh) holds
// QB blocks of 32 query vectors and takes keys [kh KT/KH, (kh+1) KT/KH) of
// every tile, in 32-key blocks:
//   S^T (32 keys x 32 queries) = K Q^T with v_mfma_f32_32x32x16_bf16, Q^T
//     from registers (lane l: query l%32, head dims 16c + 8(l/32) .. +7);
//     lane l supplies K row pi(l%32) of the block, where pi swaps bits 2 and
//     3 of the row index, so that accumulator register 8s + e of lane l
//     holds key 16s + 8(l/32) + e of the block for query l%32;
//   O^T (hd x 32 queries) += V^T P^T with the same MFMA: registers 8s..8s+7
//     of S^T, exponentiated and rounded to bf16, are exactly the B operand of
//     key step s, and the A operand is 8 consecutive keys of one V^T row (one
//     16-byte LDS read).
// One K/V fragment read from LDS thus feeds 32 queries (64 with QB = 2), and
// P never leaves registers.  Online softmax per query in base 2 with a lazily
// raised maximum; the two lanes l and l^32 of a query combine by
// permlane32_swap.  The KH key groups of a query block merge through LDS at
// the end; split-KV (gridDim.z > 1) writes unnormalised partials for the
// combine pass.
__device__ __forceinline__ int pi32(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}
// 16-byte slot XOR of a K row (HD * 2 bytes) or V^T row (KT * 2 bytes): the
// rows one 8-lane group of a fragment read touches land on distinct slots
// (16-slot rows: r & 15; 8-slot rows: rows {0-3, 8-11} and {4-7, 12-15}
// are the groups, hence bit 3 moves to bit 2)
template <int CH>
__device__ __forceinline__ int a32_swz(int r) {
  if constexpr (CH == 16) return r & 15;
  else return (r & 3) | ((r >> 1) & 4);
}
// V^T rows: the 8 lanes of a group read 8 consecutive rows at one chunk
template <int CH>
__device__ __forceinline__ int a32_vswz(int r) {
  return CH == 16 ? (r & 15) : (r & 7);
}

template <int HD, int QB>
constexpr size_t attn32_merge_bytes(int KH, int QW) {
  return KH == 1 ? 0 : (size_t)KH * QW * QB * ((HD / 32) * 16 * 64 * 4 + 64 * 8);
}

template <int HD, int KT, int STAGES, int QW, int KH, int QB, bool SPLIT>
__global__ __launch_bounds__(64 * QW * KH, 1) void attn32_kernel(
    const bf16_t* __restrict__ q, const int32_t* __restrict__ row_start,
    const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc, bf16_t* __restrict__ o, int N,
    int nq, int nkv, int keys_per_split, int M, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  static_assert(HD == 64 || HD == 128, "head dim");
  static_assert(KT == 64 || KT == 128, "key tile");
  static_assert(QB == 1 || QB == 2, "query blocks per wave");
  constexpr int NWV = QW * KH;
  constexpr int QT = QW * QB * 32;       // query vectors per workgroup
  constexpr int KW = KT / KH;            // keys per wave per tile
  static_assert(KW % 32 == 0, "a wave takes whole 32-key blocks");
  constexpr int KB = KW / 32;
  constexpr int NKC = HD / 16;           // k-steps of S (head dims)
  constexpr int NHB = HD / 32;           // 32-row blocks of O^T
  constexpr int KRB = HD * 2, KCH = KRB / 16;  // K row bytes, 16-byte chunks per row
  constexpr int VRB = KT * 2, VCH = VRB / 16;  // V^T row bytes in a tile, chunks per row
  constexpr int K_BYTES = KT * KRB, V_BYTES = HD * VRB, STAGE = K_BYTES + V_BYTES;
  constexpr int K_INSTR = K_BYTES / 1024, V_INSTR = V_BYTES / 1024;
  constexpr int IPW = (K_INSTR + V_INSTR) / NWV;  // load instructions per wave per tile
  static_assert((K_INSTR + V_INSTR) % NWV == 0, "instructions per wave");
  constexpr int QRB = HD * 2, QCH = QRB / 16;  // query vector bytes, 16-byte chunks
  constexpr int Q_INSTR = QT * QRB / 1024;
  static_assert(Q_INSTR % NWV == 0, "query load instructions per wave");
  constexpr int QIPW = Q_INSTR / NWV;
  static_assert(QIPW + STAGES * IPW < 64, "in-flight loads must fit the vmcnt counter");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qw = wave % QW, kh = wave / QW;
  const int g = lane >> 5, l32 = lane & 31;
  // XCD-aware order (workgroup i runs on XCD i % 8): consecutive workgroups
  // of one XCD take the query tiles and key ranges of one (sequence, kv
  // head), whose K/V then stream through that XCD's L2
  const int nx = gridDim.x, ny = gridDim.y;
  const int total = nx * ny * gridDim.z;
  int lin = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  if ((total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);
  const int bx = lin % nx, by = (lin / nx) % ny, bz = lin / (nx * ny);
  const int b = by / nkv, gk = by % nkv;
  const int G = nq / nkv;
  const int r0 = row_start[b], Qn = (row_start[b + 1] - r0) * G;
  const int qbase = bx * QT;
  if (qbase >= Qn) return;  // uniform over the workgroup

  bool qok[QB];
  int row[QB], head[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qv = qbase + (qw * QB + qb) * 32 + l32;
    qok[qb] = qv < Qn;
    row[qb] = r0 + (qok[qb] ? qv / G : 0);
    head[qb] = gk * G + (qok[qb] ? qv % G : 0);
  }
  const bool wave_live = qbase + qw * QB * 32 < Qn;  // wave-uniform
  const size_t slab = ((size_t)b * nkv + gk) * N * HD;
  const bf16_t* kslab = kc + slab;  // [N][HD]
  const bf16_t* vslab = vc + slab;  // [HD][N]
  const int key0 = bz * keys_per_split;
  const int key1 = min(N, key0 + keys_per_split);
  const int ntiles = key1 > key0 ? (key1 - key0) / KT : 0;
  const float scale = kLog2e / sqrtf((float)HD);

  // this lane's global source and LDS destination for each of its load
  // instructions (tile 0): lane i of instruction j fills 16-byte slot i % CH
  // of row j * (64 / CH) + i / CH, from the row's chunk slot ^ swizzle
  const bf16_t* src[IPW];
  int dst[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int j = wave + i * NWV;
    if (j < K_INSTR) {
      const int kr = j * (1024 / KRB) + lane / KCH;
      const int lc = (lane % KCH) ^ a32_swz<KCH>(kr);
      src[i] = kslab + (size_t)(key0 + kr) * HD + lc * 8;
      dst[i] = j * 1024;
    } else {
      const int jv = j - K_INSTR;
      const int vr = jv * (1024 / VRB) + lane / VCH;
      const int lc = (lane % VCH) ^ a32_vswz<VCH>(vr);
      src[i] = vslab + (size_t)vr * N + key0 + lc * 8;
      dst[i] = K_BYTES + jv * 1024;
    }
  }
  // Key tiles in rotated order: query tile bx starts at key tile bx mod
  // ntiles.  The query tiles of one (sequence, kv head) are consecutive
  // workgroups of one XCD, so they first request different tiles and the
  // head's whole K/V is in flight at once, rather than one tile at a time;
  // each then finds the tiles its siblings fetched in the XCD's L2.  The
  // online softmax does not depend on the order beyond rounding.
  const int rot = ntiles > 0 ? bx % ntiles : 0;
  auto issue = [&](int t) {
    unsigned char* st = smem + (t % STAGES) * STAGE;
    const int kt = t + rot < ntiles ? t + rot : t + rot - ntiles;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int j = wave + i * NWV;
      const size_t adv = j < K_INSTR ? (size_t)kt * KT * HD : (size_t)kt * KT;
      attn_dma16(src[i] + adv, st + dst[i]);
    }
  };

  float m_run[QB], l_run[QB];
  f32x16 oacc[QB][NHB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][hb][r] = 0.f;
  }

  // The query vectors go to LDS by the same DMA as the tiles, ahead of them:
  // then every load in flight is of one kind, completes in issue order, and
  // the wait for the first tile also covers the queries (a register load of
  // the queries made the compiler wait for every tile in flight before the
  // first MFMA).  Lane i of instruction j fills slot i % QCH of query vector
  // j * (64 / QCH) + i / QCH from its chunk slot ^ (vector & (QCH - 1));
  // vectors past the sequence's last load the tile's first one and are
  // zeroed in registers.
  unsigned char* qs = smem + STAGES * STAGE;
#pragma unroll
  for (int i = 0; i < QIPW; ++i) {
    const int j = wave + i * NWV;
    const int qi = j * (1024 / QRB) + lane / QCH;
    const int qv = qbase + qi < Qn ? qbase + qi : qbase;
    const int lc = (lane % QCH) ^ (qi & (QCH - 1));
    attn_dma16(q + (size_t)(r0 + qv / G) * nq * HD + (size_t)(gk * G + qv % G) * HD + lc * 8,
               qs + j * 1024);
  }
  // every slot of the ring is filled before the loop; from the second tile
  // on, tile t + STAGES - 1 refills the slot of tile t - 1, which every wave
  // has finished once it has passed tile t's barrier
#pragma unroll
  for (int t = 0; t < STAGES; ++t)
    if (t < ntiles) issue(t);
  if (ntiles == 0) attn_wait_vmcnt<0>();  // no DMA may land after the workgroup ends

  bf16x8 qf[QB][NKC];  // query fragments: the B operand of S^T
  const int kofs = kh * KW;  // this wave's first key in a tile
  for (int t = 0; t < ntiles; ++t) {
    if (t == 0) attn_wait_tiles<IPW, STAGES>(min(STAGES - 1, ntiles - 1));
    else attn_wait_tiles<IPW, STAGES>(min(STAGES - 2, ntiles - 1 - t));
    attn_lds_barrier();
    if (t > 0 && t + STAGES - 1 < ntiles) issue(t + STAGES - 1);
    if (!wave_live) continue;  // no valid query in this wave: loads only
    if (t == 0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qi = (qw * QB + qb) * 32 + l32;
#pragma unroll
        for (int c = 0; c < NKC; ++c) {
          const uint4 z = make_uint4(0, 0, 0, 0);
          const bf16x8 v =
              *(const bf16x8*)(qs + qi * QRB + (((2 * c + g) ^ (qi & (QCH - 1))) << 4));
          qf[qb][c] = qok[qb] ? v : *(const bf16x8*)&z;
        }
      }
    }
    const unsigned char* st = smem + (t % STAGES) * STAGE;
    f32x16 s[QB][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
      const int kr = kofs + kb * 32 + pi32(l32);
      const unsigned char* krow = st + kr * KRB;
#pragma unroll
      for (int c = 0; c < NKC; ++c) {
        const bf16x8 a = *(const bf16x8*)(krow + (((2 * c + g) ^ a32_swz<KCH>(kr)) << 4));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][c], s[qb][kb], 0, 0, 0);
      }
    }
    bf16x8 pb[QB][KB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
      mx = xor32_max(mx) * scale;
      if (__any(mx > m_run[qb] + kLazyMax)) {  // wave-uniform branch
        const float m_new = fmaxf(m_run[qb], mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);  // -inf -> 0
        l_run[qb] *= alpha;
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) oacc[qb][hb] *= alpha;
        m_run[qb] = m_new;
      }
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][8 * sb + e], scale, -m_run[qb]));
            psum += p[e];
          }
          const uint4 w = make_uint4(f2bf2(p[0], p[1]), f2bf2(p[2], p[3]), f2bf2(p[4], p[5]),
                                     f2bf2(p[6], p[7]));
          pb[qb][kb][sb] = __builtin_bit_cast(bf16x8, w);
        }
      l_run[qb] += xor32_sum(psum);
    }
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const int vr = hb * 32 + l32;
      const unsigned char* vrow = st + K_BYTES + vr * VRB;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const int ch = (kofs + kb * 32 + sb * 16) / 8 + g;
          const bf16x8 va = *(const bf16x8*)(vrow + ((ch ^ a32_vswz<VCH>(vr)) << 4));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            oacc[qb][hb] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[qb][kb][sb], oacc[qb][hb], 0, 0, 0);
        }
    }
  }

  // The key groups merge by the log-sum-exp rule in one round: every wave
  // writes its state to LDS, then wave kh merges head-dim blocks kh, kh + KH,
  // ... over the KH groups (in group order), normalises and stores them, so
  // that the merge and the stores are shared by all waves.
  constexpr int OB = NHB * 16 * 64 * 4;  // O^T registers of one query block
  constexpr int SB = OB + 64 * 8;        // + (m, l) per lane
  auto state = [&](int grp, int qb) { return smem + (size_t)((grp * QW + qw) * QB + qb) * SB; };
  if constexpr (KH > 1) {
    attn_lds_barrier();  // every wave is done with the tiles and queries in LDS
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      f32x4* mine = (f32x4*)state(kh, qb);
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          mine[(hb * 4 + r4) * 64 + lane] =
              f32x4{oacc[qb][hb][4 * r4], oacc[qb][hb][4 * r4 + 1], oacc[qb][hb][4 * r4 + 2],
                    oacc[qb][hb][4 * r4 + 3]};
      ((float2*)(state(kh, qb) + OB))[lane] = make_float2(m_run[qb], l_run[qb]);
    }
    attn_lds_barrier();
  }

  // lane l holds query l%32 and head dims 32 hb + 8 i + 4 (l/32) + j in
  // register 4 i + j of block hb
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float wgt[KH];  // weight of each group's sums
    float m = m_run[qb], l = l_run[qb];
    if constexpr (KH > 1) {
      float mg[KH], lg[KH];
      m = -INFINITY;
#pragma unroll
      for (int kg = 0; kg < KH; ++kg) {
        const float2 ml = ((const float2*)(state(kg, qb) + OB))[lane];
        mg[kg] = ml.x;
        lg[kg] = ml.y;
        m = fmaxf(m, ml.x);
      }
      l = 0.f;
#pragma unroll
      for (int kg = 0; kg < KH; ++kg) {
        wgt[kg] = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mg[kg] - m);
        l += lg[kg] * wgt[kg];
      }
    }
    if (!qok[qb]) continue;
    const int gq = row[qb] * nq + head[qb];
    const size_t base = SPLIT ? (size_t)bz * M * nq + gq : 0;
    if (SPLIT && kh == 0 && g == 0) *(float2*)(part_ml + base * 2) = make_float2(m, l);
    const float inv = 1.f / l;
    bf16_t* op = o + (size_t)row[qb] * nq * HD + (size_t)head[qb] * HD;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      if (hb % KH != kh) continue;  // wave-uniform
      f32x16 v;
      if constexpr (KH > 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = 0.f;
#pragma unroll
        for (int kg = 0; kg < KH; ++kg) {
          const f32x4* st = (const f32x4*)state(kg, qb);
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 x = st[(hb * 4 + r4) * 64 + lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * r4 + e] += wgt[kg] * x[e];
          }
        }
      } else {
        v = oacc[qb][hb];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (SPLIT) {
          *(f32x4*)(part_o + base * HD + hb * 32 + 8 * i + 4 * g) =
              f32x4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
        } else {
          *(uint2*)(op + hb * 32 + 8 * i + 4 * g) =
              make_uint2(f2bf2(v[4 * i] * inv, v[4 * i + 1] * inv),
                         f2bf2(v[4 * i + 2] * inv, v[4 * i + 3] * inv));
        }
      }
    }
  }
}

// Combine split-KV partials: o = sum_s o_s 2^(m_s - m) / sum_s l_s 2^(m_s - m),
// m = max_s m_s; one thread per 4 consecutive output columns.
template <typename T>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           int splits, int MQ, int hd,
                                                           T* __restrict__ o) {
  const int hd4 = hd / 4;
  const size_t total = (size_t)MQ * hd4;
  for (size_t f = blockIdx.x * (size_t)blockDim.x + threadIdx.x; f < total;
       f += (size_t)gridDim.x * blockDim.x) {
    const size_t gq = f / hd4;
    const int c = (int)(f % hd4) * 4;
    float m = -INFINITY;
    for (int s = 0; s < splits; ++s) m = fmaxf(m, part_ml[((size_t)s * MQ + gq) * 2]);
    float den = 0.f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < splits; ++s) {
      const float ms = part_ml[((size_t)s * MQ + gq) * 2];
      if (ms == -INFINITY) continue;
      const float w = exp2f(ms - m);
      den += part_ml[((size_t)s * MQ + gq) * 2 + 1] * w;
      num += *(const f32x4*)(part_o + ((size_t)s * MQ + gq) * hd + c) * w;
    }
    const float inv = 1.f / den;
#pragma unroll
    for (int i = 0; i < 4; ++i) st(o, gq * hd + c + i, num[i] * inv);
  }
}

// Generic kernel (float or bf16, any even hd <= 256): one wave per
// (row, query head); lanes split hd; keys visited in order with an online
// softmax in fp32.
template <typename T>
__global__ __launch_bounds__(256) void attn_generic_kernel(
    const T* __restrict__ q, const int32_t* __restrict__ row_start, int B,
    const T* __restrict__ kc, const T* __restrict__ vc, T* __restrict__ o, int M, int N, int nq,
    int nkv, int hd) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gw >= M * nq) return;
  const int row = gw / nq, h = gw % nq;
  int b = 0;
  while (b + 1 < B && row_start[b + 1] <= row) ++b;
  const int g = h * nkv / nq;
  const float scale = rsqrtf((float)hd);
  float qv[4], acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int col = lane + 64 * c;
    qv[c] = col < hd ? ld(q, (size_t)row * nq * hd + (size_t)h * hd + col) * scale : 0.f;
  }
  const size_t slab = ((size_t)b * nkv + g) * N * hd;
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j < N; ++j) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int col = lane + 64 * c;
      if (col < hd) s += qv[c] * ld(kc, slab + (size_t)j * hd + col);
    }
    s = wave_sum(s);
    const float mn = fmaxf(m, s);
    const float a = expf(m - mn), p = expf(s - mn);
    l = l * a + p;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int col = lane + 64 * c;
      acc[c] = acc[c] * a + (col < hd ? p * ld(vc, slab + (size_t)col * N + j) : 0.f);
    }
    m = mn;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int col = lane + 64 * c;
    if (col < hd) st(o, (size_t)row * nq * hd + (size_t)h * hd + col, acc[c] / l);
  }
}

namespace {

struct AttnPlan {
  bool mfma;
  int qtiles, splits, keys_per_split, stages;
  int key_halves;  // key groups: waves per query block, each over its share of every key tile
  int qblocks;     // 16-query blocks per wave
  int key_tile;    // keys per LDS tile of the DMA kernel (64 or 128)
  size_t ws;
};

constexpr size_t kAttnSplitCap = 64ull << 20;  // split-KV partials never exceed this
constexpr int kAttnCUs = 256;                    // compute units of an MI355X

// Splits the keys while fewer than 128 workgroups would be busy (the
// combine pass costs a launch plus a write and a read of every partial
// output), keeping at least one 64-key tile per split, and uses a 2-stage
// LDS ring (64 KB at hd 128).  Both choices come from a sweep on MI355X over
// M = 20 .. 1024 active rows and N = 512, 1024 keys (32 heads of 128), where
// 2 stages beat 4 at every point and more splits lost to the combine pass.
// Measured at N = 512 .. 4096 with one workgroup per (head, 64 queries): a
// workgroup takes ~0.9 us per 64-key tile whatever its wave layout (two
// query blocks per wave, which halves the LDS reads, did not change it) and
// whether 32 or 192 workgroups run, so the time is per-workgroup latency
// rather than HBM, LDS or MFMA throughput.
AttnPlan make_attn_plan_cfg(int dtype, int M, int B, int N, int nq, int nkv, int hd, int splits_in,
                            int stages_in, int kh_in, int qb_in, int kt_in) {
  AttnPlan p{};
  p.key_tile = (kt_in == 128 && N % 128 == 0) ? 128 : 64;
  p.key_halves = kh_in == 1 || kh_in == 2 || kh_in == 4 ? kh_in : 2;
  p.qblocks = qb_in == 1 || qb_in == 2 ? qb_in : 1;
  p.mfma = dtype == kBF16 && (hd == 64 || hd == 128) && nq % nkv == 0;
  p.splits = 1;
  p.keys_per_split = N;
  p.stages = 4;
  if (!p.mfma || M <= 0) return p;
  const int G = nq / nkv;
  const int mb_max = std::min(M, N);  // rows of one sequence
  p.qtiles = (mb_max * G + kAttnQ - 1) / kAttnQ;
  // estimated busy workgroups: the rows are spread over the sequences
  const int busy = std::max(1, (M * G + kAttnQ - 1) / kAttnQ) * nkv;
  const int ktiles = (N + p.key_tile - 1) / p.key_tile;
  auto ws_of = [&](int sp) { return (size_t)sp * M * nq * (hd + 2) * sizeof(float); };
  int splits = 1;
  if (splits_in > 0) {
    splits = std::min(splits_in, ktiles);
  } else {
    while (busy * splits < 128 && ktiles / (splits * 2) >= 1 && ws_of(splits * 2) <= kAttnSplitCap)
      splits *= 2;
  }
  p.splits = splits;
  const int tiles_per = (ktiles + splits - 1) / splits;
  p.keys_per_split = tiles_per * p.key_tile;
  // four key groups (16 waves) with 128-key tiles when every workgroup runs
  // at once on its own CU and walks at least 1024 keys.  Measured at M = 384,
  // 32 heads: 4% faster at N = 1024, 12% at N = 2048, 17% at N = 4096 than
  // two groups of 64-key tiles, 4% slower at N = 512.  The larger tile pays
  // only with four groups (two groups with 128-key tiles are level with
  // 64-key tiles): the per-tile cost is mostly fixed (load issue, barrier,
  // fragment reads).  With many more workgroups than CUs (N = 4096 over
  // thousands of query tiles) four groups ran about 30% slower than two.
  if (kh_in == 0 && p.keys_per_split >= 1024 && busy * splits <= 256) {
    p.key_halves = 4;
    // a split range of an even number of 64-key tiles is a whole number of
    // 128-key tiles; keys_per_split is unchanged
    if (kt_in == 0 && N % 128 == 0 && tiles_per % 2 == 0) p.key_tile = 128;
  }
  p.stages = stages_in == 2 || stages_in == 4 ? stages_in : 2;
  p.ws = splits > 1 ? ws_of(splits) : 0;
  return p;
}

AttnPlan make_attn_plan(int dtype, int M, int B, int N, int nq, int nkv, int hd) {
  return make_attn_plan_cfg(dtype, M, B, N, nq, nkv, hd, 0, 0, 0, 0, 0);
}

template <int HD, bool SPLIT, int STAGES, int KH, int QB, int KT>
void launch_attn_dma(dim3 grid, const void* q, const int32_t* row_start, const void* kc,
                     const void* vc, void* o, int N, int nq, int nkv, int kps, int M, float* po,
                     float* pml, hipStream_t s) {
  constexpr size_t ring = STAGES * (size_t)(2 * KT * HD * 2);
  constexpr size_t merge = attn_merge_bytes<HD, KH, QB>();
  constexpr size_t lds = ring > merge ? ring : merge;
  static_assert(lds <= 160 * 1024, "LDS of a CU");
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute(
        reinterpret_cast<const void*>(&attn_mfma_dma_kernel<HD, SPLIT, STAGES, KH, QB, KT>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr = true;
  }
  attn_mfma_dma_kernel<HD, SPLIT, STAGES, KH, QB, KT><<<grid, 64 * (4 / QB) * KH, lds, s>>>(
      (const bf16_t*)q, row_start, (const bf16_t*)kc, (const bf16_t*)vc, (bf16_t*)o, N, nq, nkv,
      kps, M, po, pml);
}

// Wave layouts built: (key groups, query blocks per wave) = (1, 1), (2, 1),
// (4, 1), (2, 2), (4, 2); any other request takes (2, 1).
template <int HD, bool SPLIT, int STAGES, int KT>
void launch_attn_dma_layout(int kh, int qb, dim3 grid, const void* q, const int32_t* row_start,
                            const void* kc, const void* vc, void* o, int N, int nq, int nkv,
                            int kps, int M, float* po, float* pml, hipStream_t s) {
#define DLM_ATTN_LAUNCH(KH, QB)                                                              \
  launch_attn_dma<HD, SPLIT, STAGES, KH, QB, KT>(grid, q, row_start, kc, vc, o, N, nq, nkv, kps, \
                                                 M, po, pml, s)
  if (qb == 2 && kh == 4) DLM_ATTN_LAUNCH(4, 2);
  else if (qb == 2 && kh == 2) DLM_ATTN_LAUNCH(2, 2);
  else if (kh == 4) DLM_ATTN_LAUNCH(4, 1);
  else if (kh == 1) DLM_ATTN_LAUNCH(1, 1);
  else DLM_ATTN_LAUNCH(2, 1);
#undef DLM_ATTN_LAUNCH
}

template <int HD, bool SPLIT>
void launch_attn_kernel(dim3 grid, bool dma, int stages, int kh, int qb, int kt, const void* q,
                        const int32_t* row_start,
                        const void* kc, const void* vc, void* o, int N, int nq, int nkv,
                        int kps, int M, float* po, float* pml, hipStream_t s) {
  if (dma) {
#define DLM_ATTN_STAGES(ST, KT)                                                              \
  launch_attn_dma_layout<HD, SPLIT, ST, KT>(kh, qb, grid, q, row_start, kc, vc, o, N, nq, nkv, \
                                            kps, M, po, pml, s)
    if (kt == 128) {
      DLM_ATTN_STAGES(2, 128);  // four 64 KB stages would not fit the LDS at hd 128
    } else {
      if (stages == 2) DLM_ATTN_STAGES(2, 64);
      else DLM_ATTN_STAGES(4, 64);
    }
#undef DLM_ATTN_STAGES
  } else {
    attn_mfma_kernel<HD, SPLIT><<<grid, 256, 0, s>>>((const bf16_t*)q, row_start,
                                                     (const bf16_t*)kc, (const bf16_t*)vc,
                                                     (bf16_t*)o, N, nq, nkv, kps, M, po, pml);
  }
}

template <int HD>
hipError_t run_attn_mfma(const AttnPlan& p, int M, int B, int N, int nq, int nkv,
                         const void* q, const int32_t* row_start, const void* kc,
                         const void* vc, void* o, void* ws, hipStream_t s) {
  dim3 grid(p.qtiles, B * nkv, p.splits);
  const bool dma = (N % p.key_tile) == 0;
  if (p.splits > 1) {
    float* po = (float*)ws;
    float* pml = po + (size_t)p.splits * M * nq * HD;
    launch_attn_kernel<HD, true>(grid, dma, p.stages, p.key_halves, p.qblocks, p.key_tile, q,
                                 row_start, kc, vc, o, N, nq, nkv, p.keys_per_split, M, po, pml,
                                 s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t total = (size_t)M * nq * (HD / 4);
    const int gsz = (int)std::min<size_t>((total + 255) / 256, 8192);
    attn_combine_kernel<bf16_t><<<gsz, 256, 0, s>>>(po, pml, p.splits, M * nq, HD, (bf16_t*)o);
  } else {
    launch_attn_kernel<HD, false>(grid, dma, p.stages, p.key_halves, p.qblocks, p.key_tile, q,
                                  row_start, kc, vc, o, N, nq, nkv, p.keys_per_split, M, nullptr,
                                  nullptr, s);
  }
  return hipGetLastError();
}

// ---- 32x32 MFMA kernel: layouts, plan, launch ---------------------------------

struct A32Layout {
  int kt, stages, qw, kh, qb;
};
// (keys per LDS tile, ring depth, query waves, key groups, 32-query blocks
// per wave); query vectors per workgroup = 32 qw qb.  Kept from a sweep on
// MI355X over one layer of 32 heads of 128 at N = 512 and 1024 and M = 9 ..
// 1024 (kernels timed back to back in a HIP graph, 32 caches rotated);
// dropped there: two query blocks per wave, one key group, 64-key tiles in
// 3- to 5-deep rings, and a variant without LDS that loads each wave's K / V
// fragments straight into registers (all slower at every point).
constexpr A32Layout kA32[] = {
    {128, 2, 1, 4, 1},  // 0: 32 queries, four key groups (4 waves)
    {128, 2, 2, 4, 1},  // 1: 64 queries, four key groups (8 waves)
    {128, 2, 4, 2, 1},  // 2: 128 queries, two key groups (8 waves)
    {128, 2, 2, 2, 1},  // 3: 64 queries, two key groups (4 waves)
};
constexpr int kNumA32 = sizeof(kA32) / sizeof(kA32[0]);

struct A32Plan {
  bool ok;
  int layout, qtiles, splits, keys_per_split;
  size_t ws;
};

A32Plan make_a32_plan(int dtype, int M, int B, int N, int nq, int nkv, int hd, int splits_in,
                      int layout_in) {
  A32Plan p{};
  p.ok = dtype == kBF16 && (hd == 64 || hd == 128) && nq % nkv == 0 && M > 0;
  if (!p.ok) return p;
  const int G = nq / nkv;
  int lay = layout_in;
  // query vectors per (sequence, kv head), the rows spread evenly
  const int qph = (M * G + B - 1) / B;
  if (lay < 0 || lay >= kNumA32) {
    // 64 queries per workgroup up to 64 per head (one workgroup per head,
    // 8 waves); above, the smallest query tile (32, 64, 128) whose
    // workgroups all run in one round: each holds 128 KB of LDS, so one per
    // CU, and a grid one round too large ran 1.5-1.7x slower (N = 512,
    // M = 264..300: 21.3 against 12.5 us with 64 queries; N = 1024,
    // M = 544..736: 34-36 against 23-24 us with 128)
    if (qph <= 64) {
      lay = 1;
    } else {
      lay = 2;
      for (int c : {0, 1}) {
        const int qt = 32 * kA32[c].qw * kA32[c].qb;
        if ((long long)B * nkv * ((qph + qt - 1) / qt) <= kAttnCUs) {
          lay = c;
          break;
        }
      }
    }
  }
  const A32Layout& L = kA32[lay];
  if (N % L.kt) {
    p.ok = false;
    return p;
  }
  p.layout = lay;
  const int QT = 32 * L.qw * L.qb;
  p.qtiles = (std::min(M, N) * G + QT - 1) / QT;
  const int busy = std::max(1, (M * G + QT - 1) / QT) * nkv;
  const int unit = L.kt;  // a key range is a whole number of LDS tiles
  const int ktiles = N / unit;
  auto ws_of = [&](int sp) { return (size_t)sp * M * nq * (hd + 2) * sizeof(float); };
  int splits = 1;
  if (splits_in > 0) {
    splits = std::min(splits_in, ktiles);
  } else {
    // splitting the keys (partials merged by the combine pass) paid only
    // from N = 1024, with few busy workgroups and at least two tiles per
    // range: M = 20 (32 workgroups) 4 ranges, M = 102 (128) 2 ranges
    while (N >= 1024 && busy * splits * 2 <= kAttnCUs && ktiles / (splits * 2) >= 2 &&
           ws_of(splits * 2) <= kAttnSplitCap)
      splits *= 2;
  }
  const int tiles_per = (ktiles + splits - 1) / splits;
  p.splits = (ktiles + tiles_per - 1) / tiles_per;  // no empty key range
  p.keys_per_split = tiles_per * unit;
  p.ws = p.splits > 1 ? ws_of(p.splits) : 0;
  return p;
}

template <int HD, int KT, int STAGES, int QW, int KH, int QB, bool SPLIT>
void launch_a32(dim3 grid, const void* q, const int32_t* row_start, const void* kc,
                const void* vc, void* o, int N, int nq, int nkv, int kps, int M, float* po,
                float* pml, hipStream_t s) {
  // the ring, then the workgroup's query vectors
  constexpr size_t ring = (size_t)STAGES * (KT * HD * 2 + HD * KT * 2) + 32 * QW * QB * HD * 2;
  constexpr size_t merge = attn32_merge_bytes<HD, QB>(KH, QW);
  constexpr size_t lds = ring > merge ? ring : merge;
  static_assert(lds <= 160 * 1024, "LDS of a CU");
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute(
        reinterpret_cast<const void*>(&attn32_kernel<HD, KT, STAGES, QW, KH, QB, SPLIT>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr = true;
  }
  attn32_kernel<HD, KT, STAGES, QW, KH, QB, SPLIT><<<grid, 64 * QW * KH, lds, s>>>(
      (const bf16_t*)q, row_start, (const bf16_t*)kc, (const bf16_t*)vc, (bf16_t*)o, N, nq, nkv,
      kps, M, po, pml);
}

template <int HD, bool SPLIT>
void launch_a32_layout(int lay, dim3 grid, const void* q, const int32_t* row_start,
                       const void* kc, const void* vc, void* o, int N, int nq, int nkv, int kps,
                       int M, float* po, float* pml, hipStream_t s) {
#define DLM_A32(KT, ST, QW, KH, QB)                                                              \
  launch_a32<HD, KT, ST, QW, KH, QB, SPLIT>(grid, q, row_start, kc, vc, o, N, nq, nkv, kps, M, \
                                            po, pml, s)
  switch (lay) {
    case 0: DLM_A32(128, 2, 1, 4, 1); break;
    case 1: DLM_A32(128, 2, 2, 4, 1); break;
    case 2: DLM_A32(128, 2, 4, 2, 1); break;
    default: DLM_A32(128, 2, 2, 2, 1); break;
  }
#undef DLM_A32
}

template <int HD>
hipError_t run_a32(const A32Plan& p, int M, int B, int N, int nq, int nkv, const void* q,
                   const int32_t* row_start, const void* kc, const void* vc, void* o, void* ws,
                   hipStream_t s) {
  dim3 grid(p.qtiles, B * nkv, p.splits);
  if (p.splits > 1) {
    float* po = (float*)ws;
    float* pml = po + (size_t)p.splits * M * nq * HD;
    launch_a32_layout<HD, true>(p.layout, grid, q, row_start, kc, vc, o, N, nq, nkv,
                                p.keys_per_split, M, po, pml, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t total = (size_t)M * nq * (HD / 4);
    const int gsz = (int)std::min<size_t>((total + 255) / 256, 8192);
    attn_combine_kernel<bf16_t><<<gsz, 256, 0, s>>>(po, pml, p.splits, M * nq, HD, (bf16_t*)o);
  } else {
    launch_a32_layout<HD, false>(p.layout, grid, q, row_start, kc, vc, o, N, nq, nkv,
                                 p.keys_per_split, M, nullptr, nullptr, s);
  }
  return hipGetLastError();
}

hipError_t run_a32_any(const A32Plan& p, int M, int B, int N, int nq, int nkv, int hd,
                       const void* q, const int32_t* row_start, const void* kc, const void* vc,
                       void* o, void* ws, hipStream_t s) {
  if (hd == 128) return run_a32<128>(p, M, B, N, nq, nkv, q, row_start, kc, vc, o, ws, s);
  return run_a32<64>(p, M, B, N, nq, nkv, q, row_start, kc, vc, o, ws, s);
}

}  // namespace

int attention_num_layouts() { return kNumA32; }

size_t attention_layout_ws_bytes(int dtype, int M, int B, int N, int nq, int nkv, int hd,
                                 int splits, int layout) {
  const A32Plan p = make_a32_plan(dtype, M, B, N, nq, nkv, hd, splits, layout);
  return p.ok ? p.ws : 0;
}

bool attention_layout_supported(int dtype, int N, int hd, int layout) {
  if (dtype != kBF16 || (hd != 64 && hd != 128) || layout < 0 || layout >= kNumA32) return false;
  return N % kA32[layout].kt == 0;
}

hipError_t launch_attention_layout(int dtype, int M, int B, int N, int nq, int nkv, int hd,
                                   const void* q, const int32_t* row_start, const void* kc,
                                   const void* vc, void* o, void* ws, size_t ws_bytes, int splits,
                                   int layout, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  A32Plan p = make_a32_plan(dtype, M, B, N, nq, nkv, hd, splits, layout);
  if (!p.ok) return hipErrorInvalidValue;
  if (p.ws > ws_bytes) return hipErrorInvalidValue;
  return run_a32_any(p, M, B, N, nq, nkv, hd, q, row_start, kc, vc, o, ws, s);
}

size_t attention_ws_bytes(int dtype, int M, int B, int N, int nq, int nkv, int hd) {
  const A32Plan p = make_a32_plan(dtype, M, B, N, nq, nkv, hd, 0, -1);
  if (p.ok) return p.ws;
  return make_attn_plan(dtype, M, B, N, nq, nkv, hd).ws;
}

hipError_t launch_attention_cfg(int dtype, int M, int B, int N, int nq, int nkv, int hd,
                                const void* q, const int32_t* row_start, const void* kc,
                                const void* vc, void* o, void* ws, size_t ws_bytes, int splits,
                                int stages, int key_halves, int qblocks, int key_tile,
                                hipStream_t s) {
  if (M <= 0) return hipSuccess;
  AttnPlan p = make_attn_plan_cfg(dtype, M, B, N, nq, nkv, hd, splits, stages, key_halves,
                                  qblocks, key_tile);
  if (p.mfma && p.ws > ws_bytes) {
    p.splits = 1;
    p.keys_per_split = N;
  }
  if (p.mfma) {
    if (hd == 128) return run_attn_mfma<128>(p, M, B, N, nq, nkv, q, row_start, kc, vc, o, ws, s);
    return run_attn_mfma<64>(p, M, B, N, nq, nkv, q, row_start, kc, vc, o, ws, s);
  }
  const int waves = M * nq;
  const int grid = (waves + 3) / 4;
  if (dtype == kBF16)
    attn_generic_kernel<bf16_t><<<grid, 256, 0, s>>>((const bf16_t*)q, row_start, B,
                                                     (const bf16_t*)kc, (const bf16_t*)vc,
                                                     (bf16_t*)o, M, N, nq, nkv, hd);
  else
    attn_generic_kernel<float><<<grid, 256, 0, s>>>((const float*)q, row_start, B,
                                                    (const float*)kc, (const float*)vc,
                                                    (float*)o, M, N, nq, nkv, hd);
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, int M, int B, int N, int nq, int nkv, int hd,
                            const void* q, const int32_t* row_start, const void* kc,
                            const void* vc, void* o, void* ws, size_t ws_bytes, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  A32Plan p = make_a32_plan(dtype, M, B, N, nq, nkv, hd, 0, -1);
  if (p.ok) {
    if (p.ws > ws_bytes) {  // not enough workspace: one key range
      p = make_a32_plan(dtype, M, B, N, nq, nkv, hd, 1, p.layout);
    }
    return run_a32_any(p, M, B, N, nq, nkv, hd, q, row_start, kc, vc, o, ws, s);
  }
  return launch_attention_cfg(dtype, M, B, N, nq, nkv, hd, q, row_start, kc, vc, o, ws, ws_bytes,
                              0, 0, 0, 0, 0, s);
}

size_t attention_cfg_ws_bytes(int dtype, int M, int B, int N, int nq, int nkv, int hd, int splits) {
  return make_attn_plan_cfg(dtype, M, B, N, nq, nkv, hd, splits, 0, 0, 0, 0).ws;
}

}  // namespace dlm

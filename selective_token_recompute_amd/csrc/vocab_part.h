// Partial posterior statistics of one row over a subset of the vocabulary,
// shared by the vocabulary-statistics kernels and the LM-head GEMM's fused
// statistics epilogue.
//
// SureLock page ("Stopping Computation for Converged Tokens in Masked
// Diffusion-LM Decoding"), §2 Methodology, locking condition: the step-wise
// divergence KL(p_t || p_{t-1}) of a position's posterior, gated by its
// confidence.  With an online maximum m over the visited logits z (current)
// and z' (previous step, log-normaliser lse'):
//   S0 = sum e^{z-m},  S1 = sum e^{z-m} (z - z'),   (KL(p_t || p_{t-1}))
//   T1 = sum q (z' - z), q = e^{z' - lse'}          (KL(p_{t-1} || p_t))
// and am = the smallest index attaining m.  Finished per row:
//   lse = m + log S0, conf = 1/S0,
//   KL(p_t || p_{t-1}) = S1/S0 - (lse - lse'),  KL(p_{t-1} || p_t) = T1 + lse - lse'.
// The mask token's column never counts (probability 0).
#pragma once

#include "common.h"
#include "internal.h"

namespace dlm {

struct VocabPart {
  float m, s0, s1, t1;
  int am;
};
static_assert(sizeof(VocabPart) == kVocabPartBytes, "partial layout");

__device__ __forceinline__ VocabPart vpart_empty() {
  return VocabPart{-INFINITY, 0.f, 0.f, 0.f, 0x7fffffff};
}

// Merge of two partials (commutative up to rounding; ties in m keep the
// smaller index).
__device__ __forceinline__ VocabPart vmerge(VocabPart a, VocabPart b) {
  VocabPart r;
  r.m = fmaxf(a.m, b.m);
  const float fa = (a.m == -INFINITY) ? 0.f : __expf(a.m - r.m);
  const float fb = (b.m == -INFINITY) ? 0.f : __expf(b.m - r.m);
  r.s0 = a.s0 * fa + b.s0 * fb;
  r.s1 = a.s1 * fa + b.s1 * fb;
  r.t1 = a.t1 + b.t1;
  if (a.m > b.m) r.am = a.am;
  else if (b.m > a.m) r.am = b.am;
  else r.am = min(a.am, b.am);
  return r;
}

// Folds vocabulary entry v (current logit zv, previous logit zpv) into acc:
// S1 for KLDIR 0, T1 for KLDIR 1, both for KLDIR 2.  Entries must be
// visited in increasing v by one accumulator so that the strict '>' keeps
// the smallest index among equal maxima.
template <int KLDIR>
__device__ __forceinline__ void vpart_visit(VocabPart& acc, int v, float zv, float zpv, bool hp,
                                            float lsep, int mask_id) {
  if (v == mask_id || zv == -INFINITY) {
    if (KLDIR >= 1 && hp && v != mask_id) {
      const float q = __expf(zpv - lsep);
      if (q > 0.f) acc.t1 += q * (zpv - zv);
    }
    return;
  }
  const float d = zv - zpv;
  if (zv > acc.m) {
    const float sc = (acc.m == -INFINITY) ? 0.f : __expf(acc.m - zv);
    acc.s0 = acc.s0 * sc + 1.f;
    if (KLDIR != 1) acc.s1 = acc.s1 * sc + (hp ? d : 0.f);
    acc.m = zv;
    acc.am = v;
  } else {
    const float e = __expf(zv - acc.m);
    acc.s0 += e;
    if (KLDIR != 1 && hp) acc.s1 += e * d;
  }
  if (KLDIR >= 1 && hp) {
    const float q = __expf(zpv - lsep);
    if (q > 0.f) acc.t1 += q * (zpv - zv);
  }
}

__device__ __forceinline__ VocabPart vpart_shfl_xor(const VocabPart& a, int o) {
  VocabPart b;
  b.m = __shfl_xor(a.m, o, 64);
  b.s0 = __shfl_xor(a.s0, o, 64);
  b.s1 = __shfl_xor(a.s1, o, 64);
  b.t1 = __shfl_xor(a.t1, o, 64);
  b.am = __shfl_xor(a.am, o, 64);
  return b;
}

}  // namespace dlm

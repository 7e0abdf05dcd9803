// The draft-token part of one query row, shared by the standalone merge kernel
// (draft.hip) and the fused merge pass (decode.hip), so that both compute it
// with the same operations in the same order.
//
// Within one draft step, draft token t also attends to the step's own draft
// keys 0..t, which are not in the cache yet. For query row (b, t, h) this is
//   lse_d = ln sum_{j<=t} e^{c <q, kd_j>},  out_d = sum_{j<=t} e^{c <q, kd_j> - lse_d} vd_j,
// and the row's result is the log-sum-exp merge of the cache part (out_c, lse_c)
// with it: one softmax over the cached visible keys and draft keys 0..t. c is
// the cache call's logit scale softmax_scale * s(n) ("SharpDraft: Accelerating
// Long-Context Speculative Decoding with Cardinality-Aware Query Scaling",
// Abstract), n the cached visible count. In FOLD the draft keys sit at exact
// positions next to the window, so they join its partition and the merge is
// exact ("FOLD: Position-Free Far Memory with Local Order for Long-Context
// Speculative Decoding", summary).
//
// One wave computes a row: lane l owns channels l*CPL .. l*CPL + CPL - 1,
// CPL = D / 64. Loads and arithmetic are split so that a caller can issue the
// loads early and use them after other work.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "lanes.h"

namespace da {

template <int D, int TM>
struct DraftRow {
  static constexpr int CPL = D / 64;
  float qv[CPL];
  __bf16 kx[TM][CPL], vx[TM][CPL];
};

// Loads of row (b, t, h): the query row and draft keys/values 0..TM-1 of kv
// head kvh. Every load is unconditional, from draft token min(j, t), so that
// no wait is placed under a branch.
template <int D, int TM>
__device__ __forceinline__ void draft_row_load(DraftRow<D, TM>& r, const __bf16* q, const __bf16* kd,
                                               const __bf16* vd, int32_t b, int32_t t, int32_t h, int32_t kvh,
                                               int32_t T, int32_t Hq, int32_t Hkv, int lane) {
  constexpr int CPL = D / 64;
  const int64_t qrow = ((int64_t)b * T + t) * Hq + h;
#pragma unroll
  for (int e = 0; e < CPL; ++e) r.qv[e] = (float)q[qrow * D + lane * CPL + e];
  // draft token 0 of (b, kvh); consecutive draft tokens are Hkv * D elements apart
  const int64_t row0 = ((int64_t)b * T * Hkv + kvh) * D + lane * CPL;
  const __bf16* kp = kd + row0;
  const __bf16* vp = vd + row0;
  const int64_t stride = (int64_t)Hkv * D;
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int64_t off = (j <= t ? j : t) * stride;
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      r.kx[j][e] = kp[off + e];
      r.vx[j][e] = vp[off + e];
    }
  }
}

// The draft part of the row: lse_d and the normalised out_d channels of this
// lane. c: logit scale (natural-log domain). The TM dot products are formed and
// reduced across the wave (lanes.h) for every held key, with no branch between
// them, so that their reductions overlap; keys j > t (loaded from draft token
// t) are then masked.
template <int D, int TM>
__device__ __forceinline__ void draft_row_part(const DraftRow<D, TM>& r, int32_t t, float c, float& lse_d,
                                               float (&od)[D / 64]) {
  // no multiply-add contraction, so that every kernel that inlines this rounds alike
#pragma clang fp contract(off)
  constexpr int CPL = D / 64;
  float lg[TM];
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) part = fmaf(r.qv[e], (float)r.kx[j][e], part);
    lg[j] = part;
  }
#pragma unroll
  for (int j = 0; j < TM; ++j) lg[j] = wave_sum(lg[j]);
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    lg[j] = j <= t ? c * lg[j] : -INFINITY;
    m = fmaxf(m, lg[j]);
  }
  float z = 0.f;
#pragma unroll
  for (int e = 0; e < CPL; ++e) od[e] = 0.f;
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    if (j <= t) {
      const float pj = expf(lg[j] - m);
      z += pj;
#pragma unroll
      for (int e = 0; e < CPL; ++e) od[e] = fmaf(pj, (float)r.vx[j][e], od[e]);
    }
  }
  lse_d = m + logf(z);
#pragma unroll
  for (int e = 0; e < CPL; ++e) od[e] = od[e] / z;
}

// Weights of the cache part and the draft part in the merged row, and the
// merged lse: out = wc * out_c + wd * out_d (draft_merge_out). A cache part with
// no visible key (lse_c = -inf) gets weight 0. The sums of this file are
// written as explicit fmaf so that every kernel that inlines them rounds the
// same way (contraction would otherwise be chosen per kernel).
struct DraftMerge {
  float wc, wd, lse;
};
__device__ __forceinline__ DraftMerge draft_merge(float lse_c, float lse_d) {
  const float top = fmaxf(lse_c, lse_d);
  const float ec = expf(lse_c - top), ed = expf(lse_d - top);
  const float den = ec + ed;
  return DraftMerge{ec / den, ed / den, top + logf(den)};
}

__device__ __forceinline__ float draft_merge_out(const DraftMerge& mg, float out_c, float out_d) {
  return fmaf(mg.wc, mg.wc > 0.f ? out_c : 0.f, mg.wd * out_d);
}

// Logit scale of the draft part for a sequence with n cached visible keys.
// With kappa = 0, s(n) is exactly 1 (n / n0 >= 1, so its logarithm is finite),
// and the logarithm is skipped.
__device__ __forceinline__ float draft_logit_scale(float scale, float kappa, int32_t n, int32_t n0) {
  if (kappa == 0.f) return scale;
  const double sn = 1.0 + (double)kappa * log((double)(n > n0 ? n : n0) / (double)n0);
  return (float)((double)scale * sn);
}

}  // namespace da

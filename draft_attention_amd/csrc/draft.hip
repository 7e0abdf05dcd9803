// Draft-token self-attention merged into the cache attention, for CDNA4 (gfx950).
//
// Within one draft step, draft token t also attends to the step's own draft keys
// 0..t, which are not in the cache yet. draft_attn_decode returns the cache part
// as (out, lse); this kernel computes the causal part over the draft keys and
// merges the two in place: lse <- logaddexp(lse, lse_d) and out <- the matching
// weighted sum. That is exactly one softmax over the cached visible keys and
// the draft keys 0..t. In FOLD the draft keys sit at exact positions next to the
// window, so they join its partition, and the same merge is exact. The logits
// use the cache call's scale softmax_scale * s(n), with n the cached visible
// count ("SharpDraft: Accelerating Long-Context Speculative Decoding with
// Cardinality-Aware Query Scaling", Abstract, scales by the visible keys; the
// few draft keys do not change n here).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "draft_part.h"
#include "host.h"
#include "plan.h"

namespace da {

constexpr int kLenArgs = 32;

struct MergeArgs {
  const __bf16* q;   // [B][T][Hq][D]
  const __bf16* kd;  // [B][T][Hkv][D], rotated at the draft positions
  const __bf16* vd;  // [B][T][Hkv][D]
  const int32_t* ctx_len;
  float* out;        // [B][T][Hq][D], in place
  float* lse;        // [B][T][Hq], in place
  int32_t B, T, Hq, Hkv, G, mode, W, S, n0;
  float kappa, scale;
  // Lengths of a batch of up to kLenArgs sequences, from ctx_len_host, as
  // draft_attn_decode passes them: both calls then take the query scale's n
  // from the same source (larger batches read ctx_len in device memory).
  int32_t nlen;            // B when B <= kLenArgs, else 0
  int32_t len[kLenArgs];
};

// One wave per (sequence, draft token, query head); lane l owns channels
// l*CPL .. l*CPL + CPL - 1. Every load the wave needs (its query row, the cache
// result, draft keys and values 0..t) is issued before any is used, so the call
// costs about one memory round trip; the logits are then reduced across the
// wave one draft key at a time (draft_part.h).
template <int D, int TM>
__global__ __launch_bounds__(64) void merge_draft_kernel(const MergeArgs a) {
  constexpr int CPL = D / 64;
  const int lane = threadIdx.x;
  uint32_t r = blockIdx.x;  // grid = B * T * Hq < 2^31, checked on the host
  const int32_t h = (int32_t)(r % (uint32_t)a.Hq);
  r /= (uint32_t)a.Hq;
  const int32_t t = (int32_t)(r % (uint32_t)a.T);
  const int32_t b = (int32_t)(r / (uint32_t)a.T);
  const int32_t kvh = h / a.G;
  const int64_t qrow = ((int64_t)b * a.T + t) * a.Hq + h;

  DraftRow<D, TM> dr;
  draft_row_load(dr, a.q, a.kd, a.vd, b, t, h, kvh, a.T, a.Hq, a.Hkv, lane);
  float oc[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) oc[e] = a.out[qrow * D + lane * CPL + e];
  const float lse_c = a.lse[qrow];
  const int32_t L = a.nlen > 0 ? a.len[b] : a.ctx_len[b];
  const float c = draft_logit_scale(a.scale, a.kappa, visible_count(L, a.mode, a.W, a.S), a.n0);
  float lse_d, od[CPL];
  draft_row_part(dr, t, c, lse_d, od);
  const DraftMerge mg = draft_merge(lse_c, lse_d);
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    a.out[qrow * D + lane * CPL + e] = draft_merge_out(mg, oc[e], od[e]);
  }
  if (lane == 0) a.lse[qrow] = mg.lse;
}

}  // namespace da

extern "C" int draft_attn_merge_draft(const draft_attn_params* p, const void* q, const void* k_draft,
                                      const void* v_draft, const int32_t* ctx_len_dev, const int32_t* ctx_len_host,
                                      float* out, float* lse, void* stream) {
  using namespace da;
  Prepared pr;
  const int st = prepare(p, ctx_len_host, &pr);
  if (st != DRAFT_ATTN_OK) return st;
  if (p->num_seqs == 0) return DRAFT_ATTN_OK;
  if (p->num_draft_tokens > DRAFT_ATTN_MAX_ROWS) return DRAFT_ATTN_ENOTSUP;
  if (p->out_dtype != DRAFT_ATTN_OUT_F32) return DRAFT_ATTN_ENOTSUP;  // needs the fp32 cache result
  if (!q || !k_draft || !v_draft || !ctx_len_dev || !out || !lse) return DRAFT_ATTN_EINVAL;
  auto mis = [](const void* ptr, uintptr_t al) { return ((uintptr_t)ptr & (al - 1)) != 0; };
  if (mis(q, 16) || mis(k_draft, 16) || mis(v_draft, 16) || mis(out, 8) || mis(lse, 4) || mis(ctx_len_dev, 4))
    return DRAFT_ATTN_EINVAL;
  MergeArgs a;
  a.q = (const __bf16*)q;
  a.kd = (const __bf16*)k_draft;
  a.vd = (const __bf16*)v_draft;
  a.ctx_len = ctx_len_dev;
  a.out = out;
  a.lse = lse;
  a.B = p->num_seqs;
  a.T = p->num_draft_tokens;
  a.Hq = p->num_q_heads;
  a.Hkv = p->num_kv_heads;
  a.G = pr.G;
  a.mode = p->mode;
  a.W = p->window;
  a.S = p->n_sink;
  a.n0 = p->n0;
  a.kappa = p->kappa;
  a.scale = p->softmax_scale;
  a.nlen = p->num_seqs <= kLenArgs ? p->num_seqs : 0;
  for (int32_t b = 0; b < kLenArgs; ++b) a.len[b] = b < a.nlen ? ctx_len_host[b] : 0;
  if ((int64_t)a.B * a.T * a.Hq > 0x7fffffff) return DRAFT_ATTN_EINVAL;
  const uint32_t grid = (uint32_t)((int64_t)a.B * a.T * a.Hq);
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  // The kernel holds draft keys 0..TM-1 in registers: TM is the smallest of 8,
  // 16 and 32 that covers T.
  if (p->head_dim == 64) {
    if (a.T <= 8) merge_draft_kernel<64, 8><<<grid, 64, 0, s>>>(a);
    else if (a.T <= 16) merge_draft_kernel<64, 16><<<grid, 64, 0, s>>>(a);
    else merge_draft_kernel<64, 32><<<grid, 64, 0, s>>>(a);
  } else {
    if (a.T <= 8) merge_draft_kernel<128, 8><<<grid, 64, 0, s>>>(a);
    else if (a.T <= 16) merge_draft_kernel<128, 16><<<grid, 64, 0, s>>>(a);
    else merge_draft_kernel<128, 32><<<grid, 64, 0, s>>>(a);
  }
  if (hipGetLastError() != hipSuccess) return DRAFT_ATTN_EHIP;
  return DRAFT_ATTN_OK;
}

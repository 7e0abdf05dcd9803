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

// The arguments after the leading scalars (which the kernel receives preloaded
// in scalar registers).
struct MergeArgs {
  const int32_t* ctx_len;
  int32_t mode, W, S, n0;
  float kappa, scale;
  // Lengths of a batch of up to kLenArgs sequences, from ctx_len_host, as
  // draft_attn_decode passes them: both calls then take the query scale's n
  // from the same source (larger batches read ctx_len in device memory).
  int32_t len[kLenArgs];
};

// One wave per (sequence b, draft token t, query head h) = (blockIdx.x, .y, .z);
// lane l owns channels l*CPL .. l*CPL + CPL - 1. The sequence's length is read
// first, then every load the wave needs (its query row, the cache result, draft
// keys and values 0..t) is issued before any is used, so the call costs about
// one memory round trip; the logits are then reduced across the wave
// (draft_part.h). HOSTLEN: the length comes with the arguments.
template <int D, int TM, bool HOSTLEN>
__global__ __launch_bounds__(64) void merge_draft_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ kd,
                                                         const __bf16* __restrict__ vd, float* __restrict__ out,
                                                         float* __restrict__ lse, int32_t T, int32_t Hq, int32_t Hkv,
                                                         int32_t G, const MergeArgs a) {
  constexpr int CPL = D / 64;
  const int lane = threadIdx.x;
  const int32_t b = blockIdx.x, t = blockIdx.y, h = blockIdx.z;
  const int32_t L = HOSTLEN ? a.len[b] : a.ctx_len[b];
  const int64_t qrow = ((int64_t)b * T + t) * Hq + h;

  DraftRow<D, TM> dr;
  draft_row_load(dr, q, kd, vd, b, t, h, h / G, T, Hq, Hkv, lane);
  float oc[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) oc[e] = out[qrow * D + lane * CPL + e];
  const float lse_c = lse[qrow];
  const float c = draft_logit_scale(a.scale, a.kappa, visible_count(L, a.mode, a.W, a.S), a.n0);
  float lse_d, od[CPL];
  draft_row_part(dr, t, c, lse_d, od);
  const DraftMerge mg = draft_merge(lse_c, lse_d);
#pragma unroll
  for (int e = 0; e < CPL; ++e) out[qrow * D + lane * CPL + e] = draft_merge_out(mg, oc[e], od[e]);
  if (lane == 0) lse[qrow] = mg.lse;
}

template <int D, int TM>
static void launch_merge(bool hostlen, dim3 grid, hipStream_t s, const __bf16* q, const __bf16* kd,
                         const __bf16* vd, float* out, float* lse, int32_t T, int32_t Hq, int32_t Hkv, int32_t G,
                         const MergeArgs& a) {
  if (hostlen) merge_draft_kernel<D, TM, true><<<grid, 64, 0, s>>>(q, kd, vd, out, lse, T, Hq, Hkv, G, a);
  else merge_draft_kernel<D, TM, false><<<grid, 64, 0, s>>>(q, kd, vd, out, lse, T, Hq, Hkv, G, a);
}

// The kernel holds draft keys 0..TM-1 in registers: TM is the smallest of 8,
// 16 and 32 that covers T.
template <int D>
static void launch_merge_d(bool hostlen, dim3 grid, hipStream_t s, const __bf16* q, const __bf16* kd,
                           const __bf16* vd, float* out, float* lse, int32_t T, int32_t Hq, int32_t Hkv, int32_t G,
                           const MergeArgs& a) {
  if (T <= 8) launch_merge<D, 8>(hostlen, grid, s, q, kd, vd, out, lse, T, Hq, Hkv, G, a);
  else if (T <= 16) launch_merge<D, 16>(hostlen, grid, s, q, kd, vd, out, lse, T, Hq, Hkv, G, a);
  else launch_merge<D, 32>(hostlen, grid, s, q, kd, vd, out, lse, T, Hq, Hkv, G, a);
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
  // grid (B, T, Hq) of 64-thread workgroups: T <= DRAFT_ATTN_MAX_ROWS; the
  // head count must fit the third dimension, and B * 64 threads the first
  if (p->num_q_heads > 65535 || (int64_t)p->num_seqs * 64 > 0xffffffffLL) return DRAFT_ATTN_ENOTSUP;
  MergeArgs a;
  a.ctx_len = ctx_len_dev;
  a.mode = p->mode;
  a.W = p->window;
  a.S = p->n_sink;
  a.n0 = p->n0;
  a.kappa = p->kappa;
  a.scale = p->softmax_scale;
  const bool hostlen = p->num_seqs <= kLenArgs;
  for (int32_t b = 0; b < kLenArgs; ++b) a.len[b] = hostlen && b < p->num_seqs ? ctx_len_host[b] : 0;
  const dim3 grid((uint32_t)p->num_seqs, (uint32_t)p->num_draft_tokens, (uint32_t)p->num_q_heads);
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  auto* qb = (const __bf16*)q;
  auto* kb = (const __bf16*)k_draft;
  auto* vb = (const __bf16*)v_draft;
  const int32_t T = p->num_draft_tokens, Hq = p->num_q_heads, Hkv = p->num_kv_heads;
  if (p->head_dim == 64) launch_merge_d<64>(hostlen, grid, s, qb, kb, vb, out, lse, T, Hq, Hkv, pr.G, a);
  else launch_merge_d<128>(hostlen, grid, s, qb, kb, vb, out, lse, T, Hq, Hkv, pr.G, a);
  if (hipGetLastError() != hipSuccess) return DRAFT_ATTN_EHIP;
  return DRAFT_ATTN_OK;
}

// Draft-head decode attention over a paged KV cache: HIP kernels for CDNA4
// (gfx950) and the draft_attn_decode entry point.
//
// Sources, by page title (sections in brackets):
//   [WMTP] "Windowed-MTP: Removing the Full-Context Draft-KV Tax at Million-Token
//          Context" -- Abstract (full read vs sliding window plus sinks).
//   [FOLD] "FOLD: Position-Free Far Memory with Local Order for Long-Context
//          Speculative Decoding" -- summary and abstract (local window, far memory
//          at one shared position from an unrotated side cache, decoupled softmax).
//   [SD]   "SharpDraft: Accelerating Long-Context Speculative Decoding with
//          Cardinality-Aware Query Scaling" -- Abstract (query scale by visible count).
// The exact definitions this code computes are stated in include/draft_attn.h.
//
// Design. The call is bound by HBM: every visible key costs 4*d bytes of K and V
// read once. Pass 1 deals the 32-key steps (two 16-token blocks) of every
// (sequence, kv head) round-robin to work items of at most C keys (plan.h). A
// 256-thread workgroup streams one item; its four waves take interleaved steps
// of the item and each keeps the whole GQA group x draft-token row set
// (R <= 32 rows) of its kv head in registers, so each K/V byte is loaded
// exactly once:
//   S^T[key][row] = K . Q^T   on v_mfma_f32_16x16x32_bf16 (A = K rows, B = Q rows)
//   online softmax per row    in the MFMA output layout: lane (row = l%16) holds
//                             keys 4*(l/16)+r, so row statistics reduce with two
//                             permlane swaps (lanes l^16, l^32)
//   O^T[chan][row] += V^T . P^T  on the same MFMA: A = V^T comes straight from the
//                             channel-major value block (one 16-byte load = 8
//                             consecutive keys of one channel), B = P in bf16.
// K and V fragments go from HBM to registers with 128-bit nontemporal loads and
// no LDS staging; each wave holds two steps, and a buffer's next step loads
// while the current one computes. The key permutation inside a step is chosen so that the softmax
// output of the Q.K^T product is already the B operand of the P.V product. The
// four waves' states merge through LDS into one record per item and row.
// Pass 2 merges the per-item (max, sums, unnormalised output) records with the
// log-sum-exp rule, then combines FOLD's local and far partitions with beta.
// On the single-launch path there is no pass 2: each workgroup marks its item
// done, and a workgroup that finds every item of its (sequence, kv head) done
// performs that merge itself (records and flags travel through device-scope
// accesses, since the eight XCDs' L2 caches are not coherent with each other).
// Small batches receive their lengths and item offsets with the launch
// arguments, so neither kernel starts with a dependent read of ctx_len, and
// the first sequence's addressing comes in preloaded scalar arguments, so its
// workgroups issue their first loads before the argument block arrives.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <type_traits>

#include "draft_part.h"
#include "host.h"
#include "lanes.h"
#include "plan.h"

namespace da {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxHalfDim = 64;

// Lengths and item prefix of a small batch, passed with the launch so that
// the first dependent memory read of each workgroup (the lengths) is not
// needed: the values arrive with the kernel arguments. nseq = 0 for larger
// batches, whose kernels read ctx_len from device memory instead. The host
// fills this from ctx_len_host, which the contract makes equal to ctx_len_dev.
constexpr int kArgSeqs = 32;
struct SeqTable {
  int32_t nseq;                // B when B <= kArgSeqs, else 0
  int32_t len[kArgSeqs];       // context length of each sequence
  int32_t base[kArgSeqs + 1];  // items (over all kv heads) of the sequences before it
  float c2[kArgSeqs];          // logit scale softmax_scale * s(n) * log2(e) of each sequence
};

// Logit scale in the log2 domain, softmax_scale * s(n) * log2(e), with
// s(n) = 1 + kappa ln(max(n, n0) / n0) formed in fp64 ("SharpDraft: Accelerating
// Long-Context Speculative Decoding with Cardinality-Aware Query Scaling",
// Abstract). The host forms it for the sequences of a small batch; kernels form
// it from ctx_len for larger ones.
__host__ __device__ inline float logit_scale_log2(float scale, float kappa, int32_t n, int32_t n0) {
  const double sn = 1.0 + (double)kappa * log((double)(n > n0 ? n : n0) / (double)n0);
  return (float)((double)scale * sn * 1.4426950408889634);
}

struct Pass1Args {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* ks;
  const int32_t* table;
  const int32_t* ctx_len;
  float4* stat;      // [items][rows_pad]: (max, denominator of acc, plain sum, 0), log2 domain
  float* acc;        // [items][rows_pad][D]: unnormalised partial outputs
  uint8_t* visit;    // optional [B][visit_stride]
  int64_t visit_stride;
  unsigned long long* flags;  // [items] done flags (single launch)
  const __bf16* kd;  // fused call only: draft keys / values [B][T][Hkv][D] (else null)
  const __bf16* vd;
  float* dpart;      // fused call: draft parts, out_d [B*T*Hq][D] then lse_d [B*T*Hq]
  void* out;         // [B][T][Hq][D] fp32 or bf16 (single launch)
  float* lse;        // [B][T][Hq] (single launch)
  uint32_t* status;  // optional device status word (DRAFT_ATTN_STATUS_* bits), or null
  int32_t B, T, Hq, Hkv, G, R, rows_pad, max_blocks, num_blocks;
  int32_t mode, W, S, n0, C, rope, total_items;
  int32_t out_bf16, fold_variant;
  float alpha, kappa, scale, beta;
  SeqTable seqs;
  double omega[kMaxHalfDim];  // RoPE frequencies rope_theta^(-2i/d)
};

struct Pass2Args {
  const float4* stat;
  const float* acc;
  const int32_t* ctx_len;
  void* out;
  float* lse;
  const float* dpart;  // fused call, T <= 8: draft parts written by pass 1 (out_d rows, then lse_d)
  const __bf16* q;     // fused call, T > 8: the draft part's inputs
  const __bf16* kd;
  const __bf16* vd;
  int32_t B, T, Hq, Hkv, G, R, rows_pad;
  int32_t mode, W, S, C, total_items, fold_variant, out_bf16, n0;
  float alpha, beta, kappa, scale;
  SeqTable seqs;
};

// The kernel arguments are read through the scalar cache, and their first
// reads miss: the prologue's reads, each waiting on the one before, would pay
// that miss once per cache line. Reading every 64-byte line once, with
// independent loads and one wait, pays it once (at entry, or, in workgroups
// that start from preloaded arguments, once their first loads are out).
// BYTES: the leading part of the arguments the prologue reads (at most 16
// lines: the loads all issue before the one wait).
template <int BYTES, typename T>
__device__ __forceinline__ void touch_args(const T& a) {
  static_assert(BYTES <= (int)sizeof(T) && BYTES <= 16 * 64, "touched span");
  constexpr int N = (BYTES + 63) / 64;
  const uint32_t* p = reinterpret_cast<const uint32_t*>(&a);
  uint32_t v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = i < N ? p[16 * i] : 0u;
  asm volatile("" ::"s"(v[0]), "s"(v[1]), "s"(v[2]), "s"(v[3]), "s"(v[4]), "s"(v[5]), "s"(v[6]), "s"(v[7]),
               "s"(v[8]), "s"(v[9]), "s"(v[10]), "s"(v[11]), "s"(v[12]), "s"(v[13]), "s"(v[14]), "s"(v[15]));
}

// 2^x on the transcendental unit (the cross-lane reductions are in lanes.h)
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned int pack_bf16(float lo, float hi) {
  const bf16x2 h = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(unsigned int, h);
}

// P from the score layout to the P.V B operand. pv[4t + r] is this lane's
// probability for block t of the step at slot 4(g>>1) + 8(g&1) + r. Swapping the
// upper half-wave of the block-0 values with the lower half-wave of the block-1
// values leaves lane group g holding slots 8(g&1) .. 8(g&1)+7 of block g>>1 in
// order: lanes 0-31 keep their block-0 values and receive those of lane+32;
// lanes 32-63 receive the block-1 values of lane-32 and keep their own.
__device__ __forceinline__ bf16x8 exchange_p(const float (&pv)[8]) {
  const unsigned int a0 = pack_bf16(pv[0], pv[1]), a1 = pack_bf16(pv[2], pv[3]);
  const unsigned int b0 = pack_bf16(pv[4], pv[5]), b1 = pack_bf16(pv[6], pv[7]);
  const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
  const u32x4 w = {s0[0], s1[0], s0[1], s1[1]};
  return __builtin_bit_cast(bf16x8, w);
}

// Items of all sequences before sequence `b` (wave-wide prefix over ctx_len),
// plus the per-kv-head item counts of `b`. Uniform across the wave.
struct SeqInfo {
  int32_t b, base, n, n_main;
};

__device__ __forceinline__ int32_t wave_incl_scan(int32_t x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// Finds the sequence holding global item w; ok = false when w is past the
// device-side item count.
__device__ bool locate_item(int32_t w, const int32_t* __restrict__ ctx_len, int32_t B, int32_t Hkv,
                            int32_t mode, int32_t W, int32_t S, int32_t C, SeqInfo* out) {
  const int lane = threadIdx.x & 63;
  int32_t acc = 0;
  for (int32_t b0 = 0; b0 < B; b0 += 64) {
    const int32_t b = b0 + lane;
    int32_t cnt = 0, nm = 0;
    if (b < B) cnt = seq_items(seq_ranges(ctx_len[b], mode, W, S), C, &nm) * Hkv;
    const int32_t inc = wave_incl_scan(cnt, lane);
    const int32_t total = __shfl(inc, 63, 64);
    if (w < acc + total) {
      const unsigned long long m = __ballot(acc + inc > w);
      const int ln = __ffsll(m) - 1;
      out->b = b0 + ln;
      out->base = acc + __shfl(inc - cnt, ln, 64);
      out->n = __shfl(cnt, ln, 64) / Hkv;
      out->n_main = __shfl(nm, ln, 64);
      return true;
    }
    acc += total;
  }
  return false;
}

// Prefix of item counts over sequences [0, b) and the counts of b.
__device__ void seq_prefix(int32_t b, const int32_t* __restrict__ ctx_len, int32_t Hkv, int32_t mode,
                           int32_t W, int32_t S, int32_t C, SeqInfo* out) {
  const int lane = threadIdx.x & 63;
  int32_t acc = 0;
  for (int32_t b0 = 0; b0 < b; b0 += 64) {
    const int32_t bb = b0 + lane;
    int32_t cnt = 0;
    if (bb < b) cnt = seq_items(seq_ranges(ctx_len[bb], mode, W, S), C, nullptr) * Hkv;
    const int32_t inc = wave_incl_scan(cnt, lane);
    acc += __shfl(inc, 63, 64);
  }
  int32_t nm = 0;
  out->b = b;
  out->base = acc;
  out->n = seq_items(seq_ranges(ctx_len[b], mode, W, S), C, &nm);
  out->n_main = nm;
}

// The same two lookups from the launch's sequence table (t.nseq > 0).
__device__ __forceinline__ bool locate_item_table(int32_t w, const SeqTable& t, int32_t mode, int32_t W, int32_t S,
                                                  int32_t C, SeqInfo* out) {
  if (w >= t.base[t.nseq]) return false;
  int32_t b = 0;
  while (b + 1 < t.nseq && w >= t.base[b + 1]) ++b;
  int32_t nm = 0;
  out->b = b;
  out->base = t.base[b];
  out->n = seq_items(seq_ranges(t.len[b], mode, W, S), C, &nm);
  out->n_main = nm;
  return true;
}

__device__ __forceinline__ void seq_prefix_table(int32_t b, const SeqTable& t, int32_t mode, int32_t W, int32_t S,
                                                 int32_t C, SeqInfo* out) {
  int32_t nm = 0;
  out->b = b;
  out->base = t.base[b];
  out->n = seq_items(seq_ranges(t.len[b], mode, W, S), C, &nm);
  out->n_main = nm;
}

// ---------------------------------------------------------------- pass 1
// A work item (at most C keys of one sequence, kv head and range: the range's
// steps first, first + stride, ...) is streamed by a workgroup of kWaves
// waves; wave w takes the item's steps w, w + kWaves, ... Each wave keeps its
// own online-softmax state; at the end the states
// are merged through LDS and the workgroup writes one record per query row.
constexpr int kWaves = 4;

template <int D>
struct StepRegs {
  bf16x8 k[2][D / 32];  // A operands of the two S^T key tiles, per k-step
  bf16x8 v[D / 16];     // A operands of the O^T channel tiles
  int32_t id0, id1;     // physical blocks of the step whose values are loaded (-1: masked)
  int32_t nid0, nid1;   // physical blocks of the step whose keys were loaded last
};

// Online-softmax state of one wave (log2 domain). l and l1 are lane-partial
// over the four key groups until the end of streaming.
template <int D, int RT>
struct WaveState {
  float m[RT], l[RT], l1[RT];
  f32x4 o[RT][D / 16];
};

template <int D, int RT, bool FAR, bool LO, bool SPLIT>
__device__ __forceinline__ void stream_steps(const Pass1Args& a, const int32_t* sbid, int32_t b, int32_t kvh,
                                             const Item& it, float c2,
                                             const bf16x8 (&qh)[RT][D / 32], const bf16x8 (&ql)[RT][D / 32],
                                             const bf16x8 (&qm)[RT][D / 32],
                                             WaveState<D, RT>& st) {
  constexpr int KS = D / 32, NT = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, i16 = lane & 15, g = lane >> 4;
  const __bf16* __restrict__ kpool = FAR ? a.ks : a.k;
  const __bf16* __restrict__ vpool = a.v;
  const int32_t nsteps = it.steps;
  const int32_t ka = it.a, ke = it.e;
  const int32_t vmark = it.part + 1;
  // Key tile t of a step is block t of the step; MFMA row i reads slot
  // pi(i) = (i & 3) + 4*((i >> 3) & 1) + 8*((i >> 2) & 1). In the key layout
  // [c8][slot][8] one load instruction (fixed k-step) then covers channel groups
  // 4ks..4ks+3 of all 16 slots: 1 KiB contiguous. The S^T output lane (row, g)
  // holds slots 4(g>>1) + 8(g&1) + r of each block; one permlane32 swap turns
  // that into slots 8(g&1) .. +7 of block g>>1, the value operand's key order.
  const int32_t kslot = (i16 & 3) + 4 * ((i16 >> 3) & 1) + 8 * ((i16 >> 2) & 1);
  const int32_t srel = 4 * (g >> 1) + 8 * (g & 1);  // first slot of this lane's score keys
  const bool vhi = (g >> 1) != 0;    // value keys 8g..8g+7 live in the second block for g >= 2
  const bool sharp = FAR && (a.alpha != 1.f);
  const float alpha = a.alpha;

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    st.m[rt] = -INFINITY;
    st.l[rt] = 0.f;
    st.l1[rt] = 0.f;
#pragma unroll
    for (int n = 0; n < NT; ++n) st.o[rt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // K/V are read once per call: nontemporal loads keep them from displacing
  // anything in the caches.
  // A step's keys and values load separately: in the main loop the keys of a
  // buffer's next step go in as soon as the Q.K^T products of its current step
  // have read theirs (issue_k, before that step's softmax), the values once its
  // P.V is done (issue_v). So 24 to 32 of a wave's 16-byte loads stay in flight
  // while it computes, with the registers of two steps.
  auto issue_k = [&](int32_t s, StepRegs<D>& r) {
    // Every lane reads the same two ids; making them wave-uniform lets the
    // block base addresses and the step's mask test live in scalar registers.
    r.nid0 = __builtin_amdgcn_readfirstlane(sbid[2 * s]);
    r.nid1 = __builtin_amdgcn_readfirstlane(sbid[2 * s + 1]);
    // masked block: read block 0 (in bounds), values discarded
    const int32_t kid0 = r.nid0 < 0 ? 0 : r.nid0;
    const int32_t kid1 = r.nid1 < 0 ? 0 : r.nid1;
    const size_t krow = (size_t)(g * 16 + kslot) * 8;
    const __bf16* kp0 = kpool + (size_t)((int64_t)kid0 * a.Hkv + kvh) * (D * 16) + krow;
    const __bf16* kp1 = kpool + (size_t)((int64_t)kid1 * a.Hkv + kvh) * (D * 16) + krow;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      r.k[0][ks] = __builtin_nontemporal_load((const bf16x8*)(kp0 + ks * 512));
      r.k[1][ks] = __builtin_nontemporal_load((const bf16x8*)(kp1 + ks * 512));
    }
  };
  auto issue_v = [&](StepRegs<D>& r) {
    r.id0 = r.nid0;
    r.id1 = r.nid1;
    int32_t vid = vhi ? r.id1 : r.id0;
    vid = vid < 0 ? 0 : vid;
    const __bf16* vp = vpool + ((size_t)((int64_t)vid * a.Hkv + kvh) * D + i16) * 16 + 8 * (g & 1);
#pragma unroll
    for (int n = 0; n < NT; ++n) r.v[n] = __builtin_nontemporal_load((const bf16x8*)(vp + n * 256));
  };
  auto issue = [&](int32_t s, StepRegs<D>& r) {
    issue_k(s, r);
    issue_v(r);
  };
  auto no_mid = [] {};

  // mid() runs once the step's Q.K^T products have read r.k.
  auto compute = [&](int32_t s, StepRegs<D>& r, auto&& mid) {
    const int32_t key0 = item_step_key(it, s);
    const bool clean = key0 >= ka && key0 + 32 <= ke && r.id0 >= 0 && r.id1 >= 0;
    // key (relative to key0) is scored iff its block is valid and it lies in the range
    auto key_ok = [&](int32_t rel) {
      const int32_t id = rel >= 16 ? r.id1 : r.id0;
      const int32_t key = key0 + rel;
      return id >= 0 && key >= ka && key < ke;
    };
    if (a.visit != nullptr && lane < 32 && key_ok(lane))
      a.visit[(int64_t)b * a.visit_stride + key0 + lane] = (uint8_t)vmark;
    if (!clean) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (!key_ok(8 * g + e)) {
#pragma unroll
          for (int n = 0; n < NT; ++n) r.v[n][e] = (__bf16)0.f;
        }
      }
    }
    // S^T tiles
    f32x4 sc[2][RT];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.k[t][ks], qh[rt][ks], c, 0, 0, 0);
          if (LO) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.k[t][ks], qm[rt][ks], c, 0, 0, 0);
          if (LO) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.k[t][ks], ql[rt][ks], c, 0, 0, 0);
        }
        sc[t][rt] = c;
      }
    mid();
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float x[8];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) x[4 * t + rr] = sc[t][rt][rr] * c2;
      if (!clean) {  // wave-uniform: only steps at a range edge or with a missing block
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            if (!key_ok(16 * t + srel + rr)) x[4 * t + rr] = -INFINITY;
      }
      float mx = x[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
      mx = pair_max32(pair_max16(mx));
      const float mnew = fmaxf(st.m[rt], mx);
      const float mref = mnew == -INFINITY ? 0.f : mnew;
      const float corr = ex2(st.m[rt] - mref);
      float pv[8];
      float psum = 0.f;
      if (sharp) {
        const float corr_a = ex2(alpha * (st.m[rt] - mref));
        float pasum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d0 = x[e] - mref;
          const float p1 = ex2(d0);
          const float pa = ex2(alpha * d0);
          psum += p1;
          pasum += pa;
          pv[e] = pa;
        }
        st.l1[rt] = st.l1[rt] * corr + psum;
        st.l[rt] = st.l[rt] * corr_a + pasum;
#pragma unroll
        for (int n = 0; n < NT; ++n) st.o[rt][n] *= corr_a;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = ex2(x[e] - mref);
          psum += p;
          pv[e] = p;
        }
        st.l[rt] = st.l[rt] * corr + psum;
#pragma unroll
        for (int n = 0; n < NT; ++n) st.o[rt][n] *= corr;
      }
      st.m[rt] = mnew;
      const bf16x8 pb = exchange_p(pv);
#pragma unroll
      for (int n = 0; n < NT; ++n)
        st.o[rt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.v[n], pb, st.o[rt][n], 0, 0, 0);
    }
  };

  int32_t s = wave;
  if (s < nsteps) {
    // Two buffers, each holding one of this wave's steps. In the FULL and
    // WINDOW kernels (SPLIT) a buffer's next step loads while its current step
    // computes: keys after Q.K^T, values after P.V. In each loop body every
    // load is unconditional, so the compiler's wait before each product covers
    // only that product's own loads. (With a load under a condition inside the
    // loop, the wait had to cover the newest loads as well, which left almost
    // none in flight during it.) The last steps run after the loop.
    StepRegs<D> ra, rb;
    issue(s, ra);
    if constexpr (SPLIT) {
      if (s + kWaves < nsteps) issue(s + kWaves, rb);
      while (s + 3 * kWaves < nsteps) {
        compute(s, ra, [&] { issue_k(s + 2 * kWaves, ra); });
        issue_v(ra);
        compute(s + kWaves, rb, [&] { issue_k(s + 3 * kWaves, rb); });
        issue_v(rb);
        s += 2 * kWaves;
      }
      if (s + 2 * kWaves < nsteps) {
        compute(s, ra, [&] { issue_k(s + 2 * kWaves, ra); });
        issue_v(ra);
        compute(s + kWaves, rb, no_mid);
        compute(s + 2 * kWaves, ra, no_mid);
      } else if (s + kWaves < nsteps) {
        compute(s, ra, no_mid);
        compute(s + kWaves, rb, no_mid);
      } else {
        compute(s, ra, no_mid);
      }
    } else if constexpr (!LO) {
      // (the FOLD kernels: whole-step loads, one step ahead; with the split
      // loads above their far path and the 16-sequence FOLD batch measured
      // 0.5-1% slower)
      while (s + 2 * kWaves < nsteps) {
        issue(s + kWaves, rb);
        compute(s, ra, no_mid);
        issue(s + 2 * kWaves, ra);
        compute(s + kWaves, rb, no_mid);
        s += 2 * kWaves;
      }
      if (s + kWaves < nsteps) {
        issue(s + kWaves, rb);
        compute(s, ra, no_mid);
        compute(s + kWaves, rb, no_mid);
      } else {
        compute(s, ra, no_mid);
      }
    } else {
      // The rotated far query's mid and lo terms take 64 more registers at
      // two row tiles; the loops above then run short of registers, so this
      // path keeps one compute per buffer and the stricter wait (measured
      // faster here).
      for (;;) {
        if (s + kWaves < nsteps) issue(s + kWaves, rb);
        compute(s, ra, no_mid);
        s += kWaves;
        if (s >= nsteps) break;
        if (s + kWaves < nsteps) issue(s + kWaves, ra);
        compute(s, rb, no_mid);
        s += kWaves;
        if (s >= nsteps) break;
      }
    }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    st.l[rt] = pair_add32(pair_add16(st.l[rt]));
    st.l1[rt] = sharp ? pair_add32(pair_add16(st.l1[rt])) : st.l[rt];
  }
}

// Dynamic LDS of pass 1: block ids of the item, then the merge buffers (row
// maxima, sums and partial outputs of each wave).
__host__ __device__ inline size_t pass1_sbid_bytes(int32_t C) { return ((size_t)(C / 16 + 2) * 4 + 15) & ~(size_t)15; }
__host__ __device__ inline size_t pass1_lds_bytes(int32_t C, int32_t rows_pad, int32_t D) {
  return pass1_sbid_bytes(C) + (size_t)kWaves * rows_pad * (sizeof(float) + sizeof(float2)) +
         (size_t)kWaves * rows_pad * (D + 4) * sizeof(float);
}

// Record access on the single-launch path. Work items of one group run on
// different XCDs, whose L2 caches are not coherent with each other. Records
// are therefore written and read as 8-byte device-scope accesses, which go to
// the device's coherence point directly, instead of plain accesses behind
// device-scope fences, which write back or invalidate a whole L2 each time.
// Each pair of floats travels as one 64-bit word.
__device__ __forceinline__ void store_dev4(float* p, float x, float y, float z, float w) {
  unsigned long long* q = (unsigned long long*)p;
  __hip_atomic_store(q, ((unsigned long long)__float_as_uint(y) << 32) | __float_as_uint(x), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, ((unsigned long long)__float_as_uint(w) << 32) | __float_as_uint(z), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float4 load_dev4(const float* p) {
  unsigned long long* q = (unsigned long long*)p;
  const unsigned long long a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned long long b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float4(__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)), __uint_as_float((uint32_t)b),
                     __uint_as_float((uint32_t)(b >> 32)));
}

// Partition weights of one query row from its reduced statistics (log2 domain:
// main maximum M and sum Ls; far maximum MF, plain sum ZF and sharpened sum
// ZFa). The local window weighs Z_L = 2^M Ls; the far memory weighs e^beta Z_F
// (default), e^beta Z_Fa (joint softmax) or e^beta Z_Fa^(1/alpha) (one virtual
// key), with Z_F = 2^MF ZF and Z_Fa = 2^(alpha MF) ZFa. Returns the factors fl
// and ff that turn the scaled partial-output sums of each partition into the
// output, and the row's lse (natural log).
struct RowCombine {
  float fl, ff, lse;
};
__device__ __forceinline__ RowCombine combine_row(float M, float MF, float Ls, float ZF, float ZFa, float alpha,
                                                  float beta, int32_t fold_variant) {
  const float lwL = Ls > 0.f ? M + log2f(Ls) : -INFINITY;
  float lwF = -INFINITY;
  if (ZF > 0.f) {
    const float far_log2 = fold_variant == DRAFT_ATTN_FOLD_JOINT     ? alpha * MF + log2f(ZFa)
                           : fold_variant == DRAFT_ATTN_FOLD_VIRTUAL ? MF + log2f(ZFa) / alpha
                                                                     : MF + log2f(ZF);
    lwF = beta * kLog2e + far_log2;
  }
  const float top = fmaxf(lwL, lwF);
  RowCombine r{0.f, 0.f, -INFINITY};
  if (top != -INFINITY) {
    const float wL = exp2f(lwL - top), wF = exp2f(lwF - top);
    const float den = wL + wF;
    r.fl = wL > 0.f ? wL / (den * Ls) : 0.f;
    r.ff = wF > 0.f ? wF / (den * ZFa) : 0.f;
    r.lse = (top + log2f(den)) * kLn2;
  }
  return r;
}

__device__ __forceinline__ void store_out4(void* out, bool bf16, int64_t off, float4 v) {
  if (bf16) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 h;
    h[0] = (__bf16)v.x;
    h[1] = (__bf16)v.y;
    h[2] = (__bf16)v.z;
    h[3] = (__bf16)v.w;
    *(bf16x4*)((__bf16*)out + off) = h;
  } else {
    *(float4*)((float*)out + off) = v;
  }
}

// ---------------------------------------------------------------- single-launch merge
// Run by a workgroup that found every item of its (sequence, kv head) done: it
// merges the group's n item records (items i0 .. i0 + n - 1, the first nm of
// them local) into out and lse for every query row of the group. Thread
// (row = tid / 8, sub = tid % 8) reduces the statistics of items sub, sub + 8,
// ... of one row and stages each item's final scale in s_sc; then thread tid
// sums the partial outputs of the (row, channel quad) pairs tid + 256 j, 16
// float4 loads per thread and round.
constexpr int kGroupItems = DRAFT_ATTN_MAX_GROUP_ITEMS;
// Done-flag value: an arbitrary 64-bit pattern (the first 64 fraction bits of
// sqrt(2)), which plain data left in a workspace is not expected to hold.
constexpr unsigned long long kDoneFlag = 0x6A09E667F3BCC908ull;

template <int D, int RT>
__device__ __forceinline__ void single_merge(const Pass1Args& a, int32_t b, int32_t kvh, int64_t i0, int32_t n,
                                             int32_t nm, float* s_sc) {
  constexpr int NQ = D / 4;
  constexpr int ROWS = 16 * RT;
  constexpr int NPJ = ROWS * NQ / 256;  // (row, channel quad) pairs per thread
  constexpr int IB = 16 / NPJ;          // items per round of partial-output loads
  // (Rounds three times as large, at head dim 128, measured slower: 128K
  // window single launch 16.2 -> 17.9 us, the 16-sequence batch +0.4%.)
  constexpr int SPT = kGroupItems / 8;
  static_assert(NPJ * 256 == ROWS * NQ, "pairs must tile the workgroup");
  const int tid = threadIdx.x;
  const size_t rp = (size_t)a.rows_pad;
  const int row = tid >> 3, sub = tid & 7;
  const bool row_ok = row < a.R;
  const float alpha = a.alpha;

  float4 v[NPJ][IB];
  auto load_round = [&](int32_t ib) {
#pragma unroll
    for (int j = 0; j < NPJ; ++j) {
      const int pair = tid + 256 * j;
      const int prow = pair / NQ, q4 = pair - prow * NQ;
#pragma unroll
      for (int k = 0; k < IB; ++k) {
        // unconditional load from a clamped index (see the merge kernel)
        const int32_t it = ib + k;
        const bool ok = prow < a.R && it < n;
        const int32_t itc = it < n ? it : n - 1, prc = prow < a.R ? prow : a.R - 1;
        const float4 x = load_dev4(a.acc + ((size_t)(i0 + itc) * rp + prc) * D + 4 * q4);
        v[j][k] = ok ? x : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  // The first round does not depend on the statistics: issue it first.
  load_round(0);
  float4 st[SPT];
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    const int it = sub + 8 * k;
    const int itc = it < n ? it : n - 1, rc = row_ok ? row : a.R - 1;
    const float4 x = load_dev4((const float*)&a.stat[(size_t)(i0 + itc) * rp + rc]);
    st[k] = row_ok && it < n ? x : make_float4(-INFINITY, 0.f, 0.f, 0.f);
  }
  float M = -INFINITY, MF = -INFINITY;
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    if (sub + 8 * k < nm) M = fmaxf(M, st[k].x);
    else MF = fmaxf(MF, st[k].x);
  }
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) {
    M = fmaxf(M, __shfl_xor(M, off, 64));
    MF = fmaxf(MF, __shfl_xor(MF, off, 64));
  }
  float Ls = 0.f, ZF = 0.f, ZFa = 0.f;
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    const float m = st[k].x;
    if (m == -INFINITY) continue;
    if (sub + 8 * k < nm) {
      Ls += st[k].y * exp2f(m - M);
    } else {
      ZF += st[k].z * exp2f(m - MF);
      ZFa += st[k].y * exp2f(alpha * (m - MF));
    }
  }
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) {
    Ls += __shfl_xor(Ls, off, 64);
    ZF += __shfl_xor(ZF, off, 64);
    ZFa += __shfl_xor(ZFa, off, 64);
  }
  const RowCombine cb = combine_row(M, MF, Ls, ZF, ZFa, alpha, a.beta, a.fold_variant);
  if (row < ROWS) {
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int it = sub + 8 * k;
      if (it >= n) continue;
      const float m = st[k].x;
      float sc = 0.f;
      if (m != -INFINITY) sc = it < nm ? exp2f(m - M) * cb.fl : exp2f(alpha * (m - MF)) * cb.ff;
      s_sc[row * kGroupItems + it] = sc;
    }
  }
  auto out_row = [&](int32_t r) {
    const int32_t t = r / a.G;
    const int32_t head = kvh * a.G + (r - t * a.G);
    return (int64_t)(b * a.T + t) * a.Hq + head;
  };
  if (sub == 0 && row_ok) a.lse[out_row(row)] = cb.lse;
  __syncthreads();

  float4 acc[NPJ];
#pragma unroll
  for (int j = 0; j < NPJ; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int32_t ib = 0; ib < n; ib += IB) {
    if (ib > 0) load_round(ib);
#pragma unroll
    for (int j = 0; j < NPJ; ++j) {
      const int prow = (tid + 256 * j) / NQ;
#pragma unroll
      for (int k = 0; k < IB; ++k) {
        const int32_t it = ib + k;
        if (prow < a.R && it < n) {
          const float sc = s_sc[prow * kGroupItems + it];
          acc[j].x += sc * v[j][k].x;
          acc[j].y += sc * v[j][k].y;
          acc[j].z += sc * v[j][k].z;
          acc[j].w += sc * v[j][k].w;
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NPJ; ++j) {
    const int pair = tid + 256 * j;
    const int prow = pair / NQ, q4 = pair - prow * NQ;
    if (prow < a.R) store_out4(a.out, a.out_bf16 != 0, out_row(prow) * D + 4 * q4, acc[j]);
  }
}

// Fused call: the draft part of query row r = (b * T + t) * Hq + h, formed by
// one wave of an extra pass-1 workgroup and stored for the merge kernel.
template <int D, int TM>
__device__ __forceinline__ void draft_part_store(const Pass1Args& a, int32_t r, int lane) {
  const int32_t h = r % a.Hq, bt = r / a.Hq;
  const int32_t t = bt % a.T, b = bt / a.T;
  DraftRow<D, TM> dr;
  draft_row_load(dr, a.q, a.kd, a.vd, b, t, h, h / a.G, a.T, a.Hq, a.Hkv, lane);
  const int32_t L = a.seqs.nseq > 0 ? a.seqs.len[b] : a.ctx_len[b];
  const float c = draft_logit_scale(a.scale, a.kappa, visible_count(L, a.mode, a.W, a.S), a.n0);
  float lse_d, od[D / 64];
  draft_row_part(dr, t, c, lse_d, od);
#pragma unroll
  for (int e = 0; e < D / 64; ++e) a.dpart[(int64_t)r * D + lane * (D / 64) + e] = od[e];
  if (lane == 0) a.dpart[(int64_t)a.B * a.T * a.Hq * D + r] = lse_d;
}

// Waves per SIMD, i.e. workgroups per CU, that the kernel is compiled for; the
// host planner's resident_per_cu() uses the same numbers.
constexpr int pass1_occupancy(int D, int RT) { return D == 64 ? (RT == 1 ? 3 : 2) : 1; }

template <int D, int RT, bool FOLDK, bool SINGLE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(pass1_occupancy(D, RT))))
void pass1_kernel(const __bf16* __restrict__ q, const int32_t* __restrict__ table, int32_t first_items,
                  int32_t L_first, int32_t mode_g_t, int32_t W, int32_t S, int32_t C, int32_t Hq,
                  int32_t max_blocks, int32_t num_blocks, const Pass1Args a) {
  constexpr int KS = D / 32, NT = D / 16, OS = D + 4;  // OS: padded LDS row stride (floats)
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int kArgBytes = (int)offsetof(Pass1Args, omega);  // the rotation frequencies, last, only FOLD reads
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, i16 = lane & 15, g = lane >> 4;
  const int32_t w = blockIdx.x;
  // Leading scalar arguments, which the hardware places in registers before
  // the kernel starts: the query, the block table, the launch's shape (mode,
  // G and T packed in one word) and the first sequence's length and item
  // count over its kv heads (0: no such shortcut). The first sequence's
  // workgroups find their item, query rows and table row from these alone and
  // issue those loads before the argument block arrives; the others read it
  // first.
  const int32_t mode = mode_g_t & 0xff, G = (mode_g_t >> 8) & 0xff, T = mode_g_t >> 16, R = T * G;
  const bool first = w < first_items;
  SeqInfo si;
  int32_t L = L_first;
  if (first) {
    int32_t nm = 0;
    si.b = 0;
    si.base = 0;
    si.n = seq_items(seq_ranges(L_first, mode, W, S), C, &nm);
    si.n_main = nm;
  } else {
    touch_args<kArgBytes>(a);
    if (!SINGLE && a.kd != nullptr && w >= a.total_items) {
      // Fused call: workgroups past the work items form the draft parts, one
      // query row per wave (they do not depend on the cache part, so the merge
      // kernel only loads them).
      // (The host adds these workgroups only for T <= 8: holding 16 or 32 draft
      // keys here raised the register demand of the whole kernel into spills.)
      const int32_t r = (w - a.total_items) * kWaves + wave;
      if (r < a.B * a.T * a.Hq) draft_part_store<D, 8>(a, r, lane);
      return;
    }
    const bool found = a.seqs.nseq > 0 ? locate_item_table(w, a.seqs, mode, W, S, C, &si)
                                       : locate_item(w, a.ctx_len, a.B, a.Hkv, mode, W, S, C, &si);
    if (!found) {
      // Only when ctx_len on the device disagrees with the host mirror: leave a
      // neutral record so the merge stays defined, and report it.
      const int32_t rp = a.rows_pad;
      if (tid == 0 && a.status != nullptr) atomicOr(a.status, (uint32_t)DRAFT_ATTN_STATUS_LENGTHS);
      if (tid < a.R) a.stat[(size_t)w * rp + tid] = make_float4(-INFINITY, 0.f, 0.f, 0.f);
      for (int32_t i = tid; i < a.R * D; i += 256) a.acc[(size_t)w * rp * D + i] = 0.f;
      return;
    }
    L = a.seqs.nseq > 0 ? a.seqs.len[si.b] : a.ctx_len[si.b];
  }
  int32_t* sbid = (int32_t*)smem;
  const int32_t b = si.b;
  const int32_t rel = w - si.base;
  const int32_t kvh = rel / si.n, kidx = rel - kvh * si.n;
  const Ranges rg = seq_ranges(L, mode, W, S);
  const Item it = item_of(rg, kidx, C);

  // Query rows of this kv head (loaded before the block table so both loads are
  // in flight together): row = t * G + (h - kvh * G), zero-padded to 16 * RT.
  bf16x8 qh[RT][KS], ql[RT][KS], qm[RT][KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int32_t row = 16 * rt + i16;
    const bool ok = row < R;
    const int32_t t = ok ? row / G : 0;
    const int32_t head = kvh * G + (ok ? row - t * G : 0);
    const __bf16* qp = q + ((int64_t)(b * T + t) * Hq + head) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 z;
#pragma unroll
      for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.f;
      const bf16x8 qv = *(const bf16x8*)(qp + 32 * ks);  // qp is a valid row even when !ok
      qh[rt][ks] = ok ? qv : z;
      ql[rt][ks] = z;
      qm[rt][ks] = z;
    }
  }

  // Block ids of the item's steps (two per step), validated; the second block
  // of a range's last step may lie past the range and reads as absent. Each
  // thread issues up to eight table loads before it waits for any (a loop of
  // load-then-store waits one round trip per id). A slot with no id loads
  // entry 0 of the row, which exists, and drops it. Every block staged here
  // holds at least one key of the range, so an id outside [0, num_blocks) is a
  // bad table entry: its keys are masked, and the status word reports it.
  const int32_t nblk = 2 * it.steps;
  const int32_t last_blk = (it.e - 1) >> 4;
  const int32_t* trow = table + (int64_t)b * max_blocks;
  constexpr int kStageUnroll = 8;
  bool bad_id = false;
  for (int32_t j0 = 0; j0 < nblk; j0 += 256 * kStageUnroll) {
    int32_t ids[kStageUnroll];
#pragma unroll
    for (int u = 0; u < kStageUnroll; ++u) {
      const int32_t j = j0 + 256 * u + tid;
      const int32_t blk = (item_step_key(it, j >> 1) >> 4) + (j & 1);
      const bool ok = j < nblk && blk <= last_blk && blk < max_blocks;
      const int32_t id = trow[ok ? blk : 0];
      const bool valid = id >= 0 && id < num_blocks;
      bad_id |= ok && !valid;
      ids[u] = ok && valid ? id : -1;
    }
    // the argument block, read while the first ids and the query are in flight
    if (first && j0 == 0) touch_args<kArgBytes>(a);
#pragma unroll
    for (int u = 0; u < kStageUnroll; ++u) {
      const int32_t j = j0 + 256 * u + tid;
      if (j < nblk) sbid[j] = ids[u];
    }
  }
  if (first && nblk <= 0) touch_args<kArgBytes>(a);
  if (bad_id && a.status != nullptr) atomicOr(a.status, (uint32_t)DRAFT_ATTN_STATUS_BAD_BLOCK);
  __syncthreads();

  // Logit scale in the log2 domain: softmax_scale * s(n) * log2(e).
  const float c2 = a.seqs.nseq > 0 ? a.seqs.c2[b]
                                   : logit_scale_log2(a.scale, a.kappa, visible_count(L, mode, W, S), a.n0);
  const int32_t rp = a.rows_pad;
  float* s_m = (float*)(smem + pass1_sbid_bytes(C));  // [kWaves][rp] row maxima
  float2* s_l = (float2*)(s_m + kWaves * rp);         // [kWaves][rp] (acc denominator, plain sum)
  float* s_o = (float*)(s_l + kWaves * rp);            // [kWaves][rp][OS] partial outputs

  WaveState<D, RT> st;
  const bool far_part = FOLDK && it.part == kPartFar;
  if (far_part) {
    if (a.rope == DRAFT_ATTN_ROPE_NEOX) {
      // Far query q_far = R(-P_v) q, P_v = L - W - 1 [FOLD]. Lane (i16, g) holds
      // channels 32ks + 8g + e; the rotation partner d/2 away sits in k-step
      // ks + KS/2 of the same lane. Angles are formed and reduced mod 2*pi in fp64;
      // the fp32 rotated value is split into three bf16 terms (hi, mid, lo) so
      // the Q.K^T product keeps q_far's 24 significant bits. (Two terms keep
      // about 17, which at far logits of hundreds of nats moves lse by a few
      // 1e-4; the third product costs no measurable time here.)
      const double pv = (double)(L - a.W - 1);
#pragma unroll
      for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 32 * ks + 8 * g + e;
          const double ang = -pv * a.omega[i];
          const double kq = rint(ang * 0.15915494309189535);
          double red = fma(-kq, 6.283185307179586, ang);
          red = fma(-kq, 2.4492935982947064e-16, red);
          float sn_, cs_;
          sincosf((float)red, &sn_, &cs_);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const float x1 = (float)qh[rt][ks][e];
            const float x2 = (float)qh[rt][ks + KS / 2][e];
            const float y1 = x1 * cs_ - x2 * sn_;
            const float y2 = x1 * sn_ + x2 * cs_;
            const __bf16 h1 = (__bf16)y1, h2 = (__bf16)y2;
            qh[rt][ks][e] = h1;
            qh[rt][ks + KS / 2][e] = h2;
            const __bf16 m1 = (__bf16)(y1 - (float)h1), m2 = (__bf16)(y2 - (float)h2);
            qm[rt][ks][e] = m1;
            qm[rt][ks + KS / 2][e] = m2;
            ql[rt][ks][e] = (__bf16)(y1 - (float)h1 - (float)m1);
            ql[rt][ks + KS / 2][e] = (__bf16)(y2 - (float)h2 - (float)m2);
          }
        }
      stream_steps<D, RT, true, true, false>(a, sbid, b, kvh, it, c2, qh, ql, qm, st);
    } else {
      stream_steps<D, RT, true, false, false>(a, sbid, b, kvh, it, c2, qh, ql, qm, st);
    }
  } else {
    stream_steps<D, RT, false, false, !FOLDK>(a, sbid, b, kvh, it, c2, qh, ql, qm, st);
  }

  // ---- merge the waves. Wave rt (rt < RT) combines row tile rt: every wave
  // publishes its row maxima and sums, and the partial outputs of the tiles it
  // does not combine, in LDS; after one barrier each combining wave rescales
  // the four states of its tile to the common row maxima, sums them and writes
  // the tile's records (one (stat, acc) pair per query row) itself.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = 16 * rt + i16;
    if (g == 0) {
      s_m[wave * rp + row] = st.m[rt];
      s_l[wave * rp + row] = make_float2(st.l[rt], st.l1[rt]);
    }
    if (wave != rt) {
#pragma unroll
      for (int n2 = 0; n2 < NT; ++n2) *(f32x4*)(s_o + (wave * rp + row) * OS + 16 * n2 + 4 * g) = st.o[rt][n2];
    }
  }
  __syncthreads();
  const size_t rowbase = (size_t)w * rp;
  // (the tile index must be a compile-time constant: a register array indexed
  // by the wave number would be moved to scratch memory)
  auto combine_tile = [&](auto tile) {
    constexpr int rt = decltype(tile)::value;
    const bool sharp = far_part && (a.alpha != 1.f);
    const int row = 16 * rt + i16;
    float mk[kWaves], fk[kWaves], fak[kWaves];
#pragma unroll
    for (int k = 0; k < kWaves; ++k) mk[k] = s_m[k * rp + row];
    float M = mk[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) M = fmaxf(M, mk[k]);
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      const float d0 = M == -INFINITY ? -INFINITY : mk[k] - M;
      fk[k] = ex2(d0);
      fak[k] = sharp ? ex2(a.alpha * d0) : fk[k];
    }
    float Lsum = 0.f, L1sum = 0.f;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      const float2 l = s_l[k * rp + row];
      Lsum += l.x * fak[k];
      L1sum += l.y * fk[k];
    }
    const bool live = row < a.R;
#pragma unroll
    for (int n2 = 0; n2 < NT; ++n2) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < kWaves; ++k) {
        const f32x4 o = k == rt ? st.o[rt][n2] : *(const f32x4*)(s_o + (k * rp + row) * OS + 16 * n2 + 4 * g);
        v += o * fak[k];
      }
      float* dst = a.acc + (rowbase + row) * D + 16 * n2 + 4 * g;
      if (live) {
        if constexpr (SINGLE) store_dev4(dst, v[0], v[1], v[2], v[3]);
        else *(f32x4*)dst = v;
      }
    }
    if (live && g == 0) {
      if constexpr (SINGLE) store_dev4((float*)&a.stat[rowbase + row], M, Lsum, L1sum, 0.f);
      else a.stat[rowbase + row] = make_float4(M, Lsum, L1sum, 0.f);
    }
  };
  if (wave == 0) combine_tile(std::integral_constant<int, 0>{});
  if constexpr (RT > 1) {
    if (wave == 1) combine_tile(std::integral_constant<int, 1>{});
  }
  if constexpr (SINGLE) {
    // Mark this item done, then look at the done flags of the whole group. Each
    // workgroup's flag store completes before it reads the flags, so of any two
    // late workgroups the second sees the first's flag: the last to arrive, at
    // least, finds every flag set. Workgroups that finish together often all do;
    // each of them then exchanges the group's first flag for 0, and only the one
    // that gets kDoneFlag back merges the group (and clears the other flags).
    // Flags hold kDoneFlag or 0 (every call leaves them 0); any other value, as
    // in a fresh workspace, reads as not done.
    __shared__ int s_last;
    const int64_t g0 = (int64_t)si.base + (int64_t)kvh * si.n;  // first item of the group
    const bool mergeable = si.n <= kGroupItems && g0 + si.n <= (int64_t)a.total_items;
    // Each wave waits until its record stores have completed (s_waitcnt
    // vmcnt(0); expcnt and lgkmcnt left unconstrained) before the barrier.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (wave == 0) {
      int last = 0;
      if (mergeable) {
        if (lane == 0) __hip_atomic_store(a.flags + w, kDoneFlag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        unsigned long long f = kDoneFlag;
        if (lane < si.n) f = __hip_atomic_load(a.flags + g0 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__ballot(f != kDoneFlag) == 0ull) {
          unsigned long long prev = 0ull;
          if (lane == 0)
            prev = __hip_atomic_exchange(a.flags + g0, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          last = __shfl(prev == kDoneFlag ? 1 : 0, 0, 64);
          if (last && lane > 0 && lane < si.n)
            __hip_atomic_store(a.flags + g0 + lane, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      if (lane == 0) s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    single_merge<D, RT>(a, b, kvh, g0, si.n, si.n_main, s_o);
  }
}

// ---------------------------------------------------------------- pass 2
// One workgroup of 256 threads per output row (sequence, kv head, query row).
// It reduces the row's item records to partition maxima and sums, scales and
// sums the unnormalised partial outputs, then combines FOLD's partitions.
// The record pointers, the shape and the first sequence's item counts come as
// leading scalar arguments (placed in registers before the waves start), so
// the first sequence's rows issue their record loads without waiting for the
// argument block.
// Rows with at most NG * FI items (every workload here) take one round of
// loads: each thread issues its statistics record and its partial outputs
// (thread (group g, channel quad c) owns items g, g + NG, ... : FI of them)
// before using any of them. FI (1, 2, 4 or 8) is the smallest that covers the
// launch's largest group, so no thread loads records it has no use for (4
// instead of 8 per thread took 0.3-0.6 us off the window steps). Longer rows
// stream the records in tiles.
constexpr int kMaxFastItems = 8;

// DM != 0: the fused call; the row is written already merged with its draft
// part (draft keys 0..t of the step, draft_part.h). DM == 1: pass 1's extra
// workgroups formed the part, and it is loaded with the records. DM == 16 or
// 32 (more than 8 draft tokens): wave 0 forms it here, its loads issued with
// the records', after the row's reductions.
template <int D, int DM, int FI>
__global__ __launch_bounds__(256) void pass2_kernel(const float4* __restrict__ stat, const float* __restrict__ acc,
                                                    int32_t R, int32_t Hkv, int32_t rows_pad, int32_t total_items,
                                                    int32_t n_first, int32_t nm_first, const Pass2Args a) {
  constexpr bool FUSED = DM != 0;
  constexpr int TM = DM > 1 ? DM : 1;
  constexpr int NQ = D / 4;     // float4 channel quads per row
  constexpr int NG = 256 / NQ;  // item groups
  constexpr int TILE = 1024;    // items whose scales are staged at once (long rows)
  __shared__ float s_scale[TILE];
  __shared__ float4 s_part[2][NG][NQ];
  __shared__ float s_red[4][4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int q4 = tid % NQ, grp = tid / NQ;
  const int32_t idx = blockIdx.x;
  const int32_t row = idx % R;
  const int32_t bh = idx / R;
  const int32_t kvh = bh % Hkv;
  const int32_t b = bh / Hkv;
  // The rows of the first sequence find their items from the leading scalar
  // arguments alone, which the hardware places in registers before the kernel
  // starts: their record loads go out before the argument block arrives.
  const bool first = b == 0 && n_first >= 0;
  SeqInfo si{0, 0, n_first, nm_first};
  if (!first) {
    touch_args<(int)sizeof(Pass2Args)>(a);
    if (a.seqs.nseq > 0) seq_prefix_table(b, a.seqs, a.mode, a.W, a.S, a.C, &si);
    else seq_prefix(b, a.ctx_len, Hkv, a.mode, a.W, a.S, a.C, &si);
  }
  int64_t i0 = (int64_t)si.base + (int64_t)kvh * si.n;
  int64_t im = i0 + si.n_main;
  int64_t i1 = i0 + si.n;
  const int64_t lim = total_items;
  i0 = i0 < lim ? i0 : lim;
  im = im < lim ? im : lim;
  i1 = i1 < lim ? i1 : lim;
  const size_t rp = (size_t)rows_pad;
  const int64_t n = i1 - i0;
  const float* accrow = acc + row * (size_t)D + 4 * q4;
  __shared__ float s_od[DM > 1 ? D : 1];
  __shared__ float s_lsed;
  // Output row, and the fused call's draft inputs: these need the argument
  // block, so they are read once the first record loads are out.
  int32_t t = 0, head = 0;
  int64_t orow = 0;
  float od_row = 0.f, lse_d = 0.f;
  DraftRow<D, TM> dr;
  auto draft_inputs = [&] {
    t = row / a.G;
    head = kvh * a.G + (row - t * a.G);
    orow = (int64_t)(b * a.T + t) * a.Hq + head;
    if constexpr (DM == 1) {
      const int64_t nd = (int64_t)a.B * a.T * a.Hq;
      od_row = a.dpart[orow * D + (tid < D ? tid : 0)];
      lse_d = a.dpart[nd * D + orow];
    }
    if constexpr (DM > 1) {
      if (wv == 0) draft_row_load(dr, a.q, a.kd, a.vd, b, t, head, kvh, a.T, a.Hq, Hkv, lane);
    }
  };

  // block-wide max / sum of per-thread values through the 4 waves
  auto block_max2 = [&](float& x, float& y) {
    x = wave_max(x);
    y = wave_max(y);
    if (lane == 0) { s_red[wv][0] = x; s_red[wv][1] = y; }
    __syncthreads();
    x = fmaxf(fmaxf(s_red[0][0], s_red[1][0]), fmaxf(s_red[2][0], s_red[3][0]));
    y = fmaxf(fmaxf(s_red[0][1], s_red[1][1]), fmaxf(s_red[2][1], s_red[3][1]));
    __syncthreads();
  };
  auto block_sum3 = [&](float& x, float& y, float& z) {
    x = wave_sum(x);
    y = wave_sum(y);
    z = wave_sum(z);
    if (lane == 0) { s_red[wv][0] = x; s_red[wv][1] = y; s_red[wv][2] = z; }
    __syncthreads();
    x = s_red[0][0] + s_red[1][0] + s_red[2][0] + s_red[3][0];
    y = s_red[0][1] + s_red[1][1] + s_red[2][1] + s_red[3][1];
    z = s_red[0][2] + s_red[1][2] + s_red[2][2] + s_red[3][2];
    __syncthreads();
  };

  float M, MF, Ls, ZF, ZFa;
  float4 accp[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
  if (n <= (int64_t)NG * FI) {
    // One round of loads. Each load reads a valid record (its index clamped to
    // the row's last item) and its value always enters the arithmetic: out of
    // range, a statistic gets -inf added and a partial output a zero weight.
    // A value used only under a condition lets the compiler move its load into
    // the branch and wait for it there, which would serialise the round.
    // With at most 64 records every wave loads all the statistics (lane l:
    // record l) and reduces them itself, and each thread takes the scales of
    // its records from the lanes holding them: no barrier before the weighted
    // sums. Otherwise thread tid holds record tid and the workgroup reduces.
    const bool one_wave = n <= 64;
    const int32_t sid = one_wave ? lane : tid;
    const bool has_st = sid < n;
    const int64_t nl = n > 0 ? n - 1 : 0;  // n == 0: nothing is read
    float4 v[FI];
    float4 sv = make_float4(0.f, 0.f, 0.f, 0.f);
    if (n > 0) {
#pragma unroll
      for (int k = 0; k < FI; ++k) {
        const int64_t i = grp + (int64_t)k * NG;
        v[k] = *(const float4*)(accrow + (size_t)(i0 + (i < n ? i : nl)) * rp * D);
      }
      sv = stat[(size_t)(i0 + (has_st ? sid : nl)) * rp + row];
    } else {
#pragma unroll
      for (int k = 0; k < FI; ++k) v[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (first) touch_args<(int)sizeof(Pass2Args)>(a);  // after the record loads are out
    draft_inputs();
    const float alpha = a.alpha;
    const float st_m = sv.x + (has_st ? 0.f : -INFINITY);  // record max (log2), -inf if none
    const float st_y = sv.y * (has_st ? 1.f : 0.f);
    const float st_z = sv.z * (has_st ? 1.f : 0.f);
    const bool is_main = i0 + sid < im;
    M = is_main ? st_m : -INFINITY;
    MF = is_main ? -INFINITY : st_m;
    if (one_wave) {
      M = wave_max(M);
      MF = wave_max(MF);
    } else {
      block_max2(M, MF);
    }
    float sc = 0.f;
    Ls = 0.f; ZF = 0.f; ZFa = 0.f;
    if (st_m != -INFINITY) {
      if (is_main) {
        sc = exp2f(st_m - M);
        Ls = st_y * sc;
      } else {
        sc = exp2f(alpha * (st_m - MF));
        ZF = st_z * exp2f(st_m - MF);
        ZFa = st_y * sc;
      }
    }
    if (one_wave) {
      Ls = wave_sum(Ls);
      ZF = wave_sum(ZF);
      ZFa = wave_sum(ZFa);
    } else {
      if (tid < n) s_scale[tid] = sc;
      block_sum3(Ls, ZF, ZFa);   // its barriers also publish s_scale
    }
#pragma unroll
    for (int k = 0; k < FI; ++k) {
      const int64_t i = grp + (int64_t)k * NG;
      const bool ok = i < n;
      const float s_i = one_wave ? __shfl(sc, ok ? (int)i : 0, 64) : s_scale[ok ? i : 0];
      const float sk = s_i * (ok ? 1.f : 0.f);
      const float wm = i0 + i < im ? sk : 0.f, wf = i0 + i < im ? 0.f : sk;
      accp[0].x += wm * v[k].x;
      accp[0].y += wm * v[k].y;
      accp[0].z += wm * v[k].z;
      accp[0].w += wm * v[k].w;
      accp[1].x += wf * v[k].x;
      accp[1].y += wf * v[k].y;
      accp[1].z += wf * v[k].z;
      accp[1].w += wf * v[k].w;
    }
  } else {
    // long rows: maxima, sums, then the partial outputs tile by tile
    if (first) touch_args<(int)sizeof(Pass2Args)>(a);
    draft_inputs();
    const float alpha = a.alpha;
    M = -INFINITY;
    MF = -INFINITY;
    for (int64_t i = i0 + tid; i < i1; i += 256) {
      const float m = stat[(size_t)i * rp + row].x;
      if (i < im) M = fmaxf(M, m);
      else MF = fmaxf(MF, m);
    }
    block_max2(M, MF);
    Ls = 0.f; ZF = 0.f; ZFa = 0.f;
    for (int64_t i = i0 + tid; i < i1; i += 256) {
      const float4 st = stat[(size_t)i * rp + row];
      if (st.x == -INFINITY) continue;
      if (i < im) {
        Ls += st.y * exp2f(st.x - M);
      } else {
        ZF += st.z * exp2f(st.x - MF);
        ZFa += st.y * exp2f(alpha * (st.x - MF));
      }
    }
    block_sum3(Ls, ZF, ZFa);
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      const int64_t lo = pt == 0 ? i0 : im, hi = pt == 0 ? im : i1;
      const float ref = pt == 0 ? M : MF;
      const float sh = pt == 0 ? 1.f : alpha;
      for (int64_t t0 = lo; t0 < hi; t0 += TILE) {
        const int64_t t1 = hi < t0 + TILE ? hi : t0 + TILE;
        __syncthreads();
        for (int64_t i = t0 + tid; i < t1; i += 256) {
          const float m = stat[(size_t)i * rp + row].x;
          s_scale[i - t0] = m == -INFINITY ? 0.f : exp2f(sh * (m - ref));
        }
        __syncthreads();
#pragma unroll 8
        for (int64_t i = t0 + grp; i < t1; i += NG) {
          const float4 v = *(const float4*)(accrow + (size_t)i * rp * D);
          const float sc = s_scale[i - t0];
          acc.x += sc * v.x;
          acc.y += sc * v.y;
          acc.z += sc * v.z;
          acc.w += sc * v.w;
        }
      }
      accp[pt] = acc;
    }
  }
  s_part[0][grp][q4] = accp[0];
  s_part[1][grp][q4] = accp[1];
  __syncthreads();

  const RowCombine cb = combine_row(M, MF, Ls, ZF, ZFa, a.alpha, a.beta, a.fold_variant);
  float lse_out = cb.lse;
  DraftMerge mg{1.f, 0.f, cb.lse};
  if constexpr (DM > 1) {
    if (wv == 0) {
      const int32_t L = a.seqs.nseq > 0 ? a.seqs.len[b] : a.ctx_len[b];
      const float c = draft_logit_scale(a.scale, a.kappa, visible_count(L, a.mode, a.W, a.S), a.n0);
      float ld, od[D / 64];
      draft_row_part(dr, t, c, ld, od);
#pragma unroll
      for (int e = 0; e < D / 64; ++e) s_od[lane * (D / 64) + e] = od[e];
      if (lane == 0) s_lsed = ld;
    }
    __syncthreads();
    if (tid < D) od_row = s_od[tid];
    lse_d = s_lsed;
  }
  if constexpr (FUSED) {
    mg = draft_merge(cb.lse, lse_d);
    lse_out = mg.lse;
  }
  // Final combine: thread c < D owns output channel c.
  if (tid < D) {
    const float* pm = (const float*)&s_part[0][0][0];
    const float* pf = (const float*)&s_part[1][0][0];
    float sm = 0.f, sf = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < NG; ++g2) {
      sm += pm[g2 * D + tid];
      sf += pf[g2 * D + tid];
    }
    // explicit fmaf: the separate merge call reads this value back and must
    // see the same rounding as the fused merge below
    float res = fmaf(sm, cb.fl, sf * cb.ff);
    if constexpr (FUSED) res = draft_merge_out(mg, res, od_row);
    if (a.out_bf16) ((__bf16*)a.out)[orow * D + tid] = (__bf16)res;
    else ((float*)a.out)[orow * D + tid] = res;
  }
  if (tid == 0) a.lse[orow] = lse_out;
}

// ---------------------------------------------------------------- launch
// The merge kernel's leading scalar arguments (see pass2_kernel), gathered on
// the host.
struct Pass2Lead {
  const float4* stat;
  const float* acc;
  int32_t R, Hkv, rows_pad, total_items, n_first, nm_first;
};

template <int D, int DM, int FI>
static void launch_pass2_k(uint32_t grid, hipStream_t s, const Pass2Lead& h, const Pass2Args& a) {
  pass2_kernel<D, DM, FI><<<grid, 256, 0, s>>>(h.stat, h.acc, h.R, h.Hkv, h.rows_pad, h.total_items, h.n_first,
                                               h.nm_first, a);
}

template <int D, int FI>
static void launch_pass2_fi(int dm, uint32_t grid, hipStream_t s, const Pass2Lead& h, const Pass2Args& a) {
  if (dm == 0) launch_pass2_k<D, 0, FI>(grid, s, h, a);
  else if (dm == 1) launch_pass2_k<D, 1, FI>(grid, s, h, a);
  else if (dm == 16) launch_pass2_k<D, 16, FI>(grid, s, h, a);
  else launch_pass2_k<D, 32, FI>(grid, s, h, a);
}

template <int D>
static void launch_pass2(int dm, int fi, uint32_t grid, hipStream_t s, const Pass2Lead& h, const Pass2Args& a) {
  if (fi == 1) launch_pass2_fi<D, 1>(dm, grid, s, h, a);
  else if (fi == 2) launch_pass2_fi<D, 2>(dm, grid, s, h, a);
  else if (fi == 4) launch_pass2_fi<D, 4>(dm, grid, s, h, a);
  else launch_pass2_fi<D, kMaxFastItems>(dm, grid, s, h, a);
}

template <int D, bool SINGLE>
static void launch_pass1(const Pass1Args& a, int row_tiles, bool fold, uint32_t grid, size_t lds,
                         hipStream_t s) {
  // the leading scalar arguments (see pass1_kernel)
  int32_t first_items = 0;
  if (a.seqs.nseq > 0) first_items = seq_items(seq_ranges(a.seqs.len[0], a.mode, a.W, a.S), a.C, nullptr) * a.Hkv;
  const int32_t L_first = a.seqs.nseq > 0 ? a.seqs.len[0] : 0;
  const int32_t mode_g_t = a.mode | (a.G << 8) | (a.T << 16);
  auto go = [&](auto kernel) {
    kernel<<<grid, 64 * kWaves, lds, s>>>(a.q, a.table, first_items, L_first, mode_g_t, a.W, a.S, a.C, a.Hq,
                                          a.max_blocks, a.num_blocks, a);
  };
  if (row_tiles == 1) {
    if (fold) go(pass1_kernel<D, 1, true, SINGLE>);
    else go(pass1_kernel<D, 1, false, SINGLE>);
  } else {
    if (fold) go(pass1_kernel<D, 2, true, SINGLE>);
    else go(pass1_kernel<D, 2, false, SINGLE>);
  }
}

}  // namespace da

namespace da {

// The decode call, optionally fused with the draft part (kd, vd non-null).
static int decode_impl(const draft_attn_params* p, const void* q, const void* k_cache, const void* v_cache,
                       const void* k_side, const int32_t* block_table, const int32_t* ctx_len_dev,
                       const int32_t* ctx_len_host, const void* kd, const void* vd, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream) {
  Prepared pr;
  const int st = prepare(p, ctx_len_host, &pr);
  if (st != DRAFT_ATTN_OK) return st;
  const bool fused = kd != nullptr;
  if (fused) {
    // The draft part is applied by the merge kernel, so the call always runs
    // on two kernels (the layout of the workspace does not depend on it).
    pr.single = false;
    if (!vd) return DRAFT_ATTN_EINVAL;
    if (((uintptr_t)kd & 15) != 0 || ((uintptr_t)vd & 15) != 0) return DRAFT_ATTN_EINVAL;
  }
  if ((p->prof_events[0] == nullptr) != (p->prof_events[1] == nullptr)) return DRAFT_ATTN_EINVAL;
  if (p->num_seqs == 0) return DRAFT_ATTN_OK;
  if (!q || !k_cache || !v_cache || !block_table || !ctx_len_dev || !out || !lse || !workspace)
    return DRAFT_ATTN_EINVAL;
  if ((p->mode == kFold) != (k_side != nullptr)) return DRAFT_ATTN_EINVAL;
  auto mis = [](const void* ptr, uintptr_t al) { return ((uintptr_t)ptr & (al - 1)) != 0; };
  if (mis(q, 16) || mis(k_cache, 16) || mis(v_cache, 16) || (k_side && mis(k_side, 16)) ||
      mis(out, 8) || mis(lse, 4) || mis(block_table, 4) || mis(ctx_len_dev, 4) || mis(workspace, 256) ||
      mis(p->status_flags, 4))
    return DRAFT_ATTN_EINVAL;
  if (workspace_bytes < pr.workspace_bytes) return DRAFT_ATTN_ENOSPC;
  log_plan(p, pr);

  const int D = p->head_dim;
  char* ws = (char*)workspace;
  Pass1Args a1;
  a1.q = (const __bf16*)q;
  a1.k = (const __bf16*)k_cache;
  a1.v = (const __bf16*)v_cache;
  a1.ks = (const __bf16*)k_side;
  a1.table = block_table;
  a1.ctx_len = ctx_len_dev;
  a1.stat = (float4*)(ws + pr.stat_offset);
  a1.acc = (float*)(ws + pr.acc_offset);
  a1.visit = p->debug_visit;
  a1.visit_stride = p->debug_visit_stride;
  a1.flags = (unsigned long long*)(ws + pr.flag_offset);
  // pass 1 forms the draft parts only for T <= 8 (see draft_wgs below)
  a1.kd = kd != nullptr && p->num_draft_tokens <= 8 ? (const __bf16*)kd : nullptr;
  a1.vd = a1.kd != nullptr ? (const __bf16*)vd : nullptr;
  a1.dpart = (float*)(ws + pr.draft_offset);
  a1.out = out;
  a1.lse = lse;
  a1.status = p->status_flags;
  a1.out_bf16 = p->out_dtype == DRAFT_ATTN_OUT_BF16;
  a1.fold_variant = p->fold_variant;
  a1.beta = p->beta;
  a1.B = p->num_seqs;
  a1.T = p->num_draft_tokens;
  a1.Hq = p->num_q_heads;
  a1.Hkv = p->num_kv_heads;
  a1.G = pr.G;
  a1.R = pr.rows;
  a1.rows_pad = pr.rows_pad;
  a1.max_blocks = p->max_blocks_per_seq;
  a1.num_blocks = p->num_blocks;
  a1.mode = p->mode;
  a1.W = p->window;
  a1.S = p->n_sink;
  a1.n0 = p->n0;
  a1.C = pr.chunk;
  a1.rope = p->rope;
  a1.total_items = (int32_t)pr.total_items;
  a1.alpha = p->alpha;
  a1.kappa = p->kappa;
  a1.scale = p->softmax_scale;
  // RoPE frequencies, read only by FOLD's far-query rotation.
  const bool far_rope = p->mode == kFold && p->rope == DRAFT_ATTN_ROPE_NEOX;
  if (far_rope) {
    static_assert(kMaxHalfDim <= 64, "frequency table size");
    memcpy(a1.omega, rope_table(p->rope_theta, D).omega, sizeof a1.omega);
  } else {
    memset(a1.omega, 0, sizeof a1.omega);
  }
  memset(&a1.seqs, 0, sizeof(a1.seqs));
  if (p->num_seqs <= kArgSeqs) {
    a1.seqs.nseq = p->num_seqs;
    int32_t acc = 0;
    for (int32_t b = 0; b < p->num_seqs; ++b) {
      a1.seqs.len[b] = ctx_len_host[b];
      a1.seqs.base[b] = acc;
      a1.seqs.c2[b] = logit_scale_log2(p->softmax_scale, p->kappa,
                                       visible_count(ctx_len_host[b], p->mode, p->window, p->n_sink), p->n0);
      acc += seq_items(seq_ranges(ctx_len_host[b], p->mode, p->window, p->n_sink), pr.chunk, nullptr) *
             p->num_kv_heads;
    }
    a1.seqs.base[p->num_seqs] = acc;
  }

  Pass2Args a2;
  a2.stat = a1.stat;
  a2.acc = a1.acc;
  a2.ctx_len = ctx_len_dev;
  a2.out = out;
  a2.lse = lse;
  a2.B = a1.B;
  a2.T = a1.T;
  a2.Hq = a1.Hq;
  a2.Hkv = a1.Hkv;
  a2.G = a1.G;
  a2.R = a1.R;
  a2.rows_pad = a1.rows_pad;
  a2.mode = a1.mode;
  a2.W = a1.W;
  a2.S = a1.S;
  a2.C = a1.C;
  a2.total_items = a1.total_items;
  a2.alpha = p->alpha;
  a2.beta = p->beta;
  a2.fold_variant = p->fold_variant;
  a2.out_bf16 = a1.out_bf16;
  a2.seqs = a1.seqs;
  a2.dpart = a1.dpart;
  a2.q = (const __bf16*)q;
  a2.kd = (const __bf16*)kd;
  a2.vd = (const __bf16*)vd;
  a2.n0 = p->n0;
  a2.kappa = p->kappa;
  a2.scale = p->softmax_scale;

  // Every (sequence, kv head) has at least one item, so the single kernel
  // writes every output row.
  const bool single = pr.single && pr.total_items > 0;
  // the fused call adds one workgroup per four query rows for the draft parts
  // (T <= 8: for more draft tokens the merge kernel forms the parts itself)
  const bool draft_in_pass1 = fused && p->num_draft_tokens <= 8;
  const int64_t draft_wgs =
      draft_in_pass1 ? ((int64_t)p->num_seqs * p->num_draft_tokens * p->num_q_heads + kWaves - 1) / kWaves : 0;
  if (pr.total_items + draft_wgs > 0x7fffffff) return DRAFT_ATTN_EINVAL;  // before anything is enqueued
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();  // clear a stale error so the check below reports ours
  if (p->prof_events[0]) (void)hipEventRecord((hipEvent_t)p->prof_events[0], s);
  if (pr.total_items + draft_wgs > 0) {
    const size_t lds = pass1_lds_bytes(pr.chunk, pr.rows_pad, D);
    const bool fold = p->mode == kFold;
    const uint32_t grid = (uint32_t)(pr.total_items + draft_wgs);
    if (single) {
      if (D == 64) launch_pass1<64, true>(a1, pr.row_tiles, fold, grid, lds, s);
      else launch_pass1<128, true>(a1, pr.row_tiles, fold, grid, lds, s);
    } else {
      if (D == 64) launch_pass1<64, false>(a1, pr.row_tiles, fold, grid, lds, s);
      else launch_pass1<128, false>(a1, pr.row_tiles, fold, grid, lds, s);
    }
  }
  if (p->prof_events[1]) (void)hipEventRecord((hipEvent_t)p->prof_events[1], s);
  if (!single) {
    const uint32_t rows_total = (uint32_t)((int64_t)p->num_seqs * p->num_kv_heads * pr.rows);
    const int dm = !fused ? 0 : (draft_in_pass1 ? 1 : (a2.T <= 16 ? 16 : 32));
    // leading scalar arguments: record pointers, shape, and the first
    // sequence's item counts (from the launch's sequence table; -1 without one)
    Pass2Lead h{a2.stat, a2.acc, a2.R, a2.Hkv, a2.rows_pad, a2.total_items, -1, 0};
    if (a2.seqs.nseq > 0) h.n_first = seq_items(seq_ranges(a2.seqs.len[0], a2.mode, a2.W, a2.S), a2.C, &h.nm_first);
    // records each thread of the merge kernel loads in its one round
    const int32_t ng = 256 / (D / 4);
    const int32_t fi = pr.max_group_items <= ng ? 1 : pr.max_group_items <= 2 * ng ? 2
                     : pr.max_group_items <= 4 * ng ? 4 : kMaxFastItems;
    if (D == 64) launch_pass2<64>(dm, fi, rows_total, s, h, a2);
    else launch_pass2<128>(dm, fi, rows_total, s, h, a2);
  }
  if (hipGetLastError() != hipSuccess) return DRAFT_ATTN_EHIP;
  return DRAFT_ATTN_OK;
}

}  // namespace da

namespace da {

// Scratch of the allocation-free entry point: the workspace of one call (done
// flags, partial records, draft parts), held by the library in each GPU's
// memory for the life of the process. In host code `scratch` names a host-side
// stand-in, not device memory: only the address that hipGetSymbolAddress
// returns for the current device is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[DRAFT_ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
static ScratchSlot g_scratch[kMaxDevices];

// Device address of the current device's copy of `scratch`, looked up once per
// device (with that device current) and kept.
static int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DRAFT_ATTN_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return DRAFT_ATTN_ENOTSUP;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&slot] { slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch)); });
  if (slot.err != hipSuccess || slot.ptr == nullptr) return DRAFT_ATTN_EHIP;
  *out = slot.ptr;
  return DRAFT_ATTN_OK;
}

}  // namespace da

extern "C" int draft_attn_decode_noalloc(const draft_attn_params* p, const void* q, const void* k_cache,
                                         const void* v_cache, const void* k_side, const int32_t* block_table,
                                         const int32_t* ctx_len_dev, const int32_t* ctx_len_host, void* out,
                                         float* lse, void* stream) {
  da::Prepared pr;
  const int st = da::prepare(p, ctx_len_host, &pr);
  if (st != DRAFT_ATTN_OK) return st;
  if (pr.workspace_bytes > DRAFT_ATTN_NOALLOC_SCRATCH_BYTES) return DRAFT_ATTN_ENOSPC;
  if (p->num_seqs == 0) return DRAFT_ATTN_OK;
  void* ws = nullptr;
  const int sa = da::scratch_address(&ws);
  if (sa != DRAFT_ATTN_OK) return sa;
  return da::decode_impl(p, q, k_cache, v_cache, k_side, block_table, ctx_len_dev, ctx_len_host, nullptr, nullptr,
                         out, lse, ws, DRAFT_ATTN_NOALLOC_SCRATCH_BYTES, stream);
}

namespace da {
// Launch-floor kernels of draft_attn_launch_floor: they do nothing, and take
// argument blocks of the same layout and size as pass 1 and pass 2, since the
// runtime's cost of enqueueing a launch grows with its argument block.
__global__ __launch_bounds__(256) void empty_pass1_kernel(const __bf16*, const int32_t*, int32_t, int32_t, int32_t,
                                                          int32_t, int32_t, int32_t, int32_t, int32_t, int32_t,
                                                          const Pass1Args) {}
__global__ __launch_bounds__(256) void empty_pass2_kernel(const float4*, const float*, int32_t, int32_t, int32_t,
                                                          int32_t, int32_t, int32_t, const Pass2Args) {}
}  // namespace da

extern "C" int draft_attn_launch_floor(const draft_attn_params* p, const int32_t* ctx_len_host, int32_t kernels,
                                       void* stream) {
  da::Prepared pr;
  const int st = da::prepare(p, ctx_len_host, &pr);
  if (st != DRAFT_ATTN_OK) return st;
  if (kernels != 1 && kernels != 2) return DRAFT_ATTN_EINVAL;
  if (p->num_seqs == 0 || pr.total_items == 0) return DRAFT_ATTN_OK;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  const size_t lds = da::pass1_lds_bytes(pr.chunk, pr.rows_pad, p->head_dim);
  da::Pass1Args a1;
  da::Pass2Args a2;
  memset(&a1, 0, sizeof a1);
  memset(&a2, 0, sizeof a2);
  da::empty_pass1_kernel<<<(uint32_t)pr.total_items, 256, lds, s>>>(nullptr, nullptr, 0, 0, 0, 0, 0, 0, 0, 0, 0, a1);
  if (kernels == 2) {
    const uint32_t rows_total = (uint32_t)((int64_t)p->num_seqs * p->num_kv_heads * pr.rows);
    da::empty_pass2_kernel<<<rows_total, 256, 0, s>>>(nullptr, nullptr, 0, 0, 0, 0, 0, 0, a2);
  }
  if (hipGetLastError() != hipSuccess) return DRAFT_ATTN_EHIP;
  return DRAFT_ATTN_OK;
}

extern "C" int draft_attn_decode(const draft_attn_params* p, const void* q, const void* k_cache,
                                 const void* v_cache, const void* k_side, const int32_t* block_table,
                                 const int32_t* ctx_len_dev, const int32_t* ctx_len_host, void* out,
                                 float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return da::decode_impl(p, q, k_cache, v_cache, k_side, block_table, ctx_len_dev, ctx_len_host, nullptr, nullptr,
                         out, lse, workspace, workspace_bytes, stream);
}

extern "C" int draft_attn_decode_draft(const draft_attn_params* p, const void* q, const void* k_cache,
                                       const void* v_cache, const void* k_side, const int32_t* block_table,
                                       const int32_t* ctx_len_dev, const int32_t* ctx_len_host,
                                       const void* k_draft, const void* v_draft, void* out, float* lse,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!k_draft || !v_draft) return DRAFT_ATTN_EINVAL;
  return da::decode_impl(p, q, k_cache, v_cache, k_side, block_table, ctx_len_dev, ctx_len_host, k_draft, v_draft,
                         out, lse, workspace, workspace_bytes, stream);
}

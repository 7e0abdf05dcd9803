// KV append with FOLD side-cache bookkeeping, for CDNA4 (gfx950).
//
// "FOLD: Position-Free Far Memory with Local Order for Long-Context Speculative
// Decoding" (review) keeps an unrotated side cache beside the usual rotated one
// and names its bookkeeping as part of the cost. For each newly accepted token
// at position p this kernel writes the key turned to its own position, R(p) k,
// into k_cache, the unrotated key into k_side, and the value into v_cache, at the
// slot the block table gives for p. The rotation is done in fp64 (the angle of
// a block's first slot formed and reduced by the fp64 sincos, then advanced by
// fp64 rotation steps to the block's other slots) and rounded once to bf16, to
// nearest with ties to even: the stored key is the bf16 value nearest to an
// fp64 rotation that is within a few fp64 ulps of the exact one.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include "host.h"

namespace da {

constexpr int kAppendArgSeqs = 32;

struct AppendArgs {
  const __bf16* k_new;  // [B][n_new][Hkv][D]
  const __bf16* v_new;  // [B][n_new][Hkv][D]
  const int32_t* table;
  const int32_t* pos;   // [B] position of each sequence's first new token
  __bf16* k;            // [blocks][Hkv][D/8][16][8]
  __bf16* v;            // [blocks][Hkv][D][16]
  __bf16* ks;           // like k, or null
  uint32_t* status;     // optional device status word, or null
  int32_t B, n_new, Hkv, max_blocks, num_blocks, rope;
  int32_t span;         // logical blocks one sequence's append can touch
  int32_t npos;         // B when B <= kAppendArgSeqs (positions below), else 0 (read pos)
  int32_t pos_h[kAppendArgSeqs];  // the host copy of pos, for up to kAppendArgSeqs sequences
  double omega[64];     // rope_theta^(-2i/D)
  double cos_w[64];     // cos(omega_i), sin(omega_i): one position step
  double sin_w[64];
  double cos_g[64];     // cos(G omega_i), sin(G omega_i): one slot group of
  double sin_g[64];     // G = 16 * (D/2) / 256 positions
};

// fp64 -> bf16 bits, round to nearest, ties to even, for finite values in the
// normal range: round the significand to 8 bits in the fp64 encoding (the
// result is exactly representable in fp32 and bf16), then take the fp32 bits.
__device__ __forceinline__ unsigned short bf16_bits_rne(double x) {
  unsigned long long u = __double_as_longlong(x);
  const unsigned long long lsb = (u >> 45) & 1ull;
  u += 0x00000FFFFFFFFFFFull + lsb;
  u &= ~0x00001FFFFFFFFFFFull;
  const float f = (float)__longlong_as_double(u);
  return (unsigned short)(__float_as_uint(f) >> 16);
}

// One workgroup per (sequence, logical block, kv head) that the append touches;
// it owns the new tokens of that block, slots s0 .. s1-1. They are staged in LDS
// with row-contiguous loads, rotated there, and written back as whole 16-byte
// runs of each cache layout: 16 slots of one key octet for k_cache and k_side,
// 8 slots of one channel for v_cache (a partial run at the edges of the append
// is written per slot). Large appends (NT) load and store nontemporally, since
// each byte is moved once; small ones (a decode step's accepted tokens) use
// ordinary accesses, which complete sooner and leave the new slots in cache for
// the next decode. Rotation: the first D/2 threads form the angle of the block's slot 0
// for their pair with the fp64 sincos (one per pair, not per thread: the fp64
// unit, not memory, was the limit otherwise), in wave 0, which stages nothing,
// so the sincos overlaps the other waves' loads. Wave 0 also turns it to the
// first slot of every slot group by steps of (cos G w_i, sin G w_i) and leaves
// those angles and the one-position step (cos w_i, sin w_i) in LDS, so that
// after the barrier the rotation reads nothing from memory; thread (pair i,
// slot group q) then advances one position at a time. Each step adds a few
// fp64 ulps.
template <bool NT, typename T>
__device__ __forceinline__ T load_nt(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT, typename T>
__device__ __forceinline__ void store_nt(T v, T* p) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// The arguments the prologue reads (up to the end of pos_h) span a few 64-byte
// lines of the scalar cache; each line's first read misses. Loading one word
// of every line at entry, with independent loads and one wait, pays that miss
// once instead of once per line in a chain of dependent reads.
__device__ __forceinline__ void touch_append_args(const AppendArgs& a) {
  constexpr int N = (int)((offsetof(AppendArgs, omega) + 63) / 64);
  static_assert(N <= 4, "prologue arguments span at most four lines");
  const uint32_t* p = reinterpret_cast<const uint32_t*>(&a);
  uint32_t v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = i < N ? p[16 * i] : 0u;
  asm volatile("" ::"s"(v[0]), "s"(v[1]), "s"(v[2]), "s"(v[3]));
}

template <int D, bool NT>
__global__ __launch_bounds__(256) void append_kernel(const AppendArgs a) {
  touch_append_args(a);
  constexpr int NO = D / 8;               // channel octets
  constexpr int HALF = D / 2;             // rotation pairs
  constexpr int SPT = 16 * HALF / 256;    // slots per thread in the rotation
  constexpr int LD = D + 8;               // padded LDS row (elements)
  __shared__ __align__(16) __bf16 s_k[16][LD];
  __shared__ __align__(16) __bf16 s_v[16][LD];
  __shared__ __align__(16) __bf16 s_r[16][LD];
  constexpr int NG = 256 / HALF;          // slot groups of the rotation
  __shared__ double s_c0[NG][HALF], s_s0[NG][HALF];  // angle of each group's first slot
  __shared__ double s_cw[HALF], s_sw[HALF];          // one position step
  const int tid = threadIdx.x;
  int64_t w = blockIdx.x;
  const int32_t h = (int32_t)(w % a.Hkv);
  w /= a.Hkv;
  const int32_t jj = (int32_t)(w % a.span);
  const int32_t b = (int32_t)(w / a.span);
  // Up to 32 sequences take their position from the launch arguments, so the
  // block-table and new-token loads do not wait for a read of pos first.
  const int32_t p0 = a.npos > 0 ? a.pos_h[b] : a.pos[b];
  if (p0 < 0) return;
  const int32_t j = (p0 >> 4) + jj;
  const int64_t lo64 = (int64_t)j * 16 > p0 ? (int64_t)j * 16 : p0;
  const int64_t hi64 = (int64_t)p0 + a.n_new < (int64_t)j * 16 + 16 ? (int64_t)p0 + a.n_new : (int64_t)j * 16 + 16;
  if (lo64 >= hi64 || j >= a.max_blocks) return;
  const int32_t id = a.table[(int64_t)b * a.max_blocks + j];
  if (id < 0 || id >= a.num_blocks) {  // no block allocated: nothing is written, and it is reported
    if (tid == 0 && a.status != nullptr) atomicOr(a.status, (uint32_t)DRAFT_ATTN_STATUS_APPEND_BAD_BLOCK);
    return;
  }
  const int s0 = (int)(lo64 - (int64_t)j * 16), s1 = (int)(hi64 - (int64_t)j * 16);
  const int32_t i0 = (int32_t)(lo64 - p0);  // index of slot s0's token among the new ones

  // Wave 0 forms the block's sincos while waves 1-3 stage the new tokens' keys
  // and values, 16 slots x D/8 octets of 16 bytes (wave 1 takes two octets per
  // thread when there are 256). Keeping the sincos off the staging waves keeps
  // its argument load out of their load queue: a wave's wait for one load also
  // waits for every load issued before it. A lane whose octet is outside the
  // new slots loads slot s0's octet and drops it, so that every lane of a wave
  // issues the same loads.
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  static_assert(16 * NO <= 192 + 64, "at most two staged octets per thread");
  const bool rot = a.rope == DRAFT_ATTN_ROPE_NEOX;
  if (tid < 64) {
    if (rot && tid < HALF) {
      const double om = a.omega[tid], cg = a.cos_g[tid], sg = a.sin_g[tid];
      s_cw[tid] = a.cos_w[tid];
      s_sw[tid] = a.sin_w[tid];
      double sn, cs;
      sincos((double)((int64_t)j * 16) * om, &sn, &cs);
#pragma unroll
      for (int q = 0; q < NG; ++q) {
        s_c0[q][tid] = cs;
        s_s0[q][tid] = sn;
        const double c2 = cs * cg - sn * sg;
        sn = sn * cg + cs * sg;
        cs = c2;
      }
    }
  } else {
    const int e1 = tid - 64, e2 = e1 + 192;
    const bool has1 = e1 < 16 * NO, has2 = e2 < 16 * NO;  // uniform per wave
    const int s1a = e1 / NO, c1 = e1 - s1a * NO, s2a = e2 / NO, c2 = e2 - s2a * NO;
    const bool ok1 = s1a >= s0 && s1a < s1, ok2 = s2a >= s0 && s2a < s1;
    auto src = [&](bool ok, int ss, int sc) {
      return (((size_t)b * a.n_new + (i0 + (ok ? ss : s0) - s0)) * a.Hkv + h) * D + 8 * (ok ? sc : 0);
    };
    if (has1) {
      const size_t o1 = src(ok1, s1a, c1);
      const u32x4 k1 = load_nt<NT>((const u32x4*)(a.k_new + o1));
      const u32x4 v1 = load_nt<NT>((const u32x4*)(a.v_new + o1));
      u32x4 k2 = {0u, 0u, 0u, 0u}, v2 = {0u, 0u, 0u, 0u};
      if (has2) {
        const size_t o2 = src(ok2, s2a, c2);
        k2 = load_nt<NT>((const u32x4*)(a.k_new + o2));
        v2 = load_nt<NT>((const u32x4*)(a.v_new + o2));
      }
      if (ok1) {
        *(u32x4*)&s_k[s1a][8 * c1] = k1;
        *(u32x4*)&s_v[s1a][8 * c1] = v1;
      }
      if (has2 && ok2) {
        *(u32x4*)&s_k[s2a][8 * c2] = k2;
        *(u32x4*)&s_v[s2a][8 * c2] = v2;
      }
    }
  }
  __syncthreads();

  // Rotate: thread (i, q) owns pair (i, i + D/2) of slots q*SPT .. q*SPT + SPT - 1.
  if (rot) {
    const int i = tid % HALF, q = tid / HALF;
    const int sa = q * SPT, sb = sa + SPT;
    if (sa < s1 && sb > s0) {
      double cs = s_c0[q][i], sn = s_s0[q][i];
      const double cw = s_cw[i], sw = s_sw[i];
      for (int s = sa; s < sb; ++s) {
        if (s >= s0 && s < s1) {
          const double x1 = (double)(float)s_k[s][i], x2 = (double)(float)s_k[s][i + HALF];
          const unsigned short r1 = bf16_bits_rne(x1 * cs - x2 * sn);
          const unsigned short r2 = bf16_bits_rne(x1 * sn + x2 * cs);
          s_r[s][i] = __builtin_bit_cast(__bf16, r1);
          s_r[s][i + HALF] = __builtin_bit_cast(__bf16, r2);
        }
        const double c2 = cs * cw - sn * sw;
        sn = sn * cw + cs * sw;
        cs = c2;
      }
    }
  }
  __syncthreads();
  const __bf16(*kr)[LD] = a.rope == DRAFT_ATTN_ROPE_NEOX ? s_r : s_k;

  // Keys: thread (octet c, slot s) writes 16 bytes at [c][s]; 16 consecutive
  // threads cover one octet's 256 contiguous bytes.
  const size_t blk = ((size_t)id * a.Hkv + h) * (size_t)(D * 16);
  for (int e = tid; e < 16 * NO; e += 256) {
    const int c = e / 16, s = e - c * 16;
    if (s < s0 || s >= s1) continue;
    const size_t dst = blk + ((size_t)c * 16 + s) * 8;
    store_nt<NT>(*(const u32x4*)&kr[s][8 * c], (u32x4*)(a.k + dst));
    if (a.ks != nullptr) store_nt<NT>(*(const u32x4*)&s_k[s][8 * c], (u32x4*)(a.ks + dst));
  }
  // Values: thread (channel ch, half g) writes slots 8g .. 8g+7 of channel ch.
  for (int e = tid; e < 2 * D; e += 256) {
    const int ch = e >> 1, g = e & 1;
    const int sa = 8 * g, sb = sa + 8;
    __bf16* dst = a.v + blk + (size_t)ch * 16 + sa;
    if (sa >= s0 && sb <= s1) {
      typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
      bf16x8_t o;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = s_v[sa + k][ch];
      store_nt<NT>(o, (bf16x8_t*)dst);
    } else {
      for (int k = 0; k < 8; ++k)
        if (sa + k >= s0 && sa + k < s1) dst[k] = s_v[sa + k][ch];
    }
  }
}

}  // namespace da

extern "C" int draft_attn_append(const draft_attn_append_params* p, const void* k_new, const void* v_new,
                                 const int32_t* block_table, const int32_t* pos_dev, const int32_t* pos_host,
                                 void* k_cache, void* v_cache, void* k_side, void* stream) {
  using namespace da;
  const int st = prepare_append(p, pos_host);
  if (st != DRAFT_ATTN_OK) return st;
  if (p->num_seqs == 0) return DRAFT_ATTN_OK;
  if (!k_new || !v_new || !block_table || !pos_dev || !k_cache || !v_cache) return DRAFT_ATTN_EINVAL;
  auto mis = [](const void* ptr, uintptr_t al) { return ((uintptr_t)ptr & (al - 1)) != 0; };
  if (mis(k_new, 16) || mis(v_new, 16) || mis(k_cache, 16) || mis(v_cache, 16) || (k_side && mis(k_side, 16)) ||
      mis(block_table, 4) || mis(pos_dev, 4) || mis(p->status_flags, 4))
    return DRAFT_ATTN_EINVAL;
  AppendArgs a;
  a.k_new = (const __bf16*)k_new;
  a.v_new = (const __bf16*)v_new;
  a.table = block_table;
  a.pos = pos_dev;
  a.k = (__bf16*)k_cache;
  a.v = (__bf16*)v_cache;
  a.ks = (__bf16*)k_side;
  a.status = p->status_flags;
  a.B = p->num_seqs;
  a.n_new = p->num_new;
  a.Hkv = p->num_kv_heads;
  a.max_blocks = p->max_blocks_per_seq;
  a.num_blocks = p->num_blocks;
  a.rope = p->rope;
  const int D = p->head_dim;
  if (p->rope == DRAFT_ATTN_ROPE_NEOX) {
    static_assert(16 * (64 / 2) / 256 == 64 / 32 && 16 * (128 / 2) / 256 == 128 / 32, "slot group = d/32 positions");
    const RopeTable& t = rope_table(p->rope_theta, D);
    memcpy(a.omega, t.omega, sizeof a.omega);
    memcpy(a.cos_w, t.cos_w, sizeof a.cos_w);
    memcpy(a.sin_w, t.sin_w, sizeof a.sin_w);
    memcpy(a.cos_g, t.cos_g, sizeof a.cos_g);
    memcpy(a.sin_g, t.sin_g, sizeof a.sin_g);
  } else {
    for (double* t : {a.omega, a.cos_w, a.sin_w, a.cos_g, a.sin_g}) memset(t, 0, 64 * sizeof(double));  // unread
  }
  a.span = (p->num_new + 15) / 16 + 1;
  a.npos = p->num_seqs <= kAppendArgSeqs ? p->num_seqs : 0;
  for (int32_t b = 0; b < a.npos; ++b) a.pos_h[b] = pos_host[b];
  const uint32_t grid = (uint32_t)((int64_t)a.B * a.span * a.Hkv);
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  // Streaming (nontemporal) accesses once the append moves more than the
  // infinity cache could usefully keep: 64 MiB of new keys, side keys and values.
  const bool nt = (double)a.B * a.n_new * a.Hkv * 10.0 * D > 64.0 * 1024 * 1024;
  if (D == 64) {
    if (nt) append_kernel<64, true><<<grid, 256, 0, s>>>(a);
    else append_kernel<64, false><<<grid, 256, 0, s>>>(a);
  } else {
    if (nt) append_kernel<128, true><<<grid, 256, 0, s>>>(a);
    else append_kernel<128, false><<<grid, 256, 0, s>>>(a);
  }
  if (hipGetLastError() != hipSuccess) return DRAFT_ATTN_EHIP;
  return DRAFT_ATTN_OK;
}

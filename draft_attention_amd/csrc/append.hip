// KV append with FOLD side-cache bookkeeping, for CDNA4 (gfx950).
//
// "FOLD: Position-Free Far Memory with Local Order for Long-Context Speculative
// Decoding" (review) keeps an unrotated side cache beside the usual rotated one
// and names its bookkeeping as part of the cost. For each newly accepted token
// at position p this kernel writes the key turned to its own position, R(p) k,
// into k_cache, the unrotated key into k_side, and the value into v_cache, at the
// slot the block table gives for p. The rotation is done in fp64 (angles formed
// and reduced by the fp64 sincos) and rounded once to bf16, to nearest with ties
// to even, so the stored key is the correctly rounded value of the exact rotation.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "host.h"

namespace da {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

struct AppendArgs {
  const __bf16* k_new;  // [B][n_new][Hkv][D]
  const __bf16* v_new;  // [B][n_new][Hkv][D]
  const int32_t* table;
  const int32_t* pos;   // [B] position of each sequence's first new token
  __bf16* k;            // [blocks][Hkv][D/8][16][8]
  __bf16* v;            // [blocks][Hkv][D][16]
  __bf16* ks;           // like k, or null
  int32_t B, n_new, Hkv, max_blocks, num_blocks, rope;
  double omega[64];     // rope_theta^(-2i/D)
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

// One thread per (sequence, new token, kv head, channel octet c < D/16): it owns
// channels 8c..8c+7 and their rotation partners 8c+D/2..8c+D/2+7.
template <int D>
__global__ __launch_bounds__(256) void append_kernel(const AppendArgs a) {
  constexpr int NC = D / 16;
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.B * a.n_new * a.Hkv * NC;
  if (t >= total) return;
  const int32_t c = (int32_t)(t % NC);
  t /= NC;
  const int32_t h = (int32_t)(t % a.Hkv);
  t /= a.Hkv;
  const int32_t i = (int32_t)(t % a.n_new);
  const int32_t b = (int32_t)(t / a.n_new);
  const int32_t p = a.pos[b] + i;
  if (p < 0 || (p >> 4) >= a.max_blocks) return;
  const int32_t id = a.table[(int64_t)b * a.max_blocks + (p >> 4)];
  if (id < 0 || id >= a.num_blocks) return;  // no block allocated: nothing is written
  const int32_t slot = p & 15;

  const size_t src = (((size_t)b * a.n_new + i) * a.Hkv + h) * D;
  const bf16x8 x1 = *(const bf16x8*)(a.k_new + src + 8 * c);
  const bf16x8 x2 = *(const bf16x8*)(a.k_new + src + 8 * c + D / 2);
  const bf16x8 v1 = *(const bf16x8*)(a.v_new + src + 8 * c);
  const bf16x8 v2 = *(const bf16x8*)(a.v_new + src + 8 * c + D / 2);

  const size_t blk = ((size_t)id * a.Hkv + h) * (size_t)(D * 16);
  const size_t k_lo = blk + ((size_t)c * 16 + slot) * 8;              // channel octet c
  const size_t k_hi = blk + ((size_t)(c + D / 16) * 16 + slot) * 8;   // octet c + D/16
  if (a.ks != nullptr) {
    *(bf16x8*)(a.ks + k_lo) = x1;
    *(bf16x8*)(a.ks + k_hi) = x2;
  }
  if (a.rope == DRAFT_ATTN_ROPE_NEOX) {
    u16x8 r1, r2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      double sn, cs;
      sincos((double)p * a.omega[8 * c + e], &sn, &cs);
      const double y1 = (double)(float)x1[e] * cs - (double)(float)x2[e] * sn;
      const double y2 = (double)(float)x1[e] * sn + (double)(float)x2[e] * cs;
      r1[e] = bf16_bits_rne(y1);
      r2[e] = bf16_bits_rne(y2);
    }
    *(u16x8*)(a.k + k_lo) = r1;
    *(u16x8*)(a.k + k_hi) = r2;
  } else {
    *(bf16x8*)(a.k + k_lo) = x1;
    *(bf16x8*)(a.k + k_hi) = x2;
  }
  // Values: channel-major blocks, one 2-byte store per channel.
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a.v[blk + (size_t)(8 * c + e) * 16 + slot] = v1[e];
    a.v[blk + (size_t)(8 * c + e + D / 2) * 16 + slot] = v2[e];
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
      mis(block_table, 4) || mis(pos_dev, 4))
    return DRAFT_ATTN_EINVAL;
  AppendArgs a;
  a.k_new = (const __bf16*)k_new;
  a.v_new = (const __bf16*)v_new;
  a.table = block_table;
  a.pos = pos_dev;
  a.k = (__bf16*)k_cache;
  a.v = (__bf16*)v_cache;
  a.ks = (__bf16*)k_side;
  a.B = p->num_seqs;
  a.n_new = p->num_new;
  a.Hkv = p->num_kv_heads;
  a.max_blocks = p->max_blocks_per_seq;
  a.num_blocks = p->num_blocks;
  a.rope = p->rope;
  const int D = p->head_dim;
  for (int i = 0; i < 64; ++i) a.omega[i] = i < D / 2 ? pow(p->rope_theta, -2.0 * (double)i / (double)D) : 0.0;
  const int64_t threads = (int64_t)a.B * a.n_new * a.Hkv * (D / 16);
  const uint32_t grid = (uint32_t)((threads + 255) / 256);
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  if (D == 64) append_kernel<64><<<grid, 256, 0, s>>>(a);
  else append_kernel<128><<<grid, 256, 0, s>>>(a);
  if (hipGetLastError() != hipSuccess) return DRAFT_ATTN_EHIP;
  return DRAFT_ATTN_OK;
}

// KV append with FOLD side-cache bookkeeping, for CDNA4 (gfx950).
//
// "FOLD: Position-Free Far Memory with Local Order for Long-Context Speculative
// Decoding" (review) keeps an unrotated side cache beside the usual rotated one
// and names its bookkeeping as part of the cost. For each newly accepted token
// at position p this kernel writes the key turned to its own position, R(p) k,
// into k_cache, the unrotated key into k_side, and the value into v_cache, at the
// slot the block table gives for p. The rotation is done in fp64 (angles formed
// and reduced by the fp64 sincos, then advanced by fp64 rotation steps across a
// few consecutive positions) and rounded once to bf16, to nearest with ties to
// even: the stored key is the bf16 value nearest to an fp64 rotation that is
// within a few fp64 ulps of the exact one.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "host.h"

namespace da {


struct AppendArgs {
  const __bf16* k_new;  // [B][n_new][Hkv][D]
  const __bf16* v_new;  // [B][n_new][Hkv][D]
  const int32_t* table;
  const int32_t* pos;   // [B] position of each sequence's first new token
  __bf16* k;            // [blocks][Hkv][D/8][16][8]
  __bf16* v;            // [blocks][Hkv][D][16]
  __bf16* ks;           // like k, or null
  int32_t B, n_new, Hkv, max_blocks, num_blocks, rope;
  int32_t span;         // logical blocks one sequence's append can touch
  double omega[64];     // rope_theta^(-2i/D)
  double cos_w[64];     // cos(omega_i), sin(omega_i): one position step
  double sin_w[64];
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
// is written per slot). Rotation: thread (pair i, slot group q) forms the angle
// of its first slot with the fp64 sincos and advances it one position at a time
// by the rotation (cos w_i, sin w_i), which adds a few fp64 ulps.
template <int D>
__global__ __launch_bounds__(256) void append_kernel(const AppendArgs a) {
  constexpr int NO = D / 8;               // channel octets
  constexpr int HALF = D / 2;             // rotation pairs
  constexpr int SPT = 16 * HALF / 256;    // slots per thread in the rotation
  constexpr int LD = D + 8;               // padded LDS row (elements)
  __shared__ __align__(16) __bf16 s_k[16][LD];
  __shared__ __align__(16) __bf16 s_v[16][LD];
  __shared__ __align__(16) __bf16 s_r[16][LD];
  const int tid = threadIdx.x;
  int64_t w = blockIdx.x;
  const int32_t h = (int32_t)(w % a.Hkv);
  w /= a.Hkv;
  const int32_t jj = (int32_t)(w % a.span);
  const int32_t b = (int32_t)(w / a.span);
  const int32_t p0 = a.pos[b];
  if (p0 < 0) return;
  const int32_t j = (p0 >> 4) + jj;
  const int64_t lo64 = (int64_t)j * 16 > p0 ? (int64_t)j * 16 : p0;
  const int64_t hi64 = (int64_t)p0 + a.n_new < (int64_t)j * 16 + 16 ? (int64_t)p0 + a.n_new : (int64_t)j * 16 + 16;
  if (lo64 >= hi64 || j >= a.max_blocks) return;
  const int32_t id = a.table[(int64_t)b * a.max_blocks + j];
  if (id < 0 || id >= a.num_blocks) return;  // no block allocated: nothing is written
  const int s0 = (int)(lo64 - (int64_t)j * 16), s1 = (int)(hi64 - (int64_t)j * 16);
  const int32_t i0 = (int32_t)(lo64 - p0);  // index of slot s0's token among the new ones

  // Stage the new tokens' keys and values: one 16-byte octet per thread.
  for (int e = tid; e < 16 * NO; e += 256) {
    const int s = e / NO, c = e - s * NO;
    if (s < s0 || s >= s1) continue;
    const size_t src = (((size_t)b * a.n_new + (i0 + s - s0)) * a.Hkv + h) * D + 8 * c;
    *(uint4*)&s_k[s][8 * c] = *(const uint4*)(a.k_new + src);
    *(uint4*)&s_v[s][8 * c] = *(const uint4*)(a.v_new + src);
  }
  __syncthreads();

  // Rotate: thread (i, q) owns pair (i, i + D/2) of slots q*SPT .. q*SPT + SPT - 1.
  if (a.rope == DRAFT_ATTN_ROPE_NEOX) {
    const int i = tid % HALF, q = tid / HALF;
    int sa = q * SPT, sb = sa + SPT;
    sa = sa > s0 ? sa : s0;
    sb = sb < s1 ? sb : s1;
    if (sa < sb) {
      double sn, cs;
      sincos((double)((int64_t)j * 16 + sa) * a.omega[i], &sn, &cs);
      const double cw = a.cos_w[i], sw = a.sin_w[i];
      for (int s = sa; s < sb; ++s) {
        const double x1 = (double)(float)s_k[s][i], x2 = (double)(float)s_k[s][i + HALF];
        const unsigned short r1 = bf16_bits_rne(x1 * cs - x2 * sn);
        const unsigned short r2 = bf16_bits_rne(x1 * sn + x2 * cs);
        s_r[s][i] = __builtin_bit_cast(__bf16, r1);
        s_r[s][i + HALF] = __builtin_bit_cast(__bf16, r2);
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
    *(uint4*)(a.k + dst) = *(const uint4*)&kr[s][8 * c];
    if (a.ks != nullptr) *(uint4*)(a.ks + dst) = *(const uint4*)&s_k[s][8 * c];
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
      *(bf16x8_t*)dst = o;
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
  for (int i = 0; i < 64; ++i) {
    a.omega[i] = i < D / 2 && p->rope == DRAFT_ATTN_ROPE_NEOX ? pow(p->rope_theta, -2.0 * (double)i / (double)D) : 0.0;
    a.cos_w[i] = cos(a.omega[i]);
    a.sin_w[i] = sin(a.omega[i]);
  }
  a.span = (p->num_new + 15) / 16 + 1;
  const uint32_t grid = (uint32_t)((int64_t)a.B * a.span * a.Hkv);
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  if (D == 64) append_kernel<64><<<grid, 256, 0, s>>>(a);
  else append_kernel<128><<<grid, 256, 0, s>>>(a);
  if (hipGetLastError() != hipSuccess) return DRAFT_ATTN_EHIP;
  return DRAFT_ATTN_OK;
}

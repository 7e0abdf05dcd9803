// Host-side validation and planning for draft_attn_decode. Pure C++: no HIP
// headers, so the same file also builds with g++ for sanitizer runs.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/draft_attn.h"

namespace da {

struct Prepared {
  int32_t chunk;          // C: keys per work item (multiple of 32)
  int64_t total_items;    // work items over all sequences and kv heads
  int32_t G;              // query heads per kv head
  int32_t rows;           // R = G * T query rows per (sequence, kv head)
  int32_t row_tiles;      // ceil(R / 16)
  int32_t rows_pad;       // 16 * row_tiles
  bool single;            // one kernel: a workgroup that finds its group done merges it
  int32_t max_group_items;// largest item count of one (sequence, kv head)
  size_t flag_offset;     // workspace offset of the per-item 64-bit done flags
  size_t stat_offset;     // workspace offset of the per-row statistics
  size_t acc_offset;      // workspace offset of the per-row partial outputs
  size_t draft_offset;    // workspace offset of the fused call's draft parts: out_d [B*T*Hq][d], then lse_d [B*T*Hq]
  size_t workspace_bytes; // bytes the call needs
};

// Checks every scalar argument and the host context lengths, picks the chunk
// size and sizes the workspace. Returns a DRAFT_ATTN_* status.
int prepare(const draft_attn_params* p, const int32_t* ctx_len_host, Prepared* out);

// Checks the scalar arguments and host positions of draft_attn_append.
int prepare_append(const draft_attn_append_params* p, const int32_t* pos_host);

// NeoX RoPE frequencies for head dim d (at most 128): omega_i = theta^(-2i/d),
// one position step (cos omega_i, sin omega_i) and one slot-group step of
// g = d/32 positions (cos g omega_i, sin g omega_i), zero past d/2. A pure
// function of (theta, d), kept in a per-thread memo: the 64 pow and 192 cos/sin
// calls would otherwise cost a few microseconds of host time per call.
struct RopeTable {
  double theta;
  int32_t d;
  double omega[64], cos_w[64], sin_w[64], cos_g[64], sin_g[64];
};
const RopeTable& rope_table(double theta, int32_t d);

// With DRAFT_ATTN_LOG=1 in the environment (read once), prints a decode call's
// plan to stderr: shapes, mode, chunk size, work items and launch shape.
void log_plan(const draft_attn_params* p, const Prepared& pr);

}  // namespace da

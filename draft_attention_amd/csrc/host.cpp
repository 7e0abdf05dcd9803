// Host-side validation, chunk choice, workspace sizing and plan introspection.
// See the header draft_attn.h for the argument contract.
#include "host.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "plan.h"

namespace da {

namespace {

// Chunk-size model. Each work item is streamed by one 4-wave workgroup; the
// number resident per compute unit is set by registers, and the kernel asks the
// compiler for it (head_dim 128 -> 1; head_dim 64 -> 3 with one row tile, 2
// with two). An item's four waves take its 32-key steps in turn, so an item
// of at most P keys lasts about ceil(P / 128) steps of its busiest wave: P is
// rounded up to a multiple of 128 keys, which never adds a step to any wave
// and leaves fewer items (fewer records to merge). With such items, r rounds
// over the resident slots take about r * (P + kItemOverheadKeys) key-steps,
// the overhead being an item's start-up (block-table and query loads before
// the first K/V load). The planner tries 1..kMaxRounds rounds and keeps the
// cheapest.
constexpr int32_t kComputeUnits = 256;  // MI355X
constexpr int64_t kItemOverheadKeys = 256;
constexpr int32_t kMaxRounds = 4;
constexpr int32_t kMinAutoChunk = 128;  // one 32-key step per wave
constexpr int32_t kWaveRoundKeys = 128;  // one 32-key step for each of the four waves
constexpr int32_t kMaxChunk = 65536;    // bounds the block-id table kept in LDS
constexpr int32_t kMaxLen = 1 << 30;

// The streaming kernel requests exactly this occupancy from the compiler
// (amdgpu_waves_per_eu, pass1_occupancy() in decode.hip), so the two agree.
int32_t resident_per_cu(int32_t D, int32_t row_tiles) { return D == 128 ? 1 : (row_tiles == 1 ? 3 : 2); }

int32_t round_up_32(int64_t x) { return (int32_t)((x + 31) / 32 * 32); }

int64_t count_items(const draft_attn_params* p, const int32_t* lens, int32_t P) {
  int64_t items = 0;
  for (int32_t b = 0; b < p->num_seqs; ++b)
    items += (int64_t)seq_items(seq_ranges(lens[b], p->mode, p->window, p->n_sink), P, nullptr) * p->num_kv_heads;
  return items;
}

// Smallest P in [lo, kMaxChunk] (multiple of 32) with at most `budget` items;
// kMaxChunk when none fits. Item count does not grow with P.
int32_t fit_chunk(const draft_attn_params* p, const int32_t* lens, int32_t lo, int64_t budget) {
  if (count_items(p, lens, lo) <= budget) return lo;
  int32_t bad = lo, good = kMaxChunk;
  if (count_items(p, lens, good) > budget) return good;
  while (good - bad > 32) {
    const int32_t mid = round_up_32(((int64_t)bad + good) / 2);
    if (mid >= good) break;
    if (count_items(p, lens, mid) <= budget) good = mid;
    else bad = mid;
  }
  return good;
}

int32_t choose_chunk(const draft_attn_params* p, const int32_t* lens, int64_t keyheads, int32_t row_tiles) {
  const int64_t slots = (int64_t)kComputeUnits * resident_per_cu(p->head_dim, row_tiles);
  int32_t best = kMinAutoChunk;
  int64_t best_cost = -1;
  for (int32_t r = 1; r <= kMaxRounds; ++r) {
    const int64_t budget = r * slots;
    int64_t lo = (keyheads + budget - 1) / budget;
    lo = lo < kMinAutoChunk ? kMinAutoChunk : (lo > kMaxChunk ? kMaxChunk : lo);
    int32_t P = fit_chunk(p, lens, round_up_32(lo), budget);
    P = (int32_t)((P + kWaveRoundKeys - 1) / kWaveRoundKeys * kWaveRoundKeys);
    P = P > kMaxChunk ? kMaxChunk : P;
    const int64_t items = count_items(p, lens, P);
    const int64_t rounds = (items + slots - 1) / slots;
    const int64_t cost = (rounds > 0 ? rounds : 1) * ((int64_t)P + kItemOverheadKeys);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = P;
    }
  }
  return best;
}

// Largest number of items of one (sequence, kv head) at chunk P.
int32_t max_group_items(const draft_attn_params* p, const int32_t* lens, int32_t P) {
  int32_t m = 0;
  for (int32_t b = 0; b < p->num_seqs; ++b) {
    const int32_t n = seq_items(seq_ranges(lens[b], p->mode, p->window, p->n_sink), P, nullptr);
    m = n > m ? n : m;
  }
  return m;
}

// True when some sequence has no work item (no visible key). Its output rows
// are written by the merge kernel only, so such a batch runs on two kernels.
bool has_empty_group(const draft_attn_params* p, const int32_t* lens) {
  for (int32_t b = 0; b < p->num_seqs; ++b)
    if (seq_items(seq_ranges(lens[b], p->mode, p->window, p->n_sink), kMaxChunk, nullptr) == 0) return true;
  return false;
}

// Smallest chunk >= lo (multiple of 32) with at most `cap` items per group;
// -1 when even kMaxChunk has more. Group item counts do not grow with P.
int32_t fit_group_chunk(const draft_attn_params* p, const int32_t* lens, int32_t lo, int32_t cap) {
  if (max_group_items(p, lens, lo) <= cap) return lo;
  if (max_group_items(p, lens, kMaxChunk) > cap) return -1;
  int32_t bad = lo, good = kMaxChunk;
  while (good - bad > 32) {
    const int32_t mid = round_up_32(((int64_t)bad + good) / 2);
    if (mid >= good) break;
    if (max_group_items(p, lens, mid) <= cap) good = mid;
    else bad = mid;
  }
  return good;
}

// Single-launch choice for DRAFT_ATTN_LAUNCH_AUTO. The single kernel saves the
// merge kernel and one kernel boundary, but the workgroup that completes a
// (sequence, kv head) group then merges it alone: it writes a done flag, reads
// the group's flags and reads every partial record of the group, n items *
// padded rows * d * 4 bytes, all through the device's coherence point. When
// the whole step is one round of workgroups, that tail is on the critical path,
// and on MI355X the two-kernel step now wins every such shape measured (4K to
// 1M contexts, windows of 64 to 4096 keys: by 0.8 to 6 us). When there are more
// items than resident workgroups, early groups merge while later items still
// stream, and the single launch still pays up to the largest group measured
// (160 KiB of records: the 16-sequence batch, 0.2-0.4%).
constexpr size_t kAutoSingleGroupBytesMultiRound = 160 * 1024;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool finite_f(double x) { return isfinite(x) != 0; }

}  // namespace

int prepare(const draft_attn_params* p, const int32_t* ctx_len_host, Prepared* out) {
  if (!p || !out) return DRAFT_ATTN_EINVAL;
  if (p->struct_size != sizeof(draft_attn_params)) return DRAFT_ATTN_EINVAL;
  if (p->fold_variant < DRAFT_ATTN_FOLD_B || p->fold_variant > DRAFT_ATTN_FOLD_VIRTUAL) return DRAFT_ATTN_EINVAL;
  if (p->launch < DRAFT_ATTN_LAUNCH_AUTO || p->launch > DRAFT_ATTN_LAUNCH_SINGLE) return DRAFT_ATTN_EINVAL;
  if (p->out_dtype != DRAFT_ATTN_OUT_F32 && p->out_dtype != DRAFT_ATTN_OUT_BF16) return DRAFT_ATTN_EINVAL;
  const int32_t B = p->num_seqs, T = p->num_draft_tokens, Hq = p->num_q_heads, Hkv = p->num_kv_heads;
  if (B < 0 || T < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return DRAFT_ATTN_EINVAL;
  if (p->block_size != kBlock) return DRAFT_ATTN_EINVAL;
  if (p->head_dim < 1) return DRAFT_ATTN_EINVAL;
  if (p->num_blocks < 0 || p->max_blocks_per_seq < 1) return DRAFT_ATTN_EINVAL;
  if (p->mode != kFull && p->mode != kWindow && p->mode != kFold) return DRAFT_ATTN_EINVAL;
  if (p->window < 0 || p->n_sink < 0 || p->window > kMaxLen || p->n_sink > kMaxLen) return DRAFT_ATTN_EINVAL;
  if (p->mode == kFold && p->n_sink != 0) return DRAFT_ATTN_EINVAL;
  if (p->n0 < 1) return DRAFT_ATTN_EINVAL;
  if (p->rope != DRAFT_ATTN_ROPE_NEOX && p->rope != DRAFT_ATTN_ROPE_NONE) return DRAFT_ATTN_EINVAL;
  if (!finite_f(p->alpha) || !(p->alpha > 0.f)) return DRAFT_ATTN_EINVAL;
  if (!finite_f(p->beta) || !finite_f(p->kappa)) return DRAFT_ATTN_EINVAL;
  if (!finite_f(p->softmax_scale) || !(p->softmax_scale > 0.f)) return DRAFT_ATTN_EINVAL;
  if (p->mode == kFold && p->rope == DRAFT_ATTN_ROPE_NEOX &&
      (!finite_f(p->rope_theta) || !(p->rope_theta > 0.0)))
    return DRAFT_ATTN_EINVAL;
  if (p->split_keys != 0 && (p->split_keys < 32 || p->split_keys > kMaxChunk || p->split_keys % 32 != 0))
    return DRAFT_ATTN_EINVAL;
  if (p->debug_visit && p->debug_visit_stride < 1) return DRAFT_ATTN_EINVAL;
  if (B > 0 && !ctx_len_host) return DRAFT_ATTN_EINVAL;
  if ((int64_t)p->max_blocks_per_seq * kBlock > (int64_t)kMaxLen * 2) return DRAFT_ATTN_EINVAL;

  // Context lengths, query scale and the total key count.
  int64_t keyheads = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t L = ctx_len_host[b];
    if (L < 0 || L > kMaxLen) return DRAFT_ATTN_EINVAL;
    if ((int64_t)L > (int64_t)p->max_blocks_per_seq * kBlock) return DRAFT_ATTN_EINVAL;
    if (L > 0 && p->num_blocks < 1) return DRAFT_ATTN_EINVAL;
    if (p->debug_visit && (int64_t)L > p->debug_visit_stride) return DRAFT_ATTN_EINVAL;
    const int32_t n = visible_count(L, p->mode, p->window, p->n_sink);
    const double s = 1.0 + (double)p->kappa * log((double)(n > p->n0 ? n : p->n0) / (double)p->n0);
    if (!(s > 0.0)) return DRAFT_ATTN_EINVAL;
    keyheads += (int64_t)n * Hkv;
  }

  // Kernel coverage of the library.
  if (p->head_dim != 64 && p->head_dim != 128) return DRAFT_ATTN_ENOTSUP;
  const int32_t G = Hq / Hkv;
  const int64_t R = (int64_t)G * T;
  if (R > DRAFT_ATTN_MAX_ROWS) return DRAFT_ATTN_ENOTSUP;

  const int32_t row_tiles = (int32_t)((R + 15) / 16);
  const int32_t rows_pad = 16 * row_tiles;
  int32_t C = p->split_keys != 0 ? p->split_keys : choose_chunk(p, ctx_len_host, keyheads, row_tiles);
  int32_t gmax = max_group_items(p, ctx_len_host, C);
  bool single = false;
  if (has_empty_group(p, ctx_len_host)) {
    single = false;
  } else if (p->launch == DRAFT_ATTN_LAUNCH_SINGLE) {
    single = true;
    if (gmax > DRAFT_ATTN_MAX_GROUP_ITEMS) {
      if (p->split_keys != 0) return DRAFT_ATTN_ENOTSUP;
      C = fit_group_chunk(p, ctx_len_host, C, DRAFT_ATTN_MAX_GROUP_ITEMS);
      if (C < 0) return DRAFT_ATTN_ENOTSUP;
      gmax = max_group_items(p, ctx_len_host, C);
    }
  } else if (p->launch == DRAFT_ATTN_LAUNCH_AUTO) {
    const size_t group_bytes = (size_t)gmax * rows_pad * p->head_dim * sizeof(float);
    const int64_t slots = (int64_t)kComputeUnits * resident_per_cu(p->head_dim, row_tiles);
    const bool multi_round = count_items(p, ctx_len_host, C) > slots;
    single = multi_round && gmax <= DRAFT_ATTN_MAX_GROUP_ITEMS && group_bytes <= kAutoSingleGroupBytesMultiRound;
  }
  const int64_t items = count_items(p, ctx_len_host, C);
  if (items > 0x7fffffff) return DRAFT_ATTN_EINVAL;
  if ((int64_t)B * Hkv * R > 0x7fffffff) return DRAFT_ATTN_EINVAL;

  out->chunk = C;
  out->total_items = items;
  out->G = G;
  out->rows = (int32_t)R;
  out->row_tiles = row_tiles;
  out->rows_pad = rows_pad;
  out->single = single;
  out->max_group_items = gmax;
  // Layout: [one 64-bit done flag per item] [stat] [acc] [draft parts]. The flags are
  // reserved on both paths so the layout does not depend on the launch shape.
  const size_t nrows = (size_t)items * (size_t)rows_pad;
  out->flag_offset = 0;
  out->stat_offset = align_up((size_t)items * sizeof(uint64_t), 256);
  out->acc_offset = out->stat_offset + align_up(nrows * 4 * sizeof(float), 256);
  // [draft parts] of draft_attn_decode_draft, reserved on every call so that
  // one workspace size serves both calls: B*T*Hq rows of d + 1 floats.
  out->draft_offset = out->acc_offset + align_up(nrows * (size_t)p->head_dim * sizeof(float), 256);
  const size_t drows = (size_t)B * T * Hq;
  out->workspace_bytes = align_up(out->draft_offset + drows * ((size_t)p->head_dim + 1) * sizeof(float), 256);
  if (out->workspace_bytes == 0) out->workspace_bytes = 256;
  return DRAFT_ATTN_OK;
}

void log_plan(const draft_attn_params* p, const Prepared& pr) {
  static const bool enabled = [] {
    const char* v = getenv("DRAFT_ATTN_LOG");
    return v != nullptr && v[0] == '1';
  }();
  if (!enabled) return;
  static const char* const kModes[] = {"full", "window", "fold"};
  fprintf(stderr,
          "draft_attn_decode: B=%d T=%d Hq=%d Hkv=%d d=%d mode=%s W=%d sinks=%d alpha=%g beta=%g kappa=%g "
          "chunk=%d items=%lld max_items_per_group=%d rows=%d launch=%s out=%s\n",
          p->num_seqs, p->num_draft_tokens, p->num_q_heads, p->num_kv_heads, p->head_dim, kModes[p->mode], p->window,
          p->n_sink, (double)p->alpha, (double)p->beta, (double)p->kappa, pr.chunk, (long long)pr.total_items,
          pr.max_group_items, pr.rows, pr.single ? "single" : "two_pass",
          p->out_dtype == DRAFT_ATTN_OUT_BF16 ? "bf16" : "f32");
}

int prepare_append(const draft_attn_append_params* p, const int32_t* pos_host) {
  if (!p) return DRAFT_ATTN_EINVAL;
  if (p->struct_size != sizeof(draft_attn_append_params) || p->reserved != 0) return DRAFT_ATTN_EINVAL;
  if (p->num_seqs < 0 || p->num_new < 1 || p->num_kv_heads < 1 || p->head_dim < 1) return DRAFT_ATTN_EINVAL;
  if (p->block_size != kBlock || p->max_blocks_per_seq < 1 || p->num_blocks < 0) return DRAFT_ATTN_EINVAL;
  if (p->rope != DRAFT_ATTN_ROPE_NEOX && p->rope != DRAFT_ATTN_ROPE_NONE) return DRAFT_ATTN_EINVAL;
  if (p->rope == DRAFT_ATTN_ROPE_NEOX && (!finite_f(p->rope_theta) || !(p->rope_theta > 0.0))) return DRAFT_ATTN_EINVAL;
  if (p->num_seqs > 0 && (!pos_host || p->num_blocks < 1)) return DRAFT_ATTN_EINVAL;
  for (int32_t b = 0; b < p->num_seqs; ++b) {
    if (pos_host[b] < 0) return DRAFT_ATTN_EINVAL;
    if ((int64_t)pos_host[b] + p->num_new > (int64_t)p->max_blocks_per_seq * kBlock) return DRAFT_ATTN_EINVAL;
  }
  if (p->head_dim != 64 && p->head_dim != 128) return DRAFT_ATTN_ENOTSUP;
  // grid: one workgroup per (sequence, touched logical block, kv head)
  if ((int64_t)p->num_seqs * ((p->num_new + 15) / 16 + 1) * p->num_kv_heads > (int64_t)0x7fffffff)
    return DRAFT_ATTN_EINVAL;
  return DRAFT_ATTN_OK;
}

const RopeTable& rope_table(double theta, int32_t d) {
  static thread_local RopeTable t = {0.0, 0, {}, {}, {}, {}, {}};
  if (t.d != d || memcmp(&t.theta, &theta, sizeof theta) != 0) {
    const double g = d / 32;
    for (int i = 0; i < 64; ++i) {
      t.omega[i] = i < d / 2 ? pow(theta, -2.0 * (double)i / (double)d) : 0.0;
      t.cos_w[i] = cos(t.omega[i]);
      t.sin_w[i] = sin(t.omega[i]);
      t.cos_g[i] = cos(g * t.omega[i]);
      t.sin_g[i] = sin(g * t.omega[i]);
    }
    t.theta = theta;
    t.d = d;
  }
  return t;
}

}  // namespace da

extern "C" {

void draft_attn_append_params_init(draft_attn_append_params* p) {
  if (!p) return;
  memset(p, 0, sizeof(*p));
  p->struct_size = sizeof(draft_attn_append_params);
  p->block_size = 16;
  p->rope = DRAFT_ATTN_ROPE_NEOX;
  p->rope_theta = 1e4;
}

void draft_attn_params_init(draft_attn_params* p) {
  if (!p) return;
  memset(p, 0, sizeof(*p));
  p->struct_size = sizeof(draft_attn_params);
  p->block_size = 16;
  p->mode = DRAFT_ATTN_FULL;
  p->n0 = 1;
  p->rope = DRAFT_ATTN_ROPE_NEOX;
  p->alpha = 1.f;
  p->beta = 0.f;
  p->kappa = 0.f;
  p->softmax_scale = 0.f;
  p->rope_theta = 1e4;
}

int draft_attn_workspace_size(const draft_attn_params* p, const int32_t* ctx_len_host, size_t* bytes) {
  if (!bytes) return DRAFT_ATTN_EINVAL;
  da::Prepared pr;
  const int st = da::prepare(p, ctx_len_host, &pr);
  if (st != DRAFT_ATTN_OK) return st;
  *bytes = pr.workspace_bytes;
  return DRAFT_ATTN_OK;
}

int draft_attn_plan(const draft_attn_params* p, const int32_t* ctx_len_host, int32_t* items,
                    int64_t capacity, int64_t* n_items, int32_t* chunk_keys, int32_t* launch) {
  if (!n_items || capacity < 0) return DRAFT_ATTN_EINVAL;
  da::Prepared pr;
  const int st = da::prepare(p, ctx_len_host, &pr);
  if (st != DRAFT_ATTN_OK) return st;
  int64_t w = 0;
  for (int32_t b = 0; b < p->num_seqs; ++b) {
    const da::Ranges r = da::seq_ranges(ctx_len_host[b], p->mode, p->window, p->n_sink);
    const int32_t n = da::seq_items(r, pr.chunk, nullptr);
    for (int32_t h = 0; h < p->num_kv_heads; ++h) {
      for (int32_t k = 0; k < n; ++k, ++w) {
        if (items && w < capacity) {
          const da::Item t = da::item_of(r, k, pr.chunk);
          int32_t* it = items + DRAFT_ATTN_PLAN_ITEM_INTS * w;
          it[0] = b; it[1] = h; it[2] = t.a; it[3] = t.e; it[4] = t.part; it[5] = t.first; it[6] = t.stride;
        }
      }
    }
  }
  *n_items = w;
  if (chunk_keys) *chunk_keys = pr.chunk;
  if (launch) *launch = pr.single ? DRAFT_ATTN_LAUNCH_SINGLE : DRAFT_ATTN_LAUNCH_TWO_PASS;
  return DRAFT_ATTN_OK;
}

int draft_attn_ring_size(int32_t window, int32_t n_sink, int32_t max_new, int32_t* sink_blocks,
                         int32_t* ring_len) {
  if (window < 0 || n_sink < 0 || max_new < 0 || !sink_blocks || !ring_len) return DRAFT_ATTN_EINVAL;
  if (window > (1 << 30) || n_sink > (1 << 30) || max_new > (1 << 30)) return DRAFT_ATTN_EINVAL;
  *sink_blocks = (n_sink + 15) / 16;
  *ring_len = (window + 15) / 16 + 1 + (max_new + 15) / 16;
  return DRAFT_ATTN_OK;
}

int draft_attn_ring_table(int32_t length, int32_t max_new, int32_t window, int32_t n_sink,
                          const int32_t* sink_phys, int32_t sink_blocks, const int32_t* ring_phys,
                          int32_t ring_len, int32_t* table_row, int32_t max_blocks_per_seq) {
  int32_t need_sinks = 0, need_ring = 0;
  if (draft_attn_ring_size(window, n_sink, max_new, &need_sinks, &need_ring) != DRAFT_ATTN_OK) return DRAFT_ATTN_EINVAL;
  if (length < 0 || !table_row || max_blocks_per_seq < 1) return DRAFT_ATTN_EINVAL;
  if (sink_blocks < need_sinks || ring_len < need_ring) return DRAFT_ATTN_EINVAL;
  if ((sink_blocks > 0 && !sink_phys) || !ring_phys) return DRAFT_ATTN_EINVAL;
  const int64_t end = (int64_t)length + max_new;  // one past the last position touched
  if (end > (int64_t)max_blocks_per_seq * 16) return DRAFT_ATTN_EINVAL;
  for (int32_t j = 0; j < max_blocks_per_seq; ++j) table_row[j] = -1;
  if (end == 0) return DRAFT_ATTN_OK;
  // Blocks touched: the sinks, and the window of the read through the last append.
  const int64_t s_end = n_sink < length ? n_sink : length;
  const int64_t w0 = length - window > 0 ? length - window : 0;
  for (int64_t j = 0; j < (s_end + 15) / 16; ++j)
    table_row[j] = j < sink_blocks ? sink_phys[j] : ring_phys[(j - sink_blocks) % ring_len];
  if (end > w0)
    for (int64_t j = w0 / 16; j <= (end - 1) / 16; ++j)
      table_row[j] = j < sink_blocks ? sink_phys[j] : ring_phys[(j - sink_blocks) % ring_len];
  return DRAFT_ATTN_OK;
}

const char* draft_attn_strerror(int status) {
  switch (status) {
    case DRAFT_ATTN_OK: return "ok";
    case DRAFT_ATTN_EINVAL: return "invalid argument";
    case DRAFT_ATTN_ENOSPC: return "workspace too small";
    case DRAFT_ATTN_EHIP: return "HIP launch error";
    case DRAFT_ATTN_ENOTSUP: return "shape not supported by the library's kernels";
    default: return "unknown status";
  }
}

int draft_attn_version(void) { return DRAFT_ATTN_ABI_VERSION; }

}  // extern "C"

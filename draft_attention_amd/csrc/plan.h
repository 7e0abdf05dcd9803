// Work decomposition shared by the host planner and the device kernels.
//
// A sequence's keys split into at most two ranges per mode (the visible sets of
// "Windowed-MTP: Removing the Full-Context Draft-KV Tax at Million-Token
// Context", Abstract, and the local/far split of "FOLD: Position-Free Far
// Memory with Local Order for Long-Context Speculative Decoding", summary).
// A range [a, e) is read in steps of 32 keys: pairs of 16-token blocks counted
// from the range's first block, a / 16 (keys of a step outside [a, e) are
// masked). Given a target P (a multiple of 32 keys), the range's steps are
// dealt round-robin to np = ceil(steps / (P / 32)) work items: item k takes
// steps k, k + np, k + 2 np, ... So no item reads more than P keys, the items
// of a range differ by at most one step, every block of a range belongs to one
// item, and the items of a range read neighbouring steps at the same time
// rather than places P keys apart (which, with blocks allocated in order,
// would send every workgroup to addresses a large power of two apart). Work
// items are ordered sequence-major, then kv head, then range, then item; the
// ranges of partition 0 (keys from k_cache) come before partition 1 (FOLD far
// keys from k_side). The kernels recompute this decomposition from ctx_len on
// the device instead of reading a work list, so nothing is copied from the host
// per call.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define DA_HD __host__ __device__ __forceinline__
#else
#define DA_HD static inline
#endif

namespace da {

enum : int32_t { kFull = 0, kWindow = 1, kFold = 2 };
enum : int32_t { kPartMain = 0, kPartFar = 1 };
constexpr int32_t kBlock = 16;

// At most two ranges, as named fields (no runtime-indexed arrays, so device
// code keeps them in registers).
struct Ranges {
  int32_t n;
  int32_t a0, e0, p0;  // first range [a0, e0), partition p0
  int32_t a1, e1, p1;  // second range, valid when n == 2
};

DA_HD int32_t imin(int32_t x, int32_t y) { return x < y ? x : y; }
DA_HD int32_t imax(int32_t x, int32_t y) { return x > y ? x : y; }

DA_HD Ranges make_ranges(int32_t n, int32_t a0, int32_t e0, int32_t p0, int32_t a1, int32_t e1,
                         int32_t p1) {
  Ranges r;
  r.n = n; r.a0 = a0; r.e0 = e0; r.p0 = p0; r.a1 = a1; r.e1 = e1; r.p1 = p1;
  return r;
}

// Key ranges [a, e) of one sequence of length L (validated: L, W, S >= 0).
DA_HD Ranges seq_ranges(int32_t L, int32_t mode, int32_t W, int32_t S) {
  if (L <= 0) return make_ranges(0, 0, 0, kPartMain, 0, 0, kPartMain);
  if (mode == kFull) return make_ranges(1, 0, L, kPartMain, 0, 0, kPartMain);
  const int32_t ws = imax(0, L - W);  // first key of the recent / local window
  if (mode == kWindow) {
    const int32_t s = imin(S, L);      // end of the sinks
    if (ws <= s) return make_ranges(1, 0, L, kPartMain, 0, 0, kPartMain);
    if (s > 0) return make_ranges(2, 0, s, kPartMain, ws, L, kPartMain);
    return make_ranges(1, ws, L, kPartMain, 0, 0, kPartMain);
  }
  // FOLD: local window first (partition 0), then the far memory (partition 1).
  if (ws > 0 && ws < L) return make_ranges(2, ws, L, kPartMain, 0, ws, kPartFar);
  if (ws < L) return make_ranges(1, ws, L, kPartMain, 0, 0, kPartMain);
  return make_ranges(1, 0, ws, kPartFar, 0, 0, kPartMain);
}

// Steps of the range [a, e): ceil(blocks / 2) over its blocks a / 16 .. (e - 1) / 16.
DA_HD int32_t range_steps(int32_t a, int32_t e) {
  return e > a ? ((((e - 1) >> 4) - (a >> 4)) >> 1) + 1 : 0;
}

// Number of work items of the range [a, e) under target P.
DA_HD int32_t range_chunks(int32_t a, int32_t e, int32_t P) {
  const int32_t per = P >> 5;  // steps per item at most
  return (range_steps(a, e) + per - 1) / per;
}

// Work items of one (sequence, kv head); *n_main receives those of partition 0.
DA_HD int32_t seq_items(const Ranges& r, int32_t P, int32_t* n_main) {
  const int32_t c0 = r.n > 0 ? range_chunks(r.a0, r.e0, P) : 0;
  const int32_t c1 = r.n > 1 ? range_chunks(r.a1, r.e1, P) : 0;
  if (n_main) *n_main = (r.p0 == kPartMain ? c0 : 0) + (r.p1 == kPartMain ? c1 : 0);
  return c0 + c1;
}

// Keys carrying weight in the softmax, the n of the query scale s(n)
// ("SharpDraft: Accelerating Long-Context Speculative Decoding with
// Cardinality-Aware Query Scaling", Abstract).
DA_HD int32_t visible_count(int32_t L, int32_t mode, int32_t W, int32_t S) {
  if (L <= 0) return 0;
  if (mode == kWindow) {
    const int64_t cap = (int64_t)S + (int64_t)W;
    return cap < (int64_t)L ? (int32_t)cap : L;
  }
  return L;
}

// Work item k (0 <= k < seq_items) of a (sequence, kv head): its range, its
// partition and its steps first, first + stride, ... (steps in all).
struct Item {
  int32_t a, e;    // the range [a, e)
  int32_t part;
  int32_t first;   // first step, counted within the range
  int32_t stride;  // the range's item count
  int32_t steps;   // steps of this item (>= 1)
};

DA_HD Item item_of(const Ranges& r, int32_t k, int32_t P) {
  const int32_t c0 = r.n > 0 ? range_chunks(r.a0, r.e0, P) : 0;
  const bool in0 = k < c0;
  Item it;
  it.a = in0 ? r.a0 : r.a1;
  it.e = in0 ? r.e0 : r.e1;
  it.part = in0 ? r.p0 : r.p1;
  it.first = in0 ? k : k - c0;
  it.stride = in0 ? c0 : range_chunks(r.a1, r.e1, P);
  it.steps = it.stride > 0 ? (range_steps(it.a, it.e) - it.first + it.stride - 1) / it.stride : 0;
  return it;
}

// First key of step s (0 <= s < it.steps) of an item; the step covers 32 keys.
DA_HD int32_t item_step_key(const Item& it, int32_t s) {
  return ((it.a >> 4) + 2 * (it.first + s * it.stride)) << 4;
}

}  // namespace da

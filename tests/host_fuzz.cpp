// Randomised exercise of the host validation and planner (host.cpp), built
// with AddressSanitizer and UBSan by tests/test_abi_host.py. Checks that every
// call returns a defined status, and that accepted plans stay inside [0, L).
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <random>
#include <vector>

#include "draft_attn.h"

int main() {
  std::mt19937 rng(1234);
  auto pick = [&](std::initializer_list<long long> v) { return *(v.begin() + rng() % v.size()); };
  long long accepted = 0;
  for (int iter = 0; iter < 20000; ++iter) {
    draft_attn_params p;
    draft_attn_params_init(&p);
    p.num_seqs = (int)pick({0, 1, 2, 3, 7, -1});
    p.num_draft_tokens = (int)pick({1, 2, 4, 8, 0, 33});
    p.num_kv_heads = (int)pick({1, 2, 8, 0});
    p.num_q_heads = p.num_kv_heads * (int)pick({1, 2, 4, 8, 3});
    p.head_dim = (int)pick({64, 128, 96, 0});
    p.num_blocks = (int)pick({0, 1, 100, 1 << 20});
    p.max_blocks_per_seq = (int)pick({1, 8, 300, 1 << 16, 0});
    p.mode = (int)pick({0, 1, 2, 3});
    p.window = (int)pick({0, 1, 17, 256, 4096, -5, 1 << 30});
    p.n_sink = (int)pick({0, 0, 4, 100, -1});
    p.n0 = (int)pick({1, 16, 4096, 0});
    p.alpha = (float)pick({1, 2, 4, 0, -1});
    p.beta = (float)pick({0, -1, 3});
    p.kappa = (float)pick({0, 1, -1}) * 0.1f;
    p.softmax_scale = (float)pick({0, 1}) * 0.125f;
    p.split_keys = (int)pick({0, 0, 32, 64, 48, 65536, 1 << 20});
    p.launch = (int)pick({0, 0, 1, 2, 3, -1});
    p.out_dtype = (int)pick({0, 0, 1, 2});
    std::vector<int32_t> lens(p.num_seqs > 0 ? p.num_seqs : 1);
    for (auto& L : lens) L = (int32_t)pick({0, 1, 15, 16, 17, 1000, 4800, 1 << 20, -3});
    size_t bytes = 0;
    const int st = draft_attn_workspace_size(&p, lens.data(), &bytes);
    if (st != DRAFT_ATTN_OK && st != DRAFT_ATTN_EINVAL && st != DRAFT_ATTN_ENOTSUP) {
      printf("bad status %d\n", st);
      return 1;
    }
    int64_t n = 0;
    int32_t chunk = 0;
    int32_t launch = -1;
    const int st2 = draft_attn_plan(&p, lens.data(), nullptr, 0, &n, &chunk, &launch);
    if (st2 != st) {
      printf("plan/workspace status mismatch %d %d\n", st, st2);
      return 1;
    }
    if (st != DRAFT_ATTN_OK) continue;
    ++accepted;
    if (n > 200000) continue;
    std::vector<int32_t> items(DRAFT_ATTN_PLAN_ITEM_INTS * (size_t)(n > 0 ? n : 1));
    int64_t n2 = 0;
    if (draft_attn_plan(&p, lens.data(), items.data(), n, &n2, &chunk, nullptr) != DRAFT_ATTN_OK || n2 != n) return 1;
    if (launch != DRAFT_ATTN_LAUNCH_SINGLE && launch != DRAFT_ATTN_LAUNCH_TWO_PASS) {
      printf("bad launch %d\n", launch);
      return 1;
    }
    if (p.launch == DRAFT_ATTN_LAUNCH_TWO_PASS && launch != DRAFT_ATTN_LAUNCH_TWO_PASS) {
      printf("two-pass request not honoured\n");
      return 1;
    }
    // Single launch: every (sequence, kv head) has 1..DRAFT_ATTN_MAX_GROUP_ITEMS items.
    std::vector<int64_t> per_group((size_t)p.num_seqs * p.num_kv_heads, 0);
    for (int64_t i = 0; i < n; ++i) {
      const int32_t* it = &items[DRAFT_ATTN_PLAN_ITEM_INTS * i];
      const int32_t L = lens[it[0]];
      if (it[2] < 0 || it[3] > L || it[2] >= it[3] || it[1] >= p.num_kv_heads || it[5] < 0 || it[5] >= it[6]) {
        printf("item out of range\n");
        return 1;
      }
      ++per_group[(size_t)it[0] * p.num_kv_heads + it[1]];
    }
    if (launch == DRAFT_ATTN_LAUNCH_SINGLE)
      for (int64_t c : per_group)
        if (c < 1 || c > DRAFT_ATTN_MAX_GROUP_ITEMS) {
          printf("single launch with %lld items in a group\n", (long long)c);
          return 1;
        }
    if (bytes < (size_t)n * 8 + (size_t)n * 16 * 4 * 4) {
      printf("workspace too small for the plan\n");
      return 1;
    }
  }
  printf("ok accepted=%lld\n", accepted);
  return 0;
}

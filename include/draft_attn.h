/*
 * draft_attn.h -- C ABI of libdraft_attn.so: decode attention of a speculative
 * draft head over a very long paged KV cache, on one AMD MI355X (gfx950).
 *
 * Sources (page titles; sections in brackets):
 *   [WMTP] "Windowed-MTP: Removing the Full-Context Draft-KV Tax at Million-Token
 *          Context" -- Abstract: a built-in draft head that attends over the whole
 *          cache pays a read that grows with context; a sliding window plus
 *          attention sinks on the draft only bounds that read. Its "Builds on"
 *          list names PagedAttention, RoFormer and StreamingLLM.
 *   [FOLD] "FOLD: Position-Free Far Memory with Local Order for Long-Context
 *          Speculative Decoding" -- summary, review, abstract: a local window at
 *          exact positions, all distant keys at one shared virtual position read
 *          from an unrotated side cache, and a decoupled softmax with a
 *          concentration factor alpha.
 *   [SD]   "SharpDraft: Accelerating Long-Context Speculative Decoding with
 *          Cardinality-Aware Query Scaling" -- Abstract: the query is scaled by a
 *          closed-form, fixed-slope function of the number of visible keys.
 *
 * ---------------------------------------------------------------------------
 * What one call computes. Notation: B sequences, L_b = ctx_len[b], T draft
 * tokens per sequence, Hq query heads, Hkv kv heads, G = Hq / Hkv, head dim d.
 * Query head h reads kv head h / G. All T draft tokens of a sequence attend to
 * the same L_b cached keys and not to each other (merge draft-to-draft
 * attention with the returned lse).
 *
 * 1. Visible sets, per mode:
 *    DRAFT_ATTN_FULL    V = [0, L)                                   [WMTP]
 *    DRAFT_ATTN_WINDOW  V = [0, min(n_sink, L)) U [max(0, L - W), L)  [WMTP]
 *                       (W does not count the sinks; keys keep the rotation they
 *                       were cached with -- the window masks, it does not re-index)
 *    DRAFT_ATTN_FOLD    Loc = [max(0, L - W), L), Far = [0, max(0, L - W)) [FOLD]
 *                       (no sinks: n_sink must be 0)
 * 2. Query scale [SD]; the page prints no formula, this library fixes
 *        s(n) = 1 + kappa * ln(max(n, n0) / n0),
 *    n = |V| for FULL and WINDOW, n = L for FOLD. Logit scale
 *    c = softmax_scale * s(n). kappa = 0 is the unmodified drafter. s(n) scales
 *    fp32 logits, never the bf16 query, and needs no workspace.
 * 3. Logits l_j = c * <q, k_j>, k_j from k_cache, over V (FULL, WINDOW) or Loc
 *    (FOLD). FOLD far logits phi_j = c * <q_far, u_j>, u_j from k_side, with
 *    q_far = R(-P_v) q and P_v = L - W - 1: every far key sits at the position
 *    of the newest far key. R(a) is NeoX rotate-half RoPE: for i < d/2 the pair
 *    (x_i, x_{i+d/2}) turns by a * rope_theta^(-2i/d) [WMTP, Builds on:
 *    RoFormer]. DRAFT_ATTN_ROPE_NONE makes R the identity (NoPE drafters).
 * 4. FULL, WINDOW:  lse = ln sum_V e^{l_j},  out = sum_V e^{l_j - lse} v_j.
 * 5. FOLD decoupled softmax; the page prints no formula, this library fixes
 *        Z_L = sum_Loc e^{l_j},  Z_F = sum_Far e^{phi_j},  Z_Fa = sum_Far e^{alpha phi_j}
 *        lse = ln(Z_L + e^beta Z_F)
 *        out = (sum_Loc e^{l_j} v_j + e^beta Z_F sum_Far (e^{alpha phi_j} / Z_Fa) v_j) / e^lse
 *    alpha sharpens weights inside the far memory only; the far memory's total
 *    weight against the window is e^beta Z_F / Z_L [FOLD, abstract]. alpha = 1,
 *    beta = 0 is one softmax over Loc U Far.
 * 6. An empty visible set gives out = 0 and lse = -inf.
 * 7. fold_variant selects other readings of FOLD's alpha/beta (same Z_L, Z_F, Z_Fa):
 *    DRAFT_ATTN_FOLD_B       (0, default) as in 5.
 *    DRAFT_ATTN_FOLD_JOINT   (1) one softmax with far logits alpha phi_j + beta:
 *                            lse = ln(Z_L + e^beta Z_Fa); alpha also scales the far total.
 *    DRAFT_ATTN_FOLD_VIRTUAL (2) the far memory is one virtual key with logit
 *                            beta + ln(Z_Fa)/alpha and value sum_Far (e^{alpha phi_j}/Z_Fa) v_j:
 *                            lse = ln(Z_L + e^beta Z_Fa^(1/alpha)).
 *    All three are one softmax over Loc U Far at alpha = 1, beta = 0.
 * Numerics: bf16 inputs; logits, sums and outputs accumulate in fp32, and the
 * probabilities that weight the values are rounded to bf16 (relative to the
 * running maximum, so the dominant key's weight is exactly 1). FOLD's rotated
 * far query is kept as three bf16 terms (all 24 bits of its fp32 value), so
 * logits and lse are at fp32 level in every mode.
 *
 * ---------------------------------------------------------------------------
 * Layouts. All tensors are device memory owned by the caller; the library
 * never retains, frees or allocates them.
 *   q            bf16 [B][T][Hq][d], already RoPE-rotated by the caller at
 *                its own positions. 16-byte aligned.
 *   k_cache      bf16 [num_blocks][Hkv][d/8][16][8]: rotated keys in 16-token
 *                blocks; channel 8c + j of the key in slot s sits at [c][s][j], so
 *                the 16 keys' copies of one 8-channel group are contiguous (256 B)
 *                and a 64-lane 16-byte load covers 1 KiB contiguous. 16-byte aligned.
 *   v_cache      bf16 [num_blocks][Hkv][d][16]: values, channel-major inside a
 *                block (one channel's 16 slots contiguous), so a 16-byte load
 *                holds eight consecutive keys of one channel. 16-byte aligned.
 *   k_side       bf16 [num_blocks][Hkv][d/8][16][8]: unrotated keys, same layout
 *                and block ids as k_cache; read for FOLD's far keys only. NULL
 *                unless FOLD.
 *   block_table  int32 [B][max_blocks_per_seq]: key j of sequence b lives in
 *                block block_table[b][j / 16], slot j % 16 [WMTP, Builds on:
 *                PagedAttention]. Entries for blocks the mode never reads are
 *                not read and may hold anything (e.g. -1). An entry that is read
 *                (its block holds a key of the visible set) and lies outside
 *                [0, num_blocks) is treated as a block of masked keys (never
 *                dereferenced), and sets DRAFT_ATTN_STATUS_BAD_BLOCK in
 *                *status_flags when that pointer is set.
 *   ctx_len_dev  int32 [B] on the device, the same values as ctx_len_host;
 *                the kernels read it when B > 32 (smaller batches receive the
 *                host values with the launch arguments);
 *   ctx_len_host int32 [B] on the host, read for validation, grid and
 *                workspace sizing. A mismatch gives wrong results but no
 *                out-of-bounds access (and sets DRAFT_ATTN_STATUS_LENGTHS when
 *                a kernel notices it). Because grids are sized from the host
 *                lengths, a call captured in a HIP graph is bound to the host
 *                lengths of the capture: re-capture when they change.
 *   out          [B][T][Hq][d], written: fp32 (8-byte aligned) or, with
 *                out_dtype DRAFT_ATTN_OUT_BF16, bf16 rounded to nearest even
 *                from the fp32 result (8-byte aligned).
 *   lse          fp32 [B][T][Hq], natural log, written. 4-byte aligned.
 *   workspace    device scratch of at least draft_attn_workspace_size() bytes,
 *                256-byte aligned; its contents on entry do not matter. Its
 *                first bytes hold one 64-bit done flag per work item for the
 *                single-launch path; every call leaves them zero.
 *
 * Calls are asynchronous on `stream` (a hipStream_t). The library allocates
 * nothing, synchronises nothing and keeps no shared mutable state (its only
 * cache is a per-thread memo of the RoPE frequency table, a pure function of
 * rope_theta and head_dim): concurrent calls on different streams with
 * distinct workspaces are safe; calls that share a workspace must not overlap
 * in time.
 *
 * Errors: every check runs on the host before anything is enqueued, and a
 * non-zero return means nothing was enqueued. DRAFT_ATTN_EHIP reports a launch
 * failure seen by hipGetLastError() after enqueueing.
 *
 * Device-side status: the host cannot see the contents of device tables. When
 * params.status_flags points to a device uint32, the kernels OR the
 * DRAFT_ATTN_STATUS_* bits below into it when they meet such a problem (a bad
 * block id, lengths that disagree); the caller clears the word and reads it
 * after the stream has completed. NULL: nothing is reported (the default).
 *
 * Debugging: with DRAFT_ATTN_LOG=1 in the environment (read once, at the first
 * call), draft_attn_decode prints each call's plan to stderr: shapes, mode,
 * chunk size, work items and launch shape. Nothing else reads the environment.
 */
#ifndef DRAFT_ATTN_H
#define DRAFT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DRAFT_ATTN_ABI_VERSION 4

/* modes */
#define DRAFT_ATTN_FULL 0
#define DRAFT_ATTN_WINDOW 1
#define DRAFT_ATTN_FOLD 2

/* rotary encoding of the FOLD far query */
#define DRAFT_ATTN_ROPE_NEOX 0
#define DRAFT_ATTN_ROPE_NONE 1

/* FOLD parameterisations (fold_variant) */
#define DRAFT_ATTN_FOLD_B 0
#define DRAFT_ATTN_FOLD_JOINT 1
#define DRAFT_ATTN_FOLD_VIRTUAL 2

/* launch shapes (launch) */
#define DRAFT_ATTN_LAUNCH_AUTO 0    /* the library picks one of the two below */
#define DRAFT_ATTN_LAUNCH_TWO_PASS 1 /* streaming kernel, then a merge kernel */
#define DRAFT_ATTN_LAUNCH_SINGLE 2  /* one kernel: a workgroup that finds every
                                       item of its (sequence, kv head) done
                                       merges it */

/* output element types (out_dtype) */
#define DRAFT_ATTN_OUT_F32 0
#define DRAFT_ATTN_OUT_BF16 1

/* status codes */
#define DRAFT_ATTN_OK 0
#define DRAFT_ATTN_EINVAL (-1)   /* bad argument, shape, pointer or alignment */
#define DRAFT_ATTN_ENOSPC (-2)   /* workspace_bytes below draft_attn_workspace_size() */
#define DRAFT_ATTN_EHIP (-3)     /* the HIP runtime reported a launch error */
#define DRAFT_ATTN_ENOTSUP (-4)  /* valid, but the library has no kernel for it */

/* bits ORed into *status_flags by the kernels (device-side status above) */
#define DRAFT_ATTN_STATUS_BAD_BLOCK 1u        /* decode read a table entry outside [0, num_blocks):
                                                 its keys were masked */
#define DRAFT_ATTN_STATUS_LENGTHS 2u          /* ctx_len_dev held fewer work items than ctx_len_host */
#define DRAFT_ATTN_STATUS_APPEND_BAD_BLOCK 4u /* append met a table entry outside [0, num_blocks):
                                                 those tokens were not written */

/* Kernel support of the library: head_dim 64 or 128, block_size 16, and
 * G * T <= DRAFT_ATTN_MAX_ROWS query rows per (sequence, kv head). */
#define DRAFT_ATTN_MAX_ROWS 32

typedef struct draft_attn_params {
  uint32_t struct_size;        /* sizeof(draft_attn_params) */
  int32_t num_seqs;            /* B >= 0 (0: nothing to do) */
  int32_t num_draft_tokens;    /* T >= 1 */
  int32_t num_q_heads;         /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;        /* Hkv >= 1 */
  int32_t head_dim;            /* d: 64 or 128 */
  int32_t block_size;          /* must be 16 */
  int32_t num_blocks;          /* physical blocks in each pool */
  int32_t max_blocks_per_seq;  /* row stride of block_table; 16 * it >= every L */
  int32_t mode;                /* DRAFT_ATTN_FULL / _WINDOW / _FOLD */
  int32_t window;              /* W >= 0 (WINDOW, FOLD; ignored by FULL) */
  int32_t n_sink;              /* sinks >= 0 (WINDOW; must be 0 for FOLD; ignored by FULL) */
  int32_t n0;                  /* SharpDraft reference count, >= 1 */
  int32_t rope;                /* DRAFT_ATTN_ROPE_NEOX or _NONE (FOLD far query) */
  float alpha;                 /* FOLD concentration factor, finite, > 0 */
  float beta;                  /* FOLD far log-weight, finite */
  float kappa;                 /* SharpDraft slope, finite, with s(n) > 0 for every n */
  float softmax_scale;         /* finite, > 0; usually 1/sqrt(d) */
  double rope_theta;           /* RoPE base, finite, > 0 (FOLD with NEOX) */
  uint8_t* debug_visit;        /* optional device map [B][debug_visit_stride]: the kernel
                                  writes 1 for each key scored from k_cache and 2 for
                                  each key scored from k_side; untouched bytes keep
                                  the caller's value. NULL: off (the fast path). */
  int64_t debug_visit_stride;  /* >= max L when debug_visit is set */
  void* prof_events[2];        /* optional hipEvent_t pair recorded on `stream` just
                                  before and just after the streaming pass; NULL: off */
  int32_t split_keys;          /* most keys per work item: 0 = chosen by the library,
                                  else a multiple of 32 in [32, 65536] */
  int32_t fold_variant;        /* DRAFT_ATTN_FOLD_B (default), _JOINT or _VIRTUAL */
  int32_t launch;              /* DRAFT_ATTN_LAUNCH_AUTO (default), _TWO_PASS or _SINGLE.
                                  SINGLE needs at most DRAFT_ATTN_MAX_GROUP_ITEMS work
                                  items per (sequence, kv head): with split_keys 0 the
                                  library raises the chunk until that holds, with a
                                  fixed split_keys the call returns DRAFT_ATTN_ENOTSUP.
                                  A batch holding a sequence with no visible key runs
                                  on two kernels whatever the setting (its rows are
                                  written by the merge kernel) */
  int32_t out_dtype;           /* DRAFT_ATTN_OUT_F32 (default) or _BF16 */
  uint32_t* status_flags;      /* optional device word: the kernels OR DRAFT_ATTN_STATUS_* bits
                                  into it (4-byte aligned); NULL: off */
} draft_attn_params;

/* int32 values per work item written by draft_attn_plan. */
#define DRAFT_ATTN_PLAN_ITEM_INTS 7

/* Work items one workgroup merges on the single-launch path. */
#define DRAFT_ATTN_MAX_GROUP_ITEMS 64

/* Fill *p with defaults: FULL mode, block_size 16, alpha 1, beta 0, kappa 0,
 * n0 1, NEOX with rope_theta 1e4, softmax_scale 0 (the caller sets it), all
 * pointers NULL, struct_size set. Shapes stay 0. Never fails for non-NULL p. */
void draft_attn_params_init(draft_attn_params* p);

/* Workspace bytes that draft_attn_decode needs for these params and context
 * lengths (host array of num_seqs entries). The size depends on shapes, mode,
 * window, n_sink, split_keys and the lengths; it does not depend on alpha,
 * beta or kappa. Returns DRAFT_ATTN_OK or the status draft_attn_decode would
 * return for a validation failure. */
int draft_attn_workspace_size(const draft_attn_params* p, const int32_t* ctx_len_host,
                              size_t* bytes);

/* Enqueue one decode-attention call (definitions above) on `stream`.
 * q, k_cache, v_cache, k_side, block_table, ctx_len_dev, out, lse, workspace:
 * device pointers; ctx_len_host: host pointer. k_side must be non-NULL exactly
 * when mode is DRAFT_ATTN_FOLD. Returns a DRAFT_ATTN_* status. */
int draft_attn_decode(const draft_attn_params* p, const void* q, const void* k_cache,
                      const void* v_cache, const void* k_side, const int32_t* block_table,
                      const int32_t* ctx_len_dev, const int32_t* ctx_len_host, void* out,
                      float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Allocation-free decode, for callers that cannot allocate device memory or be
 * handed a workspace: code under HIP graph capture, tight serving loops and
 * harnesses that forbid allocation. The same call and result as
 * draft_attn_decode (bit for bit), without the workspace arguments: the partial
 * records live in a scratch array of DRAFT_ATTN_NOALLOC_SCRATCH_BYTES that the
 * library holds in device memory, one per GPU, for the life of the process. The
 * call allocates nothing and frees nothing. Its first call on a device (the
 * current device, which must own `stream` and every pointer) looks up that
 * device's copy of the array once.
 * A call whose draft_attn_workspace_size exceeds the scratch size returns
 * DRAFT_ATTN_ENOSPC before enqueueing anything. Every call on one GPU uses the
 * same array: calls that overlap in time on one GPU (on different streams, or
 * from different threads) race and give wrong results; serialise them. The
 * array keeps the last call's contents, which no call depends on (each call's
 * single-launch done flags are left zero, as with a workspace). */
#define DRAFT_ATTN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

int draft_attn_decode_noalloc(const draft_attn_params* p, const void* q, const void* k_cache,
                              const void* v_cache, const void* k_side, const int32_t* block_table,
                              const int32_t* ctx_len_dev, const int32_t* ctx_len_host, void* out,
                              float* lse, void* stream);

/* Measurement aid. A window step reads a constant number of keys whatever the
 * context ["Windowed-MTP: Removing the Full-Context Draft-KV Tax at
 * Million-Token Context", Abstract: the window bounds the draft's KV working set
 * to a constant], so its time is mostly fixed cost. This enqueues the launch
 * shape draft_attn_decode would use for these params and lengths with kernels
 * that do nothing: with kernels = 1, one kernel with the streaming pass's grid,
 * workgroup size, LDS and argument block; with kernels = 2, that kernel and
 * then one with the merge pass's grid and argument block. (The runtime's cost
 * of enqueueing a launch grows with the size of its argument block, so empty
 * kernels without arguments would understate it.) The time of such a step is
 * the launch floor under the decode call. Validation as for draft_attn_decode;
 * kernels must be 1 or 2. */
int draft_attn_launch_floor(const draft_attn_params* p, const int32_t* ctx_len_host, int32_t kernels,
                            void* stream);

/* Host-only introspection of the work decomposition a call would use: the
 * chunk size in keys (*chunk_keys: the most keys of one work item), the launch
 * shape (*launch: _TWO_PASS or _SINGLE) and the work items in launch order,
 * DRAFT_ATTN_PLAN_ITEM_INTS int32 each:
 *   {seq, kv_head, range_begin, range_end, partition, first_step, step_stride}.
 * A work item reads part of one key range [range_begin, range_end) of a
 * sequence's visible set (partition 0: keys read from k_cache; 1: FOLD far keys
 * read from k_side). The range is read in steps of 32 keys, pairs of 16-token
 * blocks counted from block range_begin / 16; the item takes the range's steps
 * first_step, first_step + step_stride, ... (step_stride is the range's item
 * count), keeping the keys of each step that lie in the range. The items of a
 * range thus share its steps round-robin and cover it exactly once. Writes at
 * most `capacity` items to `items` (may be NULL) and the total to *n_items;
 * chunk_keys and launch may be NULL. */
int draft_attn_plan(const draft_attn_params* p, const int32_t* ctx_len_host, int32_t* items,
                    int64_t capacity, int64_t* n_items, int32_t* chunk_keys, int32_t* launch);

/* ---------------------------------------------------------------------------
 * Draft-token self-attention, merged into a draft_attn_decode result in place.
 * Within one draft step, draft token t also attends to the step's own draft keys
 * 0..t, which are not in the cache yet. Given the cache attention (out, lse) of
 * the same step and params, this computes, per (b, t, h),
 *   lse_d = ln sum_{j<=t} e^{c <q, kd_j>},  out_d = sum_{j<=t} e^{c <q, kd_j> - lse_d} vd_j
 * and replaces (out, lse) by the merge of the two: lse <- logaddexp(lse, lse_d),
 * out <- e^{lse_old - lse} out + e^{lse_d - lse} out_d. The result is one softmax
 * over the cached visible keys and draft keys 0..t; in FOLD the draft keys join
 * the local window (they sit at exact positions next to it). c is the cache
 * call's scale softmax_scale * s(n), n the cached visible count (a reading: the
 * pages do not say whether the draft's own keys count).
 * q: bf16 [B][T][Hq][d] (the same queries as the decode call); k_draft (already
 * rotated at positions L_b + t) and v_draft: bf16 [B][T][Hkv][d]; out, lse: as
 * written by draft_attn_decode. p, ctx_len_dev and ctx_len_host: as for that call.
 * The merge needs the fp32 cache result: out_dtype DRAFT_ATTN_OUT_BF16 returns
 * DRAFT_ATTN_ENOTSUP, as do num_q_heads above 65535 and num_seqs above 2^26
 * (the merge kernel's grid spans the query heads in one dimension and the
 * sequences, 64 threads each, in another). */
int draft_attn_merge_draft(const draft_attn_params* p, const void* q, const void* k_draft, const void* v_draft,
                           const int32_t* ctx_len_dev, const int32_t* ctx_len_host, float* out, float* lse,
                           void* stream);

/* draft_attn_decode and draft_attn_merge_draft in one call: the cache
 * attention of the step, already merged with the draft part (same definitions
 * and arguments as those two calls; k_draft, v_draft as for merge_draft,
 * non-NULL, 16-byte aligned). With up to 8 draft tokens, extra workgroups of the
 * streaming kernel form the draft parts beside the cache pass; with more, the
 * merge kernel forms them. Either way the merge kernel writes each row already
 * merged, so the call runs on two kernels whatever `launch` says, saves the
 * separate merge launch, and may write out in bf16 (rounded once, from the
 * merged fp32 value). With out_dtype F32 the results equal those of the two
 * calls bit for bit. Errors as for draft_attn_decode; the workspace is sized by
 * draft_attn_workspace_size with the same params (it always reserves the draft
 * parts, B * T * Hq * (d + 1) floats). */
int draft_attn_decode_draft(const draft_attn_params* p, const void* q, const void* k_cache,
                            const void* v_cache, const void* k_side, const int32_t* block_table,
                            const int32_t* ctx_len_dev, const int32_t* ctx_len_host, const void* k_draft,
                            const void* v_draft, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * KV append with FOLD side-cache bookkeeping. For token i < num_new of sequence
 * b, at position p = pos[b] + i, in block block_table[b][p / 16] and slot p % 16:
 *   k_cache <- R(p) k_new[b][i]  rounded to bf16 (to nearest, ties to even) from
 *                                the fp64 rotation; with DRAFT_ATTN_ROPE_NONE the
 *                                key is copied unchanged
 *   k_side  <- k_new[b][i]       (when k_side is not NULL)
 *   v_cache <- v_new[b][i]
 * R(p) is the NeoX rotation of the header above at angle p * rope_theta^(-2i/d).
 * The unrotated side cache is what FOLD's far memory reads ["FOLD: Position-Free
 * Far Memory with Local Order for Long-Context Speculative Decoding", review].
 * k_new, v_new: bf16 [B][num_new][Hkv][d] device, 16-byte aligned; pos_dev /
 * pos_host: int32 [B] on device / host with the same values (for up to 32
 * sequences the kernel takes the positions from pos_host, passed with the
 * launch, so a captured call is bound to the host positions of the capture);
 * caches as for draft_attn_decode. Every written block must be allocated in block_table; a
 * token whose table entry lies outside [0, num_blocks) is not written (and
 * sets DRAFT_ATTN_STATUS_APPEND_BAD_BLOCK in *status_flags when that is set). Nothing
 * outside the new tokens' slots is touched. Validation is host-side and runs
 * before anything is enqueued. */
typedef struct draft_attn_append_params {
  uint32_t struct_size;        /* sizeof(draft_attn_append_params) */
  int32_t num_seqs;            /* B >= 0 */
  int32_t num_new;             /* tokens appended per sequence, >= 1 */
  int32_t num_kv_heads;        /* Hkv >= 1 */
  int32_t head_dim;            /* 64 or 128 */
  int32_t block_size;          /* must be 16 */
  int32_t num_blocks;          /* physical blocks in each pool */
  int32_t max_blocks_per_seq;  /* row stride of block_table; pos + num_new <= 16 * it */
  int32_t rope;                /* DRAFT_ATTN_ROPE_NEOX or _NONE */
  int32_t reserved;            /* must be 0 */
  double rope_theta;           /* finite, > 0 with NEOX */
  uint32_t* status_flags;      /* optional device word: DRAFT_ATTN_STATUS_APPEND_BAD_BLOCK is
                                  ORed into it for a token not written; NULL: off */
} draft_attn_append_params;

/* Defaults: block_size 16, NEOX with rope_theta 1e4, struct_size set. */
void draft_attn_append_params_init(draft_attn_append_params* p);

int draft_attn_append(const draft_attn_append_params* p, const void* k_new, const void* v_new,
                      const int32_t* block_table, const int32_t* pos_dev, const int32_t* pos_host,
                      void* k_cache, void* v_cache, void* k_side, void* stream);

/* ---------------------------------------------------------------------------
 * Ring-buffer draft cache for WINDOW mode. A window step reads only the sinks
 * [0, n_sink) and the recent window [L - W, L), so a sequence needs only
 * sink_blocks = ceil(n_sink / 16) fixed blocks plus a ring of ring_len blocks
 * that the recent window cycles through; the rest of the draft KV is never read
 * and need not be kept ["Windowed-MTP: Removing the Full-Context Draft-KV Tax
 * at Million-Token Context", Abstract: unread draft KV reclaimed by a compact
 * ring buffer]. Logical block j maps to sink_phys[j] for j < sink_blocks and to
 * ring_phys[(j - sink_blocks) % ring_len] otherwise.
 *
 * draft_attn_ring_size: the smallest sink_blocks and ring_len for a window W,
 * n_sink sinks and appends of up to max_new tokens between two window reads
 * (ring_len = ceil(W / 16) + 1 + ceil(max_new / 16)).
 *
 * draft_attn_ring_table: fill the block-table row (max_blocks_per_seq entries)
 * of a sequence of current length `length` that is about to be read in WINDOW
 * mode and then receive up to max_new appended tokens: entries of the blocks the
 * read or the appends touch get their physical block, every other entry -1.
 * Returns DRAFT_ATTN_EINVAL when ring_len or sink_blocks is smaller than
 * draft_attn_ring_size reports or a touched block lies past max_blocks_per_seq.
 * Host-only; the decode and append kernels are unchanged. */
int draft_attn_ring_size(int32_t window, int32_t n_sink, int32_t max_new, int32_t* sink_blocks,
                         int32_t* ring_len);
int draft_attn_ring_table(int32_t length, int32_t max_new, int32_t window, int32_t n_sink,
                          const int32_t* sink_phys, int32_t sink_blocks, const int32_t* ring_phys,
                          int32_t ring_len, int32_t* table_row, int32_t max_blocks_per_seq);

/* Static description of a status code. */
const char* draft_attn_strerror(int status);

/* DRAFT_ATTN_ABI_VERSION of the loaded library. */
int draft_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DRAFT_ATTN_H */

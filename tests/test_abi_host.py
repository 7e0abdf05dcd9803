"""Host side of the C ABI, on the CPU: exported symbols, the params struct
layout, every validation path, and the work decomposition against the
oracle's index sets. Nothing here launches a kernel."""

import ctypes
import os
import random
import re
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "draft_attn.h")


def da():
    import draft_attention_amd
    return draft_attention_amd


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[a-z][\w \*]*?\b(draft_attn_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert {"draft_attn_decode", "draft_attn_workspace_size", "draft_attn_strerror",
            "draft_attn_version", "draft_attn_plan", "draft_attn_params_init"} <= set(names)
    lib = ctypes.CDLL(da().LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert da().lib.draft_attn_version() == da().ABI_VERSION == 4


def test_params_layout_matches_the_c_compiler(tmp_path):
    fields = [f for f, _ in da().Params._fields_]
    src = tmp_path / "layout.c"
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', 'int main(void) {',
             'printf("%zu\\n", sizeof(draft_attn_params));']
    lines += [f'printf("%zu\\n", offsetof(draft_attn_params, {f}));' for f in fields]
    lines += ['return 0; }']
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", str(src), "-o", str(exe)], check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(da().Params)
    for f, off in zip(fields, vals[1:]):
        assert getattr(da().Params, f).offset == off, f


def test_append_params_layout_matches_the_c_compiler(tmp_path):
    fields = [f for f, _ in da().AppendParams._fields_]
    src = tmp_path / "alayout.c"
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', 'int main(void) {',
             'printf("%zu\\n", sizeof(draft_attn_append_params));']
    lines += [f'printf("%zu\\n", offsetof(draft_attn_append_params, {f}));' for f in fields]
    lines += ['return 0; }']
    src.write_text("\n".join(lines))
    exe = tmp_path / "alayout"
    subprocess.run(["gcc", "-std=c99", str(src), "-o", str(exe)], check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(da().AppendParams)
    for f, off in zip(fields, vals[1:]):
        assert getattr(da().AppendParams, f).offset == off, f


def _append_call(p, pos=(0, 5), **ptrs):
    P = dict(k=0x10000, v=0x20000, table=0x30000, posd=0x40000, kc=0x50000, vc=0x60000, ks=None)
    P.update(ptrs)
    host = (ctypes.c_int32 * max(len(pos), 1))(*pos)
    return da().lib.draft_attn_append(ctypes.byref(p), P["k"], P["v"], P["table"], P["posd"], host, P["kc"], P["vc"],
                                      P["ks"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(num_seqs=-1), -1), (dict(num_new=0), -1), (dict(num_kv_heads=0), -1), (dict(head_dim=96), -4),
    (dict(max_blocks_per_seq=0), -1), (dict(rope=7), -1), (dict(rope_theta=-1.0), -1), (dict(num_blocks=0), -1),
])
def test_append_validation(kw, status):
    base = dict(num_seqs=2, num_new=4, num_kv_heads=2, head_dim=128, num_blocks=16, max_blocks_per_seq=4)
    base.update(kw)
    assert _append_call(da().make_append_params(**base)) == status


def test_append_positions_pointers_and_alignment():
    mk = lambda **kw: da().make_append_params(**dict(dict(num_seqs=2, num_new=4, num_kv_heads=2, head_dim=128,
                                                          num_blocks=16, max_blocks_per_seq=4), **kw))
    assert _append_call(mk(), pos=(-1, 0)) == -1
    assert _append_call(mk(), pos=(61, 0)) == -1            # 61 + 4 > 64 slots
    for name in ("k", "v", "table", "posd", "kc", "vc"):
        assert _append_call(mk(), **{name: None}) == -1, name
    assert _append_call(mk(), k=0x10008) == -1
    assert _append_call(mk(), ks=0x70004) == -1
    p = mk()
    p.reserved = 3
    assert _append_call(p) == -1
    assert _append_call(mk(status_flags=0x80001)) == -1   # the status word needs 4-byte alignment
    assert _append_call(mk(num_seqs=0), pos=()) == 0
    assert _append_call(mk(rope="none", rope_theta=0.0), pos=(0, 0), k=None) == -1   # theta unused, pointer checked


def test_status_strings():
    for st in (0, -1, -2, -3, -4):
        assert da().strerror(st) and da().strerror(st) != "unknown status"
    assert da().strerror(-99) == "unknown status"


# ----------------------------------------------------------------------------- validation
BASE = dict(num_seqs=2, num_draft_tokens=4, num_q_heads=8, num_kv_heads=2, head_dim=128, num_blocks=64,
            max_blocks_per_seq=32, mode="window", window=100, n_sink=4, n0=16)
LENS = [300, 17]


def call(params, lens=LENS, side=None, fold=False, ws_bytes=1 << 30, **ptrs):
    """draft_attn_decode with fake, aligned device addresses: only reached code is host validation."""
    P = dict(q=0x10000, k=0x20000, v=0x30000, ks=0x40000 if fold else None, table=0x50000, ctx=0x60000,
             out=0x70000, lse=0x80000, ws=0x100000)
    P.update(ptrs)
    host = (ctypes.c_int32 * max(len(lens), 1))(*lens)
    return da().lib.draft_attn_decode(ctypes.byref(params), P["q"], P["k"], P["v"], P["ks"], P["table"],
                                      P["ctx"], host, P["out"], P["lse"], P["ws"], ws_bytes, None)


def params(**kw):
    d = dict(BASE)
    d.update(kw)
    return da().make_params(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(num_seqs=-1), -1), (dict(num_draft_tokens=0), -1), (dict(num_q_heads=7), -1),
    (dict(num_kv_heads=0), -1), (dict(head_dim=96), -4), (dict(head_dim=0), -1),
    (dict(num_q_heads=16, num_draft_tokens=5), -4),     # G*T = 40 rows > 32
    (dict(mode=7), -1), (dict(window=-1), -1), (dict(n_sink=-2), -1),
    (dict(mode="fold", n_sink=4), -1), (dict(n0=0), -1), (dict(rope=5), -1),
    (dict(alpha=0.0), -1), (dict(alpha=-1.0), -1), (dict(alpha=float("inf")), -1),
    (dict(beta=float("nan")), -1), (dict(kappa=float("inf")), -1), (dict(kappa=-10.0), -1),
    (dict(softmax_scale=0.0), -1), (dict(softmax_scale=float("nan")), -1),
    (dict(split_keys=48), -1), (dict(split_keys=16), -1), (dict(split_keys=1 << 20), -1),
    (dict(max_blocks_per_seq=10), -1),                  # 160 keys < L = 300
    (dict(num_blocks=0), -1),
])
def test_invalid_params_are_rejected_before_launch(kw, status):
    fold = kw.get("mode") == "fold"
    p = params(**kw)
    assert call(p, fold=fold) == status
    n = ctypes.c_size_t(0)
    host = (ctypes.c_int32 * 2)(*LENS)
    assert da().lib.draft_attn_workspace_size(ctypes.byref(p), host, ctypes.byref(n)) == status


def test_struct_size_reserved_and_theta_checked():
    p = params()
    p.struct_size = 64
    assert call(p) == -1
    p = params()
    p.fold_variant = 3
    assert call(p) == -1
    p = params(mode="fold", n_sink=0, rope_theta=0.0)
    assert call(p, fold=True) == -1
    p = params(mode="fold", n_sink=0, rope="none", rope_theta=0.0)   # theta unused without rotation
    assert da().workspace_size(p, LENS) > 0


def test_bad_lengths_pointers_and_alignment():
    assert call(params(), lens=[-1, 5]) == -1
    p = params()
    assert da().lib.draft_attn_decode(ctypes.byref(p), 0x1000, 0x1000, 0x1000, None, 0x1000, 0x1000, None,
                                      0x1000, 0x1000, 0x1000, 1 << 30, None) == -1   # no host lengths
    for name in ("q", "k", "v", "table", "ctx", "out", "lse", "ws"):
        assert call(params(), **{name: None}) == -1, name
    assert call(params(), q=0x10008) == -1            # bf16 tensors need 16-byte alignment
    assert call(params(), v=0x30004) == -1
    assert call(params(), out=0x70004) == -1
    assert call(params(), ws=0x100010) == -1
    assert call(params(status_flags=0x90002)) == -1   # the status word needs 4-byte alignment
    assert call(params(status_flags=0x90004), ws_bytes=0) == -2   # aligned: the checks go on
    # k_side exactly when FOLD
    assert call(params(), ks=0x40000) == -1
    assert call(params(mode="fold", n_sink=0), fold=True, ks=None) == -1


def test_workspace_too_small_and_prof_events():
    p = params()
    need = da().workspace_size(p, LENS)
    assert call(p, ws_bytes=need - 1) == -2
    p = params(prof_events=(0x1234, 0))
    p.prof_events[1] = None
    assert call(p) == -1


def test_noalloc_refuses_a_call_beyond_its_scratch():
    # 16 sequences of 1M keys at 8 kv heads need more partial records than the
    # library's scratch holds: refused on the host, before anything is enqueued
    # (fake, aligned device addresses, as above).
    lens = [1 << 20] * 16
    p = da().make_params(num_seqs=16, num_draft_tokens=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
                         num_blocks=16 << 16, max_blocks_per_seq=1 << 16)
    assert da().workspace_size(p, lens) > da().NOALLOC_SCRATCH_BYTES
    host = (ctypes.c_int32 * 16)(*lens)
    st = da().lib.draft_attn_decode_noalloc(ctypes.byref(p), 0x10000, 0x20000, 0x30000, None, 0x50000, 0x60000,
                                            host, 0x70000, 0x80000, None)
    assert st == da().ENOSPC
    p.num_draft_tokens = 0                               # validation comes first
    assert da().lib.draft_attn_decode_noalloc(ctypes.byref(p), 0x10000, 0x20000, 0x30000, None, 0x50000,
                                              0x60000, host, 0x70000, 0x80000, None) == -1


def test_noalloc_scratch_size_matches_the_header():
    text = open(HEADER).read()
    assert "#define DRAFT_ATTN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)" in text
    assert da().NOALLOC_SCRATCH_BYTES == 16 << 20


def test_launch_floor_validated_before_launch():
    host = (ctypes.c_int32 * 2)(*LENS)
    f = da().lib.draft_attn_launch_floor
    assert f(ctypes.byref(params()), host, 3, None) == -1
    assert f(ctypes.byref(params()), host, 0, None) == -1
    assert f(ctypes.byref(params(num_kv_heads=0)), host, 1, None) == -1
    assert f(ctypes.byref(params(num_seqs=0)), host, 2, None) == 0


def test_debug_visit_stride_checked():
    p = params(debug_visit=0x9000, debug_visit_stride=100)
    assert call(p) == -1          # L = 300 > stride


def test_empty_batch_is_a_noop():
    p = params(num_seqs=0)
    assert call(p, lens=[]) == 0


def test_workspace_independent_of_alpha_beta_kappa():
    base = da().workspace_size(params(mode="fold", n_sink=0), LENS)
    for kw in (dict(alpha=4.0), dict(beta=-3.0), dict(kappa=0.5), dict(alpha=0.1, beta=2.0, kappa=-0.1)):
        assert da().workspace_size(params(mode="fold", n_sink=0, **kw), LENS) == base


# ----------------------------------------------------------------------------- work decomposition
def _item_keys(item):
    """Keys a work item scores, from the documented item format: the 32-key steps
    first, first + stride, ... of its range, counted from block range_begin // 16,
    each clipped to [range_begin, range_end)."""
    _, _, a, e, _, first, stride = item
    base = a // 16
    nsteps = ((e - 1) // 16 - base) // 2 + 1
    parts = [np.arange(max(a, 16 * (base + 2 * t)), min(e, 16 * (base + 2 * t) + 32))
             for t in range(first, nsteps, stride)]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def _check_plan(mode, W, S, lens, Hkv, split):
    p = params(num_seqs=len(lens), num_kv_heads=Hkv, num_q_heads=Hkv * 2, num_draft_tokens=2, mode=mode,
               window=W, n_sink=S, split_keys=split, max_blocks_per_seq=max(1, (max(lens) + 15) // 16),
               num_blocks=1 << 20)
    items, C = da().plan(p, lens)
    assert C % 32 == 0 and (split == 0 or C == split)
    assert split != 0 or C % 128 == 0, "the library's chunk is whole rounds of the four waves' steps"
    seen, ranges = {}, {}
    prev = (-1, -1, -1)
    for item in items:
        b, h, a, e, part, first, stride = item
        assert 0 <= b < len(lens) and 0 <= h < Hkv and 0 <= a < e <= lens[b] and part in (0, 1)
        assert 0 <= first < stride
        keys = _item_keys(item)
        assert 0 < keys.size <= C, "item empty or longer than the target"
        assert (b, h, part) >= prev, "launch order is sequence, kv head, partition"
        prev = (b, h, part)
        seen.setdefault((b, h, part), []).append(keys)
        ranges.setdefault((b, h, a, e), []).append((first, stride))
    for (b, h, a, e), fs in ranges.items():
        stride = fs[0][1]
        assert fs == [(k, stride) for k in range(stride)], "a range's items take its steps round-robin, in order"
    for b, L in enumerate(lens):
        main, far = oracle.index_sets(L, mode, W, S)
        for h in range(Hkv):
            for part, want in ((0, main), (1, far)):
                got = np.concatenate(seen.get((b, h, part), []) or [np.zeros(0, dtype=np.int64)])
                assert np.array_equal(np.sort(got), want), (b, h, part)
                assert np.unique(got).size == got.size, "overlapping items"
    assert da().workspace_size(p, lens) >= len(items) * 16 * (128 + 4) * 4


def test_plan_covers_the_oracle_index_sets():
    rnd = random.Random(0)
    for _ in range(150):
        mode = rnd.choice(["full", "window", "fold"])
        lens = [rnd.choice([0, 1, 15, 16, 17, 31, 32, 33, rnd.randint(0, 5000)]) for _ in range(rnd.randint(1, 5))]
        W = rnd.choice([0, 1, 16, 31, 100, 4096, rnd.randint(0, 3000)])
        S = 0 if mode == "fold" else rnd.choice([0, 1, 4, 20, 100])
        split = rnd.choice([0, 32, 64, 96, 256])
        _check_plan(mode, W, S, lens, rnd.choice([1, 2, 8]), split)


def test_auto_chunk_size_balances_the_workloads():
    # One sequence of 2^20 keys, 8 kv heads: 256 equal items (one per compute unit).
    p = params(num_seqs=1, num_q_heads=32, num_kv_heads=8, num_draft_tokens=8, mode="full",
               max_blocks_per_seq=1 << 16, num_blocks=1 << 17)
    items, C = da().plan(p, [1 << 20])
    assert C == 32768 and len(items) == 256 and {_item_keys(it).size for it in items} == {32768}
    assert {it[6] for it in items} == {32}, "each head's 1024 steps dealt to 32 items"
    # FOLD at 256K with a 4096 window: no item exceeds C, at most one per compute unit.
    p = params(num_seqs=1, num_q_heads=32, num_kv_heads=8, num_draft_tokens=6, mode="fold", n_sink=0, window=4096,
               max_blocks_per_seq=1 << 14, num_blocks=1 << 15)
    items, C = da().plan(p, [262144])
    assert len(items) <= 256 and max(_item_keys(it).size for it in items) <= C
    # Ragged batches: the items of a sequence differ by at most one step (plus a
    # partial last block) and none exceeds C.
    lens = [40000, 300000, 123457]
    p = params(num_seqs=3, num_q_heads=16, num_kv_heads=4, num_draft_tokens=2, mode="full",
               max_blocks_per_seq=(300000 + 15) // 16, num_blocks=1 << 20)
    items, C = da().plan(p, lens)
    for b in range(3):
        sizes = [_item_keys(it).size for it in items if it[0] == b and it[1] == 0]
        assert sum(sizes) == lens[b] and max(sizes) - min(sizes) < 64 and max(sizes) <= C


def test_items_deal_a_range_s_steps_round_robin():
    for L in (1, 31, 32, 33, 1000, 4097, 100003):
        for P in (32, 64, 96, 4096):
            p = params(num_seqs=1, mode="full", split_keys=P, max_blocks_per_seq=(L + 15) // 16, num_blocks=1 << 16)
            items, C = da().plan(p, [L])
            head0 = [it for it in items if it[1] == 0]
            nsteps = -(-L // 32)
            want = -(-nsteps // (P // 32))
            assert len(head0) == want
            assert [it[2:] for it in head0] == [(0, L, 0, k, want) for k in range(want)]
            steps = [len(range(k, nsteps, want)) for k in range(want)]
            assert max(steps) - min(steps) <= 1 and max(steps) <= P // 32
            got = np.concatenate([_item_keys(it) for it in head0])
            assert np.array_equal(np.sort(got), np.arange(L))


def test_host_logic_under_sanitizers(tmp_path):
    """host.cpp (validation + planner) built with g++ ASan/UBSan and fuzzed by a small driver."""
    drv = os.path.join(ROOT, "tests", "host_fuzz.cpp")
    src = os.path.join(ROOT, "draft_attention_amd", "csrc", "host.cpp")
    exe = tmp_path / "host_fuzz"
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "include"), drv, src, "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "ok" in res.stdout


# ----------------------------------------------------------------------------- ring buffer
def test_ring_size_and_table_cover_exactly_the_touched_blocks():
    rnd = random.Random(5)
    for _ in range(300):
        W, S, n_new = rnd.choice([0, 1, 16, 100, 256]), rnd.choice([0, 1, 4, 16, 20]), rnd.choice([0, 1, 7, 40])
        sb, rl = da().ring_size(W, S, n_new)
        assert sb == -(-S // 16) and rl == -(-W // 16) + 1 + -(-n_new // 16)
        L = rnd.randint(0, 3000)
        MB = (L + n_new + 15) // 16 + 1
        sinks = [1000 + i for i in range(sb)]
        ring = [2000 + i for i in range(rl)]
        row = da().ring_table(L, n_new, W, S, sinks, ring, MB)
        main, _ = oracle.index_sets(L, "window", W, S)
        touched = set(int(j) // 16 for j in main) | set(p // 16 for p in range(L, L + n_new))
        assert {j for j, x in enumerate(row) if x >= 0} == touched
        phys = [row[j] for j in sorted(touched)]
        assert len(set(phys)) == len(phys), "two touched blocks share a physical block"
        for j in touched:
            assert row[j] == (sinks[j] if j < sb else ring[(j - sb) % rl])
    # rings smaller than the minimum are refused
    sb, rl = da().ring_size(100, 4, 7)
    with pytest.raises(da().DraftAttnError):
        da().ring_table(500, 7, 100, 4, [0] * sb, list(range(rl - 1)), 64)


# ----------------------------------------------------------------------------- launch shape, output type
def test_launch_and_out_dtype_validated():
    for bad in (3, -1):
        p = params()
        p.launch = bad
        assert call(p) == -1
    p = params()
    p.out_dtype = 2
    assert call(p) == -1
    p = params(out_dtype="bf16")
    assert call(p, out=0x70002) == -1                 # bf16 out still needs 8-byte alignment


def _group_counts(items):
    counts = {}
    for (b, h, *_) in items:
        counts[(b, h)] = counts.get((b, h), 0) + 1
    return counts


def test_single_launch_limits_items_per_group():
    # Forced single launch with the library's chunk: the chunk grows until no
    # (sequence, kv head) has more than MAX_GROUP_ITEMS items.
    lens = [1 << 20, 5000]
    p = params(num_seqs=2, num_q_heads=32, num_kv_heads=8, num_draft_tokens=8, mode="full", launch="single",
               max_blocks_per_seq=1 << 16, num_blocks=1 << 17)
    items, C = da().plan(p, lens)
    assert da().launch_of(p, lens) == "single"
    counts = _group_counts(items)
    assert len(counts) == 16 and max(counts.values()) <= da().MAX_GROUP_ITEMS
    # With a fixed chunk that leaves too many items per group, single is refused.
    p = params(num_seqs=2, num_q_heads=32, num_kv_heads=8, num_draft_tokens=8, mode="full", launch="single",
               split_keys=4096, max_blocks_per_seq=1 << 16, num_blocks=1 << 17)
    assert call(p, lens=lens) == -4
    # A forced two-pass launch is always honoured.
    p = params(num_seqs=2, num_q_heads=32, num_kv_heads=8, num_draft_tokens=8, mode="window", window=128,
               n_sink=4, launch="two_pass", max_blocks_per_seq=1 << 16, num_blocks=1 << 17)
    assert da().launch_of(p, lens) == "two_pass"


def test_batch_with_an_empty_sequence_runs_on_two_kernels():
    for launch in ("auto", "single"):
        p = params(launch=launch)
        assert da().launch_of(p, [300, 0]) == "two_pass"
    assert da().launch_of(params(launch="single"), [300, 17]) == "single"


def test_auto_launch_rule():
    # Single launch exactly when the step has more items than resident
    # workgroups (256 compute units times 1 for d = 128, 3 or 2 for d = 64 with
    # one or two row tiles) and the largest group's partial records (items *
    # padded rows * d * 4 bytes) fit in 160 KiB.
    rnd = random.Random(3)
    seen = set()
    for _ in range(200):
        mode = rnd.choice(["full", "window", "fold"])
        lens = [rnd.choice([17, 300, 4096, 40000, 1 << 17]) for _ in range(rnd.randint(1, 24))]
        T = rnd.choice([1, 2, 4, 8])
        d = rnd.choice([64, 128])
        Hkv = rnd.choice([2, 8])
        p = params(num_seqs=len(lens), num_q_heads=4 * Hkv, num_kv_heads=Hkv, num_draft_tokens=T, head_dim=d,
                   mode=mode, window=rnd.choice([16, 256, 2048, 4096]), n_sink=0 if mode == "fold" else 4,
                   max_blocks_per_seq=(max(lens) + 15) // 16, num_blocks=1 << 14)
        items, _ = da().plan(p, lens)
        gmax = max(_group_counts(items).values())
        tiles = (4 * T + 15) // 16
        slots = 256 * (1 if d == 128 else (3 if tiles == 1 else 2))
        cap = 160 * 1024 if len(items) > slots else -1
        want = "single" if gmax <= da().MAX_GROUP_ITEMS and gmax * 16 * tiles * d * 4 <= cap else "two_pass"
        assert da().launch_of(p, lens) == want, (mode, lens, T, d)
        seen.add((want, len(items) > slots))
    assert seen == {("single", True), ("two_pass", True), ("two_pass", False)}, seen


def test_merge_draft_refuses_bf16_output():
    p = params(out_dtype="bf16")
    host = (ctypes.c_int32 * 2)(*LENS)
    st = da().lib.draft_attn_merge_draft(ctypes.byref(p), 0x10000, 0x20000, 0x30000, 0x60000, host, 0x70000,
                                         0x80000, None)
    assert st == -4


def test_merge_draft_refuses_more_query_heads_than_its_grid_spans():
    # one grid dimension of the merge kernel spans the query heads (at most
    # 65535); refused on the host, before anything is enqueued
    host = (ctypes.c_int32 * 2)(*LENS)
    p = params(num_q_heads=65536, num_kv_heads=8192, num_draft_tokens=1)
    st = da().lib.draft_attn_merge_draft(ctypes.byref(p), 0x10000, 0x20000, 0x30000, 0x60000, host, 0x70000,
                                         0x80000, None)
    assert st == -4


def test_fused_decode_draft_validates_the_draft_pointers():
    # Checked on the host before anything is enqueued (no GPU needed): both
    # draft pointers are required and must be 16-byte aligned.
    p = params()
    host = (ctypes.c_int32 * 2)(*LENS)
    f = da().lib.draft_attn_decode_draft
    common = (0x10000, 0x20000, 0x30000, None, 0x40000, 0x50000, host)
    tail = (0x80000, 0x90000, 0x100000, 1, None)   # a 1-byte workspace: ENOSPC once everything else passes
    assert f(ctypes.byref(p), *common, None, None, *tail) == -1
    assert f(ctypes.byref(p), *common, 0x60000, None, *tail) == -1
    assert f(ctypes.byref(p), *common, 0x60008, 0x70000, *tail) == -1
    assert f(ctypes.byref(p), *common, 0x60000, 0x70004, *tail) == -1
    assert f(ctypes.byref(p), *common, 0x60000, 0x70000, *tail) == -2


# ----------------------------------------------------------------------------- binding argument checks
def test_binding_rejects_host_tensors_and_wrong_dtypes():
    # These checks run before any GPU call, so they are safe without a GPU.
    import torch
    q = torch.zeros((1, 2, 4, 64), dtype=torch.bfloat16)
    k = torch.zeros((3, 1, 8, 16, 8), dtype=torch.bfloat16)
    v = torch.zeros((3, 1, 64, 16), dtype=torch.bfloat16)
    table = torch.zeros((1, 3), dtype=torch.int32)
    ctx = torch.tensor([40], dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        da().decode(q, k, v, table, ctx, ctx_lens=[40])
    with pytest.raises(ValueError, match="GPU"):
        da().append(q[:, :, :1], q[:, :, :1], table, ctx, k, v, pos_host=[0])
    with pytest.raises(ValueError, match="GPU"):
        da().merge_draft(q, q[:, :, :1], q[:, :, :1], ctx, torch.zeros((1, 2, 4, 64)), torch.zeros((1, 2, 4)),
                         num_blocks=3, max_blocks_per_seq=3, num_kv_heads=1, ctx_lens=[40])


def test_binding_expect_checks_dtype_shape_and_contiguity():
    import torch
    dev = torch.device("cuda", 0)            # only compared, never used to allocate
    t = torch.zeros((2, 3), dtype=torch.float32)

    class Fake:                               # a CPU tensor that reports a GPU device
        def __init__(self, x):
            self._x = x
        def __getattr__(self, k):
            return getattr(self._x, k)
        device = dev
    da()._expect(Fake(t), "x", torch.float32, (2, None), dev)
    with pytest.raises(ValueError, match="dtype"):
        da()._expect(Fake(t.to(torch.float64)), "x", torch.float32, (2, 3), dev)
    with pytest.raises(ValueError, match="shape"):
        da()._expect(Fake(t), "x", torch.float32, (3, 3), dev)
    with pytest.raises(ValueError, match="contiguous"):
        da()._expect(Fake(t.t()), "x", torch.float32, (3, 2), dev)

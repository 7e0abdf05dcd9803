"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bars: max|d out| <= 1e-2 and max|d lse| <= 1e-3 for bf16 inputs with fp32
accumulation; the set of keys each call scores (the debug visit map) must
equal the oracle's index sets bit for bit. Inputs come from the seeded
generator in ``synth``; unused pool slots are NaN, so any read outside the
visible set poisons the result.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
LSE_TOL = 1e-3


def _da():
    import draft_attention_amd as da  # raises if the library is not built
    return da


def to_dev(x):
    dev = torch.device("cuda:0")
    return {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in x.items()}


def np_inputs(x):
    out = {}
    for k, v in x.items():
        if torch.is_tensor(v):
            v = v.cpu()
            out[k] = v.float().numpy() if v.is_floating_point() else v.numpy()
        else:
            out[k] = v
    return out


def expected_visit(ctx_lens, stride, mode, window=0, n_sink=0, **_):
    m = np.zeros((len(ctx_lens), stride), dtype=np.uint8)
    for b, L in enumerate(ctx_lens):
        main, far = oracle.index_sets(L, mode, window, n_sink)
        m[b, main] = 1
        m[b, far] = 2
    return m


def run_gpu(g, kw, split=0, visit=True, theta=5e5, stream=None, launch="auto"):
    da = _da()
    side = g["k_side"] if kw["mode"] == "fold" else None
    vis = None
    if visit:
        stride = max(max(g["ctx_lens"]), 1)
        vis = torch.zeros((len(g["ctx_lens"]), stride), dtype=torch.uint8, device="cuda:0")
    out, lse = da.decode(g["q"], g["k_cache"], g["v_cache"], g["block_table"], g["ctx_len"], k_side=side,
                         ctx_lens=g["ctx_lens"], rope_theta=theta, split_keys=split, debug_visit=vis,
                         stream=stream, launch=launch, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), (None if vis is None else vis.cpu().numpy())


def compare(out, lse, ref, label, pairs=None, G=None):
    if pairs is not None:
        sel = np.zeros(ref["lse"].shape, dtype=bool)
        for (b, g) in pairs:
            sel[b, :, g * G:(g + 1) * G] = True
        out, lse = out[sel], lse[sel]
        rout, rlse = ref["out"][sel], ref["lse"][sel]
    else:
        rout, rlse = ref["out"], ref["lse"]
    assert np.all(np.isfinite(out)), f"{label}: non-finite output"
    empty = np.isneginf(rlse)
    assert np.array_equal(np.isneginf(lse), empty), f"{label}: empty-set rows differ"
    dout = float(np.abs(out - rout).max()) if out.size else 0.0
    dlse = float(np.abs(lse[~empty] - rlse[~empty]).max()) if (~empty).any() else 0.0
    print(f"{label}: max|dout|={dout:.3e} max|dlse|={dlse:.3e}", flush=True)
    assert dout <= OUT_TOL and dlse <= LSE_TOL, (label, dout, dlse)


def check(x, kw, split=0, theta=5e5, label="", launch="auto"):
    g = to_dev(x)
    out, lse, vis = run_gpu(g, kw, split=split, theta=theta, launch=launch)
    n = np_inputs(x)
    ref = oracle.decode(n["q"], n["k_cache"], n["v_cache"], n["block_table"], x["ctx_lens"],
                        k_side=n["k_side"], rope_theta=theta, **kw)
    compare(out, lse, ref, label or str(kw))
    want = expected_visit(x["ctx_lens"], vis.shape[1], **kw)
    assert np.array_equal(vis, want), f"{label or kw}: visited key set differs from the oracle's"
    return out, lse


# ----------------------------------------------------------------------------- small shapes
def test_tiny_ctx4k_gqa4_d64_full_and_window():
    w = synth.workloads()["tiny_4k_gqa4_d64"]
    x = synth.make_inputs(ctx_lens=w.ctx_lens, T=w.T, Hq=w.Hq, Hkv=w.Hkv, d=w.d, seed=0)
    for kw in w.runs:
        check(x, kw, theta=w.rope_theta, label=f"tiny {kw}")


@pytest.mark.parametrize("launch", ["two_pass", "single"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G,T", [(4, 4), (4, 8), (1, 1), (8, 3), (2, 5)])
def test_full_and_window_shapes(d, G, T, launch):
    Hkv = 2
    x = synth.make_inputs(ctx_lens=[1000, 37, 4097, 16], T=T, Hq=G * Hkv, Hkv=Hkv, d=d, seed=G * 10 + T)
    for kw in (dict(mode="full"), dict(mode="window", window=300, n_sink=4),
               dict(mode="window", window=0, n_sink=7), dict(mode="window", window=2000, n_sink=0)):
        check(x, kw, label=f"d={d} G={G} T={T} {launch} {kw}", launch=launch)


@pytest.mark.parametrize("launch", ["two_pass", "single"])
@pytest.mark.parametrize("rope", ["neox", "none"])
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (2.0, 0.0), (4.0, -1.0), (0.5, 1.5)])
def test_fold_modes(rope, alpha, beta, launch):
    x = synth.make_inputs(ctx_lens=[20000, 700, 4096, 4097, 5], T=6, Hq=16, Hkv=4, d=128, seed=5,
                          fold=True, needle_frac=0.01)
    kw = dict(mode="fold", window=4096, alpha=alpha, beta=beta, rope=rope)
    check(x, kw, label=f"fold {launch} {kw}", launch=launch)


def test_fold_small_window_and_zero_window():
    x = synth.make_inputs(ctx_lens=[3000, 1, 64], T=2, Hq=4, Hkv=2, d=64, seed=8, fold=True)
    for W in (0, 1, 17, 64):
        check(x, dict(mode="fold", window=W, alpha=3.0, beta=-0.5), label=f"fold W={W}")


@pytest.mark.parametrize("launch", ["two_pass", "single"])
def test_query_scaling_batched_ragged(launch):
    # The empty sequence (L = 0) is included once; without it the batch takes
    # the requested launch shape.
    for lens in ([0, 1, 17, 5000, 33333, 4096, 12000], [1, 17, 5000, 33333, 4096, 12000]):
        x = synth.make_inputs(ctx_lens=lens, T=4, Hq=32, Hkv=8, d=128, seed=9, fold=True)
        for kw in (dict(mode="full", kappa=0.1, n0=4096),
                   dict(mode="window", window=1024, n_sink=4, kappa=0.3, n0=256),
                   dict(mode="fold", window=4096, alpha=2.0, beta=0.0, kappa=0.1, n0=4096),
                   dict(mode="full", kappa=-0.05, n0=16)):
            check(x, kw, label=f"ragged {len(lens)} seqs {launch} {kw}", launch=launch)


@pytest.mark.parametrize("split,launch", [(32, "two_pass"), (64, "two_pass"), (96, "two_pass"), (512, "two_pass"),
                                          (4096, "two_pass"), (65536, "two_pass"), (160, "single"), (512, "single"),
                                          (4096, "single"), (65536, "single")])
def test_split_size_sweep(split, launch):
    x = synth.make_inputs(ctx_lens=[9000, 333], T=4, Hq=8, Hkv=2, d=128, seed=12, fold=True)
    for kw in (dict(mode="full"), dict(mode="window", window=1000, n_sink=4),
               dict(mode="fold", window=1000, alpha=2.0, beta=-1.0)):
        check(x, kw, split=split, label=f"split={split} {launch} {kw}", launch=launch)


@pytest.mark.parametrize("d", [64, 128])
def test_every_steps_per_wave_count(d):
    # The streaming loop has a main part (three or more steps left per wave) and
    # a tail of one or two steps; chunks of 128 m keys give each of the four
    # waves exactly m steps (the last, ragged item fewer), for m = 1 .. 7.
    for m in range(1, 8):
        split = 128 * m
        x = synth.make_inputs(ctx_lens=[3 * split + 77, split - 16], T=4, Hq=8, Hkv=2, d=d, seed=60 + m, fold=True)
        for kw in (dict(mode="full"), dict(mode="fold", window=split + 40, alpha=2.0, beta=-1.0)):
            check(x, kw, split=split, label=f"d={d} {m} steps per wave {kw}")


def test_fold_far_logit_precision_at_large_logits():
    # The rotated far query is held as three bf16 terms (its full 24 fp32
    # bits), so far logits, and lse through them, stay at fp32 level even
    # when needle keys with a large alpha and kappa push |lse| to hundreds of
    # nats: the same relative bound holds with and without the rotation.
    # (Two terms keep about 17 bits and miss it by some 8x.)
    x = synth.make_inputs(ctx_lens=[1900, 3000], T=6, Hq=8, Hkv=4, d=64, seed=70, fold=True, needle_frac=0.02)
    n = np_inputs(x)
    g = to_dev(x)
    for rope, rel in (("neox", 2.0 ** -20), ("none", 2.0 ** -20)):
        kw = dict(mode="fold", window=17, alpha=3.0, beta=0.0, kappa=0.3, n0=1, fold_variant="A", rope=rope)
        out, lse, _ = run_gpu(g, kw, visit=False)
        ref = oracle.decode(n["q"], n["k_cache"], n["v_cache"], n["block_table"], x["ctx_lens"],
                            k_side=n["k_side"], rope_theta=5e5, **kw)
        big = float(np.abs(ref["lse"]).max())
        assert big > 100, "the case is meant to have large logits"
        err = np.abs(lse - ref["lse"])
        assert np.all(err <= rel * np.abs(ref["lse"]) + 1e-5), (rope, float(err.max()), big)
        assert float(np.abs(out - ref["out"]).max()) <= 1e-2


def test_needles_full_attention():
    x = synth.make_inputs(ctx_lens=[30000], T=8, Hq=32, Hkv=8, d=128, seed=13, needle_frac=0.01)
    check(x, dict(mode="full"), label="needles full")
    check(x, dict(mode="window", window=4096, n_sink=4), label="needles window")


@pytest.mark.parametrize("launch", ["two_pass", "single"])
def test_batch_above_the_argument_table(launch):
    # Up to 32 sequences travel with the launch arguments; larger batches are
    # located from ctx_len in device memory. 40 ragged sequences, one empty.
    rnd = np.random.default_rng(50)
    lens = [int(v) for v in rnd.integers(1, 3000, size=40)]
    lens[7] = 0
    x = synth.make_inputs(ctx_lens=lens, T=2, Hq=8, Hkv=2, d=64, seed=50, fold=True)
    for kw in (dict(mode="full", kappa=0.1, n0=256), dict(mode="window", window=500, n_sink=4),
               dict(mode="fold", window=700, alpha=2.0, beta=-1.0)):
        check(x, kw, label=f"40 seqs {launch} {kw}", launch=launch)
    x = synth.make_inputs(ctx_lens=[v if v else 5 for v in lens], T=2, Hq=8, Hkv=2, d=64, seed=51)
    check(x, dict(mode="window", window=300, n_sink=4), label=f"40 seqs, none empty, {launch}", launch=launch)


def test_device_lengths_that_disagree_are_reported():
    # Batches above 32 sequences read ctx_len from device memory. When it holds
    # fewer work items than the host lengths the call was planned from, the
    # kernels leave neutral records for the missing items (no access goes out of
    # bounds) and set DRAFT_ATTN_STATUS_LENGTHS; with matching lengths the word
    # stays zero.
    da = _da()
    dev = torch.device("cuda:0")
    lens = [300 + 7 * i for i in range(39)] + [20000]
    x = synth.make_inputs(ctx_lens=lens, T=2, Hq=8, Hkv=2, d=64, seed=52)
    g = to_dev(x)
    p = da.make_params(num_seqs=40, num_draft_tokens=2, num_q_heads=8, num_kv_heads=2, head_dim=64,
                       num_blocks=x["k_cache"].shape[0], max_blocks_per_seq=x["block_table"].shape[1])
    items, _ = da.plan(p, lens)
    assert sum(1 for it in items if it[0] == 39) > 2, "the last sequence must span several items"
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    _decode(g, dict(mode="full"), status=status)
    assert int(status.item()) == 0
    short = g["ctx_len"].clone()
    short[39] = 16
    da.decode(g["q"], g["k_cache"], g["v_cache"], g["block_table"], short, ctx_lens=lens, status=status,
              rope_theta=5e5, mode="full")
    torch.cuda.synchronize()
    assert int(status.item()) == da.STATUS_LENGTHS


# ----------------------------------------------------------------------------- paging behaviour
def test_unread_blocks_may_be_invalid():
    # Blocks wholly outside the window are never read: give them -1 table entries.
    L, W, S = 5000, 700, 4
    x = synth.make_inputs(ctx_lens=[L], T=2, Hq=8, Hkv=2, d=128, seed=14)
    kw = dict(mode="window", window=W, n_sink=S)
    base, _ = check(x, kw)
    t = x["block_table"].clone()
    keep = set(range((S + 15) // 16)) | set(range((L - W) // 16, (L + 15) // 16))
    for j in range(t.shape[1]):
        if j not in keep:
            t[0, j] = -1
    y = dict(x, block_table=t)
    out, _ = check(y, kw)
    assert np.array_equal(out, base)


def _repage(n, table, keep, Hkv, d):
    """Host pools holding exactly the kept logical keys of each sequence, in
    order, in fresh blocks: (k_cache, v_cache, k_side, block_table, lengths)."""
    nblk = [(len(kk) + 15) // 16 for kk in keep]
    NB, MB = max(sum(nblk), 1), max(max(nblk), 1)
    k = np.full((NB, Hkv, d // 8, 16, 8), np.nan)
    ks = np.full((NB, Hkv, d // 8, 16, 8), np.nan)
    v = np.full((NB, Hkv, d, 16), np.nan)
    t = np.full((len(keep), MB), -1, dtype=np.int64)
    nb = 0
    for b, kk in enumerate(keep):
        for i, j in enumerate(kk):
            if i % 16 == 0:
                t[b, i // 16] = nb
                nb += 1
            sb, ss, db, ds = table[b, j // 16], j % 16, t[b, i // 16], i % 16
            k[db, :, :, ds, :] = n["k_cache"][sb, :, :, ss, :]
            ks[db, :, :, ds, :] = n["k_side"][sb, :, :, ss, :]
            v[db, :, :, ds] = n["v_cache"][sb, :, :, ss]
    return k, v, ks, t, [len(kk) for kk in keep]


@pytest.mark.parametrize("launch", ["two_pass", "single"])
def test_table_entries_outside_the_pool_are_masked_and_reported(launch):
    # The pools hold three more blocks than the num_blocks passed, all NaN. A
    # table entry that is read and names one of them, or is -1, must be masked
    # (a broken mask shows up as NaN, and no access leaves the allocation) and
    # must set DRAFT_ATTN_STATUS_BAD_BLOCK. Reference: the oracle over a cache
    # re-paged with exactly the keys that remain (kappa = 0, so the visible
    # count does not enter; FOLD without rotation, so the shared position does
    # not either).
    da = _da()
    dev = torch.device("cuda:0")
    lens, Hkv, d = [3000, 700], 2, 128
    x = synth.make_inputs(ctx_lens=lens, T=4, Hq=8, Hkv=Hkv, d=d, seed=30, fold=True)
    NB = x["k_cache"].shape[0]

    def widen(t):
        return torch.cat([t, torch.full((3,) + tuple(t.shape[1:]), float("nan"), dtype=t.dtype)])

    g = to_dev(dict(x, k_cache=widen(x["k_cache"]), v_cache=widen(x["v_cache"]), k_side=widen(x["k_side"])))
    n = np_inputs(x)
    cases = [  # (mode arguments, {(sequence, logical block): bad entry})
        (dict(mode="full"), {(0, 10): NB, (0, 100): NB + 2, (1, 5): -1, (1, 43): NB + 1}),
        (dict(mode="window", window=1000, n_sink=20), {(0, 1): NB + 1, (0, 150): NB, (1, 3): -1}),
        (dict(mode="fold", window=512, alpha=2.0, beta=-1.0, rope="none"), {(0, 20): NB, (1, 2): NB + 1}),
    ]
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    for kw, bad in cases:
        # a clean call leaves the word at zero
        out0, _ = da.decode(g["q"], g["k_cache"], g["v_cache"], g["block_table"], g["ctx_len"],
                            k_side=g["k_side"] if kw["mode"] == "fold" else None, ctx_lens=lens, num_blocks=NB,
                            status=status, launch=launch, **kw)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, kw
        t = x["block_table"].clone()
        for (b, j), e in bad.items():
            t[b, j] = e
        vis = torch.zeros((2, max(lens)), dtype=torch.uint8, device=dev)
        out, lse = da.decode(g["q"], g["k_cache"], g["v_cache"], t.to(dev), g["ctx_len"],
                             k_side=g["k_side"] if kw["mode"] == "fold" else None, ctx_lens=lens, num_blocks=NB,
                             status=status, debug_visit=vis, launch=launch, **kw)
        torch.cuda.synchronize()
        assert int(status.item()) == da.STATUS_BAD_BLOCK, (kw, int(status.item()))
        status.zero_()
        keep, want = [], expected_visit(lens, max(lens), **kw)
        for b, L in enumerate(lens):
            main, far = oracle.index_sets(L, kw["mode"], kw.get("window", 0), kw.get("n_sink", 0))
            masked = {j for (bb, j) in bad if bb == b}
            keys = [int(j) for j in np.concatenate([far, main]) if j // 16 not in masked]
            keep.append(keys)
            for j in masked:
                want[b, 16 * j:16 * j + 16] = 0
        assert np.array_equal(vis.cpu().numpy(), want), f"{kw}: masked keys were scored"
        k, v, ks, t2, l2 = _repage(n, x["block_table"].numpy(), keep, Hkv, d)
        if kw["mode"] == "fold":
            assert all(len(kk) > kw["window"] for kk in keep)   # the local window is unchanged
            ref = oracle.decode(n["q"], k, v, t2, l2, k_side=ks, **kw)
        else:
            ref = oracle.decode(n["q"], k, v, t2, l2, "full")
        compare(out.cpu().numpy(), lse.cpu().numpy(), ref, f"bad entries {launch} {kw}")


def _relabel_blocks(x, perm):
    """The same cache with physical block perm[i] moved to position i."""
    inv = torch.argsort(perm)
    t = x["block_table"]
    t2 = torch.where(t >= 0, inv[t.clamp(min=0).long()].to(torch.int32), t)
    return dict(x, k_cache=x["k_cache"][perm], v_cache=x["v_cache"][perm], k_side=x["k_side"][perm],
                block_table=t2)


def test_block_shuffle_gives_identical_results():
    x = synth.make_inputs(ctx_lens=[3000, 50], T=4, Hq=8, Hkv=2, d=128, seed=15, fold=True)
    NB = x["k_cache"].shape[0]
    y = _relabel_blocks(x, torch.randperm(NB, generator=torch.Generator().manual_seed(1)))
    for kw in (dict(mode="full"), dict(mode="fold", window=512, alpha=2.0, beta=-1.0)):
        a, la = check(x, kw)
        b, lb = check(y, kw)
        assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_in_order_block_table_gives_identical_results():
    # Blocks allocated in table order (sequence by sequence) against a shuffled
    # pool, with a split that gives each range many work items, so that the
    # round-robin dealing of steps crosses many block boundaries.
    x = synth.make_inputs(ctx_lens=[20000, 1500, 77], T=4, Hq=8, Hkv=2, d=128, seed=16, fold=True)
    NB = x["k_cache"].shape[0]
    used = [int(i) for i in x["block_table"].flatten().tolist() if i >= 0]
    assert len(set(used)) == len(used)
    rest = sorted(set(range(NB)) - set(used))
    y = _relabel_blocks(x, torch.tensor(used + rest))
    t = y["block_table"]
    assert all(int(t[0, j]) == j for j in range((20000 + 15) // 16)), "table not in order"
    for split in (0, 1024):
        for kw in (dict(mode="full"), dict(mode="window", window=3000, n_sink=20),
                   dict(mode="fold", window=1000, alpha=4.0, beta=-1.0)):
            a, la = check(x, kw, split=split, label=f"shuffled {kw} split={split}")
            b, lb = check(y, kw, split=split, label=f"in order {kw} split={split}")
            assert np.array_equal(a, b) and np.array_equal(la, lb), f"{kw} split={split}"


def _permute_sequences(x, perm):
    y = dict(x)
    y["q"] = x["q"][perm]
    y["block_table"] = x["block_table"][perm]
    y["ctx_len"] = x["ctx_len"][perm]
    y["ctx_lens"] = [x["ctx_lens"][i] for i in perm]
    return y


@pytest.mark.parametrize("lens,perm,launch", [
    ([3000, 1234, 517, 0, 64], [2, 0, 4, 1, 3], "two_pass"),
    ([3000, 1234, 517, 0, 64], [2, 0, 4, 1, 3], "single"),
    ([300 + 37 * i for i in range(40)], list(range(39, -1, -1)), "two_pass"),
], ids=["5seq-two_pass", "5seq-single", "40seq-two_pass"])
def test_sequence_position_does_not_change_its_result(lens, perm, launch):
    # The first sequence's workgroups start from preloaded kernel arguments, the
    # others from the argument block, and beyond 32 sequences every workgroup
    # finds its sequence from ctx_len on the device: a sequence's result is the
    # same bits whatever its position in the batch.
    x = synth.make_inputs(ctx_lens=lens, T=4, Hq=8, Hkv=2, d=128, seed=19, fold=True)
    y = _permute_sequences(x, perm)
    for kw in (dict(mode="full"), dict(mode="window", window=700, n_sink=4),
               dict(mode="fold", window=900, alpha=2.0, beta=-1.0)):
        a = run_gpu(to_dev(x), kw, launch=launch)
        b = run_gpu(to_dev(y), kw, launch=launch)
        assert np.array_equal(a[0][perm], b[0]) and np.array_equal(a[1][perm], b[1]), (kw, launch)
        assert np.array_equal(a[2][perm], b[2]), (kw, launch)


def test_deterministic_and_stream_safe():
    da = _da()
    x = synth.make_inputs(ctx_lens=[8000, 900], T=4, Hq=16, Hkv=4, d=128, seed=16, fold=True)
    g = to_dev(x)
    kw = dict(mode="fold", window=1024, alpha=2.0, beta=-1.0)
    a = run_gpu(g, kw)
    b = run_gpu(g, kw)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for s, kw2 in ((s1, kw), (s2, dict(mode="full"))):
        with torch.cuda.stream(s):
            side = g["k_side"] if kw2["mode"] == "fold" else None
            outs.append(da.decode(g["q"], g["k_cache"], g["v_cache"], g["block_table"], g["ctx_len"],
                                  k_side=side, ctx_lens=g["ctx_lens"], rope_theta=5e5, **kw2))
    torch.cuda.synchronize()
    c = run_gpu(g, dict(mode="full"))
    assert np.array_equal(outs[0][0].cpu().numpy(), a[0])
    assert np.array_equal(outs[1][0].cpu().numpy(), c[0])


def test_empty_batch_and_all_empty_sequences():
    da = _da()
    x = synth.make_inputs(ctx_lens=[0, 0], T=1, Hq=2, Hkv=1, d=64, seed=17)
    g = to_dev(x)
    out, lse = da.decode(g["q"], g["k_cache"], g["v_cache"], g["block_table"], g["ctx_len"], ctx_lens=[0, 0])
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


# ----------------------------------------------------------------------------- full-size workloads
def _full_size_inputs(w, seed=0):
    dev = torch.device("cuda:0")
    return synth.make_inputs(ctx_lens=w.ctx_lens, T=w.T, Hq=w.Hq, Hkv=w.Hkv, d=w.d, seed=seed, device=dev,
                             fold=w.fold, needle_frac=w.needle_frac)


def _head_subcache(w, kw, x, g, bsel):
    """fp32 host copies of just kv head g's blocks that hold visible keys of the
    sequences bsel, with their table rows renumbered to the copy."""
    G = w.Hq // w.Hkv
    table = x["block_table"].cpu()
    rows = table[bsel].clone()
    for i, b in enumerate(bsel):
        main, far = oracle.index_sets(w.ctx_lens[b], kw["mode"], kw.get("window", 0), kw.get("n_sink", 0))
        read = np.zeros(rows.shape[1], dtype=bool)
        read[np.concatenate([main, far]) // 16] = True
        rows[i, torch.from_numpy(~read)] = -1
    used = torch.unique(rows[rows >= 0])
    remap = torch.full((int(table.max()) + 1,), -1, dtype=torch.int64)
    remap[used.long()] = torch.arange(used.numel())
    sub_table = np.where(rows.numpy() >= 0, remap[rows.clamp(min=0).long()].numpy(), -1)
    idx = used.long().to(x["k_cache"].device)
    sub = dict(q=x["q"][bsel][:, :, g * G:(g + 1) * G].float().cpu().numpy(),
               k=x["k_cache"][idx, g:g + 1].float().cpu().numpy(),
               v=x["v_cache"][idx, g:g + 1].float().cpu().numpy(),
               ks=None if x["k_side"] is None else x["k_side"][idx, g:g + 1].float().cpu().numpy())
    return sub, sub_table


def _sampled(w, kw, pairs, x=None, seed=0):
    """Full-size inputs generated on the GPU (or given); the GPU call runs in the
    launch configuration the bench times, on every sequence and head; the oracle
    runs in full on the sampled (seq, kv head) pairs."""
    if x is None:
        x = _full_size_inputs(w, seed)
    out, lse, vis = run_gpu(x, kw, visit=True, theta=w.rope_theta)
    want = expected_visit(w.ctx_lens, vis.shape[1], **kw)
    assert np.array_equal(vis, want)
    heads = sorted({g for _, g in pairs})
    G = w.Hq // w.Hkv
    for g in heads:
        bsel = sorted({b for b, gg in pairs if gg == g})
        sub, sub_table = _head_subcache(w, kw, x, g, bsel)
        ref = oracle.decode(sub["q"], sub["k"], sub["v"], sub_table, [w.ctx_lens[b] for b in bsel],
                            k_side=sub["ks"], rope_theta=w.rope_theta, **kw)
        o = out[:, :, g * G:(g + 1) * G][bsel]
        ls = lse[:, :, g * G:(g + 1) * G][bsel]
        compare(o, ls, ref, f"{w.name} {kw} kv={g} seqs={bsel}")
        del sub


def test_full_size_llama8b_128k():
    w = synth.workloads()["llama8b_128k"]
    x = _full_size_inputs(w)
    for kw in w.runs:
        _sampled(w, kw, pairs=[(0, g) for g in range(w.Hkv)], x=x)


def test_full_size_needles_1m():
    w = synth.workloads()["needles_1m"]
    x = _full_size_inputs(w)
    for kw in w.runs:
        _sampled(w, kw, pairs=[(0, g) for g in range(w.Hkv)], x=x)


@pytest.mark.parametrize("name,run", [("llama8b_128k", 1), ("needles_1m", 1), ("fold_256k", 3)])
def test_full_size_fused_draft_step(name, run):
    # a step of the workload with the step's draft keys, as one fused call (the
    # window steps are the shape bench.py's draft-step entries time; FOLD at
    # alpha = 2, beta = -1): every kv head against the oracle's single softmax
    # over the step's keys and draft keys 0..t, and the fused result equal to
    # decode + merge_draft bit for bit
    da = _da()
    w = synth.workloads()[name]
    kw = w.runs[run]
    x = _full_size_inputs(w)
    side = x["k_side"] if kw["mode"] == "fold" else None
    B = len(w.ctx_lens)
    gen = torch.Generator(device="cuda:0").manual_seed(91)
    kd = (torch.randn((B, w.T, w.Hkv, w.d), generator=gen, device="cuda:0") * 2).to(torch.bfloat16)
    vd = torch.randn((B, w.T, w.Hkv, w.d), generator=gen, device="cuda:0").to(torch.bfloat16)
    fo, fl = da.decode(x["q"], x["k_cache"], x["v_cache"], x["block_table"], x["ctx_len"], ctx_lens=x["ctx_lens"],
                       k_side=side, rope_theta=w.rope_theta, k_draft=kd, v_draft=vd, **kw)
    o2, l2 = da.decode(x["q"], x["k_cache"], x["v_cache"], x["block_table"], x["ctx_len"], ctx_lens=x["ctx_lens"],
                       k_side=side, rope_theta=w.rope_theta, launch="two_pass", **kw)
    da.merge_draft(x["q"], kd, vd, x["ctx_len"], o2, l2, num_blocks=x["k_cache"].shape[0],
                   max_blocks_per_seq=x["block_table"].shape[1], num_kv_heads=w.Hkv, ctx_lens=x["ctx_lens"],
                   rope_theta=w.rope_theta, **kw)
    torch.cuda.synchronize()
    assert torch.equal(fo, o2) and torch.equal(fl, l2)
    out, lse = fo.cpu().numpy(), fl.cpu().numpy()
    G = w.Hq // w.Hkv
    bsel = list(range(B))
    for g in range(w.Hkv):
        sub, sub_table = _head_subcache(w, kw, x, g, bsel)
        ref = oracle.decode_with_draft(sub["q"], sub["k"], sub["v"], sub_table, w.ctx_lens, kw["mode"],
                                       kd[:, :, g:g + 1].float().cpu().numpy(), vd[:, :, g:g + 1].float().cpu().numpy(),
                                       k_side=sub["ks"], rope_theta=w.rope_theta,
                                       **{k: v for k, v in kw.items() if k != "mode"})
        compare(out[:, :, g * G:(g + 1) * G], lse[:, :, g * G:(g + 1) * G], ref, f"{name} fused {kw} kv={g}")


def test_full_size_fold_256k():
    # every alpha/beta pair of the workload, each on two kv heads; over the six
    # pairs every kv head is checked
    w = synth.workloads()["fold_256k"]
    x = _full_size_inputs(w)
    for i, kw in enumerate(w.runs):
        _sampled(w, kw, pairs=[(0, (2 * i) % w.Hkv), (0, (2 * i + 5) % w.Hkv)], x=x)


def test_full_size_batch16_ragged():
    # every sequence of the batch, each on one kv head (two sequences per head)
    w = synth.workloads()["batch16_ragged"]
    x = _full_size_inputs(w)
    for kw in w.runs:
        _sampled(w, kw, pairs=[(b, b % w.Hkv) for b in range(len(w.ctx_lens))], x=x)


@pytest.mark.parametrize("launch,fused", [("two_pass", False), ("single", False), ("auto", True)])
def test_graph_replay_matches_eager(launch, fused):
    # The call captured in a HIP graph, replayed several times with eager work in
    # between; every replay must equal the eager result bit for bit. A
    # workspace filled with garbage before a replay must not matter.
    da = _da()
    x = synth.make_inputs(ctx_lens=[7000, 333], T=4, Hq=16, Hkv=4, d=128, seed=21, fold=True)
    g = to_dev(x)
    kw = dict(mode="fold", window=1024, alpha=2.0, beta=-1.0, kappa=0.1, n0=256)
    out = torch.empty((2, 4, 16, 128), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((2, 4, 16), dtype=torch.float32, device="cuda:0")
    p = da.make_params(num_seqs=2, num_draft_tokens=4, num_q_heads=16, num_kv_heads=4, head_dim=128,
                       num_blocks=g["k_cache"].shape[0], max_blocks_per_seq=g["block_table"].shape[1], **kw)
    ws = torch.empty(da.workspace_size(p, g["ctx_lens"]), dtype=torch.uint8, device="cuda:0")
    # fused: the call with the step's draft keys (draft_attn_decode_draft)
    gen = torch.Generator(device="cuda:0").manual_seed(22)
    kd = torch.randn((2, 4, 4, 128), generator=gen, device="cuda:0").to(torch.bfloat16) if fused else None
    vd = torch.randn((2, 4, 4, 128), generator=gen, device="cuda:0").to(torch.bfloat16) if fused else None

    def call():
        da.decode(g["q"], g["k_cache"], g["v_cache"], g["block_table"], g["ctx_len"], k_side=g["k_side"],
                  ctx_lens=g["ctx_lens"], out=out, lse=lse, workspace=ws, rope_theta=5e5, launch=launch,
                  k_draft=kd, v_draft=vd, **kw)

    call()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for i in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(0xAB)                      # the workspace's contents on entry must not matter
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"replay {i}"
        eager = (g["q"].float() * 2).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(eager)


@pytest.mark.parametrize("variant", ["A", "B'"])
def test_fold_parameterisations(variant):
    # The joint-softmax and virtual-key readings of FOLD's alpha/beta (fold_variant).
    x = synth.make_inputs(ctx_lens=[20000, 700, 4097, 5], T=6, Hq=16, Hkv=4, d=128, seed=25, fold=True,
                          needle_frac=0.01)
    g = to_dev(x)
    n = np_inputs(x)
    for alpha, beta, rope in ((1.0, 0.0, "neox"), (2.0, -1.0, "neox"), (4.0, 0.5, "none"), (0.5, 1.0, "neox")):
        kw = dict(mode="fold", window=4096, alpha=alpha, beta=beta, rope=rope)
        out, lse = _da().decode(g["q"], g["k_cache"], g["v_cache"], g["block_table"], g["ctx_len"], k_side=g["k_side"],
                                ctx_lens=g["ctx_lens"], rope_theta=5e5, fold_variant=variant, **kw)
        torch.cuda.synchronize()
        ref = oracle.decode(n["q"], n["k_cache"], n["v_cache"], n["block_table"], x["ctx_lens"], k_side=n["k_side"],
                            rope_theta=5e5, fold_variant=variant, **kw)
        compare(out.cpu().numpy(), lse.cpu().numpy(), ref, f"fold variant {variant} {kw}")


# ----------------------------------------------------------------------------- single launch, bf16 output
def _decode(g, kw, **extra):
    da = _da()
    side = g["k_side"] if kw["mode"] == "fold" else None
    out, lse = da.decode(g["q"], g["k_cache"], g["v_cache"], g["block_table"], g["ctx_len"], k_side=side,
                         ctx_lens=g["ctx_lens"], rope_theta=5e5, **kw, **extra)
    torch.cuda.synchronize()
    return out, lse


def test_single_launch_reuses_one_workspace_across_shapes():
    # Calls of different shapes share one workspace, first filled with garbage.
    # Each must match the oracle, and each leaves its done flags at zero.
    da = _da()
    ws = torch.full((64 << 20,), 0x5C, dtype=torch.uint8, device="cuda:0")
    cases = [([3000, 700, 41], 4, 16, 4, 128, dict(mode="window", window=512, n_sink=4)),
             ([9000], 8, 32, 8, 128, dict(mode="full")),
             ([5000, 12], 2, 8, 2, 64, dict(mode="fold", window=1000, alpha=2.0, beta=-0.5)),
             ([3000, 700, 41], 4, 16, 4, 128, dict(mode="window", window=512, n_sink=4))]
    for i, (lens, T, Hq, Hkv, d, kw) in enumerate(cases):
        x = synth.make_inputs(ctx_lens=lens, T=T, Hq=Hq, Hkv=Hkv, d=d, seed=40 + i, fold=kw["mode"] == "fold")
        g = to_dev(x)
        out, lse = _decode(g, kw, workspace=ws, launch="single")
        n = np_inputs(x)
        ref = oracle.decode(n["q"], n["k_cache"], n["v_cache"], n["block_table"], x["ctx_lens"],
                            k_side=n["k_side"], rope_theta=5e5, **kw)
        compare(out.cpu().numpy(), lse.cpu().numpy(), ref, f"shared workspace call {i} {kw}")
        p = da.make_params(num_seqs=len(lens), num_draft_tokens=T, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                           num_blocks=x["k_cache"].shape[0], max_blocks_per_seq=x["block_table"].shape[1],
                           launch="single", **kw)
        assert da.launch_of(p, lens) == "single"
        n_items = len(da.plan(p, lens)[0])
        flags = ws[:8 * n_items].cpu()
        assert int(flags.count_nonzero()) == 0, f"call {i} left a done flag set"


@pytest.mark.parametrize("d", [64, 128])
def test_single_launch_at_the_group_item_limit(d):
    # 64 items per (sequence, kv head), the most one workgroup merges, and a
    # chunk the library raises itself to reach the limit.
    da = _da()
    x = synth.make_inputs(ctx_lens=[8192, 8000, 100], T=8, Hq=8, Hkv=2, d=d, seed=44, fold=True)
    items, C = da.plan(da.make_params(num_seqs=3, num_draft_tokens=8, num_q_heads=8, num_kv_heads=2, head_dim=d,
                                      num_blocks=x["k_cache"].shape[0], max_blocks_per_seq=x["block_table"].shape[1],
                                      split_keys=128, launch="single"), x["ctx_lens"])
    assert sum(1 for it in items if it[0] == 0 and it[1] == 0) == da.MAX_GROUP_ITEMS
    for kw in (dict(mode="full"), dict(mode="fold", window=2048, alpha=3.0, beta=0.5)):
        check(x, kw, split=128, label=f"64 items d={d} {kw}", launch="single")
    x = synth.make_inputs(ctx_lens=[40000, 3], T=2, Hq=8, Hkv=2, d=d, seed=45)
    check(x, dict(mode="full"), split=0, label=f"raised chunk d={d}", launch="single")


@pytest.mark.parametrize("launch", ["two_pass", "single"])
def test_bf16_output(launch):
    # bf16 output is the fp32 result of the same path rounded to nearest even,
    # bit for bit; against the oracle the bar widens by bf16's half ulp.
    x = synth.make_inputs(ctx_lens=[5000, 300, 17], T=4, Hq=16, Hkv=4, d=128, seed=46, fold=True,
                          needle_frac=0.01)
    g = to_dev(x)
    n = np_inputs(x)
    for kw in (dict(mode="full"), dict(mode="window", window=1000, n_sink=4),
               dict(mode="fold", window=1000, alpha=2.0, beta=-1.0)):
        o32, l32 = _decode(g, kw, launch=launch)
        o16, l16 = _decode(g, kw, launch=launch, out_dtype="bf16")
        assert o16.dtype == torch.bfloat16
        assert torch.equal(o16, o32.to(torch.bfloat16)), f"{kw}: not the rounded fp32 result"
        assert torch.equal(l16, l32)
        ref = oracle.decode(n["q"], n["k_cache"], n["v_cache"], n["block_table"], x["ctx_lens"],
                            k_side=n["k_side"], rope_theta=5e5, **kw)
        err = np.abs(o16.float().cpu().numpy() - ref["out"])
        bound = OUT_TOL + 2.0 ** -8 * np.abs(ref["out"])
        print(f"bf16 {launch} {kw}: max excess {float((err - bound).max()):.3e}", flush=True)
        assert np.all(err <= bound), kw


def test_single_and_two_pass_agree_on_the_benchmark_shapes():
    # Same inputs through both launch shapes at benchmark-like head counts.
    x = synth.make_inputs(ctx_lens=[20000], T=4, Hq=32, Hkv=8, d=128, seed=47, fold=True)
    g = to_dev(x)
    for kw in (dict(mode="window", window=2048, n_sink=4), dict(mode="full"),
               dict(mode="fold", window=4096, alpha=2.0, beta=-1.0, kappa=0.1, n0=4096)):
        o1, l1 = _decode(g, kw, launch="two_pass")
        o2, l2 = _decode(g, kw, launch="single")
        dout = float((o1 - o2).abs().max())
        dlse = float((l1 - l2).abs().max())
        print(f"single vs two-pass {kw}: max|dout|={dout:.2e} max|dlse|={dlse:.2e}", flush=True)
        assert dout <= 1e-4 and dlse <= 1e-5


def test_plan_log_on_request(tmp_path):
    # DRAFT_ATTN_LOG=1 is read once per process, so the call runs in a short child process.
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import torch, draft_attention_amd as da, synth\n"
            "x = synth.make_inputs(ctx_lens=[3000, 40], T=2, Hq=8, Hkv=2, d=128, seed=1, device='cuda')\n"
            "da.decode(x['q'], x['k_cache'], x['v_cache'], x['block_table'], x['ctx_len'], ctx_lens=[3000, 40],\n"
            "          mode='window', window=512, n_sink=4)\n"
            "torch.cuda.synchronize()\n")
    env = dict(os.environ, DRAFT_ATTN_LOG="1")
    res = subprocess.run([sys.executable, "-c", code], env=env, cwd=root, capture_output=True, text=True, timeout=180)
    assert res.returncode == 0, res.stderr[-2000:]
    line = [ln for ln in res.stderr.splitlines() if ln.startswith("draft_attn_decode:")]
    assert len(line) == 1 and "B=2 T=2 Hq=8 Hkv=2 d=128 mode=window W=512 sinks=4" in line[0], res.stderr[-2000:]
    assert "launch=" in line[0] and "items=" in line[0]

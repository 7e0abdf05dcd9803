"""GPU parity of the KV append (draft_attn_append) against the oracle.

The bar is bit equality of all three pools: the side cache and the values are
copies, and the rotated key is the correctly rounded bf16 value of the fp64
rotation on both sides. Pool slots the append must not touch hold NaN, so any
stray write shows up.
"""

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def _da():
    import draft_attention_amd as da
    return da


def _np(t):
    return None if t is None else t.detach().cpu().double().numpy()


def _pools_equal(a, b):
    return np.array_equal(a, b, equal_nan=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("rope,side", [("neox", True), ("none", True), ("neox", False)])
def test_append_matches_oracle_bit_for_bit(d, rope, side):
    da = _da()
    dev = torch.device("cuda:0")
    lens = [40, 3, 200]                      # existing lengths: appends start mid-block and at block 0
    n_new, Hkv = 11, 4
    x = synth.make_inputs(ctx_lens=[L + n_new for L in lens], T=1, Hq=Hkv, Hkv=Hkv, d=d, seed=31, fold=True)
    g = torch.Generator().manual_seed(5)
    kn = (torch.randn((3, n_new, Hkv, d), generator=g) * 3).to(torch.bfloat16)
    vn = torch.randn((3, n_new, Hkv, d), generator=g).to(torch.bfloat16)
    kc, vc, ks = x["k_cache"].to(dev), x["v_cache"].to(dev), x["k_side"].to(dev)
    pos = torch.tensor(lens, dtype=torch.int32, device=dev)
    da.append(kn.to(dev), vn.to(dev), x["block_table"].to(dev), pos, kc, vc, ks if side else None, rope=rope,
              rope_theta=5e5, pos_host=lens)
    torch.cuda.synchronize()
    rk, rv, rs = oracle.append(_np(kn), _np(vn), x["block_table"].numpy(), lens, _np(x["k_cache"]),
                               _np(x["v_cache"]), _np(x["k_side"]) if side else None, rope=rope, rope_theta=5e5)
    assert _pools_equal(_np(kc), rk)
    assert _pools_equal(_np(vc), rv)
    if side:
        assert _pools_equal(_np(ks), rs)
    else:
        assert _pools_equal(_np(ks), _np(x["k_side"]))


def test_append_far_positions_and_unallocated_blocks():
    # Positions near 2^20 (angles up to ~1e6 rad), and a token whose block is not
    # allocated (-1 table entry): nothing is written for it.
    da = _da()
    dev = torch.device("cuda:0")
    d, Hkv, n_new = 128, 2, 20
    MB = 65536
    start = (1 << 20) - 37
    blocks = list(range(start // 16, (start + n_new - 1) // 16 + 1))
    NB = len(blocks) + 1
    table = torch.full((1, MB), -1, dtype=torch.int32)
    for i, j in enumerate(blocks[:-1]):                     # the last block stays unallocated
        table[0, j] = i
    kc = torch.full((NB, Hkv, d // 8, 16, 8), float("nan"), dtype=torch.bfloat16)
    vc = torch.full((NB, Hkv, d, 16), float("nan"), dtype=torch.bfloat16)
    ks = kc.clone()
    g = torch.Generator().manual_seed(6)
    kn = torch.randn((1, n_new, Hkv, d), generator=g).to(torch.bfloat16)
    vn = torch.randn((1, n_new, Hkv, d), generator=g).to(torch.bfloat16)
    gk, gv, gs = kc.to(dev), vc.to(dev), ks.to(dev)
    da.append(kn.to(dev), vn.to(dev), table.to(dev), torch.tensor([start], dtype=torch.int32, device=dev),
              gk, gv, gs, rope="neox", rope_theta=5e5, pos_host=[start])
    torch.cuda.synchronize()
    keep = [i for i in range(n_new) if (start + i) // 16 != blocks[-1]]
    rk, rv, rs = oracle.append(_np(kn)[:, keep], _np(vn)[:, keep], np.where(table.numpy() < 0, 0, table.numpy()),
                               [start], _np(kc), _np(vc), _np(ks), rope="neox", rope_theta=5e5)
    assert len(keep) < n_new
    assert _pools_equal(_np(gk), rk) and _pools_equal(_np(gv), rv) and _pools_equal(_np(gs), rs)


def test_append_entries_outside_the_pool_are_skipped_and_reported():
    # The pools hold two more blocks than the num_blocks passed, all NaN, and
    # one new token's block entry names one of them: that block's tokens are not
    # written (the extra blocks stay NaN), the rest are written as the oracle
    # writes them, and DRAFT_ATTN_STATUS_APPEND_BAD_BLOCK is set.
    da = _da()
    dev = torch.device("cuda:0")
    d, Hkv, n_new = 128, 2, 20
    lens = [40, 90]
    x = synth.make_inputs(ctx_lens=[L + n_new for L in lens], T=1, Hq=Hkv, Hkv=Hkv, d=d, seed=33, fold=True)
    NB = x["k_cache"].shape[0]

    def widen(t):
        return torch.cat([t, torch.full((2,) + tuple(t.shape[1:]), float("nan"), dtype=t.dtype)])

    kc, vc, ks = (widen(x[k]).to(dev) for k in ("k_cache", "v_cache", "k_side"))
    before = [_np(t) for t in (kc, vc, ks)]
    table = x["block_table"].clone()
    bad_blk = (lens[1] + n_new - 1) // 16          # sequence 1's last touched block
    table[1, bad_blk] = NB + 1
    g = torch.Generator().manual_seed(8)
    kn = torch.randn((2, n_new, Hkv, d), generator=g).to(torch.bfloat16)
    vn = torch.randn((2, n_new, Hkv, d), generator=g).to(torch.bfloat16)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    da.append(kn.to(dev), vn.to(dev), table.to(dev), torch.tensor(lens, dtype=torch.int32, device=dev), kc, vc, ks,
              rope="neox", rope_theta=5e5, pos_host=lens, num_blocks=NB, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == da.STATUS_APPEND_BAD_BLOCK
    # oracle: sequence 0 whole, sequence 1 without the tokens of the bad block
    rk, rv, rs = oracle.append(_np(kn)[:1], _np(vn)[:1], table.numpy()[:1], lens[:1], *before, rope="neox",
                               rope_theta=5e5)
    keep = [i for i in range(n_new) if (lens[1] + i) // 16 != bad_blk]
    assert 0 < len(keep) < n_new and keep == list(range(len(keep)))
    rk, rv, rs = oracle.append(_np(kn)[1:, keep], _np(vn)[1:, keep], table.numpy()[1:], lens[1:], rk, rv, rs,
                               rope="neox", rope_theta=5e5)
    assert _pools_equal(_np(kc), rk) and _pools_equal(_np(vc), rv) and _pools_equal(_np(ks), rs)
    assert np.all(np.isnan(_np(kc)[NB:])) and np.all(np.isnan(_np(vc)[NB:]))
    # a clean append leaves the word at zero
    status.zero_()
    da.append(kn.to(dev), vn.to(dev), x["block_table"].to(dev), torch.tensor(lens, dtype=torch.int32, device=dev),
              kc, vc, ks, rope="neox", rope_theta=5e5, pos_host=lens, num_blocks=NB, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0


def test_cache_built_by_appends_then_decoded():
    # Prefill three sequences entirely through the append kernel (chunks of 64 and
    # a ragged tail), check the pools against the oracle's appends, then decode
    # full and FOLD on the GPU-built cache against the oracle on its own cache.
    da = _da()
    dev = torch.device("cuda:0")
    lens = [1000, 77, 2500]
    d, Hkv, Hq, T = 128, 2, 8, 4
    x = synth.make_inputs(ctx_lens=lens, T=T, Hq=Hq, Hkv=Hkv, d=d, seed=41, fold=True)
    g = torch.Generator().manual_seed(7)
    total = max(lens)
    kr = torch.randn((3, total, Hkv, d), generator=g).to(torch.bfloat16)
    vr = torch.randn((3, total, Hkv, d), generator=g).to(torch.bfloat16)
    kc, vc, ks = x["k_cache"].to(dev), x["v_cache"].to(dev), x["k_side"].to(dev)
    table = x["block_table"].to(dev)
    rk, rv, rs = _np(x["k_cache"]), _np(x["v_cache"]), _np(x["k_side"])
    done = [0, 0, 0]
    while any(done[b] < lens[b] for b in range(3)):
        # every sequence appends the same number of tokens per call; finished ones
        # append into positions past their length in their own (spare) capacity
        chunk = 64
        for b in range(3):
            if done[b] >= lens[b]:
                continue
            n = min(chunk, lens[b] - done[b])
            sel = slice(done[b], done[b] + n)
            kb, vb = kr[b:b + 1, sel].contiguous(), vr[b:b + 1, sel].contiguous()
            da.append(kb.to(dev), vb.to(dev), table[b:b + 1], torch.tensor([done[b]], dtype=torch.int32, device=dev),
                      kc, vc, ks, rope="neox", rope_theta=5e5, pos_host=[done[b]])
            rk, rv, rs = oracle.append(_np(kb), _np(vb), x["block_table"].numpy()[b:b + 1], [done[b]], rk, rv, rs,
                                       rope="neox", rope_theta=5e5)
            done[b] += n
    torch.cuda.synchronize()
    assert _pools_equal(_np(kc), rk) and _pools_equal(_np(vc), rv) and _pools_equal(_np(ks), rs)
    q = x["q"].to(dev)
    ctx = x["ctx_len"].to(dev)
    for kw in (dict(mode="full"), dict(mode="fold", window=300, alpha=2.0, beta=-1.0)):
        side = ks if kw["mode"] == "fold" else None
        out, lse = da.decode(q, kc, vc, table, ctx, k_side=side, ctx_lens=lens, rope_theta=5e5, **kw)
        torch.cuda.synchronize()
        ref = oracle.decode(_np(x["q"]), rk, rv, x["block_table"].numpy(), lens, k_side=rs, rope_theta=5e5, **kw)
        dout = float(np.abs(out.cpu().numpy() - ref["out"]).max())
        dlse = float(np.abs(lse.cpu().numpy() - ref["lse"]).max())
        print(f"appended cache {kw}: max|dout|={dout:.3e} max|dlse|={dlse:.3e}", flush=True)
        assert dout <= 1e-2 and dlse <= 1e-3


def test_prepared_append_matches_the_direct_call():
    da = _da()
    dev = torch.device("cuda:0")
    lens = [40, 3]
    x = synth.make_inputs(ctx_lens=[L + 37 for L in lens], T=1, Hq=2, Hkv=2, d=128, seed=33, fold=True)
    g = torch.Generator().manual_seed(8)
    kn = torch.randn((2, 37, 2, 128), generator=g).to(torch.bfloat16).to(dev)
    vn = torch.randn((2, 37, 2, 128), generator=g).to(torch.bfloat16).to(dev)
    pos = torch.tensor(lens, dtype=torch.int32, device=dev)
    pools1 = [x[k].to(dev) for k in ("k_cache", "v_cache", "k_side")]
    pools2 = [t.clone() for t in pools1]
    da.append(kn, vn, x["block_table"].to(dev), pos, *pools1, rope_theta=5e5, pos_host=lens)
    call = da.prepare_append(kn, vn, x["block_table"].to(dev), pos, *pools2, rope_theta=5e5, pos_host=lens)
    call()
    torch.cuda.synchronize()
    for a, b in zip(pools1, pools2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("d,n_new", [(128, 30000), (64, 60000)])
def test_large_append_streaming_path_matches_oracle(d, n_new):
    # An append that moves more than 64 MiB takes the kernel's streaming
    # (nontemporal) variant: n_new tokens x 2 kv heads x 10 d bytes. Every new
    # slot must be written (and nothing else: the pools start as NaN), and two
    # samples of 1000 tokens, at the start (mid-block) and at the end of the
    # append, must equal the oracle's appends bit for bit.
    da = _da()
    dev = torch.device("cuda:0")
    Hkv, start = 2, 777
    assert n_new * Hkv * 10 * d > 64 * 1024 * 1024
    first, last = start // 16, (start + n_new - 1) // 16
    NB = last - first + 1
    table = torch.full((1, last + 1), -1, dtype=torch.int32)
    table[0, first:] = torch.arange(NB, dtype=torch.int32)
    g = torch.Generator().manual_seed(9)
    kn = (torch.randn((1, n_new, Hkv, d), generator=g) * 2).to(torch.bfloat16)
    vn = torch.randn((1, n_new, Hkv, d), generator=g).to(torch.bfloat16)
    nan_k = torch.full((NB, Hkv, d // 8, 16, 8), float("nan"), dtype=torch.bfloat16)
    nan_v = torch.full((NB, Hkv, d, 16), float("nan"), dtype=torch.bfloat16)
    gk, gv, gs = nan_k.to(dev), nan_v.to(dev), nan_k.clone().to(dev)
    da.append(kn.to(dev), vn.to(dev), table.to(dev), torch.tensor([start], dtype=torch.int32, device=dev),
              gk, gv, gs, rope="neox", rope_theta=5e5, pos_host=[start])
    torch.cuda.synchronize()
    ck, cv, cs = _np(gk), _np(gv), _np(gs)
    for pool in (ck, cv, cs):
        assert int((~np.isnan(pool)).sum()) == n_new * Hkv * d
    tab = table.numpy()
    for a in (0, n_new - 1000):
        sel = slice(a, a + 1000)
        rk, rv, rs = oracle.append(_np(kn)[:, sel], _np(vn)[:, sel], tab, [start + a], _np(nan_k), _np(nan_v),
                                   _np(nan_k), rope="neox", rope_theta=5e5)
        for ref, got in ((rk, ck), (rv, cv), (rs, cs)):
            m = ~np.isnan(ref)
            assert int(m.sum()) == 1000 * Hkv * d
            assert np.array_equal(ref[m], got[m])


@pytest.mark.parametrize("case", ["decode", "prefill"])
def test_bench_append_cases_match_the_oracle(case):
    # The append exactly as bench.py times it (its inputs and a prepared call):
    # the decode-time case (16 sequences x 8 accepted tokens at ragged
    # positions, 8 kv heads, d = 128) checked on every written slot, the
    # 64K-token prefill on 512 tokens at each end of the chunk; bit for bit.
    import bench
    da = _da()
    x = bench.append_inputs(case, 0)
    call = da.prepare_append(x["kn"], x["vn"], x["table"], x["posd"], x["kc"], x["vc"], x["ks"], rope="neox",
                             rope_theta=5e5, pos_host=x["pos"])
    call()
    torch.cuda.synchronize()
    tab = x["table"].cpu().numpy()
    n_new, B, Hkv, d = x["n_new"], x["B"], x["Hkv"], x["d"]
    windows = [(0, n_new)] if case == "decode" else [(0, 512), (n_new - 512, n_new)]
    for a, e in windows:
        # the physical blocks the window writes, as a compact pool with its own table
        logical = sorted({(b, (x["pos"][b] + i) // 16) for b in range(B) for i in range(a, e)})
        phys = [int(tab[b, j]) for b, j in logical]
        sub_tab = np.full(tab.shape, -1, dtype=np.int64)
        for k, (b, j) in enumerate(logical):
            sub_tab[b, j] = k
        idx = torch.tensor(phys, dtype=torch.long, device=x["kc"].device)
        got = [_np(t[idx]) for t in (x["kc"], x["vc"], x["ks"])]
        zk = np.zeros((len(phys), Hkv, d // 8, 16, 8))
        zv = np.zeros((len(phys), Hkv, d, 16))
        ref = oracle.append(_np(x["kn"][:, a:e]), _np(x["vn"][:, a:e]), sub_tab, [p + a for p in x["pos"]],
                            zk, zv, zk.copy(), rope="neox", rope_theta=5e5)
        # compare the slots the window writes
        mask_k = np.zeros(zk.shape, dtype=bool)
        mask_v = np.zeros(zv.shape, dtype=bool)
        for b in range(B):
            for i in range(a, e):
                p = x["pos"][b] + i
                k = int(sub_tab[b, p // 16])
                mask_k[k, :, :, p % 16, :] = True
                mask_v[k, :, :, p % 16] = True
        for r, g, m in zip(ref, got, (mask_k, mask_v, mask_k)):
            assert int(m.sum()) == B * (e - a) * Hkv * d
            assert np.array_equal(r[m], g[m]), (case, a, e)

"""Seeded random configurations through the C ABI against the fp64 oracle:
batch size, draft tokens, GQA ratio, head dim, mode, window, sinks, alpha,
beta, kappa, rope, FOLD reading, lengths (ragged, with partial blocks and
empty sequences), chunk size, launch shape and output dtype all vary. Same
bars as the parity tests; the visited key set must equal the oracle's."""

import math
import os
import random

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

# 48 by default; a longer sweep: DRAFT_ATTN_FUZZ_CASES=600
N_CASES = int(os.environ.get("DRAFT_ATTN_FUZZ_CASES", "48"))


def draw(rnd):
    d = rnd.choice([64, 128])
    Hkv = rnd.choice([1, 2, 4])
    G = rnd.choice([1, 2, 4, 8])
    T = rnd.randint(1, max(1, 32 // G))
    B = rnd.randint(1, 5)
    lens = [rnd.choice([0, 1, 15, 16, 17, 31, 33, rnd.randint(1, 600), rnd.randint(600, 6000)]) for _ in range(B)]
    mode = rnd.choice(["full", "window", "fold"])
    kw = dict(mode=mode)
    if mode == "window":
        kw.update(window=rnd.choice([0, 1, 16, 100, 512, 5000]), n_sink=rnd.choice([0, 1, 4, 20]))
    if mode == "fold":
        kw.update(window=rnd.choice([0, 1, 17, 256, 2000]), alpha=rnd.choice([0.5, 1.0, 2.0, 3.0]),
                  beta=rnd.choice([-1.5, 0.0, 0.7]), rope=rnd.choice(["neox", "none"]),
                  fold_variant=rnd.choice(["B", "A", "B'"]))
    if rnd.random() < 0.4:
        kw.update(kappa=rnd.choice([-0.05, 0.1, 0.3]), n0=rnd.choice([1, 16, 256]))
    split = rnd.choice([0, 0, 32, 96, 256, 384, 640, 1024])
    launch = rnd.choice(["auto", "two_pass", "single"])
    out_dtype = rnd.choice(["f32", "f32", "bf16"])
    needle = rnd.choice([0.0, 0.0, 0.02])
    # drawn last, so the earlier fields of every case stay as they were: about a
    # quarter of the cases take the fused call with the step's draft keys, under
    # every FOLD reading
    fused = rnd.random() < 0.25
    # about one case in ten is a batch of 33 to 40 sequences: more than the 32
    # whose lengths travel with the kernel arguments
    if rnd.random() < 0.1:
        lens = lens + [rnd.choice([0, 5, 16, 40, rnd.randint(1, 300)]) for _ in range(33 - B + rnd.randint(0, 7))]
    return dict(d=d, Hkv=Hkv, G=G, T=T, lens=lens, kw=kw, split=split, launch=launch, out_dtype=out_dtype,
                needle=needle, fused=fused)


CASES = [draw(random.Random(1000 + i)) for i in range(N_CASES)]


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(N_CASES)])
def test_random_configuration_matches_the_oracle(case):
    import draft_attention_amd as da
    c = case
    x = synth.make_inputs(ctx_lens=c["lens"], T=c["T"], Hq=c["G"] * c["Hkv"], Hkv=c["Hkv"], d=c["d"], seed=7,
                          fold=c["kw"]["mode"] == "fold", needle_frac=c["needle"])
    dev = torch.device("cuda:0")
    g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in x.items()}
    stride = max(max(c["lens"]), 1)
    vis = torch.zeros((len(c["lens"]), stride), dtype=torch.uint8, device=dev)
    side = g["k_side"] if c["kw"]["mode"] == "fold" else None
    kd = vd = None
    if c["fused"]:
        gen = torch.Generator().manual_seed(hash((c["d"], c["T"], tuple(c["lens"]))) % (1 << 31))
        kd = (torch.randn((len(c["lens"]), c["T"], c["Hkv"], c["d"]), generator=gen) * 2).to(torch.bfloat16)
        vd = torch.randn((len(c["lens"]), c["T"], c["Hkv"], c["d"]), generator=gen).to(torch.bfloat16)
    try:
        out, lse = da.decode(g["q"], g["k_cache"], g["v_cache"], g["block_table"], g["ctx_len"], k_side=side,
                             ctx_lens=c["lens"], rope_theta=5e5, split_keys=c["split"], launch=c["launch"],
                             out_dtype=c["out_dtype"], debug_visit=vis,
                             k_draft=None if kd is None else kd.to(dev), v_draft=None if vd is None else vd.to(dev),
                             **c["kw"])
    except da.DraftAttnError as e:
        # the only refusal a valid draw can meet: single launch with a fixed chunk
        # that leaves more than MAX_GROUP_ITEMS items in a group
        assert e.status == da.ENOTSUP and c["launch"] == "single" and c["split"], (c, e)
        return
    torch.cuda.synchronize()
    n = {k: (v.float().numpy() if torch.is_tensor(v) and v.is_floating_point() else v) for k, v in x.items()}
    if kd is None:
        ref = oracle.decode(n["q"], n["k_cache"], n["v_cache"], x["block_table"].numpy(), c["lens"],
                            k_side=n["k_side"], rope_theta=5e5, **c["kw"])
    else:
        kw = {k: v for k, v in c["kw"].items() if k != "mode"}
        ref = oracle.decode_with_draft(n["q"], n["k_cache"], n["v_cache"], x["block_table"].numpy(), c["lens"],
                                       c["kw"]["mode"], kd.float().numpy(), vd.float().numpy(), k_side=n["k_side"],
                                       rope_theta=5e5, **kw)
    if kd is not None and c["out_dtype"] == "f32" and c["launch"] != "single":
        # the same step as two calls (decode on two kernels, as the fused call
        # always runs, then the separate draft merge) equals the fused call bit
        # for bit
        kw = {k: v for k, v in c["kw"].items() if k != "fold_variant"}
        o2, l2 = da.decode(g["q"], g["k_cache"], g["v_cache"], g["block_table"], g["ctx_len"], k_side=side,
                           ctx_lens=c["lens"], rope_theta=5e5, split_keys=c["split"], launch="two_pass",
                           **c["kw"])
        da.merge_draft(g["q"], kd.to(dev), vd.to(dev), g["ctx_len"], o2, l2, num_blocks=g["k_cache"].shape[0],
                       max_blocks_per_seq=g["block_table"].shape[1], num_kv_heads=c["Hkv"], ctx_lens=c["lens"],
                       rope_theta=5e5, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o2, out) and torch.equal(l2, lse), c
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    empty = np.isneginf(ref["lse"])
    assert np.array_equal(np.isneginf(l), empty), c
    bound = 1e-2 + (2.0 ** -8 * np.abs(ref["out"]) if c["out_dtype"] == "bf16" else 0.0)
    dout = np.abs(o - ref["out"])
    dlse = float(np.abs(l[~empty] - ref["lse"][~empty]).max()) if (~empty).any() else 0.0
    print(f"{c['kw']} d={c['d']} G={c['G']} T={c['T']} lens={c['lens']} split={c['split']} {c['launch']} "
          f"{'fused ' if c['fused'] else ''}"
          f"{c['out_dtype']}: max|dout|={float(dout.max()) if dout.size else 0:.2e} max|dlse|={dlse:.2e}", flush=True)
    assert np.all(np.isfinite(o)) and np.all(dout <= bound) and dlse <= 1e-3, c
    want = np.zeros_like(vis.cpu().numpy())
    for b, L in enumerate(c["lens"]):
        main, far = oracle.index_sets(L, c["kw"]["mode"], c["kw"].get("window", 0), c["kw"].get("n_sink", 0))
        want[b, main] = 1
        want[b, far] = 2
    assert np.array_equal(vis.cpu().numpy(), want), c

"""GPU parity of draft-token self-attention merged into the cache attention
(draft_attn_decode followed by draft_attn_merge_draft) against the oracle's
single softmax over cached visible keys and draft keys 0..t."""

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kw", [
    dict(mode="full"),
    dict(mode="window", window=500, n_sink=4),
    dict(mode="fold", window=700, alpha=2.0, beta=-1.0),
    dict(mode="full", kappa=0.2, n0=256),
    dict(mode="fold", window=300, alpha=4.0, beta=0.5, kappa=0.1, n0=64, rope="none"),
    dict(mode="fold", window=700, alpha=2.0, beta=-1.0, fold_variant="A"),
    dict(mode="fold", window=300, alpha=0.5, beta=1.0, kappa=0.1, n0=64, fold_variant="B'"),
], ids=["full", "window", "fold", "full-kappa", "fold-kappa-nope", "fold-A", "fold-Bprime-kappa"])
@pytest.mark.parametrize("d,T,G", [(128, 4, 4), (64, 8, 2), (128, 1, 8), (128, 32, 1)])
def test_decode_then_merge_draft(kw, d, T, G):
    import draft_attention_amd as da
    dev = torch.device("cuda:0")
    lens = [0, 5, 3000, 1234]
    Hkv = 2
    x = synth.make_inputs(ctx_lens=lens, T=T, Hq=G * Hkv, Hkv=Hkv, d=d, seed=61, fold=True)
    g = torch.Generator().manual_seed(62)
    kd = (torch.randn((4, T, Hkv, d), generator=g) * 2).to(torch.bfloat16)
    vd = torch.randn((4, T, Hkv, d), generator=g).to(torch.bfloat16)
    q, kc, vc, ks = (x[k].to(dev) for k in ("q", "k_cache", "v_cache", "k_side"))
    table, ctx = x["block_table"].to(dev), x["ctx_len"].to(dev)
    side = ks if kw["mode"] == "fold" else None
    out, lse = da.decode(q, kc, vc, table, ctx, k_side=side, ctx_lens=lens, rope_theta=5e5, **kw)
    # the merge does not depend on the FOLD reading: each reading's far mass is
    # already in the cache result's lse
    mkw = {k: v for k, v in kw.items() if k != "fold_variant"}
    da.merge_draft(q, kd.to(dev), vd.to(dev), ctx, out, lse, num_blocks=kc.shape[0],
                   max_blocks_per_seq=table.shape[1], num_kv_heads=Hkv, ctx_lens=lens, rope_theta=5e5, **mkw)
    torch.cuda.synchronize()
    n = {k: (v.float().numpy() if torch.is_tensor(v) and v.is_floating_point() else v) for k, v in x.items()}
    ref = oracle.decode_with_draft(n["q"], n["k_cache"], n["v_cache"], x["block_table"].numpy(), lens, kw["mode"],
                                   kd.float().numpy(), vd.float().numpy(), k_side=n["k_side"], rope_theta=5e5,
                                   **{k: v for k, v in kw.items() if k != "mode"})
    dout = float(np.abs(out.cpu().numpy() - ref["out"]).max())
    dlse = float(np.abs(lse.cpu().numpy() - ref["lse"]).max())
    print(f"merge_draft {kw} d={d} T={T} G={G}: max|dout|={dout:.3e} max|dlse|={dlse:.3e}", flush=True)
    assert np.all(np.isfinite(out.cpu().numpy()))
    assert dout <= 1e-2 and dlse <= 1e-3


def test_prepared_merge_draft_matches_the_direct_call():
    import draft_attention_amd as da
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(63)
    B, T, Hq, Hkv, d = 3, 6, 8, 2, 128
    q = torch.randn((B, T, Hq, d), generator=g, device=dev).to(torch.bfloat16)
    kd = torch.randn((B, T, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
    vd = torch.randn((B, T, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
    out0 = torch.randn((B, T, Hq, d), generator=g, device=dev)
    lse0 = torch.randn((B, T, Hq), generator=g, device=dev)
    lens = [100, 2000, 7]
    ctx = torch.tensor(lens, dtype=torch.int32, device=dev)
    kw = dict(num_blocks=200, max_blocks_per_seq=130, num_kv_heads=Hkv, ctx_lens=lens, kappa=0.1, n0=64)
    o1, l1 = out0.clone(), lse0.clone()
    da.merge_draft(q, kd, vd, ctx, o1, l1, **kw)
    o2, l2 = out0.clone(), lse0.clone()
    call = da.prepare_merge_draft(q, kd, vd, ctx, o2, l2, **kw)
    call()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("kw", [
    dict(mode="full"),
    dict(mode="window", window=500, n_sink=4),
    dict(mode="fold", window=700, alpha=2.0, beta=-1.0),
    dict(mode="fold", window=300, alpha=4.0, beta=0.5, kappa=0.1, n0=64, rope="none"),
    dict(mode="fold", window=700, alpha=2.0, beta=-1.0, fold_variant="A"),
    dict(mode="fold", window=300, alpha=3.0, beta=0.5, fold_variant="B'"),
], ids=["full", "window", "fold", "fold-kappa-nope", "fold-A", "fold-Bprime"])
@pytest.mark.parametrize("d,T,G", [(128, 4, 4), (64, 8, 2), (128, 1, 8), (128, 32, 1), (64, 12, 2)])
def test_fused_decode_draft_equals_the_two_calls(kw, d, T, G):
    # draft_attn_decode_draft applies the draft part inside the decode's merge
    # kernel with the same arithmetic as the separate merge call: fp32 results
    # equal bit for bit, on either launch setting (the fused call always runs on
    # two kernels), and bf16 output is the fused fp32 value rounded once.
    import draft_attention_amd as da
    dev = torch.device("cuda:0")
    lens = [0, 5, 3000, 1234]
    Hkv = 2
    x = synth.make_inputs(ctx_lens=lens, T=T, Hq=G * Hkv, Hkv=Hkv, d=d, seed=71, fold=True)
    g = torch.Generator().manual_seed(72)
    kd = (torch.randn((4, T, Hkv, d), generator=g) * 2).to(torch.bfloat16).to(dev)
    vd = torch.randn((4, T, Hkv, d), generator=g).to(torch.bfloat16).to(dev)
    q, kc, vc, ks = (x[k].to(dev) for k in ("q", "k_cache", "v_cache", "k_side"))
    table, ctx = x["block_table"].to(dev), x["ctx_len"].to(dev)
    side = ks if kw["mode"] == "fold" else None
    out, lse = da.decode(q, kc, vc, table, ctx, k_side=side, ctx_lens=lens, rope_theta=5e5, launch="two_pass", **kw)
    mkw = {k: v for k, v in kw.items() if k != "fold_variant"}
    da.merge_draft(q, kd, vd, ctx, out, lse, num_blocks=kc.shape[0], max_blocks_per_seq=table.shape[1],
                   num_kv_heads=Hkv, ctx_lens=lens, rope_theta=5e5, **mkw)
    for launch in ("auto", "single"):
        fo, fl = da.decode(q, kc, vc, table, ctx, k_side=side, ctx_lens=lens, rope_theta=5e5, launch=launch,
                           k_draft=kd, v_draft=vd, **kw)
        torch.cuda.synchronize()
        assert torch.equal(fo, out) and torch.equal(fl, lse), (kw, launch)
    bo, bl = da.decode(q, kc, vc, table, ctx, k_side=side, ctx_lens=lens, rope_theta=5e5, out_dtype="bf16",
                       k_draft=kd, v_draft=vd, **kw)
    torch.cuda.synchronize()
    assert torch.equal(bo, out.to(torch.bfloat16)) and torch.equal(bl, lse)


@pytest.mark.parametrize("kw", [dict(mode="full", kappa=0.1, n0=64), dict(mode="window", window=200, n_sink=4)],
                         ids=["full-kappa", "window"])
def test_draft_merge_of_a_batch_beyond_the_argument_lengths(kw):
    # 40 sequences: more than the 32 whose lengths travel with the kernel
    # arguments, so both the separate merge and the fused call read ctx_len in
    # device memory. Checked against the oracle, and fused against two calls.
    import draft_attention_amd as da
    dev = torch.device("cuda:0")
    rnd = np.random.default_rng(81)
    lens = [int(v) for v in rnd.integers(0, 700, size=40)]
    lens[3] = 0
    B, T, Hkv, G, d = len(lens), 3, 2, 2, 64
    x = synth.make_inputs(ctx_lens=lens, T=T, Hq=G * Hkv, Hkv=Hkv, d=d, seed=82)
    g = torch.Generator().manual_seed(83)
    kd = (torch.randn((B, T, Hkv, d), generator=g) * 2).to(torch.bfloat16)
    vd = torch.randn((B, T, Hkv, d), generator=g).to(torch.bfloat16)
    q, kc, vc = (x[k].to(dev) for k in ("q", "k_cache", "v_cache"))
    table, ctx = x["block_table"].to(dev), x["ctx_len"].to(dev)
    out, lse = da.decode(q, kc, vc, table, ctx, ctx_lens=lens, launch="two_pass", **kw)
    da.merge_draft(q, kd.to(dev), vd.to(dev), ctx, out, lse, num_blocks=kc.shape[0],
                   max_blocks_per_seq=table.shape[1], num_kv_heads=Hkv, ctx_lens=lens, **kw)
    fo, fl = da.decode(q, kc, vc, table, ctx, ctx_lens=lens, k_draft=kd.to(dev), v_draft=vd.to(dev), **kw)
    torch.cuda.synchronize()
    assert torch.equal(fo, out) and torch.equal(fl, lse)
    n = {k: (v.float().numpy() if torch.is_tensor(v) and v.is_floating_point() else v) for k, v in x.items()}
    ref = oracle.decode_with_draft(n["q"], n["k_cache"], n["v_cache"], x["block_table"].numpy(), lens, kw["mode"],
                                   kd.float().numpy(), vd.float().numpy(),
                                   **{k: v for k, v in kw.items() if k != "mode"})
    dout = float(np.abs(out.cpu().numpy() - ref["out"]).max())
    dlse = float(np.abs(lse.cpu().numpy() - ref["lse"]).max())
    print(f"merge_draft batch of {B} {kw}: max|dout|={dout:.3e} max|dlse|={dlse:.3e}", flush=True)
    assert dout <= 1e-2 and dlse <= 1e-3

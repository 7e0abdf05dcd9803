"""The allocation-free entry point (draft_attn_decode_noalloc) through the C ABI:
two calls in a row, the second with a smaller input, each equal bit for bit to
draft_attn_decode on the same inputs and within the oracle's bars."""

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def _np(x):
    return {k: (v.float().cpu().numpy() if torch.is_tensor(v) and v.is_floating_point() else
                (v.cpu().numpy() if torch.is_tensor(v) else v)) for k, v in x.items()}


@pytest.mark.parametrize("launch", ["two_pass", "single"])
def test_noalloc_equals_decode_on_two_calls_in_a_row(launch):
    import draft_attention_amd as da
    dev = torch.device("cuda:0")
    cases = [  # the second input is smaller than the first (fewer items, rows and keys)
        (dict(ctx_lens=[40000, 3000, 17], T=6, Hq=16, Hkv=4, d=128, seed=81, fold=True),
         dict(mode="fold", window=1024, alpha=2.0, beta=-1.0, kappa=0.1, n0=256)),
        (dict(ctx_lens=[2500, 33], T=2, Hq=8, Hkv=2, d=64, seed=82, fold=True),
         dict(mode="window", window=700, n_sink=4)),
    ]
    for i, (shape, kw) in enumerate(cases):
        x = synth.make_inputs(**shape)
        g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in x.items()}
        side = g["k_side"] if kw["mode"] == "fold" else None
        ref_out, ref_lse = da.decode(g["q"], g["k_cache"], g["v_cache"], g["block_table"], g["ctx_len"], k_side=side,
                                     ctx_lens=x["ctx_lens"], rope_theta=5e5, launch=launch, **kw)
        out = torch.full_like(ref_out, float("nan"))
        lse = torch.full_like(ref_lse, float("nan"))
        da.decode_noalloc(g["q"], g["k_cache"], g["v_cache"], g["block_table"], g["ctx_len"], out=out, lse=lse,
                          ctx_lens=x["ctx_lens"], k_side=side, rope_theta=5e5, launch=launch, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), (i, launch)
        n = _np(x)
        ref = oracle.decode(n["q"], n["k_cache"], n["v_cache"], n["block_table"], x["ctx_lens"], k_side=n["k_side"],
                            rope_theta=5e5, **kw)
        dout = float(np.abs(out.cpu().numpy() - ref["out"]).max())
        dlse = float(np.abs(lse.cpu().numpy() - ref["lse"]).max())
        print(f"noalloc call {i} {launch} {kw}: max|dout|={dout:.3e} max|dlse|={dlse:.3e}", flush=True)
        assert dout <= 1e-2 and dlse <= 1e-3


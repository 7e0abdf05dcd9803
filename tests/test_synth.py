"""Properties of the seeded input generator (layout, padding, determinism)."""

import math

import numpy as np
import torch

import synth


def test_layout_padding_and_determinism():
    a = synth.make_inputs(ctx_lens=[37, 16, 0, 50], T=2, Hq=4, Hkv=2, d=8, seed=3, fold=True)
    b = synth.make_inputs(ctx_lens=[37, 16, 0, 50], T=2, Hq=4, Hkv=2, d=8, seed=3, fold=True)
    for key in ("q", "k_cache", "v_cache", "k_side", "block_table", "ctx_len"):
        assert torch.equal(torch.nan_to_num(a[key].float(), 123.0), torch.nan_to_num(b[key].float(), 123.0))
    assert a["q"].shape == (4, 2, 4, 8) and a["q"].dtype == torch.bfloat16
    NB = 3 + 1 + 0 + 4 + 2
    assert a["k_cache"].shape == (NB, 2, 1, 16, 8)
    assert a["v_cache"].shape == (NB, 2, 8, 16)
    t = a["block_table"]
    assert t.shape == (4, 4) and t.dtype == torch.int32
    used = t[t >= 0].tolist()
    assert sorted(used) == sorted(set(used)) and len(used) == 8
    assert t[2].tolist() == [-1] * 4 and t[1, 1:].tolist() == [-1] * 3
    # slots past L are NaN, slots below L are finite
    blk = int(t[0, 2])
    assert torch.isnan(a["k_cache"][blk, :, :, 5:, :].float()).all()
    assert torch.isfinite(a["k_cache"][blk, :, :, :5, :].float()).all()
    assert torch.isnan(a["v_cache"][blk, :, :, 5:].float()).all()
    assert torch.isnan(a["k_side"][blk, :, :, 5:, :].float()).all()
    spare = sorted(set(range(NB)) - set(used))
    assert all(torch.isnan(a["k_cache"][s].float()).all() for s in spare)
    c = synth.make_inputs(ctx_lens=[37, 16, 0, 50], T=2, Hq=4, Hkv=2, d=8, seed=4, fold=True)
    assert not torch.equal(torch.nan_to_num(a["q"].float()), torch.nan_to_num(c["q"].float()))


def test_values_are_bf16_roundings_of_normal_draws():
    x = synth.make_inputs(ctx_lens=[4096], T=1, Hq=1, Hkv=1, d=64, seed=0, fill="zero")
    k = x["k_cache"].float().numpy().ravel()
    assert abs(k.mean()) < 0.01 and abs(k.std() - 1) < 0.01
    assert np.array_equal(torch.from_numpy(k).to(torch.bfloat16).float().numpy(), k)


def test_needles_scale_keys_in_both_caches():
    L = 3200
    kw = dict(ctx_lens=[L], T=1, Hq=1, Hkv=1, d=16, seed=1, fold=True, fill="zero")
    x = synth.make_inputs(needle_frac=0.01, **kw)
    y = synth.make_inputs(needle_frac=0.0, **kw)
    for key in ("k_cache", "k_side"):
        a = x[key].float().permute(0, 1, 3, 2, 4).reshape(-1, 16)   # one row per (block, head, slot)
        b = y[key].float().permute(0, 1, 3, 2, 4).reshape(-1, 16)
        scaled = torch.all(a == 8 * b, dim=1) & torch.any(b != 0, dim=1)
        same = torch.all(a == b, dim=1)
        assert torch.all(scaled | same)
        assert scaled.sum().item() == 32
        if key == "k_cache":
            rows = scaled
        else:
            assert torch.equal(rows, scaled)
    assert torch.equal(x["v_cache"], y["v_cache"])


def test_ragged_lengths_are_log_uniform_in_range():
    lens = synth.ragged_lengths(1000, 32768, 524288, seed=0)
    assert min(lens) >= 32768 and max(lens) < 524288
    logs = np.log(lens)
    assert abs(np.median(logs) - 0.5 * (math.log(32768) + math.log(524288))) < 0.15
    assert synth.ragged_lengths(16, 32768, 524288, 0) == synth.workloads(0)["batch16_ragged"].ctx_lens

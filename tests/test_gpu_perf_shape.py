"""Performance shape on the GPU: a FULL step costs in proportion to the context
it reads; a WINDOW step (window + sinks) costs about the same at any context
length, since it reads the same number of keys ("Windowed-MTP: Removing the
Full-Context Draft-KV Tax at Million-Token Context", Abstract); a FOLD step
reads the same bytes as FULL ("FOLD: Position-Free Far Memory with Local Order
for Long-Context Speculative Decoding", review: the far memory is read whole,
without retrieval), so it costs about what FULL does. Bounds are loose: these
check shapes, not speeds."""

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def step_us(L, kw, T=4, reps=30, fold=False):
    import draft_attention_amd as da
    dev = torch.device("cuda:0")
    x = synth.make_inputs(ctx_lens=[L], T=T, Hq=32, Hkv=8, d=128, seed=3, device=dev, fold=fold, fill="zero")
    call = da.prepare(x["q"], x["k_cache"], x["v_cache"], x["block_table"], x["ctx_len"], ctx_lens=[L],
                      k_side=x["k_side"] if fold else None, rope_theta=5e5, **kw)
    for _ in range(5):
        call()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        call()
    b.record()
    torch.cuda.synchronize()
    del x, call
    torch.cuda.empty_cache()
    return a.elapsed_time(b) * 1e3 / reps


def test_full_step_grows_with_context_and_window_step_does_not():
    full = {L: step_us(L, dict(mode="full")) for L in (1 << 18, 1 << 20)}
    ratio = full[1 << 20] / full[1 << 18]
    print(f"FULL 256K {full[1 << 18]:.1f} us, 1M {full[1 << 20]:.1f} us: x{ratio:.2f} for 4x the keys", flush=True)
    assert 3.0 <= ratio <= 4.6
    win = {L: step_us(L, dict(mode="window", window=2048, n_sink=4)) for L in (1 << 14, 1 << 18, 1 << 20)}
    print("WINDOW 2048+4: " + ", ".join(f"{L >> 10}K {t:.1f} us" for L, t in win.items()), flush=True)
    assert max(win.values()) <= 1.5 * min(win.values())
    assert win[1 << 20] * 10 < full[1 << 20]


def test_fold_step_costs_about_a_full_step():
    L = 1 << 18
    full = step_us(L, dict(mode="full"), T=6)
    fold = step_us(L, dict(mode="fold", window=4096, alpha=2.0, beta=-1.0), T=6, fold=True)
    print(f"256K, 6 draft tokens: FULL {full:.1f} us, FOLD {fold:.1f} us", flush=True)
    assert 0.8 * full <= fold <= 1.25 * full


def test_launch_floor_runs_the_call_shape_and_stays_below_the_step():
    # draft_attn_launch_floor enqueues the decode call's launches (grids, LDS,
    # argument blocks) with empty kernels; on one or two kernels it must run
    # cleanly, and a real window step must not be cheaper than its own floor
    # by more than noise
    import draft_attention_amd as da
    L, W = 1 << 17, 2048
    p = da.make_params(num_seqs=1, num_draft_tokens=4, num_q_heads=32, num_kv_heads=8, head_dim=128,
                       num_blocks=(L >> 4) + 16, max_blocks_per_seq=(L >> 4) + 8, mode="window", window=W,
                       n_sink=4)
    floors = {}
    for nk in (1, 2):
        call = da.prepare_launch_floor(p, [L], nk)
        for _ in range(5):
            call()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(30):
            call()
        b.record()
        torch.cuda.synchronize()
        floors[nk] = a.elapsed_time(b) * 1e3 / 30
    step = step_us(L, dict(mode="window", window=W, n_sink=4))
    print(f"floor one kernel {floors[1]:.2f} us, two {floors[2]:.2f} us; window step {step:.2f} us", flush=True)
    assert floors[1] > 0 and floors[2] > 0
    assert step > 0.8 * floors[2]

"""Ring-buffer draft cache for WINDOW mode: a sequence grown by appends into a
ring of (sinks + window + append) blocks decodes bit-identically to the same
sequence kept in a full cache, at every step, while holding a constant number
of blocks; at every 20th step and the last, the ring decode also matches the
fp64 oracle run on host copies of the ring pools and table (max|d out| <= 1e-2,
max|d lse| <= 1e-3, visited keys bit-exact), before and after the ring wraps."""

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


def test_window_decode_over_a_ring_equals_the_full_cache():
    import draft_attention_amd as da
    dev = torch.device("cuda:0")
    W, S, n_new, d, Hkv, Hq, T = 200, 4, 7, 128, 2, 8, 2
    starts = [0, 35]                       # sequence 1 starts from a 35-token prefill
    steps = 260
    final = [s + steps * n_new for s in starts]
    MB = max(final) // 16 + 2
    sb, rl = da.ring_size(W, S, n_new)
    # full cache: each sequence owns every block of its positions
    NBf = 2 * MB
    kf = torch.zeros((NBf, Hkv, d // 8, 16, 8), dtype=torch.bfloat16, device=dev)
    vf = torch.zeros((NBf, Hkv, d, 16), dtype=torch.bfloat16, device=dev)
    tf = torch.tensor([[b * MB + j for j in range(MB)] for b in range(2)], dtype=torch.int32, device=dev)
    # ring cache: sink blocks + a ring per sequence, nothing else
    per = sb + rl
    kr = torch.zeros((2 * per, Hkv, d // 8, 16, 8), dtype=torch.bfloat16, device=dev)
    vr = torch.zeros((2 * per, Hkv, d, 16), dtype=torch.bfloat16, device=dev)
    sinks = [list(range(b * per, b * per + sb)) for b in range(2)]
    rings = [list(range(b * per + sb, (b + 1) * per)) for b in range(2)]
    g = torch.Generator().manual_seed(71)
    L = [0, 0]

    def ring_rows():
        return torch.tensor([da.ring_table(L[b], n_new, W, S, sinks[b], rings[b], MB) for b in range(2)],
                            dtype=torch.int32, device=dev)

    # prefill sequence 1 in appends of n_new tokens, through both tables
    while L[1] < starts[1]:
        kp = torch.randn((1, n_new, Hkv, d), generator=g).to(torch.bfloat16).to(dev)
        vp = torch.randn((1, n_new, Hkv, d), generator=g).to(torch.bfloat16).to(dev)
        pos = torch.tensor([L[1]], dtype=torch.int32, device=dev)
        da.append(kp, vp, tf[1:2], pos, kf, vf, rope_theta=5e5, pos_host=[L[1]])
        row = torch.tensor([da.ring_table(L[1], n_new, W, S, sinks[1], rings[1], MB)], dtype=torch.int32, device=dev)
        da.append(kp, vp, row, pos, kr, vr, rope_theta=5e5, pos_host=[L[1]])
        L[1] += n_new
    q = torch.randn((2, T, Hq, d), generator=g).to(torch.bfloat16).to(dev)
    qn = q.float().cpu().numpy()
    checked, wrapped = 0, False
    for step in range(steps):
        rt = ring_rows()
        if min(L) > 0:
            ctx = torch.tensor(L, dtype=torch.int32, device=dev)
            of, lf = da.decode(q, kf, vf, tf, ctx, mode="window", window=W, n_sink=S, ctx_lens=L)
            vis = torch.zeros((2, max(L)), dtype=torch.uint8, device=dev)
            orr, lr = da.decode(q, kr, vr, rt, ctx, mode="window", window=W, n_sink=S, ctx_lens=L, debug_visit=vis)
            torch.cuda.synchronize()
            assert torch.equal(of, orr) and torch.equal(lf, lr), f"step {step} lengths {L}"
            if step % 20 == 0 or step == steps - 1:
                # the oracle on the ring's own pools and table: its -1 entries are
                # never read, and the window's blocks sit where the ring put them
                table = rt.cpu().numpy()
                ref = oracle.decode(qn, kr.float().cpu().numpy(), vr.float().cpu().numpy(), table, L, "window",
                                    window=W, n_sink=S)
                dout = float(np.abs(orr.cpu().numpy() - ref["out"]).max())
                dlse = float(np.abs(lr.cpu().numpy() - ref["lse"]).max())
                assert dout <= 1e-2 and dlse <= 1e-3, (step, L, dout, dlse)
                want = np.zeros((2, max(L)), dtype=np.uint8)
                for b in range(2):
                    main, _ = oracle.index_sets(L[b], "window", W, S)
                    want[b, main] = 1
                assert np.array_equal(vis.cpu().numpy(), want), f"step {step}: visited keys differ"
                checked += 1
                wrapped |= (max(L) + 15) // 16 > per
        kn = torch.randn((2, n_new, Hkv, d), generator=g).to(torch.bfloat16).to(dev)
        vn = torch.randn((2, n_new, Hkv, d), generator=g).to(torch.bfloat16).to(dev)
        pos = torch.tensor(L, dtype=torch.int32, device=dev)
        da.append(kn, vn, tf, pos, kf, vf, rope_theta=5e5, pos_host=L)
        da.append(kn, vn, rt, pos, kr, vr, rope_theta=5e5, pos_host=L)
        L = [x + n_new for x in L]
    torch.cuda.synchronize()
    assert L == final
    assert checked >= 10 and wrapped, (checked, wrapped)
    full_blocks = sum((x + 15) // 16 for x in final)
    print(f"ring: {2 * per} blocks for lengths {final} (full cache: {full_blocks})", flush=True)
    assert 2 * per < full_blocks / 5

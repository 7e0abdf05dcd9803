"""Seeded synthetic inputs for draft-head decode attention.

Shared by the tests, the bench and the oracle leg. It holds none of the
attention arithmetic: it only draws random bf16 tensors and lays them out in
the paged format that the library and the oracle both document:

  q           bf16 [B, T, Hq, d]
  k_cache     bf16 [NB, Hkv, d/8, 16, 8]  rotated keys; within a block, channel
                                      8c + j of slot s sits at [c, s, j]
  k_side      bf16 [NB, Hkv, d/8, 16, 8]  unrotated keys (FOLD far memory), optional
  v_cache     bf16 [NB, Hkv, d, 16]   values, channel-major blocks
  block_table int32 [B, MB]           -1 past a sequence's last block
  ctx_len     int32 [B]

Recipe. Every value is an N(0, 1) float32 draw from a seeded torch generator,
rounded to bf16 (round-to-nearest-even). The rotated and the side key caches
are drawn independently: a rotation of an isotropic Gaussian key is again an
isotropic Gaussian, and the attention path reads each cache as given. Needle
keys (a fraction of positions chosen uniformly without replacement) are the
same draws scaled by a power of two (exact in bf16), in both key caches.
Physical blocks are a seeded random permutation of the pool. Pool slots that
hold no key (past L in a sequence's last block, and spare blocks no sequence
owns) are NaN for parity runs, so a read outside the visible set shows up in
the output, or 0 for timing runs.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

BLOCK = 16


def _randn_bf16(shape, gen, device, chunk_rows=1 << 14):
    """N(0,1) fp32 draws rounded to bf16, generated in row chunks to bound temporaries."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(shape[0], -1)
    for s in range(0, shape[0], chunk_rows):
        e = min(shape[0], s + chunk_rows)
        flat[s:e] = torch.randn((e - s, flat.shape[1]), generator=gen, device=device).to(torch.bfloat16)
    return out


def make_inputs(*, ctx_lens, T: int, Hq: int, Hkv: int, d: int, seed: int = 0, device="cpu",
                fold: bool = False, needle_frac: float = 0.0, needle_scale: float = 8.0,
                fill: str = "nan", spare_blocks: int = 2, shuffle: bool = True,
                max_blocks_per_seq: int | None = None):
    """Draw one batch of inputs. Returns a dict of tensors on ``device``."""
    ctx_lens = [int(x) for x in ctx_lens]
    B = len(ctx_lens)
    nblk = [(L + BLOCK - 1) // BLOCK for L in ctx_lens]
    MB = max(max(nblk) if nblk else 0, 1) if max_blocks_per_seq is None else int(max_blocks_per_seq)
    if any(n > MB for n in nblk):
        raise ValueError("max_blocks_per_seq too small for ctx_lens")
    used = sum(nblk)
    NB = used + int(spare_blocks)
    host = torch.Generator().manual_seed(int(seed))
    dev_gen = host if torch.device(device).type == "cpu" else \
        torch.Generator(device=device).manual_seed(int(seed) + 1)

    perm = torch.randperm(NB, generator=host) if shuffle else torch.arange(NB)
    table = torch.full((B, MB), -1, dtype=torch.int32)
    pos = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[pos:pos + n].to(torch.int32)
        pos += n
    spare = perm[used:]

    q = _randn_bf16((B, T, Hq, d), dev_gen, device)
    if d % 8:
        raise ValueError("head_dim must be a multiple of 8")
    k = _randn_bf16((NB, Hkv, d // 8, BLOCK, 8), dev_gen, device)
    v = _randn_bf16((NB, Hkv, d, BLOCK), dev_gen, device)
    ks = _randn_bf16((NB, Hkv, d // 8, BLOCK, 8), dev_gen, device) if fold else None

    # Needles: chosen logical positions get keys scaled by needle_scale in both key caches.
    if needle_frac > 0:
        for b, L in enumerate(ctx_lens):
            cnt = int(round(needle_frac * L))
            if cnt == 0:
                continue
            pos_j = torch.randperm(L, generator=host)[:cnt]
            blocks = table[b, (pos_j // BLOCK)].long().to(device)
            slots = (pos_j % BLOCK).to(device)
            k[blocks, :, :, slots, :] *= needle_scale
            if ks is not None:
                ks[blocks, :, :, slots, :] *= needle_scale

    fill_val = float("nan") if fill == "nan" else 0.0
    pad_blocks, pad_slot0 = [], []
    for b, L in enumerate(ctx_lens):
        if L % BLOCK:
            pad_blocks.append(int(table[b, L // BLOCK]))
            pad_slot0.append(L % BLOCK)
    for blk, s0 in zip(pad_blocks, pad_slot0):
        k[blk, :, :, s0:, :] = fill_val
        v[blk, :, :, s0:] = fill_val
        if ks is not None:
            ks[blk, :, :, s0:, :] = fill_val
    if spare.numel():
        sp = spare.to(device)
        k[sp] = fill_val
        v[sp] = fill_val
        if ks is not None:
            ks[sp] = fill_val

    return dict(q=q, k_cache=k, v_cache=v, k_side=ks, block_table=table.to(device),
                ctx_len=torch.tensor(ctx_lens, dtype=torch.int32).to(device),
                ctx_lens=list(ctx_lens))


def ragged_lengths(n: int, lo: int, hi: int, seed: int):
    """n lengths floor(exp(U(ln lo, ln hi))) from a seeded generator (log-uniform)."""
    g = torch.Generator().manual_seed(int(seed))
    u = torch.rand(n, generator=g, dtype=torch.float64)
    return [int(math.floor(math.exp(math.log(lo) + x * (math.log(hi) - math.log(lo))))) for x in u.tolist()]


@dataclass
class Workload:
    """One synthetic workload shaped like the pages' decoding setups."""
    name: str
    ctx_lens: list
    T: int
    Hq: int
    Hkv: int
    d: int
    rope_theta: float
    runs: list = field(default_factory=list)   # list of dicts of per-call mode arguments
    needle_frac: float = 0.0
    fold: bool = False


def workloads(seed: int = 0):
    """The five workloads: a tiny CPU-checkable case, a Llama-3-8B-shaped draft
    layer at 128K, a million-token step with needles, a FOLD split at 256K, and a
    ragged 16-sequence batch with SharpDraft-style query scaling."""
    sq = dict(kappa=0.1, n0=4096)
    return {
        "tiny_4k_gqa4_d64": Workload(
            "tiny_4k_gqa4_d64", [4096], T=2, Hq=4, Hkv=1, d=64, rope_theta=1e4,
            runs=[dict(mode="full"), dict(mode="window", window=256, n_sink=4)]),
        "llama8b_128k": Workload(
            "llama8b_128k", [131072], T=4, Hq=32, Hkv=8, d=128, rope_theta=5e5,
            runs=[dict(mode="full"), dict(mode="window", window=2048, n_sink=4)]),
        "needles_1m": Workload(
            "needles_1m", [1 << 20], T=8, Hq=32, Hkv=8, d=128, rope_theta=5e5, needle_frac=0.01,
            runs=[dict(mode="full"), dict(mode="window", window=4096, n_sink=4)]),
        "fold_256k": Workload(
            "fold_256k", [262144], T=6, Hq=32, Hkv=8, d=128, rope_theta=5e5, fold=True,
            runs=[dict(mode="fold", window=4096, alpha=a, beta=bt) for a in (1.0, 2.0, 4.0) for bt in (0.0, -1.0)]),
        "batch16_ragged": Workload(
            "batch16_ragged", ragged_lengths(16, 32768, 524288, seed), T=4, Hq=32, Hkv=8, d=128,
            rope_theta=5e5, fold=True,
            runs=[dict(mode="full", **sq), dict(mode="fold", window=4096, alpha=2.0, beta=0.0, **sq)]),
    }

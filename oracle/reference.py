"""NumPy fp64 oracle: draft-head decode attention over a paged KV cache.

TEST INFRASTRUCTURE (see the package docstring): imported only by tests/,
``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg.

Sources, by page title (sections in brackets):
  [WMTP] "Windowed-MTP: Removing the Full-Context Draft-KV Tax at Million-Token
         Context" -- Abstract; the page's "Builds on" list names PagedAttention
         (paged KV), RoFormer (rotary positions) and StreamingLLM (attention sinks).
  [FOLD] "FOLD: Position-Free Far Memory with Local Order for Long-Context
         Speculative Decoding" -- summary, review and abstract.
  [SD]   "SharpDraft: Accelerating Long-Context Speculative Decoding with
         Cardinality-Aware Query Scaling" -- Abstract.

Notation: B sequences; L = ctx_len[b]; T draft tokens per sequence; Hq query
heads; Hkv kv heads; G = Hq // Hkv; head dim d; 16-token blocks. Query head h
reads kv head h // G. All T draft tokens of a sequence see the same L cached
keys (draft tokens do not attend to each other here).

Layouts (the library documents the same ones):
  q           [B, T, Hq, d]      queries, already rotated by the caller
  k_cache     [NB, Hkv, d/8, 16, 8]  RoPE-rotated keys: within a block, channel
                                 8c + j of the key in slot s sits at [c, s, j]
  k_side      [NB, Hkv, d/8, 16, 8]  unrotated keys, read for FOLD's far memory
  v_cache     [NB, Hkv, d, 16]   values, channel-major inside a block
  block_table [B, MB]            key j of sequence b lives in physical block
                                 block_table[b, j // 16] at slot j % 16 [WMTP,
                                 Builds on: PagedAttention]

What is computed, per sequence b, draft token t and query head h:
 1. Visible sets (integer).
      full    V = [0, L): the draft reads the whole cache [WMTP, Abstract].
      window  V = [0, min(n_sink, L)) U [max(0, L-W), L): a sliding window of W
              keys plus n_sink attention-sink keys, on the draft only [WMTP,
              Abstract]. W does not count the sinks. Keys keep the rotation
              they were cached with: the window only masks.
      fold    Loc = [max(0, L-W), L) at exact positions and Far = [0, max(0, L-W))
              at one shared virtual position [FOLD, summary and abstract]. FOLD
              names no sinks.
 2. Visible count n = |V| (full, window) or L (fold: every cached key carries
    weight). Query scale s(n) = 1 + kappa * ln(max(n, n0) / n0): SharpDraft's
    closed-form fixed-slope scaling by the number of visible keys [SD,
    Abstract]; the page gives no formula, this form is the library's.
    Logit scale c = softmax_scale * s(n).
 3. Logits l_j = c * <q, k_j> over V (full, window) or Loc (fold), k_j from
    k_cache. Fold's far logits phi_j = c * <q_far, u_j>, u_j from k_side, with
    q_far = R(-P_v) q and P_v = L - W - 1 (the newest far key's true position).
    R(a) is NeoX rotate-half RoPE [WMTP, Builds on: RoFormer]: for i < d/2 the
    pair (x_i, x_{i+d/2}) turns by the angle a * theta_rope^(-2i/d).
 4. full / window:  lse = ln sum_V e^{l_j};  out = sum_V e^{l_j - lse} v_j.
 5. fold, decoupled softmax [FOLD, abstract: sharpen attention inside the far
    memory and set its total weight against the window separately; summary:
    concentration factor alpha]:
      Z_L = sum_Loc e^{l_j},  Z_F = sum_Far e^{phi_j},  Z_Fa = sum_Far e^{alpha phi_j}
      lse = ln(Z_L + e^beta Z_F)
      out = (sum_Loc e^{l_j} v_j + e^beta Z_F sum_Far (e^{alpha phi_j} / Z_Fa) v_j) / e^lse
    alpha reshapes weights only inside the far memory; the far memory's total
    weight relative to the window is e^beta Z_F / Z_L. With alpha = 1 and
    beta = 0 this is one softmax over Loc U Far.
 6. An empty visible set gives out = 0 and lse = -inf.
 7. Alternative FOLD parameterisations (``fold_variant``), same definitions of
    Z_L, Z_F, Z_Fa:
      "A"  joint softmax with far logits alpha phi_j + beta:
           lse = ln(Z_L + e^beta Z_Fa); far key j weighs e^(alpha phi_j + beta - lse)
      "B'" far memory as one virtual key with logit beta + ln(Z_Fa)/alpha and value
           sum_Far (e^{alpha phi_j} / Z_Fa) v_j: lse = ln(Z_L + e^beta Z_Fa^(1/alpha))
    All three reduce to one softmax over Loc U Far at alpha = 1, beta = 0.
"""

from __future__ import annotations

import math

import numpy as np

MODES = ("full", "window", "fold")
BLOCK = 16


def index_sets(L: int, mode: str, window: int = 0, n_sink: int = 0):
    """Return (main, far) sorted int64 key-index arrays for one sequence.

    ``main`` is V for full/window and Loc for fold; ``far`` is Far for fold and
    empty otherwise. [WMTP, Abstract] for the window and sinks; [FOLD, summary]
    for the local/far split.
    """
    L = int(L)
    empty = np.zeros(0, dtype=np.int64)
    if mode == "full":
        return np.arange(L, dtype=np.int64), empty
    if mode == "window":
        sinks = np.arange(min(int(n_sink), L), dtype=np.int64)
        recent = np.arange(max(0, L - int(window)), L, dtype=np.int64)
        return np.union1d(sinks, recent).astype(np.int64), empty
    if mode == "fold":
        start = max(0, L - int(window))
        return np.arange(start, L, dtype=np.int64), np.arange(0, start, dtype=np.int64)
    raise ValueError(f"unknown mode {mode!r}")


def visible_count(L: int, mode: str, window: int = 0, n_sink: int = 0) -> int:
    """n in SharpDraft's s(n): keys that carry weight in the softmax [SD, Abstract]."""
    main, far = index_sets(L, mode, window, n_sink)
    return int(main.size + far.size)


def query_scale(n: int, kappa: float, n0: int) -> float:
    """s(n) = 1 + kappa * ln(max(n, n0) / n0) [SD, Abstract; form fixed by this library]."""
    return 1.0 + float(kappa) * math.log(max(int(n), int(n0)) / int(n0))


def rope_rotate(x, pos: float, theta: float) -> np.ndarray:
    """NeoX rotate-half RoPE of x[..., d] by position ``pos`` (may be negative).

    Pair (x_i, x_{i+d/2}) turns by pos * theta^(-2i/d) [WMTP, Builds on:
    RoFormer]. Angles are formed in fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    omega = float(theta) ** (-2.0 * np.arange(h, dtype=np.float64) / d)
    ang = float(pos) * omega
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos], axis=-1)


def gather_keys(pool, table_row, idx, kvh: int) -> np.ndarray:
    """Rows of a key pool [NB, Hkv, d/8, 16, 8] for logical keys ``idx`` -> [n, d] fp64."""
    idx = np.asarray(idx, dtype=np.int64)
    blocks = np.asarray(table_row, dtype=np.int64)[idx // BLOCK]
    rows = pool[blocks, kvh, :, idx % BLOCK, :]          # [n, d/8, 8]
    return np.asarray(rows, dtype=np.float64).reshape(idx.size, pool.shape[2] * pool.shape[4])


def gather_values(pool, table_row, idx, kvh: int) -> np.ndarray:
    """Rows of a channel-major value pool [NB, Hkv, d, 16] for logical keys ``idx`` -> [n, d] fp64."""
    idx = np.asarray(idx, dtype=np.int64)
    blocks = np.asarray(table_row, dtype=np.int64)[idx // BLOCK]
    return np.asarray(pool[blocks, kvh, :, idx % BLOCK], dtype=np.float64)


def _logsumexp(x: np.ndarray) -> np.ndarray:
    """ln sum exp over the last axis, max-shifted; -inf for an empty axis."""
    if x.shape[-1] == 0:
        return np.full(x.shape[:-1], -np.inf)
    m = x.max(axis=-1)
    return m + np.log(np.exp(x - m[..., None]).sum(axis=-1))


def _far_log_mass(fold_variant: str, alpha: float, beta: float, lse_F, lse_Fa):
    """Log of the far memory's total weight against the local window's Z_L, per
    reading of FOLD's alpha/beta [FOLD, abstract: the far memory's total weight is
    controlled apart from the sharpening inside it]: "B" beta + ln Z_F (default),
    "A" beta + ln Z_Fa (joint softmax), "B'" beta + ln(Z_Fa)/alpha (one virtual key)."""
    return {"B": beta + lse_F, "A": beta + lse_Fa, "B'": beta + lse_Fa / alpha}[fold_variant]


def decode(q, k_cache, v_cache, block_table, ctx_len, mode: str, *, window: int = 0,
           n_sink: int = 0, alpha: float = 1.0, beta: float = 0.0, kappa: float = 0.0,
           n0: int = 1, softmax_scale: float | None = None, rope: str = "neox",
           rope_theta: float = 1e4, k_side=None, pairs=None, details: bool = False,
           fold_variant: str = "B"):
    """Decode attention of every draft query against its sequence's cache.

    Arguments follow the layouts in the module docstring. ``pairs`` optionally
    restricts work to a set of (b, kv_head) pairs; rows outside it are NaN.
    Returns a dict with ``out`` [B, T, Hq, d] and ``lse`` [B, T, Hq] (natural
    log), and with ``details=True`` a per-(b, kv_head) dict of index sets,
    weights, scale and partition log-sums.
    """
    if mode not in MODES:
        raise ValueError(f"unknown mode {mode!r}")
    q = np.asarray(q, dtype=np.float64)
    B, T, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    if k_cache.shape[2] * k_cache.shape[4] != d:
        raise ValueError("key pool layout must be [NB, Hkv, d/8, 16, 8]")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    out = np.full((B, T, Hq, d), np.nan)
    lse = np.full((B, T, Hq), np.nan)
    info = {}
    for b in range(B):
        L = int(ctx_len[b])
        main, far = index_sets(L, mode, window, n_sink)
        n = int(main.size + far.size)
        c = scale * query_scale(n, kappa, n0)
        row = block_table[b]
        for g in range(Hkv):
            if pairs is not None and (b, g) not in pairs:
                continue
            # R = T*G query rows of this kv head, row r = t*G + (h - g*G)
            Q = q[b, :, g * G:(g + 1) * G, :].reshape(T * G, d)
            K = gather_keys(k_cache, row, main, g)
            V = gather_values(v_cache, row, main, g)
            logits = c * (Q @ K.T)
            if mode == "fold":
                P_v = L - int(window) - 1
                Qf = rope_rotate(Q, -P_v, rope_theta) if rope == "neox" else Q
                U = gather_keys(k_side, row, far, g)
                Vf = gather_values(v_cache, row, far, g)
                phi = c * (Qf @ U.T)
                lse_L = _logsumexp(logits)
                lse_F = _logsumexp(phi)
                lse_Fa = _logsumexp(alpha * phi)
                # log of the far memory's total weight, per parameterisation
                far_mass = _far_log_mass(fold_variant, alpha, beta, lse_F, lse_Fa)
                tot = np.logaddexp(lse_L, far_mass)
                with np.errstate(invalid="ignore"):  # -inf - -inf only when a partition is empty
                    w_loc = np.exp(logits - tot[:, None])
                    w_far = np.exp(far_mass - tot)[:, None] * np.exp(alpha * phi - lse_Fa[:, None])
                o = w_loc @ V + w_far @ Vf
            else:
                tot = _logsumexp(logits)
                w_loc = np.exp(logits - tot[:, None])
                w_far = np.zeros((T * G, 0))
                lse_L, lse_F, lse_Fa = tot, np.full(T * G, -np.inf), np.full(T * G, -np.inf)
                o = w_loc @ V
            if n == 0:
                o = np.zeros((T * G, d))
            out[b, :, g * G:(g + 1) * G, :] = o.reshape(T, G, d)
            lse[b, :, g * G:(g + 1) * G] = tot.reshape(T, G)
            if details:
                info[(b, g)] = dict(main=main, far=far, scale=c, n=n, w_main=w_loc, w_far=w_far,
                                    lse_main=lse_L, lse_far=lse_F, lse_far_alpha=lse_Fa)
    res = dict(out=out, lse=lse)
    if details:
        res["details"] = info
    return res


# ----------------------------------------------------------------------------- cache append
def bf16_round(x) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even), returned as fp64.

    Written from the definition: with e = floor(log2|x|), bf16 spacing near x is
    2^(e-7); the two neighbours are exact dyadic numbers, so comparing distances
    in fp64 is exact. Zero stays zero; finite inputs in the normal range only.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    xs = x[nz]
    _, e = np.frexp(np.abs(xs))            # |x| = f * 2^e with f in [0.5, 1)
    ulp = np.ldexp(1.0, e - 8)              # 8 significant bits
    lo = np.floor(xs / ulp) * ulp
    hi = lo + ulp
    dlo, dhi = xs - lo, hi - xs
    lo_even = (np.floor(xs / ulp) % 2) == 0
    out[nz] = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo_even, lo, hi)))
    return out


def append(k_new, v_new, block_table, pos, k_cache, v_cache, k_side=None, rope: str = "neox",
           rope_theta: float = 1e4):
    """Write newly accepted tokens into the paged caches; returns updated copies.

    Token i of sequence b sits at position p = pos[b] + i, in block
    block_table[b, p // 16] at slot p % 16. The rotated cache receives the key
    turned to its own position, R(p) k, rounded to bf16; the side cache keeps the
    unrotated key for FOLD's far memory ("FOLD: Position-Free Far Memory with
    Local Order for Long-Context Speculative Decoding", review: the unrotated
    side cache and its bookkeeping); the value cache receives v. k_new, v_new:
    [B, n_new, Hkv, d] (bf16 values as fp64).
    """
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    B, n_new, Hkv, d = k_new.shape
    kc, vc = np.array(k_cache, dtype=np.float64), np.array(v_cache, dtype=np.float64)
    ks = None if k_side is None else np.array(k_side, dtype=np.float64)
    for b in range(B):
        for i in range(n_new):
            p = int(pos[b]) + i
            blk, slot = int(block_table[b][p // BLOCK]), p % BLOCK
            for h in range(Hkv):
                raw = k_new[b, i, h]
                rot = bf16_round(rope_rotate(raw, p, rope_theta)) if rope == "neox" else raw
                kc[blk, h, :, slot, :] = rot.reshape(d // 8, 8)
                if ks is not None:
                    ks[blk, h, :, slot, :] = raw.reshape(d // 8, 8)
                vc[blk, h, :, slot] = v_new[b, i, h]
    return kc, vc, ks


# ----------------------------------------------------------------------------- draft tokens
def decode_with_draft(q, k_cache, v_cache, block_table, ctx_len, mode: str, k_draft, v_draft, *,
                      window: int = 0, n_sink: int = 0, alpha: float = 1.0, beta: float = 0.0,
                      kappa: float = 0.0, n0: int = 1, softmax_scale: float | None = None,
                      rope: str = "neox", rope_theta: float = 1e4, k_side=None, fold_variant: str = "B"):
    """Cache attention plus causal attention among the draft tokens, as one softmax.

    Draft token t of sequence b also attends to the step's own draft keys
    k_draft[b, 0..t] (already rotated at their positions L_b + t'), which are not
    in the cache yet. They sit at exact positions next to the window, so for FOLD
    they join the local partition, and the far memory's log-weight is that of
    the chosen reading (``fold_variant``, as in ``decode``). Reading (no page
    states it): their logits use the same scale c = softmax_scale * s(n) as the
    cached keys, with n the cached visible count. q: [B, T, Hq, d]; k_draft,
    v_draft: [B, T, Hkv, d].
    """
    q = np.asarray(q, dtype=np.float64)
    kd = np.asarray(k_draft, dtype=np.float64)
    vd = np.asarray(v_draft, dtype=np.float64)
    B, T, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    out = np.zeros((B, T, Hq, d))
    lse = np.zeros((B, T, Hq))
    for b in range(B):
        L = int(ctx_len[b])
        main, far = index_sets(L, mode, window, n_sink)
        c = scale * query_scale(int(main.size + far.size), kappa, n0)
        row = block_table[b]
        for g in range(Hkv):
            K = gather_keys(k_cache, row, main, g)
            V = gather_values(v_cache, row, main, g)
            if mode == "fold":
                U = gather_keys(k_side, row, far, g)
                Vf = gather_values(v_cache, row, far, g)
            for t in range(T):
                Q = q[b, t, g * G:(g + 1) * G, :]                       # [G, d]
                Km = np.concatenate([K, kd[b, :t + 1, g, :]])           # main keys + draft keys <= t
                Vm = np.concatenate([V, vd[b, :t + 1, g, :]])
                logits = c * (Q @ Km.T)
                if mode == "fold":
                    Qf = rope_rotate(Q, -(L - int(window) - 1), rope_theta) if rope == "neox" else Q
                    phi = c * (Qf @ U.T)
                    lse_L, lse_F, lse_Fa = _logsumexp(logits), _logsumexp(phi), _logsumexp(alpha * phi)
                    mass = _far_log_mass(fold_variant, alpha, beta, lse_F, lse_Fa)
                    tot = np.logaddexp(lse_L, mass)
                    with np.errstate(invalid="ignore"):
                        w_far = np.exp(mass - tot)[:, None] * np.exp(alpha * phi - lse_Fa[:, None])
                    o = np.exp(logits - tot[:, None]) @ Vm + (w_far @ Vf if far.size else 0.0)
                else:
                    tot = _logsumexp(logits)
                    o = np.exp(logits - tot[:, None]) @ Vm
                out[b, t, g * G:(g + 1) * G] = o
                lse[b, t, g * G:(g + 1) * G] = tot
    return dict(out=out, lse=lse)

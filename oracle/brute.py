"""Brute-force decode attention in pure Python scalars (8-64 token inputs).

TEST INFRASTRUCTURE (see the package docstring). Written apart from
``oracle.reference`` -- membership predicates instead of range arithmetic,
per-element pool reads, complex-number RoPE, explicit per-key weights -- so the
two pin each other on tiny inputs. Same definitions and citations as
``oracle.reference``:
  [WMTP] "Windowed-MTP: Removing the Full-Context Draft-KV Tax at Million-Token
         Context", Abstract (window + sinks, paged KV, RoPE).
  [FOLD] "FOLD: Position-Free Far Memory with Local Order for Long-Context
         Speculative Decoding", summary and abstract (local window, shared-position
         far memory, decoupled softmax).
  [SD]   "SharpDraft: Accelerating Long-Context Speculative Decoding with
         Cardinality-Aware Query Scaling", Abstract (query scale by visible count).
"""

from __future__ import annotations

import cmath
import math


def _is_main(j: int, L: int, mode: str, W: int, S: int) -> bool:
    """Key j takes part in the main (rotated-cache) softmax."""
    if j < 0 or j >= L:
        return False
    if mode == "full":
        return True
    if mode == "window":
        return j < S or j >= L - W
    return j >= L - W  # fold: local window


def _is_far(j: int, L: int, mode: str, W: int) -> bool:
    return mode == "fold" and 0 <= j < L - W


def rotate(x, pos: float, theta: float):
    """NeoX RoPE as complex multiplication: z_i = x_i + i*x_{i+d/2}, z_i *= e^{i pos w_i}."""
    d = len(x)
    h = d // 2
    y = [0.0] * d
    for i in range(h):
        w = theta ** (-2.0 * i / d)
        z = complex(x[i], x[i + h]) * cmath.exp(1j * pos * w)
        y[i], y[i + h] = z.real, z.imag
    return y


def _key(pool, table, b, g, j, d):
    blk = int(table[b][j // 16])
    return [float(pool[blk][g][i // 8][j % 16][i % 8]) for i in range(d)]


def _val(pool, table, b, g, j, d):
    blk = int(table[b][j // 16])
    return [float(pool[blk][g][i][j % 16]) for i in range(d)]


def _dot(a, b):
    s = 0.0
    for x, y in zip(a, b):
        s += x * y
    return s


def decode(q, k_cache, v_cache, block_table, ctx_len, mode: str, *, window: int = 0,
           n_sink: int = 0, alpha: float = 1.0, beta: float = 0.0, kappa: float = 0.0,
           n0: int = 1, softmax_scale=None, rope: str = "neox", rope_theta: float = 1e4,
           k_side=None, fold_variant: str = "B"):
    """Return (out, lse, weights): nested lists out[b][t][h][i], lse[b][t][h] and
    weights[b][t][h] = {key: (partition, weight)} with partition 'main' or 'far'."""
    B, T, Hq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k_cache[0])
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    W, S = int(window), int(n_sink)
    out, lse, weights = [], [], []
    for b in range(B):
        L = int(ctx_len[b])
        mains = [j for j in range(L) if _is_main(j, L, mode, W, S)]
        fars = [j for j in range(L) if _is_far(j, L, mode, W)]
        n = len(mains) + len(fars)
        c = scale * (1.0 + kappa * math.log(max(n, n0) / n0))
        ob, lb, wb = [], [], []
        for t in range(T):
            ot, lt, wt = [], [], []
            for h in range(Hq):
                g = h // G
                qv = [float(q[b][t][h][i]) for i in range(d)]
                ell = {j: c * _dot(qv, _key(k_cache, block_table, b, g, j, d)) for j in mains}
                phi = {}
                if fars:
                    qf = rotate(qv, -(L - W - 1), rope_theta) if rope == "neox" else qv
                    phi = {j: c * _dot(qf, _key(k_side, block_table, b, g, j, d)) for j in fars}
                if n == 0:
                    ot.append([0.0] * d)
                    lt.append(-math.inf)
                    wt.append({})
                    continue
                w = {}
                if mode != "fold":
                    m = max(ell.values())
                    z = sum(math.exp(v - m) for v in ell.values())
                    log_den = m + math.log(z)
                    for j, v in ell.items():
                        w[j] = ("main", math.exp(v - log_den))
                else:
                    parts = []
                    if ell:
                        mL = max(ell.values())
                        parts.append(mL + math.log(sum(math.exp(v - mL) for v in ell.values())))
                    if phi:
                        mF = max(phi.values())
                        zF = sum(math.exp(v - mF) for v in phi.values())
                        zFa = sum(math.exp(alpha * (v - mF)) for v in phi.values())
                        if fold_variant == "A":      # joint softmax, far logits alpha*phi + beta
                            log_far_mass = beta + alpha * mF + math.log(zFa)
                        elif fold_variant == "B'":   # one virtual key, logit beta + ln(Z_Fa)/alpha
                            log_far_mass = beta + mF + math.log(zFa) / alpha
                        else:
                            log_far_mass = beta + mF + math.log(zF)
                        parts.append(log_far_mass)
                    top = max(parts)
                    log_den = top + math.log(sum(math.exp(p - top) for p in parts))
                    for j, v in ell.items():
                        w[j] = ("main", math.exp(v - log_den))
                    if phi:
                        far_share = math.exp(log_far_mass - log_den)
                        for j, v in phi.items():
                            w[j] = ("far", far_share * math.exp(alpha * (v - mF)) / zFa)
                o = [0.0] * d
                for j, (part, wj) in w.items():
                    vj = _val(v_cache, block_table, b, g, j, d)
                    for i in range(d):
                        o[i] += wj * vj[i]
                ot.append(o)
                lt.append(log_den)
                wt.append(w)
            ob.append(ot)
            lb.append(lt)
            wb.append(wt)
        out.append(ob)
        lse.append(lb)
        weights.append(wb)
    return out, lse, weights

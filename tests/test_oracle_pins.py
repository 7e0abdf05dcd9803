"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test names the fact it checks. None re-derives the oracle's own formula:
they use closed forms worked out by hand, an independently written brute
force (``oracle.brute``), textbook identities of rotations and softmax, and the
reductions that the pages state in words:
  - a window that covers the context is plain full attention
    ("Windowed-MTP: Removing the Full-Context Draft-KV Tax at Million-Token
    Context", Abstract: the window only drops keys);
  - FOLD with no sharpening (alpha = 1) and no reweighting (beta = 0) is one
    softmax over local and far keys ("FOLD: Position-Free Far Memory with Local
    Order for Long-Context Speculative Decoding", abstract and review);
  - kappa = 0 leaves the drafter unmodified ("SharpDraft: Accelerating
    Long-Context Speculative Decoding with Cardinality-Aware Query Scaling",
    Abstract).
"""

import math
import os

import numpy as np
import pytest

from oracle import brute, reference as ref

# tests/test_oracle_mutations.py runs this file against deliberately broken
# copies of oracle/reference.py (named by ORACLE_REFERENCE_PATH) and expects it
# to fail for each of them.
if os.environ.get("ORACLE_REFERENCE_PATH"):
    import importlib.util
    _spec = importlib.util.spec_from_file_location("oracle_reference_mutant", os.environ["ORACLE_REFERENCE_PATH"])
    ref = importlib.util.module_from_spec(_spec)
    _spec.loader.exec_module(ref)

BLOCK = 16


# ----------------------------------------------------------------------------- helpers
def paged(ctx_lens, Hkv, d, seed, side=False, shuffle=True, nan_pad=True, spare=2):
    """Small paged pools as fp64 NumPy arrays (bf16-representable values are not
    needed for oracle pins). Unused slots are NaN so stray reads poison results."""
    rng = np.random.default_rng(seed)
    nblk = [(L + BLOCK - 1) // BLOCK for L in ctx_lens]
    NB = sum(nblk) + spare
    MB = max(max(nblk), 1)
    perm = rng.permutation(NB) if shuffle else np.arange(NB)
    table = np.full((len(ctx_lens), MB), -1, dtype=np.int64)
    p = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[p:p + n]
        p += n
    k = rng.standard_normal((NB, Hkv, d // 8, BLOCK, 8))
    v = rng.standard_normal((NB, Hkv, d, BLOCK))
    ks = rng.standard_normal((NB, Hkv, d // 8, BLOCK, 8)) if side else None
    if nan_pad:
        for b, L in enumerate(ctx_lens):
            if L % BLOCK:
                blk = table[b, L // BLOCK]
                k[blk, :, :, L % BLOCK:, :] = np.nan
                v[blk, :, :, L % BLOCK:] = np.nan
                if side:
                    ks[blk, :, :, L % BLOCK:, :] = np.nan
        for blk in perm[sum(nblk):]:
            k[blk] = np.nan
            v[blk] = np.nan
            if side:
                ks[blk] = np.nan
    return k, v, ks, table


def repage(keys, vals, d):
    """Pack explicit per-key rows [n, d] into a fresh one-sequence, one-head pool."""
    n = keys.shape[0]
    nb = max((n + BLOCK - 1) // BLOCK, 1)
    k = key_pool(nb, 1, d)
    v = np.zeros((nb, 1, d, BLOCK))
    for j in range(n):
        put_key(k, j // BLOCK, 0, j % BLOCK, keys[j])
        v[j // BLOCK, 0, :, j % BLOCK] = vals[j]
    return k, v, np.arange(nb)[None, :]


def key_pool(nb, hkv, d):
    """Zero key pool in the library's layout [NB, Hkv, d/8, 16, 8]."""
    return np.zeros((nb, hkv, d // 8, BLOCK, 8))


def put_key(pool, blk, h, slot, vec):
    """Write key vector vec[d] into block blk, kv head h, slot: channel 8c + j -> [c, slot, j]."""
    d = len(vec)
    pool[blk, h, :, slot, :] = np.asarray(vec, dtype=float).reshape(d // 8, 8)


def logical_rows(pool_k, pool_v, table_row, g, L, d):
    """All L logical key/value rows of one sequence, read element by element."""
    K = np.array([[pool_k[table_row[j // BLOCK], g, i // 8, j % BLOCK, i % 8] for i in range(d)] for j in range(L)])
    V = np.array([[pool_v[table_row[j // BLOCK], g, i, j % BLOCK] for i in range(d)] for j in range(L)])
    return K.reshape(L, d), V.reshape(L, d)


# ----------------------------------------------------------------------------- index sets
@pytest.mark.parametrize("mode", ["full", "window", "fold"])
def test_index_sets_match_membership_predicates(mode):
    for L in list(range(0, 70)) + [255, 256, 257]:
        for W in (0, 1, 5, 16, 33, 100, 300):
            for S in ((0, 1, 4, 20) if mode == "window" else (0,)):
                main, far = ref.index_sets(L, mode, W, S)
                want_main = [j for j in range(L) if brute._is_main(j, L, mode, W, S)]
                want_far = [j for j in range(L) if brute._is_far(j, L, mode, W)]
                assert main.tolist() == want_main, (L, W, S)
                assert far.tolist() == want_far, (L, W, S)


def test_index_set_sizes_of_the_pages_workloads():
    # Window of 256 plus 4 sinks over 4096 keys.
    assert ref.visible_count(4096, "window", 256, 4) == 260
    # Window of 4096 plus 4 sinks at 2^20 keys keeps 4100 keys: about 99.6% dropped,
    # consistent with the Windowed-MTP abstract's "~99% at 1M".
    n = ref.visible_count(1 << 20, "window", 4096, 4)
    assert n == 4100 and 1 - n / (1 << 20) > 0.99
    # FOLD at 262144 with a 4096 window: 258048 far keys, 4096 local.
    main, far = ref.index_sets(262144, "fold", 4096)
    assert (main.size, far.size) == (4096, 258048)
    assert main[0] == far[-1] + 1
    # Sinks overlapping the window are not double counted.
    assert ref.visible_count(10, "window", 8, 4) == 10
    assert ref.visible_count(0, "window", 8, 4) == 0


# ----------------------------------------------------------------------------- query scale
def test_query_scale_closed_forms():
    assert ref.query_scale(10 ** 6, 0.0, 4096) == 1.0          # kappa = 0: unmodified drafter
    assert ref.query_scale(100, 0.37, 4096) == 1.0             # below n0: no scaling
    assert ref.query_scale(4096, 0.37, 4096) == 1.0
    assert abs(ref.query_scale(8 * 4096, 0.1, 4096) - (1 + 0.3 * math.log(2))) < 1e-15  # ln 8 = 3 ln 2
    assert abs(ref.query_scale(2 * 4096, 0.5, 4096) - (1 + 0.5 * math.log(2))) < 1e-15
    # fixed slope: s(2n) - s(n) = kappa ln 2 for n >= n0
    for n in (5000, 123456, 1 << 20):
        assert abs(ref.query_scale(2 * n, 0.2, 4096) - ref.query_scale(n, 0.2, 4096) - 0.2 * math.log(2)) < 1e-12


# ----------------------------------------------------------------------------- rotary positions
def test_rope_closed_forms():
    # d = 2: the single pair turns by pos radians (theta^0 = 1).
    for pos in (0.0, 0.5, -1.25, 3.0):
        y = ref.rope_rotate([1.0, 0.0], pos, 1e4)
        assert np.allclose(y, [math.cos(pos), math.sin(pos)], atol=1e-15)
        y = ref.rope_rotate([0.0, 1.0], pos, 1e4)
        assert np.allclose(y, [-math.sin(pos), math.cos(pos)], atol=1e-15)
    # d = 4, theta = 1e4: the second pair turns at 10^-2 rad per position.
    y = ref.rope_rotate([0.0, 1.0, 0.0, 0.0], 100.0, 1e4)
    assert np.allclose(y, [0.0, math.cos(1.0), 0.0, math.sin(1.0)], atol=1e-14)
    # position 0 is the identity
    x = np.random.default_rng(0).standard_normal(8)
    assert np.array_equal(ref.rope_rotate(x, 0.0, 5e5), x)


def test_rope_group_properties_and_complex_form():
    rng = np.random.default_rng(1)
    for d in (2, 8, 64, 128):
        x = rng.standard_normal(d)
        y = rng.standard_normal(d)
        for a, b in ((3.0, 7.0), (1e6 - 5, 2.5), (-40000.0, 1.0)):
            ra = ref.rope_rotate(x, a, 5e5)
            # norm preserved; R(b) R(a) = R(a + b); R(-a) R(a) = I
            assert abs(np.linalg.norm(ra) - np.linalg.norm(x)) < 1e-12
            assert np.allclose(ref.rope_rotate(ra, b, 5e5), ref.rope_rotate(x, a + b, 5e5), atol=1e-9)
            assert np.allclose(ref.rope_rotate(ra, -a, 5e5), x, atol=1e-9)
            # relative position: <R(a)x, R(b)y> = <x, R(b-a)y>
            lhs = ref.rope_rotate(x, a, 5e5) @ ref.rope_rotate(y, b, 5e5)
            rhs = x @ ref.rope_rotate(y, b - a, 5e5)
            assert abs(lhs - rhs) < 1e-8
            # complex-multiplication form of the same rotation
            assert np.allclose(ref.rope_rotate(x, a, 5e5), brute.rotate(list(x), a, 5e5), atol=1e-9)


# ----------------------------------------------------------------------------- hand-derived cases
def test_two_key_closed_form():
    # q = e0, keys e0 and e1 (d = 8, other channels 0), scale 1: logits (1, 0).
    d = 8
    k = key_pool(1, 1, d)
    put_key(k, 0, 0, 0, np.eye(d)[0])
    put_key(k, 0, 0, 1, np.eye(d)[1])
    v = np.zeros((1, 1, d, BLOCK)); v[0, 0, 0, 0] = 2; v[0, 0, 1, 1] = 4
    q = np.eye(d)[0].reshape(1, 1, 1, d)
    r = ref.decode(q, k, v, np.array([[0]]), [2], "full", softmax_scale=1.0)
    e = math.e
    assert abs(r["lse"][0, 0, 0] - math.log(e + 1)) < 1e-15
    assert np.allclose(r["out"][0, 0, 0], [2 * e / (e + 1), 4 / (e + 1)] + [0] * 6, atol=1e-15)


def test_fold_hand_example():
    # L = 3, W = 1: Loc = {2}, Far = {0, 1}. No rotation, scale 1, q = e0.
    # local logit 0; far logits (1, 0); alpha = 2, beta = -1.
    # Z_L = 1, Z_F = e + 1, Z_Fa = e^2 + 1, lse = ln(1 + (e + 1)/e) = ln(2 + 1/e).
    # out = (v2 + e^-1 (e+1) (e^2 v0 + v1)/(e^2 + 1)) / (2 + 1/e)
    d = 8
    k = key_pool(1, 1, d)
    ks = key_pool(1, 1, d)
    put_key(ks, 0, 0, 0, np.eye(d)[0])
    v = np.zeros((1, 1, d, BLOCK)); v[0, 0, 0, 0] = 1; v[0, 0, 1, 1] = 1; v[0, 0, :2, 2] = 3
    q = np.eye(d)[0].reshape(1, 1, 1, d)
    r = ref.decode(q, k, v, np.array([[0]]), [3], "fold", window=1, alpha=2.0, beta=-1.0,
                   softmax_scale=1.0, rope="none", k_side=ks)
    e = math.e
    den = 2 + 1 / e
    far = (e + 1) / e / (e * e + 1)
    want = (np.array([3.0, 3.0] + [0] * 6) + far * np.array([e * e, 1.0] + [0] * 6)) / den
    assert abs(r["lse"][0, 0, 0] - math.log(den)) < 1e-15
    assert np.allclose(r["out"][0, 0, 0], want, atol=1e-15)


def test_key_and_value_layouts():
    # Value: key j, channel i holds 1000 j + i. A window of one key picks key L - 1.
    d, L = 8, 21
    k = key_pool(2, 1, d); v = np.zeros((2, 1, d, BLOCK))
    for j in range(L):
        for i in range(d):
            v[j // BLOCK, 0, i, j % BLOCK] = 1000 * j + i
    q = np.zeros((1, 1, 1, d))
    r = ref.decode(q, k, v, np.array([[0, 1]]), [L], "window", window=1, n_sink=0)
    assert np.array_equal(r["out"][0, 0, 0], [20000 + i for i in range(d)])
    r = ref.decode(q, k, v, np.array([[1, 0]]), [L], "window", window=1, n_sink=0)
    assert np.array_equal(r["out"][0, 0, 0], [1000 * 4 + i for i in range(d)])  # block swap: key 20 -> blk 0 slot 4
    # Key: channel 8c + j of slot s sits at [c, s, j]; one key (slot 5 of block 0) with channel 11 set.
    d = 16
    k = key_pool(1, 1, d)
    k[0, 0, 1, 5, 3] = 2.0                      # channel 8*1 + 3 = 11 of slot 5
    v = np.zeros((1, 1, d, BLOCK)); v[0, 0, 0, :6] = np.arange(6)
    q = np.zeros((1, 1, 1, d)); q[0, 0, 0, 11] = 1.0
    r = ref.decode(q, k, v, np.array([[0]]), [6], "full", softmax_scale=1.0)
    # logits: 2 for key 5, 0 otherwise -> lse = ln(5 + e^2)
    assert abs(r["lse"][0, 0, 0] - math.log(5 + math.e ** 2)) < 1e-14


# ----------------------------------------------------------------------------- brute force
CASES = [
    dict(mode="full"),
    dict(mode="window", window=7, n_sink=3),
    dict(mode="window", window=20, n_sink=0),
    dict(mode="window", window=0, n_sink=5),
    dict(mode="full", kappa=0.3, n0=8),
    dict(mode="window", window=9, n_sink=2, kappa=-0.05, n0=4),
    dict(mode="fold", window=9, alpha=1.0, beta=0.0),
    dict(mode="fold", window=9, alpha=3.0, beta=-1.0),
    dict(mode="fold", window=5, alpha=0.5, beta=0.7, kappa=0.2, n0=8),
    dict(mode="fold", window=40, alpha=2.0, beta=0.0),
    dict(mode="fold", window=0, alpha=2.0, beta=-0.5),
    dict(mode="fold", window=9, alpha=4.0, beta=-1.0, rope="none"),
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_oracle_matches_brute_force(case):
    ctx = [37, 8, 0, 64, 21]
    Hkv, G, T, d = 2, 2, 2, 8
    k, v, ks, table = paged(ctx, Hkv, d, seed=7, side=True)
    q = np.random.default_rng(3).standard_normal((len(ctx), T, Hkv * G, d)) * 1.5
    args = dict(case)
    r = ref.decode(q, k, v, table, ctx, k_side=ks, rope_theta=100.0, details=True, **args)
    bo, bl, bw = brute.decode(q, k, v, table, ctx, k_side=ks, rope_theta=100.0, **args)
    for b, L in enumerate(ctx):
        for t in range(T):
            for h in range(Hkv * G):
                assert np.allclose(r["out"][b, t, h], bo[b][t][h], atol=1e-12, rtol=0), (b, t, h)
                if math.isinf(bl[b][t][h]):
                    assert r["lse"][b, t, h] == -math.inf
                else:
                    assert abs(r["lse"][b, t, h] - bl[b][t][h]) < 1e-12
        # weights: the same key sets and values, summing to 1
        for g in range(Hkv):
            det = r["details"][(b, g)]
            for t in range(T):
                for hl in range(G):
                    row = t * G + hl
                    w = bw[b][t][g * G + hl]
                    mains = sorted(j for j, (p, _) in w.items() if p == "main")
                    fars = sorted(j for j, (p, _) in w.items() if p == "far")
                    assert mains == det["main"].tolist() and fars == det["far"].tolist()
                    wm = np.array([w[j][1] for j in mains])
                    wf = np.array([w[j][1] for j in fars])
                    assert np.allclose(det["w_main"][row], wm, atol=1e-13)
                    assert np.allclose(det["w_far"][row], wf, atol=1e-13)
                    if L:
                        assert abs(det["w_main"][row].sum() + det["w_far"][row].sum() - 1) < 1e-12


# ----------------------------------------------------------------------------- closed-form special cases
@pytest.mark.parametrize("mode,kw", [("full", {}), ("window", dict(window=10, n_sink=3)),
                                     ("fold", dict(window=10, alpha=1.0, beta=0.0))])
def test_zero_query_gives_uniform_weights(mode, kw):
    ctx = [45, 13]
    d = 8
    k, v, ks, table = paged(ctx, 1, d, seed=11, side=True)
    q = np.zeros((2, 1, 2, d))
    r = ref.decode(q, k, v, table, ctx, mode, k_side=ks, **kw)
    for b, L in enumerate(ctx):
        main, far = ref.index_sets(L, mode, kw.get("window", 0), kw.get("n_sink", 0))
        idx = np.concatenate([main, far])
        _, V = logical_rows(k, v, table[b], 0, L, d)
        assert abs(r["lse"][b, 0, 0] - math.log(idx.size)) < 1e-13
        assert np.allclose(r["out"][b, 0, 1], V[idx].mean(axis=0), atol=1e-13)


def test_zero_query_fold_general_alpha_beta():
    # All logits 0: Z_L = nL, Z_F = Z_Fa = nF, lse = ln(nL + e^beta nF),
    # out = (sum_Loc v + e^beta nF mean_Far v) / (nL + e^beta nF) for any alpha.
    L, W, d = 50, 12, 8
    k, v, ks, table = paged([L], 1, d, seed=5, side=True)
    _, V = logical_rows(k, v, table[0], 0, L, d)
    for alpha, beta in ((1.0, 0.0), (3.0, -2.0), (0.25, 1.5)):
        r = ref.decode(np.zeros((1, 1, 1, d)), k, v, table, [L], "fold", window=W,
                       alpha=alpha, beta=beta, k_side=ks)
        nL, nF = W, L - W
        den = nL + math.exp(beta) * nF
        want = (V[L - W:].sum(axis=0) + math.exp(beta) * nF * V[:L - W].mean(axis=0)) / den
        assert abs(r["lse"][0, 0, 0] - math.log(den)) < 1e-13
        assert np.allclose(r["out"][0, 0, 0], want, atol=1e-13)


def test_single_key_and_constant_values():
    d = 8
    k, v, ks, table = paged([1, 30], 1, d, seed=2, side=True)
    q = np.random.default_rng(4).standard_normal((2, 3, 1, d))
    r = ref.decode(q, k, v, table, [1, 30], "full")
    K0, V0 = logical_rows(k, v, table[0], 0, 1, d)
    for t in range(3):
        assert np.allclose(r["out"][0, t, 0], V0[0], atol=1e-15)
        assert abs(r["lse"][0, t, 0] - q[0, t, 0] @ K0[0] / math.sqrt(d)) < 1e-14
    # constant values: out equals the constant whatever the weights
    vc = np.full_like(v, 2.5)
    for mode, kw in (("full", {}), ("window", dict(window=7, n_sink=2)),
                     ("fold", dict(window=7, alpha=3.0, beta=-0.5))):
        r = ref.decode(q, k, vc, table, [1, 30], mode, k_side=ks, **kw)
        assert np.allclose(r["out"], 2.5, atol=1e-13)


def test_empty_context():
    d = 8
    k, v, ks, table = paged([0, 5], 1, d, seed=2, side=True)
    q = np.ones((2, 1, 1, d))
    for mode, kw in (("full", {}), ("window", dict(window=3, n_sink=1)), ("fold", dict(window=3, alpha=2.0))):
        r = ref.decode(q, k, v, table, [0, 5], mode, k_side=ks, **kw)
        assert np.all(r["out"][0] == 0) and np.all(r["lse"][0] == -np.inf)
        assert np.all(np.isfinite(r["out"][1]))
    r = ref.decode(q, k, v, table, [0, 5], "window", window=0, n_sink=0)
    assert np.all(r["out"] == 0) and np.all(r["lse"] == -np.inf)


# ----------------------------------------------------------------------------- reductions the pages fix
def test_window_covering_context_is_full_attention():
    ctx = [33, 70, 5]
    d = 16
    k, v, _, table = paged(ctx, 2, d, seed=9)
    q = np.random.default_rng(1).standard_normal((3, 2, 4, d))
    full = ref.decode(q, k, v, table, ctx, "full")
    for W, S in ((70, 0), (1000, 4), (66, 4), (0, 70)):
        win = ref.decode(q, k, v, table, ctx, "window", window=W, n_sink=S)
        assert np.allclose(win["out"], full["out"], atol=1e-14)
        assert np.allclose(win["lse"], full["lse"], atol=1e-14)


def test_window_equals_full_attention_over_the_kept_keys():
    L, W, S, d = 90, 20, 4, 8
    k, v, _, table = paged([L], 1, d, seed=12)
    q = np.random.default_rng(2).standard_normal((1, 2, 3, d))
    K, V = logical_rows(k, v, table[0], 0, L, d)
    keep = [j for j in range(L) if j < S or j >= L - W]
    k2, v2, t2 = repage(K[keep], V[keep], d)
    win = ref.decode(q, k, v, table, [L], "window", window=W, n_sink=S)
    full = ref.decode(q, k2, v2, t2, [len(keep)], "full")
    assert np.allclose(win["out"], full["out"], atol=1e-14)
    assert np.allclose(win["lse"], full["lse"], atol=1e-14)


def test_fold_alpha1_beta0_no_rotation_same_cache_is_full_attention():
    ctx = [77, 19]
    d = 8
    k, v, _, table = paged(ctx, 2, d, seed=13)
    q = np.random.default_rng(5).standard_normal((2, 3, 4, d))
    full = ref.decode(q, k, v, table, ctx, "full")
    for W in (0, 10, 19, 50, 100):
        fold = ref.decode(q, k, v, table, ctx, "fold", window=W, alpha=1.0, beta=0.0, rope="none", k_side=k)
        assert np.allclose(fold["out"], full["out"], atol=1e-13)
        assert np.allclose(fold["lse"], full["lse"], atol=1e-13)


def test_fold_far_keys_sit_at_the_shared_position():
    # alpha = 1, beta = 0 with NeoX: FOLD equals full attention over a cache in which each
    # far key is its unrotated side key rotated to P_v = L - W - 1 (complex-form RoPE).
    L, W, d, theta = 60, 13, 8, 100.0
    k, v, ks, table = paged([L], 1, d, seed=21, side=True)
    q = np.random.default_rng(6).standard_normal((1, 2, 2, d))
    K, V = logical_rows(k, v, table[0], 0, L, d)
    U, _ = logical_rows(ks, v, table[0], 0, L, d)
    P_v = L - W - 1
    mat = np.array([brute.rotate(list(U[j]), P_v, theta) if j < L - W else K[j] for j in range(L)])
    k2, v2, t2 = repage(mat, V, d)
    fold = ref.decode(q, k, v, table, [L], "fold", window=W, alpha=1.0, beta=0.0, k_side=ks, rope_theta=theta)
    full = ref.decode(q, k2, v2, t2, [L], "full")
    assert np.allclose(fold["out"], full["out"], atol=1e-12)
    assert np.allclose(fold["lse"], full["lse"], atol=1e-12)


def test_fold_window_covering_context_is_full_attention():
    ctx = [30, 64]
    d = 8
    k, v, ks, table = paged(ctx, 1, d, seed=14, side=True)
    q = np.random.default_rng(8).standard_normal((2, 2, 2, d))
    full = ref.decode(q, k, v, table, ctx, "full")
    for alpha, beta in ((1.0, 0.0), (4.0, -1.0), (0.5, 2.0)):
        fold = ref.decode(q, k, v, table, ctx, "fold", window=64, alpha=alpha, beta=beta, k_side=ks)
        assert np.allclose(fold["out"], full["out"], atol=1e-14)
        assert np.allclose(fold["lse"], full["lse"], atol=1e-14)


def test_fold_partition_log_weights():
    # lse(beta) = logaddexp(lse_Loc, beta + lse_Far) with both sides computed as plain full
    # attention over re-paged caches (far side with the query rotated to -P_v); and lse does
    # not depend on alpha, which reshapes weights only inside the far memory.
    L, W, d, theta = 75, 16, 8, 1e4
    k, v, ks, table = paged([L], 1, d, seed=31, side=True)
    q = np.random.default_rng(9).standard_normal((1, 1, 1, d)) * 2
    K, V = logical_rows(k, v, table[0], 0, L, d)
    U, _ = logical_rows(ks, v, table[0], 0, L, d)
    kl, vl, tl = repage(K[L - W:], V[L - W:], d)
    kf, vf, tf = repage(U[:L - W], V[:L - W], d)
    qf = np.array(brute.rotate(list(q[0, 0, 0]), -(L - W - 1), theta)).reshape(1, 1, 1, d)
    lse_loc = ref.decode(q, kl, vl, tl, [W], "full", softmax_scale=1 / math.sqrt(d))["lse"][0, 0, 0]
    lse_far = ref.decode(qf, kf, vf, tf, [L - W], "full", softmax_scale=1 / math.sqrt(d))["lse"][0, 0, 0]
    for beta in (0.0, -1.0, 2.5):
        lses = []
        for alpha in (1.0, 2.0, 4.0, 0.3):
            r = ref.decode(q, k, v, table, [L], "fold", window=W, alpha=alpha, beta=beta, k_side=ks,
                           rope_theta=theta)
            lses.append(r["lse"][0, 0, 0])
        assert max(lses) - min(lses) < 1e-13
        assert abs(lses[0] - np.logaddexp(lse_loc, beta + lse_far)) < 1e-13


def test_fold_large_alpha_concentrates_on_the_best_far_key():
    L, W, d = 40, 4, 8
    k, v, ks, table = paged([L], 1, d, seed=41, side=True)
    q = np.random.default_rng(10).standard_normal((1, 1, 1, d))
    U, V = logical_rows(ks, v, table[0], 0, L, d)
    qf = ref.rope_rotate(q[0, 0, 0], -(L - W - 1), 1e4)
    phi = U[:L - W] @ qf
    best = int(np.argmax(phi))
    gap = np.sort(phi)[-1] - np.sort(phi)[-2]
    assert gap > 0.01
    # beta large: the far memory holds essentially all weight; alpha large: one key wins
    r = ref.decode(q, k, v, table, [L], "fold", window=W, alpha=20000.0, beta=60.0, k_side=ks,
                   softmax_scale=1.0)
    assert np.allclose(r["out"][0, 0, 0], V[best], atol=1e-9)


def test_kappa_zero_is_a_noop_and_scale_equals_query_multiplication():
    ctx = [50, 9000 // 100]
    d = 8
    k, v, ks, table = paged(ctx, 1, d, seed=15, side=True)
    q = np.random.default_rng(12).standard_normal((2, 2, 2, d))
    for mode, kw in (("full", {}), ("window", dict(window=16, n_sink=4)),
                     ("fold", dict(window=16, alpha=2.0, beta=-1.0))):
        base = ref.decode(q, k, v, table, ctx, mode, k_side=ks, **kw)
        zero = ref.decode(q, k, v, table, ctx, mode, k_side=ks, kappa=0.0, n0=3, **kw)
        assert np.array_equal(base["out"], zero["out"]) and np.array_equal(base["lse"], zero["lse"])
        # n below n0: s = 1
        big = ref.decode(q, k, v, table, ctx, mode, k_side=ks, kappa=0.7, n0=10 ** 6, **kw)
        assert np.array_equal(base["out"], big["out"])
        # kappa > 0 equals multiplying each sequence's queries by s(n) with kappa = 0
        kap = ref.decode(q, k, v, table, ctx, mode, k_side=ks, kappa=0.3, n0=4, **kw)
        qs = q.copy()
        for b, L in enumerate(ctx):
            n = len([j for j in range(L) if brute._is_main(j, L, mode, kw.get("window", 0), kw.get("n_sink", 0))
                     or brute._is_far(j, L, mode, kw.get("window", 0))])
            qs[b] *= 1 + 0.3 * math.log(max(n, 4) / 4)
        scaled = ref.decode(qs, k, v, table, ctx, mode, k_side=ks, **kw)
        assert np.allclose(kap["out"], scaled["out"], atol=1e-13)
        assert np.allclose(kap["lse"], scaled["lse"], atol=1e-13)


def test_gqa_head_mapping():
    # Query head h reads kv head h // G: give kv head g the constant value g + 1.
    ctx, Hkv, G, d = [20], 3, 4, 8
    k, v, _, table = paged(ctx, Hkv, d, seed=16, nan_pad=False)
    for g in range(Hkv):
        v[:, g] = g + 1
    q = np.random.default_rng(13).standard_normal((1, 2, Hkv * G, d))
    r = ref.decode(q, k, v, table, ctx, "full")
    for h in range(Hkv * G):
        assert np.allclose(r["out"][0, :, h], h // G + 1, atol=1e-13)


def test_block_table_shuffle_invariance():
    ctx = [70, 33]
    d = 8
    k, v, ks, table = paged(ctx, 2, d, seed=17, side=True)
    q = np.random.default_rng(14).standard_normal((2, 2, 4, d))
    perm = np.random.default_rng(99).permutation(k.shape[0])
    inv = np.argsort(perm)          # new block inv[p] holds old block p
    k2, v2, ks2 = k[perm], v[perm], ks[perm]
    t2 = np.where(table >= 0, inv[np.maximum(table, 0)], -1)
    for mode, kw in (("full", {}), ("window", dict(window=9, n_sink=2)), ("fold", dict(window=9, alpha=2.0))):
        a = ref.decode(q, k, v, table, ctx, mode, k_side=ks, **kw)
        bb = ref.decode(q, k2, v2, t2, ctx, mode, k_side=ks2, **kw)
        assert np.array_equal(a["out"], bb["out"]) and np.array_equal(a["lse"], bb["lse"])


# ----------------------------------------------------------------------------- cache append
def test_bf16_rounding_closed_forms():
    u = 2.0 ** -7                                    # bf16 spacing in [1, 2)
    cases = {1.0: 1.0, 1 + u / 2: 1.0, 1 + 3 * u / 2: 1 + 2 * u,        # ties go to even
             1 + u / 2 + 2 ** -30: 1 + u, 1 + u / 2 - 2 ** -30: 1.0,
             -(1 + 3 * u / 2): -(1 + 2 * u), 3.0 + 2 ** -20: 3.0, 0.0: 0.0,
             2 ** -100 * (1 + u / 2): 2 ** -100, 255.5: 256.0, 254.5: 254.0}
    for x, want in cases.items():
        assert ref.bf16_round(np.array([x]))[0] == want, x
    # agrees with torch's float32 -> bf16 rounding on float32-representable inputs
    import torch
    xs = np.random.default_rng(0).standard_normal(20000).astype(np.float32).astype(np.float64) * 7
    t = torch.from_numpy(xs.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(ref.bf16_round(xs), t)


def test_append_places_tokens_at_their_positions():
    # Tokens appended at positions pos[b] + i are read back at those logical positions,
    # the side cache holds the raw key, the rotated cache R(p) k rounded to bf16.
    rng = np.random.default_rng(3)
    Hkv, d, theta = 2, 16, 1e4
    lens = [5, 30]
    k, v, ks, table = paged([48, 48], Hkv, d, seed=4, side=True, nan_pad=False)
    kn = rng.standard_normal((2, 7, Hkv, d))
    vn = rng.standard_normal((2, 7, Hkv, d))
    kc, vc, ksc = ref.append(kn, vn, table, lens, k, v, ks, rope="neox", rope_theta=theta)
    for b, L in enumerate(lens):
        for h in range(Hkv):
            K, V = logical_rows(kc, vc, table[b], h, 48, d)
            U, _ = logical_rows(ksc, vc, table[b], h, 48, d)
            K0, V0 = logical_rows(k, v, table[b], h, 48, d)
            for i in range(7):
                p = L + i
                assert np.array_equal(U[p], kn[b, i, h]) and np.array_equal(V[p], vn[b, i, h])
                want = ref.bf16_round(np.array(brute.rotate(list(kn[b, i, h]), p, theta)))
                assert np.array_equal(K[p], want)
            untouched = [j for j in range(48) if not (L <= j < L + 7)]
            assert np.array_equal(K[untouched], K0[untouched]) and np.array_equal(V[untouched], V0[untouched])
    # no rotation: the rotated cache receives the raw key
    kc2, _, _ = ref.append(kn, vn, table, lens, k, v, None, rope="none")
    K, _ = logical_rows(kc2, vc, table[1], 0, 48, d)
    assert np.array_equal(K[30], kn[1, 0, 0])


def test_appended_cache_fold_reduces_to_full_attention():
    # A cache written by append: FOLD with alpha = 1, beta = 0 on (rotated cache, side
    # cache) equals full attention over a cache whose far keys are the side keys rotated
    # to the shared position -- the side cache really holds the unrotated keys.
    rng = np.random.default_rng(8)
    Hkv, d, theta, L = 1, 16, 1e4, 40
    k, v, ks, table = paged([L], Hkv, d, seed=9, side=True, nan_pad=False)
    kn = rng.standard_normal((1, L, Hkv, d))
    vn = rng.standard_normal((1, L, Hkv, d))
    kc, vc, ksc = ref.append(kn, vn, table, [0], k, v, ks, rope="neox", rope_theta=theta)
    q = rng.standard_normal((1, 2, 2, d))
    W = 9
    P_v = L - W - 1
    K, V = logical_rows(kc, vc, table[0], 0, L, d)
    U, _ = logical_rows(ksc, vc, table[0], 0, L, d)
    mat = np.array([brute.rotate(list(U[j]), P_v, theta) if j < L - W else K[j] for j in range(L)])
    k2, v2, t2 = repage(mat, V, d)
    fold = ref.decode(q, kc, vc, table, [L], "fold", window=W, alpha=1.0, beta=0.0, k_side=ksc, rope_theta=theta)
    full = ref.decode(q, k2, v2, t2, [L], "full")
    assert np.allclose(fold["out"], full["out"], atol=1e-12) and np.allclose(fold["lse"], full["lse"], atol=1e-12)


# ----------------------------------------------------------------------------- draft tokens
def _draft_inputs(ctx, T, Hkv, G, d, seed):
    k, v, ks, table = paged(ctx, Hkv, d, seed=seed, side=True, nan_pad=False, spare=4)
    rng = np.random.default_rng(seed + 1)
    q = rng.standard_normal((len(ctx), T, Hkv * G, d))
    kd = rng.standard_normal((len(ctx), T, Hkv, d))
    vd = rng.standard_normal((len(ctx), T, Hkv, d))
    return k, v, ks, table, q, kd, vd


def test_draft_tokens_equal_decode_over_the_extended_cache():
    # Token t's result equals plain decode over the cache with draft keys 0..t
    # appended as cache entries (kappa = 0, so the visible count does not matter).
    ctx, T, Hkv, G, d = [37, 13], 3, 2, 2, 8        # draft positions L..L+2 stay inside allocated blocks
    k, v, ks, table, q, kd, vd = _draft_inputs(ctx, T, Hkv, G, d, seed=51)
    assert all(table[b, (L + T - 1) // BLOCK] >= 0 for b, L in enumerate(ctx))
    # FOLD under each reading of alpha/beta: the draft keys join the local
    # partition, so the far memory's log-weight is the reading's own.
    for mode, kw in (("full", {}), ("window", dict(window=9, n_sink=2)), ("fold", dict(window=9, alpha=2.0, beta=-1.0)),
                     ("fold", dict(window=9, alpha=2.0, beta=-1.0, fold_variant="A")),
                     ("fold", dict(window=9, alpha=0.5, beta=0.7, fold_variant="B'"))):
        res = ref.decode_with_draft(q, k, v, table, ctx, mode, kd, vd, k_side=ks, rope_theta=100.0, **kw)
        for b, L in enumerate(ctx):
            for t in range(T):
                k2, v2, ks2 = k.copy(), v.copy(), ks.copy()
                for tt in range(t + 1):         # write draft key tt at position L + tt
                    p = L + tt
                    for h in range(Hkv):
                        put_key(k2, table[b, p // BLOCK], h, p % BLOCK, kd[b, tt, h])
                        put_key(ks2, table[b, p // BLOCK], h, p % BLOCK, np.full(d, np.nan))
                        v2[table[b, p // BLOCK], h, :, p % BLOCK] = vd[b, tt, h]
                # the window / local window grows with the appended keys: W + t + 1
                kw2 = dict(kw)
                if "window" in kw2:
                    kw2["window"] = kw["window"] + t + 1
                r2 = ref.decode(q[b:b + 1, t:t + 1], k2, v2, table[b:b + 1], [L + t + 1], mode, k_side=ks2,
                                rope_theta=100.0, **kw2)
                # (FOLD's shared far position is unchanged: L + t + 1 - (W + t + 1) - 1 = L - W - 1)
                assert np.allclose(res["out"][b, t], r2["out"][0, 0], atol=1e-12), (mode, b, t)
                assert np.allclose(res["lse"][b, t], r2["lse"][0, 0], atol=1e-12), (mode, b, t)


def test_draft_tokens_on_an_empty_cache_are_causal_attention():
    T, Hkv, G, d = 4, 1, 2, 8
    k, v, ks, table, q, kd, vd = _draft_inputs([0], T, Hkv, G, d, seed=52)
    res = ref.decode_with_draft(q, k, v, table, [0], "full", kd, vd, softmax_scale=0.5)
    for t in range(T):
        for h in range(G):
            logits = [0.5 * q[0, t, h] @ kd[0, j, 0] for j in range(t + 1)]
            m = max(logits)
            z = sum(math.exp(x - m) for x in logits)
            want = sum(math.exp(x - m) / z * vd[0, j, 0] for j, x in enumerate(logits))
            assert np.allclose(res["out"][0, t, h], want, atol=1e-13)
            assert abs(res["lse"][0, t, h] - (m + math.log(z))) < 1e-13


def test_draft_tokens_keep_the_cached_visible_count_for_kappa():
    # Reading: the query scale uses the cached visible count n, not n + t + 1.
    ctx, T, Hkv, G, d = [50], 2, 1, 1, 8
    k, v, ks, table, q, kd, vd = _draft_inputs(ctx, T, Hkv, G, d, seed=53)
    s = ref.query_scale(50, 0.4, 4)
    a = ref.decode_with_draft(q, k, v, table, ctx, "full", kd, vd, kappa=0.4, n0=4)
    b_ = ref.decode_with_draft(q * s, k, v, table, ctx, "full", kd, vd)
    assert np.allclose(a["out"], b_["out"], atol=1e-13) and np.allclose(a["lse"], b_["lse"], atol=1e-13)


# ----------------------------------------------------------------------------- FOLD parameterisations
@pytest.mark.parametrize("variant", ["A", "B'"])
def test_fold_variants_match_brute_force(variant):
    ctx = [37, 8, 64, 21]
    Hkv, G, T, d = 2, 2, 2, 8
    k, v, ks, table = paged(ctx, Hkv, d, seed=17, side=True)
    q = np.random.default_rng(23).standard_normal((len(ctx), T, Hkv * G, d)) * 1.5
    for alpha, beta, W in ((1.0, 0.0, 9), (3.0, -1.0, 9), (0.5, 0.7, 5), (2.0, 0.0, 0)):
        kw = dict(window=W, alpha=alpha, beta=beta, k_side=ks, rope_theta=100.0, fold_variant=variant)
        r = ref.decode(q, k, v, table, ctx, "fold", **kw)
        bo, bl, _ = brute.decode(q, k, v, table, ctx, "fold", **kw)
        assert np.allclose(r["out"], np.array(bo), atol=1e-12)
        assert np.allclose(r["lse"], np.array(bl), atol=1e-12)


def test_fold_variants_reduce_to_the_union_softmax_and_hand_values():
    ctx = [60, 30]
    d = 8
    k, v, ks, table = paged(ctx, 1, d, seed=18, side=True)
    q = np.random.default_rng(24).standard_normal((2, 2, 2, d))
    base = ref.decode(q, k, v, table, ctx, "fold", window=10, alpha=1.0, beta=0.0, k_side=ks)
    for variant in ("A", "B'"):
        r = ref.decode(q, k, v, table, ctx, "fold", window=10, alpha=1.0, beta=0.0, k_side=ks, fold_variant=variant)
        assert np.allclose(r["out"], base["out"], atol=1e-13) and np.allclose(r["lse"], base["lse"], atol=1e-13)
    # Hand example of test_fold_hand_example (local logit 0, far logits 1 and 0, alpha 2, beta -1):
    #   A:  lse = ln(1 + e^-1 (e^2 + 1)),  B': lse = ln(1 + e^-1 (e^2 + 1)^(1/2))
    e = math.e
    kk = key_pool(1, 1, 8)
    kside = key_pool(1, 1, 8)
    put_key(kside, 0, 0, 0, np.eye(8)[0])
    vv = np.zeros((1, 1, 8, BLOCK)); vv[0, 0, 0, 0] = 1; vv[0, 0, 1, 1] = 1; vv[0, 0, :2, 2] = 3
    qq = np.eye(8)[0].reshape(1, 1, 1, 8)
    for variant, mass in (("A", (e * e + 1) / e), ("B'", math.sqrt(e * e + 1) / e)):
        r = ref.decode(qq, kk, vv, np.array([[0]]), [3], "fold", window=1, alpha=2.0, beta=-1.0, softmax_scale=1.0,
                       rope="none", k_side=kside, fold_variant=variant)
        assert abs(r["lse"][0, 0, 0] - math.log(1 + mass)) < 1e-14
        far_out = np.array([e * e, 1.0] + [0] * 6) / (e * e + 1)
        want = (np.array([3.0, 3.0] + [0] * 6) + mass * far_out) / (1 + mass)
        assert np.allclose(r["out"][0, 0, 0], want, atol=1e-14)

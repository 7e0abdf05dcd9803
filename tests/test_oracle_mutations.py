"""The oracle's pins catch plausible mistakes: each case below plants one
mistake in a copy of oracle/reference.py (on the CPU) and runs the pin suite
(tests/test_oracle_pins.py) against that copy, which must fail."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "reference.py")

# (name, text in oracle/reference.py, replacement)
MUTATIONS = [
    ("window start off by one", "recent = np.arange(max(0, L - int(window)), L", "recent = np.arange(max(0, L - int(window) + 1), L"),
    ("one sink too many", "sinks = np.arange(min(int(n_sink), L)", "sinks = np.arange(min(int(n_sink) + 1, L)"),
    ("fold boundary off by one", "start = max(0, L - int(window))", "start = max(0, L - int(window) - 1)"),
    ("shared position off by one", "P_v = L - int(window) - 1\n", "P_v = L - int(window)\n"),
    ("far query rotated the wrong way", "Qf = rope_rotate(Q, -P_v, rope_theta)", "Qf = rope_rotate(Q, P_v, rope_theta)"),
    ("rope frequency exponent", "omega = float(theta) ** (-2.0 * np.arange(h", "omega = float(theta) ** (-1.0 * np.arange(h"),
    ("rope pair sign", "x1 * sin + x2 * cos], axis=-1)", "x1 * sin - x2 * cos], axis=-1)"),
    ("rope pairs adjacent channels", "x1, x2 = x[..., :h], x[..., h:]", "x1, x2 = x[..., 0::2], x[..., 1::2]"),
    ("beta dropped", 'return {"B": beta + lse_F,', 'return {"B": lse_F,'),
    ("alpha leaks into the far mass", 'return {"B": beta + lse_F,', 'return {"B": beta + lse_Fa,'),
    ("far weights not normalised by Z_Fa", "np.exp(alpha * phi - lse_Fa[:, None])\n                o = w_loc", "np.exp(alpha * phi - lse_F[:, None])\n                o = w_loc"),
    ("variant A with the unsharpened mass", '"A": beta + lse_Fa,', '"A": beta + lse_F,'),
    ("variant B' without the 1/alpha", '"B\'": beta + lse_Fa / alpha}', '"B\'": beta + lse_Fa}'),
    ("visible count ignores the window", "n = int(main.size + far.size)\n        c = scale", "n = L\n        c = scale"),
    ("query scale without log", "return 1.0 + float(kappa) * math.log(max(int(n), int(n0)) / int(n0))",
     "return 1.0 + float(kappa) * (max(int(n), int(n0)) / int(n0) - 1)"),
    ("GQA head map h % Hkv", "Q = q[b, :, g * G:(g + 1) * G, :].reshape(T * G, d)", "Q = q[b, :, g::Hkv, :].reshape(T * G, d)"),
    ("slot from the block index", "return np.asarray(pool[blocks, kvh, :, idx % BLOCK], dtype=np.float64)",
     "return np.asarray(pool[blocks, kvh, :, (idx + 1) % BLOCK], dtype=np.float64)"),
    ("key channel groups swapped", "rows = pool[blocks, kvh, :, idx % BLOCK, :]          # [n, d/8, 8]",
     "rows = pool[blocks, kvh, :, idx % BLOCK, :][:, ::-1, :]"),
    ("softmax scale 1/d", "scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)\n    out = np.full",
     "scale = 1.0 / d if softmax_scale is None else float(softmax_scale)\n    out = np.full"),
    ("empty set gives NaN", "if n == 0:\n                o = np.zeros((T * G, d))", "if n == 0:\n                o = np.full((T * G, d), np.nan)"),
    ("bf16 ties away from even", "np.where(lo_even, lo, hi)", "np.where(lo_even, hi, lo)"),
    ("append rotates to p + 1", "rot = bf16_round(rope_rotate(raw, p, rope_theta))", "rot = bf16_round(rope_rotate(raw, p + 1, rope_theta))"),
    ("draft step ignores the FOLD reading", " mass = _far_log_mass(fold_variant,", ' mass = _far_log_mass("B",'),
    ("draft token sees only earlier drafts", "Km = np.concatenate([K, kd[b, :t + 1, g, :]])", "Km = np.concatenate([K, kd[b, :t, g, :]])"),
]


def test_every_mutation_text_is_present():
    src = open(SRC).read()
    for name, old, _ in MUTATIONS:
        assert src.count(old) == 1, name


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_the_mutation(tmp_path, name, old, new):
    src = open(SRC).read()
    mutant = tmp_path / "reference_mutant.py"
    mutant.write_text(src.replace(old, new))
    env = dict(os.environ, ORACLE_REFERENCE_PATH=str(mutant))
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    assert res.returncode != 0, f"the pins did not catch: {name}\n{res.stdout[-2000:]}"


def test_unmodified_copy_passes(tmp_path):
    # Control: the same mechanism on an exact copy must pass, so the failures above
    # come from the planted mistakes and not from loading the copy.
    copy = tmp_path / "reference_copy.py"
    copy.write_text(open(SRC).read())
    env = dict(os.environ, ORACLE_REFERENCE_PATH=str(copy))
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                          os.path.join(ROOT, "tests", "test_golden.py")],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    assert res.returncode == 0, res.stdout[-2000:]

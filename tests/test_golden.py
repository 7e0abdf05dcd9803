"""The oracle against hand-worked cases with closed-form results
(``tests/golden/closed_forms.json``; each case carries its derivation and the
page it follows). Both implementations, NumPy and pure Python, must reproduce
every case to 1e-12."""

import json
import math
import os

import numpy as np
import pytest

from oracle import brute, reference as ref

# Like the pins, this file can run against a deliberately broken copy of the
# NumPy oracle (tests/test_oracle_mutations.py).
if os.environ.get("ORACLE_REFERENCE_PATH"):
    import importlib.util
    _spec = importlib.util.spec_from_file_location("oracle_reference_mutant", os.environ["ORACLE_REFERENCE_PATH"])
    ref = importlib.util.module_from_spec(_spec)
    _spec.loader.exec_module(ref)

HERE = os.path.dirname(os.path.abspath(__file__))
CASES = json.load(open(os.path.join(HERE, "golden", "closed_forms.json")))["cases"]
D = 8
NAMES = {"ln": math.log, "sqrt": math.sqrt, "exp": math.exp, "cos": math.cos, "sin": math.sin, "e": math.e}


def val(x):
    """A number or a closed-form expression of the fixture."""
    if isinstance(x, (int, float)):
        return float(x)
    return float(eval(x, {"__builtins__": {}}, NAMES))  # fixture expressions only: arithmetic and NAMES


def rows(spec, L):
    m = np.zeros((L, D))
    for j, chans in (spec or {}).items():
        for c, x in chans.items():
            m[int(j), int(c)] = val(x)
    return m


def pools(case):
    L = case["L"]
    keys, side = rows(case.get("keys"), L), rows(case.get("side"), L)
    k = np.zeros((1, 1, D // 8, 16, 8))
    ks = np.zeros_like(k)
    v = np.zeros((1, 1, D, 16))
    for j in range(L):
        k[0, 0, :, j, :] = keys[j].reshape(D // 8, 8)
        ks[0, 0, :, j, :] = side[j].reshape(D // 8, 8)
        v[0, 0, 0, j] = j
        v[0, 0, 1, j] = 1.0
    q = np.zeros((1, 1, 1, D))
    for c, x in case["q"].items():
        q[0, 0, 0, int(c)] = val(x)
    return q, k, v, ks


def kwargs(case):
    return dict(window=case.get("window", 0), n_sink=case.get("n_sink", 0), alpha=val(case.get("alpha", 1.0)),
                beta=val(case.get("beta", 0.0)), kappa=val(case.get("kappa", 0.0)), n0=case.get("n0", 1),
                softmax_scale=1.0, rope=case.get("rope", "neox"), rope_theta=case.get("rope_theta", 1e4),
                fold_variant=case.get("fold_variant", "B"))


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_numpy_oracle_reproduces_the_closed_form(case):
    q, k, v, ks = pools(case)
    r = ref.decode(q, k, v, np.zeros((1, 1), dtype=np.int64), [case["L"]], case["mode"],
                   k_side=ks if case["mode"] == "fold" else None, **kwargs(case))
    out, lse = r["out"][0, 0, 0], float(r["lse"][0, 0, 0])
    assert abs(lse - val(case["expect"]["lse"])) < 1e-12, (lse, case["expect"]["lse"])
    assert abs(out[0] - val(case["expect"]["out0"])) < 1e-12, (out[0], case["expect"]["out0"])
    assert abs(out[1] - 1.0) < 1e-12 and np.all(out[2:] == 0.0)


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_brute_force_oracle_reproduces_the_closed_form(case):
    q, k, v, ks = pools(case)
    out, lse, _ = brute.decode(q.tolist(), k.tolist(), v.tolist(), [[0]], [case["L"]], case["mode"],
                               k_side=ks.tolist() if case["mode"] == "fold" else None, **kwargs(case))
    assert abs(lse[0][0][0] - val(case["expect"]["lse"])) < 1e-12
    assert abs(out[0][0][0][0] - val(case["expect"]["out0"])) < 1e-12
    assert abs(out[0][0][0][1] - 1.0) < 1e-12

"""Pins of the epilogue oracle (oracle/epilogue.py) against what the pages'
output equation fixes ([KDA-blog] "Kimi k3 技术报告详解（1）——架构再升华",
section "Gated MLA"): a hand-worked example, closed forms of RMSNorm and the
sigmoid gate, and invariances. Planted mistakes in a copy of the oracle
source must each fail at least one pin."""
import inspect
import json
import os

import numpy as np
import pytest

import oracle.epilogue as epi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gated_rmsnorm_worked.json")


def _pins(f):
    """Run every pin against the function `f`; raises AssertionError on the first miss."""
    ex = json.load(open(GOLDEN))
    y = f(np.array(ex["o"]), np.array(ex["gate_logits"]), np.array(ex["weight"]), ex["eps"])
    np.testing.assert_allclose(y, ex["y"], rtol=1e-14)
    # RMSNorm of a constant vector is its sign (eps = 0); sigmoid(50) = 1 to fp64
    for c in (3.5, -0.25):
        y = f(np.full((2, 7), c), np.full((2, 7), 50.0), None, 0.0)
        np.testing.assert_allclose(y, np.sign(c) * np.ones((2, 7)), rtol=1e-14)
    rng = np.random.default_rng(3)
    o = rng.standard_normal((4, 3, 16))
    z = rng.standard_normal((4, 3, 16))
    w = rng.standard_normal(16)
    # positive scale invariance and oddness (eps = 0)
    np.testing.assert_allclose(f(5.0 * o, z, w, 0.0), f(o, z, w, 0.0), rtol=1e-13)
    np.testing.assert_allclose(f(-o, z, w, 0.0), -f(o, z, w, 0.0), rtol=1e-13)
    # unit root-mean-square before gate and weight
    y = f(o, np.full_like(z, 50.0), None, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-13)
    # zero gate logits halve; a very negative logit closes the gate
    np.testing.assert_allclose(f(o, np.zeros_like(z), w, 0.0), 0.5 * f(o, np.full_like(z, 50.0), w, 0.0),
                               rtol=1e-13)
    assert np.all(np.abs(f(o, np.full_like(z, -800.0), w, 0.0)) == 0.0)
    # eps: a zero vector stays zero; eps shrinks small vectors as mean(o^2)/(mean(o^2)+eps)
    assert np.all(f(np.zeros((2, 8)), np.zeros((2, 8)), None, 1e-6) == 0.0)
    small = np.full((1, 8), 1e-3)
    np.testing.assert_allclose(f(small, np.full((1, 8), 50.0), None, 1e-6),
                               1e-3 / np.sqrt(1e-6 + 1e-6), rtol=1e-13)


def test_oracle_meets_every_pin():
    _pins(epi.oracle_gated_rmsnorm)


MUTANTS = [
    ("mean -> sum", "np.mean(o64 * o64, axis=-1, keepdims=True)", "np.sum(o64 * o64, axis=-1, keepdims=True)"),
    ("no sqrt", "np.sqrt(mean_sq + eps)", "(mean_sq + eps)"),
    ("eps outside root", "np.sqrt(mean_sq + eps)", "(np.sqrt(mean_sq) + eps)"),
    ("gate sign", "np.exp(-z64)", "np.exp(z64)"),
    ("weight ignored", "normed = normed * _f64(weight)", "normed = normed"),
    ("gate ignored", "return gate * normed", "return normed"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new):
    src = inspect.getsource(epi)
    assert src.count(old) == 1, name
    ns = {}
    exec(compile(src.replace(old, new), "mutant_epilogue", "exec"), ns)
    with pytest.raises(AssertionError):
        _pins(ns["oracle_gated_rmsnorm"])

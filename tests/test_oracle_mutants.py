"""The pins must catch plausible mistakes in the oracle.

Each case copies ``oracle/kda_oracle.c``, plants one mistake (a dropped term,
a wrong sign or index, a transposed operand, an off-by-one in the cumulative
decay), builds the mutant on the CPU and checks that at least one pin rejects
it. The committed oracle itself is never modified.
"""
import os
import subprocess
import tempfile

import numpy as np
import pytest
from scipy.special import expit

import oracle.oracle as orc

SRC = os.path.join(os.path.dirname(orc.__file__), "kda_oracle.c")

MUTANTS = {
    "no_decay": ("S[i * Dv + j] *= a;", ";"),
    "decay_reciprocal": ("double a = exp(gt[i]);", "double a = exp(-gt[i]);"),
    "delta_sign": ("u[j] = bt * (vt[j] - u[j]);", "u[j] = bt * (vt[j] + u[j]);"),
    "beta_on_old_only": ("u[j] = bt * (vt[j] - u[j]);", "u[j] = vt[j] - bt * u[j];"),
    "retrieve_with_query": ("u[j] += S[i * Dv + j] * kt[i];", "u[j] += S[i * Dv + j] * qt[i];"),
    "transposed_readout": ("ot[j] += S[i * Dv + j] * qt[i];", "ot[j] += S[j * Dv + i] * qt[i];"),
    "write_dropped": ("S[i * Dv + j] += kt[i] * u[j];", "S[i * Dv + j] += 0.0 * kt[i] * u[j];"),
    "read_before_write": None,  # output read from S_{t-1} (steps 4 and 5 swapped)
    "scale_ignored": ("for (int j = 0; j < Dv; ++j) ot[j] *= scale;", ""),
    "beta_wrong_head": ("jb->beta + t0 * H + h, H", "jb->beta + t0 * H, H"),
    "gate_drops_exp_A": ("g[i] = g_min * sigmoid(scale * z[i]);", "g[i] = g_min * sigmoid(z[i]);"),
    "gate_sign": ("g[i] = g_min * sigmoid(scale * z[i]);", "g[i] = g_min * sigmoid(-scale * z[i]);"),
    "cumsum_exclusive": ("run += g[i];\n          out[i] = run;", "out[i] = run;\n          run += g[i];"),
    "cumsum_no_restart": ("if ((t - cu[n]) % chunk == 0) run = 0.0;", ""),
    "initial_state_ignored": ("memcpy(S, jb->h0 + (size_t)unit * ssz, sizeof(double) * ssz);",
                              "memset(S, 0, sizeof(double) * ssz);"),
}


def _swap_write_and_read(src):
    i4 = src.index("    /* 4. S += k d^T */")
    i5 = src.index("    /* 5. o = scale * S^T q */")
    end = src.index("  }\n  free(u);")
    return src[:i4] + src[i5:end] + src[i4:i5] + src[end:]


def _build_mutant(name, tmpdir):
    src = open(SRC).read()
    if MUTANTS[name] is None:
        mutated = _swap_write_and_read(src)
    else:
        old, new = MUTANTS[name]
        assert src.count(old) == 1, f"mutation anchor for {name} not unique/present"
        mutated = src.replace(old, new)
    assert mutated != src
    path = os.path.join(tmpdir, f"{name}.c")
    open(path, "w").write(mutated)
    so = os.path.join(tmpdir, f"lib_{name}.so")
    subprocess.run(["gcc", "-O2", "-std=gnu99", "-shared", "-fPIC", path, "-o", so, "-lm",
                    "-lpthread"], check=True)
    return so


def _pins(lib):
    """Run a compact set of the pins against the library at `lib`; return the
    names of the pins that fail."""
    import json
    from tests.test_oracle_pins import GOLDEN, _brute_force_unit, _rand_problem
    from tests.chunk_mirror import chunk_form_pages
    failed = []

    def check(name, ok):
        if not ok:
            failed.append(name)

    # hand-worked example
    spec = json.load(open(os.path.join(GOLDEN, "hand_worked_recurrence.json")))
    x = {k: np.array(v) for k, v in spec["inputs"].items()}
    o, S = orc.oracle_recurrence(x["q"][None, :, None], x["k"][None, :, None],
                                 x["v"][None, :, None], np.log(x["alpha"])[None, :, None],
                                 x["beta"][None, :, None], lib_path=lib)
    check("hand", np.allclose(o[0, :, 0], spec["expected"]["o"], atol=1e-12)
          and np.allclose(S[0, 0], spec["expected"]["final_state"], atol=1e-12))
    # brute force with initial state and two heads
    rng = np.random.default_rng(1)
    q, k, v, g, beta = _rand_problem(rng, 1, 9, 2, 5, 5)
    S0 = rng.standard_normal((1, 2, 5, 5))
    o, S = orc.oracle_recurrence(q, k, v, g, beta, S0, lib_path=lib)
    ok = True
    for h in range(2):
        o_ref, S_ref = _brute_force_unit(q[0, :, h], k[0, :, h], v[0, :, h], g[0, :, h],
                                         beta[0, :, h], S0[0, h])
        ok &= np.allclose(o[0, :, h], o_ref, atol=1e-10) and np.allclose(S[0, h], S_ref, atol=1e-10)
    check("brute", ok)
    # scale is a plain factor
    o2, _ = orc.oracle_recurrence(q, k, v, g, beta, S0, scale=0.5, lib_path=lib)
    check("scale", np.allclose(o2, 0.5 * o, atol=1e-13))
    # gate closed forms
    gspec = json.load(open(os.path.join(GOLDEN, "gate_closed_forms.json")))
    ok = True
    for c in gspec["cases"]:
        gv = orc.oracle_gate(np.full((1, 1, 1, 1), c["z"]), np.array([c["A"]]), gspec["g_min"],
                             lib_path=lib)
        ok &= abs(gv.item() - c["g"]) < 1e-12
    check("gate", ok)
    # cumsum vs numpy per chunk (dense, two chunks per sequence)
    gg = rng.standard_normal((2, 40, 1, 3))
    cs = orc.oracle_cumsum(gg, 16, lib_path=lib)
    ref = np.concatenate([np.cumsum(gg[:, s:s + 16], axis=1) for s in range(0, 40, 16)], axis=1)
    check("cumsum", np.allclose(cs, ref, atol=1e-12))
    # chunk form of the pages
    qq, kk, vv, g2, b2 = _rand_problem(rng, 1, 40, 1, 6, 4)
    oo, SS = orc.oracle_recurrence(qq, kk, vv, g2, b2, lib_path=lib)
    oc, Sc = chunk_form_pages(qq[0, :, 0], kk[0, :, 0], vv[0, :, 0], g2[0, :, 0], b2[0, :, 0],
                              np.zeros((6, 4)), 16)
    check("chunk_form", np.allclose(oo[0, :, 0], oc, atol=1e-10) and np.allclose(SS[0, 0], Sc, atol=1e-10))
    return failed


def test_unmutated_oracle_passes_compact_pins():
    with tempfile.TemporaryDirectory() as d:
        so = os.path.join(d, "lib_clean.so")
        subprocess.run(["gcc", "-O2", "-std=gnu99", "-shared", "-fPIC", SRC, "-o", so, "-lm",
                        "-lpthread"], check=True)
        assert _pins(so) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    with tempfile.TemporaryDirectory() as d:
        so = _build_mutant(name, d)
        failed = _pins(so)
        assert failed, f"mutant {name} passed every pin"

"""The backward's context split: for dense sequences with few (sequence,
head) chains, kda_chunk_bwd runs both scans over pieces of each sequence
(state maps, entry states chained forward; zero-start gradients, exit
gradients chained back through the transposed maps) and then every piece
from its true entry state or exit gradient.

Each case is checked against the fp64 oracle's derivative and against the
same call run unsplit (a workspace without the split region), at the
backward's bf16 tolerance. With the default gate (log-decay about -2.5 per
token) a piece's map underflows to zero within a few tiles, so the split
must give the unsplit bits; a gate near zero keeps states and gradients
alive across every piece, so the composed maps decide the result there.
long256k, whose oracle would hold 262,145 fp64 states per unit, is compared
split against unsplit over every element.
"""
import pytest
import torch

from gated_delta_rule_92_amd import bwd_workspace_size, chunk_bwd, chunk_fwd_train
from gated_delta_rule_92_amd.inputs import make_inputs
from oracle import oracle_backward, oracle_gate, oracle_recurrence
from tests.gpu_helpers import TOL_BF16, rel_err, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dh0")
# On a 256-CU device: B=1 H=2 T=20000 takes 64 pieces of 320 tokens (the
# last one empty), T=4096 16 pieces of 256, B=2 H=4 T=6016 32 pieces of 192
# (the last of 64).
CASES = [
    ("B=1 H=2 T=20000 logits h0 dhT", dict(B=1, H=2, T=20000, gate="logits", h0=0.02, dh=True)),
    ("B=2 H=4 T=6016 logdecay h0", dict(B=2, H=4, T=6016, gate="logdecay", h0=0.02, dh=False)),
    ("slow decay B=1 H=2 T=4096 h0 dhT",
     dict(B=1, H=2, T=4096, gate="slow", h0=0.02, dh=True)),
    ("slow decay B=1 H=2 T=20000 h0 dhT",
     dict(B=1, H=2, T=20000, gate="slow", h0=0.02, dh=True)),
]


def _gate(d, kind):
    """(gate input for the kernel, gate mode, log-decay for the oracle)."""
    if kind == "logits":
        return d["z"], "logits", oracle_gate(d["z"], None, -5.0)
    if kind == "slow":
        g = (-0.002 * torch.sigmoid(d["z"])).contiguous()  # per-token log-decay in [-0.002, 0]
        return g, "logdecay", g
    g = torch.from_numpy(oracle_gate(d["z"], None, -5.0)).float()
    return g, "logdecay", g


def _unsplit_workspace(B, T, H, D):
    # the base layout of packed sequences (N = B + 1) is at least the dense
    # one and far smaller than the split region: kda_chunk_bwd runs unsplit
    return torch.empty(bwd_workspace_size(B, T, H, D, D, B + 1, 64, torch.bfloat16),
                       dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_split_backward_matches_oracle_and_unsplit(name, kw):
    print(f"\n[case] split backward: {name}", flush=True)
    B, H, T, D = kw["B"], kw["H"], kw["T"], 128
    d = make_inputs(B, T, H, D, D, torch.bfloat16, h0_std=kw["h0"], seed=71)
    gen = torch.Generator().manual_seed(72)
    do = torch.randn(B, T, H, D, generator=gen).to(torch.bfloat16)
    dhT = torch.randn(B, H, D, D, generator=gen) if kw["dh"] else None
    g_in, mode, g_ref = _gate(d, kw["gate"])
    dd = to_dev(d)
    ins = (dd["q"], dd["k"], dd["v"], g_in.cuda(), dd["beta"])
    dev = lambda x: None if x is None else x.cuda()  # noqa: E731
    split = chunk_bwd(*ins, do.cuda(), dd["h0"], dev(dhT), None, gate=mode)
    plain = chunk_bwd(*ins, do.cuda(), dd["h0"], dev(dhT), None, gate=mode,
                      workspace=_unsplit_workspace(B, T, H, D))
    torch.cuda.synchronize()
    ref = oracle_backward(d["q"], d["k"], d["v"], g_ref, d["beta"], do, d["h0"], dhT, None, 1.0)
    errs = {n: rel_err(split[n], ref[n]) for n in GRADS}
    base = {n: rel_err(plain[n], ref[n]) for n in GRADS}
    vs = {n: rel_err(split[n], plain[n].double().cpu()) for n in GRADS}
    print("  split vs oracle  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    print("  plain vs oracle  " + " ".join(f"{n}={e:.2e}" for n, e in base.items()), flush=True)
    print("  split vs plain   " + " ".join(f"{n}={e:.2e}" for n, e in vs.items()) +
          f" (tol {TOL_BF16:g})", flush=True)
    assert all(e <= TOL_BF16 for e in errs.values()), errs
    assert all(e <= TOL_BF16 for e in vs.values()), vs
    if kw["gate"] == "slow":
        # the entry states and exit gradients came from the composed maps,
        # whose rounding differs from the unsplit chain's somewhere
        assert any(e > 0 for e in vs.values()), "the split path did not run"


@pytest.mark.parametrize("kind", ["logits", "slow"])
def test_split_training_pair(kind):
    """kda_chunk_fwd_train over the same pieces (maps, entry states, every
    piece with output and checkpoints) then kda_chunk_bwd_saved, which runs
    the reverse split only: o, the final state and the gradients against the
    oracle, and the gradients equal to kda_chunk_bwd's (also split) bit for
    bit."""
    print(f"\n[case] split training pair: B=1 H=2 T=20000 {kind}", flush=True)
    B, H, T, D = 1, 2, 20000, 128
    d = make_inputs(B, T, H, D, D, torch.bfloat16, h0_std=0.02, seed=73)
    gen = torch.Generator().manual_seed(74)
    do = torch.randn(B, T, H, D, generator=gen).to(torch.bfloat16)
    dhT = torch.randn(B, H, D, D, generator=gen)
    g_in, mode, g_ref = _gate(d, kind)
    dd = to_dev(d)
    ins = (dd["q"], dd["k"], dd["v"], g_in.cuda(), dd["beta"])
    o, hT, ws = chunk_fwd_train(*ins, dd["h0"], None, gate=mode)
    got = chunk_bwd(*ins, do.cuda(), dd["h0"], dhT.cuda(), None, gate=mode, workspace=ws,
                    saved=True)
    full = chunk_bwd(*ins, do.cuda(), dd["h0"], dhT.cuda(), None, gate=mode)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle_recurrence(d["q"], d["k"], d["v"], g_ref, d["beta"], d["h0"], None)
    eo, eh = rel_err(o, o_ref), rel_err(hT, h_ref)
    ref = oracle_backward(d["q"], d["k"], d["v"], g_ref, d["beta"], do, d["h0"], dhT, None, 1.0)
    errs = {n: rel_err(got[n], ref[n]) for n in GRADS}
    same = {n: torch.equal(got[n], full[n]) for n in GRADS}
    print(f"  o={eo:.2e} final_state={eh:.2e} " +
          " ".join(f"{n}={e:.2e}" for n, e in errs.items()) + f" (tol {TOL_BF16:g})", flush=True)
    print(f"  saved == kda_chunk_bwd: {same}", flush=True)
    assert eo <= TOL_BF16 and eh <= TOL_BF16
    assert all(e <= TOL_BF16 for e in errs.values()), errs
    assert all(same.values()), same


@pytest.mark.parametrize("kind", ["logits", "slow"])
def test_split_backward_long256k_matches_unsplit(kind):
    print(f"\n[case] split backward: long256k B=1 H=32 T=262144 {kind}, every element vs unsplit",
          flush=True)
    B, H, T, D = 1, 32, 262144, 128
    d = make_inputs(B, T, H, D, D, torch.bfloat16, h0_std=0.0, seed=75, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(76)
    do = torch.randn(B, T, H, D, generator=gen, device="cuda").to(torch.bfloat16)
    dhT = torch.randn(B, H, D, D, generator=gen, device="cuda")
    g_in, mode, _ = _gate(d, kind) if kind == "slow" else (d["z"], "logits", None)
    ins = (d["q"], d["k"], d["v"], g_in, d["beta"])
    split = chunk_bwd(*ins, do, None, dhT, None, gate=mode)
    torch.cuda.synchronize()
    plain = chunk_bwd(*ins, do, None, dhT, None, gate=mode,
                      workspace=_unsplit_workspace(B, T, H, D))
    torch.cuda.synchronize()
    errs = {}
    for n in GRADS:
        a, b = split[n].float(), plain[n].float()
        assert torch.isfinite(a).all(), n
        errs[n] = float((a - b).abs().max() / b.abs().max().clamp_min(1e-30))
    print("  split vs plain " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) +
          f" (tol {TOL_BF16:g})", flush=True)
    assert all(e <= TOL_BF16 for e in errs.values()), errs

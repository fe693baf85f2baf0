"""The training pair kda_chunk_fwd_train / kda_chunk_bwd_saved.

kda_chunk_fwd_train runs the forward and the backward's checkpoint scan in one
pass (the pipelined kernel with both outputs); kda_chunk_bwd_saved then skips
that scan. Same kernels, same inputs: o and the final state must equal
kda_chunk_fwd's, and every gradient kda_chunk_bwd's, bit for bit. Small cases
are also checked against the oracle's derivative; train8k (B=8, H=32, T=8192)
is compared with the regular pair over every element.
"""
import pytest
import torch

from gated_delta_rule_92_amd import chunk_bwd, chunk_fwd, chunk_fwd_train
from gated_delta_rule_92_amd.inputs import make_inputs
from oracle import oracle_backward, oracle_gate
from tests.gpu_helpers import TOL_BF16, rel_err, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dh0")
CASES = [
    ("dense B=2 H=2 T=1000 logits h0", dict(B=2, T=1000, lengths=None), "logits"),
    ("packed 6 sequences H=2 logits h0", dict(B=1, T=0, lengths=[700, 0, 33, 1290, 64, 517]),
     "logits"),
    ("dense B=1 H=2 T=333 logdecay h0", dict(B=1, T=333, lengths=None), "logdecay"),
]


def _pair(d, dd, gate, g_in, do_d, dhT_d):
    o_r, h_r = chunk_fwd(dd["q"], dd["k"], dd["v"], g_in, dd["beta"], dd["h0"], dd["cu_seqlens"],
                         gate=gate)
    o_t, h_t, ws = chunk_fwd_train(dd["q"], dd["k"], dd["v"], g_in, dd["beta"], dd["h0"],
                                   dd["cu_seqlens"], gate=gate)
    full = chunk_bwd(dd["q"], dd["k"], dd["v"], g_in, dd["beta"], do_d, dd["h0"], dhT_d,
                     dd["cu_seqlens"], gate=gate)
    saved = chunk_bwd(dd["q"], dd["k"], dd["v"], g_in, dd["beta"], do_d, dd["h0"], dhT_d,
                      dd["cu_seqlens"], gate=gate, workspace=ws, saved=True)
    torch.cuda.synchronize()
    return (o_r, h_r), (o_t, h_t), full, saved


@pytest.mark.parametrize("name,kw,gate", CASES, ids=[c[0] for c in CASES])
def test_training_pair_equals_forward_and_backward(name, kw, gate):
    print(f"\n[case] training pair: {name}", flush=True)
    H, D = 2, 128
    d = make_inputs(kw["B"], kw["T"], H, D, D, torch.bfloat16, h0_std=0.02, lengths=kw["lengths"],
                    seed=61)
    B, T = d["q"].shape[0], d["q"].shape[1]
    N = B if d["cu_seqlens"] is None else d["cu_seqlens"].numel() - 1
    gen = torch.Generator().manual_seed(62)
    do = torch.randn(B, T, H, D, generator=gen).to(torch.bfloat16)
    dhT = torch.randn(N, H, D, D, generator=gen)
    g64 = oracle_gate(d["z"], None, -5.0)
    g_host = d["z"] if gate == "logits" else torch.from_numpy(g64).float()
    dd = to_dev(d)
    (o_r, h_r), (o_t, h_t), full, saved = _pair(d, dd, gate, g_host.cuda(), do.cuda(), dhT.cuda())
    assert torch.equal(o_t, o_r) and torch.equal(h_t, h_r)
    same = {n: torch.equal(saved[n], full[n]) for n in GRADS}
    ref = oracle_backward(d["q"], d["k"], d["v"], g64 if gate == "logits" else g_host, d["beta"],
                          do, d["h0"], dhT, d["cu_seqlens"], 1.0)
    errs = {n: rel_err(saved[n], ref[n]) for n in GRADS}
    print("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) + f" (tol {TOL_BF16:g}); "
          f"equal to kda_chunk_bwd: {all(same.values())}", flush=True)
    assert all(same.values()), same
    assert all(e <= TOL_BF16 for e in errs.values()), errs


def test_training_pair_train8k_equals_forward_and_backward():
    print("\n[case] training pair: train8k B=8 H=32 T=8192, every element", flush=True)
    B, T, H, D = 8, 8192, 32, 128
    d = make_inputs(B, T, H, D, D, torch.bfloat16, h0_std=0.0, lengths=None, seed=63,
                    device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(64)
    do = torch.randn(B, T, H, D, generator=gen, device="cuda").to(torch.bfloat16)
    dhT = torch.randn(B, H, D, D, generator=gen, device="cuda")
    (o_r, h_r), (o_t, h_t), full, saved = _pair(None, d, "logits", d["z"], do, dhT)
    assert torch.equal(o_t, o_r) and torch.equal(h_t, h_r)
    for n in GRADS:
        assert torch.equal(saved[n], full[n]), n
    print("  o, final state and all six gradients equal the regular pair's", flush=True)

"""The chunk forward and backward captured into a HIP graph (torch.cuda.graph)
and replayed.

Two calls are captured: a long dense sequence with few (sequence, head) units,
whose automatic context split kda_chunk_fwd takes by itself (on a stream that
is being captured it keeps the one-stream schedule, equal pieces, where eager
calls of this shape run the first piece on the library's second stream), and
a packed batch whose longest-first order is computed into the workspace. The
graph is replayed three times with eager work and synchronisations between the
replays, and every replay is checked: against the oracle at the forward's
tolerance, and against the eager call of the same inputs.

The backward (kda_chunk_bwd: checkpoint scan, reverse scan, per-chunk
gradients, and for packed sequences the longest-first order it computes into
the workspace; for the long dense sequence both scans' context split: piece
table, split pass, compositions, scans over the pieces) is captured the same
way, and so is the training pair (kda_chunk_fwd_train, kda_chunk_bwd_saved).
Both are deterministic, so every replay must equal the eager call bit for
bit, besides matching the oracle.
"""
import pytest
import torch

from gated_delta_rule_92_amd import chunk_bwd, chunk_fwd, workspace_size
from gated_delta_rule_92_amd.inputs import make_inputs
from gated_delta_rule_92_amd.ops import bwd_workspace_size
from oracle import oracle_backward, oracle_forward, oracle_gate
from tests.gpu_helpers import TOL_BF16, rel_err, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

CASES = [
    ("dense B=1 H=2 T=20000 (automatic context split)", dict(B=1, T=20000, lengths=None)),
    ("packed 6 sequences H=2 (longest-first order)",
     dict(B=1, T=0, lengths=[700, 0, 33, 1290, 64, 517])),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_captured_forward_replays(name, kw):
    print(f"\n[case] graph capture: {name}", flush=True)
    H = 2
    d = make_inputs(kw["B"], kw["T"], H, 128, 128, torch.bfloat16, h0_std=0.02,
                    lengths=kw["lengths"], seed=51)
    dd = to_dev(d)
    B, T = d["q"].shape[0], d["q"].shape[1]
    N = B if d["cu_seqlens"] is None else d["cu_seqlens"].numel() - 1
    ws = workspace_size(B, T, H, 128, 128, N, 64, torch.bfloat16)
    wsp = torch.zeros(max(ws, 1), dtype=torch.uint8, device="cuda")
    o = torch.zeros_like(dd["v"])
    hT = torch.zeros((N, H, 128, 128), dtype=torch.float32, device="cuda")

    def call():
        chunk_fwd(dd["q"], dd["k"], dd["v"], dd["z"], dd["beta"], dd["h0"], dd["cu_seqlens"],
                  gate="logits", o=o, final_state=hT, workspace=wsp)

    # eager reference (for the dense case: the first-out schedule)
    o_eager, h_eager = chunk_fwd(dd["q"], dd["k"], dd["v"], dd["z"], dd["beta"], dd["h0"],
                                 dd["cu_seqlens"], gate="logits")
    # warm up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    ref = oracle_forward(d["q"], d["k"], d["v"], d["z"], d["beta"], d["h0"], d["cu_seqlens"], None,
                         -5.0)
    for replay in range(3):
        # eager work between replays: clobber the outputs and the workspace
        o.fill_(float("nan"))
        hT.fill_(float("nan"))
        wsp.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eo, es = rel_err(o, ref[0]), rel_err(hT, ref[1])
        do = rel_err(o, o_eager.double().cpu())
        ds = rel_err(hT, h_eager.double().cpu())
        print(f"  replay {replay}: vs oracle err_o={eo:.3e} err_state={es:.3e}; vs eager "
              f"o {do:.3e} state {ds:.3e} (tol {TOL_BF16:g})", flush=True)
        assert eo <= TOL_BF16 and es <= TOL_BF16
        assert do <= TOL_BF16 and ds <= TOL_BF16


BWD_CASES = [
    ("dense B=1 H=2 T=1000 logits", dict(B=1, T=1000, lengths=None)),
    ("packed 6 sequences H=2 with h0 and dhT", dict(B=1, T=0, lengths=[700, 0, 33, 1290, 64, 517])),
    ("dense B=1 H=2 T=20000 (context split of both scans)", dict(B=1, T=20000, lengths=None)),
]
GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


@pytest.mark.parametrize("name,kw", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_captured_backward_replays(name, kw):
    print(f"\n[case] graph capture, backward: {name}", flush=True)
    H, D = 2, 128
    d = make_inputs(kw["B"], kw["T"], H, D, D, torch.bfloat16, h0_std=0.02, lengths=kw["lengths"],
                    seed=53)
    B, T = d["q"].shape[0], d["q"].shape[1]
    N = B if d["cu_seqlens"] is None else d["cu_seqlens"].numel() - 1
    gen = torch.Generator().manual_seed(54)
    do = torch.randn(B, T, H, D, generator=gen).to(torch.bfloat16)
    dhT = torch.randn(N, H, D, D, generator=gen)
    dd = to_dev(d)
    do_d, dhT_d = do.cuda(), dhT.cuda()
    wsp = torch.zeros(max(bwd_workspace_size(B, T, H, D, D, N, 64, torch.bfloat16), 1),
                      dtype=torch.uint8, device="cuda")

    def call():
        return chunk_bwd(dd["q"], dd["k"], dd["v"], dd["z"], dd["beta"], do_d, dd["h0"], dhT_d,
                         dd["cu_seqlens"], gate="logits", workspace=wsp)

    eager = {n: t.clone() for n, t in call().items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = call()
    torch.cuda.synchronize()
    ref = oracle_backward(d["q"], d["k"], d["v"], oracle_gate(d["z"], None, -5.0), d["beta"], do,
                          d["h0"], dhT, d["cu_seqlens"], 1.0)
    for replay in range(3):
        # eager work between replays: clobber the gradients and the workspace
        for t in out.values():
            t.fill_(float("nan"))
        wsp.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        errs = {n: rel_err(out[n], ref[n]) for n in GRADS}
        same = all(torch.equal(out[n], eager[n]) for n in GRADS)
        print(f"  replay {replay}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) +
              f" (tol {TOL_BF16:g}); equal to eager: {same}", flush=True)
        assert same
        assert all(e <= TOL_BF16 for e in errs.values()), errs


TRAIN_CASES = [
    ("packed 6 sequences H=2", dict(T=0, lengths=[700, 0, 33, 1290, 64, 517])),
    ("dense B=1 H=2 T=20000 (context split)", dict(T=20000, lengths=None)),
]


@pytest.mark.parametrize("name,kw", TRAIN_CASES, ids=[c[0] for c in TRAIN_CASES])
def test_captured_training_pair_replays(name, kw):
    """kda_chunk_fwd_train and kda_chunk_bwd_saved captured together (packed
    sequences: both compute the longest-first order into the backward
    workspace; the long dense sequence: both take the context split, the
    forward leaving the maps' transposes for the backward): every replay
    equals the eager pair bit for bit."""
    print(f"\n[case] graph capture, training pair: {name}", flush=True)
    from gated_delta_rule_92_amd import chunk_fwd_train
    H, D = 2, 128
    d = make_inputs(1, kw["T"], H, D, D, torch.bfloat16, h0_std=0.02, lengths=kw["lengths"],
                    seed=55)
    B, T = d["q"].shape[0], d["q"].shape[1]
    N = B if d["cu_seqlens"] is None else d["cu_seqlens"].numel() - 1
    gen = torch.Generator().manual_seed(56)
    do = torch.randn(B, T, H, D, generator=gen).to(torch.bfloat16).cuda()
    dhT = torch.randn(N, H, D, D, generator=gen).cuda()
    dd = to_dev(d)
    wsp = torch.zeros(bwd_workspace_size(B, T, H, D, D, N, 64, torch.bfloat16), dtype=torch.uint8,
                      device="cuda")
    ins = (dd["q"], dd["k"], dd["v"], dd["z"], dd["beta"])

    def call():
        o, hT, _ = chunk_fwd_train(*ins, dd["h0"], dd["cu_seqlens"], gate="logits",
                                   bwd_workspace=wsp)
        g = chunk_bwd(*ins, do, dd["h0"], dhT, dd["cu_seqlens"], gate="logits", workspace=wsp,
                      saved=True)
        return dict(o=o, hT=hT, **g)

    eager = {n: t.clone() for n, t in call().items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = call()
    torch.cuda.synchronize()
    for replay in range(3):
        for t in out.values():
            t.fill_(float("nan"))
        wsp.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same = {n: torch.equal(out[n], eager[n]) for n in eager}
        print(f"  replay {replay}: equal to eager: {all(same.values())}", flush=True)
        assert all(same.values()), same

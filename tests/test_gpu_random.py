"""Seeded random parity sweep: forward (kda_chunk_fwd) and backward
(kda_chunk_bwd) against the fp64 oracle on problems whose shape is drawn from
a fixed seed: dense or packed sequences (0 to 300 tokens, empty ones
included), 1 to 3 heads, d_k and d_v in {64, 128} independently, bf16 or fp32,
gate logits or per-token log-decay, with or without an initial state and a
final-state gradient, output scale in [0.5, 1.5]. A second sweep draws long
dense problems that kda_chunk_fwd runs as a context split, and a third such
problems for kda_chunk_bwd, whose two scans split the same way. The same bar as
the other parity tests: max|gpu - ref| / max|ref| <= 2e-2 (bf16) and 1e-4
(fp32) per output array. For bf16 d_k = d_v = 128 problems the training pair
(kda_chunk_fwd_train, kda_chunk_bwd_saved) must also equal the plain calls bit
for bit.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_92_amd import chunk_bwd, chunk_fwd
from gated_delta_rule_92_amd.inputs import make_inputs
from oracle import oracle_backward, oracle_forward, oracle_gate, oracle_recurrence
from tests.gpu_helpers import rel_err, tol_for

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _problem(seed):
    rng = np.random.default_rng(1000 + seed)
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    Dk, Dv = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
    H = int(rng.integers(1, 4))
    packed = rng.random() < 0.6
    if packed:
        n = int(rng.integers(1, 7))
        lengths = [int(x) for x in rng.integers(0, 301, n)]
        if rng.random() < 0.3:
            lengths[int(rng.integers(0, n))] = 0
        B, T = 1, 0
    else:
        lengths = None
        B, T = int(rng.integers(1, 4)), int(rng.integers(1, 301))
    spec = dict(dtype=dtype, Dk=Dk, Dv=Dv, H=H, B=B, T=T, lengths=lengths,
                gate="logits" if rng.random() < 0.6 else "logdecay",
                h0=rng.random() < 0.5, dh=rng.random() < 0.6,
                scale=float(np.round(rng.uniform(0.5, 1.5), 3)))
    return spec


def _label(s):
    shape = f"lengths={s['lengths']}" if s["lengths"] is not None else f"B={s['B']} T={s['T']}"
    return (f"{'bf16' if s['dtype'] == torch.bfloat16 else 'fp32'} Dk={s['Dk']} Dv={s['Dv']} "
            f"H={s['H']} {shape} gate={s['gate']} h0={s['h0']} dhT={s['dh']} scale={s['scale']}")


@pytest.mark.parametrize("seed", range(40))
def test_random_problem_forward_and_backward(seed):
    s = _problem(seed)
    print(f"\n[case] random {seed}: {_label(s)}", flush=True)
    d = make_inputs(s["B"], s["T"], s["H"], s["Dk"], s["Dv"], s["dtype"],
                    h0_std=0.02 if s["h0"] else 0.0, lengths=s["lengths"], seed=2000 + seed)
    N = d["N"]
    if d["q"].shape[1] == 0:
        pytest.skip("no tokens drawn")
    tol = tol_for(s["dtype"])
    g64 = oracle_gate(d["z"], None, -5.0)
    g_in = d["z"] if s["gate"] == "logits" else torch.from_numpy(g64).float()
    g_ref = g64 if s["gate"] == "logits" else torch.from_numpy(g64).float()
    dev = lambda x: None if x is None else x.cuda()  # noqa: E731

    o, hT = chunk_fwd(dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(g_in), dev(d["beta"]),
                      dev(d["h0"]), dev(d["cu_seqlens"]), gate=s["gate"], scale=s["scale"])
    torch.cuda.synchronize()
    if s["gate"] == "logits":
        ro, rs = oracle_forward(d["q"], d["k"], d["v"], d["z"], d["beta"], d["h0"],
                                d["cu_seqlens"], None, -5.0, s["scale"])
    else:
        ro, rs = oracle_recurrence(d["q"], d["k"], d["v"], g_ref, d["beta"], d["h0"],
                                   d["cu_seqlens"], s["scale"])
    eo, es = rel_err(o, ro), rel_err(hT, rs)
    print(f"  forward err_o={eo:.2e} err_state={es:.2e} tol={tol:g}", flush=True)
    assert eo <= tol and es <= tol

    gen = torch.Generator().manual_seed(3000 + seed)
    do = torch.randn(d["v"].shape, generator=gen).to(s["dtype"])
    dhT = torch.randn(N, s["H"], s["Dk"], s["Dv"], generator=gen) if s["dh"] else None
    got = chunk_bwd(dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(g_in), dev(d["beta"]), dev(do),
                    dev(d["h0"]), dev(dhT), dev(d["cu_seqlens"]), gate=s["gate"],
                    scale=s["scale"])
    torch.cuda.synchronize()
    ref = oracle_backward(d["q"], d["k"], d["v"], g_ref, d["beta"], do, d["h0"], dhT,
                          d["cu_seqlens"], s["scale"])
    errs = {n: rel_err(got[n], ref[n]) for n in ("dq", "dk", "dv", "dg", "dbeta", "dh0")}
    print("  backward " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert np.all(np.isfinite(got[n].double().cpu().numpy())), n
        assert e <= tol, (n, e)

    if s["dtype"] == torch.bfloat16 and s["Dk"] == 128 and s["Dv"] == 128:
        # the training pair (one pass for the forward and the backward's
        # checkpoints, then the backward without its first scan) equals the
        # plain calls bit for bit
        from gated_delta_rule_92_amd import chunk_fwd_train
        o2, h2, ws = chunk_fwd_train(dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(g_in),
                                     dev(d["beta"]), dev(d["h0"]), dev(d["cu_seqlens"]),
                                     gate=s["gate"], scale=s["scale"])
        got2 = chunk_bwd(dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(g_in), dev(d["beta"]), dev(do),
                         dev(d["h0"]), dev(dhT), dev(d["cu_seqlens"]), gate=s["gate"],
                         scale=s["scale"], workspace=ws, saved=True)
        torch.cuda.synchronize()
        same = torch.equal(o2, o) and torch.equal(h2, hT) and \
            all(torch.equal(got2[n], got[n]) for n in errs)
        print(f"  training pair equal to the plain calls: {same}", flush=True)
        assert same


def _split_problem(seed):
    """A dense bf16 d = 128 problem long enough, with few enough heads, that
    kda_chunk_fwd splits it by itself (P = CUs / (B H) >= 4 pieces and
    T (0.9 - 3/P) > 300): on a 256-CU device 1 to 2 sequences of 2,000 to
    24,000 tokens with 1 to 8 heads; gate logits, per-token log-decay or its
    cumulative sum within 64-token chunks."""
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(1, 3))
    H = int(rng.choice([1, 2, 4, 8]))
    T = int(rng.integers(2000, 24001))
    return dict(B=B, H=H, T=T, gate=str(rng.choice(["logits", "logdecay", "cumsum"])),
                h0=bool(rng.random() < 0.7), scale=float(np.round(rng.uniform(0.5, 1.5), 3)))


@pytest.mark.parametrize("seed", range(12))
def test_random_automatic_split(seed):
    """kda_chunk_fwd on random long dense problems that take the automatic
    context split (equal pieces or first-out, as the cost model picks), every
    element against the unsplit oracle; the piece table is checked to start
    every piece on a 64-token chunk boundary and to end at T."""
    from gated_delta_rule_92_amd import gate as gate_fn
    from gated_delta_rule_92_amd import workspace_size
    s = _split_problem(seed)
    print(f"\n[case] random split {seed}: B={s['B']} H={s['H']} T={s['T']} gate={s['gate']} "
          f"h0={s['h0']} scale={s['scale']}", flush=True)
    d = make_inputs(s["B"], s["T"], s["H"], 128, 128, torch.bfloat16,
                    h0_std=0.02 if s["h0"] else 0.0, seed=6000 + seed)
    dd = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    if s["gate"] == "logits":
        g = dd["z"]
    else:
        g = gate_fn(dd["z"], None, -5.0, 64 if s["gate"] == "cumsum" else 0, None)
    ws = workspace_size(s["B"], s["T"], s["H"], 128, 128, s["B"], 64, torch.bfloat16)
    wsp = torch.zeros(max(ws, 1), dtype=torch.uint8, device="cuda")
    o, hT = chunk_fwd(dd["q"], dd["k"], dd["v"], g, dd["beta"], dd["h0"], gate=s["gate"],
                      scale=s["scale"], workspace=wsp)
    torch.cuda.synchronize()
    if ws >= 4 * 2:
        table = wsp[:4 * 66].view(torch.int32).cpu().tolist()
        if table[0] == 0 and s["T"] in table[1:]:
            P = table[1:].index(s["T"]) + 1
            print(f"  pieces: {P}, first {table[1]}, second {table[2] - table[1] if P > 1 else 0}",
                  flush=True)
            assert all(t % 64 == 0 for t in table[:P])
    ro, rs = oracle_forward(d["q"], d["k"], d["v"], d["z"], d["beta"], d["h0"], None, None, -5.0,
                            s["scale"])
    eo, es = rel_err(o, ro), rel_err(hT, rs)
    print(f"  err_o={eo:.2e} err_state={es:.2e}", flush=True)
    assert eo <= 2e-2 and es <= 2e-2


def _split_bwd_problem(seed):
    """A long dense bf16 d = 128 problem whose backward scans split (as
    _split_problem), with gate logits, per-token log-decay, or a log-decay in
    [-0.002, 0] that keeps states and gradients alive across every piece, so
    that the composed maps decide the result."""
    rng = np.random.default_rng(7000 + seed)
    B = int(rng.integers(1, 3))
    H = int(rng.choice([1, 2, 4, 8]))
    T = int(rng.integers(2000, 24001))
    return dict(B=B, H=H, T=T, gate=str(rng.choice(["logits", "logdecay", "slow"])),
                h0=bool(rng.random() < 0.7), dh=bool(rng.random() < 0.7),
                scale=float(np.round(rng.uniform(0.5, 1.5), 3)))


@pytest.mark.parametrize("seed", range(6))
def test_random_split_backward(seed):
    """kda_chunk_bwd on random long dense problems that take the context
    split of both scans: every element of every sequence of up to two heads
    against the oracle's derivative (the heads are independent, so the oracle
    runs on those heads alone), and every element of all heads against the
    same call in a workspace without the split region (unsplit)."""
    from gated_delta_rule_92_amd.ops import bwd_workspace_size
    s = _split_bwd_problem(seed)
    print(f"\n[case] random split backward {seed}: B={s['B']} H={s['H']} T={s['T']} "
          f"gate={s['gate']} h0={s['h0']} dhT={s['dh']} scale={s['scale']}", flush=True)
    B, H, T, D = s["B"], s["H"], s["T"], 128
    d = make_inputs(B, T, H, D, D, torch.bfloat16, h0_std=0.02 if s["h0"] else 0.0,
                    seed=8000 + seed)
    gen = torch.Generator().manual_seed(9000 + seed)
    do = torch.randn(B, T, H, D, generator=gen).to(torch.bfloat16)
    dhT = torch.randn(B, H, D, D, generator=gen) if s["dh"] else None
    if s["gate"] == "logits":
        g_in, mode, g_ref = d["z"], "logits", oracle_gate(d["z"], None, -5.0)
    elif s["gate"] == "slow":
        g_in = (-0.002 * torch.sigmoid(d["z"])).contiguous()
        mode, g_ref = "logdecay", g_in
    else:
        g_in = torch.from_numpy(oracle_gate(d["z"], None, -5.0)).float()
        mode, g_ref = "logdecay", g_in
    dev = lambda x: None if x is None else x.cuda()  # noqa: E731
    ins = (dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(g_in), dev(d["beta"]), dev(do), dev(d["h0"]),
           dev(dhT), None)
    split = chunk_bwd(*ins, gate=mode, scale=s["scale"])
    base = torch.empty(bwd_workspace_size(B, T, H, D, D, B + 1, 64, torch.bfloat16),
                       dtype=torch.uint8, device="cuda")
    plain = chunk_bwd(*ins, gate=mode, scale=s["scale"], workspace=base)
    torch.cuda.synchronize()
    names = ("dq", "dk", "dv", "dg", "dbeta", "dh0")
    vs = {n: rel_err(split[n], plain[n].double().cpu()) for n in names}
    heads = [0] if H == 1 else [0, H - 1]
    sl = lambda x: None if x is None else x[:, :, heads].contiguous()  # noqa: E731
    slh = lambda x: None if x is None else x[:, heads].contiguous()  # noqa: E731
    g_sl = g_ref[:, :, heads] if isinstance(g_ref, np.ndarray) else sl(g_ref)
    ref = oracle_backward(sl(d["q"]), sl(d["k"]), sl(d["v"]), g_sl, sl(d["beta"]), sl(do),
                          slh(d["h0"]), slh(dhT), None, s["scale"])
    errs = {}
    for n in names:
        x = split[n][:, heads] if n == "dh0" else split[n][:, :, heads]
        errs[n] = rel_err(x, ref[n])
    print("  split vs oracle (heads %s) " % heads +
          " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    print("  split vs unsplit " + " ".join(f"{n}={e:.2e}" for n, e in vs.items()), flush=True)
    assert all(e <= 2e-2 for e in errs.values()), errs
    assert all(e <= 2e-2 for e in vs.values()), vs

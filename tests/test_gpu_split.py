"""GPU parity for the context-split path (one-GPU form of splitting a
sequence across devices): per-segment state maps (kda_chunk_transition),
their composition (kda_compose_states) and the split forward, each against
the fp64 oracle's unsplit run or plain fp64 arithmetic.

Bar: max|gpu - ref| / max|ref| <= 2e-2 for bf16 inputs (o, final state and
state maps), <= 1e-4 for the fp32 composition.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_92_amd import chunk_fwd, chunk_fwd_split, compose_states, gate, transition
from gated_delta_rule_92_amd.inputs import make_inputs, make_workload
from oracle import oracle_forward, oracle_recurrence
from tests.gpu_helpers import TOL_BF16, TOL_FP32, rel_err, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _print_case(name):
    print(f"\n[case] {name}", flush=True)


def test_transition_matches_oracle():
    """M from the pipelined kernel's transition mode equals the oracle run
    with v = 0 from S = I (the state map), per (sequence, head)."""
    _print_case("transition, varlen bf16 d=128")
    lens = [130, 1, 64, 300, 0, 47]
    H = 2
    d = make_inputs(1, 0, H, 128, 128, torch.bfloat16, lengths=lens, seed=31)
    dd = to_dev(d)
    M = transition(dd["k"], dd["z"], dd["beta"], dd["cu_seqlens"], gate="logits")
    torch.cuda.synchronize()
    N = len(lens)
    eye = torch.eye(128).expand(N, H, 128, 128).contiguous()
    zeros = torch.zeros(1, sum(lens), H, 128)
    _, ref = oracle_forward(d["q"], d["k"], zeros, d["z"], d["beta"], eye, d["cu_seqlens"],
                            None, -5.0)
    err = rel_err(M, ref)
    print(f"  err_M={err:.3e} tol={TOL_BF16:g}", flush=True)
    assert err <= TOL_BF16
    assert torch.equal(M[4].cpu(), eye[4])   # empty sequence: the identity


@pytest.mark.parametrize("P,Dv,Dk", [(5, 40, 128), (1, 16, 128), (2, 128, 128), (3, 7, 128), (4, 24, 64)])
def test_compose_matches_fp64_chain(P, Dv, Dk):
    _print_case(f"compose, fp32, P={P} Dk={Dk} Dv={Dv}")
    gen = torch.Generator().manual_seed(32 + P)
    nseq, H = 2, 3
    M = (torch.eye(Dk) + 0.05 * torch.randn(nseq * P, H, Dk, Dk, generator=gen)).contiguous()
    b = torch.randn(nseq * P, H, Dk, Dv, generator=gen)
    S0 = torch.randn(nseq, H, Dk, Dv, generator=gen)
    for init in (S0, None):
        out = compose_states(M.cuda(), b.cuda(), None if init is None else init.cuda(), nseq, P)
        torch.cuda.synchronize()
        M64, b64 = M.double().numpy(), b.double().numpy()
        ref = np.empty(b64.shape)
        for s in range(nseq):
            cur = np.zeros((H, Dk, Dv)) if init is None else init[s].double().numpy()
            for p in range(P):
                ref[s * P + p] = cur
                cur = np.einsum("hij,hjc->hic", M64[s * P + p], cur) + b64[s * P + p]
        err = rel_err(out, ref)
        print(f"  init={'yes' if init is not None else 'none'} err={err:.3e} tol={TOL_FP32:g}",
              flush=True)
        assert err <= TOL_FP32


CASES = [
    ("dense B=2 T=300 P=3", dict(B=2, T=300, lengths=None, h0_std=0.02), 3, "logits"),
    ("varlen P=2", dict(B=1, T=0, lengths=[0, 1, 63, 64, 65, 130, 257, 16], h0_std=0.02), 2,
     "logits"),
    ("varlen P=5 cumsum gate", dict(B=1, T=0, lengths=[700, 129, 64], h0_std=0.0), 5, "cumsum"),
    ("dense B=1 T=1000 P=8 logdecay", dict(B=1, T=1000, lengths=None, h0_std=0.02), 8,
     "logdecay"),
    # Lp = 64: pieces 5-7 of each sequence are empty
    ("dense B=2 T=300 P=8 empty trailing pieces", dict(B=2, T=300, lengths=None, h0_std=0.02), 8,
     "logits"),
]


@pytest.mark.parametrize("name,kw,P,mode", CASES, ids=[c[0] for c in CASES])
def test_split_forward_matches_unsplit_oracle(name, kw, P, mode):
    _print_case(f"split forward: {name}")
    H = 2
    d = make_inputs(kw["B"], kw["T"], H, 128, 128, torch.bfloat16, h0_std=kw["h0_std"],
                    lengths=kw["lengths"], seed=33)
    dd = to_dev(d)
    if mode == "logits":
        g = dd["z"]
    else:
        g = gate(dd["z"], None, -5.0, 64 if mode == "cumsum" else 0, dd["cu_seqlens"])
    o, hT = chunk_fwd_split(dd["q"], dd["k"], dd["v"], g, dd["beta"], dd["h0"], dd["cu_seqlens"],
                            segments=P, gate=mode)
    o_ref_gpu, hT_ref_gpu = chunk_fwd(dd["q"], dd["k"], dd["v"], g, dd["beta"], dd["h0"],
                                      dd["cu_seqlens"], gate=mode)
    torch.cuda.synchronize()
    ref = oracle_forward(d["q"], d["k"], d["v"], d["z"], d["beta"], d["h0"], d["cu_seqlens"],
                         None, -5.0)
    eo, es = rel_err(o, ref[0]), rel_err(hT, ref[1])
    print(f"  vs oracle err_o={eo:.3e} err_state={es:.3e} tol={TOL_BF16:g}; vs unsplit GPU "
          f"{rel_err(o, o_ref_gpu.double().cpu().numpy()):.3e}", flush=True)
    assert eo <= TOL_BF16 and es <= TOL_BF16
    del hT_ref_gpu


def test_packed_piece_table():
    """The piece table kda_chunk_fwd_split builds on the device from
    cu_seqlens: every sequence in `segments` consecutive pieces of
    64 * ceil(ceil(L / P) / 64) tokens, the last taking the rest."""
    import ctypes
    from gated_delta_rule_92_amd import _lib
    from gated_delta_rule_92_amd.ops import _ptr, _stream
    _print_case("packed piece table")
    lens, P, H = [0, 1, 63, 64, 65, 700, 130], 3, 2
    d = make_inputs(1, 0, H, 128, 128, torch.bfloat16, lengths=lens, seed=36)
    dd = to_dev(d)
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    assert lib.kda_chunk_fwd_split_workspace_size(1, sum(lens), H, 128, 128, len(lens), P, 64,
                                                  _lib.KDA_BFLOAT16, ctypes.byref(n)) == 0
    ws = torch.zeros(n.value, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(dd["v"])
    rc = lib.kda_chunk_fwd_split(_ptr(dd["q"]), _ptr(dd["k"]), _ptr(dd["v"]), _lib.KDA_BFLOAT16,
                                 _ptr(dd["z"]), _lib.KDA_GATE_LOGITS, None, -5.0, _ptr(dd["beta"]),
                                 None, _ptr(dd["cu_seqlens"]), len(lens), 1, sum(lens), H, 128, 128,
                                 64, P, 1.0, _ptr(o), None, _ptr(ws), n.value,
                                 _stream(torch.device("cuda")))
    assert rc == 0
    table = ws[:4 * (len(lens) * P + 1)].view(torch.int32).cpu().tolist()
    want, start = [], 0
    for L in lens:
        per = -(-(-(-L // P)) // 64) * 64
        want += [start + min(p * per, L) for p in range(P)]
        start += L
    want.append(start)
    assert table == want
    ref = oracle_forward(d["q"], d["k"], d["v"], d["z"], d["beta"], None, d["cu_seqlens"], None, -5.0)
    assert rel_err(o, ref[0]) <= TOL_BF16


def _first_out_plan(T, cus_per_unit, chunk=64):
    """The piece table of the first-out split the library plans for one dense
    sequence (its cost model: a split-pass token costs 1.12 forward tokens,
    a composition step 30 tokens, the fork to the second stream and the
    join back 200; middle pieces of a tokens, a first piece of about
    1.12 a, both whole chunks, the last piece the rest), or None when it
    plans equal pieces."""
    P = min(cus_per_unit, T // 256, 64)
    Lp = -(-(-(-T // P)) // chunk) * chunk
    best, best_cost = None, 2.12 * Lp + 30 * (P - 1)
    for Pf in range(3, cus_per_unit + 2):
        if Pf - 1 > 64:
            break
        a = -(-int(T / ((Pf - 1) + 1.12)) // chunk) * chunk
        L0 = int(1.12 * a) // chunk * chunk
        last = T - L0 - (Pf - 2) * a
        if last > a:
            L0 += -(-(last - a) // chunk) * chunk
            last = T - L0 - (Pf - 2) * a
        if a < 256 or L0 < a or last <= 0:
            continue
        cost = max(L0, 1.12 * a) + a + 30 * (Pf - 2) + 200
        if cost < best_cost:
            best, best_cost = [0] + [L0 + p * a for p in range(Pf - 1)] + [T], cost
    return best


def test_split_long256k_schedules_agree():
    """The 256K-token single sequence at full size (32 heads): kda_chunk_fwd's
    automatic split (on a 256-CU device the first-out schedule, 9 pieces:
    the first of 32,256 tokens run with output on the library's second
    stream, 7 of 28,800, the last of 28,288) and the explicit 8-segment
    split (equal pieces,
    one stream) give the same bits. With this workload's gate every piece's
    state map underflows to zero within a few tiles, so both equal the
    unsplit chain; test_gpu_parity checks the automatic split's every
    element against the oracle."""
    _print_case("split forward: long256k, automatic (first-out) vs explicit 8 segments")
    from gated_delta_rule_92_amd import workspace_size
    d = make_workload("long256k", device="cuda")
    T = d["q"].shape[1]
    ws = workspace_size(1, T, 32, 128, 128, 1, 64, torch.bfloat16)
    wsp = torch.empty(ws, dtype=torch.uint8, device="cuda")
    o_a, h_a = chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["beta"], d["h0"], d["cu_seqlens"],
                         gate="logits", workspace=wsp)
    torch.cuda.synchronize()
    table = wsp[:4 * 10].view(torch.int32).cpu().tolist()
    print(f"  automatic split: piece table {table}", flush=True)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        want = _first_out_plan(T, 8)
        assert want == [0] + [32256 + p * 28800 for p in range(8)] + [T]
        assert table == want
    o_e, h_e = chunk_fwd_split(d["q"], d["k"], d["v"], d["z"], d["beta"], d["h0"],
                               d["cu_seqlens"], segments=8, gate="logits")
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_e) and torch.equal(h_a, h_e)


@pytest.mark.parametrize("T,H,first_out,want", [
    # equal pieces of 320 tokens: pieces 13-15 are empty
    (4160, 16, False, [min(p * 320, 4160) for p in range(17)]),
    # first-out: a first piece of 576 tokens with output on the second
    # stream, 37 of 512 and a last one of 480
    (20000, 2, True, [0] + [576 + p * 512 for p in range(38)] + [20000]),
])
def test_automatic_splits_with_ragged_and_empty_pieces(T, H, first_out, want):
    """Dense B=1 with an initial state: kda_chunk_fwd's automatic split, its
    piece table as planned on a 256-CU device, every element against the
    unsplit oracle."""
    _print_case(f"automatic split: B=1 H={H} T={T}")
    from gated_delta_rule_92_amd import workspace_size
    B = 1
    d = make_inputs(B, T, H, 128, 128, torch.bfloat16, h0_std=0.02, seed=37)
    dd = to_dev(d)
    ws = workspace_size(B, T, H, 128, 128, B, 64, torch.bfloat16)
    wsp = torch.zeros(ws, dtype=torch.uint8, device="cuda")
    o, hT = chunk_fwd(dd["q"], dd["k"], dd["v"], dd["z"], dd["beta"], dd["h0"], gate="logits",
                      workspace=wsp)
    torch.cuda.synchronize()
    table = wsp[:4 * len(want)].view(torch.int32).cpu().tolist()
    print(f"  piece table {table}", flush=True)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert _first_out_plan(T, 256 // H) == (want if first_out else None)
        assert table == want
    ref = oracle_forward(d["q"], d["k"], d["v"], d["z"], d["beta"], d["h0"], None, None, -5.0)
    eo, es = rel_err(o, ref[0]), rel_err(hT, ref[1])
    print(f"  err_o={eo:.3e} err_state={es:.3e} tol={TOL_BF16:g}", flush=True)
    assert eo <= TOL_BF16 and es <= TOL_BF16


@pytest.mark.parametrize("mode", ["cumsum", "logdecay"])
def test_first_out_split_with_precomputed_gates(mode):
    """The first-out automatic split (B=1, H=2, T=20000 with an initial
    state; on a 256-CU device a first piece of 576 tokens, then 37 of 512
    and 480) fed the gate as per-token log-decay or as its cumulative sum
    within 64-token chunks (kda_gate's output): every piece starts on a chunk
    boundary, so each piece's tiles rebase the chunk-local sums correctly.
    Every element against the unsplit oracle."""
    _print_case(f"first-out split, gate input {mode}: B=1 H=2 T=20000")
    from gated_delta_rule_92_amd import workspace_size
    B, T, H = 1, 20000, 2
    d = make_inputs(B, T, H, 128, 128, torch.bfloat16, h0_std=0.02, seed=38)
    dd = to_dev(d)
    g = gate(dd["z"], None, -5.0, 64 if mode == "cumsum" else 0, None)
    ws = workspace_size(B, T, H, 128, 128, B, 64, torch.bfloat16)
    wsp = torch.zeros(ws, dtype=torch.uint8, device="cuda")
    o, hT = chunk_fwd(dd["q"], dd["k"], dd["v"], g, dd["beta"], dd["h0"], gate=mode,
                      workspace=wsp)
    torch.cuda.synchronize()
    table = wsp[:4 * 40].view(torch.int32).cpu().tolist()
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert table == [0] + [576 + p * 512 for p in range(38)] + [T]
    assert all(t % 64 == 0 for t in table[:-1])
    ref = oracle_forward(d["q"], d["k"], d["v"], d["z"], d["beta"], d["h0"], None, None, -5.0)
    eo, es = rel_err(o, ref[0]), rel_err(hT, ref[1])
    print(f"  err_o={eo:.3e} err_state={es:.3e} tol={TOL_BF16:g}", flush=True)
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_chunk_fwd_splits_long_dense_sequences_by_itself():
    """kda_chunk_fwd on a long dense sequence with few (sequence, head) units
    takes the context split when its workspace holds it (the size query asks
    for it); with a workspace too small for it the same call runs one serial
    chain per unit. Both against the unsplit oracle, and the split's final
    state written over the initial state it started from."""
    _print_case("automatic split: dense B=1 H=2 T=16384")
    from gated_delta_rule_92_amd import workspace_size
    B, T, H = 1, 16384, 2
    ws = workspace_size(B, T, H, 128, 128, B, 64, torch.bfloat16)
    assert ws > 0
    d = make_inputs(B, T, H, 128, 128, torch.bfloat16, h0_std=0.02, seed=34)
    dd = to_dev(d)
    wsp = torch.zeros(ws, dtype=torch.uint8, device="cuda")
    o_split, hT_split = chunk_fwd(dd["q"], dd["k"], dd["v"], dd["z"], dd["beta"], dd["h0"],
                                  gate="logits", workspace=wsp)
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    o_one, hT_one = chunk_fwd(dd["q"], dd["k"], dd["v"], dd["z"], dd["beta"], dd["h0"],
                              gate="logits", workspace=small)
    state = dd["h0"].clone()
    o_alias, _ = chunk_fwd(dd["q"], dd["k"], dd["v"], dd["z"], dd["beta"], state, gate="logits",
                           final_state=state)
    torch.cuda.synchronize()
    ref = oracle_forward(d["q"], d["k"], d["v"], d["z"], d["beta"], d["h0"], None, None, -5.0)
    for name, o, hT in (("split", o_split, hT_split), ("one chain", o_one, hT_one),
                        ("split, final state over initial", o_alias, state)):
        eo, es = rel_err(o, ref[0]), rel_err(hT, ref[1])
        print(f"  {name}: err_o={eo:.3e} err_state={es:.3e} tol={TOL_BF16:g}", flush=True)
        assert eo <= TOL_BF16 and es <= TOL_BF16
    # the split ran: its piece table opens the workspace (on a 256-CU device
    # the first-out schedule: 32 pieces of 512 tokens)
    table = wsp[:4 * 66].view(torch.int32).cpu().tolist()
    P = table.index(T)
    print(f"  pieces: P={P} table {table[:P + 1]}", flush=True)
    assert table[0] == 0 and 4 <= P <= 65
    assert all(0 < b - a and a % 64 == 0 for a, b in zip(table[:P], table[1:P + 1]))
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        want = _first_out_plan(T, 128)
        assert want == [p * 512 for p in range(33)]
        assert table[:P + 1] == want
    # With this gate a piece's state map underflows to zero within a few
    # tiles, so every piece starts from exactly the state the unsplit chain
    # has there and both paths give the same bits.
    assert torch.equal(o_split, o_one)


@pytest.mark.parametrize("T", [4096, 16384])
def test_split_with_slowly_decaying_state(T):
    """A gate near zero keeps the state alive across every piece, so the
    entry states come from the composed maps, not from underflow: the split
    (explicit and automatic) against the unsplit oracle. On a 256-CU device
    the automatic split of T = 4096 has 16 equal pieces, that of T = 16384
    is first-out (32 pieces of 512, the first with output on the second
    stream and the entry states of the others chained from its final
    state)."""
    _print_case(f"split, slow decay: dense B=1 H=2 T={T}, P = 8 and automatic")
    B, H = 1, 2
    d = make_inputs(B, T, H, 128, 128, torch.bfloat16, h0_std=0.02, seed=35)
    g = (-0.002 * torch.sigmoid(d["z"])).contiguous()  # per-token log-decay in [-0.002, 0]
    dd = to_dev(d)
    gd = g.cuda()
    o8, h8 = chunk_fwd_split(dd["q"], dd["k"], dd["v"], gd, dd["beta"], dd["h0"], None,
                             segments=8, gate="logdecay")
    oa, ha = chunk_fwd(dd["q"], dd["k"], dd["v"], gd, dd["beta"], dd["h0"], gate="logdecay")
    torch.cuda.synchronize()
    ref = oracle_recurrence(d["q"], d["k"], d["v"], g, d["beta"], d["h0"], None)
    for name, o, hT in (("explicit P=8", o8, h8), ("automatic", oa, ha)):
        eo, es = rel_err(o, ref[0]), rel_err(hT, ref[1])
        print(f"  {name}: err_o={eo:.3e} err_state={es:.3e} tol={TOL_BF16:g}", flush=True)
        assert eo <= TOL_BF16 and es <= TOL_BF16


@pytest.mark.parametrize("T", [4096, 20000])
@pytest.mark.parametrize("stress", ["g_min_everywhere", "g_zero", "beta_one", "large_values"])
def test_automatic_split_under_numeric_stress(T, stress):
    """Extreme inputs through kda_chunk_fwd's automatic split (dense B=1, H=2,
    initial state; on a 256-CU device T = 4096 takes 16 equal pieces and
    T = 20000 the first-out schedule): the gate at its lower bound on every
    token (largest in-tile reciprocals), no decay at all (every piece's state
    map stays a product of (I - beta k k^T), so each entry state depends on
    the whole history through the composition), every token fully written,
    and values 100 times larger. Every element against the unsplit oracle."""
    _print_case(f"automatic split under stress {stress}: B=1 H=2 T={T}")
    d = make_inputs(1, T, 2, 128, 128, torch.bfloat16, h0_std=0.02, seed=39)
    if stress == "g_min_everywhere":
        d["z"] = torch.full_like(d["z"], 40.0)        # sigmoid -> 1, g = g_min
    elif stress == "g_zero":
        d["z"] = torch.full_like(d["z"], -200.0)      # sigmoid -> 0, g = 0
    elif stress == "beta_one":
        d["beta"] = torch.ones_like(d["beta"])
    elif stress == "large_values":
        d["v"] = (d["v"].float() * 100).to(torch.bfloat16)
    dd = to_dev(d)
    o, hT = chunk_fwd(dd["q"], dd["k"], dd["v"], dd["z"], dd["beta"], dd["h0"], gate="logits")
    torch.cuda.synchronize()
    ref = oracle_forward(d["q"], d["k"], d["v"], d["z"], d["beta"], d["h0"], None, None, -5.0)
    eo, es = rel_err(o, ref[0]), rel_err(hT, ref[1])
    print(f"  err_o={eo:.3e} err_state={es:.3e} tol={TOL_BF16:g}", flush=True)
    assert eo <= TOL_BF16 and es <= TOL_BF16

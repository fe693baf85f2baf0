"""kda_chunk_fwd_noalloc (the forward for callers that cannot allocate: its
workspace is the library's static device scratch) against kda_chunk_fwd with
a workspace of the size the query asks for, called through the C ABI, on
consecutive calls with shrinking inputs, so the second call sees the first
call's leftovers in the shared scratch. Both must meet the oracle's bar and
agree with each other to it: where kda_chunk_fwd splits with its first piece
on a second stream, kda_chunk_fwd_noalloc (which creates no stream) takes the
equal-piece split, whose rounding may differ; elsewhere they run the same
kernels and give the same bits."""
import ctypes

import pytest
import torch

from gated_delta_rule_92_amd import _lib, chunk_fwd
from gated_delta_rule_92_amd.inputs import make_inputs
from gated_delta_rule_92_amd.ops import _ptr, _stream
from oracle import oracle_forward
from tests.gpu_helpers import TOL_BF16, rel_err, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _noalloc(dd, o, hT):
    lib = _lib.load()
    cu = dd["cu_seqlens"]
    B, T, H, Dk = dd["q"].shape
    Dv = dd["v"].shape[-1]
    N = B if cu is None else cu.numel() - 1
    return lib.kda_chunk_fwd_noalloc(_ptr(dd["q"]), _ptr(dd["k"]), _ptr(dd["v"]),
                                     _lib.KDA_BFLOAT16, _ptr(dd["z"]), _lib.KDA_GATE_LOGITS, None,
                                     -5.0, _ptr(dd["beta"]), _ptr(dd["h0"]), _ptr(cu), N, B, T, H,
                                     Dk, Dv, 64, 1.0, _ptr(o), _ptr(hT),
                                     _stream(torch.device("cuda")))


CALLS = [  # (label, B, T, H, lengths): a context split of 16 pieces, then of 8, then packed
    ("dense B=1 H=16 T=4096 (split, 16 pieces)", 1, 4096, 16, None),
    ("dense B=1 H=16 T=2048 (split, 8 pieces)", 1, 2048, 16, None),
    ("packed 5 sequences H=4 (longest-first order)", 1, 0, 4, [300, 0, 17, 130, 64]),
]


def test_noalloc_matches_chunk_fwd_on_consecutive_calls():
    for i, (label, B, T, H, lengths) in enumerate(CALLS):
        print(f"\n[case] noalloc call {i}: {label}", flush=True)
        d = make_inputs(B, T, H, 128, 128, torch.bfloat16, h0_std=0.02, lengths=lengths,
                        seed=40 + i)
        dd = to_dev(d)
        o = torch.full_like(dd["v"], float("nan"))
        hT = torch.full((d["N"], H, 128, 128), float("nan"), device="cuda")
        assert _noalloc(dd, o, hT) == _lib.KDA_SUCCESS
        o_ref, hT_ref = chunk_fwd(dd["q"], dd["k"], dd["v"], dd["z"], dd["beta"], dd["h0"],
                                  dd["cu_seqlens"], gate="logits")
        torch.cuda.synchronize()
        same = torch.equal(o, o_ref) and torch.equal(hT, hT_ref)
        do, ds = rel_err(o, o_ref.double().cpu()), rel_err(hT, hT_ref.double().cpu())
        ref = oracle_forward(d["q"], d["k"], d["v"], d["z"], d["beta"], d["h0"], d["cu_seqlens"],
                             None, -5.0)
        eo, es = rel_err(o, ref[0]), rel_err(hT, ref[1])
        print(f"  vs kda_chunk_fwd: same bits {same}, o {do:.3e}, state {ds:.3e}; "
              f"vs oracle: err_o={eo:.3e} err_state={es:.3e}", flush=True)
        assert do <= TOL_BF16 and ds <= TOL_BF16
        if lengths is not None:  # packed sequences: no split, the same kernels
            assert same
        assert eo <= TOL_BF16 and es <= TOL_BF16


def test_automatic_splits_fit_the_scratch():
    """The workspace the size query asks for (what the no-allocation entry
    point takes from its scratch) fits the 64 MiB scratch for the automatic
    splits of the 4096-token (16 pieces of 16 heads) and 256K-token (8 equal
    pieces for this entry point, 9 for kda_chunk_fwd's first-out schedule;
    the query asks for the larger) single sequences on this device. (Sizes beyond the scratch
    are rejected before anything is enqueued; that path needs a device with
    more compute units and is exercised by the host-check build.)"""
    lib = _lib.load()
    for (T, H) in ((4096, 16), (262144, 32)):
        n = ctypes.c_size_t(0)
        assert lib.kda_chunk_fwd_workspace_size(1, T, H, 128, 128, 1, 64, _lib.KDA_BFLOAT16,
                                                ctypes.byref(n)) == 0
        print(f"  T={T} H={H}: workspace {n.value} bytes", flush=True)
        assert 0 < n.value <= (64 << 20)

"""Device-side failure reporting (kda_device_status): failures only the
device can see reach the host through the device's flags word.

- A bounded producer/consumer wait that gives up: the spin limit is lowered
  from the host (kda_debug_set_spin_limit) so that the waits of the
  pipelined kernel give up at once; every kernel still finishes (a workgroup
  that gave up stops waiting) and KDA_DEVICE_WAIT_TIMEOUT is reported.
- A per-token log-decay below -5.5 passed directly (log-decay or cumsum
  input): a 16-token tile's reciprocal decay factors overflow, and
  KDA_DEVICE_DECAY_OUT_OF_RANGE is reported ([Baidu-1] "Kimi K3 Core
  Techniques Explained ...", §1.2: the gate's lower bound keeps 16-token
  tiles finite). Both chunk kernels (pipelined bf16 d = 128, tile kernel for
  other shapes) report it.
After each case the flags are cleared, and a valid call leaves them clear and
meets the oracle's bar."""
import pytest
import torch

from gated_delta_rule_92_amd import chunk_fwd, debug_set_spin_limit, device_status, gate
from gated_delta_rule_92_amd._lib import KDA_DEVICE_DECAY_OUT_OF_RANGE, KDA_DEVICE_WAIT_TIMEOUT
from gated_delta_rule_92_amd.inputs import make_inputs
from oracle import oracle_forward
from tests.gpu_helpers import rel_err, to_dev, tol_for

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _print_case(name):
    print(f"\n[case] {name}", flush=True)


def _valid_call_is_clean(dtype=torch.bfloat16, D=128):
    d = make_inputs(1, 200, 2, D, D, dtype, h0_std=0.02, seed=50)
    dd = to_dev(d)
    o, hT = chunk_fwd(dd["q"], dd["k"], dd["v"], dd["z"], dd["beta"], dd["h0"], gate="logits")
    torch.cuda.synchronize()
    assert device_status() == 0
    ref = oracle_forward(d["q"], d["k"], d["v"], d["z"], d["beta"], d["h0"], None, None, -5.0)
    assert rel_err(o, ref[0]) <= tol_for(dtype) and rel_err(hT, ref[1]) <= tol_for(dtype)


def test_wait_give_up_is_reported():
    _print_case("spin limit 1: the pipelined kernel's waits give up")
    device_status(clear=True)
    _valid_call_is_clean()
    d = make_inputs(2, 300, 2, 128, 128, torch.bfloat16, h0_std=0.02, seed=51)
    dd = to_dev(d)
    try:
        debug_set_spin_limit(1)
        chunk_fwd(dd["q"], dd["k"], dd["v"], dd["z"], dd["beta"], dd["h0"], gate="logits")
        torch.cuda.synchronize()
    finally:
        debug_set_spin_limit(0)
    flags = device_status(clear=True)
    print(f"  flags={flags:#x}", flush=True)
    assert flags & KDA_DEVICE_WAIT_TIMEOUT
    assert device_status() == 0
    _valid_call_is_clean()


@pytest.mark.parametrize("dtype,Dk,Dv", [(torch.bfloat16, 128, 128), (torch.bfloat16, 64, 64),
                                         (torch.float32, 64, 64)])
@pytest.mark.parametrize("mode", ["logdecay", "cumsum"])
def test_log_decay_below_the_bound_is_reported(dtype, Dk, Dv, mode):
    _print_case(f"log-decay -6 passed as {mode}, {dtype} Dk={Dk} Dv={Dv}")
    device_status(clear=True)
    d = make_inputs(1, 100, 2, Dk, Dv, dtype, h0_std=0.02, seed=52)
    dd = to_dev(d)
    g6 = torch.full_like(dd["z"], -6.0)
    g = g6 if mode == "logdecay" else gate(torch.full_like(dd["z"], 60.0), None, -6.0, 64)
    if mode == "cumsum":
        assert abs(float(g[0, 15, 0, 0]) - (-96.0)) < 1e-3    # 16 tokens at -6
    chunk_fwd(dd["q"], dd["k"], dd["v"], g, dd["beta"], dd["h0"], gate=mode)
    torch.cuda.synchronize()
    flags = device_status(clear=True)
    print(f"  flags={flags:#x}", flush=True)
    assert flags & KDA_DEVICE_DECAY_OUT_OF_RANGE
    # the same sizes with a log-decay inside the bound: nothing reported
    g5 = torch.full_like(dd["z"], -5.5)
    chunk_fwd(dd["q"], dd["k"], dd["v"], g5 if mode == "logdecay" else gate(
        torch.full_like(dd["z"], 60.0), None, -5.5, 64), dd["beta"], dd["h0"], gate=mode)
    torch.cuda.synchronize()
    assert device_status() == 0

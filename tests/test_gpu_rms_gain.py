"""GPU parity of the RMSNorm gain's gradient (vdn_vda_backward_readout with
d_rms_weight) against the oracle's (oracle/vda_grad.py: the float64 autograd
of the forward, pinned by finite differences), with the tolerance of the other
bfloat16 gradients (max relative error <= 2e-2 over the d_v vector).

The same call must leave dq and dgate bit for bit as the call without the gain
gradient makes them (the same arithmetic, in the same order), and two calls
must give the same gradient bit for bit (it is summed in a fixed order)."""

import numpy as np
import pytest

from oracle import vda_grad
from frame_wise_delta_02_amd import synth
import gpu_harness as G
import test_gpu_backward as GB

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_case(request):
    G.say(request.node.nodeid)
    yield


# every head width; a given gain and none (a gain of ones); the bridge, the
# raw query, two batches; and the 768p frame size on two heads
CASES = ["bwd_128_gain", "bwd_128", "bwd_64_bridge", "bwd_32", "bwd_16", "bwd_64_ql2_gain", "bwd_B2_chunk3",
         "bwd_T1", "768p_two_heads"]


def _case(name):
    if name == "768p_two_heads":
        return dict(w=GB.BASE.scaled(name=name, H=2), gain=True)
    return GB.CASES[name]


@pytest.mark.parametrize("name", CASES)
def test_gain_gradient(name):
    import torch
    from frame_wise_delta_02_amd import binding as bd
    case = _case(name)
    w, bridge, ql2 = case["w"], case.get("bridge", False), case.get("query_l2", False)
    x = synth.make_inputs(w)
    if ql2:
        GB._raw_queries(x, w)
    dy = GB._dy(w)
    rw = np.random.default_rng(5).uniform(0.5, 1.5, w.d) if case.get("gain") else None
    out, ws, desc, dev = G.run_forward(x, w, epilogue=True, rms_weight=rw, bridge=bridge, query_l2=ql2)
    dy_d = G.to_device(dy, w.dtype)
    rw_d = None if rw is None else torch.from_numpy(rw.astype(np.float32)).cuda()
    kw = dict(grid=(w.grid_h, w.grid_w), n_text=w.L, chunk=w.chunk, epilogue=True, bridge=bridge, query_l2=ql2,
              l2_eps=GB.L2_EPS)
    G.say(f"backward_readout {name} without the gain gradient")
    dq0, dg0, _ = bd.backward_readout(dev["q"], dev["gate"], rw_d, dev["alpha"], dy_d, ws, **kw)
    torch.cuda.synchronize()
    got = []
    for i in range(2):
        G.say(f"backward_readout {name} with the gain gradient, call {i + 1}")
        dgamma = torch.full((w.d,), float("nan"), dtype=torch.float32, device="cuda")
        dq, dg, _ = bd.backward_readout(dev["q"], dev["gate"], rw_d, dev["alpha"], dy_d, ws, d_rms_weight=dgamma,
                                        **kw)
        torch.cuda.synchronize()
        assert torch.equal(dq.view(torch.int16), dq0.view(torch.int16)), "dq changed"
        assert torch.equal(dg.view(torch.int16), dg0.view(torch.int16)), "dgate changed"
        got.append(dgamma.cpu().numpy().astype(np.float64))
    assert np.array_equal(got[0], got[1]), "two calls differ"
    f = G.oracle_view({k: x[k] for k in ("q", "k", "v", "beta", "k_text", "v_text", "beta_text", "gate")}, w)
    gain = rw if rw is not None else np.ones(w.d)
    ref = vda_grad.backward(f["q"], f["k"], f["v"], x["alpha"].astype(np.float64), f["beta"], f["k_text"],
                            f["v_text"], f["beta_text"], G.oracle_view({"dy": dy}, w)["dy"], gate=f["gate"],
                            rms_weight=gain, chunk=w.chunk, bridge=bridge, query_l2=GB.L2_EPS if ql2 else None)
    err = GB._rel(got[0], ref["dgamma"])
    G.say(f"{name}: dgamma max rel err {err:.3e}")
    assert err <= G.TOL["bf16"], err

"""selective_scan under torch autograd: its gradients are the backward entry point's, bit for
bit (the workspace path is reproducible), for every differentiable input, with and without
a padding mask, and when only part of the inputs need gradients or only one output is used.
The backward entry point itself is checked against the float64 oracle in test_gpu_bwd.py."""
import numpy as np
import pytest

import selective_scan_fwd_amd as ssm
from gpu_util import announce, dev, torch
from ssm_workloads import WORKLOADS, make_inputs, make_mask

pytestmark = pytest.mark.gpu

NAMES = ("u", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")


def leaves(inp, io, requires=NAMES):
    t = {k: dev(inp[k], io) for k in ("u", "delta", "B", "C", "z")}
    t.update({k: dev(inp[k], "f32") for k in ("A", "D", "delta_bias", "h0")})
    for k in requires:
        t[k].requires_grad_(True)
    return t


def same(a, b):
    t = torch()
    if a.dtype == t.bfloat16:
        a, b = a.view(t.int16), b.view(t.int16)
    return bool(t.equal(a, b))


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("masked", [False, True])
def test_autograd_equals_backward_entry(io, masked):
    t = torch()
    w = WORKLOADS["tiny"].with_(batch=2, dim=24, dstate=16, seqlen=700, io=io, gate=True,
                                initial_state=True, seed=80)
    announce(f"{w.describe()} autograd masked={masked}")
    inp = make_inputs(w)
    mask = t.from_numpy(make_mask(w.batch, w.seqlen, "random", seed=81)).cuda() if masked else None
    x = leaves(inp, io)
    out, fin = ssm.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"],
                                  z=x["z"], delta_bias=x["delta_bias"], delta_softplus=True,
                                  h0=x["h0"], mask=mask)
    gen = t.Generator(device="cuda")
    gen.manual_seed(82)
    wout = t.randn(out.shape, device="cuda", generator=gen).to(out.dtype)
    wfin = t.randn(fin.shape, device="cuda", generator=gen)
    ((out.float() * wout.float()).sum() + (fin * wfin).sum()).backward()

    d = {k: v.detach() for k, v in x.items()}
    _, _, states = ssm.scan_train(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                                  z=d["z"], delta_bias=d["delta_bias"], delta_softplus=True,
                                  h0=d["h0"], mask=mask)
    g = ssm.scan_backward(d["u"], d["delta"], d["A"], d["B"], d["C"], states, wout, D=d["D"],
                          z=d["z"], delta_bias=d["delta_bias"], delta_softplus=True,
                          dfinal=wfin, mask=mask)
    want = {"u": g["du"], "delta": g["ddelta"], "A": g["dA"], "B": g["dB"].to(x["B"].dtype),
            "C": g["dC"].to(x["C"].dtype), "D": g["dD"], "z": g["dz"],
            "delta_bias": g["dbias"], "h0": g["dh0"]}
    for k in NAMES:
        assert x[k].grad is not None, k
        assert x[k].grad.dtype == x[k].dtype, k
        assert same(x[k].grad, want[k]), f"{k}: autograd gradient differs"
    print(f"[autograd] {w.describe()} masked={masked}: nine gradients bitwise equal", flush=True)


def test_autograd_partial_inputs_and_outputs():
    """Only u and A need gradients and only final_state enters the loss: their gradients
    equal the entry point's with dout = 0; the other inputs get none."""
    t = torch()
    w = WORKLOADS["tiny"].with_(batch=1, dim=16, dstate=8, seqlen=900, io="bf16", gate=True,
                                initial_state=True, seed=83)
    announce(f"{w.describe()} autograd partial")
    inp = make_inputs(w)
    x = leaves(inp, "bf16", requires=("u", "A"))
    out, fin = ssm.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"],
                                  z=x["z"], delta_bias=x["delta_bias"], delta_softplus=True,
                                  h0=x["h0"])
    fin.sum().backward()
    d = {k: v.detach() for k, v in x.items()}
    _, _, states = ssm.scan_train(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                                  z=d["z"], delta_bias=d["delta_bias"], delta_softplus=True,
                                  h0=d["h0"])
    g = ssm.scan_backward(d["u"], d["delta"], d["A"], d["B"], d["C"], states,
                          t.zeros_like(d["u"]), D=d["D"], z=d["z"], delta_bias=d["delta_bias"],
                          delta_softplus=True, dfinal=t.ones_like(fin), want_dh0=False)
    assert same(x["u"].grad, g["du"]) and same(x["A"].grad, g["dA"])
    for k in ("delta", "B", "C", "D", "z", "delta_bias", "h0"):
        assert x[k].grad is None, k
    assert np.isfinite(x["u"].grad.float().cpu().numpy()).all()

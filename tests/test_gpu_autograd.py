"""selective_scan under torch autograd: its gradients are the backward entry point's, bit for
bit (the workspace path is reproducible), for every differentiable input, with and without
a padding mask, and when only part of the inputs need gradients or only one output is used.
The backward entry point itself is checked against the float64 oracle in test_gpu_bwd.py."""
import numpy as np
import pytest

import selective_state_space_fwd_amd as ssm
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


def test_strided_inputs_are_copied():
    """Strided views (B and C as slices of a [batch, seqlen, 2N] projection, u transposed)
    give bitwise the same results as contiguous copies, through scan, selective_scan and
    scan_backward."""
    t = torch()
    w = WORKLOADS["tiny"].with_(batch=2, dim=12, dstate=16, seqlen=300, io="bf16", gate=True,
                                initial_state=True, seed=84)
    announce(f"{w.describe()} strided inputs")
    inp = make_inputs(w)
    x = leaves(inp, "bf16", requires=())
    proj = t.cat([x["B"].transpose(1, 2), x["C"].transpose(1, 2)], dim=2).contiguous()
    Bv, Cv = proj[..., :w.dstate].transpose(1, 2), proj[..., w.dstate:].transpose(1, 2)
    uv = x["u"].transpose(1, 2).contiguous().transpose(1, 2)
    assert not (Bv.is_contiguous() or Cv.is_contiguous() or uv.is_contiguous())
    kw = dict(D=x["D"], z=x["z"], delta_bias=x["delta_bias"], delta_softplus=True, h0=x["h0"])
    o1, f1 = ssm.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], **kw)
    o2, f2 = ssm.scan(uv, x["delta"], x["A"], Bv, Cv, **kw)
    assert same(o1, o2) and same(f1, f2)
    _, _, st = ssm.scan_train(x["u"], x["delta"], x["A"], x["B"], x["C"], **kw)
    dout = t.ones_like(o1)
    kb = dict(D=x["D"], z=x["z"], delta_bias=x["delta_bias"], delta_softplus=True)
    g1 = ssm.scan_backward(x["u"], x["delta"], x["A"], x["B"], x["C"], st, dout, **kb)
    g2 = ssm.scan_backward(uv, x["delta"], x["A"], Bv, Cv, st, dout.transpose(1, 2).contiguous()
                           .transpose(1, 2), **kb)
    for k, v in g1.items():
        if v is not None:
            assert same(v, g2[k]), k

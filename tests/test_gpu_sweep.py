"""A seeded sweep of random shapes and option sets through every entry point, against the
float64 oracles: the hand-picked cases of the other GPU tests cover the boundaries one at a
time; here sizes (ragged tails, one-step and short sequences, odd channel and state counts)
and optional inputs (D, z, bias, softplus, h0, padding mask) are drawn together, so that
combinations nobody listed are exercised too. Every case is small enough for the oracle to
finish in well under a second, and each is named before its GPU step."""
import numpy as np
import pytest

import oracle
import selective_state_space_fwd_amd as ssm
from gpu_util import announce, dev, host, torch
from ssm_workloads import (RTOL, WATCH, RTOL_STATE, SSD_WORKLOADS, WORKLOADS, f32_to_bf16_bits,
                           make_inputs, make_mask, make_ssd_inputs, parity, widen)

pytestmark = pytest.mark.gpu

RTOL_F32_OUT = 1e-4


def draw_scan_case(i):
    r = np.random.default_rng(9000 + i)
    io = ("f32", "bf16")[i % 2]
    seqlen = int(r.integers(1, 33)) if r.random() < 0.3 else int(r.integers(33, 2600))
    dstate = int(r.choice([1, 2, 3, 4, 7, 8, 15, 16, 17, 24, 32, 40, 63, 64]))
    opts = {k: bool(r.random() < 0.7) for k in ("D", "z", "bias", "softplus", "h0")}
    opts["mask"] = bool(r.random() < 0.3)
    return dict(io=io, batch=int(r.integers(1, 4)), dim=int(r.integers(1, 41)), dstate=dstate,
                seqlen=seqlen, seed=9100 + i, **opts)


def scan_inputs(c):
    w = WORKLOADS["tiny"].with_(batch=c["batch"], dim=c["dim"], dstate=c["dstate"],
                                seqlen=c["seqlen"], io=c["io"], gate=True,
                                initial_state=c["h0"], a_kind="scaled", seed=c["seed"])
    inp = make_inputs(w)
    if not c["D"]:
        inp["D"] = None
    if not c["z"]:
        inp["z"] = None
    if not c["bias"]:
        inp["delta_bias"] = None
    if not c["softplus"]:  # delta is then the step size itself: keep it positive and small
        raw = np.abs(widen(inp["delta"], c["io"])) * 0.05 + 1e-3
        inp["delta"] = raw.astype(np.float32) if c["io"] == "f32" else f32_to_bf16_bits(raw)
        if inp["delta_bias"] is not None:
            inp["delta_bias"] = np.abs(inp["delta_bias"]) * 0.01
    mask = make_mask(c["batch"], c["seqlen"], "random", seed=c["seed"]) if c["mask"] else None
    return w, inp, mask


def label(c):
    opts = "".join(k[0] if c[k] else "-" for k in ("D", "z", "bias", "softplus", "h0", "mask"))
    return (f"b{c['batch']}d{c['dim']}N{c['dstate']}L{c['seqlen']} {c['io']} opts={opts} "
            f"seed={c['seed']}")


def widened(inp, io):
    return {k: (None if inp[k] is None else
                (widen(inp[k], io) if k in ("u", "delta", "B", "C", "z") else inp[k]))
            for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")}


def on_device(inp, io, mask):
    g = {k: dev(inp[k], io) for k in ("u", "delta", "B", "C", "z")}
    g.update({k: dev(inp[k], "f32") for k in ("A", "D", "delta_bias", "h0")})
    g["mask"] = None if mask is None else torch().from_numpy(mask).cuda()
    return g


@pytest.mark.parametrize("i", range(100))
def test_sweep_forward(i):
    c = draw_scan_case(i)
    announce("forward " + label(c))
    w, inp, mask = scan_inputs(c)
    g = on_device(inp, c["io"], mask)
    out, fin = ssm.scan(g["u"], g["delta"], g["A"], g["B"], g["C"], D=g["D"], z=g["z"],
                        delta_bias=g["delta_bias"], delta_softplus=c["softplus"], h0=g["h0"],
                        mask=g["mask"])
    torch().cuda.synchronize()
    x = widened(inp, c["io"])
    ref_out, ref_fin = oracle.scan_ref(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"],
                                       x["delta_bias"], c["softplus"], x["h0"], mask=mask)
    ro = parity(host(out), ref_out, RTOL[c["io"]], WATCH[c["io"]])
    rf = parity(host(fin), ref_fin, RTOL_STATE)
    print(f"[sweep] forward {label(c)}: out {ro} | final {rf}", flush=True)
    assert ro.ok and rf.ok, f"{label(c)}: out {ro} final {rf}"


@pytest.mark.parametrize("i", range(32))
def test_sweep_backward(i):
    c = draw_scan_case(100 + i)
    c["seqlen"] = max(c["seqlen"], 1)
    announce("backward " + label(c))
    w, inp, mask = scan_inputs(c)
    io = c["io"]
    g = on_device(inp, io, mask)
    r = np.random.default_rng(c["seed"] + 1)
    dout = r.standard_normal(inp["u"].shape).astype(np.float32)
    dout = dout if io == "f32" else f32_to_bf16_bits(dout)
    dfin = r.standard_normal((c["batch"], c["dim"], c["dstate"])).astype(np.float32)
    _, _, states = ssm.scan_train(g["u"], g["delta"], g["A"], g["B"], g["C"], D=g["D"], z=g["z"],
                                  delta_bias=g["delta_bias"], delta_softplus=c["softplus"],
                                  h0=g["h0"], mask=g["mask"])
    grads = ssm.scan_backward(g["u"], g["delta"], g["A"], g["B"], g["C"], states, dev(dout, io),
                              D=g["D"], z=g["z"], delta_bias=g["delta_bias"],
                              delta_softplus=c["softplus"], dfinal=dev(dfin, "f32"),
                              mask=g["mask"])
    torch().cuda.synchronize()
    x = widened(inp, io)
    ref = oracle.scan_bwd_ref(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"],
                              x["delta_bias"], c["softplus"], x["h0"], widen(dout, io),
                              dfin.astype(np.float64), mask=mask)
    for k, want in ref.items():
        if want is None:
            assert grads.get(k) is None, f"{label(c)}: {k} should be absent"
            continue
        per_element = k in ("du", "ddelta", "dz")
        rtol = RTOL[io] if per_element else RTOL_F32_OUT
        rep = parity(host(grads[k]), want, rtol, WATCH[io] if per_element else None)
        print(f"[sweep] backward {label(c)} {k}: {rep}", flush=True)
        assert rep.ok, f"{label(c)} {k}: {rep}"


@pytest.mark.parametrize("i", range(24))
def test_sweep_ssd(i):
    r = np.random.default_rng(9500 + i)
    w = SSD_WORKLOADS["ssd_tiny"].with_(
        batch=int(r.integers(1, 3)), nheads=int(r.integers(1, 5)),
        headdim=int(r.choice([16, 32, 48, 64, 80])), dstate=int(r.choice([64, 128, 256])),
        seqlen=int(r.integers(1, 33)) if r.random() < 0.25 else int(r.integers(33, 900)),
        initial_state=bool(r.random() < 0.6), seed=9600 + i)
    use = {k: bool(r.random() < 0.7) for k in ("D", "z", "dt_bias", "softplus")}
    masked = bool(r.random() < 0.3)
    name = f"{w.describe()} opts={''.join(k[0] if v else '-' for k, v in use.items())}" \
           f"{'m' if masked else '-'}"
    announce("ssd " + name)
    inp = make_ssd_inputs(w)
    for k in ("D", "z", "dt_bias"):
        if not use[k]:
            inp[k] = None
    if not use["softplus"]:
        raw = np.abs(widen(inp["dt"], "bf16")) * 0.05 + 1e-3
        inp["dt"] = f32_to_bf16_bits(raw)
        if inp["dt_bias"] is not None:
            inp["dt_bias"] = np.abs(inp["dt_bias"]) * 0.01
    mask = make_mask(w.batch, w.seqlen, "random", seed=w.seed) if masked else None
    g = {k: dev(inp[k], "bf16") for k in ("x", "dt", "B", "C", "z")}
    f = {k: dev(inp[k], "f32") for k in ("A", "D", "dt_bias", "h0")}
    out, fin = ssm.ssd(g["x"], g["dt"], f["A"], g["B"], g["C"], D=f["D"], z=g["z"],
                       dt_bias=f["dt_bias"], dt_softplus=use["softplus"], h0=f["h0"],
                       mask=None if mask is None else torch().from_numpy(mask).cuda())
    torch().cuda.synchronize()
    wd = lambda k: None if inp[k] is None else widen(inp[k], "bf16")
    ref_out, ref_fin = oracle.ssd_ref(wd("x"), wd("dt"), inp["A"], wd("B"), wd("C"), inp["D"],
                                      wd("z"), inp["dt_bias"], use["softplus"], inp["h0"],
                                      mask=mask)
    ro, rf = parity(host(out), ref_out, RTOL["bf16"]), parity(host(fin), ref_fin, RTOL_STATE)
    print(f"[sweep] ssd {name}: out {ro} | final {rf}", flush=True)
    assert ro.ok and rf.ok, f"{name}: out {ro} final {rf}"

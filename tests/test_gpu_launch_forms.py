"""The two launch forms of the fp32 chunked scan, each forced through the
SSM_WAVES_PER_CHANNEL_* hint, against the float64 oracle.

fp32 launches split each channel's states over two waves when every workgroup fits on the
device at once, and use one wave per channel otherwise; the small shapes the other tests use
all take the split form on their own. Here both forms run on the same inputs: vector rows
(whole 16-byte words) and element-wise rows (odd lengths), several chunks with an initial
state and the gate, 1, 17 and 64 states, a padding mask, and the training forward followed by
the backward. The two forms scan every state in the same order, so final and saved states
must be bitwise equal between them; y is summed over the states in another order, so outputs
agree to float32 rounding.

Bar: the parity metric of ssm_workloads.compare, rtol 1e-4 (float32 storage) on out,
final_state, the saved states and every gradient.
"""
import numpy as np
import pytest

import oracle
import selective_state_space_fwd_amd as ssm
from gpu_util import announce, dev, host, run_hip, torch
from ssm_workloads import RTOL, RTOL_STATE, WORKLOADS, make_inputs, make_mask, parity, widen

pytestmark = pytest.mark.gpu

FORMS = [1, 2]
SHAPES = [
    # (batch, dim, dstate, seqlen): vector rows (L % 4 == 0) and element-wise rows (odd L),
    # one and several 1024-step chunks, ragged tails, 1 / 17 / 64 states
    (2, 5, 16, 600), (1, 6, 16, 1024), (2, 3, 16, 1537), (1, 4, 17, 1537), (1, 5, 1, 777),
    (1, 3, 64, 2100), (2, 9, 16, 63), (1, 7, 16, 4099),
]


def _oracle(inp, mask=None):
    io = inp["io"]
    return oracle.scan_ref(widen(inp["u"], io), widen(inp["delta"], io), inp["A"],
                           widen(inp["B"], io), widen(inp["C"], io), inp["D"],
                           widen(inp["z"], io), inp["delta_bias"], True, inp["h0"], mask=mask)


def _check(got_out, got_fin, ref, label):
    ro = parity(got_out, ref[0], RTOL["f32"])
    rf = parity(got_fin, ref[1], RTOL_STATE)
    print(f"[forms] {label}: out {ro} | final {rf}", flush=True)
    assert ro.ok and rf.ok, label


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}d{}N{}L{}".format(*s))
def test_forms_against_the_oracle_and_each_other(shape):
    b, d, n, L = shape
    w = WORKLOADS["tiny"].with_(batch=b, dim=d, dstate=n, seqlen=L, io="f32", gate=True,
                                initial_state=True, a_kind="scaled" if n != 16 else "s4d",
                                seed=900 + L + n)
    inp = make_inputs(w)
    ref = _oracle(inp)
    res = {}
    for k in FORMS:
        announce(f"{w.describe()} waves_per_channel={k}")
        res[k] = run_hip(inp, waves_per_channel=k)
        _check(*res[k], ref, f"{w.describe()} form {k}")
    assert np.array_equal(res[1][1], res[2][1]), "final states differ between the forms"
    rep = parity(res[1][0], res[2][0], 1e-5)
    assert rep.ok, f"outputs of the two forms: {rep}"


@pytest.mark.parametrize("kind", ["lengths", "random"])
@pytest.mark.parametrize("form", FORMS)
def test_forms_with_a_padding_mask(form, kind):
    w = WORKLOADS["tiny"].with_(batch=3, dim=5, dstate=16, seqlen=1537, io="f32", gate=True,
                                initial_state=True, seed=940)
    announce(f"{w.describe()} mask {kind} waves_per_channel={form}")
    inp = make_inputs(w)
    mask = make_mask(w.batch, w.seqlen, kind, seed=941)
    g = {k: dev(inp[k], "f32") for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias",
                                         "h0")}
    out, fin = ssm.scan(g["u"], g["delta"], g["A"], g["B"], g["C"], D=g["D"], z=g["z"],
                        delta_bias=g["delta_bias"], delta_softplus=True, h0=g["h0"],
                        mask=torch().from_numpy(mask).cuda(), waves_per_channel=form)
    torch().cuda.synchronize()
    _check(host(out), host(fin), _oracle(inp, mask), f"{w.describe()} mask {kind} form {form}")


def test_forms_training_forward_then_backward():
    """scan_train in each form (bitwise the same saved and final states), then the backward
    from those states against the backward oracle."""
    w = WORKLOADS["tiny"].with_(batch=2, dim=6, dstate=16, seqlen=1537, io="f32", gate=True,
                                initial_state=True, seed=950)
    inp = make_inputs(w)
    rng = np.random.default_rng(951)
    dout = rng.standard_normal(inp["u"].shape).astype(np.float32)
    dfin = rng.standard_normal((w.batch, w.dim, w.dstate)).astype(np.float32)
    g = {k: dev(inp[k], "f32") for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias",
                                         "h0")}
    ref = oracle.scan_bwd_ref(widen(inp["u"], "f32"), widen(inp["delta"], "f32"), inp["A"],
                              widen(inp["B"], "f32"), widen(inp["C"], "f32"), inp["D"],
                              widen(inp["z"], "f32"), inp["delta_bias"], True, inp["h0"],
                              dout.astype(np.float64), dfin.astype(np.float64))
    saved = {}
    for form in FORMS:
        announce(f"{w.describe()} training forward + backward waves_per_channel={form}")
        out, fin, states = ssm.scan_train(g["u"], g["delta"], g["A"], g["B"], g["C"], D=g["D"],
                                          z=g["z"], delta_bias=g["delta_bias"],
                                          delta_softplus=True, h0=g["h0"],
                                          waves_per_channel=form)
        grads = ssm.scan_backward(g["u"], g["delta"], g["A"], g["B"], g["C"], states,
                                  dev(dout, "f32"), D=g["D"], z=g["z"],
                                  delta_bias=g["delta_bias"], delta_softplus=True,
                                  dfinal=dev(dfin, "f32"))
        torch().cuda.synchronize()
        saved[form] = (host(fin), host(states))
        _check(host(out), host(fin), _oracle(inp), f"{w.describe()} training form {form}")
        for k, r in ref.items():
            if r is None:
                continue
            rep = parity(host(grads[k]), r, RTOL["f32"])
            print(f"[forms] backward form {form} {k}: {rep}", flush=True)
            assert rep.ok, f"form {form} {k}: {rep}"
    assert np.array_equal(saved[1][0], saved[2][0])
    assert np.array_equal(saved[1][1], saved[2][1])


def test_automatic_choice_matches_a_forced_form():
    """With no hint the library picks one of the two forms: its outputs are bitwise those of
    one forced form (which one depends on the device's compute-unit count)."""
    w = WORKLOADS["tiny"].with_(batch=2, dim=40, dstate=16, seqlen=1100, io="f32", gate=True,
                                initial_state=True, seed=960)
    announce(f"{w.describe()} automatic form")
    inp = make_inputs(w)
    auto = run_hip(inp)
    forced = [run_hip(inp, waves_per_channel=k) for k in FORMS]
    assert any(np.array_equal(auto[0], f[0]) and np.array_equal(auto[1], f[1]) for f in forced)


@pytest.mark.parametrize("n", [16, 8, 17])
def test_six_channel_two_wave_shape(n):
    """1 100 channels: too many for the two-wave form in four-channel workgroups to run in
    one round on a 256-CU device, few enough in six-channel ones, which the library then
    takes (late input loads, three waves per SIMD, each wave forming the step sizes of half
    of a lane's steps). The states are scanned as in the forced two-wave launch (four-channel
    workgroups), so the final state is bitwise that launch's; the D skip joins y in the other
    wave's share for half of the steps, so out agrees to float32 rounding; both against the
    oracle; the training forward writes the same out bit for bit."""
    w = WORKLOADS["tiny"].with_(batch=1, dim=1100, dstate=n, seqlen=1100, io="f32", gate=True,
                                initial_state=True, a_kind="scaled" if n != 16 else "s4d",
                                seed=970 + n)
    announce(f"{w.describe()} six-channel two-wave shape")
    inp = make_inputs(w)
    auto = run_hip(inp)
    two = run_hip(inp, waves_per_channel=2)
    assert np.array_equal(auto[1], two[1]), "final states differ from the forced two-wave launch"
    np.testing.assert_allclose(auto[0], two[0], rtol=1e-5, atol=1e-5 * float(np.abs(two[0]).max()))
    _check(auto[0], auto[1], _oracle(inp), f"{w.describe()} automatic")
    t = torch()
    g = {k: dev(inp[k], "f32") for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")}
    out, fin, _ = ssm.scan_train(g["u"], g["delta"], g["A"], g["B"], g["C"], D=g["D"], z=g["z"],
                                 delta_bias=g["delta_bias"], delta_softplus=True, h0=g["h0"])
    t.cuda.synchronize()
    assert np.array_equal(host(out), auto[0]) and np.array_equal(host(fin), auto[1])

"""Pins of the backward oracle (oracle/ssm_ref_bwd.c), on the CPU.

The pages define only the forward scan, so the backward oracle is pinned against the
forward oracle (itself pinned in test_oracle_pins.py) by facts that hold for any correct
derivative:

  * central finite differences of L = sum(dout * out) + sum(dfinal * final_state), for
    every element of every input, with softplus, gate, skip, bias and initial state on,
    and again with all of them off;
  * adjoint (dot-product) identities: out is linear in u, in B, in C and in h0 when the
    other inputs are fixed, so <dout, out(v)> = <grad, v> for any v, at a size where
    finite differences would be slow;
  * chaining: the backward of a sequence equals the backward of its second half
    followed by that of its first half, handed the second half's initial-state gradient
    as its final-state gradient (the carry a chunked backward relies on).
A plausible slip (a missing term, a wrong index between a_t and a_{t+1}, h_t in place of
h_{t-1}, a gate derivative without its z (1 - sigmoid) term) fails at least one of them.
"""
import numpy as np
import pytest

import oracle
from ssm_workloads import WORKLOADS, make_inputs


def f64_inputs(batch, dim, dstate, seqlen, seed, gate=True, h0=True, scaled=True):
    w = WORKLOADS["tiny"].with_(batch=batch, dim=dim, dstate=dstate, seqlen=seqlen, io="f32",
                                gate=gate, initial_state=h0,
                                a_kind="scaled" if scaled else "s4d", seed=seed)
    inp = make_inputs(w)
    f = lambda x: None if x is None else np.asarray(x, np.float64)
    return {k: f(inp[k]) for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")}


def loss(inp, dout, dfinal, softplus):
    out, fin = oracle.scan_ref(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                               inp["z"], inp["delta_bias"], softplus, inp["h0"], nthreads=1)
    val = float(np.sum(dout * out))
    if dfinal is not None:
        val += float(np.sum(dfinal * fin))
    return val


def grads(inp, dout, dfinal, softplus):
    return oracle.scan_bwd_ref(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                               inp["z"], inp["delta_bias"], softplus, inp["h0"], dout, dfinal,
                               nthreads=2)


GRAD_OF = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
           "z": "dz", "delta_bias": "dbias", "h0": "dh0"}


def check_fd(inp, dout, dfinal, softplus, names):
    g = grads(inp, dout, dfinal, softplus)
    for name in names:
        x = inp[name]
        an = g[GRAD_OF[name]]
        fd = np.empty_like(x)
        flat, fdf = x.reshape(-1), fd.reshape(-1)
        for i in range(flat.size):
            keep = flat[i]
            eps = 1e-6 * max(1.0, abs(keep))
            flat[i] = keep + eps
            lp = loss(inp, dout, dfinal, softplus)
            flat[i] = keep - eps
            lm = loss(inp, dout, dfinal, softplus)
            flat[i] = keep
            fdf[i] = (lp - lm) / (2 * eps)
        scale = np.max(np.abs(fd)) + 1e-30
        err = np.max(np.abs(fd - an)) / scale
        assert err < 1e-6, f"d/d{name}: max error {err:.2e} (scale {scale:.3e})"


def test_finite_differences_everything_on():
    inp = f64_inputs(2, 3, 4, 9, seed=501)
    rng = np.random.default_rng(502)
    dout = rng.standard_normal(inp["u"].shape)
    dfinal = rng.standard_normal(inp["h0"].shape)
    check_fd(inp, dout, dfinal, True, list(GRAD_OF))


def test_finite_differences_everything_off():
    inp = f64_inputs(2, 3, 5, 7, seed=503, gate=False, h0=False)
    inp["D"] = None
    inp["delta_bias"] = None
    inp["delta"] = np.abs(inp["delta"]) * 0.3 + 0.01       # positive step sizes
    rng = np.random.default_rng(504)
    dout = rng.standard_normal(inp["u"].shape)
    check_fd(inp, dout, None, False, ["u", "delta", "A", "B", "C"])


def test_finite_differences_above_softplus_threshold():
    """Above 20 the forward returns x itself, so the step-size derivative is 1."""
    inp = f64_inputs(1, 2, 3, 6, seed=505)
    inp["delta"] = inp["delta"] + 25.0
    inp["A"] = inp["A"] * 0.01                              # keep exp(s A) away from 0
    rng = np.random.default_rng(506)
    dout = rng.standard_normal(inp["u"].shape)
    check_fd(inp, dout, None, True, ["delta", "delta_bias"])


def adjoint(inp, softplus, name, use_dfinal=False, seed=0):
    rng = np.random.default_rng(seed)
    dout = rng.standard_normal(inp["u"].shape)
    dfinal = rng.standard_normal((inp["u"].shape[0], inp["u"].shape[1], inp["A"].shape[1])) \
        if use_dfinal else None
    g = grads(inp, dout, dfinal, softplus)[GRAD_OF[name]]
    v = rng.standard_normal(inp[name].shape)
    probe = dict(inp)
    probe[name] = v
    out, fin = oracle.scan_ref(probe["u"], probe["delta"], probe["A"], probe["B"], probe["C"],
                               probe["D"], probe["z"], probe["delta_bias"], softplus,
                               probe["h0"])
    lhs = float(np.sum(dout * out)) + (float(np.sum(dfinal * fin)) if use_dfinal else 0.0)
    rhs = float(np.sum(g * v))
    assert abs(lhs - rhs) <= 1e-10 * (abs(lhs) + np.sqrt(np.sum(dout ** 2))), (name, lhs, rhs)


@pytest.mark.parametrize("name", ["u", "B", "C", "h0"])
def test_adjoint_identities(name):
    inp = f64_inputs(2, 5, 8, 300, seed=507)
    if name in ("B", "C", "h0"):
        inp["D"] = None            # out is then linear (not affine) in B, C and h0
    if name in ("u", "B", "C"):
        inp["h0"] = None
    if name == "h0":
        inp["u"] = np.zeros_like(inp["u"])
    adjoint(inp, True, name, use_dfinal=(name == "h0"), seed=508)


def test_backward_chains_through_the_state():
    inp = f64_inputs(2, 4, 6, 40, seed=509)
    rng = np.random.default_rng(510)
    dout = rng.standard_normal(inp["u"].shape)
    dfinal = rng.standard_normal(inp["h0"].shape)
    full = grads(inp, dout, dfinal, True)
    cut = 17
    time_axis = ("u", "delta", "z", "B", "C")
    first = {k: (v[..., :cut] if k in time_axis else v) for k, v in inp.items()}
    second = {k: (v[..., cut:] if k in time_axis else v) for k, v in inp.items()}
    _, mid = oracle.scan_ref(first["u"], first["delta"], first["A"], first["B"], first["C"],
                             first["D"], first["z"], first["delta_bias"], True, first["h0"])
    second["h0"] = mid
    g2 = grads(second, dout[..., cut:], dfinal, True)
    g1 = grads(first, dout[..., :cut], g2["dh0"], True)
    for k in ("du", "ddelta", "dz"):
        np.testing.assert_allclose(np.concatenate([g1[k], g2[k]], axis=2), full[k],
                                   rtol=1e-11, atol=1e-12)
    for k in ("dB", "dC"):
        np.testing.assert_allclose(np.concatenate([g1[k], g2[k]], axis=2), full[k],
                                   rtol=1e-11, atol=1e-12)
    for k in ("dA", "dD", "dbias"):
        np.testing.assert_allclose(g1[k] + g2[k], full[k], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g1["dh0"], full["dh0"], rtol=1e-11, atol=1e-12)


def test_thread_count_does_not_change_the_result():
    inp = f64_inputs(2, 9, 4, 50, seed=511)
    rng = np.random.default_rng(512)
    dout = rng.standard_normal(inp["u"].shape)
    a = oracle.scan_bwd_ref(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                            inp["z"], inp["delta_bias"], True, inp["h0"], dout, None, nthreads=1)
    b = oracle.scan_bwd_ref(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                            inp["z"], inp["delta_bias"], True, inp["h0"], dout, None, nthreads=4)
    for k in a:
        if a[k] is not None:
            np.testing.assert_allclose(a[k], b[k], rtol=1e-13, atol=1e-14)


def test_empty_sequence_passes_the_final_gradient_through():
    inp = f64_inputs(1, 3, 4, 5, seed=513)
    inp = {k: (v[..., :0] if k in ("u", "delta", "z", "B", "C") else v) for k, v in inp.items()}
    rng = np.random.default_rng(514)
    dfinal = rng.standard_normal(inp["h0"].shape)
    g = grads(inp, np.zeros(inp["u"].shape), dfinal, True)
    np.testing.assert_array_equal(g["dh0"], dfinal)
    assert not g["dA"].any() and not g["dD"].any() and not g["dbias"].any()


def test_finite_differences_with_padding_mask():
    """Padding positions (mhpq.cn/news/1057127 section 4) keep the state; the backward
    oracle must be the derivative of that forward, padding included."""
    inp = f64_inputs(2, 3, 4, 11, seed=515)
    rng = np.random.default_rng(516)
    mask = (rng.random((2, 11)) > 0.35).astype(np.uint8)
    mask[0, :3] = 0
    mask[1, -3:] = 0
    dout = rng.standard_normal(inp["u"].shape)
    dfinal = rng.standard_normal(inp["h0"].shape)

    def loss_m(i, do, df, sp):
        out, fin = oracle.scan_ref(i["u"], i["delta"], i["A"], i["B"], i["C"], i["D"], i["z"],
                                   i["delta_bias"], sp, i["h0"], nthreads=1, mask=mask)
        return float(np.sum(do * out)) + float(np.sum(df * fin))

    g = oracle.scan_bwd_ref(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                            inp["z"], inp["delta_bias"], True, inp["h0"], dout, dfinal,
                            nthreads=2, mask=mask)
    for name in GRAD_OF:
        x = inp[name]
        an = g[GRAD_OF[name]]
        fd = np.empty_like(x)
        flat, fdf = x.reshape(-1), fd.reshape(-1)
        for i in range(flat.size):
            keep = flat[i]
            eps = 1e-6 * max(1.0, abs(keep))
            flat[i] = keep + eps
            lp = loss_m(inp, dout, dfinal, True)
            flat[i] = keep - eps
            lm = loss_m(inp, dout, dfinal, True)
            flat[i] = keep
            fdf[i] = (lp - lm) / (2 * eps)
        scale = np.max(np.abs(fd)) + 1e-30
        err = np.max(np.abs(fd - an)) / scale
        assert err < 1e-6, f"d/d{name} with mask: max error {err:.2e}"
    # nothing flows into the step size of a padding position
    assert not g["ddelta"][np.broadcast_to(mask[:, None, :] == 0, g["ddelta"].shape)].any()

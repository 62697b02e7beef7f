"""Pins of the Mamba-2 (SSD) oracles (oracle/ssd.py), on the CPU.

The three formulations come from different passages and share no arithmetic:
  * ssd_ref: the recurrence (the pinned Mamba-1 C oracle with A and the step size
    broadcast per head; ybb.press/ai-applications/14118.html section 2.2);
  * ssd_dense_ref: one semiseparable matrix per (batch, head)
    (mhpq.cn/news/1077344 section 5.1);
  * ssd_chunked_ref: blocks with an inter-block scan of states (same page, section 5.2).
Their agreement to float64 rounding pins each against the others: a wrong head mapping,
a dropped dt_s, an exponent summed over the wrong range (a_s included, or a_t left out),
B and C swapped, or a missing carried-state term makes one of them differ. Closed forms
and a brute-force loop fix the special cases independently of all three.
"""
import numpy as np
import pytest

import oracle
from ssm_workloads import SSD_WORKLOADS, make_mask, make_ssd_inputs, widen


def f64_case(batch, nheads, headdim, dstate, seqlen, seed, gate=True, h0=True):
    w = SSD_WORKLOADS["ssd_tiny"].with_(batch=batch, nheads=nheads, headdim=headdim,
                                        dstate=dstate, seqlen=seqlen, io="f32", gate=gate,
                                        initial_state=h0, seed=seed)
    inp = make_ssd_inputs(w)
    return {k: (None if v is None else np.asarray(v, np.float64))
            for k, v in inp.items() if k != "io"}


def run(fn, c, softplus=True, mask=None, **kw):
    return fn(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["z"], c["dt_bias"], softplus,
              c["h0"], mask=mask, **kw)


def close(a, b, rtol=1e-11):
    for u, v in zip(a, b):
        scale = np.max(np.abs(v)) + 1e-300
        assert np.max(np.abs(u - v)) <= rtol * scale, np.max(np.abs(u - v)) / scale


@pytest.mark.parametrize("shape", [(2, 3, 4, 5, 37), (1, 2, 8, 16, 64), (2, 4, 2, 3, 1),
                                   (1, 1, 1, 1, 9)],
                         ids=lambda s: "b{}h{}p{}N{}L{}".format(*s))
def test_recurrence_equals_semiseparable_matrix(shape):
    c = f64_case(*shape, seed=900 + sum(shape))
    close(run(oracle.ssd_ref, c), run(oracle.ssd_dense_ref, c))


@pytest.mark.parametrize("chunk", [1, 7, 16, 64, 100])
def test_block_form_equals_recurrence(chunk):
    c = f64_case(2, 3, 4, 6, 53, seed=910)
    close(run(oracle.ssd_chunked_ref, c, chunk=chunk), run(oracle.ssd_ref, c))


def test_all_forms_agree_without_optional_inputs():
    c = f64_case(2, 2, 3, 4, 30, seed=911, gate=False, h0=False)
    c["D"] = None
    c["dt_bias"] = None
    c["dt"] = np.abs(c["dt"]) * 0.2 + 0.01
    ref = run(oracle.ssd_ref, c, softplus=False)
    close(run(oracle.ssd_dense_ref, c, softplus=False), ref)
    close(run(oracle.ssd_chunked_ref, c, softplus=False, chunk=8), ref)


@pytest.mark.parametrize("kind", ["lengths", "random", "zeros"])
def test_padding_mask_in_every_form(kind):
    c = f64_case(3, 2, 4, 5, 41, seed=912)
    m = make_mask(3, 41, kind, seed=913)
    ref = run(oracle.ssd_ref, c, mask=m)
    close(run(oracle.ssd_dense_ref, c, mask=m), ref)
    close(run(oracle.ssd_chunked_ref, c, mask=m, chunk=16), ref)
    if kind == "zeros":
        assert np.array_equal(ref[1], c["h0"])


def test_no_decay_closed_form():
    """A = 0 and a constant step size c: the state is a plain running sum, so
    y_t[p] = c * sum_{s<=t} (C_t . B_s) x_s[p] + D x_t[p]."""
    c = f64_case(1, 2, 3, 4, 12, seed=914, gate=False, h0=False)
    c["A"] = np.zeros(2)
    c["dt"] = np.full_like(c["dt"], 0.3)
    c["dt_bias"] = None
    out, fin = run(oracle.ssd_ref, c, softplus=False)
    x, B, C, D = c["x"][0], c["B"][0], c["C"][0], c["D"]
    for p in range(6):
        for t in range(12):
            want = 0.3 * sum(float(C[:, t] @ B[:, s]) * x[p, s] for s in range(t + 1))
            want += D[p] * x[p, t]
            assert abs(out[0, p, t] - want) <= 1e-12 * (1 + abs(want))
        np.testing.assert_allclose(fin[0, p], 0.3 * (B * x[p][None, :]).sum(axis=1),
                                   rtol=1e-12, atol=1e-14)


def test_brute_force_loop():
    """Tiny case by an explicit loop over heads, channels, steps and states, written
    here independently of the three oracle forms."""
    c = f64_case(1, 2, 2, 3, 6, seed=915)
    out, fin = run(oracle.ssd_ref, c)
    x, dt, A, B, C, D, z, bias, h0 = (c[k] for k in ("x", "dt", "A", "B", "C", "D", "z",
                                                      "dt_bias", "h0"))
    for d in range(4):
        h = d // 2
        st = h0[0, d].copy()
        for t in range(6):
            v = dt[0, h, t] + bias[h]
            s = np.log1p(np.exp(v)) if v <= 20 else v
            st = np.exp(s * A[h]) * st + s * B[0, :, t] * x[0, d, t]
            y = float(C[0, :, t] @ st) + D[d] * x[0, d, t]
            y *= z[0, d, t] / (1 + np.exp(-z[0, d, t]))
            assert abs(out[0, d, t] - y) <= 1e-12 * (1 + abs(y))
        np.testing.assert_allclose(fin[0, d], st, rtol=1e-12, atol=1e-15)


def test_single_step_closed_form():
    c = f64_case(2, 2, 3, 4, 1, seed=916)
    out, fin = run(oracle.ssd_ref, c)
    s = np.logaddexp(0.0, c["dt"][:, :, 0] + c["dt_bias"][None, :])        # [b, h]
    sd = np.repeat(s, 3, axis=1)                                             # [b, d]
    Ad = np.repeat(c["A"], 3)
    want_f = np.exp(sd * Ad[None, :])[:, :, None] * c["h0"] \
        + (sd * c["x"][:, :, 0])[:, :, None] * c["B"][:, None, :, 0]
    np.testing.assert_allclose(fin, want_f, rtol=1e-12)
    y = np.einsum("bdn,bn->bd", want_f, c["C"][:, :, 0]) + c["D"][None, :] * c["x"][:, :, 0]
    zz = c["z"][:, :, 0]
    np.testing.assert_allclose(out[:, :, 0], y * zz / (1 + np.exp(-zz)), rtol=1e-12)


def test_heads_are_independent():
    """Changing one head's inputs leaves every other head's channels bitwise unchanged."""
    c = f64_case(1, 3, 2, 4, 20, seed=917)
    a = run(oracle.ssd_ref, c)
    c2 = dict(c)
    c2["dt"] = c["dt"].copy()
    c2["dt"][:, 1] += 1.0
    c2["A"] = c["A"].copy()
    c2["A"][1] *= 2
    b = run(oracle.ssd_ref, c2)
    keep = [0, 1, 4, 5]
    assert np.array_equal(a[0][:, keep], b[0][:, keep]) and np.array_equal(a[1][:, keep],
                                                                            b[1][:, keep])
    assert not np.allclose(a[0][:, 2:4], b[0][:, 2:4])


def test_empty_sequence():
    c = f64_case(1, 2, 2, 3, 0, seed=918)
    out, fin = run(oracle.ssd_ref, c)
    assert out.shape == (1, 4, 0)
    assert np.array_equal(fin, c["h0"])
    d_out, d_fin = run(oracle.ssd_dense_ref, c)
    assert np.array_equal(d_fin, c["h0"])


def test_bf16_inputs_widen_exactly():
    w = SSD_WORKLOADS["ssd_tiny"].with_(seqlen=40)
    inp = make_ssd_inputs(w)
    x = widen(inp["x"], "bf16")
    # bf16 values carry 8 significant bits: the widened value times 2^k is an integer
    m, _ = np.frexp(x[x != 0])
    assert np.all((m * 256) == np.round(m * 256))

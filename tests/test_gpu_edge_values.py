"""Edge values through the GPU forward, against the float64 oracle.

* Step-size arguments at and above softplus' threshold of 20 (the oracle returns x itself
  there; the kernel's max(x, 0) + log1p(exp(-|x|)) differs from that by less than 3e-9
  relative).
* Non-finite inputs: NaN in u, in the raw step size and in B; -inf in the raw step size
  (softplus(-inf) = 0: an identity step, everything stays finite); +inf and -inf in z. The
  parity metric counts elements whose finiteness differs between the two results
  (nonfinite_mismatch) and requires none; the finite elements keep the usual bar.
* A > 0 on some states (Δ·A > 0, so exp(Δ·A) > 1 and those states grow), in a range where
  nothing overflows.

fp32 storage (rtol 1e-4 on out and final_state) and bf16 storage (2e-2 on out).
"""
import numpy as np
import pytest

import oracle
from gpu_util import announce, run_hip
from ssm_workloads import (RTOL, WATCH, RTOL_STATE, WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits,
                           make_inputs, parity, widen)

pytestmark = pytest.mark.gpu


def _oracle(inp):
    io = inp["io"]
    return oracle.scan_ref(widen(inp["u"], io), widen(inp["delta"], io), inp["A"],
                           widen(inp["B"], io), widen(inp["C"], io), inp["D"],
                           widen(inp["z"], io), inp["delta_bias"], True, inp["h0"])


def _set(inp, key, idx, value):
    """Write one value into a stored (fp32 or bf16-bits) input array."""
    a = inp[key]
    if a.dtype == np.uint16:
        a[idx] = f32_to_bf16_bits(np.array([value], np.float32))[0]
    else:
        a[idx] = np.float32(value)


def _check(got, ref, io, label, expect_nonfinite=False):
    ro, rf = parity(got[0], ref[0], RTOL[io], WATCH[io]), parity(got[1], ref[1], RTOL_STATE)
    print(f"[edge] {label}: out {ro} | final {rf}", flush=True)
    assert ro.ok and rf.ok, label
    if expect_nonfinite:
        assert not np.all(np.isfinite(ref[0])), "the case should produce non-finite outputs"


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_softplus_at_and_above_its_threshold(io):
    w = WORKLOADS["tiny"].with_(batch=2, dim=6, seqlen=1100, io=io, gate=True,
                                initial_state=True, seed=1800)
    announce(f"{w.describe()} softplus threshold")
    inp = make_inputs(w)
    inp["delta_bias"][:] = 0.0  # the raw step size is softplus' argument
    rng = np.random.default_rng(1801)
    values = [19.5, 19.99, 20.0, 20.01, 20.5, 25.0, 40.0, 88.0, 100.0, 1e4]
    for v in values:
        for _ in range(3):
            b, d, t = rng.integers(w.batch), rng.integers(w.dim), rng.integers(w.seqlen)
            _set(inp, "delta", (b, d, t), v)
    _check(run_hip(inp), _oracle(inp), io, f"{w.describe()} softplus threshold")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_non_finite_inputs(io):
    w = WORKLOADS["tiny"].with_(batch=2, dim=8, seqlen=1300, io=io, gate=True,
                                initial_state=True, seed=1810)
    announce(f"{w.describe()} non-finite inputs")
    inp = make_inputs(w)
    _set(inp, "u", (0, 1, 300), np.nan)       # that channel: NaN from step 300 on
    _set(inp, "delta", (0, 2, 700), np.nan)   # that channel: NaN from step 700 on
    _set(inp, "delta", (1, 3, 100), -np.inf)  # softplus(-inf) = 0: an identity step
    _set(inp, "B", (1, 4, 1200), np.nan)      # batch row 1, state 4: every channel from 1200
    _set(inp, "z", (1, 0, 50), np.inf)        # one output +-inf
    _set(inp, "z", (1, 1, 60), -np.inf)       # one output NaN (y * -inf * 0)
    ref = _oracle(inp)
    assert np.isnan(ref[0][0, 1, 300:]).all() and np.isfinite(ref[0][0, 1, :300]).all()
    assert np.isfinite(ref[0][1, 3, :1200]).all() and np.isnan(ref[0][1, :, 1200:]).all()
    _check(run_hip(inp), ref, io, f"{w.describe()} non-finite inputs", expect_nonfinite=True)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_positive_delta_times_A(io):
    w = WORKLOADS["tiny"].with_(batch=2, dim=5, dstate=8, seqlen=900, io=io, gate=False,
                                a_kind="scaled", initial_state=True, seed=1820)
    announce(f"{w.describe()} A > 0 on some states")
    inp = make_inputs(w)
    inp["A"][:, 2] = 0.05                     # growth exp(0.05 dt) per step
    inp["A"][:, 5] = np.abs(inp["A"][:, 5]) * 0.01
    ref = _oracle(inp)
    assert np.all(np.isfinite(ref[0])) and np.abs(ref[1][:, :, 2]).max() > np.abs(inp["h0"]).max()
    _check(run_hip(inp), ref, io, f"{w.describe()} A > 0")

"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on the same
seeded, stored inputs.

Bar (the per-element metric of ssm_workloads.compare):
  * out: rtol 1e-4 for float32 storage; 2e-2 for bfloat16 storage (bf16 output rounding
    included), and for bf16 also the tighter regression watch 2^-8 (1 + 1e-4) + 1e-4, which
    a float32 result within 1e-4 keeps after rounding to bf16;
  * final_state (always float32, never rounded to bf16): rtol 1e-4.
Small and medium cases compare every element; the full-size workloads compare a seeded
sample of rows (plus the first and last) that the oracle computes one by one, in the
same launch configuration the benchmark times.
"""
import numpy as np
import pytest

import oracle
from gpu_util import announce, run_hip
from ssm_workloads import (RTOL, RTOL_STATE, WATCH, WORKLOADS, f32_to_bf16_bits, make_inputs,
                           parity, widen)

pytestmark = pytest.mark.gpu


def oracle_full(inp, softplus=True, use_D=True, use_z=True, use_bias=True):
    io = inp["io"]
    return oracle.scan_ref(
        widen(inp["u"], io), widen(inp["delta"], io), inp["A"], widen(inp["B"], io),
        widen(inp["C"], io), inp["D"] if use_D else None,
        widen(inp["z"], io) if use_z else None,
        inp["delta_bias"] if use_bias else None, softplus, inp["h0"])


def assert_parity(io, got_out, got_fin, ref_out, ref_fin, label):
    ro = parity(got_out, ref_out, RTOL[io], WATCH[io])
    rf = parity(got_fin, ref_fin, RTOL_STATE)
    print(f"[parity] {label}: out {ro} | final {rf}", flush=True)
    assert ro.ok, f"{label} out: {ro}"
    assert rf.ok, f"{label} final_state: {rf}"


# ----------------------------------------------------------------- full comparisons

SMALL = WORKLOADS["tiny"]
SHAPES = [
    # (batch, dim, dstate, seqlen): ragged tails around the 512-step chunk and the 8-step
    # lane block, one-step and one-lane sequences, odd channel counts, several states
    (1, 64, 16, 256), (2, 13, 16, 1), (1, 5, 16, 2), (1, 7, 16, 7), (2, 9, 16, 63),
    (1, 8, 16, 64), (1, 8, 16, 65), (1, 6, 16, 511), (1, 6, 16, 512), (1, 6, 16, 513),
    (2, 5, 16, 1000), (1, 4, 16, 1537), (1, 3, 16, 4099),
    (1, 6, 1, 300), (1, 6, 3, 300), (1, 6, 17, 300), (2, 6, 32, 777), (1, 6, 64, 1030),
]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}d{}N{}L{}".format(*s))
def test_parity_shapes(shape, io):
    b, d, n, L = shape
    w = SMALL.with_(batch=b, dim=d, dstate=n, seqlen=L, io=io, gate=(io == "bf16"),
                    a_kind="scaled" if n != 16 else "s4d", seed=100 + L + n)
    announce(w.describe())
    inp = make_inputs(w)
    got = run_hip(inp)
    ref = oracle_full(inp)
    assert_parity(io, *got, *ref, w.describe())


@pytest.mark.parametrize("variant", ["no_D", "no_z", "no_bias", "no_softplus", "h0",
                                     "bare"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_parity_optional_inputs(variant, io):
    w = SMALL.with_(batch=2, dim=24, seqlen=700, io=io, gate=True,
                    initial_state=(variant == "h0"), seed=7)
    announce(f"{w.describe()} {variant}")
    inp = make_inputs(w)
    kw = dict(use_D=variant not in ("no_D", "bare"), use_z=variant not in ("no_z", "bare"),
              use_bias=variant not in ("no_bias", "bare"),
              softplus=variant not in ("no_softplus", "bare"))
    if not kw["softplus"]:
        # without softplus, delta + bias is the step size itself: keep both positive
        raw = widen(inp["delta"], io)
        pos = np.abs(raw) * 0.05 + 1e-3
        inp["delta"] = (pos.astype(np.float32) if io == "f32"
                        else f32_to_bf16_bits(pos.astype(np.float32)))
        inp["delta_bias"] = np.abs(inp["delta_bias"]) * np.float32(0.01)
    got = run_hip(inp, **kw)
    ref = oracle_full(inp, **kw)
    assert_parity(io, *got, *ref, f"{w.describe()} {variant}")


def test_parity_tiny_workload():
    w = WORKLOADS["tiny"]
    announce(w.describe())
    inp = make_inputs(w)
    assert_parity(w.io, *run_hip(inp), *oracle_full(inp), w.describe())


@pytest.mark.slow
def test_parity_long_workload_full():
    w = WORKLOADS["long"]
    announce(w.describe())
    inp = make_inputs(w)
    assert_parity(w.io, *run_hip(inp), *oracle_full(inp), w.describe())


def test_parity_decode_workload_full():
    w = WORKLOADS["decode"]
    announce(w.describe())
    inp = make_inputs(w)
    assert_parity(w.io, *run_hip(inp), *oracle_full(inp), w.describe())


# ----------------------------------------------------------------- full-size, sampled rows

@pytest.mark.slow
@pytest.mark.parametrize("name", ["layer", "verylong", "widestate"])
def test_parity_full_size_sampled(name):
    w = WORKLOADS[name]
    announce(w.describe())
    inp = make_inputs(w)
    out, fin = run_hip(inp)
    rows = oracle.sample_rows(w.batch, w.dim, 64, w.seed)
    ref_out, ref_fin = oracle.scan_rows(inp, rows)
    bi = np.array([r[0] for r in rows])
    di = np.array([r[1] for r in rows])
    assert_parity(w.io, out[bi, di], fin[bi, di], ref_out, ref_fin,
                  f"{w.describe()} ({len(rows)} sampled rows)")
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(fin))


@pytest.mark.parametrize("rows", [(1, 1023), (2, 512), (1, 1025), (3, 700)],
                         ids=lambda r: "b{}d{}".format(*r))
def test_parity_fp32_around_the_state_split(rows):
    """fp32 launches whose workgroups (4 channels each) all fit on the device at once split
    each channel's states over two waves; larger ones use one wave per channel. Both sides of
    the threshold on a 256-CU device (256 and 257 workgroups), every element."""
    b, d = rows
    w = SMALL.with_(batch=b, dim=d, dstate=16, seqlen=600, io="f32", gate=True,
                    initial_state=True, seed=140 + d)
    announce(w.describe())
    inp = make_inputs(w)
    got = run_hip(inp)
    ref = oracle_full(inp)
    assert_parity("f32", got[0], got[1], ref[0], ref[1], w.describe())

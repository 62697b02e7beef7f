"""GPU parity of the short-sequence path (seqlen <= 32: decode and state passing) against
the float64 oracle, through the C ABI.

Sequences of at most 32 steps run one lane per (channel, four states) stepping through
time (one lane per state when dstate is not a multiple of four or a state pointer is not
16-byte aligned); longer ones run the chunked scan. These cases cover that kernel's own
mapping: dstate not a power of two or not a multiple of four (idle lanes, the one-state
form), 1 and 64 states, channel counts that leave a wavefront partly empty, every
optional input, unaligned state pointers, the 32/33-step boundary between the two
kernels, and a decode loop that carries the state from call to call.
"""
import numpy as np
import pytest

import oracle
import selective_state_space_fwd_amd as ssm
from gpu_util import announce, dev, host, run_hip, torch
from ssm_workloads import RTOL, WATCH, RTOL_STATE, WORKLOADS, make_inputs, parity, widen

pytestmark = pytest.mark.gpu

BASE = WORKLOADS["decode"]


def oracle_full(inp, softplus=True, use_D=True, use_z=True, use_bias=True):
    io = inp["io"]
    return oracle.scan_ref(
        widen(inp["u"], io), widen(inp["delta"], io), inp["A"], widen(inp["B"], io),
        widen(inp["C"], io), inp["D"] if use_D else None,
        widen(inp["z"], io) if use_z and inp["z"] is not None else None,
        inp["delta_bias"] if use_bias else None, softplus, inp["h0"])


def check(io, got, ref, label):
    ro = parity(got[0], ref[0], RTOL[io], WATCH[io])
    rf = parity(got[1], ref[1], RTOL_STATE)
    print(f"[parity] {label}: out {ro} | final {rf}", flush=True)
    assert ro.ok, f"{label} out: {ro}"
    assert rf.ok, f"{label} final_state: {rf}"


SHORT_SHAPES = [
    # (batch, dim, dstate, seqlen)
    (2, 13, 16, 1), (3, 5, 64, 1), (2, 7, 1, 1), (1, 9, 3, 2), (2, 6, 17, 5),
    (1, 8, 33, 16), (2, 4, 64, 32), (1, 5, 16, 32), (1, 5, 16, 33), (1, 3, 2, 40),
    (2, 11, 12, 3), (1, 7, 20, 9), (2, 5, 44, 1), (1, 3, 4, 2),
]


@pytest.mark.parametrize("h0", [False, True], ids=["zero_state", "h0"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHORT_SHAPES, ids=lambda s: "b{}d{}N{}L{}".format(*s))
def test_short_shapes(shape, io, h0):
    b, d, n, L = shape
    w = BASE.with_(batch=b, dim=d, dstate=n, seqlen=L, io=io, gate=(io == "bf16"),
                   initial_state=h0, seed=300 + 7 * L + n)
    announce(w.describe())
    inp = make_inputs(w)
    check(io, run_hip(inp), oracle_full(inp), w.describe())


@pytest.mark.parametrize("variant", ["no_D", "no_z", "no_bias", "no_softplus", "bare"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_short_optional_inputs(variant, io):
    w = BASE.with_(batch=2, dim=24, dstate=16, seqlen=8, io=io, gate=True, seed=41)
    announce(f"{w.describe()} {variant}")
    inp = make_inputs(w)
    kw = dict(use_D=variant not in ("no_D", "bare"), use_z=variant not in ("no_z", "bare"),
              use_bias=variant not in ("no_bias", "bare"),
              softplus=variant not in ("no_softplus", "bare"))
    if not kw["softplus"]:
        # without softplus, delta + bias is the step size itself: keep it positive
        from ssm_workloads import f32_to_bf16_bits
        raw = widen(inp["delta"], io)
        pos = (np.abs(raw) * 0.05 + 1e-3).astype(np.float32)
        inp["delta"] = pos if io == "f32" else f32_to_bf16_bits(pos)
        inp["delta_bias"] = np.abs(inp["delta_bias"]) * 0.01
    check(io, run_hip(inp, **kw), oracle_full(inp, **kw), f"{w.describe()} {variant}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_loop_carries_state(io):
    """Twelve one-step calls, each starting from the previous call's final state, equal
    one twelve-step run."""
    steps = 12
    w = BASE.with_(batch=2, dim=40, dstate=64, seqlen=steps, io=io, gate=True,
                   initial_state=True, seed=43)
    announce(f"{w.describe()} decode loop")
    inp = make_inputs(w)
    ref_out, ref_fin = oracle_full(inp)
    state = inp["h0"].astype(np.float32)
    outs = []
    for t in range(steps):
        step = {k: (v[..., t:t + 1] if k in ("u", "delta", "z", "B", "C") else v)
                for k, v in inp.items()}
        step["h0"] = state
        o, f = run_hip(step)
        outs.append(o)
        state = f.astype(np.float32)
    check(io, (np.concatenate(outs, axis=2), state.astype(np.float64)), (ref_out, ref_fin),
          f"{w.describe()} decode loop")


def test_decode_workload_full():
    w = WORKLOADS["decode"]
    announce(w.describe())
    inp = make_inputs(w)
    check(w.io, run_hip(inp), oracle_full(inp), w.describe())


def test_short_zero_input_keeps_only_decay():
    """u = 0: the state only decays, h_L = h0 * exp(A * sum dt), exactly the oracle's
    product to float32 rounding; out is C . h (no D term since u = 0)."""
    w = BASE.with_(batch=1, dim=6, dstate=16, seqlen=9, io="f32", gate=False,
                   initial_state=True, seed=44)
    announce(f"{w.describe()} zero input")
    inp = make_inputs(w)
    inp["u"] = np.zeros_like(inp["u"])
    check("f32", run_hip(inp), oracle_full(inp), f"{w.describe()} zero input")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_short_unaligned_state_pointers(io):
    """A and the state tensors placed 4 bytes past a 16-byte boundary: the kernel falls
    back from four states per lane to one, with the same results."""
    t = torch()
    w = BASE.with_(batch=2, dim=24, dstate=16, seqlen=3, io=io, initial_state=True, seed=45)
    announce(f"{w.describe()} unaligned A and state")
    inp = make_inputs(w)
    g = {k: dev(inp[k], io) for k in ("u", "delta", "B", "C", "z")}
    f = {k: dev(inp[k], "f32") for k in ("D", "delta_bias")}

    def offset(a):
        flat = t.empty(a.size + 1, dtype=t.float32, device="cuda")
        view = flat[1:].view(a.shape)
        view.copy_(t.from_numpy(np.ascontiguousarray(a, dtype=np.float32)))
        return view

    A, h0, fin = offset(inp["A"]), offset(inp["h0"]), offset(inp["h0"])
    assert A.data_ptr() % 16 == 4 and fin.data_ptr() % 16 == 4
    out, fin = ssm.scan(g["u"], g["delta"], A, g["B"], g["C"], D=f["D"], z=g["z"],
                        delta_bias=f["delta_bias"], delta_softplus=True, h0=h0,
                        final_state=fin)
    t.cuda.synchronize()
    check(io, (host(out), host(fin)), oracle_full(inp), f"{w.describe()} unaligned")

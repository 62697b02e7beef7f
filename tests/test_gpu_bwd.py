"""GPU backward pass (through the C ABI) against the float64 backward oracle, and the
forward's saved states against the forward oracle.

Bar, per tensor (the metric of ssm_workloads.compare, max |g - r| / (|r| + rms(r))):
  * du, ddelta, dz: 1e-4 with float32 storage, 2e-2 with bfloat16 storage (one rounding
    to bf16 on store, as for out);
  * dA, dB, dC, dD, dbias, dh0 and the saved states (always float32): 1e-4, which leaves
    about two orders of magnitude over the float32 rounding of sums of up to ~1e4 terms.
By default the channel- and batch-summed gradients (dA, dB, dC, dD, dbias) go through the
workspace path (per-workgroup partial sums added in a fixed order), so every gradient is
compared bit for bit between runs; the float-atomic path (no workspace) is checked against
the oracle too, and against the workspace path within float32 rounding.
"""
import numpy as np
import pytest

import oracle
import selective_state_space_fwd_amd as ssm
from gpu_util import announce, dev, host, torch
from ssm_workloads import RTOL, WATCH, WORKLOADS, f32_to_bf16_bits, make_inputs, parity, widen

pytestmark = pytest.mark.gpu

RTOL_F32_OUT = 1e-4
PER_ELEMENT = ("du", "ddelta", "dz")


def setup(w, softplus=True, use_D=True, use_z=True, use_bias=True, dfinal=True, seed=0):
    inp = make_inputs(w)
    if not use_z:
        inp["z"] = None
    if not use_D:
        inp["D"] = None
    if not use_bias:
        inp["delta_bias"] = None
    if not softplus:
        raw = widen(inp["delta"], w.io)
        pos = (np.abs(raw) * 0.05 + 1e-3).astype(np.float32)
        inp["delta"] = pos if w.io == "f32" else f32_to_bf16_bits(pos)
        if inp["delta_bias"] is not None:  # delta + bias is the step size: keep it positive
            inp["delta_bias"] = np.abs(inp["delta_bias"]) * 0.01
    rng = np.random.default_rng(seed + 991)
    dout = rng.standard_normal(inp["u"].shape).astype(np.float32)
    if w.io == "bf16":
        dout = f32_to_bf16_bits(dout)
    dfin = rng.standard_normal((w.batch, w.dim, w.dstate)).astype(np.float32) if dfinal else None
    return inp, dout, dfin


def run_gpu(inp, dout, dfin, softplus, deterministic=True, workspace=None, unsplit=False):
    io = inp["io"]
    g = {k: dev(inp[k], io) for k in ("u", "delta", "B", "C", "z")}
    f = {k: dev(inp[k], "f32") for k in ("A", "D", "delta_bias", "h0")}
    out, fin, states = ssm.scan_train(g["u"], g["delta"], f["A"], g["B"], g["C"], D=f["D"],
                                      z=g["z"], delta_bias=f["delta_bias"],
                                      delta_softplus=softplus, h0=f["h0"])
    grads = ssm.scan_backward(g["u"], g["delta"], f["A"], g["B"], g["C"], states,
                              dev(dout, io), D=f["D"], z=g["z"], delta_bias=f["delta_bias"],
                              delta_softplus=softplus,
                              dfinal=None if dfin is None else dev(dfin, "f32"),
                              deterministic=deterministic, workspace=workspace,
                              unsplit=unsplit)
    torch().cuda.synchronize()
    res = {k: (None if v is None else host(v)) for k, v in grads.items()}
    return host(out), host(fin), host(states), res


def run_oracle(inp, dout, dfin, softplus):
    io = inp["io"]
    return oracle.scan_bwd_ref(
        widen(inp["u"], io), widen(inp["delta"], io), inp["A"], widen(inp["B"], io),
        widen(inp["C"], io), inp["D"], None if inp["z"] is None else widen(inp["z"], io),
        inp["delta_bias"], softplus, inp["h0"], widen(dout, io),
        None if dfin is None else dfin.astype(np.float64))


def compare(io, got, ref, label):
    for k, r in ref.items():
        if r is None:
            assert got.get(k) is None, f"{label}: {k} should be absent"
            continue
        rtol = RTOL[io] if k in PER_ELEMENT else RTOL_F32_OUT
        rep = parity(got[k], r, rtol, WATCH[io] if k in PER_ELEMENT else None)
        print(f"[grad] {label} {k}: {rep}", flush=True)
        assert rep.ok, f"{label} {k}: {rep}"


SHAPES = [
    # (batch, dim, dstate, seqlen): one step, a ragged tail, one and several 256-step
    # intervals, ragged channel counts, 1 to 64 states
    (2, 5, 16, 1), (1, 7, 3, 7), (2, 9, 16, 100), (1, 6, 16, 256), (1, 6, 16, 257),
    (1, 6, 16, 512), (1, 6, 16, 513),
    (2, 5, 4, 1500), (1, 3, 64, 700), (1, 10, 1, 300), (1, 4, 17, 2049),
]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}d{}N{}L{}".format(*s))
def test_backward_shapes(shape, io):
    b, d, n, L = shape
    w = WORKLOADS["tiny"].with_(batch=b, dim=d, dstate=n, seqlen=L, io=io, gate=True,
                                initial_state=True, a_kind="scaled", seed=600 + L + n)
    announce(w.describe() + " backward")
    inp, dout, dfin = setup(w, seed=L)
    *_, got = run_gpu(inp, dout, dfin, True)
    compare(io, got, run_oracle(inp, dout, dfin, True), w.describe())


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_backward_long_sequence(io):
    """16 384 steps: the state adjoint carried across 64 intervals of 256 steps, right to left,
    and the states restarted from 64 saved ones; a channel count that leaves the last
    workgroup partly empty and its last wave with one channel."""
    w = WORKLOADS["tiny"].with_(batch=1, dim=37, dstate=16, seqlen=16384, io=io, gate=True,
                                initial_state=True, a_kind="scaled", seed=640)
    announce(w.describe() + " backward, long sequence")
    inp, dout, dfin = setup(w, seed=640)
    *_, got = run_gpu(inp, dout, dfin, True)
    compare(io, got, run_oracle(inp, dout, dfin, True), w.describe() + " long")


@pytest.mark.parametrize("variant", ["no_D", "no_z", "no_bias", "no_softplus", "no_dfinal",
                                     "bare"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_backward_optional_inputs(variant, io):
    w = WORKLOADS["tiny"].with_(batch=2, dim=12, dstate=16, seqlen=600, io=io, gate=True,
                                initial_state=variant not in ("bare",), seed=61)
    announce(f"{w.describe()} backward {variant}")
    bare = variant == "bare"
    kw = dict(softplus=variant not in ("no_softplus", "bare"),
              use_D=variant not in ("no_D", "bare"), use_z=variant not in ("no_z", "bare"),
              use_bias=variant not in ("no_bias", "bare"),
              dfinal=variant not in ("no_dfinal", "bare"))
    inp, dout, dfin = setup(w, seed=62, **kw)
    *_, got = run_gpu(inp, dout, dfin, kw["softplus"])
    compare(io, got, run_oracle(inp, dout, dfin, kw["softplus"]), f"{w.describe()} {variant}")
    if bare:
        assert got["dD"] is None and got["dz"] is None and got["dbias"] is None


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("seqlen", [1700, 2048])  # bf16 rows: element-wise, then whole words
def test_saved_states_and_forward_unchanged(io, seqlen):
    w = WORKLOADS["tiny"].with_(batch=2, dim=6, dstate=16, seqlen=seqlen, io=io, gate=True,
                                initial_state=True, seed=63)
    announce(w.describe() + " saved states")
    inp, dout, dfin = setup(w, seed=63)
    out, fin, states, _ = run_gpu(inp, dout, dfin, True)
    # the training forward writes the same out and final state as the plain forward
    from gpu_util import run_hip
    o2, f2 = run_hip(inp)
    assert np.array_equal(out, o2) and np.array_equal(fin, f2)
    # entry k is the state entering step SSM_CKPT_INTERVAL k
    io_ = inp["io"]
    for k in range(states.shape[2]):
        t = ssm.SSM_CKPT_INTERVAL * k
        if t == 0:
            ref = inp["h0"].astype(np.float64)
        else:
            _, ref = oracle.scan_ref(
                widen(inp["u"][..., :t], io_), widen(inp["delta"][..., :t], io_), inp["A"],
                widen(inp["B"][..., :t], io_), widen(inp["C"][..., :t], io_), inp["D"],
                widen(inp["z"][..., :t], io_), inp["delta_bias"], True, inp["h0"])
        rep = parity(states[:, :, k], ref, RTOL_F32_OUT)
        assert rep.ok, f"state {k}: {rep}"


ALL_GRADS = ("du", "ddelta", "dz", "dh0", "dA", "dB", "dC", "dD", "dbias")


def test_backward_per_element_outputs_are_deterministic():
    """Atomic path: the per-element gradients and dh0 are still reproducible."""
    w = WORKLOADS["tiny"].with_(batch=2, dim=16, dstate=16, seqlen=1100, io="bf16", gate=True,
                                initial_state=True, seed=64)
    announce(w.describe() + " determinism (atomics)")
    inp, dout, dfin = setup(w, seed=64)
    *_, g1 = run_gpu(inp, dout, dfin, True, deterministic=False)
    *_, g2 = run_gpu(inp, dout, dfin, True, deterministic=False)
    for k in ("du", "ddelta", "dz", "dh0"):
        assert np.array_equal(g1[k], g2[k]), k


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_backward_workspace_sums_are_reproducible(io):
    """Workspace path: every gradient, the summed ones included, is bitwise the same from
    run to run (several workgroups per batch row, a ragged channel count and tail)."""
    w = WORKLOADS["tiny"].with_(batch=3, dim=37, dstate=16, seqlen=1300, io=io, gate=True,
                                initial_state=True, seed=66)
    announce(w.describe() + " determinism (workspace)")
    inp, dout, dfin = setup(w, seed=66)
    *_, g1 = run_gpu(inp, dout, dfin, True)
    *_, g2 = run_gpu(inp, dout, dfin, True)
    for k in ALL_GRADS:
        assert np.array_equal(g1[k], g2[k]), k
    compare(io, g1, run_oracle(inp, dout, dfin, True), w.describe())


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(2, 9, 16, 100), (1, 4, 17, 2049), (2, 37, 64, 600)],
                         ids=lambda s: "b{}d{}N{}L{}".format(*s))
def test_backward_atomic_path(shape, io):
    """The float-atomic path (no workspace) against the oracle."""
    b, d, n, L = shape
    w = WORKLOADS["tiny"].with_(batch=b, dim=d, dstate=n, seqlen=L, io=io, gate=True,
                                initial_state=True, a_kind="scaled", seed=700 + L + n)
    announce(w.describe() + " backward (atomics)")
    inp, dout, dfin = setup(w, seed=L + 1)
    *_, got = run_gpu(inp, dout, dfin, True, deterministic=False)
    compare(io, got, run_oracle(inp, dout, dfin, True), w.describe() + " atomics")


def test_backward_workspace_reused_and_paths_agree():
    """One caller-held workspace, larger than needed, serves two different problems in a
    row; on the same problem the two summation paths agree within float32 rounding and, with
    the sequences kept whole (SSM_BWD_UNSPLIT, as the atomic path keeps them), the
    per-element gradients are identical."""
    t = torch()
    need = max(ssm.ssm_scan_bwd_workspace_bytes(2, 40, 16, 900, ssm.SSM_IO_BF16),
               ssm.ssm_scan_bwd_workspace_bytes(1, 24, 8, 1500, ssm.SSM_IO_BF16))
    ws = t.full((need + 4096,), 0x7F, dtype=t.uint8, device="cuda")  # stale contents
    for i, (b, d, n, L) in enumerate([(2, 40, 16, 900), (1, 24, 8, 1500)]):
        w = WORKLOADS["tiny"].with_(batch=b, dim=d, dstate=n, seqlen=L, io="bf16", gate=True,
                                    initial_state=True, seed=67 + i)
        announce(w.describe() + " workspace reuse")
        inp, dout, dfin = setup(w, seed=67 + i)
        *_, gw = run_gpu(inp, dout, dfin, True, workspace=ws, unsplit=True)
        compare("bf16", gw, run_oracle(inp, dout, dfin, True), w.describe() + " reused ws")
        *_, ga = run_gpu(inp, dout, dfin, True, deterministic=False)
        for k in ("du", "ddelta", "dz", "dh0"):
            assert np.array_equal(gw[k], ga[k]), k
        for k in ("dA", "dB", "dC", "dD", "dbias"):
            rep = parity(ga[k], gw[k].astype(np.float64), 1e-5)
            print(f"[paths] {k}: {rep}", flush=True)
            assert rep.ok, f"{k}: {rep}"


def _segments(b, d, L, io):
    """The segments the library cuts each sequence into here: the workspace sizes with and
    without SSM_BWD_UNSPLIT differ exactly when it cuts (the carries and per-segment slots)."""
    flags = ssm.SSM_IO_BF16 if io == "bf16" else ssm.SSM_IO_F32
    return (ssm.ssm_scan_bwd_workspace_bytes(b, d, 16, L, flags)
            > ssm.ssm_scan_bwd_workspace_bytes(b, d, 16, L, flags | ssm.SSM_BWD_UNSPLIT))


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(4, 320, 16, 2700), (1, 37, 16, 4100), (2, 40, 16, 600)],
                         ids=lambda s: "b{}d{}N{}L{}".format(*s))
def test_backward_segments(shape, io):
    """Few channels, long sequences: the workspace path cuts each sequence into segments
    (on a 256-CU device: 6 segments of two intervals, the last of one, for the first shape;
    one interval each for the others), each scanned from the adjoint carried into it. Every
    gradient against the oracle, bitwise reproducible, and within float32 rounding of the
    uncut backward."""
    b, d, n, L = shape
    w = WORKLOADS["tiny"].with_(batch=b, dim=d, dstate=n, seqlen=L, io=io, gate=True,
                                initial_state=True, seed=800 + L)
    announce(w.describe() + " backward in segments")
    if not _segments(b, d, L, io):  # a device with fewer compute units may not cut this shape
        pytest.skip("this device keeps these sequences whole")
    inp, dout, dfin = setup(w, seed=L + 3)
    *_, g1 = run_gpu(inp, dout, dfin, True)
    compare(io, g1, run_oracle(inp, dout, dfin, True), w.describe() + " segments")
    *_, g2 = run_gpu(inp, dout, dfin, True)
    for k in ALL_GRADS:
        assert np.array_equal(g1[k], g2[k]), k
    *_, gu = run_gpu(inp, dout, dfin, True, unsplit=True)
    for k in ALL_GRADS:
        # bf16 per-element outputs: float32 values 1e-5 apart may round one bf16 step apart
        tol = 2.0 ** -8 * 1.01 if (io == "bf16" and k in PER_ELEMENT) else 1e-5
        rep = parity(g1[k].astype(np.float32), gu[k].astype(np.float64), tol)
        print(f"[segments vs whole] {k}: {rep}", flush=True)
        assert rep.ok, f"{k}: {rep}"


def test_backward_layer_workload_full():
    """The benchmark's layer shape (b4 d2048 N16 L2048 bf16, gated): every gradient
    against the oracle, whole tensors."""
    w = WORKLOADS["layer"]
    announce(w.describe() + " backward")
    inp, dout, dfin = setup(w, seed=65)
    *_, got = run_gpu(inp, dout, dfin, True)
    compare(w.io, got, run_oracle(inp, dout, dfin, True), w.describe())

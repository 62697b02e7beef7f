"""GPU parity of the Mamba-2 (SSD) forward (through the C ABI) against the float64
recurrence oracle (oracle.ssd_ref, pinned in test_oracle_ssd_pins.py).

Bars (the metric of ssm_workloads.compare): out 2e-2 (bf16 storage: the kernel rounds the
block matrix and the carried state to bf16 for its matrix products, and out once on
store), final_state 1e-4 (fp32; the state update keeps fp32-level accuracy by splitting its
bf16 operand in two halves).

Shapes cover: 1, 2 and 3 state tiles per wave (dstate 64, 128, 256); headdim 16 and 48
(a channel group with an idle half); sequences of 1 step, of one and several 64-step
blocks, ragged tails, and lengths that are not a multiple of 8 (the element-wise path);
every optional input; padding masks; the full ssd workload.
"""
import numpy as np
import pytest

import oracle
import selective_state_space_fwd_amd as ssm
from gpu_util import announce, dev, host, torch
from ssm_workloads import (RTOL, RTOL_STATE, SSD_WORKLOADS, f32_to_bf16_bits, make_mask,
                           make_ssd_inputs, parity, widen)

pytestmark = pytest.mark.gpu


def run_gpu(inp, softplus=True, use=("D", "z", "dt_bias", "h0"), mask=None, workspace=None):
    t = torch()
    g = {k: dev(inp[k], "bf16") for k in ("x", "dt", "B", "C", "z")}
    f = {k: dev(inp[k], "f32") for k in ("A", "D", "dt_bias", "h0")}
    pick = lambda k, src: src[k] if k in use else None
    out, fin = ssm.ssd(g["x"], g["dt"], f["A"], g["B"], g["C"], D=pick("D", f),
                       z=pick("z", g), dt_bias=pick("dt_bias", f), dt_softplus=softplus,
                       h0=pick("h0", f), mask=None if mask is None else t.from_numpy(mask).cuda(),
                       workspace=workspace)
    t.cuda.synchronize()
    return host(out), host(fin)


def run_oracle(inp, softplus=True, use=("D", "z", "dt_bias", "h0"), mask=None):
    w = lambda k: widen(inp[k], "bf16")
    pick = lambda k, v: v if k in use else None
    return oracle.ssd_ref(w("x"), w("dt"), inp["A"], w("B"), w("C"), pick("D", inp["D"]),
                          pick("z", None if inp["z"] is None else w("z")),
                          pick("dt_bias", inp["dt_bias"]), softplus, pick("h0", inp["h0"]),
                          mask=mask)


def check(got, ref, label):
    ro = parity(got[0], ref[0], RTOL["bf16"])
    rf = parity(got[1], ref[1], RTOL_STATE)
    print(f"[parity] {label}: out {ro} | final {rf}", flush=True)
    assert ro.ok, f"{label} out: {ro}"
    assert rf.ok, f"{label} final_state: {rf}"


SHAPES = [
    # (batch, nheads, headdim, dstate, seqlen)
    (1, 2, 64, 64, 64), (2, 3, 32, 64, 100), (1, 2, 16, 128, 1), (2, 2, 48, 128, 200),
    (1, 1, 64, 256, 300), (2, 4, 64, 128, 1024), (1, 2, 32, 64, 2047), (3, 2, 32, 128, 4096),
    (1, 3, 64, 256, 777),
]


@pytest.mark.parametrize("h0", [False, True], ids=["zero_state", "h0"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}h{}x{}N{}L{}".format(*s))
def test_ssd_shapes(shape, h0):
    b, nh, p, n, L = shape
    w = SSD_WORKLOADS["ssd_tiny"].with_(batch=b, nheads=nh, headdim=p, dstate=n, seqlen=L,
                                        initial_state=h0, seed=1000 + L + n + p)
    announce(w.describe())
    inp = make_ssd_inputs(w)
    check(run_gpu(inp), run_oracle(inp), w.describe())


@pytest.mark.parametrize("variant", ["no_D", "no_z", "no_bias", "no_softplus", "bare"])
def test_ssd_optional_inputs(variant):
    w = SSD_WORKLOADS["ssd_tiny"].with_(batch=2, nheads=2, headdim=32, dstate=64, seqlen=640,
                                        initial_state=True, seed=1100)
    announce(f"{w.describe()} {variant}")
    inp = make_ssd_inputs(w)
    use = {"no_D": ("z", "dt_bias", "h0"), "no_z": ("D", "dt_bias", "h0"),
           "no_bias": ("D", "z", "h0"), "no_softplus": ("D", "z", "dt_bias", "h0"),
           "bare": ()}[variant]
    softplus = variant not in ("no_softplus", "bare")
    if not softplus:  # positive step sizes without softplus
        raw = widen(inp["dt"], "bf16")
        inp["dt"] = f32_to_bf16_bits((np.abs(raw) * 0.05 + 1e-3).astype(np.float32))
        inp["dt_bias"] = np.abs(inp["dt_bias"]) * 0.01
    check(run_gpu(inp, softplus, use), run_oracle(inp, softplus, use), f"{w.describe()} {variant}")


@pytest.mark.parametrize("kind", ["lengths", "left", "random", "zeros"])
@pytest.mark.parametrize("L", [50, 1000])
def test_ssd_padding_mask(kind, L):
    w = SSD_WORKLOADS["ssd_tiny"].with_(batch=3, nheads=2, headdim=32, dstate=128, seqlen=L,
                                        initial_state=True, seed=1200 + L)
    announce(f"{w.describe()} mask={kind}")
    inp = make_ssd_inputs(w)
    mask = make_mask(3, L, kind, seed=1201 + L)
    got = run_gpu(inp, mask=mask)
    check(got, run_oracle(inp, mask=mask), f"{w.describe()} mask={kind}")
    if kind == "zeros":
        assert np.array_equal(got[1], inp["h0"].astype(np.float64))


def test_ssd_deterministic_and_workspace_reuse():
    t = torch()
    w = SSD_WORKLOADS["ssd_tiny"].with_(batch=2, nheads=4, headdim=64, dstate=128, seqlen=1500,
                                        seed=1300)
    announce(w.describe() + " determinism")
    inp = make_ssd_inputs(w)
    ws = t.empty(ssm.ssm_ssd_workspace_bytes(2, 4, 128, 1500), dtype=t.uint8, device="cuda")
    a = run_gpu(inp, workspace=ws)
    b = run_gpu(inp, workspace=ws)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_ssd_chained_calls_equal_one_call():
    """Two calls handing the final state on (state passing) against one call, both against
    the oracle; the split is not at a block boundary."""
    w = SSD_WORKLOADS["ssd_tiny"].with_(batch=2, nheads=2, headdim=32, dstate=64, seqlen=300,
                                        initial_state=True, seed=1400)
    announce(w.describe() + " chained")
    inp = make_ssd_inputs(w)
    cut = 131
    first = {k: (v[..., :cut] if k in ("x", "dt", "B", "C", "z") else v) for k, v in inp.items()}
    second = {k: (v[..., cut:] if k in ("x", "dt", "B", "C", "z") else v) for k, v in inp.items()}
    o1, f1 = run_gpu({k: (np.ascontiguousarray(v) if isinstance(v, np.ndarray) else v)
                      for k, v in first.items()})
    second["h0"] = f1.astype(np.float32)
    o2, f2 = run_gpu({k: (np.ascontiguousarray(v) if isinstance(v, np.ndarray) else v)
                      for k, v in second.items()})
    ref = run_oracle(inp)
    check((np.concatenate([o1, o2], axis=2), f2), ref, w.describe() + " chained")


def test_ssd_workload_full():
    """The benchmark's SSD shape (b4, 32 heads x 64, N128, L2048, bf16, gated): whole
    tensors against the oracle."""
    w = SSD_WORKLOADS["ssd"]
    announce(w.describe())
    inp = make_ssd_inputs(w)
    check(run_gpu(inp), run_oracle(inp), w.describe())


@pytest.mark.parametrize("dstate", [64, 128])
def test_ssd_large_decay_blocks(dstate):
    """Blocks whose decay exceeds the separable form's span (120 in natural-log units; the
    kernel then forms the decayed block matrix) beside blocks within it. A is set per head
    so that a head's median 64-step block decays by 0.3, 1, 3 and 10 times that span: the
    second head has blocks on both sides of it."""
    w = SSD_WORKLOADS["ssd_tiny"].with_(batch=2, nheads=4, headdim=32, dstate=dstate,
                                        seqlen=700, initial_state=True, seed=1500 + dstate)
    announce(f"{w.describe()} large decay")
    inp = make_ssd_inputs(w)
    raw = widen(inp["dt"], "bf16") + inp["dt_bias"][None, :, None]
    step = np.where(raw <= 20, np.logaddexp(0.0, raw), raw)[..., :640]
    block_sum = np.median(step.reshape(2, 4, 10, 64).sum(-1), axis=(0, 2))   # per head
    inp["A"] = (-120.0 * np.array([0.3, 1.0, 3.0, 10.0]) / block_sum).astype(np.float32)
    span = -(step * inp["A"][None, :, None]).reshape(2, 4, 10, 64).sum(-1)
    assert (span[:, 1] > 120).any() and (span[:, 1] <= 120).any()
    check(run_gpu(inp), run_oracle(inp), f"{w.describe()} large decay")

"""GPU padding mask (through the C ABI) against the float64 oracle with the same mask.

A padding step (mask 0) keeps the state and still emits C h + D u of that state
(mhpq.cn/news/1057127 section 4). Masks are drawn by ssm_workloads.make_mask: right- and
left-padded batches of different lengths, scattered padding, all real, all padding. The
shapes cover both forward kernels (at most 32 steps, and the chunked scan with several
1024-step chunks and a ragged tail), the saved states of a training forward, and the
backward pass. Bars are those of the unmasked tests (RTOL per storage type for
per-element tensors, 1e-4 for float32 states and summed gradients).
"""
import numpy as np
import pytest

import oracle
import selective_state_space_fwd_amd as ssm
from gpu_util import announce, dev, host, torch
from ssm_workloads import (RTOL, WATCH, RTOL_STATE, WORKLOADS, f32_to_bf16_bits, make_inputs,
                           make_mask, parity, widen)

pytestmark = pytest.mark.gpu

RTOL_F32_OUT = 1e-4
PER_ELEMENT = ("du", "ddelta", "dz")


def case(b, d, n, L, io, seed, h0=True):
    w = WORKLOADS["tiny"].with_(batch=b, dim=d, dstate=n, seqlen=L, io=io, gate=True,
                                initial_state=h0, a_kind="scaled", seed=seed)
    return w, make_inputs(w)


def gpu_inputs(inp):
    io = inp["io"]
    g = {k: dev(inp[k], io) for k in ("u", "delta", "B", "C", "z")}
    g.update({k: dev(inp[k], "f32") for k in ("A", "D", "delta_bias", "h0")})
    return g


def gpu_fwd(inp, mask, mask_dtype="uint8"):
    t = torch()
    g = gpu_inputs(inp)
    m = None
    if mask is not None:
        m = t.from_numpy(mask).to("cuda")
        if mask_dtype == "bool":
            m = m.bool()
    out, fin = ssm.scan(g["u"], g["delta"], g["A"], g["B"], g["C"], D=g["D"], z=g["z"],
                        delta_bias=g["delta_bias"], delta_softplus=True, h0=g["h0"], mask=m)
    t.cuda.synchronize()
    return host(out), host(fin)


def oracle_fwd(inp, mask, upto=None):
    io = inp["io"]
    cut = (lambda x: x) if upto is None else (lambda x: x[..., :upto])
    return oracle.scan_ref(
        widen(cut(inp["u"]), io), widen(cut(inp["delta"]), io), inp["A"],
        widen(cut(inp["B"]), io), widen(cut(inp["C"]), io), inp["D"],
        widen(cut(inp["z"]), io), inp["delta_bias"], True, inp["h0"],
        mask=None if mask is None else np.ascontiguousarray(cut(mask)))


def check(io, got, ref, label):
    ro = parity(got[0], ref[0], RTOL[io], WATCH[io])
    rf = parity(got[1], ref[1], RTOL_STATE)
    print(f"[parity] {label}: out {ro} | final {rf}", flush=True)
    assert ro.ok, f"{label} out: {ro}"
    assert rf.ok, f"{label} final_state: {rf}"


FWD_SHAPES = [
    # (batch, dim, dstate, seqlen): short kernel (<= 32 steps), then the chunked scan with
    # one chunk, a ragged tail, several chunks; ragged channel counts
    (3, 7, 16, 1), (3, 5, 16, 20), (2, 6, 64, 32), (3, 9, 16, 33), (2, 5, 16, 1000),
    (3, 6, 16, 2500), (2, 10, 4, 4096),
]


@pytest.mark.parametrize("kind", ["lengths", "left", "random"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", FWD_SHAPES, ids=lambda s: "b{}d{}N{}L{}".format(*s))
def test_masked_forward(shape, io, kind):
    b, d, n, L = shape
    w, inp = case(b, d, n, L, io, seed=800 + L + n)
    mask = make_mask(b, L, kind, seed=801 + L)
    label = f"{w.describe()} mask={kind}"
    announce(label)
    check(io, gpu_fwd(inp, mask), oracle_fwd(inp, mask), label)


@pytest.mark.parametrize("L", [20, 1500])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_mask_of_ones_is_bitwise_the_unmasked_scan(io, L):
    w, inp = case(2, 9, 16, L, io, seed=810 + L)
    announce(f"{w.describe()} mask=ones vs no mask")
    a = gpu_fwd(inp, None)
    m = gpu_fwd(inp, make_mask(2, L, "ones", 0))
    assert np.array_equal(a[0], m[0]) and np.array_equal(a[1], m[1])


@pytest.mark.parametrize("L", [7, 1100])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_all_padding_keeps_the_initial_state(io, L):
    w, inp = case(2, 6, 16, L, io, seed=820 + L)
    mask = make_mask(2, L, "zeros", 0)
    label = f"{w.describe()} mask=zeros"
    announce(label)
    got = gpu_fwd(inp, mask)
    # a zero step size gives exp(0) = 1 and a zero input term: the state is h0 exactly
    assert np.array_equal(got[1], inp["h0"].astype(np.float64))
    check(io, got, oracle_fwd(inp, mask), label)


def test_bool_mask_equals_uint8_mask():
    w, inp = case(2, 5, 16, 700, "bf16", seed=830)
    mask = make_mask(2, 700, "random", 831)
    announce(f"{w.describe()} bool mask")
    a = gpu_fwd(inp, mask)
    b = gpu_fwd(inp, mask, mask_dtype="bool")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_masked_saved_states(io):
    """Entry k of the training forward's saved states is the masked state entering step
    SSM_CKPT_INTERVAL k."""
    w, inp = case(2, 6, 16, 1700, io, seed=840)
    mask = make_mask(2, 1700, "random", 841)
    mask[0, 900:] = 0
    announce(f"{w.describe()} masked saved states")
    t = torch()
    g = gpu_inputs(inp)
    out, fin, states = ssm.scan_train(g["u"], g["delta"], g["A"], g["B"], g["C"], D=g["D"],
                                      z=g["z"], delta_bias=g["delta_bias"],
                                      delta_softplus=True, h0=g["h0"],
                                      mask=t.from_numpy(mask).to("cuda"))
    t.cuda.synchronize()
    o2, f2 = gpu_fwd(inp, mask)
    assert np.array_equal(host(out), o2) and np.array_equal(host(fin), f2)
    states = host(states)
    for k in range(states.shape[2]):
        ref = inp["h0"].astype(np.float64) if k == 0 else oracle_fwd(inp, mask, upto=ssm.SSM_CKPT_INTERVAL * k)[1]
        rep = parity(states[:, :, k], ref, RTOL_F32_OUT)
        assert rep.ok, f"state {k}: {rep}"


def bwd_case(w, inp, seed):
    rng = np.random.default_rng(seed)
    dout = rng.standard_normal(inp["u"].shape).astype(np.float32)
    if w.io == "bf16":
        dout = f32_to_bf16_bits(dout)
    dfin = rng.standard_normal((w.batch, w.dim, w.dstate)).astype(np.float32)
    return dout, dfin


def gpu_bwd(inp, dout, dfin, mask):
    t = torch()
    io = inp["io"]
    g = gpu_inputs(inp)
    m = t.from_numpy(mask).to("cuda")
    _, _, states = ssm.scan_train(g["u"], g["delta"], g["A"], g["B"], g["C"], D=g["D"],
                                  z=g["z"], delta_bias=g["delta_bias"], delta_softplus=True,
                                  h0=g["h0"], mask=m)
    grads = ssm.scan_backward(g["u"], g["delta"], g["A"], g["B"], g["C"], states,
                              dev(dout, io), D=g["D"], z=g["z"], delta_bias=g["delta_bias"],
                              delta_softplus=True, dfinal=dev(dfin, "f32"), mask=m)
    t.cuda.synchronize()
    return {k: (None if v is None else host(v)) for k, v in grads.items()}


def oracle_bwd(inp, dout, dfin, mask):
    io = inp["io"]
    return oracle.scan_bwd_ref(
        widen(inp["u"], io), widen(inp["delta"], io), inp["A"], widen(inp["B"], io),
        widen(inp["C"], io), inp["D"], widen(inp["z"], io), inp["delta_bias"], True,
        inp["h0"], widen(dout, io), dfin.astype(np.float64), mask=mask)


def compare_grads(io, got, ref, label):
    for k, r in ref.items():
        if r is None:
            assert got.get(k) is None, f"{label}: {k} should be absent"
            continue
        rep = parity(got[k], r, RTOL[io] if k in PER_ELEMENT else RTOL_F32_OUT,
                     WATCH[io] if k in PER_ELEMENT else None)
        print(f"[grad] {label} {k}: {rep}", flush=True)
        assert rep.ok, f"{label} {k}: {rep}"


BWD_SHAPES = [(3, 5, 16, 9), (3, 7, 16, 600), (2, 5, 8, 1500), (3, 4, 17, 2049)]


@pytest.mark.parametrize("kind", ["lengths", "left", "random", "zeros"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", BWD_SHAPES, ids=lambda s: "b{}d{}N{}L{}".format(*s))
def test_masked_backward(shape, io, kind):
    b, d, n, L = shape
    w, inp = case(b, d, n, L, io, seed=850 + L + n)
    mask = make_mask(b, L, kind, seed=851 + L)
    label = f"{w.describe()} backward mask={kind}"
    announce(label)
    dout, dfin = bwd_case(w, inp, 852 + L)
    got = gpu_bwd(inp, dout, dfin, mask)
    compare_grads(io, got, oracle_bwd(inp, dout, dfin, mask), label)
    pad = np.broadcast_to(mask[:, None, :] == 0, got["ddelta"].shape)
    assert not got["ddelta"][pad].any(), "a padding step's step size got a gradient"


def test_masked_layer_workload_full():
    """The layer shape (b4 d2048 N16 L2048 bf16, gated) as a right-padded batch of four
    sequences of different lengths: forward and backward, whole tensors, against the
    oracle."""
    w = WORKLOADS["layer"]
    inp = make_inputs(w)
    mask = make_mask(w.batch, w.seqlen, "lengths", seed=860)
    announce(w.describe() + " mask=lengths forward+backward")
    check(w.io, gpu_fwd(inp, mask), oracle_fwd(inp, mask), w.describe() + " mask")
    dout, dfin = bwd_case(w, inp, 861)
    compare_grads(w.io, gpu_bwd(inp, dout, dfin, mask), oracle_bwd(inp, dout, dfin, mask),
                  w.describe() + " mask")

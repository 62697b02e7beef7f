"""A second launch shape of the chunked scan kernel, against the oracle and the default build.

libssmscan_shape2.so is the Mamba-1 scan built with other compile-time launch parameters:
4 channels per workgroup and 4 states per LDS stage for bf16 storage (the default build has
8 and 2), 2 channels per workgroup and 1 state per stage for fp32 (default 4 and 2); both
keep 16 steps per lane (a 1024-step chunk, four 256-step saved-state intervals). The mapping
of channels to workgroups and of states to stages changes; the arithmetic of each state, and
the order in which y sums the states, do not. With one wave per channel (fp32 forced through
SSM_WAVES_PER_CHANNEL_1) every output and saved state must therefore be bitwise equal to the
default build's, and both within the float64 oracle's bar (1e-4 fp32, 2e-2 bf16 out; 1e-4
states).
"""
import ctypes

import numpy as np
import pytest

import oracle
import selective_state_space_fwd_amd as ssm
from gpu_util import announce, dev, host, torch
from selective_state_space_fwd_amd.build import SHAPE2_LIB_PATH
from ssm_workloads import RTOL, WATCH, RTOL_STATE, WORKLOADS, make_inputs, make_mask, parity, widen

pytestmark = pytest.mark.gpu

_shape2 = None


def shape2_lib():
    global _shape2
    if _shape2 is None:
        ssm.lib()  # binds the HIP runtime of torch first
        L = ctypes.CDLL(SHAPE2_LIB_PATH)
        vp, i64, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32
        L.ssm_scan_fwd_masked.argtypes = [vp] * 9 + [u32, vp, vp, vp, i64, i64, i64, i64, vp]
        L.ssm_scan_fwd_masked.restype = ctypes.c_int
        _shape2 = L
    return _shape2


def run(L, inp, mask=None, ckpt=False):
    """One masked-entry call (mask and saved states optional) through library L."""
    t = torch()
    io = inp["io"]
    g = {k: dev(inp[k], io) for k in ("u", "delta", "B", "C", "z")}
    f = {k: dev(inp[k], "f32") for k in ("A", "D", "delta_bias", "h0")}
    batch, dim, L_ = inp["u"].shape
    n = inp["A"].shape[1]
    out = t.empty_like(g["u"])
    fin = f["h0"].clone() if f["h0"] is not None else t.empty((batch, dim, n), device="cuda")
    states = t.empty((batch, dim, -(-L_ // ssm.SSM_CKPT_INTERVAL), n), device="cuda") if ckpt else None
    m = None if mask is None else t.from_numpy(mask).cuda()
    flags = (ssm.SSM_IO_BF16 if io == "bf16" else ssm.SSM_IO_F32) | ssm.SSM_DELTA_SOFTPLUS
    flags |= ssm.SSM_INITIAL_STATE if f["h0"] is not None else 0
    flags |= ssm.SSM_WAVES_PER_CHANNEL_1
    P = lambda x: None if x is None else x.data_ptr()
    st = L.ssm_scan_fwd_masked(P(g["u"]), P(g["delta"]), P(f["A"]), P(g["B"]), P(g["C"]),
                               P(f["D"]), P(g["z"]), P(f["delta_bias"]), P(m), flags, P(out),
                               P(fin), P(states), batch, dim, n, L_,
                               t.cuda.current_stream().cuda_stream)
    assert st == ssm.SSM_OK, ssm.ssm_scan_strerror(st)
    t.cuda.synchronize()
    return host(out), host(fin), None if states is None else host(states)


SHAPES = [
    # (batch, dim, dstate, seqlen): several workgroups with a ragged last one, vector and
    # element-wise rows, one and several chunks, ragged tails, 1 / 5 / 16 / 17 / 64 states
    (2, 13, 16, 600), (1, 9, 16, 2048), (2, 7, 17, 1537), (1, 6, 5, 777), (1, 5, 64, 1100),
    (3, 4, 1, 300), (1, 11, 16, 4099),
]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}d{}N{}L{}".format(*s))
def test_second_launch_shape(shape, io):
    b, d, n, L = shape
    w = WORKLOADS["tiny"].with_(batch=b, dim=d, dstate=n, seqlen=L, io=io, gate=True,
                                initial_state=True, a_kind="scaled" if n != 16 else "s4d",
                                seed=1700 + L + n)
    announce(f"{w.describe()} second launch shape")
    inp = make_inputs(w)
    got = run(shape2_lib(), inp, ckpt=True)
    base = run(ssm.lib(), inp, ckpt=True)
    for k, (x, y) in enumerate(zip(got, base)):
        assert np.array_equal(x, y), f"output {k} differs from the default build"
    ro, rf = oracle.scan_ref(widen(inp["u"], io), widen(inp["delta"], io), inp["A"],
                             widen(inp["B"], io), widen(inp["C"], io), inp["D"],
                             widen(inp["z"], io), inp["delta_bias"], True, inp["h0"])
    po, pf = parity(got[0], ro, RTOL[io], WATCH[io]), parity(got[1], rf, RTOL_STATE)
    print(f"[shape2] {w.describe()}: out {po} | final {pf}", flush=True)
    assert po.ok and pf.ok


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_second_launch_shape_masked(io):
    w = WORKLOADS["tiny"].with_(batch=3, dim=9, dstate=16, seqlen=1300, io=io, gate=True,
                                initial_state=True, seed=1750)
    announce(f"{w.describe()} second launch shape, padding mask")
    inp = make_inputs(w)
    mask = make_mask(w.batch, w.seqlen, "random", seed=1751)
    got = run(shape2_lib(), inp, mask=mask)
    base = run(ssm.lib(), inp, mask=mask)
    assert np.array_equal(got[0], base[0]) and np.array_equal(got[1], base[1])
    ro, rf = oracle.scan_ref(widen(inp["u"], io), widen(inp["delta"], io), inp["A"],
                             widen(inp["B"], io), widen(inp["C"], io), inp["D"],
                             widen(inp["z"], io), inp["delta_bias"], True, inp["h0"], mask=mask)
    assert parity(got[0], ro, RTOL[io], WATCH[io]).ok and parity(got[1], rf, RTOL_STATE).ok

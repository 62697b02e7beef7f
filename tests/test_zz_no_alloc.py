"""The allocation-free Mamba-2 forward (ssm_ssd_fwd_noalloc, for callers that cannot allocate)
against the entry point that takes a workspace (ssm_ssd_fwd), through the C ABI.

Both run the same kernels on the same inputs, so their outputs and final states must be
bitwise equal; both are also checked against the float64 recurrence oracle at the SSD bars
(out 2e-2 with bf16 storage, final_state 1e-4). Two problems run one after the other, the
second smaller, so the second call finds the first call's contents in the static buffer; a
third call repeats the first problem after the second.
"""
import numpy as np
import pytest

import oracle
import selective_state_space_fwd_amd as ssm
from gpu_util import announce, dev, host, torch
from ssm_workloads import RTOL, RTOL_STATE, SSD_WORKLOADS, make_mask, make_ssd_inputs, parity, widen

pytestmark = pytest.mark.gpu


def _run(inp, w, noalloc, mask=None):
    t = torch()
    g = {k: dev(inp[k], "bf16") for k in ("x", "dt", "B", "C", "z")}
    f = {k: dev(inp[k], "f32") for k in ("A", "D", "dt_bias", "h0")}
    out = t.empty_like(g["x"])
    fin = (f["h0"].clone() if f["h0"] is not None
           else t.empty((w.batch, w.dim, w.dstate), device="cuda", dtype=t.float32))
    m = None if mask is None else t.from_numpy(mask).cuda()
    flags = ssm.SSM_IO_BF16 | ssm.SSM_DELTA_SOFTPLUS | (
        ssm.SSM_INITIAL_STATE if f["h0"] is not None else 0)
    P = lambda x: None if x is None else x.data_ptr()
    stream = t.cuda.current_stream().cuda_stream
    common = (P(g["x"]), P(g["dt"]), P(f["A"]), P(g["B"]), P(g["C"]), P(f["D"]), P(g["z"]),
              P(f["dt_bias"]), P(m), flags, P(out), P(fin))
    sizes = (w.batch, w.nheads, w.headdim, w.dstate, w.seqlen, stream)
    if noalloc:
        st = ssm.ssm_ssd_fwd_noalloc(*common, *sizes)
    else:
        need = ssm.ssm_ssd_workspace_bytes(w.batch, w.nheads, w.dstate, w.seqlen)
        ws = t.empty((max(need, 1),), device="cuda", dtype=t.uint8)
        st = ssm.ssm_ssd_fwd(*common, P(ws), ws.numel(), *sizes)
    assert st == ssm.SSM_OK, ssm.ssm_scan_strerror(st)
    t.cuda.synchronize()
    return host(out), host(fin)


def _oracle(inp, mask=None):
    W = lambda k: widen(inp[k], "bf16")
    return oracle.ssd_ref(W("x"), W("dt"), inp["A"], W("B"), W("C"), inp["D"], W("z"),
                          inp["dt_bias"], True, inp["h0"], mask=mask)


CASES = [
    # (batch, nheads, headdim, dstate, seqlen, h0, mask): the larger first, then a smaller
    # one, then the larger again
    (2, 4, 64, 128, 700, True, None),
    (1, 2, 32, 64, 130, False, "lengths"),
    (2, 4, 64, 128, 700, True, None),
]


def test_noalloc_matches_the_workspace_entry_point_on_consecutive_calls():
    for i, (b, nh, p, n, L, h0, mk) in enumerate(CASES):
        w = SSD_WORKLOADS["ssd_tiny"].with_(batch=b, nheads=nh, headdim=p, dstate=n,
                                            seqlen=L, initial_state=h0, seed=1300 + L + n)
        need = ssm.ssm_ssd_workspace_bytes(b, nh, n, L)
        assert 0 < need <= ssm.SSM_SSD_NOALLOC_SCRATCH_BYTES
        announce(f"noalloc call {i}: {w.describe()} mask={mk} workspace={need} B")
        inp = make_ssd_inputs(w)
        mask = None if mk is None else make_mask(b, L, mk, seed=1301)
        got = _run(inp, w, noalloc=True, mask=mask)
        want = _run(inp, w, noalloc=False, mask=mask)
        assert np.array_equal(got[0], want[0]), "out differs from ssm_ssd_fwd"
        assert np.array_equal(got[1], want[1]), "final_state differs from ssm_ssd_fwd"
        ref = _oracle(inp, mask)
        ro, rf = parity(got[0], ref[0], RTOL["bf16"]), parity(got[1], ref[1], RTOL_STATE)
        print(f"[noalloc] {w.describe()}: out {ro} | final {rf}", flush=True)
        assert ro.ok and rf.ok


def test_noalloc_full_ssd_workload():
    """The Mamba-2 bench workload (b4, 32 heads of 64 channels, 128 states, 2048 steps) fits
    the static buffer; outputs bitwise those of the workspace entry point."""
    w = SSD_WORKLOADS["ssd"]
    announce(f"noalloc {w.describe()}")
    inp = make_ssd_inputs(w)
    got = _run(inp, w, noalloc=True)
    want = _run(inp, w, noalloc=False)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])

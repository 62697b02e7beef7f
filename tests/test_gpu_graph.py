"""The forward entry points under HIP graph capture (torch.cuda.CUDAGraph records the
launches the library makes on the capturing stream).

A serving loop captures its per-token work once and replays it; the library's forward
calls enqueue kernels only (no memset, no host synchronisation, no allocation), so they
record as plain kernel nodes. Each test replays its graph several times, with the
program's own eager work and synchronisations between the replays, and checks every
replay bitwise against the same calls made eagerly (same kernels, no atomics, so the
results are reproducible), and the eager results against the float64 oracle.

Cases: a decode loop of one-token calls carrying the state in place (the state cache of
ybb.press/ai-applications/14118.html section 5.1, one call per generated token), the
chunked forward at a layer-like shape with new inputs written into the captured buffers
between replays, the Mamba-2 (SSD) forward with a caller-held workspace, and a training
step (forward with saved states, then the backward with its workspace, whose fixed-order
sums make every gradient bitwise reproducible).
"""
import numpy as np
import pytest

import oracle
import selective_state_space_fwd_amd as ssm
from gpu_util import announce, dev, host, torch
from ssm_workloads import (RTOL, WATCH, RTOL_STATE, SSD_WORKLOADS, WORKLOADS, make_inputs,
                           make_ssd_inputs, parity, widen)

pytestmark = pytest.mark.gpu

REPLAYS = 3


def check(io, got, ref, label):
    ro = parity(got[0], ref[0], RTOL[io], WATCH[io])
    rf = parity(got[1], ref[1], RTOL_STATE)
    print(f"[parity] {label}: out {ro} | final {rf}", flush=True)
    assert ro.ok, f"{label} out: {ro}"
    assert rf.ok, f"{label} final_state: {rf}"


def same(a, b):
    t = torch()
    return bool(t.equal(a.view(t.int16) if a.dtype == t.bfloat16 else a,
                        b.view(t.int16) if b.dtype == t.bfloat16 else b))


def unrelated_eager_work(t):
    """Work of the program's own between replays: torch kernels and a library call on
    buffers the graph does not use."""
    a = t.randn(512, 512, device="cuda")
    (a @ a).sum().item()
    w = WORKLOADS["tiny"].with_(batch=1, dim=8, seqlen=100, seed=77)
    inp = make_inputs(w)
    g = {k: dev(inp[k], "f32") for k in ("u", "delta", "B", "C", "A", "D", "delta_bias")}
    ssm.scan(g["u"], g["delta"], g["A"], g["B"], g["C"], D=g["D"],
             delta_bias=g["delta_bias"], delta_softplus=True)
    t.cuda.synchronize()


def test_graph_decode_loop():
    """Sixteen one-token calls at the decode shape (b8, 2048 channels, 64 states, bf16,
    gated), each reading and overwriting the same fp32 state tensor, captured once."""
    t = torch()
    steps = 16
    w = WORKLOADS["decode"].with_(seqlen=steps, seed=501)
    announce(f"{w.describe()} graph decode loop")
    inp = make_inputs(w)
    tok = [{k: dev(np.ascontiguousarray(inp[k][..., s:s + 1]), w.io)
            for k in ("u", "delta", "B", "C", "z")} for s in range(steps)]
    par = {k: dev(inp[k], "f32") for k in ("A", "D", "delta_bias", "h0")}
    state = par["h0"].clone()

    def loop(outs):
        for s in range(steps):
            g = tok[s]
            ssm.scan(g["u"], g["delta"], par["A"], g["B"], g["C"], D=par["D"], z=g["z"],
                     delta_bias=par["delta_bias"], delta_softplus=True, h0=state,
                     final_state=state, out=outs[s])

    eager_out = [t.empty_like(tok[s]["u"]) for s in range(steps)]
    loop(eager_out)
    t.cuda.synchronize()
    eager_state = state.clone()
    ref = oracle.scan_ref(widen(inp["u"], w.io), widen(inp["delta"], w.io), inp["A"],
                          widen(inp["B"], w.io), widen(inp["C"], w.io), inp["D"],
                          widen(inp["z"], w.io), inp["delta_bias"], True, inp["h0"])
    got = (np.concatenate([host(o) for o in eager_out], axis=2), host(eager_state))
    check(w.io, got, ref, f"{w.describe()} eager decode loop")

    graph_out = [t.empty_like(tok[s]["u"]) for s in range(steps)]
    graph = t.cuda.CUDAGraph()
    state.copy_(par["h0"])
    t.cuda.synchronize()
    with t.cuda.graph(graph):
        loop(graph_out)
    for r in range(REPLAYS):
        state.copy_(par["h0"])
        for o in graph_out:
            o.zero_()
        unrelated_eager_work(t)
        graph.replay()
        t.cuda.synchronize()
        assert all(same(a, b) for a, b in zip(graph_out, eager_out)), f"replay {r}: out"
        assert same(state, eager_state), f"replay {r}: final state"
        print(f"[graph] decode replay {r}: bitwise equal to the eager loop", flush=True)


def test_graph_chunked_forward_new_inputs():
    """The chunked kernel (several chunks, a ragged tail) captured once; before each replay
    new inputs are copied into the captured buffers."""
    t = torch()
    w = WORKLOADS["layer"].with_(batch=2, dim=256, seqlen=1000, initial_state=True, seed=502)
    announce(f"{w.describe()} graph chunked forward")
    keys_io = ("u", "delta", "B", "C", "z")
    keys_f = ("A", "D", "delta_bias", "h0")
    sets = [make_inputs(w.with_(seed=502 + i)) for i in range(REPLAYS)]
    stat = {k: dev(sets[0][k], w.io) for k in keys_io}
    stat.update({k: dev(sets[0][k], "f32") for k in keys_f})
    out = t.empty_like(stat["u"])
    fin = t.empty_like(stat["h0"])

    def call(o, f):
        ssm.scan(stat["u"], stat["delta"], stat["A"], stat["B"], stat["C"], D=stat["D"],
                 z=stat["z"], delta_bias=stat["delta_bias"], delta_softplus=True,
                 h0=stat["h0"], out=o, final_state=f)

    call(out, fin)                                   # warm-up outside the capture
    t.cuda.synchronize()
    graph = t.cuda.CUDAGraph()
    with t.cuda.graph(graph):
        call(out, fin)
    for r, inp in enumerate(sets):
        for k in keys_io:
            stat[k].copy_(dev(inp[k], w.io))
        for k in keys_f:
            stat[k].copy_(dev(inp[k], "f32"))
        e_out, e_fin = t.empty_like(out), t.empty_like(fin)
        call(e_out, e_fin)
        t.cuda.synchronize()
        out.zero_()
        fin.zero_()
        unrelated_eager_work(t)
        graph.replay()
        t.cuda.synchronize()
        assert same(out, e_out) and same(fin, e_fin), f"replay {r} differs from eager"
        if r == 0:
            ref = oracle.scan_ref(widen(inp["u"], w.io), widen(inp["delta"], w.io), inp["A"],
                                  widen(inp["B"], w.io), widen(inp["C"], w.io), inp["D"],
                                  widen(inp["z"], w.io), inp["delta_bias"], True, inp["h0"])
            check(w.io, (host(out), host(fin)), ref, f"{w.describe()} graph replay")
        print(f"[graph] chunked replay {r}: bitwise equal to eager", flush=True)


def test_graph_ssd_forward():
    """The SSD kernels (step factors, block products, then the per-head pass) captured
    with a workspace held by the caller."""
    t = torch()
    w = SSD_WORKLOADS["ssd_tiny"].with_(batch=2, nheads=4, headdim=64, dstate=128,
                                        seqlen=700, initial_state=True, seed=503)
    announce(f"{w.describe()} graph ssd")
    inp = make_ssd_inputs(w)
    g = {k: dev(inp[k], "bf16") for k in ("x", "dt", "B", "C", "z")}
    f = {k: dev(inp[k], "f32") for k in ("A", "D", "dt_bias", "h0")}
    ws = t.empty(ssm.ssm_ssd_workspace_bytes(w.batch, w.nheads, w.dstate, w.seqlen),
                 dtype=t.uint8, device="cuda")
    out = t.empty_like(g["x"])
    fin = t.empty_like(f["h0"])

    def call(o, fs):
        ssm.ssd(g["x"], g["dt"], f["A"], g["B"], g["C"], D=f["D"], z=g["z"],
                dt_bias=f["dt_bias"], dt_softplus=True, h0=f["h0"], out=o, final_state=fs,
                workspace=ws)

    e_out, e_fin = t.empty_like(out), t.empty_like(fin)
    call(e_out, e_fin)
    t.cuda.synchronize()
    w_ = lambda k: widen(inp[k], "bf16")
    ref = oracle.ssd_ref(w_("x"), w_("dt"), inp["A"], w_("B"), w_("C"), inp["D"], w_("z"),
                         inp["dt_bias"], True, inp["h0"])
    check("bf16", (host(e_out), host(e_fin)), ref, f"{w.describe()} eager")
    graph = t.cuda.CUDAGraph()
    with t.cuda.graph(graph):
        call(out, fin)
    for r in range(REPLAYS):
        out.zero_()
        fin.zero_()
        ws.zero_()
        unrelated_eager_work(t)
        graph.replay()
        t.cuda.synchronize()
        assert same(out, e_out) and same(fin, e_fin), f"replay {r} differs from eager"
        print(f"[graph] ssd replay {r}: bitwise equal to eager", flush=True)


def test_graph_training_step():
    """ssm_scan_fwd_ckpt then ssm_scan_bwd (workspace path) captured as one graph: every
    replay's outputs, saved states and gradients equal the eager step's bit for bit."""
    t = torch()
    w = WORKLOADS["layer"].with_(batch=2, dim=96, seqlen=1300, initial_state=True, seed=504)
    announce(f"{w.describe()} graph training step")
    inp = make_inputs(w)
    g = {k: dev(inp[k], w.io) for k in ("u", "delta", "B", "C", "z")}
    f = {k: dev(inp[k], "f32") for k in ("A", "D", "delta_bias", "h0")}
    gen = t.Generator(device="cuda")
    gen.manual_seed(505)
    dout = t.randn(g["u"].shape, device="cuda", generator=gen).to(g["u"].dtype)
    dfinal = t.randn((w.batch, w.dim, w.dstate), device="cuda", generator=gen)
    flags = ssm.SSM_IO_BF16 | ssm.SSM_DELTA_SOFTPLUS
    ws = t.empty(ssm.ssm_scan_bwd_workspace_bytes(w.batch, w.dim, w.dstate, w.seqlen, flags),
                 dtype=t.uint8, device="cuda")

    def step():
        out, fin, states = ssm.scan_train(g["u"], g["delta"], f["A"], g["B"], g["C"], D=f["D"],
                                          z=g["z"], delta_bias=f["delta_bias"],
                                          delta_softplus=True, h0=f["h0"])
        grads = ssm.scan_backward(g["u"], g["delta"], f["A"], g["B"], g["C"], states, dout,
                                  D=f["D"], z=g["z"], delta_bias=f["delta_bias"],
                                  delta_softplus=True, dfinal=dfinal, workspace=ws)
        return {"out": out, "fin": fin, "states": states, **grads}

    eager = {k: v.clone() for k, v in step().items() if v is not None}
    t.cuda.synchronize()
    ref = oracle.scan_ref(widen(inp["u"], w.io), widen(inp["delta"], w.io), inp["A"],
                          widen(inp["B"], w.io), widen(inp["C"], w.io), inp["D"],
                          widen(inp["z"], w.io), inp["delta_bias"], True, inp["h0"])
    check(w.io, (host(eager["out"]), host(eager["fin"])), ref, f"{w.describe()} eager step")
    graph = t.cuda.CUDAGraph()
    with t.cuda.graph(graph):
        captured = step()
    for r in range(REPLAYS):
        for v in captured.values():
            if v is not None:
                v.zero_()
        ws.zero_()
        unrelated_eager_work(t)
        graph.replay()
        t.cuda.synchronize()
        for k, v in eager.items():
            assert same(captured[k], v), f"replay {r}: {k} differs from eager"
        print(f"[graph] training step replay {r}: bitwise equal to eager", flush=True)

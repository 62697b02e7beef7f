"""Shared helpers of the GPU tests: move a workload's stored inputs to the device, run
the HIP path through the C ABI, and read results back as float64."""
import sys

import numpy as np

import selective_state_space_fwd_amd as ssm
from ssm_workloads import bf16_bits_to_f32


def torch():
    import torch as _t
    return _t


def announce(msg):
    """Name the case before the GPU step, so a crash can be attributed from the log."""
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev(x, io, device="cuda"):
    t = torch()
    if x is None:
        return None
    if x.dtype == np.uint16:
        return t.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(t.bfloat16)
    return t.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def host(x):
    """Device tensor -> float64 numpy (bf16 widened exactly)."""
    t = torch()
    if x.dtype == t.bfloat16:
        bits = x.view(t.int16).cpu().numpy().view(np.uint16)
        return bf16_bits_to_f32(bits).astype(np.float64)
    return x.detach().cpu().numpy().astype(np.float64)


def run_hip(inputs, softplus=True, use_D=True, use_z=True, use_bias=True, device="cuda",
            waves_per_channel=None):
    """Run the GPU scan on a workload dict (storage form). Returns (out, final) float64.
    waves_per_channel: the launch-shape hint (None: the library chooses)."""
    io = inputs["io"]
    g = {k: dev(inputs[k], io, device) for k in ("u", "delta", "B", "C", "z")}
    f = {k: dev(inputs[k], "f32", device) for k in ("A", "D", "delta_bias", "h0")}
    out, fin = ssm.scan(g["u"], g["delta"], f["A"], g["B"], g["C"],
                        D=f["D"] if use_D else None,
                        z=g["z"] if use_z else None,
                        delta_bias=f["delta_bias"] if use_bias else None,
                        delta_softplus=softplus, h0=f["h0"],
                        waves_per_channel=waves_per_channel)
    torch().cuda.synchronize()
    return host(out), host(fin)

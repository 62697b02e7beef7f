"""The Python binding in a fresh process that touches the library before importing torch.

PyTorch for ROCm ships its own HIP runtime under the same SONAME as the system one. The
binding imports torch before it loads libssmscan.so, so that the library binds to torch's
runtime; loaded first, it would bring in the system runtime and the process would hold two,
the library's seeing no device. This runs one small forward in a subprocess whose first
call into the package is a host-only query, and checks it against the oracle.
"""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys
sys.path.insert(0, {root!r})
import selective_state_space_fwd_amd as ssm
assert "torch" not in sys.modules
n = ssm.ssm_scan_ckpt_count(1000)          # first use of the library: a host-only call
import numpy as np
import oracle
from ssm_workloads import RTOL, RTOL_STATE, WORKLOADS, make_inputs, parity, widen
import torch
w = WORKLOADS["tiny"].with_(batch=2, dim=8, seqlen=300, seed=31)
inp = make_inputs(w)
d = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
out, fin = ssm.scan(d(inp["u"]), d(inp["delta"]), d(inp["A"]), d(inp["B"]), d(inp["C"]),
                    D=d(inp["D"]), delta_bias=d(inp["delta_bias"]), delta_softplus=True)
torch.cuda.synchronize()
ro, rf = oracle.scan_ref(widen(inp["u"], "f32"), widen(inp["delta"], "f32"), inp["A"],
                         widen(inp["B"], "f32"), widen(inp["C"], "f32"), inp["D"], None,
                         inp["delta_bias"], True)
po = parity(out.cpu().numpy(), ro, RTOL["f32"])
pf = parity(fin.cpu().numpy(), rf, RTOL_STATE)
print("n_ckpt", n, "out", po, "final", pf, flush=True)
assert n == 4 and po.ok and pf.ok
print("BINDING-OK", flush=True)
"""


def test_library_loaded_before_torch_still_runs_on_the_gpu():
    r = subprocess.run([sys.executable, "-c", SCRIPT.format(root=ROOT)], capture_output=True,
                       text=True, timeout=240)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0 and "BINDING-OK" in r.stdout

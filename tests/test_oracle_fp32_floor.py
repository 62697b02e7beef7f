"""The rounding floor of a float32 implementation of the scan, per workload.

The float32 instantiation of the oracle (the same sequential loop, float32 arithmetic,
expf and log1pf) is compared with the float64 one on the values the GPU sees. Its error
is what any float32 evaluation of the method carries before reassociation; the parity
tolerance for float32 storage (1e-4) must sit above it, and it does by one to two orders
of magnitude. The pages say floating-point reassociation makes parallel and serial
results differ in their last bits, and that long scans let rounding drift grow
(mhpq.cn/news/1077344, section 4, on numerical stability of the parallel scan).

Whole tensors for the smaller workloads; seeded rows (oracle.sample_rows) of the two
large ones. Run with -s to see the table.
"""
import numpy as np
import pytest

import oracle
from ssm_workloads import RTOL, RTOL_STATE, WORKLOADS, make_inputs, parity, widen

# workload -> rows sampled (None: the whole tensor)
CASES = [("tiny", None), ("long", None), ("layer", None), ("verylong", 12),
         ("widestate", 16), ("decode", None)]


def _floor(name, nrows):
    w = WORKLOADS[name]
    inp = make_inputs(w)
    io = inp["io"]
    if nrows is None:
        args = (widen(inp["u"], io), widen(inp["delta"], io), inp["A"], widen(inp["B"], io),
                widen(inp["C"], io), inp["D"], widen(inp["z"], io), inp["delta_bias"], True,
                inp["h0"])
        o64, f64 = oracle.scan_ref(*args)
        o32, f32 = oracle.scan_ref(*args, precision="f32")
    else:
        rows = oracle.sample_rows(w.batch, w.dim, nrows, seed=w.seed)
        o64, f64 = oracle.scan_rows(inp, rows)
        o32, f32 = oracle.scan_rows(inp, rows, precision="f32")
    return w, parity(o32, o64, RTOL["f32"]), parity(f32, f64, RTOL_STATE)


@pytest.mark.parametrize("name,nrows", CASES)
def test_float32_floor_is_below_the_tolerance(name, nrows):
    w, po, pf = _floor(name, nrows)
    print(f"\nfloat32 floor {w.describe()} ({'all rows' if nrows is None else f'{nrows}+ rows'}): "
          f"out err {po.err:.2e} normwise {po.normwise:.2e}; "
          f"final err {pf.err:.2e} normwise {pf.normwise:.2e}")
    # The floor must leave the float32 tolerance at least a factor of 10 of room.
    assert po.nonfinite_mismatch == 0 and pf.nonfinite_mismatch == 0
    assert po.err <= RTOL["f32"] / 10, po
    assert pf.err <= RTOL_STATE / 10, pf
    # ... and it is not zero: the float32 loop really rounds in float32.
    assert po.err > 1e-9

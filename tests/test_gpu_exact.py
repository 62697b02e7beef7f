"""GPU checks with exact answers, and properties that hold at any size.

  * the pages' prefix-sum example and a 65536-step exact carry: bitwise; the same carry at
    the largest B/C rows the API accepts (2^31 - 128 bytes per batch row);
  * the wave-level combine routine on integer pairs: bitwise, every lane;
  * run-to-run determinism: bitwise;
  * chaining two calls through final_state, delta = 0, zero input, B = 0, empty sizes.
"""
import numpy as np
import pytest

import oracle
import selective_state_space_fwd_amd as ssm
from golden_io import load
from gpu_util import announce, host, run_hip, torch
from ssm_workloads import (RTOL, RTOL_STATE, WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits,
                           make_inputs, parity, widen)

pytestmark = pytest.mark.gpu


def prefix_problem(x, N=16, dim=1, io="f32"):
    """A = 0, delta = 1 (no softplus), B = C = e_0: the scan is a prefix sum of u."""
    L = len(x)
    u = np.tile(np.asarray(x, np.float32), (1, dim, 1))
    Bm = np.zeros((1, N, L), np.float32)
    Bm[0, 0] = 1.0
    st = (lambda a: f32_to_bf16_bits(a)) if io == "bf16" else (lambda a: a)
    return {"io": io, "u": st(u), "delta": st(np.ones((1, dim, L), np.float32)),
            "A": np.zeros((dim, N), np.float32), "B": st(Bm), "C": st(Bm.copy()),
            "D": None, "z": None, "delta_bias": None, "h0": None}


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prefix_sum_example_bitwise(io):
    announce(f"prefix-sum example {io}")
    g = load("prefix_sum.txt")
    out, fin = run_hip(prefix_problem(g["input"], io=io), softplus=False)
    assert out[0, 0].tolist() == g["inclusive_scan"]
    assert fin[0, 0, 0] == g["inclusive_scan"][-1] and not fin[0, 0, 1:].any()


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_long_exact_carry_bitwise(io):
    L = 65536
    announce(f"exact carry L={L} {io}")
    out, fin = run_hip(prefix_problem(np.ones(L), dim=3, io=io), softplus=False)
    expect = np.arange(1, L + 1, dtype=np.float64)
    if io == "bf16":
        expect = bf16_bits_to_f32(f32_to_bf16_bits(expect.astype(np.float32))).astype(np.float64)
    for d in range(3):
        assert np.array_equal(out[0, d], expect)
    assert np.all(fin[0, :, 0] == L)


@pytest.mark.slow
def test_exact_carry_at_the_offset_limit():
    """The largest B/C rows the API accepts: 64 states x (2^24 - 1) steps of bf16 per batch
    row is 2^31 - 128 bytes, the top of the 32-bit offsets inside a row. u = 1, A = 0,
    delta = 1 and B = C = e_0 make every output the exact step count t + 1 (below 2^24,
    so exact in float32; bf16 out is its round-to-nearest-even), in both batch rows."""
    t = torch()
    L, N, batch, dim = (1 << 24) - 1, 64, 2, 2
    announce(f"exact carry at the offset limit: b{batch} d{dim} N{N} L{L} bf16")
    u = t.ones((batch, dim, L), dtype=t.bfloat16, device="cuda")
    delta = t.ones_like(u)
    Bm = t.zeros((batch, N, L), dtype=t.bfloat16, device="cuda")
    Bm[:, 0] = 1.0
    Cm = Bm.clone()
    A = t.zeros((dim, N), dtype=t.float32, device="cuda")
    out, fin = ssm.scan(u, delta, A, Bm, Cm)
    t.cuda.synchronize()
    idx = t.arange(1, L + 1, device="cuda", dtype=t.float32)
    expect = idx.to(t.bfloat16)          # round-to-nearest-even of the exact t + 1
    for b in range(batch):
        for d in range(dim):
            assert t.equal(out[b, d].view(t.int16), expect.view(t.int16)), (b, d)
    assert t.all(fin[:, :, 0] == L) and not t.any(fin[:, :, 1:])


def test_wave_combine_lane_wiring_bitwise():
    t = torch()
    announce("wave combine debug kernel")
    groups = 32
    rng = np.random.default_rng(21)
    # a in {-1, 0, 1} and small integer b: every product and sum is exact in float32
    a = rng.integers(-1, 2, 64 * groups).astype(np.float32)
    b = rng.integers(-8, 9, 64 * groups).astype(np.float32)
    a[::7] = 1.0
    da, db = t.from_numpy(a).cuda(), t.from_numpy(b).cuda()
    ao, bo = t.empty_like(da), t.empty_like(db)
    st = ssm.ssm_scan_debug_wave_combine(da.data_ptr(), db.data_ptr(), ao.data_ptr(),
                                         bo.data_ptr(), groups, t.cuda.current_stream().cuda_stream)
    assert st == ssm.SSM_OK
    t.cuda.synchronize()
    ga, gb = ao.cpu().numpy(), bo.cpu().numpy()
    ea, eb = np.empty_like(a), np.empty_like(b)
    for g in range(groups):
        acc = (1.0, 0.0)
        for i in range(64 * g, 64 * g + 64):
            acc = (a[i] * acc[0], a[i] * acc[1] + b[i])  # (acc) o (a_i, b_i)
            ea[i], eb[i] = acc
    assert np.array_equal(gb, eb), np.nonzero(gb != eb)[0][:10]
    assert np.array_equal(ga, ea), np.nonzero(ga != ea)[0][:10]


def test_run_to_run_bitwise_determinism():
    w = WORKLOADS["layer"].with_(batch=2, dim=64)
    announce(w.describe() + " determinism")
    inp = make_inputs(w)
    o1, f1 = run_hip(inp)
    o2, f2 = run_hip(inp)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


@pytest.mark.parametrize("split", [1024, 777, 1])
def test_chaining_two_calls(split):
    w = WORKLOADS["tiny"].with_(batch=2, dim=16, seqlen=2048, io="bf16", gate=True, seed=31)
    announce(w.describe() + f" chaining at {split}")
    inp = make_inputs(w)
    full_out, full_fin = run_hip(inp)
    first = {k: (v[..., :split] if k in ("u", "delta", "z", "B", "C") else v)
             for k, v in inp.items()}
    second = {k: (v[..., split:] if k in ("u", "delta", "z", "B", "C") else v)
              for k, v in inp.items()}
    o1, f1 = run_hip(first)
    second["h0"] = f1.astype(np.float32)
    o2, f2 = run_hip(second)
    chained = np.concatenate([o1, o2], axis=2)
    assert parity(chained, full_out, RTOL["bf16"]).ok
    assert parity(f2, full_fin, RTOL_STATE).ok


def test_delta_zero_zero_input_and_skip_only():
    w = WORKLOADS["tiny"].with_(batch=2, dim=8, seqlen=300, initial_state=True, seed=32)
    announce(w.describe() + " special cases")
    inp = make_inputs(w)
    # delta = 0 with no bias and no softplus: the state never moves
    z0 = dict(inp, delta=np.zeros_like(inp["delta"]))
    out, fin = run_hip(z0, softplus=False, use_bias=False)
    assert np.array_equal(fin, inp["h0"].astype(np.float64))
    ref_out, _ = oracle.scan_ref(widen(z0["u"], "f32"), np.zeros(z0["u"].shape), z0["A"],
                                 z0["B"], z0["C"], z0["D"], None, None, False, z0["h0"])
    assert parity(out, ref_out, RTOL["f32"]).ok
    # zero input from a zero state: exactly zero everywhere
    zz = dict(inp, u=np.zeros_like(inp["u"]), h0=None)
    out, fin = run_hip(zz)
    assert not out.any() and not fin.any()
    # B = 0 from a zero state: only the skip path, y = D u (bitwise in float32)
    bz = dict(inp, B=np.zeros_like(inp["B"]), h0=None)
    out, fin = run_hip(bz)
    assert np.array_equal(out, (inp["D"][None, :, None] * inp["u"]).astype(np.float64))
    assert not fin.any()


def test_empty_sizes():
    t = torch()
    announce("empty sizes")
    A = t.full((4, 16), -1.0, device="cuda")
    u = t.zeros((2, 4, 0), device="cuda")
    Bm = t.zeros((2, 16, 0), device="cuda")
    out, fin = ssm.scan(u, u, A, Bm, Bm)
    t.cuda.synchronize()
    assert out.shape == (2, 4, 0) and (fin == 0).all()
    h0 = t.randn((2, 4, 16), device="cuda")
    out, fin = ssm.scan(u, u, A, Bm, Bm, h0=h0)
    t.cuda.synchronize()
    assert t.equal(fin, h0)
    u0 = t.zeros((0, 4, 8), device="cuda")
    out, fin = ssm.scan(u0, u0, A, t.zeros((0, 16, 8), device="cuda"),
                        t.zeros((0, 16, 8), device="cuda"))
    t.cuda.synchronize()
    assert out.shape == (0, 4, 8)


def test_invalid_shapes_rejected_before_launch():
    t = torch()
    u = t.zeros((1, 4, 8), device="cuda")
    with pytest.raises(ValueError):
        ssm.scan(u, u, t.zeros((4, 16), device="cuda"), t.zeros((1, 16, 7), device="cuda"),
                 t.zeros((1, 16, 8), device="cuda"))
    with pytest.raises(ssm.SsmScanError):
        ssm.scan(u, u, t.zeros((4, 65), device="cuda"), t.zeros((1, 65, 8), device="cuda"),
                 t.zeros((1, 65, 8), device="cuda"))

"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each expected value comes from a worked
example printed on the pages (tests/golden/), a closed form, a library routine, or an
independent evaluation order (explicit products, a Blelloch tree over the combine).
A dropped term, a wrong sign, an index or operand mix-up in ssm_ref.c fails at least
one of them:
  * y from h_{t-1} instead of h_t ............ prefix sum, chunk example
  * wrong sign or scale inside exp ............ LTI closed form, decay, brute force
  * softplus / bias / gate / D mistakes ....... brute force (library softplus, expit)
  * B or C indexed [b,t,n] instead of [b,n,t] . brute force (N != L, random B and C)
  * row / channel offsets ..................... brute force over batch 2 x dim 3
  * initial state ignored ..................... chunk example, decay, delta = 0
  * combine order reversed .................... combine-vs-recurrence, Blelloch tree
"""
import math

import numpy as np
import pytest
from scipy.special import expit

import oracle
from golden_io import load


def run(u, delta, A, B, C, D=None, z=None, bias=None, softplus=False, h0=None,
        precision="f64"):
    return oracle.scan_ref(u, delta, A, B, C, D, z, bias, softplus, h0, nthreads=2,
                           precision=precision)


def onehot_problem(x, N=16):
    """A = 0 (transition 1), delta = 1, B = C = e_0: the scan reduces to a prefix sum."""
    L = len(x)
    u = np.asarray(x, np.float64).reshape(1, 1, L)
    delta = np.ones((1, 1, L))
    A = np.zeros((1, N))
    B = np.zeros((1, N, L))
    B[0, 0, :] = 1.0
    C = B.copy()
    return u, delta, A, B, C


# ---------------------------------------------------------------- worked examples

@pytest.mark.parametrize("precision", ["f64", "f32"])
def test_prefix_sum_example(precision):
    g = load("prefix_sum.txt")
    out, fin = run(*onehot_problem(g["input"]), precision=precision)
    assert out[0, 0].tolist() == g["inclusive_scan"]
    assert fin[0, 0, 0] == g["inclusive_scan"][-1]
    assert np.all(fin[0, 0, 1:] == 0)


def test_long_exact_carry():
    # u = 1 everywhere: y_t = t + 1, exact in binary floating point up to 2^53.
    L = 65536
    out, fin = run(*onehot_problem(np.ones(L)))
    assert np.array_equal(out[0, 0], np.arange(1, L + 1, dtype=np.float64))
    assert fin[0, 0, 0] == L


def blelloch_inclusive(xs, op, identity, levels=None):
    """Work-efficient tree scan: up-sweep, then down-sweep to the exclusive scan, then
    one more op with each element. len(xs) must be a power of two."""
    x = list(xs)
    n = len(x)
    assert n & (n - 1) == 0
    depth = int(math.log2(n))
    for d in range(depth):
        stride = 2 ** (d + 1)
        for k in range(0, n, stride):
            x[k + stride - 1] = op(x[k + 2 ** d - 1], x[k + stride - 1])
        if levels is not None:
            levels.append(list(x))
    x[n - 1] = identity
    for d in reversed(range(depth)):
        stride = 2 ** (d + 1)
        for k in range(0, n, stride):
            left = x[k + 2 ** d - 1]
            x[k + 2 ** d - 1] = x[k + stride - 1]
            x[k + stride - 1] = op(x[k + stride - 1], left)
    return [op(e, v) for e, v in zip(x, xs)]


def combine(o1, o2):
    """Compose two steps h -> a h + b, first o1 then o2 (the pages' combine)."""
    a1, b1 = o1
    a2, b2 = o2
    return (a2 * a1, a2 * b1 + b2)


def test_blelloch_upsweep_levels():
    g = load("blelloch_upsweep.txt")
    levels = []
    scan = blelloch_inclusive(g["input"], lambda a, b: a + b, 0.0, levels)
    assert levels[0] == g["level2"]
    assert levels[1] == g["level1"]
    assert levels[2] == g["level0"]
    assert scan == g["inclusive_scan"]


@pytest.mark.parametrize("L", [16, 64])
def test_blelloch_over_combine_matches_recurrence(L):
    rng = np.random.default_rng(11 + L)
    delta = rng.uniform(0.01, 0.5, L)
    a_coef = -rng.uniform(0.5, 4.0)
    Bv = rng.standard_normal(L)
    u = rng.standard_normal(L)
    pairs = [(math.exp(delta[t] * a_coef), delta[t] * Bv[t] * u[t]) for t in range(L)]
    scan = blelloch_inclusive(pairs, combine, (1.0, 0.0))
    out, _ = run(u.reshape(1, 1, L), delta.reshape(1, 1, L), np.array([[a_coef]]),
                 Bv.reshape(1, 1, L), np.ones((1, 1, L)))
    h_tree = np.array([b for _, b in scan])
    np.testing.assert_allclose(out[0, 0], h_tree, rtol=1e-13, atol=1e-15)


def test_split_and_carry_example():
    g = load("split_carry.txt")
    x = g["input"]
    assert list(np.cumsum(x[:2])) == g["left_scan"]
    assert list(np.cumsum(x[2:])) == g["right_scan"]
    assert g["result"] == g["left_scan"] + [v + g["left_scan"][-1] for v in g["right_scan"]]
    out, _ = run(*onehot_problem(x))
    assert out[0, 0].tolist() == g["result"]
    u, delta, A, B, C = onehot_problem(x)
    out1, fin1 = run(u[..., :2], delta[..., :2], A, B[..., :2], C[..., :2])
    out2, _ = run(u[..., 2:], delta[..., 2:], A, B[..., 2:], C[..., 2:], h0=fin1)
    assert out1[0, 0].tolist() == g["left_scan"]
    assert out2[0, 0].tolist() == g["result"][2:]


def test_chunk_example():
    g = load("chunk_example.txt")
    a = np.array(g["a_diag"])
    N = len(a)
    k = int(g["chunk"][0])
    rng = np.random.default_rng(5)
    h0 = rng.standard_normal(N)
    beta = rng.standard_normal(N)
    x = rng.standard_normal(2 * k)
    L = 2 * k
    A = np.log(a).reshape(1, N)                  # exp(1 * log a) = a
    Bm = np.broadcast_to(beta[:, None], (N, L)).reshape(1, N, L).copy()
    args = dict(A=A, C=np.zeros((1, N, k)), h0=h0.reshape(1, 1, N))
    _, h3 = run(x[:k].reshape(1, 1, k), np.ones((1, 1, k)), B=Bm[..., :k], **args)
    a_hat = np.exp(np.log(a))
    expect3 = a_hat ** 3 * h0 + a_hat ** 2 * beta * x[0] + a_hat * beta * x[1] + beta * x[2]
    np.testing.assert_allclose(h3[0, 0], expect3, rtol=1e-14)
    _, h6 = run(x.reshape(1, 1, L), np.ones((1, 1, L)), A, Bm, np.zeros((1, N, L)),
                h0=h0.reshape(1, 1, N))
    expect6 = a_hat ** 3 * expect3 + a_hat ** 2 * beta * x[3] + a_hat * beta * x[4] + beta * x[5]
    np.testing.assert_allclose(h6[0, 0], expect6, rtol=1e-14)


def test_decay_example():
    g = load("decay.txt")
    steps = int(g["steps"][0])
    for a, approx, tol in zip(g["a"], g["approx"], g["printed_abs_tolerance"]):
        L = steps
        _, fin = run(np.zeros((1, 1, L)), np.ones((1, 1, L)), np.array([[math.log(a)]]),
                     np.zeros((1, 1, L)), np.zeros((1, 1, L)), h0=np.ones((1, 1, 1)))
        assert abs(fin[0, 0, 0] - approx) <= tol
        assert fin[0, 0, 0] == pytest.approx(a ** steps, rel=1e-10)


# ---------------------------------------------------------------- algebra of the combine

def test_combine_associative_identity_noncommutative():
    rng = np.random.default_rng(3)
    for _ in range(200):
        # small integers: every product and sum below is exact in float64
        x, y, w = [(float(rng.integers(-9, 10)), float(rng.integers(-9, 10))) for _ in range(3)]
        assert combine(combine(x, y), w) == combine(x, combine(y, w))
        assert combine((1.0, 0.0), x) == x and combine(x, (1.0, 0.0)) == x
    assert combine((2.0, 3.0), (5.0, 7.0)) != combine((5.0, 7.0), (2.0, 3.0))


def test_combine_matches_two_and_three_steps():
    rng = np.random.default_rng(4)
    N = 4
    for trial in range(20):
        L = 3
        delta = rng.uniform(0.01, 1.0, L)
        A = -rng.uniform(0.1, 3.0, N)
        Bm = rng.standard_normal((N, L))
        u = rng.standard_normal(L)
        h0 = rng.standard_normal(N)
        ops = [(np.exp(delta[t] * A), delta[t] * Bm[:, t] * u[t]) for t in range(L)]
        _, fin = run(u.reshape(1, 1, L), delta.reshape(1, 1, L), A.reshape(1, N),
                     Bm.reshape(1, N, L), np.zeros((1, N, L)), h0=h0.reshape(1, 1, N))
        left = combine(combine(ops[0], ops[1]), ops[2])
        right = combine(ops[0], combine(ops[1], ops[2]))
        for a, b in (left, right):
            np.testing.assert_allclose(fin[0, 0], a * h0 + b, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- closed forms

def lti_problem(rng, batch, dim, N, L, dt):
    A = -np.arange(1, N + 1)[None, :] * rng.uniform(0.5, 1.5, (dim, N))
    beta = rng.standard_normal((batch, N))
    gamma = rng.standard_normal((batch, N))
    Bm = np.repeat(beta[:, :, None], L, axis=2)
    Cm = np.repeat(gamma[:, :, None], L, axis=2)
    Dv = rng.standard_normal(dim)
    delta = np.full((batch, dim, L), dt)
    return A, beta, gamma, Bm, Cm, Dv, delta


def test_lti_convolution_form():
    """Constant delta, B, C: y_k = D u_k + sum_i K_i u_{k-i}, K_i = sum_n C_n Abar_n^i dt B_n
    (ybb.press, 'Mamba state-space model ... CUDA kernel optimisation', section 1.3)."""
    rng = np.random.default_rng(6)
    batch, dim, N, L, dt = 2, 3, 8, 300, 0.05
    A, beta, gamma, Bm, Cm, Dv, delta = lti_problem(rng, batch, dim, N, L, dt)
    u = rng.standard_normal((batch, dim, L))
    out, _ = run(u, delta, A, Bm, Cm, Dv)
    for b in range(batch):
        for d in range(dim):
            abar = np.exp(dt * A[d])
            powers = abar[None, :] ** np.arange(L)[:, None]           # [L, N]
            K = powers @ (gamma[b] * dt * beta[b])                    # [L]
            y = np.convolve(u[b, d], K)[:L] + Dv[d] * u[b, d]
            rms = np.sqrt(np.mean(y ** 2))
            assert np.max(np.abs(out[b, d] - y) / (np.abs(y) + rms)) < 1e-12


def test_lti_impulse_and_step():
    rng = np.random.default_rng(7)
    batch, dim, N, L, dt = 1, 2, 6, 200, 0.1
    A, beta, gamma, Bm, Cm, Dv, delta = lti_problem(rng, batch, dim, N, L, dt)
    impulse = np.zeros((batch, dim, L))
    impulse[..., 0] = 1.0
    out, _ = run(impulse, delta, A, Bm, Cm)
    step = np.ones((batch, dim, L))
    _, fin = run(step, delta, A, Bm, Cm)
    for d in range(dim):
        abar = np.exp(dt * A[d])
        k = np.arange(L)[:, None]
        np.testing.assert_allclose(out[0, d], (abar ** k) @ (gamma[0] * dt * beta[0]),
                                   rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(fin[0, d], dt * beta[0] * (1 - abar ** L) / (1 - abar),
                                   rtol=1e-12)


# ---------------------------------------------------------------- brute force

def brute_force(u, delta, A, Bm, Cm, Dv, z, bias, h0):
    """Unrolled expansion h_t = (prod_{r<=t} dA_r) h0 + sum_{s<=t} (prod_{s<r<=t} dA_r) dBu_s
    (mhpq.cn/news/1057127 section 3; jsqmd.com section 3.1), softplus via logaddexp and
    the gate via expit, evaluated with explicit products."""
    batch, dim, L = u.shape
    N = A.shape[1]
    out = np.zeros_like(u)
    fin = np.zeros((batch, dim, N))
    for b in range(batch):
        for d in range(dim):
            dt = np.logaddexp(0.0, delta[b, d] + (bias[d] if bias is not None else 0.0))
            dA = np.exp(dt[:, None] * A[d][None, :])                   # [L, N]
            dBu = dt[:, None] * Bm[b].T * u[b, d][:, None]             # [L, N]
            for t in range(L):
                h = np.prod(dA[: t + 1], axis=0) * h0[b, d]
                for s in range(t + 1):
                    h = h + np.prod(dA[s + 1: t + 1], axis=0) * dBu[s]
                y = np.dot(Cm[b, :, t], h) + (Dv[d] * u[b, d, t] if Dv is not None else 0.0)
                out[b, d, t] = y if z is None else y * z[b, d, t] * expit(z[b, d, t])
            fin[b, d] = h
    return out, fin


def test_brute_force_small():
    rng = np.random.default_rng(8)
    batch, dim, N, L = 2, 3, 5, 7
    u = rng.standard_normal((batch, dim, L))
    delta = 0.5 * rng.standard_normal((batch, dim, L))
    bias = np.log(np.expm1(rng.uniform(1e-3, 1e-1, dim)))
    A = -rng.uniform(0.5, 8.0, (dim, N))
    Bm = rng.standard_normal((batch, N, L))
    Cm = rng.standard_normal((batch, N, L))
    Dv = rng.standard_normal(dim)
    z = rng.standard_normal((batch, dim, L))
    h0 = rng.standard_normal((batch, dim, N))
    out, fin = run(u, delta, A, Bm, Cm, Dv, z, bias, True, h0)
    ob, fb = brute_force(u, delta, A, Bm, Cm, Dv, z, bias, h0)
    np.testing.assert_allclose(out, ob, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fin, fb, rtol=1e-12, atol=1e-14)


def test_softplus_threshold_branch():
    # Above 20 the oracle returns x itself; the true softplus differs by log1p(e^-x) < 3e-9.
    L, N = 3, 2
    delta = np.array([[[19.5, 20.5, 40.0]]])
    rng = np.random.default_rng(9)
    u, Bm, Cm = rng.standard_normal((1, 1, L)), rng.standard_normal((1, N, L)), rng.standard_normal((1, N, L))
    A = -np.array([[0.01, 0.02]])
    out, _ = run(u, delta, A, Bm, Cm, softplus=True)
    ob, _ = brute_force(u, delta, A, Bm, Cm, None, None, None, np.zeros((1, 1, N)))
    np.testing.assert_allclose(out, ob, rtol=1e-8)


# ---------------------------------------------------------------- special cases & properties

def test_delta_zero_keeps_state():
    rng = np.random.default_rng(10)
    batch, dim, N, L = 2, 2, 4, 9
    u = rng.standard_normal((batch, dim, L))
    Cm = rng.standard_normal((batch, N, L))
    Dv = rng.standard_normal(dim)
    h0 = rng.standard_normal((batch, dim, N))
    out, fin = run(u, np.zeros((batch, dim, L)), -rng.uniform(1, 2, (dim, N)),
                   rng.standard_normal((batch, N, L)), Cm, Dv, h0=h0)
    assert np.array_equal(fin, h0)
    expect = np.einsum("bnl,bdn->bdl", Cm, h0) + Dv[None, :, None] * u
    np.testing.assert_allclose(out, expect, rtol=1e-14, atol=1e-15)


def test_decode_single_step():
    rng = np.random.default_rng(12)
    batch, dim, N = 2, 3, 8
    u = rng.standard_normal((batch, dim, 1))
    delta = rng.standard_normal((batch, dim, 1))
    bias = rng.uniform(-3, 0, dim)
    A = -rng.uniform(0.5, 8.0, (dim, N))
    Bm, Cm = rng.standard_normal((batch, N, 1)), rng.standard_normal((batch, N, 1))
    Dv, z = rng.standard_normal(dim), rng.standard_normal((batch, dim, 1))
    h0 = rng.standard_normal((batch, dim, N))
    out, fin = run(u, delta, A, Bm, Cm, Dv, z, bias, True, h0)
    dt = np.logaddexp(0.0, delta[..., 0] + bias[None, :])                     # [b, d]
    h1 = np.exp(dt[..., None] * A[None]) * h0 + dt[..., None] * Bm[:, None, :, 0] * u
    y = np.einsum("bdn,bn->bd", h1, Cm[..., 0]) + Dv[None] * u[..., 0]
    np.testing.assert_allclose(fin, h1, rtol=1e-14)
    np.testing.assert_allclose(out[..., 0], y * z[..., 0] * expit(z[..., 0]), rtol=1e-13)


@pytest.mark.parametrize("split", [100, 77, 1, 199])
def test_chaining_is_bitwise(split):
    rng = np.random.default_rng(13)
    batch, dim, N, L = 2, 3, 6, 200
    u = rng.standard_normal((batch, dim, L))
    delta = 0.5 * rng.standard_normal((batch, dim, L))
    bias = rng.uniform(-5, -1, dim)
    A = -rng.uniform(0.5, 8.0, (dim, N))
    Bm, Cm = rng.standard_normal((batch, N, L)), rng.standard_normal((batch, N, L))
    Dv, z = rng.standard_normal(dim), rng.standard_normal((batch, dim, L))
    full, fin = run(u, delta, A, Bm, Cm, Dv, z, bias, True)
    s = split
    o1, f1 = run(u[..., :s], delta[..., :s], A, Bm[..., :s], Cm[..., :s], Dv, z[..., :s], bias, True)
    o2, f2 = run(u[..., s:], delta[..., s:], A, Bm[..., s:], Cm[..., s:], Dv, z[..., s:], bias,
                 True, h0=f1)
    assert np.array_equal(np.concatenate([o1, o2], axis=2), full)
    assert np.array_equal(f2, fin)


def test_linearity_zero_and_skip_only():
    rng = np.random.default_rng(14)
    batch, dim, N, L = 2, 3, 5, 50
    delta = 0.5 * rng.standard_normal((batch, dim, L))
    bias = rng.uniform(-5, -1, dim)
    A = -rng.uniform(0.5, 8.0, (dim, N))
    Bm, Cm = rng.standard_normal((batch, N, L)), rng.standard_normal((batch, N, L))
    Dv = rng.standard_normal(dim)
    u1, u2 = rng.standard_normal((2, batch, dim, L))
    al, be = 0.75, -1.25
    y1, _ = run(u1, delta, A, Bm, Cm, Dv, None, bias, True)
    y2, _ = run(u2, delta, A, Bm, Cm, Dv, None, bias, True)
    y12, _ = run(al * u1 + be * u2, delta, A, Bm, Cm, Dv, None, bias, True)
    np.testing.assert_allclose(y12, al * y1 + be * y2, rtol=1e-11, atol=1e-13)
    # zero input and zero state give exactly zero
    y0, f0 = run(np.zeros((batch, dim, L)), delta, A, Bm, Cm, Dv, None, bias, True)
    assert not y0.any() and not f0.any()
    # B = 0: only the skip path remains, exactly D * u (and gated: times silu(z))
    yd, fd = run(u1, delta, A, np.zeros_like(Bm), Cm, Dv, None, bias, True)
    assert np.array_equal(yd, Dv[None, :, None] * u1) and not fd.any()
    z = rng.standard_normal((batch, dim, L))
    yg, _ = run(u1, delta, A, np.zeros_like(Bm), Cm, Dv, z, bias, True)
    np.testing.assert_allclose(yg, Dv[None, :, None] * u1 * z * expit(z), rtol=1e-14)


def test_empty_and_degenerate_shapes():
    A = -np.ones((3, 4))
    out, fin = run(np.zeros((2, 3, 0)), np.zeros((2, 3, 0)), A, np.zeros((2, 4, 0)),
                   np.zeros((2, 4, 0)), h0=np.full((2, 3, 4), 2.5))
    assert out.shape == (2, 3, 0) and np.all(fin == 2.5)
    out, fin = run(np.zeros((0, 3, 5)), np.zeros((0, 3, 5)), A, np.zeros((0, 4, 5)),
                   np.zeros((0, 4, 5)))
    assert out.shape == (0, 3, 5) and fin.shape == (0, 3, 4)


# ---------------------------------------------------------------- padding mask
# mhpq.cn/news/1057127 section 4: at a padding position (mask 0) the state is inherited from
# the previous step instead of updated; the output there is still C h + D u of that state.

def _masked_case(seed, batch=2, dim=3, N=4, L=40):
    from ssm_workloads import WORKLOADS, make_inputs
    w = WORKLOADS["tiny"].with_(batch=batch, dim=dim, dstate=N, seqlen=L, io="f32", gate=True,
                                initial_state=True, a_kind="scaled", seed=seed)
    inp = make_inputs(w)
    f = lambda x: None if x is None else np.asarray(x, np.float64)
    return {k: f(inp[k]) for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")}


def _run(inp, mask=None):
    return oracle.scan_ref(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                           inp["z"], inp["delta_bias"], True, inp["h0"], mask=mask, nthreads=1)


def test_mask_of_ones_is_no_mask():
    inp = _masked_case(701)
    a = _run(inp)
    b = _run(inp, mask=np.ones((2, 40), np.uint8))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_length_mask_is_the_prefix_scan():
    """mask = (t < len_b): outputs before len_b and the final state are those of the scan
    of the first len_b steps alone; after len_b the state is frozen and the output is
    C_t h + D u_t (gated) of that frozen state."""
    inp = _masked_case(702)
    lens = [25, 40]
    mask = np.zeros((2, 40), np.uint8)
    for b, n in enumerate(lens):
        mask[b, :n] = 1
    out, fin = _run(inp, mask)
    for b, n in enumerate(lens):
        pre = {k: (v[b:b + 1] if k in ("u", "delta", "z", "B", "C", "h0") else v) for k, v in inp.items()}
        pre = {k: (v[..., :n] if k in ("u", "delta", "z", "B", "C") else v) for k, v in pre.items()}
        o, f = _run(pre)
        assert np.array_equal(out[b, :, :n], o[0]) and np.array_equal(fin[b], f[0])
        for t in range(n, 40):
            y = np.einsum("n,dn->d", inp["C"][b, :, t], fin[b]) + inp["D"] * inp["u"][b, :, t]
            zz = inp["z"][b, :, t]
            y = y * zz / (1 + np.exp(-zz))
            np.testing.assert_allclose(out[b, :, t], y, rtol=1e-13, atol=1e-15)


def test_interior_padding_is_deleting_those_steps():
    inp = _masked_case(703, batch=1)
    rng = np.random.default_rng(704)
    mask = (rng.random((1, 40)) > 0.3).astype(np.uint8)
    out, fin = _run(inp, mask)
    keep = np.nonzero(mask[0])[0]
    comp = {k: (v[..., keep] if k in ("u", "delta", "z", "B", "C") else v) for k, v in inp.items()}
    o, f = _run(comp)
    assert np.array_equal(out[0][:, keep], o[0]) and np.array_equal(fin, f)


# ---------------------------------------------------------------- row sampling (scan_rows)

def _whole(inp, precision):
    from ssm_workloads import widen
    io = inp["io"]
    return oracle.scan_ref(widen(inp["u"], io), widen(inp["delta"], io), inp["A"],
                           widen(inp["B"], io), widen(inp["C"], io), inp["D"],
                           widen(inp["z"], io), inp["delta_bias"], True, inp["h0"],
                           nthreads=2, precision=precision)


@pytest.mark.parametrize("precision", ["f64", "f32"])
@pytest.mark.parametrize("kind", ["f32", "bf16-gated-h0"])
def test_scan_rows_equals_the_whole_scan(kind, precision):
    """The sampled-row oracle behind the full-size parity checks: over every (b, d) of a
    small workload it must return exactly the rows of one whole-tensor scan. A slip in its
    slicing (B or C of the wrong batch row, A or D of the wrong channel, the wrong h0 row,
    a missing bias or gate, bf16 not widened) changes a row and fails here."""
    from ssm_workloads import Workload, make_inputs
    if kind == "f32":
        w = Workload("rows", 2, 5, 3, 70, "f32", seed=11)
    else:
        w = Workload("rows", 3, 4, 17, 90, "bf16", gate=True, a_kind="scaled",
                     bc_scale=0.125, initial_state=True, seed=12)
    inp = make_inputs(w)
    out, fin = _whole(inp, precision)
    rows = [(b, d) for b in range(w.batch) for d in range(w.dim)]
    ro, rf = oracle.scan_rows(inp, rows, delta_softplus=True, precision=precision)
    assert np.array_equal(ro, out.reshape(w.batch * w.dim, w.seqlen).astype(np.float64))
    assert np.array_equal(rf, fin.reshape(w.batch * w.dim, w.dstate).astype(np.float64))
    # rows in a scrambled order come back in that order
    pick = [rows[i] for i in (7, 0, len(rows) - 1, 3)]
    so, sf = oracle.scan_rows(inp, pick, delta_softplus=True, precision=precision)
    for i, (b, d) in enumerate(pick):
        assert np.array_equal(so[i], out[b, d].astype(np.float64))
        assert np.array_equal(sf[i], fin[b, d].astype(np.float64))


def test_sample_rows_covers_the_ends():
    rows = oracle.sample_rows(4, 2048, 64, seed=2)
    assert rows[0] == (0, 0) and rows[-1] == (3, 2047)
    assert len(set(rows)) == len(rows) and rows == sorted(rows)
    assert all(0 <= b < 4 and 0 <= d < 2048 for b, d in rows)


# ---------------------------------------------------------------- the float32 instantiation

def test_f32_instantiation_brute_force_and_decay():
    """ssm_ref_scan_f32 (used only to report the float32 rounding floor) against the
    brute-force expansion and the decay example, where A != 0, so its exp, log1p and
    softplus branch are exercised; float32 rounding bounds the distance."""
    rng = np.random.default_rng(13)
    batch, dim, N, L = 2, 3, 5, 7
    u = rng.standard_normal((batch, dim, L))
    delta = 0.5 * rng.standard_normal((batch, dim, L))
    bias = np.log(np.expm1(rng.uniform(1e-3, 1e-1, dim)))
    A = -rng.uniform(0.5, 8.0, (dim, N))
    Bm = rng.standard_normal((batch, N, L))
    Cm = rng.standard_normal((batch, N, L))
    Dv = rng.standard_normal(dim)
    z = rng.standard_normal((batch, dim, L))
    h0 = rng.standard_normal((batch, dim, N))
    f32 = lambda x: np.asarray(x, np.float32).astype(np.float64)  # the values f32 sees
    args = [f32(x) for x in (u, delta, A, Bm, Cm, Dv, z, bias)]
    out, fin = run(*args, True, f32(h0), precision="f32")
    ob, fb = brute_force(*args[:6], args[6], args[7], f32(h0))
    for g, r in ((out, ob), (fin, fb)):
        scale = np.abs(r) + np.sqrt(np.mean(r ** 2))
        assert np.max(np.abs(g - r) / scale) < 2e-6
    g = load("decay.txt")
    steps = int(g["steps"][0])
    for a, approx, tol in zip(g["a"], g["approx"], g["printed_abs_tolerance"]):
        _, fin = run(np.zeros((1, 1, steps)), np.ones((1, 1, steps)), np.array([[math.log(a)]]),
                     np.zeros((1, 1, steps)), np.zeros((1, 1, steps)), h0=np.ones((1, 1, 1)),
                     precision="f32")
        assert abs(float(fin[0, 0, 0]) - approx) <= tol
        assert float(fin[0, 0, 0]) == pytest.approx(a ** steps, rel=1e-4)

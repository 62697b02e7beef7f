"""Python face of the CPU oracle (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg may
import this package. The GPU library neither links nor calls it, and this package
imports nothing from the GPU package.

``scan_ref`` runs the float64 sequential definition in ``ssm_ref.c`` over whole
tensors; ``scan_rows`` runs it on selected (batch, channel) rows of a large workload,
widening only the slices those rows read. ``scan_bwd_ref`` runs the reverse-mode
derivative of that definition (``ssm_ref_bwd.c``). ``ssd_ref``, ``ssd_dense_ref`` and
``ssd_chunked_ref`` (``ssd.py``) are the Mamba-2 (scalar A per head) forward by its
recurrence, its semiseparable-matrix form and its block decomposition.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile
from typing import Dict, Iterable, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libssmref.so")
_SOURCES = ["ssm_ref.c", "ssm_ref_bwd.c"]
_lib = None


def build() -> str:
    """Compile libssmref.so with gcc (host only, OpenMP over rows, no fast-math)."""
    srcs = [os.path.join(_HERE, s) for s in _SOURCES]
    fd, tmp = tempfile.mkstemp(prefix="libssmref.", suffix=".so.tmp", dir=_HERE)
    os.close(fd)
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, *srcs, "-lm"]
    try:
        subprocess.run(cmd, check=True, cwd=_HERE, capture_output=True, text=True)
    except subprocess.CalledProcessError as e:
        os.unlink(tmp)
        raise RuntimeError(f"oracle build failed:\n{e.stderr}") from e
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    for name, ct in (("ssm_ref_scan_f64", ctypes.c_double), ("ssm_ref_scan_f32", ctypes.c_float)):
        fn = getattr(lib, name)
        p = ctypes.POINTER(ct)
        fn.argtypes = [p, p, p, p, p, p, p, p, ctypes.c_int, p, ctypes.c_void_p, p, p,
                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                       ctypes.c_int]
        fn.restype = ctypes.c_int
    p = ctypes.POINTER(ctypes.c_double)
    fn = lib.ssm_ref_scan_bwd_f64
    fn.argtypes = [p, p, p, p, p, p, p, p, ctypes.c_int, p, ctypes.c_void_p, p, p,
                   p, p, p, p, p, p, p, p, p,
                   ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
    fn.restype = ctypes.c_int
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _mask_arg(mask, batch, seqlen):
    """A [batch, seqlen] padding mask as a contiguous uint8 array (None: no padding)."""
    if mask is None:
        return None, None
    m = np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8)
    if m.shape != (batch, seqlen):
        raise ValueError("oracle: mask shape")
    return m, m.ctypes.data_as(ctypes.c_void_p)


def scan_ref(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
             h0=None, nthreads: Optional[int] = None, precision: str = "f64", mask=None
             ) -> Tuple[np.ndarray, np.ndarray]:
    """Sequential selective scan on the CPU. Arrays are real-valued numpy arrays with
    the shapes given in ssm_ref.h; returns (out [B,D,L], final_state [B,D,N]). mask
    [batch, seqlen] (optional): 0 marks a padding position, where the state is kept."""
    lib = _load()
    dt = np.float64 if precision == "f64" else np.float32
    ct = ctypes.c_double if precision == "f64" else ctypes.c_float
    fn = lib.ssm_ref_scan_f64 if precision == "f64" else lib.ssm_ref_scan_f32

    def arr(x):
        return None if x is None else np.ascontiguousarray(x, dtype=dt)

    u, delta, A, B, C = map(arr, (u, delta, A, B, C))
    D, z, delta_bias, h0 = map(arr, (D, z, delta_bias, h0))
    batch, dim, seqlen = u.shape
    dstate = A.shape[1]
    if delta.shape != u.shape or A.shape != (dim, dstate) or B.shape != (batch, dstate, seqlen) \
            or C.shape != B.shape:
        raise ValueError("oracle: inconsistent shapes")
    if z is not None and z.shape != u.shape:
        raise ValueError("oracle: z shape")
    if h0 is not None and h0.shape != (batch, dim, dstate):
        raise ValueError("oracle: h0 shape")
    out = np.empty((batch, dim, seqlen), dtype=dt)
    fin = np.empty((batch, dim, dstate), dtype=dt)

    def ptr(x):
        return None if x is None else x.ctypes.data_as(ctypes.POINTER(ct))

    m, mp = _mask_arg(mask, batch, seqlen)
    rc = fn(ptr(u), ptr(delta), ptr(A), ptr(B), ptr(C), ptr(D), ptr(z), ptr(delta_bias),
            1 if delta_softplus else 0, ptr(h0), mp, ptr(out), ptr(fin),
            batch, dim, dstate, seqlen, int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle returned {rc}")
    return out, fin


def scan_bwd_ref(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
                 h0=None, dout=None, dfinal=None, nthreads: Optional[int] = None, mask=None
                 ) -> Dict[str, Optional[np.ndarray]]:
    """Gradients of L = sum(dout * out) + sum(dfinal * final_state) with respect to every
    input of ``scan_ref`` (float64). Returns a dict with du, ddelta [B,D,L], dA [D,N],
    dB, dC [B,N,L], dD [D] (None without D), dz [B,D,L] (None without z), dbias [D]
    (None without a bias) and dh0 [B,D,N] (the gradient with respect to the initial
    state, zero or given)."""
    lib = _load()
    f64 = lambda x: None if x is None else np.ascontiguousarray(x, dtype=np.float64)
    u, delta, A, B, C, D, z, delta_bias, h0, dout, dfinal = map(
        f64, (u, delta, A, B, C, D, z, delta_bias, h0, dout, dfinal))
    batch, dim, seqlen = u.shape
    dstate = A.shape[1]
    if delta.shape != u.shape or A.shape != (dim, dstate) or B.shape != (batch, dstate, seqlen) \
            or C.shape != B.shape or dout is None or dout.shape != u.shape:
        raise ValueError("oracle: inconsistent shapes")
    if dfinal is not None and dfinal.shape != (batch, dim, dstate):
        raise ValueError("oracle: dfinal shape")
    g = {"du": np.empty_like(u), "ddelta": np.empty_like(u), "dA": np.empty_like(A),
         "dB": np.empty_like(B), "dC": np.empty_like(C),
         "dD": None if D is None else np.empty_like(D),
         "dz": None if z is None else np.empty_like(z),
         "dbias": None if delta_bias is None else np.empty_like(delta_bias),
         "dh0": np.empty((batch, dim, dstate))}
    ptr = lambda x: None if x is None else x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    m, mp = _mask_arg(mask, batch, seqlen)
    rc = lib.ssm_ref_scan_bwd_f64(
        ptr(u), ptr(delta), ptr(A), ptr(B), ptr(C), ptr(D), ptr(z), ptr(delta_bias),
        1 if delta_softplus else 0, ptr(h0), mp, ptr(dout), ptr(dfinal),
        ptr(g["du"]), ptr(g["ddelta"]), ptr(g["dA"]), ptr(g["dB"]), ptr(g["dC"]),
        ptr(g["dD"]), ptr(g["dz"]), ptr(g["dbias"]), ptr(g["dh0"]),
        batch, dim, dstate, seqlen, int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle backward returned {rc}")
    return g


def _widen(x, io):
    if x is None:
        return None
    if io == "bf16" and x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def scan_rows(inputs: Dict[str, Optional[np.ndarray]], rows: Iterable[Tuple[int, int]],
              delta_softplus: bool = True, nthreads: Optional[int] = None,
              precision: str = "f64") -> Tuple[np.ndarray, np.ndarray]:
    """Oracle outputs for selected (b, d) rows of a workload given in storage form
    (float32 arrays, or bf16 bit patterns when inputs['io'] == 'bf16').
    Returns out_rows [R, L] and final_rows [R, N] in float64. Each row is computed by
    ``scan_ref`` on that row's slices alone (u, delta, z [b, d]; B, C [b]; A, D, bias [d];
    h0 [b, d]), so it equals the same row of a whole-tensor ``scan_ref`` call bit for bit."""
    io = inputs["io"]
    rows = list(rows)
    L = inputs["u"].shape[2]
    N = inputs["A"].shape[1]
    outs = np.empty((len(rows), L))
    fins = np.empty((len(rows), N))
    for i, (b, d) in enumerate(rows):
        sl = lambda name: None if inputs.get(name) is None else inputs[name][b:b + 1, d:d + 1]
        o, f = scan_ref(
            _widen(sl("u"), io), _widen(sl("delta"), io),
            np.asarray(inputs["A"][d:d + 1], np.float64),
            _widen(inputs["B"][b:b + 1], io), _widen(inputs["C"][b:b + 1], io),
            None if inputs.get("D") is None else np.asarray(inputs["D"][d:d + 1], np.float64),
            _widen(sl("z"), io),
            None if inputs.get("delta_bias") is None
            else np.asarray(inputs["delta_bias"][d:d + 1], np.float64),
            delta_softplus,
            None if inputs.get("h0") is None else np.asarray(inputs["h0"][b:b + 1, d:d + 1],
                                                              np.float64),
            nthreads=1, precision=precision,
        )
        outs[i] = o[0, 0]
        fins[i] = f[0, 0]
    return outs, fins


def sample_rows(batch: int, dim: int, count: int, seed: int) -> Sequence[Tuple[int, int]]:
    """A seeded sample of (b, d) rows that always includes the first and the last row."""
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    total = batch * dim
    pick = set(rng.choice(total, size=min(count, total), replace=False).tolist())
    pick.update({0, total - 1})
    return [(r // dim, r % dim) for r in sorted(pick)]


from .ssd import ssd_chunked_ref, ssd_dense_ref, ssd_ref  # noqa: E402  (uses scan_ref)

"""Mamba-2 (SSD) forward oracles, float64 (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg may
use this module. It shares nothing with the GPU library.

What is computed. Mamba-2 keeps Mamba-1's selective recurrence and constrains A to one
scalar per head (ybb.press/ai-applications/14118.html, section 2.2). With nheads heads of
headdim channels each, channel d belongs to head d // headdim, and for batch row b,
step t, state n:

    dt_t   = softplus(dt[b, h, t] + dt_bias[h])      (bias and softplus optional)
    h_t    = exp(dt_t * A[h]) * h_{t-1} + dt_t * B[b, n, t] * x[b, d, t]
    y_t    = sum_n C[b, n, t] * h_t[n] + D[d] * x[b, d, t],   out = y_t * silu(z)

A padding position (mask 0) keeps the state (mhpq.cn/news/1057127 section 4).

Three formulations, each written from a different page passage:

* ``ssd_ref``: the recurrence itself. It is the Mamba-1 scan of ``scan_ref`` with A
  broadcast over the states of a channel and the head's step size broadcast over its
  channels, so the sequential C definition (pinned on its own) does the work.
* ``ssd_dense_ref``: the semiseparable-matrix ("duality") form of mhpq.cn/news/1077344
  section 5.1: y = M x with M[t, s] = (C_t . B_s) exp(a_{s+1} + ... + a_t) dt_s for s <= t,
  a_t = dt_t A. Quadratic in the sequence length; small cases only.
* ``ssd_chunked_ref``: the block decomposition of mhpq.cn/news/1077344 section 5.2: the
  sequence cut into blocks; inside a block the same matrix form, between blocks a scan
  of the block-end states.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from . import scan_ref


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _shapes(x, dt, A, B, C):
    batch, dim, seqlen = x.shape
    nheads = A.shape[0]
    if A.ndim != 1 or dim % max(nheads, 1) != 0:
        raise ValueError("ssd oracle: A must be [nheads] and dim a multiple of nheads")
    headdim = dim // nheads if nheads else 0
    dstate = B.shape[1]
    if dt.shape != (batch, nheads, seqlen) or B.shape != (batch, dstate, seqlen) \
            or C.shape != B.shape:
        raise ValueError("ssd oracle: inconsistent shapes")
    return batch, nheads, headdim, dstate, seqlen


def ssd_ref(x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=False, h0=None,
            mask=None, nthreads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """The SSD forward by its recurrence. x, z: [batch, nheads*headdim, seqlen];
    dt: [batch, nheads, seqlen]; A, dt_bias: [nheads]; B, C: [batch, dstate, seqlen];
    D: [nheads*headdim]; h0: [batch, nheads*headdim, dstate]; mask: [batch, seqlen].
    Returns (out, final_state) in float64."""
    x, dt, A, B, C, D, z, dt_bias, h0 = map(_f64, (x, dt, A, B, C, D, z, dt_bias, h0))
    batch, nheads, headdim, dstate, seqlen = _shapes(x, dt, A, B, C)
    # channel d of head h = d // headdim takes that head's scalar A and step size
    A_full = np.repeat(A, headdim)[:, None] * np.ones((1, dstate))
    delta = np.repeat(dt, headdim, axis=1)
    bias = None if dt_bias is None else np.repeat(dt_bias, headdim)
    return scan_ref(x, delta, A_full, B, C, D, z, bias, dt_softplus, h0, nthreads=nthreads,
                    mask=mask)


def _step_sizes(dt, dt_bias, dt_softplus, mask):
    """dt after bias and softplus, [batch, nheads, seqlen]; zero at padding steps."""
    s = dt if dt_bias is None else dt + dt_bias[None, :, None]
    if dt_softplus:
        s = np.where(s <= 20.0, np.logaddexp(0.0, s), s)
    if mask is not None:
        s = s * (np.asarray(mask)[:, None, :] != 0)
    return s


def _gate(y, z):
    return y if z is None else y * z / (1.0 + np.exp(-z))


def ssd_dense_ref(x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=False, h0=None,
                  mask=None) -> Tuple[np.ndarray, np.ndarray]:
    """The SSD forward as one lower-triangular (semiseparable) matrix per (batch, head)
    applied to the head's channels. Same arguments and result as ``ssd_ref``."""
    x, dt, A, B, C, D, z, dt_bias, h0 = map(_f64, (x, dt, A, B, C, D, z, dt_bias, h0))
    batch, nheads, P, N, L = _shapes(x, dt, A, B, C)
    s = _step_sizes(dt, dt_bias, dt_softplus, mask)
    out = np.zeros_like(x)
    fin = np.zeros((batch, nheads * P, N))
    for b in range(batch):
        G = C[b].T @ B[b]                                     # G[t, s] = C_t . B_s
        for h in range(nheads):
            cum = np.cumsum(s[b, h] * A[h])                   # sum of a_r for r <= t
            seg = cum[:, None] - cum[None, :]                 # sum of a_r for s < r <= t
            decay = np.exp(np.where(np.tril(np.ones((L, L), bool)), seg, -np.inf))
            M = G * decay * s[b, h][None, :]
            ch = slice(h * P, (h + 1) * P)
            y = x[b, ch] @ M.T                                # y[p, t] = sum_s M[t, s] x[p, s]
            # the final state: every input decayed to the last step
            w = np.exp(cum[-1] - cum) * s[b, h] if L else np.zeros(0)
            f = (x[b, ch] * w[None, :]) @ B[b].T              # [P, N]
            if h0 is not None:
                y += (h0[b, ch] @ C[b]) * np.exp(cum)[None, :]
                if L:
                    f += h0[b, ch] * np.exp(cum[-1])
                else:
                    f += h0[b, ch]
            if D is not None:
                y += D[ch, None] * x[b, ch]
            out[b, ch] = y
            fin[b, ch] = f
    return _gate(out, z), fin


def ssd_chunked_ref(x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=False,
                    h0=None, mask=None, chunk: int = 64) -> Tuple[np.ndarray, np.ndarray]:
    """The SSD forward by blocks of ``chunk`` steps: inside a block the matrix form
    (block-diagonal part plus the carried state read through C), between blocks the
    scan H_c = exp(sum of the block's a) H_{c-1} + S_c of the block-end states."""
    x, dt, A, B, C, D, z, dt_bias, h0 = map(_f64, (x, dt, A, B, C, D, z, dt_bias, h0))
    batch, nheads, P, N, L = _shapes(x, dt, A, B, C)
    s = _step_sizes(dt, dt_bias, dt_softplus, mask)
    out = np.zeros_like(x)
    fin = np.zeros((batch, nheads * P, N))
    for b in range(batch):
        for h in range(nheads):
            ch = slice(h * P, (h + 1) * P)
            H = np.zeros((P, N)) if h0 is None else h0[b, ch].copy()
            for c0 in range(0, L, chunk):
                t = slice(c0, min(c0 + chunk, L))
                sc, xc, Bc, Cc = s[b, h, t], x[b, ch, t], B[b, :, t], C[b, :, t]
                cum = np.cumsum(sc * A[h])
                seg = cum[:, None] - cum[None, :]
                Lm = np.exp(np.where(np.tril(np.ones((len(cum),) * 2, bool)), seg, -np.inf))
                y = xc @ ((Cc.T @ Bc) * Lm * sc[None, :]).T   # within the block
                y += (H @ Cc) * np.exp(cum)[None, :]          # the carried state
                S = (xc * (np.exp(cum[-1] - cum) * sc)[None, :]) @ Bc.T
                H = np.exp(cum[-1]) * H + S
                out[b, ch, t] = y
            if D is not None:
                out[b, ch] += D[ch, None] * x[b, ch]
            fin[b, ch] = H
    return _gate(out, z), fin

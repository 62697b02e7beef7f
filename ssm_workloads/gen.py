"""Seeded input generation for the selective-scan forward.

The value distributions follow the pages' description of a Mamba-1 layer scan:
  * input u and a raw step size drawn per (batch, channel, time);
  * a per-channel step-size bias chosen so that softplus(bias) is uniform in
    [1e-3, 1e-1] (the usual Mamba dt initialisation; softplus(log(expm1(dt))) = dt);
  * diagonal A with the S4D-real pattern A[d, n] = -(n + 1), or that pattern scaled per
    (channel, state) by U(0.5, 1.5) for the wide-state workload;
  * input-dependent B and C of shape [batch, dstate, seqlen], shared by all channels;
  * a skip weight D per channel and, for gated workloads, a gate input z.

Draw order (one numpy PCG64 stream per workload, seeded with the workload's seed), each
array drawn in C order of its shape:
  1. u      ~ N(0, 1)             [batch, dim, seqlen]
  2. delta  ~ 0.5 * N(0, 1)       [batch, dim, seqlen]   (raw, before bias and softplus)
  3. dt     ~ U(1e-3, 1e-1)       [dim]  ->  delta_bias = log(expm1(dt))
  4. B      ~ bc_scale * N(0, 1)  [batch, dstate, seqlen]
  5. C      ~ bc_scale * N(0, 1)  [batch, dstate, seqlen]
  6. D      ~ N(0, 1)             [dim]
  7. z      ~ N(0, 1)             [batch, dim, seqlen]   (gated workloads only)
  8. s      ~ U(0.5, 1.5)         [dim, dstate]          (scaled-A workloads only)
  9. h0     ~ N(0, 1)             [batch, dim, dstate]   (workloads that start from a state)

Normal draws are made in float32. For bf16 workloads, u, delta, B, C and z are rounded
once from float32 to bfloat16 with round-to-nearest-even; the stored bits are what both
the GPU path and the oracle read. A, D, delta_bias and h0 are always float32.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    dim: int
    dstate: int
    seqlen: int
    io: str = "f32"            # storage dtype of u, delta, B, C, z, out: "f32" or "bf16"
    gate: bool = False         # z present (out = y * silu(z))
    a_kind: str = "s4d"        # "s4d": A = -(n+1);  "scaled": A = -(n+1) * U(0.5, 1.5)
    bc_scale: float = 1.0      # standard deviation of B and C
    initial_state: bool = False
    seed: int = 0

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def elements(self) -> int:
        return self.batch * self.dim * self.seqlen

    @property
    def tuples(self) -> int:
        return self.batch * self.dim * self.seqlen * self.dstate

    def algorithmic_bytes(self) -> int:
        """Bytes the operation must move: each input read once, each output written once."""
        s = 2 if self.io == "bf16" else 4
        per_elem = s * (2 + (1 if self.gate else 0) + 1)            # u, delta, [z], out
        n = self.batch * self.dim * self.seqlen * per_elem
        n += self.batch * self.dstate * self.seqlen * 2 * s          # B, C
        n += self.dim * self.dstate * 4 + self.dim * 4 * 2           # A, D, delta_bias
        n += self.batch * self.dim * self.dstate * 4                 # final_state written
        if self.initial_state:
            n += self.batch * self.dim * self.dstate * 4             # h0 read
        return n

    def bwd_algorithmic_bytes(self, ckpt_interval: int = 512) -> int:
        """Bytes the backward pass must move: the forward's inputs, dout, the saved states
        and dfinal read once; every gradient written once (dB, dC, dA, dD, dbias, dh0 in
        float32; du, ddelta, dz in the storage type)."""
        s = 2 if self.io == "bf16" else 4
        g = 1 if self.gate else 0
        elems = self.batch * self.dim * self.seqlen
        n = elems * s * ((3 + g) + (2 + g))                          # u, delta, [z], dout; du, ddelta, [dz]
        n += self.batch * self.dstate * self.seqlen * 2 * (s + 4)    # B, C read; dB, dC written
        n += self.dim * self.dstate * 4 * 2 + self.dim * 4 * 4       # A, dA; D, bias, dD, dbias
        n_ckpt = -(-self.seqlen // ckpt_interval)
        n += self.batch * self.dim * self.dstate * 4 * (n_ckpt + 2)  # saved states, dfinal, dh0
        return n

    def describe(self) -> str:
        gate = " gated" if self.gate else ""
        h0 = " from-h0" if self.initial_state else ""
        return (f"{self.name}: b{self.batch} d{self.dim} N{self.dstate} L{self.seqlen} "
                f"{self.io}{gate}{h0}")


# The workloads the pages' problem statement is measured on.  "layer" is the headline:
# a Mamba-1 layer's scan at batch 4, 2048 channels, 16 states, 2048 steps, bf16 I/O.
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, 64, 16, 256, "f32", seed=0),
    "long": Workload("long", 2, 512, 16, 8192, "f32", seed=1),
    "layer": Workload("layer", 4, 2048, 16, 2048, "bf16", gate=True, seed=2),
    "verylong": Workload("verylong", 1, 1536, 16, 65536, "f32", seed=3),
    "widestate": Workload("widestate", 8, 2048, 64, 4096, "bf16", gate=True,
                          a_kind="scaled", bc_scale=0.125, seed=4),
    "decode": Workload("decode", 8, 2048, 64, 1, "bf16", gate=True, a_kind="scaled",
                       bc_scale=0.125, initial_state=True, seed=4),
}


@dataclass(frozen=True)
class SsdWorkload:
    """A Mamba-2 (SSD) forward: nheads heads of headdim channels, one scalar A and one
    step size per head, B and C shared by all heads of a batch row."""
    name: str
    batch: int
    nheads: int
    headdim: int
    dstate: int
    seqlen: int
    io: str = "bf16"
    gate: bool = True
    initial_state: bool = False
    seed: int = 0

    def with_(self, **kw) -> "SsdWorkload":
        return dataclasses.replace(self, **kw)

    @property
    def dim(self) -> int:
        return self.nheads * self.headdim

    def algorithmic_bytes(self) -> int:
        s = 2 if self.io == "bf16" else 4
        n = self.batch * self.dim * self.seqlen * s * (2 + (1 if self.gate else 0))  # x, [z], out
        n += self.batch * self.nheads * self.seqlen * s                 # dt
        n += self.batch * self.dstate * self.seqlen * 2 * s             # B, C
        n += self.nheads * 4 * 2 + self.dim * 4                         # A, dt_bias, D
        n += self.batch * self.dim * self.dstate * 4                    # final_state written
        if self.initial_state:
            n += self.batch * self.dim * self.dstate * 4                # h0 read
        return n

    def describe(self) -> str:
        gate = " gated" if self.gate else ""
        h0 = " from-h0" if self.initial_state else ""
        return (f"{self.name}: b{self.batch} h{self.nheads}x{self.headdim} N{self.dstate} "
                f"L{self.seqlen} {self.io}{gate}{h0}")


SSD_WORKLOADS: Dict[str, SsdWorkload] = {
    # A Mamba-2 layer's scan at the layer workload's batch, width and length: 32 heads of
    # 64 channels, 128 states (the larger state the block form makes affordable).
    "ssd": SsdWorkload("ssd", 4, 32, 64, 128, 2048, "bf16", gate=True, seed=5),
    "ssd_tiny": SsdWorkload("ssd_tiny", 1, 2, 64, 64, 256, "bf16", gate=True, seed=6),
}


def make_ssd_inputs(w: SsdWorkload) -> Dict[str, Optional[np.ndarray]]:
    """Draw one SSD workload's inputs (streamed arrays in storage form).

    Draw order (PCG64 seeded with w.seed), each array in C order:
      1. x      ~ N(0, 1)                  [batch, nheads*headdim, seqlen]
      2. dt     ~ 0.5 * N(0, 1)            [batch, nheads, seqlen]   (raw)
      3. dt0    ~ exp(U(log 1e-3, log 1e-1)) [nheads] -> dt_bias = log(expm1(dt0))
      4. A      = -U(1, 16)                [nheads]
      5. B      ~ N(0, 1) / sqrt(dstate)   [batch, dstate, seqlen]
      6. C      ~ N(0, 1) / sqrt(dstate)   [batch, dstate, seqlen]
      7. D      ~ N(0, 1)                  [nheads*headdim]
      8. z      ~ N(0, 1)                  [batch, nheads*headdim, seqlen]  (gated only)
      9. h0     ~ N(0, 1)                  [batch, nheads*headdim, dstate]  (from-h0 only)
    """
    rng = np.random.Generator(np.random.PCG64(w.seed))
    f32 = np.float32
    Bn, H, P, N, L = w.batch, w.nheads, w.headdim, w.dstate, w.seqlen
    x = rng.standard_normal((Bn, H * P, L), dtype=f32)
    dt = rng.standard_normal((Bn, H, L), dtype=f32) * f32(0.5)
    dt0 = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=H))
    dt_bias = np.log(np.expm1(dt0)).astype(f32)
    A = (-rng.uniform(1.0, 16.0, size=H)).astype(f32)
    scale = f32(1.0 / np.sqrt(N))
    Bm = rng.standard_normal((Bn, N, L), dtype=f32) * scale
    Cm = rng.standard_normal((Bn, N, L), dtype=f32) * scale
    Dv = rng.standard_normal(H * P, dtype=f32)
    z = rng.standard_normal((Bn, H * P, L), dtype=f32) if w.gate else None
    h0 = rng.standard_normal((Bn, H * P, N), dtype=f32) if w.initial_state else None
    return {
        "io": w.io,
        "x": _store(x, w.io),
        "dt": _store(dt, w.io),
        "A": A,
        "B": _store(Bm, w.io),
        "C": _store(Cm, w.io),
        "D": Dv,
        "z": _store(z, w.io) if z is not None else None,
        "dt_bias": dt_bias,
        "h0": h0,
    }


def make_mask(batch: int, seqlen: int, kind: str, seed: int) -> np.ndarray:
    """A seeded padding mask [batch, seqlen] uint8 (1 = real step, 0 = padding).

    kind "lengths": a batch of sequences of different lengths padded on the right to
    seqlen (len_b ~ U{1..seqlen}, the last row always full length);
    "left": the same lengths padded on the left; "random": each step padding with
    probability 0.3; "ones" / "zeros": all real / all padding.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    m = np.zeros((batch, seqlen), np.uint8)
    if kind in ("lengths", "left"):
        lens = rng.integers(1, seqlen + 1, size=batch) if seqlen else np.zeros(batch, int)
        if batch:
            lens[-1] = seqlen
        for b, n in enumerate(lens):
            if kind == "lengths":
                m[b, :n] = 1
            else:
                m[b, seqlen - n:] = 1
    elif kind == "random":
        m[...] = rng.random((batch, seqlen)) >= 0.3
    elif kind == "ones":
        m[...] = 1
    elif kind != "zeros":
        raise ValueError(f"unknown mask kind {kind!r}")
    return m


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even; returns the uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
               >> np.uint32(16)).astype(np.uint16)
    nan = (b & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        rounded[nan] = np.uint16(0x7FC0)
    return rounded


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def widen(x: Optional[np.ndarray], io: str) -> Optional[np.ndarray]:
    """Stored values (float32 array or bf16 bits) as float64, exactly."""
    if x is None:
        return None
    if io == "bf16" and x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def _store(x: np.ndarray, io: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if io == "bf16" else np.ascontiguousarray(x, np.float32)


def make_inputs(w: Workload) -> Dict[str, Optional[np.ndarray]]:
    """Draw one workload's inputs. Streamed arrays come back in storage form."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    Bn, Dd, N, L = w.batch, w.dim, w.dstate, w.seqlen
    f32 = np.float32

    u = rng.standard_normal((Bn, Dd, L), dtype=f32)
    delta = rng.standard_normal((Bn, Dd, L), dtype=f32) * f32(0.5)
    dt = rng.uniform(1e-3, 1e-1, size=Dd)
    delta_bias = np.log(np.expm1(dt)).astype(f32)
    Bm = rng.standard_normal((Bn, N, L), dtype=f32)
    Cm = rng.standard_normal((Bn, N, L), dtype=f32)
    if w.bc_scale != 1.0:
        Bm *= f32(w.bc_scale)
        Cm *= f32(w.bc_scale)
    Dv = rng.standard_normal(Dd, dtype=f32)
    z = rng.standard_normal((Bn, Dd, L), dtype=f32) if w.gate else None
    idx = np.arange(1, N + 1, dtype=np.float64)
    if w.a_kind == "s4d":
        A = np.broadcast_to(-idx, (Dd, N)).astype(f32)
    elif w.a_kind == "scaled":
        s = rng.uniform(0.5, 1.5, size=(Dd, N))
        A = (-idx[None, :] * s).astype(f32)
    else:
        raise ValueError(f"unknown a_kind {w.a_kind!r}")
    h0 = rng.standard_normal((Bn, Dd, N), dtype=f32) if w.initial_state else None

    return {
        "io": w.io,
        "u": _store(u, w.io),
        "delta": _store(delta, w.io),
        "A": np.ascontiguousarray(A),
        "B": _store(Bm, w.io),
        "C": _store(Cm, w.io),
        "D": Dv,
        "z": _store(z, w.io) if z is not None else None,
        "delta_bias": delta_bias,
        "h0": h0,
    }

"""Seeded synthetic workloads for the selective-scan forward, and the parity metric.

This package is shared by the tests, the benchmark and the oracle's callers. It holds
no step of the scan itself: it draws inputs, rounds them to the storage dtype, widens
stored values back to float, and measures the distance between two result tensors.

Shapes (all C-contiguous):
    u, delta, z, out : [batch, dim, seqlen]
    B, C             : [batch, dstate, seqlen]   (input-dependent, shared by all channels)
    A                : [dim, dstate]  float32
    D, delta_bias    : [dim]          float32
    h0, final_state  : [batch, dim, dstate] float32
    mask             : [batch, seqlen] uint8 (optional; 0 = padding step)

Mamba-2 (SSD) workloads (``SSD_WORKLOADS``, ``make_ssd_inputs``): x, z, out
[batch, nheads*headdim, seqlen]; dt [batch, nheads, seqlen]; A, dt_bias [nheads] float32;
B, C [batch, dstate, seqlen]; D [nheads*headdim] float32.
"""
from .gen import (
    SSD_WORKLOADS,
    WORKLOADS,
    SsdWorkload,
    Workload,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_inputs,
    make_mask,
    make_ssd_inputs,
    widen,
)
from .compare import RTOL, RTOL_STATE, WATCH, ParityReport, parity

__all__ = [
    "WORKLOADS",
    "Workload",
    "SSD_WORKLOADS",
    "SsdWorkload",
    "make_ssd_inputs",
    "make_inputs",
    "make_mask",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "widen",
    "parity",
    "ParityReport",
    "RTOL",
    "RTOL_STATE",
    "WATCH",
]

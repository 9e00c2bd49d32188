"""Shared helpers for GPU parity tests: oracle references and the error metric.

Output tolerance (floating point): the 2e-3 bound is applied to
  E = max_j max(0, |o_gpu - o_ref| - ulp_bf16(o_ref)/2) / max_j' |o_ref[j']|
per (sequence, head), with o_ref the unrounded fp64 oracle output: the bf16
store of the result alone may cost half an ulp (2^-9 relative), which a plain
relative bound of 2e-3 could not absorb, so only the error beyond that store
is charged, relative to the head's largest output.
"""
from __future__ import annotations

import math

import numpy as np

import mla_inputs as mi
import oracle

E_TOL = 2e-3
LSE_TOL = 1e-3
# lse is an fp32 result computed from fp32 scores, so at large magnitudes (a cache scaled by 300 gives
# |lse| near 1e4) its resolution is relative: the bound adds 64 fp32 ulps of |lse|, which leaves it at
# 1e-3 + 4e-5 for the workloads' |lse| of about 10
LSE_REL = 2.0 ** -18


def lse_bound(ref_l: np.ndarray) -> np.ndarray:
    """Allowed |lse_gpu - lse_ref| per output (ref_l: fp64 oracle lse, -inf for empty sequences)."""
    a = np.where(np.isfinite(ref_l), np.abs(ref_l), 0.0)
    return LSE_TOL + LSE_REL * a


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


def e_metric(o_gpu: np.ndarray, o_ref: np.ndarray) -> np.ndarray:
    """E per leading index (..., 512) -> (...)."""
    excess = np.maximum(0.0, np.abs(o_gpu.astype(np.float64) - o_ref) - bf16_ulp(o_ref) / 2)
    denom = np.max(np.abs(o_ref), axis=-1)
    denom = np.where(denom > 0, denom, 1.0)
    return np.max(excess, axis=-1) / denom


def bf16_tensor_to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def reference(rows_per_seq, q: np.ndarray, bits_c: int, scale: float, heads=None, n_sink=4, n_recent=128):
    """Oracle (out [B, nh, 512], lse [B, nh]) for each sequence's rows (uint16 [N, 576])."""
    outs, lses = [], []
    for b, rows in enumerate(rows_per_seq):
        o, l = oracle.decode_sequence(rows, q[b], scale, bits_c, heads, n_sink, n_recent)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)

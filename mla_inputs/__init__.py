"""Seeded synthetic inputs for the low-bit MLA decode path.

This module only draws random numbers and rounds them to bf16; it holds none
of the method's arithmetic (no quantization, packing, selection or
attention).  Both the CPU oracle and the HIP path consume what it returns.

Workloads follow the shapes the QuantMLA pages describe for MLA models
(content latent d_c = 512, decoupled RoPE key d_r = 64; ai.info summary,
"What This Paper Is About"; onedev.kr review, "What it is") and the value
recipe:

* content latent c ~ N(0, 1) with 8 outlier channels scaled by 20 (the
  channels are drawn once per workload and shared by every token);
* RoPE key k_r = RoPE(theta = 10000, position) applied to N(0, 1) vectors,
  rotating interleaved pairs (2j, 2j+1) by pos * 10000^(-2j/64), in fp64;
* q_c, q_r ~ N(0, 1);
* every value is rounded to float32 (RNE) and then to bf16 (RNE).

Rows are generated in fixed 4096-token chunks, each with its own
``SeedSequence(seed, spawn_key=...)``, so any chunk of any sequence can be
regenerated on its own (the oracle uses this to check samples of full-size
caches).  bf16 tensors are returned as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

D_C = 512
D_R = 64
D = D_C + D_R
CHUNK = 4096
N_OUTLIERS = 8
OUTLIER_GAIN = 20.0
ROPE_THETA = 10000.0

# spawn-key streams (fixed order; never renumber)
_S_OUTLIER, _S_ROWS, _S_Q, _S_PERM, _S_LEN = 1, 2, 3, 4, 5


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> float32 (RNE) -> bf16 (RNE) bit patterns."""
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float64).astype(np.float32))


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def outlier_channels(seed: int) -> np.ndarray:
    """The 8 content channels scaled by 20, drawn once per workload."""
    return np.sort(_rng(seed, _S_OUTLIER).choice(D_C, size=N_OUTLIERS, replace=False)).astype(np.int64)


def _chunk(seed: int, b: int, k: int, outliers: np.ndarray) -> np.ndarray:
    """bf16 rows [CHUNK, 576] for tokens [k*CHUNK, (k+1)*CHUNK) of sequence b."""
    g = _rng(seed, _S_ROWS, b, k)
    c = g.standard_normal((CHUNK, D_C))
    c[:, outliers] *= OUTLIER_GAIN
    kr = g.standard_normal((CHUNK, D_R))
    pos = np.arange(k * CHUNK, (k + 1) * CHUNK, dtype=np.float64)[:, None]
    j = np.arange(D_R // 2, dtype=np.float64)[None, :]
    ang = pos * ROPE_THETA ** (-2.0 * j / D_R)
    cs, sn = np.cos(ang), np.sin(ang)
    x0, x1 = kr[:, 0::2], kr[:, 1::2]
    rot = np.empty_like(kr)
    rot[:, 0::2] = x0 * cs - x1 * sn
    rot[:, 1::2] = x0 * sn + x1 * cs
    out = np.empty((CHUNK, D), dtype=np.uint16)
    out[:, :D_C] = to_bf16(c)
    out[:, D_C:] = to_bf16(rot)
    return out


def rows(seed: int, b: int, n: int, outliers: np.ndarray | None = None, start: int = 0,
         threads: int = 8) -> np.ndarray:
    """bf16 rows [n, 576] (c || k_r) of tokens [start, start+n) of sequence b."""
    if outliers is None:
        outliers = outlier_channels(seed)
    out = np.empty((n, D), dtype=np.uint16)
    if n == 0:
        return out
    k0, k1 = start // CHUNK, (start + n - 1) // CHUNK

    def work(k):
        ch = _chunk(seed, b, k, outliers)
        lo, hi = max(start, k * CHUNK), min(start + n, (k + 1) * CHUNK)
        out[lo - start:hi - start] = ch[lo - k * CHUNK:hi - k * CHUNK]

    ks = range(k0, k1 + 1)
    if threads > 1 and k1 > k0:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(work, ks))
    else:
        for k in ks:
            work(k)
    return out


def queries(seed: int, batch: int, heads: int) -> np.ndarray:
    """bf16 q_c || q_r [batch, heads, 576], N(0, 1)."""
    return to_bf16(_rng(seed, _S_Q).standard_normal((batch, heads, D)))


def page_permutation(seed: int, num_pages: int) -> np.ndarray:
    """Shuffled physical page order."""
    return _rng(seed, _S_PERM).permutation(num_pages).astype(np.int32)


def loguniform_lengths(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """Context lengths floor(exp(U(ln lo, ln hi)))."""
    u = _rng(seed, _S_LEN).uniform(math.log(lo), math.log(hi), size=batch)
    return np.minimum(np.floor(np.exp(u)).astype(np.int64), hi).astype(np.int32)


@dataclass
class Workload:
    name: str
    seed: int
    batch: int
    heads: int
    bits_c: int
    seq_lens: np.ndarray
    page_tokens: int = 64
    n_sink: int = 4
    n_recent: int = 128
    scale: float = field(default_factory=lambda: float(np.float32(1.0 / math.sqrt(192.0))))
    steps_append: int = 0  # tokens appended per sequence per timed step (mixed serving batch)

    @property
    def total_tokens(self) -> int:
        return int(np.sum(self.seq_lens, dtype=np.int64))

    def pages_per_seq(self) -> np.ndarray:
        return (self.seq_lens.astype(np.int64) + self.page_tokens - 1) // self.page_tokens


def workload(name: str) -> Workload:
    """Named synthetic workloads (shapes of the pages' MLA models)."""
    if name == "tiny_c4r4":            # B1, H16, 1K
        return Workload(name, 1, 1, 16, 4, np.array([1024], np.int32))
    if name == "dsv2lite_c4r4_32k":    # B32, H16, 32K
        return Workload(name, 2, 32, 16, 4, np.full(32, 32768, np.int32))
    if name == "dsv2lite_c4r4_128k":   # B8, H16, 128K (few-head point at 128K)
        return Workload(name, 6, 8, 16, 4, np.full(8, 131072, np.int32))
    if name == "dsv3_c4r4_128k":       # B8, H128, 128K
        return Workload(name, 3, 8, 128, 4, np.full(8, 131072, np.int32))
    if name == "dsv3_c2r4_128k":       # C2R4 of the above
        return Workload(name, 4, 8, 128, 2, np.full(8, 131072, np.int32))
    if name == "mixed_c4r4_serving":   # B64, H128, log-uniform 1K..128K, 1 token appended per step
        return Workload(name, 5, 64, 128, 4, loguniform_lengths(5, 64, 1024, 131072), steps_append=1)
    raise KeyError(name)


WORKLOADS = ["tiny_c4r4", "dsv2lite_c4r4_32k", "dsv2lite_c4r4_128k", "dsv3_c4r4_128k",
             "dsv3_c2r4_128k", "mixed_c4r4_serving"]

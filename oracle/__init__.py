"""CPU oracle for the low-bit MLA decode path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  It shares no code with the
HIP library (``bit_mla_kv_amd``) and never imports it; both sides only share
the seeded input generator in ``mla_inputs``.

The arithmetic lives in ``mla_oracle.c`` (plain C, fp32 quantizer, fp64
attention, OpenMP); this module builds it with gcc, loads it with ctypes and
adds the placement of packed tokens into the paged cache layout:

* page = [content codes: page_tokens rows x (512*bits_c/8) B]
         [RoPE-key codes: page_tokens rows x 32 B]
         [metadata: page_tokens rows x 9 dwords (bf16 s | bf16 z << 16)]
* token t of a slot lives in page ``block_table[slot][t // page_tokens]``,
  row ``t % page_tokens``;
* ``sink[slot][i]`` holds row i for i < min(n_sink, N);
* ``recent[slot][p % n_recent]`` holds row p for p in [max(0, N - n_recent), N).

Readings of the pages that this follows are listed in the C file's header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB = os.path.join(_BUILD, "libmla_oracle.so")

D_C, D_R, G = 512, 64, 64
D = D_C + D_R
N_GROUPS = 9
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (always, when force)."""
    os.makedirs(_BUILD, exist_ok=True)
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        L.mlo_quantize_tokens.argtypes = [P, ctypes.c_int64, ctypes.c_int, P, P, P]
        L.mlo_select.argtypes = [P, P, P, P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, P]
        L.mlo_attend.argtypes = [P, ctypes.c_int64, P, P, ctypes.c_int, ctypes.c_double, P, P]
        L.mlo_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(lib().mlo_num_threads())


def quantize(rows: np.ndarray, bits_c: int):
    """Per-token quantize + pack.  rows: uint16 [n, 576] (bf16 bits).

    Returns (codes_c uint8 [n, 512*bits_c/8], codes_r uint8 [n, 32],
    meta uint32 [n, 9])."""
    rows = np.ascontiguousarray(rows, dtype=np.uint16)
    n = rows.shape[0]
    cc = np.empty((n, D_C * bits_c // 8), np.uint8)
    cr = np.empty((n, D_R // 2), np.uint8)
    meta = np.empty((n, N_GROUPS), np.uint32)
    lib().mlo_quantize_tokens(_p(rows), n, bits_c, _p(cc), _p(cr), _p(meta))
    return cc, cr, meta


def select(rows, codes_c, codes_r, meta, bits_c: int, n_sink: int = 4, n_recent: int = 128) -> np.ndarray:
    """fp64 [N, 576]: the one representation each token enters attention with."""
    rows = np.ascontiguousarray(rows, dtype=np.uint16)
    n = rows.shape[0]
    out = np.empty((n, D), np.float64)
    lib().mlo_select(_p(rows), _p(np.ascontiguousarray(codes_c)), _p(np.ascontiguousarray(codes_r)),
                     _p(np.ascontiguousarray(meta)), n, bits_c, n_sink, n_recent, _p(out))
    return out


def attend(sel: np.ndarray, q: np.ndarray, scale: float, heads=None):
    """Exact attention (fp64).  q: uint16 [H, 576].  Returns (out [nh, 512], lse [nh])."""
    sel = np.ascontiguousarray(sel, dtype=np.float64)
    q = np.ascontiguousarray(q, dtype=np.uint16)
    if heads is None:
        heads = np.arange(q.shape[0])
    heads = np.ascontiguousarray(heads, dtype=np.int32)
    out = np.empty((len(heads), D_C), np.float64)
    lse = np.empty(len(heads), np.float64)
    lib().mlo_attend(_p(sel), sel.shape[0], _p(q), _p(heads), len(heads), float(scale), _p(out), _p(lse))
    return out, lse


def decode_sequence(rows, q, scale, bits_c, heads=None, n_sink=4, n_recent=128):
    """Quantize -> select -> attend for one sequence.  rows: [N, 576] bf16 bits."""
    cc, cr, meta = quantize(rows, bits_c)
    sel = select(rows, cc, cr, meta, bits_c, n_sink, n_recent)
    return attend(sel, q, scale, heads)


# ---------------------------------------------------------------- layout
def page_bytes(bits_c: int, page_tokens: int = 64) -> int:
    return page_tokens * (D_C * bits_c // 8 + D_R // 2 + 4 * N_GROUPS)


def place_pages(pages: np.ndarray, block_table_row: np.ndarray, codes_c, codes_r, meta, bits_c: int,
                page_tokens: int = 64) -> None:
    """Write the packed copies of tokens [0, N) of one slot into its pages."""
    n = codes_c.shape[0]
    cb = D_C * bits_c // 8
    off_r = page_tokens * cb
    off_m = off_r + page_tokens * (D_R // 2)
    for p0 in range(0, n, page_tokens):
        k = min(page_tokens, n - p0)
        pg = pages[int(block_table_row[p0 // page_tokens])]
        pg[0:k * cb] = codes_c[p0:p0 + k].reshape(-1)
        pg[off_r:off_r + k * (D_R // 2)] = codes_r[p0:p0 + k].reshape(-1)
        pg[off_m:off_m + k * 4 * N_GROUPS] = meta[p0:p0 + k].reshape(-1).view(np.uint8)


def bf16_buffers(rows: np.ndarray, n_sink: int = 4, n_recent: int = 128):
    """Expected sink rows {i: row} and ring rows {p % n_recent: row} for one slot."""
    n = rows.shape[0]
    sink = {i: rows[i] for i in range(min(n_sink, n))}
    ring = {p % n_recent: rows[p] for p in range(max(0, n - n_recent), n)}
    return sink, ring


def timed(fn, *a, **k):
    t = time.perf_counter()
    r = fn(*a, **k)
    return r, time.perf_counter() - t

"""Python binding of the MI355X low-bit MLA KV-cache library (libmla_lowbit.so).

Argument marshalling only: every step of the hot path runs in the HIP
kernels behind the C ABI in ``include/mla_lowbit.h``.  PyTorch provides
device memory and streams.  Importing this package raises if the built
library is missing; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_lowbit.so")

ABI_VERSION = 1
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_DEVICE = range(5)
D_C, D_R = 512, 64
D = D_C + D_R


class MlaLowbitError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


class Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("abi_version", "d_c", "d_r", "bits_c", "bits_r", "group", "page_tokens", "n_sink", "n_recent")]


class CacheDesc(ctypes.Structure):
    _fields_ = [("layout", Layout), ("pages", ctypes.c_void_p), ("num_pages", ctypes.c_int64),
                ("sink", ctypes.c_void_p), ("recent", ctypes.c_void_p), ("num_slots", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("max_pages_per_seq", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.mla_lowbit_page_bytes.argtypes = [ctypes.POINTER(Layout)]
    L.mla_lowbit_page_bytes.restype = SZ
    L.mla_lowbit_quantize_append.argtypes = [ctypes.POINTER(CacheDesc), P, P, P, P, I32, P]
    L.mla_lowbit_quantize_append.restype = ctypes.c_int
    L.mla_lowbit_decode_workspace_bytes.argtypes = [ctypes.POINTER(Layout), I32, I32, I32]
    L.mla_lowbit_decode_workspace_bytes.restype = SZ
    L.mla_lowbit_decode.argtypes = [ctypes.POINTER(CacheDesc), P, P, P, I32, I32, I32, ctypes.c_float, P, P, P, SZ, P]
    L.mla_lowbit_decode.restype = ctypes.c_int
    L.mla_lowbit_decode_multi.argtypes = [ctypes.POINTER(CacheDesc), P, P, P, I32, I32, I32, I32, ctypes.c_float,
                                          P, P, P, SZ, P]
    L.mla_lowbit_decode_multi.restype = ctypes.c_int
    L.mla_lowbit_decode_noalloc.argtypes = [ctypes.POINTER(CacheDesc), P, P, P, I32, I32, I32, ctypes.c_float, P, P, P]
    L.mla_lowbit_decode_noalloc.restype = ctypes.c_int
    L.mla_lowbit_status_string.argtypes = [ctypes.c_int]
    L.mla_lowbit_status_string.restype = ctypes.c_char_p
    L.mla_lowbit_profile_decode_events.argtypes = [P, P]
    L.mla_lowbit_profile_decode_events.restype = ctypes.c_int
    L.mla_lowbit_last_error.argtypes = []
    L.mla_lowbit_last_error.restype = ctypes.c_char_p
    return L


lib = _load()
EXPORTS = ("mla_lowbit_page_bytes", "mla_lowbit_quantize_append", "mla_lowbit_decode_workspace_bytes",
           "mla_lowbit_decode", "mla_lowbit_decode_multi", "mla_lowbit_decode_noalloc", "mla_lowbit_profile_decode_events",
           "mla_lowbit_status_string", "mla_lowbit_last_error")
SCRATCH_BYTES = 80 << 20  # MLA_LOWBIT_SCRATCH_BYTES


def _check(status: int) -> None:
    if status != OK:
        raise MlaLowbitError(status, lib.mla_lowbit_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def make_layout(bits_c: int = 4, n_sink: int = 4, n_recent: int = 128, bits_r: int = 4) -> Layout:
    return Layout(ABI_VERSION, D_C, D_R, bits_c, bits_r, 64, 64, n_sink, n_recent)


def page_bytes(layout: Layout) -> int:
    return int(lib.mla_lowbit_page_bytes(ctypes.byref(layout)))


@dataclass
class PagedCache:
    """Caller-owned cache buffers (torch device tensors) and their C descriptor."""
    layout: Layout
    pages: torch.Tensor        # uint8 [num_pages, page_bytes]
    sink: torch.Tensor         # bf16 [num_slots, n_sink, 576]
    recent: torch.Tensor       # bf16 [num_slots, n_recent, 576]
    block_table: torch.Tensor  # int32 [num_slots, max_pages_per_seq]

    @classmethod
    def allocate(cls, layout: Layout, num_pages: int, num_slots: int, max_pages_per_seq: int,
                 block_table: torch.Tensor | None = None, device="cuda") -> "PagedCache":
        pb = page_bytes(layout)
        if pb == 0:
            raise MlaLowbitError(ERR_UNSUPPORTED, lib.mla_lowbit_last_error().decode())
        pages = torch.zeros((num_pages, pb), dtype=torch.uint8, device=device)
        sink = torch.zeros((num_slots, max(layout.n_sink, 1), D), dtype=torch.bfloat16, device=device)
        recent = torch.zeros((num_slots, layout.n_recent, D), dtype=torch.bfloat16, device=device)
        if block_table is None:
            block_table = torch.full((num_slots, max_pages_per_seq), -1, dtype=torch.int32)
        block_table = block_table.to(device=device, dtype=torch.int32).contiguous()
        return cls(layout, pages, sink, recent, block_table)

    @property
    def desc(self) -> CacheDesc:
        return CacheDesc(self.layout, self.pages.data_ptr(), self.pages.shape[0], self.sink.data_ptr(),
                         self.recent.data_ptr(), self.block_table.shape[0], self.block_table.data_ptr(),
                         self.block_table.shape[1])


def quantize_append(cache: PagedCache, kv_new: torch.Tensor, token_slot: torch.Tensor, token_pos: torch.Tensor,
                    slot_len_after: torch.Tensor, stream=None) -> None:
    """mla_lowbit_quantize_append: kv_new bf16 [n, 576]; int32 index tensors on the device."""
    n = kv_new.shape[0]
    d = cache.desc
    _check(lib.mla_lowbit_quantize_append(ctypes.byref(d), _ptr(kv_new), _ptr(token_slot), _ptr(token_pos),
                                          _ptr(slot_len_after), n, _stream(stream)))


def profile_decode_events(start, stop) -> None:
    """Arm two hipEvent_t handles (ints) around the next decode kernel on this thread."""
    _check(lib.mla_lowbit_profile_decode_events(start, stop))


def decode_workspace_bytes(layout: Layout, batch: int, num_heads: int, max_seq_len: int) -> int:
    return int(lib.mla_lowbit_decode_workspace_bytes(ctypes.byref(layout), batch, num_heads, max_seq_len))


def decode(cache: PagedCache, q: torch.Tensor, seq_slot: torch.Tensor, seq_len: torch.Tensor, max_seq_len: int,
           softmax_scale: float, out: torch.Tensor, lse: torch.Tensor | None, workspace: torch.Tensor,
           stream=None) -> None:
    """mla_lowbit_decode: q bf16 [B, H, 576] -> out bf16 [B, H, 512], lse fp32 [B, H]."""
    batch, heads = q.shape[0], q.shape[1]
    d = cache.desc
    _check(lib.mla_lowbit_decode(ctypes.byref(d), _ptr(q), _ptr(seq_slot), _ptr(seq_len), batch, heads,
                                 max_seq_len, float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))


def decode_multi(cache: PagedCache, q: torch.Tensor, seq_slot: torch.Tensor, seq_len: torch.Tensor,
                 max_seq_len: int, softmax_scale: float, out: torch.Tensor, lse: torch.Tensor | None,
                 workspace: torch.Tensor, stream=None) -> None:
    """mla_lowbit_decode_multi: q bf16 [B, q_len, H, 576] -> out bf16 [B, q_len, H, 512], lse fp32
    [B, q_len, H]; query i of a sequence sees its first seq_len - (q_len - 1 - i) tokens."""
    batch, q_len, heads = q.shape[0], q.shape[1], q.shape[2]
    d = cache.desc
    _check(lib.mla_lowbit_decode_multi(ctypes.byref(d), _ptr(q), _ptr(seq_slot), _ptr(seq_len), batch, q_len, heads,
                                       max_seq_len, float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(stream)))


def decode_noalloc(cache: PagedCache, q: torch.Tensor, seq_slot: torch.Tensor, seq_len: torch.Tensor,
                   max_seq_len: int, softmax_scale: float, out: torch.Tensor, lse: torch.Tensor | None,
                   stream=None) -> None:
    """mla_lowbit_decode_noalloc: mla_lowbit_decode on the library's built-in device scratch."""
    batch, heads = q.shape[0], q.shape[1]
    d = cache.desc
    _check(lib.mla_lowbit_decode_noalloc(ctypes.byref(d), _ptr(q), _ptr(seq_slot), _ptr(seq_len), batch, heads,
                                         max_seq_len, float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream)))


def alloc_workspace(layout: Layout, batch: int, heads: int, max_seq_len: int, device="cuda") -> torch.Tensor:
    n = decode_workspace_bytes(layout, batch, heads, max_seq_len)
    if n == 0:
        raise MlaLowbitError(ERR_UNSUPPORTED, "unsupported decode shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def default_scale() -> float:
    """fp32(1/sqrt(d_head_qk)) with the absorbed-MLA head width 192 (128 nope + 64 rope)."""
    return float(torch.tensor(1.0 / math.sqrt(192.0), dtype=torch.float32))

"""Convenience: allocate a paged cache for a batch of sequence lengths and
prefill it through mla_lowbit_quantize_append (the HIP writer)."""
from __future__ import annotations

import numpy as np
import torch

from . import D, PagedCache, Layout, quantize_append


def block_table_for(seq_lens, perm: np.ndarray | None = None, page_tokens: int = 64, spare_tokens: int = 0,
                    spare_pages: int = 0):
    """Give every sequence ceil((N + spare_tokens)/page_tokens) pages, taken in order from `perm`
    (a permutation of the pool: shuffled physical order).  Returns (table [B, max_pages] int32, num_pages)."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    need = np.maximum(1, (seq_lens + spare_tokens + page_tokens - 1) // page_tokens)
    total = int(need.sum()) + spare_pages
    if perm is None:
        perm = np.arange(total, dtype=np.int32)
    assert len(perm) >= total
    total = max(total, len(perm), int(np.max(perm)) + 1)  # the pool spans every page the permutation names
    table = np.full((len(seq_lens), int(need.max())), -1, np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += int(n)
    return table, total


def to_device_bf16(rows_u16: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(rows_u16).view(np.int16)).view(torch.bfloat16).to(device)


def prefill(cache: PagedCache, slot: int, rows_u16: np.ndarray, start: int = 0, len_after: int | None = None,
            chunk: int = 1 << 16, stream=None) -> None:
    """Append rows [n, 576] (bf16 bits) as positions start.. of `slot` in chunks."""
    n = rows_u16.shape[0]
    dev = cache.pages.device
    if len_after is None:
        len_after = start + n
    lens = torch.zeros(cache.block_table.shape[0], dtype=torch.int32, device=dev)
    lens[slot] = len_after
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        kv = to_device_bf16(rows_u16[c0:c1], dev)
        slots = torch.full((c1 - c0,), slot, dtype=torch.int32, device=dev)
        pos = torch.arange(start + c0, start + c1, dtype=torch.int32, device=dev)
        quantize_append(cache, kv, slots, pos, lens, stream=stream)


def allocate_for(layout: Layout, seq_lens, perm=None, spare_tokens: int = 0, device="cuda") -> PagedCache:
    table, total = block_table_for(seq_lens, perm, spare_tokens=spare_tokens)
    return PagedCache.allocate(layout, total, len(seq_lens), table.shape[1], torch.from_numpy(table), device)


__all__ = ["block_table_for", "to_device_bf16", "prefill", "allocate_for", "D"]

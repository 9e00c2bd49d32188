"""Failure reporting of the decode path (marked gpu).

The kernels never fault or hang on bad device-resident data: a handshake wait between the two waves
of a 16-head pair is bounded, and a block-table entry outside the pool is read as page 0.  Both
events are counted in the workspace header, and with MLA_LOWBIT_VALIDATE=1 the library checks the
index data on the host before enqueueing and turns non-zero counters into MLA_LOWBIT_ERR_DEVICE
after the call.  The give-up path is forced from the host with a spin limit of 0 polls, so every
wave still runs its loop to the end and the kernels exit normally.
"""
import math
import os

import numpy as np
import pytest
import torch

import mla_inputs as mi

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_mla_kv_amd as m
from bit_mla_kv_amd import cache_builder as cb

SCALE = float(np.float32(1.0 / math.sqrt(192.0)))
HDR_GIVE_UPS, HDR_BAD_PAGES, HDR_BAD_SEQS, HDR_DROPPED = 4, 5, 6, 7


class Env:
    def __init__(self, **kv):
        self.kv = kv

    def __enter__(self):
        self.old = {k: os.environ.get(k) for k in self.kv}
        os.environ.update({k: str(v) for k, v in self.kv.items()})

    def __exit__(self, *a):
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def setup(heads, lens=(900, 300), bits_c=4):
    rows = [mi.rows(70, b, n) for b, n in enumerate(lens)]
    layout = m.make_layout(bits_c)
    cache = cb.allocate_for(layout, list(lens), mi.page_permutation(70, sum((n + 63) // 64 for n in lens) + 3))
    for b, r in enumerate(rows):
        cb.prefill(cache, b, r)
    dev = cache.pages.device
    B = len(lens)
    q = cb.to_device_bf16(mi.queries(70, B, heads).reshape(B * heads, -1), dev).view(B, heads, 576)
    out = torch.empty((B, heads, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, heads), dtype=torch.float32, device=dev)
    ws = m.alloc_workspace(layout, B, heads, max(lens), dev)
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    return cache, q, slots, sl, max(lens), out, lse, ws


def header(ws):
    torch.cuda.synchronize()
    return ws[:32].view(torch.int32).cpu().numpy()


@pytest.mark.parametrize("heads", [16, 128])
def test_validate_mode_passes_good_inputs(heads):
    cache, q, slots, sl, mx, out, lse, ws = setup(heads)
    m.decode(cache, q, slots, sl, mx, SCALE, out, lse, ws)
    ref = out.clone()
    with Env(MLA_LOWBIT_VALIDATE=1):
        m.decode(cache, q, slots, sl, mx, SCALE, out, lse, ws)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    h = header(ws)
    assert h[HDR_GIVE_UPS] == h[HDR_BAD_PAGES] == h[HDR_BAD_SEQS] == h[HDR_DROPPED] == 0


def test_forced_handshake_give_ups_are_counted_and_reported():
    """Spin limit 0: every wait of the 16-head kernel gives up at once.  Without validation the
    call returns OK and the count is in the header; with validation it returns ERR_DEVICE."""
    cache, q, slots, sl, mx, out, lse, ws = setup(16)
    with Env(MLA_LOWBIT_SPIN_LIMIT=0):
        m.decode(cache, q, slots, sl, mx, SCALE, out, lse, ws)
        assert header(ws)[HDR_GIVE_UPS] > 0
        with Env(MLA_LOWBIT_VALIDATE=1):
            with pytest.raises(m.MlaLowbitError) as e:
                m.decode(cache, q, slots, sl, mx, SCALE, out, lse, ws)
    assert e.value.status == m.ERR_DEVICE and "gave up" in str(e.value)
    m.decode(cache, q, slots, sl, mx, SCALE, out, lse, ws)  # the default bound again: no give-up
    assert header(ws)[HDR_GIVE_UPS] == 0


@pytest.mark.parametrize("heads", [16, 128])
def test_bad_page_id_counted_and_rejected(heads):
    """A block-table entry outside the pool in a sequence's packed range: the kernels read page 0
    instead and count it; validation rejects the call before anything is enqueued."""
    cache, q, slots, sl, mx, out, lse, ws = setup(heads)
    good = cache.block_table.clone()
    cache.block_table[0, 3] = cache.pages.shape[0] + 5
    m.decode(cache, q, slots, sl, mx, SCALE, out, lse, ws)
    assert header(ws)[HDR_BAD_PAGES] > 0
    with Env(MLA_LOWBIT_VALIDATE=1):
        with pytest.raises(m.MlaLowbitError) as e:
            m.decode(cache, q, slots, sl, mx, SCALE, out, lse, ws)
    assert e.value.status == m.ERR_INVALID_ARG and "block_table[0][3]" in str(e.value)
    cache.block_table.copy_(good)
    m.decode(cache, q, slots, sl, mx, SCALE, out, lse, ws)
    assert header(ws)[HDR_BAD_PAGES] == 0


def test_validate_rejects_bad_lengths_slots_and_shared_pages():
    cache, q, slots, sl, mx, out, lse, ws = setup(16)
    with Env(MLA_LOWBIT_VALIDATE=1):
        too_long = sl.clone()
        too_long[1] = mx + 1
        with pytest.raises(m.MlaLowbitError, match="seq_len"):
            m.decode(cache, q, slots, too_long, mx, SCALE, out, lse, ws)
        bad_slot = slots.clone()
        bad_slot[0] = 7
        with pytest.raises(m.MlaLowbitError, match="seq_slot"):
            m.decode(cache, q, bad_slot, sl, mx, SCALE, out, lse, ws)
        shared = cache.block_table.clone()
        cache.block_table[1, 2] = cache.block_table[0, 2]
        with pytest.raises(m.MlaLowbitError, match="tables of slots"):
            m.decode(cache, q, slots, sl, mx, SCALE, out, lse, ws)
        cache.block_table.copy_(shared)


def test_validate_append_arguments():
    cache, q, slots, sl, mx, out, lse, ws = setup(16)
    dev = cache.pages.device
    kv = cb.to_device_bf16(mi.rows(71, 0, 2), dev)
    i32 = lambda v: torch.tensor(v, dtype=torch.int32, device=dev)
    with Env(MLA_LOWBIT_VALIDATE=1):
        m.quantize_append(cache, kv, i32([0, 1]), i32([900, 300]), i32([901, 301]))  # good
        with pytest.raises(m.MlaLowbitError, match="appears twice"):
            m.quantize_append(cache, kv, i32([0, 0]), i32([900, 900]), i32([901, 301]))
        with pytest.raises(m.MlaLowbitError, match="token_pos"):
            m.quantize_append(cache, kv, i32([0, 1]), i32([900, 301]), i32([901, 301]))
        with pytest.raises(m.MlaLowbitError, match="token_slot"):
            m.quantize_append(cache, kv, i32([0, 2]), i32([900, 300]), i32([901, 301]))

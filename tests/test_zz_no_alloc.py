"""The allocation-free decode entry point mla_lowbit_decode_noalloc (marked gpu).

It runs the same plan, decode and combine kernels as mla_lowbit_decode on the library's built-in
device scratch instead of a caller workspace.  Two calls in a row, the second with a smaller input
(and another head count and code width), each compared with mla_lowbit_decode on the same inputs
(bit-identical: same kernels, same plan) and with the oracle (the parity bounds); the scratch keeps
the first call's contents, which the second must not depend on.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import mla_inputs as mi
from parity import E_TOL, bf16_tensor_to_f64, e_metric, lse_bound, reference

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_mla_kv_amd as m
from bit_mla_kv_amd import cache_builder as cb

SCALE = float(np.float32(1.0 / math.sqrt(192.0)))


def _case(seed, lens, heads, bits_c):
    rows = [mi.rows(seed, b, n) for b, n in enumerate(lens)]
    layout = m.make_layout(bits_c)
    cache = cb.allocate_for(layout, lens, mi.page_permutation(seed, sum(max(1, (n + 63) // 64) for n in lens) + 3))
    for b, r in enumerate(rows):
        if r.shape[0]:
            cb.prefill(cache, b, r)
    dev = cache.pages.device
    B = len(lens)
    q_host = mi.queries(seed, B, heads)
    q = cb.to_device_bf16(q_host.reshape(B * heads, -1), dev).view(B, heads, 576)
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    return rows, q_host, cache, q, slots, sl


def _run_both(rows, q_host, cache, q, slots, sl, bits_c):
    B, H = q.shape[0], q.shape[1]
    mx = max(max(int(x) for x in sl.tolist()), 1)
    dev = cache.pages.device
    out_ws = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    lse_ws = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = m.alloc_workspace(cache.layout, B, H, mx, dev)
    m.decode(cache, q, slots, sl, mx, SCALE, out_ws, lse_ws, ws)
    out = torch.full((B, H, 512), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=dev)
    m.decode_noalloc(cache, q, slots, sl, mx, SCALE, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_ws.view(torch.int16))
    assert torch.equal(lse, lse_ws)
    ro, rl = reference(rows, q_host, bits_c, SCALE)
    o = bf16_tensor_to_f64(out)
    assert np.all(np.isfinite(o))
    assert e_metric(o, ro).max() <= E_TOL
    l = lse.cpu().numpy().astype(np.float64)
    both = np.isneginf(l) & np.isneginf(rl)
    with np.errstate(invalid="ignore"):
        assert np.all(np.where(both, 0.0, np.abs(l - rl)) <= lse_bound(rl))


def test_noalloc_two_calls_match_decode():
    # first call: 128 heads (64-head kernel), C4, eight sequences up to 6000 tokens
    lens1 = [6000, 4100, 777, 133, 0, 2049, 5, 3000]
    _run_both(*_case(80, lens1, 128, 4), 4)
    # second call, smaller: 16 heads (16-head kernel), C2, two sequences
    lens2 = [700, 3]
    _run_both(*_case(81, lens2, 16, 2), 2)


def test_noalloc_rejects_shapes_beyond_its_scratch():
    rows, q_host, cache, q, slots, sl = _case(82, [100], 16, 4)
    need = m.decode_workspace_bytes(cache.layout, 256, 128, 1 << 17)
    assert need > m.SCRATCH_BYTES
    d = cache.desc
    st = m.lib.mla_lowbit_decode_noalloc(ctypes.byref(d), q.data_ptr(), slots.data_ptr(), sl.data_ptr(), 256, 128,
                                         1 << 17, SCALE, q.data_ptr(), None, None)
    assert st == m.ERR_WORKSPACE
    assert "scratch" in m.lib.mla_lowbit_last_error().decode()

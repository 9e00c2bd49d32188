"""Full-size parity (marked gpu): every workload the benchmark times, at its full size and in the
launch configuration it times (one quantize-append of a token per sequence, then the decode with the
default split plan), checked on every (sequence, head) output against the oracle, which computes each
sequence while the cache is being filled.  Every output row is held to the same bound as the
small-size tests (E <= 2e-3 after the bf16 store, |lse error| <= 1e-3).
"""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle
from parity import E_TOL, bf16_tensor_to_f64, e_metric, lse_bound

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_mla_kv_amd as m
from bit_mla_kv_amd import cache_builder as cb

FULL = ["dsv2lite_c4r4_32k", "dsv2lite_c4r4_128k", "dsv3_c4r4_128k", "dsv3_c2r4_128k", "mixed_c4r4_serving"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_every_row(name):
    w = mi.workload(name)
    B, H = w.batch, w.heads
    dev = torch.device("cuda:0")
    final = w.seq_lens.astype(np.int64)
    start = final - 1
    layout = m.make_layout(w.bits_c)
    perm = mi.page_permutation(w.seed, int(((final + 63) // 64).sum()) + 8)
    cache = cb.allocate_for(layout, start, perm, spare_tokens=1, device=dev)
    outl = mi.outlier_channels(w.seed)
    new = np.empty((B, 576), np.uint16)
    q_host = mi.queries(w.seed, B, H)
    ref_o = np.empty((B, H, 512))
    ref_l = np.empty((B, H))
    for b in range(B):
        rows = mi.rows(w.seed, b, int(final[b]), outl, threads=16)
        cb.prefill(cache, b, rows[:start[b]])
        new[b] = rows[start[b]]
        ref_o[b], ref_l[b] = oracle.decode_sequence(rows, q_host[b], w.scale, w.bits_c)
        del rows
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    m.quantize_append(cache, cb.to_device_bf16(new, dev), slots,
                      torch.tensor(start, dtype=torch.int32, device=dev),
                      torch.tensor(final, dtype=torch.int32, device=dev))
    q = cb.to_device_bf16(q_host.reshape(B * H, -1), dev).view(B, H, 576)
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = m.alloc_workspace(layout, B, H, int(final.max()), dev)
    m.decode(cache, q, slots, torch.tensor(final, dtype=torch.int32, device=dev), int(final.max()), w.scale,
             out, lse, ws)
    torch.cuda.synchronize()
    o_all = bf16_tensor_to_f64(out)
    l_all = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o_all)) and np.all(np.isfinite(l_all)), name
    E = e_metric(o_all, ref_o)
    worst = np.unravel_index(E.argmax(), E.shape)
    assert E.max() <= E_TOL, f"{name}: E max {E.max():.3e} at (sequence, head) {worst}"
    err = np.abs(l_all - ref_l)
    assert np.all(err <= lse_bound(ref_l)), f"{name}: lse err {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}"
    print(f"{name}: {B * H} rows, E max {E.max():.3e}, lse err max {err.max():.3e}", flush=True)


def test_full_size_multi_query():
    """Four query tokens per sequence on the 16-head 128K workload (the queries share one read of
    the cache as one 64-row group): every sequence, query and head; query i sees the first
    N - (3 - i) tokens in the representation the cache holds at length N."""
    w = mi.workload("dsv2lite_c4r4_128k")
    B, H, QL = w.batch, w.heads, 4
    dev = torch.device("cuda:0")
    lens = w.seq_lens.astype(np.int64)
    layout = m.make_layout(w.bits_c)
    cache = cb.allocate_for(layout, lens, mi.page_permutation(w.seed, int(((lens + 63) // 64).sum()) + 8), device=dev)
    outl = mi.outlier_channels(w.seed)
    q_host = mi.queries(w.seed + 7, B * QL, H).reshape(B, QL, H, 576)
    ref_o = np.empty((B, QL, H, 512))
    ref_l = np.empty((B, QL, H))
    for b in range(B):
        rows = mi.rows(w.seed, b, int(lens[b]), outl, threads=16)
        cb.prefill(cache, b, rows)
        n = rows.shape[0]
        cc, cr, meta = oracle.quantize(rows, w.bits_c)
        sel = oracle.select(rows, cc, cr, meta, w.bits_c)
        for i in range(QL):
            ref_o[b, i], ref_l[b, i] = oracle.attend(sel[: n - (QL - 1 - i)], q_host[b, i], w.scale)
        del rows, sel
    q = cb.to_device_bf16(q_host.reshape(B * QL * H, -1), dev).view(B, QL, H, 576)
    out = torch.empty((B, QL, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, QL, H), dtype=torch.float32, device=dev)
    ws = m.alloc_workspace(layout, B, QL * H, int(lens.max()), dev)
    m.decode_multi(cache, q, torch.arange(B, dtype=torch.int32, device=dev),
                   torch.tensor(lens, dtype=torch.int32, device=dev), int(lens.max()), w.scale, out, lse, ws)
    torch.cuda.synchronize()
    o_all = bf16_tensor_to_f64(out)
    l_all = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o_all)) and np.all(np.isfinite(l_all))
    E = e_metric(o_all, ref_o)
    assert E.max() <= E_TOL, f"E max {E.max():.3e} at (sequence, query, head) {np.unravel_index(E.argmax(), E.shape)}"
    assert np.all(np.abs(l_all - ref_l) <= lse_bound(ref_l))


@pytest.mark.parametrize("heads,bits_c", [(128, 4), (16, 2)])
def test_million_token_context(heads, bits_c):
    """The longest context of the pages' latency sweep (1M tokens), beside a short sequence in the
    same batch: one 1,048,576-token sequence and one of 777 tokens, decoded with the default split
    plan (the long one split over every CU, the short one in one or two items).  Every head of
    both sequences against the oracle, same bounds as above."""
    seed = 11 + bits_c
    lens = np.array([1 << 20, 777], np.int64)
    B = len(lens)
    dev = torch.device("cuda:0")
    layout = m.make_layout(bits_c)
    perm = mi.page_permutation(seed, int(((lens + 63) // 64).sum()))
    cache = cb.allocate_for(layout, lens, perm, device=dev)
    outl = mi.outlier_channels(seed)
    kept = {}
    for b in range(B):
        kept[b] = mi.rows(seed, b, int(lens[b]), outl, threads=16)
        cb.prefill(cache, b, kept[b])
    q_host = mi.queries(seed, B, heads)
    q = cb.to_device_bf16(q_host.reshape(B * heads, -1), dev).view(B, heads, 576)
    out = torch.empty((B, heads, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, heads), dtype=torch.float32, device=dev)
    ws = m.alloc_workspace(layout, B, heads, int(lens.max()), dev)
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    scale = float(np.float32(1.0 / np.sqrt(192.0)))
    m.decode(cache, q, slots, torch.tensor(lens, dtype=torch.int32, device=dev), int(lens.max()), scale,
             out, lse, ws)
    torch.cuda.synchronize()
    o_all = bf16_tensor_to_f64(out)
    l_all = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o_all)) and np.all(np.isfinite(l_all))
    for b in range(B):
        hs = list(range(heads))
        ro, rl = oracle.decode_sequence(kept[b], q_host[b], scale, bits_c, heads=hs)
        E = e_metric(o_all[b, hs], ro)
        assert E.max() <= E_TOL, f"H{heads} C{bits_c} seq {b} heads {hs}: E {E}"
        err = np.abs(l_all[b, hs] - rl)
        assert np.all(err <= lse_bound(rl)), f"H{heads} C{bits_c} seq {b}: lse err {err.max():.3e}"

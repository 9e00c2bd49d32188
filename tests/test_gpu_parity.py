"""GPU parity of the HIP path against the CPU oracle (marked gpu).

Writer: packed pages, sink and ring bytes are bit-exact with the oracle's
quantize + placement.  Decode: outputs within E <= 2e-3 (tests/parity.py),
lse within 1e-3, plus invariances (page order, split count, run-to-run,
stream vs bulk append) and NaN canaries proving each token is read exactly
once from exactly one representation.
"""
import math
import os

import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle
from parity import E_TOL, bf16_tensor_to_f64, e_metric, lse_bound, reference

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_mla_kv_amd as m
from bit_mla_kv_amd import cache_builder as cb

SCALE = float(np.float32(1.0 / math.sqrt(192.0)))


def build(rows_per_seq, bits_c, seed=0, n_sink=4, n_recent=128, spare_tokens=0, perm_seed=None):
    lens = [r.shape[0] for r in rows_per_seq]
    layout = m.make_layout(bits_c, n_sink, n_recent)
    need = [max(1, (n + spare_tokens + 63) // 64) for n in lens]
    total = sum(need) + 3
    perm = mi.page_permutation(seed if perm_seed is None else perm_seed, total)
    cache = cb.allocate_for(layout, lens, perm, spare_tokens=spare_tokens)
    for b, rows in enumerate(rows_per_seq):
        if rows.shape[0]:
            cb.prefill(cache, b, rows)
    torch.cuda.synchronize()
    return cache


def run_decode(cache, q_u16, lens, max_len=None):
    B, H = q_u16.shape[0], q_u16.shape[1]
    dev = cache.pages.device
    max_len = max(lens) if max_len is None else max_len
    q = cb.to_device_bf16(q_u16.reshape(B * H, -1), dev).view(B, H, 576)
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = m.alloc_workspace(cache.layout, B, H, max(max_len, 1), dev)
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    m.decode(cache, q, slots, sl, max(max_len, 1), SCALE, out, lse, ws)
    torch.cuda.synchronize()
    return out, lse


def check(out, lse, ref_o, ref_l, tag=""):
    o = bf16_tensor_to_f64(out)
    E = e_metric(o, ref_o)
    assert np.all(np.isfinite(o)), tag
    assert E.max() <= E_TOL, f"{tag} E max {E.max():.3e} at {np.unravel_index(E.argmax(), E.shape)}"
    l = lse.cpu().numpy().astype(np.float64)
    both_inf = np.isneginf(l) & np.isneginf(ref_l)
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(l - ref_l))
    assert np.all(err <= lse_bound(ref_l)), f"{tag} lse err {err.max():.3e} (|lse| up to {np.nanmax(np.abs(l)):.3g})"
    return E.max()


# ------------------------------------------------------------------- writer
def expected_pool(cache, rows_per_seq, bits_c):
    pool = np.zeros(tuple(cache.pages.shape), np.uint8)
    bt = cache.block_table.cpu().numpy()
    for b, rows in enumerate(rows_per_seq):
        if rows.shape[0]:
            cc, cr, meta = oracle.quantize(rows, bits_c)
            oracle.place_pages(pool, bt[b], cc, cr, meta, bits_c)
    return pool


def check_bf16_buffers(cache, rows_per_seq, n_sink=4, n_recent=128):
    sink = cache.sink.view(torch.int16).cpu().numpy().view(np.uint16)
    ring = cache.recent.view(torch.int16).cpu().numpy().view(np.uint16)
    for b, rows in enumerate(rows_per_seq):
        s, r = oracle.bf16_buffers(rows, n_sink, n_recent)
        for i, v in s.items():
            assert np.array_equal(sink[b, i], v), (b, i)
        for i, v in r.items():
            assert np.array_equal(ring[b, i], v), (b, i)


@pytest.mark.parametrize("bits_c", [4, 2])
def test_writer_bitexact(bits_c):
    lens = [1024, 200, 131, 5, 0, 64]
    rows = [mi.rows(21, b, n) for b, n in enumerate(lens)]
    cache = build(rows, bits_c, seed=21)
    pool = cache.pages.cpu().numpy()
    exp = expected_pool(cache, rows, bits_c)
    bad = np.argwhere(pool != exp)
    assert bad.size == 0, f"{len(bad)} bytes differ, first {bad[:4].tolist()}"
    check_bf16_buffers(cache, rows)


def test_writer_outlier_and_edge_values():
    """Rows with huge dynamic range, constant groups and signed zeros stay bit-exact."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((256, 576)) * np.exp(rng.uniform(-30, 30, (256, 1)))
    x[:, rng.choice(576, 16, replace=False)] *= 1000
    rows = mi.to_bf16(x)
    rows[3, 64:128] = rows[3, 64]
    rows[4, :] = 0
    rows[5, ::2] = 0x8000
    for bits_c in (4, 2):
        cache = build([rows], bits_c, seed=22)
        assert np.array_equal(cache.pages.cpu().numpy(), expected_pool(cache, [rows], bits_c))


def test_writer_stream_equals_bulk():
    """Appending one token (or small chunks) at a time gives the same cache as one bulk append."""
    n = 333
    rows = mi.rows(23, 0, n)
    bulk = build([rows], 4, seed=23)
    layout = m.make_layout(4)
    stream = cb.allocate_for(layout, [n], mi.page_permutation(23, 6 + 3))
    cuts = [0, 1, 2, 3, 4, 5, 70, 71, 200, 201, 333]
    for a, b in zip(cuts[:-1], cuts[1:]):
        cb.prefill(stream, 0, rows[a:b], start=a, len_after=b)
    torch.cuda.synchronize()
    assert np.array_equal(stream.pages.cpu().numpy(), bulk.pages.cpu().numpy())
    check_bf16_buffers(stream, [rows])


def _append(cache, rows_by_slot, items, lens_after):
    """One quantize_append call: items = [(slot, pos)], rows taken from rows_by_slot[slot][pos]."""
    dev = cache.pages.device
    kv = np.stack([rows_by_slot[s][p] for s, p in items])
    m.quantize_append(cache, cb.to_device_bf16(kv, dev),
                      torch.tensor([s for s, _ in items], dtype=torch.int32, device=dev),
                      torch.tensor([p for _, p in items], dtype=torch.int32, device=dev),
                      torch.tensor(lens_after, dtype=torch.int32, device=dev))


@pytest.mark.parametrize("bits_c", [4, 2])
def test_writer_chunked_prefill_and_rebuild(bits_c):
    """Chunked prefill with several slots' tokens interleaved in one call, then a preempted slot
    rebuilt from position 0 on other pages (recompute) while other slots keep appending: the final
    pages, sink and ring rows are bit-exact with the oracle's bulk quantization."""
    rng = np.random.default_rng(24)
    lens = [500, 300, 140, 300]  # slot 3 only lends its pages to slot 1's rebuild
    rows = [mi.rows(24, b, n) for b, n in enumerate(lens)]
    stale = mi.rows(25, 1, 200)  # slot 1's content before it is preempted
    layout = m.make_layout(bits_c)
    cache = cb.allocate_for(layout, lens, mi.page_permutation(24, sum((n + 63) // 64 for n in lens) + 3))
    first = [(0, p) for p in range(300)] + [(1, p) for p in range(200)] + [(2, p) for p in range(140)]
    first = [first[i] for i in rng.permutation(len(first))]
    _append(cache, [rows[0], stale, rows[2], None], first, [300, 200, 140, 0])
    # preemption: slot 1 takes slot 3's pages and is recomputed from position 0 in two chunks
    cache.block_table[1] = cache.block_table[3]
    second = [(0, p) for p in range(300, 500)] + [(1, p) for p in range(150)]
    second = [second[i] for i in rng.permutation(len(second))]
    _append(cache, rows, second, [500, 150, 140, 0])
    _append(cache, rows, [(1, p) for p in range(150, 300)], [500, 300, 140, 0])
    torch.cuda.synchronize()
    pool = cache.pages.cpu().numpy()
    bt = cache.block_table.cpu().numpy()
    for b in (0, 1, 2):
        cc, cr, meta = oracle.quantize(rows[b], bits_c)
        exp = np.zeros_like(pool)
        oracle.place_pages(exp, bt[b], cc, cr, meta, bits_c)
        used = bt[b][: (lens[b] + 63) // 64]
        assert np.array_equal(pool[used], exp[used]), f"slot {b}"
    check_bf16_buffers(cache, rows[:3] + [np.zeros((0, 576), np.uint16)])


# ------------------------------------------------------------------- decode
def test_decode_tiny_c4r4():
    """The tiny workload: batch 1, 16 heads, 1024 tokens."""
    w = mi.workload("tiny_c4r4")
    rows = [mi.rows(w.seed, 0, 1024)]
    q = mi.queries(w.seed, 1, 16)
    cache = build(rows, 4, seed=w.seed)
    out, lse = run_decode(cache, q, [1024])
    ro, rl = reference(rows, q, 4, SCALE)
    check(out, lse, ro, rl, "tiny")


EDGE_LENS = [0, 1, 3, 4, 5, 63, 64, 65, 131, 132, 133, 134, 196, 197, 198, 260, 700, 2049]


@pytest.mark.parametrize("heads", [16, 32, 48, 64, 96, 128])
@pytest.mark.parametrize("bits_c", [4, 2])
def test_decode_edge_lengths(heads, bits_c):
    seed = 30 + heads + bits_c
    rows = [mi.rows(seed, b, n) for b, n in enumerate(EDGE_LENS)]
    q = mi.queries(seed, len(EDGE_LENS), heads)
    cache = build(rows, bits_c, seed=seed)
    out, lse = run_decode(cache, q, EDGE_LENS)
    ro, rl = reference(rows, q, bits_c, SCALE)
    check(out, lse, ro, rl, f"H{heads} C{bits_c}")
    o = bf16_tensor_to_f64(out)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0].cpu().numpy()))  # N = 0


@pytest.mark.parametrize("heads", [16, 64])
def test_decode_many_sequences(heads):
    """130 sequences (the split plan scans sequences 64 at a time), lengths 0 .. 1500 mixed."""
    rng = np.random.default_rng(47 + heads)
    lens = [int(x) for x in rng.integers(0, 1500, size=130)]
    lens[0], lens[63], lens[64], lens[129] = 0, 133, 1, 1500
    rows = [mi.rows(47, b, n) for b, n in enumerate(lens)]
    q = mi.queries(47, len(lens), heads)
    cache = build(rows, 4, seed=47)
    out, lse = run_decode(cache, q, lens)
    ro, rl = reference(rows, q, 4, SCALE)
    check(out, lse, ro, rl, f"B130 H{heads}")


@pytest.mark.parametrize("heads", [16, 64])
def test_decode_large_batch_plan(heads):
    """600 sequences: above the planner's register path (512), so its per-pass path runs;
    also 300 (register path, tails in sequence order above 256)."""
    for B in (600, 300):
        rng = np.random.default_rng(49 + heads + B)
        lens = [int(x) for x in rng.integers(0, 400, size=B)]
        lens[0], lens[B - 1] = 0, 700
        rows = [mi.rows(49, b, n) for b, n in enumerate(lens)]
        q = mi.queries(49, B, heads)
        cache = build(rows, 4, seed=49)
        out, lse = run_decode(cache, q, lens)
        ro, rl = reference(rows, q, 4, SCALE)
        check(out, lse, ro, rl, f"B{B} H{heads}")


def test_decode_heads_256():
    lens = [900, 3000]
    rows = [mi.rows(41, b, n) for b, n in enumerate(lens)]
    q = mi.queries(41, 2, 256)
    cache = build(rows, 4, seed=41)
    out, lse = run_decode(cache, q, lens)
    ro, rl = reference(rows, q, 4, SCALE)
    check(out, lse, ro, rl, "H256")


@pytest.mark.parametrize("heads,bits_c", [(192, 2), (192, 4), (80, 4), (112, 2)])
def test_decode_odd_head_group_counts(heads, bits_c):
    """Head counts whose groups do not pair up: three 64-head groups (192, the 64-head kernel) and five
    or seven 16-head groups (80, 112), so the grid's head-group index and the XCD-interleaved item
    index take every residue; every (sequence, head) row against the oracle."""
    lens = [0, 133, 2500, 7000]
    rows = [mi.rows(43, b, n) for b, n in enumerate(lens)]
    q = mi.queries(43, len(lens), heads)
    cache = build(rows, bits_c, seed=43)
    out, lse = run_decode(cache, q, lens)
    ro, rl = reference(rows, q, bits_c, SCALE)
    check(out, lse, ro, rl, f"H{heads} C{bits_c}")


@pytest.mark.parametrize("heads", [16, 128])
def test_decode_max_len_far_above_lengths(heads):
    """max_seq_len of 2^20 with short sequences: the host sizes the workspace and the grid for the
    bound, the device plan splits only the tokens present, and the surplus workgroups find no item."""
    lens = [5, 900, 3000]
    rows = [mi.rows(44, b, n) for b, n in enumerate(lens)]
    q = mi.queries(44, len(lens), heads)
    cache = build(rows, 4, seed=44)
    out, lse = run_decode(cache, q, lens, max_len=1 << 20)
    ro, rl = reference(rows, q, 4, SCALE)
    check(out, lse, ro, rl, f"H{heads} max_len 2^20")


@pytest.mark.parametrize("heads", [16, 128])
def test_decode_permuted_and_repeated_slots(heads):
    """A batch that reads the cache slots out of order, one slot twice (with different queries) and
    leaves one slot unread: each batch entry attends over its own slot's tokens."""
    slot_lens = [300, 0, 2500, 133, 77]
    rows = [mi.rows(45, s_, n) for s_, n in enumerate(slot_lens)]
    cache = build(rows, 4, seed=45)
    order = [2, 0, 3, 0, 4]
    lens = [slot_lens[s_] for s_ in order]
    q_u16 = mi.queries(45, len(order), heads)
    dev = cache.pages.device
    B, H = len(order), heads
    q = cb.to_device_bf16(q_u16.reshape(B * H, -1), dev).view(B, H, 576)
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = m.alloc_workspace(cache.layout, B, H, max(lens), dev)
    m.decode(cache, q, torch.tensor(order, dtype=torch.int32, device=dev),
             torch.tensor(lens, dtype=torch.int32, device=dev), max(lens), SCALE, out, lse, ws)
    torch.cuda.synchronize()
    ro, rl = reference([rows[s_] for s_ in order], q_u16, 4, SCALE)
    check(out, lse, ro, rl, f"H{heads} slots {order}")


def test_all_bf16_mode():
    """n_recent >= N: every token from bf16, equals standard attention (oracle in all-bf16 mode)."""
    lens = [300, 1000]
    rows = [mi.rows(42, b, n) for b, n in enumerate(lens)]
    q = mi.queries(42, 2, 16)
    cache = build(rows, 4, seed=42, n_recent=1024)
    out, lse = run_decode(cache, q, lens)
    ro, rl = reference(rows, q, 4, SCALE, n_recent=1024)
    check(out, lse, ro, rl, "all-bf16")


@pytest.mark.parametrize("heads", [16, 64])
def test_all_bf16_long_window_chunks(heads):
    """A long recent window (n_recent >= N): the bf16 token lists are split over many items
    (chunks of 64 P tokens, P pages per split), merged exactly by the combine; the output must not
    depend on the chunking."""
    lens = [3000, 700, 1, 0]
    rows = [mi.rows(46, b, n) for b, n in enumerate(lens)]
    q = mi.queries(46, len(lens), heads)
    cache = build(rows, 4, seed=46, n_recent=4096)
    ro, rl = reference(rows, q, 4, SCALE, n_recent=4096)
    outs = []
    for pps in ("1", "3", None):
        if pps is not None:
            os.environ["MLA_LOWBIT_PAGES_PER_SPLIT"] = pps
        try:
            out, lse = run_decode(cache, q, lens)
        finally:
            os.environ.pop("MLA_LOWBIT_PAGES_PER_SPLIT", None)
        check(out, lse, ro, rl, f"all-bf16 H{heads} pps={pps}")
        outs.append(bf16_tensor_to_f64(out))
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 4e-3 * np.max(np.abs(outs[0]))


HDR_DIRECT = 2  # workspace header word: workgroups that wrote their sequence's final outputs


@pytest.mark.parametrize("heads,bits_c", [(16, 4), (16, 2), (64, 4), (128, 2)])
def test_one_item_sequences_written_by_the_decode(heads, bits_c):
    """A sequence with no packed tokens and one bf16 chunk (here every N <= n_sink + n_recent, N = 0
    included) is decoded by one work item, whose workgroups write its final bf16 outputs and lse;
    the combine leaves it alone and merges the longer ones.  out and lse start as NaN, so a row
    that nobody writes fails; header word 2 counts the workgroups that wrote directly."""
    lens = [0, 1, 5, 64, 132, 133, 900, 3000]
    rows = [mi.rows(33, b, n) for b, n in enumerate(lens)]
    cache = build(rows, bits_c, seed=33)
    B, dev = len(lens), cache.pages.device
    q = mi.queries(33, B, heads)
    qd = cb.to_device_bf16(q.reshape(B * heads, -1), dev).view(B, heads, 576)
    out = torch.full((B, heads, 512), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, heads), float("nan"), dtype=torch.float32, device=dev)
    ws = m.alloc_workspace(cache.layout, B, heads, max(lens), dev)
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    m.decode(cache, qd, slots, torch.tensor(lens, dtype=torch.int32, device=dev), max(lens), SCALE, out, lse, ws)
    torch.cuda.synchronize()
    ref_o, ref_l = reference(rows, q, bits_c, SCALE)
    check(out, lse, ref_o, ref_l, f"one-item H{heads} C{bits_c}")
    workgroups_per_item = heads // 64 if heads % 64 == 0 else heads // 16
    n_direct = sum(n <= 132 for n in lens)
    assert int(ws[:32].view(torch.int32)[HDR_DIRECT].item()) == n_direct * workgroups_per_item


def run_decode_multi(cache, q_u16, lens, max_len=None):
    """q_u16 [B, q_len, H, 576] -> (out [B, q_len, H, 512], lse [B, q_len, H])."""
    B, QL, H = q_u16.shape[:3]
    dev = cache.pages.device
    max_len = max(max(lens), 1) if max_len is None else max_len
    q = cb.to_device_bf16(q_u16.reshape(B * QL * H, -1), dev).view(B, QL, H, 576)
    out = torch.empty((B, QL, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, QL, H), dtype=torch.float32, device=dev)
    ws = m.alloc_workspace(cache.layout, B, QL * H, max_len, dev)
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    m.decode_multi(cache, q, slots, sl, max_len, SCALE, out, lse, ws)
    torch.cuda.synchronize()
    return out, lse


def reference_multi(rows_per_seq, q, bits_c):
    """Query i of a sequence of N tokens: the oracle's selection at length N (which tokens are
    bf16 is fixed by the cache), attended over its first N - (q_len - 1 - i) rows."""
    B, QL, H = q.shape[:3]
    ro = np.zeros((B, QL, H, 512))
    rl = np.full((B, QL, H), -np.inf)
    for b, rows in enumerate(rows_per_seq):
        n = rows.shape[0]
        if n == 0:
            continue
        cc, cr, meta = oracle.quantize(rows, bits_c)
        sel = oracle.select(rows, cc, cr, meta, bits_c)
        for i in range(QL):
            n_vis = n - (QL - 1 - i)
            if n_vis > 0:
                ro[b, i], rl[b, i] = oracle.attend(sel[:n_vis], q[b, i], SCALE)
    return ro, rl


@pytest.mark.parametrize("heads,q_len", [(16, 2), (16, 4), (128, 2), (64, 3)])
def test_decode_multi_query(heads, q_len):
    """Several query tokens per sequence with causal visibility; the queries share the cache read
    (16 heads x 4 queries run as one 64-row group)."""
    lens = [0, 1, 3, 132, 135, 200, 700, 2049]
    rows = [mi.rows(47, b, n) for b, n in enumerate(lens)]
    q = mi.queries(47, len(lens) * q_len, heads).reshape(len(lens), q_len, heads, 576)
    cache = build(rows, 4, seed=47)
    out, lse = run_decode_multi(cache, q, lens)
    ro, rl = reference_multi(rows, q, 4)
    check(out, lse, ro, rl, f"multi H{heads} q_len {q_len}")


@pytest.mark.parametrize("bits_c", [4, 2])
def test_decode_multi_query_window_limit(bits_c):
    """q_len = n_recent + 1 (the largest allowed): with a 3-token recent window, four queries;
    the tokens the early queries do not see are exactly the window's, and the window is shorter
    than the queries' spread for the first one."""
    lens = [1, 4, 9, 70, 300]
    rows = [mi.rows(51, b, n) for b, n in enumerate(lens)]
    q = mi.queries(51, len(lens) * 4, 16).reshape(len(lens), 4, 16, 576)
    cache = build(rows, bits_c, seed=51, n_recent=3)
    out, lse = run_decode_multi(cache, q, lens)
    ro = np.zeros((len(lens), 4, 16, 512))
    rl = np.full((len(lens), 4, 16), -np.inf)
    for b, r in enumerate(rows):
        cc, cr, meta = oracle.quantize(r, bits_c)
        sel = oracle.select(r, cc, cr, meta, bits_c, 4, 3)
        for i in range(4):
            n_vis = r.shape[0] - (3 - i)
            if n_vis > 0:
                ro[b, i], rl[b, i] = oracle.attend(sel[:n_vis], q[b, i], SCALE)
    check(out, lse, ro, rl, f"multi window limit C{bits_c}")


def test_decode_multi_single_query_is_decode():
    lens = [700, 2049]
    rows = [mi.rows(48, b, n) for b, n in enumerate(lens)]
    q = mi.queries(48, 2, 16)
    cache = build(rows, 4, seed=48)
    o1, l1 = run_decode(cache, q, lens)
    o2, l2 = run_decode_multi(cache, q.reshape(2, 1, 16, 576), lens)
    assert torch.equal(o1, o2.view(2, 16, 512)) and torch.equal(l1, l2.view(2, 16))


@pytest.mark.parametrize("n_sink,n_recent", [(0, 1), (0, 128), (64, 16), (7, 200)])
@pytest.mark.parametrize("heads", [16, 64])
def test_decode_window_layouts(n_sink, n_recent, heads):
    """Other sink / recent windows of the layout: no sink, a one-token recent window, the largest
    sink; writer bytes bit-exact and decode against the oracle with the same windows."""
    lens = [0, 1, 5, 63, 64, 65, 300, 1000]
    rows = [mi.rows(50, b, n) for b, n in enumerate(lens)]
    q = mi.queries(50, len(lens), heads)
    cache = build(rows, 4, seed=50, n_sink=n_sink, n_recent=n_recent)
    check_bf16_buffers(cache, rows, n_sink=n_sink, n_recent=n_recent)
    out, lse = run_decode(cache, q, lens)
    ro, rl = [], []
    for b, r in enumerate(rows):
        o, l = oracle.decode_sequence(r, q[b], SCALE, 4, None, n_sink, n_recent)
        ro.append(o)
        rl.append(l)
    check(out, lse, np.stack(ro), np.stack(rl), f"sink {n_sink} recent {n_recent} H{heads}")


@pytest.mark.parametrize("heads", [16, 64, 128])
@pytest.mark.parametrize("bits_c", [4, 2])
def test_exactly_once_canaries(heads, bits_c):
    """NaN in every representation a token must NOT be read from leaves the output unchanged: the
    packed copies of sink, recent and past-the-end rows of each page (content codes 0xFF, NaN scales
    and zeros), unused ring rows and sink rows.  Runs the 16-head kernel (H16) and the 64-head one
    (H64, H128), whose packed tiles mask such rows inside a page."""
    lens = [1000, 150, 2, 0, 197]
    rows = [mi.rows(43, b, n) for b, n in enumerate(lens)]
    q = mi.queries(43, len(lens), heads)
    cache = build(rows, bits_c, seed=43)
    out0, lse0 = run_decode(cache, q, lens)
    bt = cache.block_table.cpu().numpy()
    pages = cache.pages.cpu().numpy()
    cbytes = 64 * bits_c
    meta_off = 64 * (cbytes + 32)
    nan_meta = np.frombuffer(np.array([0x7FC07FC0] * 9, np.uint32).tobytes(), np.uint8)
    for b, n in enumerate(lens):
        npg = max(1, (n + 63) // 64)
        for t in range(npg * 64):
            bf = t < 4 or t >= n - 128 or t >= n
            if not bf:
                continue
            pg, r = bt[b, t // 64], t % 64
            pages[pg, meta_off + 36 * r: meta_off + 36 * r + 36] = nan_meta
            pages[pg, r * cbytes:(r + 1) * cbytes] = 0xFF
    cache.pages.copy_(torch.from_numpy(pages))
    ring = cache.recent.view(torch.int16).cpu().numpy()
    sink = cache.sink.view(torch.int16).cpu().numpy()
    for b, n in enumerate(lens):
        live = {p % 128 for p in range(max(0, n - 128), n)}
        for i in range(128):
            if i not in live:
                ring[b, i] = np.int16(0x7FC0)
        for i in range(min(4, n), 4):
            sink[b, i] = np.int16(0x7FC0)
    cache.recent.copy_(torch.from_numpy(ring).view(torch.bfloat16))
    cache.sink.copy_(torch.from_numpy(sink).view(torch.bfloat16))
    out1, lse1 = run_decode(cache, q, lens)
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse0, lse1)
    ro, rl = reference(rows, q, bits_c, SCALE)
    check(out1, lse1, ro, rl, f"canary H{heads} C{bits_c}")


def test_page_order_invariance_and_determinism():
    lens = [5000, 777]
    rows = [mi.rows(44, b, n) for b, n in enumerate(lens)]
    q = mi.queries(44, 2, 64)
    c1 = build(rows, 4, seed=44, perm_seed=1)
    c2 = build(rows, 4, seed=44, perm_seed=2)
    assert not torch.equal(c1.block_table, c2.block_table)
    o1, l1 = run_decode(c1, q, lens)
    o1b, l1b = run_decode(c1, q, lens)
    o2, l2 = run_decode(c2, q, lens)
    assert torch.equal(o1.view(torch.int16), o1b.view(torch.int16)) and torch.equal(l1, l1b)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


@pytest.mark.parametrize("heads", [16, 128])
def test_split_count_invariance(heads):
    """The same decode with 1, 4, 37 and 1000 pages per split (from one split per page to one
    split per sequence): every result within the bound, and all within 4e-3 of each other."""
    lens = [9000, 4100]
    rows = [mi.rows(45, b, n) for b, n in enumerate(lens)]
    q = mi.queries(45, 2, heads)
    cache = build(rows, 4, seed=45)
    ro, rl = reference(rows, q, 4, SCALE)
    outs = []
    for pps in ("1", "4", "37", "1000"):
        os.environ["MLA_LOWBIT_PAGES_PER_SPLIT"] = pps
        try:
            out, lse = run_decode(cache, q, lens)
        finally:
            del os.environ["MLA_LOWBIT_PAGES_PER_SPLIT"]
        check(out, lse, ro, rl, f"pps={pps}")
        outs.append(bf16_tensor_to_f64(out))
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 4e-3 * np.max(np.abs(outs[0]))


def test_serving_step_append_then_decode():
    """One token appended per sequence (its predecessor 128 back migrates to packed), then decode."""
    lens = [1500, 129, 4000, 10]
    rows_full = [mi.rows(46, b, n + 3) for b, n in enumerate(lens)]
    q = mi.queries(46, len(lens), 128)
    layout = m.make_layout(4)
    perm = mi.page_permutation(46, 200)
    cache = cb.allocate_for(layout, lens, perm, spare_tokens=3)
    for b, n in enumerate(lens):
        cb.prefill(cache, b, rows_full[b][:n])
    cur = list(lens)
    for step in range(3):
        kv = np.stack([rows_full[b][cur[b]] for b in range(len(lens))])
        dev = cache.pages.device
        slots = torch.arange(len(lens), dtype=torch.int32, device=dev)
        pos = torch.tensor(cur, dtype=torch.int32, device=dev)
        after = pos + 1
        m.quantize_append(cache, cb.to_device_bf16(kv, dev), slots, pos, after)
        cur = [c + 1 for c in cur]
        out, lse = run_decode(cache, q, cur, max_len=max(lens) + 3)
        ro, rl = reference([rows_full[b][:cur[b]] for b in range(len(lens))], q, 4, SCALE)
        check(out, lse, ro, rl, f"step{step}")


def _scaled(u16, mult):
    return mi.to_bf16(mi.bf16_bits_to_f32(u16).astype(np.float64) * mult)


# cache multiplier, query multiplier: the workloads' values (x1); a cache scaled up with queries
# scaled down so that the scores keep the workloads' spread (the PV scales then reach 2^13, where an
# fp16 product p * s with p up to 2^8 would overflow); a cache scaled down with queries scaled up
# (PV scales near 2^-15, fp16 subnormals unless normalised); a large cache with unscaled queries
# (sharply peaked softmax); "ramp": token magnitudes growing from x1e-3 to x300 along the sequence
# with queries x1e-2, so that a work item's PV scales grow by 2^18 while the early tokens keep
# their weight
VALUE_RANGES = [(1.0, 1.0), (300.0, 1.0 / 300.0), (1e-4, 1e2), (1e-4, 1e3), (300.0, 1.0), ("ramp", 1e-2)]


@pytest.mark.parametrize("heads", [16, 128])
@pytest.mark.parametrize("bits_c", [4, 2])
@pytest.mark.parametrize("cache_mult,q_mult", VALUE_RANGES, ids=lambda v: str(v))
def test_decode_value_range(cache_mult, q_mult, bits_c, heads):
    """Cache values from about 1e-4 to 3e4 in magnitude against the oracle, same bounds."""
    lens = [0, 5, 133, 700, 3000]
    rows = []
    for b, n in enumerate(lens):
        r = mi.rows(52, b, n)
        if cache_mult == "ramp":
            f = 10.0 ** np.linspace(-3.0, np.log10(300.0), max(n, 1))[:n, None]
            rows.append(mi.to_bf16(mi.bf16_bits_to_f32(r).astype(np.float64) * f))
        else:
            rows.append(_scaled(r, cache_mult))
    q = _scaled(mi.queries(52, len(lens), heads), q_mult)
    cache = build(rows, bits_c, seed=52)
    out, lse = run_decode(cache, q, lens)
    ro, rl = reference(rows, q, bits_c, SCALE)
    check(out, lse, ro, rl, f"cache x{cache_mult} q x{q_mult:.3g} C{bits_c} H{heads}")


def _random_config(seed):
    rng = np.random.default_rng(1000 + seed)
    heads = int(rng.choice([16, 32, 48, 64, 96, 128]))
    bits_c = int(rng.choice([4, 2]))
    B = int(rng.integers(1, 25))
    lens = [int(x) for x in np.exp(rng.uniform(0, np.log(20000), size=B)).astype(np.int64) - 1]
    n_sink, n_recent = [(4, 128), (0, 17), (9, 300), (4, 1)][int(rng.integers(0, 4))]
    return heads, bits_c, lens, n_sink, n_recent


@pytest.mark.parametrize("seed", range(12))
def test_decode_random_configs(seed):
    """Seeded random shapes against the oracle on every (sequence, head) row: head count (both
    kernels), bit width, batch 1..24, log-uniform lengths 0..20K (so the plan mixes full chunks,
    tails and bf16 items, and the combine one or several partials per row) and sink / recent
    window sizes."""
    heads, bits_c, lens, n_sink, n_recent = _random_config(seed)
    rows = [mi.rows(2000 + seed, b, n) for b, n in enumerate(lens)]
    q = mi.queries(2000 + seed, len(lens), heads)
    cache = build(rows, bits_c, seed=2000 + seed, n_sink=n_sink, n_recent=n_recent)
    out, lse = run_decode(cache, q, lens)
    ro, rl = reference(rows, q, bits_c, SCALE, n_sink=n_sink, n_recent=n_recent)
    check(out, lse, ro, rl, f"seed {seed}: H{heads} C{bits_c} B{len(lens)} sink {n_sink} recent {n_recent}")

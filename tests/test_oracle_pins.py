"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test names what it pins and why a plausible mistake in the oracle would
fail it (dropped RoPE term, wrong window, wrong sign or bit order, wrong lse).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SCALE = float(np.float32(1.0 / math.sqrt(192.0)))


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def _bf16(x):
    return mi.to_bf16(np.asarray(x, np.float64))


def _f(bits):
    return mi.bf16_bits_to_f32(bits).astype(np.float64)


# ----------------------------------------------------------------- P3: worked examples
def _example_group(ex):
    inp = ex["input"]
    if inp["kind"] == "mod":
        vals = inp["sign"] * (np.arange(64) % inp["m"]).astype(np.float64)
    elif inp["kind"] == "list":
        vals = np.full(64, inp["fill"], np.float64)
        vals[:len(inp["head"])] = inp["head"]
    else:
        vals = np.linspace(inp["lo"], inp["hi"], 64)
    g = _bf16(vals)
    if inp["kind"] == "list" and inp["head"][:1] == [-0.0]:
        g[0] = 0x8000  # keep the sign of -0.0 explicitly
    return g


def _codes(packed_row, bits, n=64):
    per = 8 // bits
    return np.array([(packed_row[i // per] >> ((i % per) * bits)) & ((1 << bits) - 1) for i in range(n)])


@pytest.mark.parametrize("ex", json.load(open(os.path.join(GOLDEN, "quantizer_examples.json")))["examples"],
                         ids=lambda e: e["name"])
def test_quantizer_worked_examples(ex):
    """Hand-derived bit patterns (tests/golden/quantizer_examples.json)."""
    bits = ex["bits"]
    grp = _example_group(ex)
    row = np.zeros((1, 576), np.uint16)
    row[0, 64:128] = grp                     # content group 1
    if bits == 4:
        row[0, 512:576] = grp                # RoPE-key group (always 4 bit)
    for bc in ([4, 2] if bits == 4 else [2]):
        cc, cr, meta = oracle.quantize(row, bc)
        gb = 64 * bc // 8
        targets = [(cc[0, gb:2 * gb], 1)] if bc == bits else []
        if bits == 4:
            targets.append((cr[0], 8))
        for packed, g in targets:
            assert meta[0, g] & 0xFFFF == int(ex["s_bits"], 16), hex(meta[0, g])
            assert meta[0, g] >> 16 == int(ex["z_bits"], 16), hex(meta[0, g])
            if "bytes" in ex:
                assert bytes(packed).hex().upper() == ex["bytes"]
            codes = _codes(packed, bits)
            if "codes_head" in ex:
                h = ex["codes_head"]
                assert list(codes[:len(h)]) == h
            if "codes_fill" in ex:
                assert (codes[len(ex["codes_head"]):] == ex["codes_fill"]).all()
            if "codes_last" in ex:
                assert codes[-1] == ex["codes_last"]
        # zero groups quantize to s = 0, z = +0
        assert meta[0, 0] == 0


# ----------------------------------------------------------------- P4: round-trip invariant
@pytest.mark.parametrize("bits_c", [4, 2])
def test_roundtrip_bound(bits_c):
    """|x - xhat| <= s/2 per element, code(min) = 0, code(max) = Lb (dequantized by hand here)."""
    rng = np.random.default_rng(7)
    n = 4000
    x = rng.standard_normal((n, 576))
    x[:, rng.choice(512, 8, replace=False)] *= 20
    x[: n // 4] *= np.exp(rng.uniform(-20, 20, (n // 4, 1)))     # wide exponent range
    rows = _bf16(x)
    rows[5, 0:64] = rows[5, 0]                                   # a constant group
    cc, cr, meta = oracle.quantize(rows, bits_c)
    xf = _f(rows)
    lb_c = (1 << bits_c) - 1
    for t in range(0, n, 7):
        for g in range(9):
            bits = bits_c if g < 8 else 4
            lb = (1 << bits) - 1
            packed = cc[t, g * 64 * bits_c // 8:(g + 1) * 64 * bits_c // 8] if g < 8 else cr[t]
            q = _codes(packed, bits)
            s = _f(np.array([meta[t, g] & 0xFFFF], np.uint16))[0]
            z = _f(np.array([meta[t, g] >> 16], np.uint16))[0]
            xs = xf[t, g * 64:(g + 1) * 64]
            xhat = s * q + z
            # allowance: fp32 rounding of (x - mn)/s can move a value off an exact tie
            assert np.all(np.abs(xs - xhat) <= s / 2 * (1 + 2.0 ** -20) + 1e-300), (t, g)
            assert z == xs.min()
            if s > 0:
                assert q[np.argmin(xs)] == 0 and q[np.argmax(xs)] == lb
            else:
                assert np.all(xs == xs[0]) and np.all(q == 0)
    assert lb_c in (3, 15)


# ----------------------------------------------------------------- helpers (independent of the oracle)
def _unpack_page_token(pages, bt_row, t, bits_c, page_tokens=64):
    """Decode token t's packed copy straight from page bytes (layout documented in oracle/__init__)."""
    pg = pages[int(bt_row[t // page_tokens])]
    r = t % page_tokens
    cb = 64 * bits_c
    off_r = page_tokens * cb
    off_m = off_r + page_tokens * 32
    meta = pg[off_m + r * 36: off_m + r * 36 + 36].view(np.uint32)
    cbytes = pg[r * cb:(r + 1) * cb]
    rbytes = pg[off_r + r * 32: off_r + r * 32 + 32]
    out = np.empty(576)
    for ch in range(576):
        if ch < 512:
            per = 8 // bits_c
            code = (int(cbytes[ch // per]) >> ((ch % per) * bits_c)) & ((1 << bits_c) - 1)
        else:
            code = (int(rbytes[(ch - 512) // 2]) >> (((ch - 512) % 2) * 4)) & 15
        md = int(meta[ch // 64])
        s = float(mi.bf16_bits_to_f32(np.array([md & 0xFFFF], np.uint16))[0])
        z = float(mi.bf16_bits_to_f32(np.array([md >> 16], np.uint16))[0])
        out[ch] = s * code + z
    return out


def _brute_attention(K, q, scale):
    """Direct fp64 softmax attention with explicit loops over tokens."""
    qd = _f(q)
    outs, lses = [], []
    for h in range(qd.shape[0]):
        sc = [scale * float(np.dot(qd[h], K[t])) for t in range(K.shape[0])]
        m = max(sc)
        w = [math.exp(s - m) for s in sc]
        l = sum(w)
        o = sum(w[t] * K[t, :512] for t in range(K.shape[0])) / l
        outs.append(o)
        lses.append(m + math.log(l))
    return np.array(outs), np.array(lses)


# ----------------------------------------------------------------- P1: all-BF16 == standard MLA
def test_all_bf16_equals_standard_attention():
    """With every token in the BF16 window, oracle == torch softmax(scale QK^T) V (fp64, CPU)."""
    n, h = 300, 16
    rows = mi.rows(11, 0, n)
    q = mi.queries(11, 1, h)[0]
    out, lse = oracle.decode_sequence(rows, q, SCALE, 4, n_recent=n)
    K = torch.from_numpy(_f(rows))
    Q = torch.from_numpy(_f(q))
    s = SCALE * (Q @ K.T)
    ref = torch.softmax(s, dim=-1) @ K[:, :512]
    ref_lse = torch.logsumexp(s, dim=-1)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=1e-13)


# ----------------------------------------------------------------- P2: absorbed == explicit-head MLA
def test_absorbed_equals_explicit_heads():
    """Scores through W_UK and outputs through W_UV equal the absorbed latent form."""
    rng = np.random.default_rng(3)
    n, h, dh = 200, 4, 128
    rows = mi.rows(12, 0, n)
    cc, cr, meta = oracle.quantize(rows, 4)
    sel = oracle.select(rows, cc, cr, meta, 4)
    w_uk = rng.integers(-1, 2, (h, dh, 512)).astype(np.float64)
    w_uv = rng.standard_normal((h, dh, 512))
    q_nope = rng.integers(-1, 2, (h, dh)).astype(np.float64)
    q_pe = _f(mi.queries(12, 1, h)[0][:, 512:])
    q_c = np.einsum("hd,hdc->hc", q_nope, w_uk)          # integers |.| <= 128: exact in bf16
    q = np.concatenate([_bf16(q_c), _bf16(q_pe)], axis=1)
    assert np.array_equal(_f(q[:, :512]), q_c)
    out_lat, _ = oracle.attend(sel, q, SCALE)
    for hh in range(h):
        k_nope = sel[:, :512] @ w_uk[hh].T                # per-head keys [n, dh]
        v = sel[:, :512] @ w_uv[hh].T                     # per-head values [n, dh]
        s = SCALE * (k_nope @ q_nope[hh] + sel[:, 512:] @ q_pe[hh])
        p = np.exp(s - s.max())
        p /= p.sum()
        explicit = p @ v
        np.testing.assert_allclose(w_uv[hh] @ out_lat[hh], explicit, rtol=1e-10, atol=1e-10)


# ----------------------------------------------------------------- P5: q = 0 closed form + selection
@pytest.mark.parametrize("bits_c", [4, 2])
@pytest.mark.parametrize("n", [1, 4, 5, 131, 132, 133, 700])
def test_zero_query_uniform_and_selection(n, bits_c):
    """q = 0: output = mean of the selected rows, lse = ln N; selected rows follow the window rule,
    and every packed token equals its copy decoded straight from the page bytes (4- and 2-bit)."""
    rows = mi.rows(13, 0, n)
    cc, cr, meta = oracle.quantize(rows, bits_c)
    npages = (n + 63) // 64
    pages = np.zeros((npages + 3, oracle.page_bytes(bits_c)), np.uint8)
    bt = mi.page_permutation(13, npages + 3)[:npages]
    oracle.place_pages(pages, bt, cc, cr, meta, bits_c)
    sel = oracle.select(rows, cc, cr, meta, bits_c)
    raw = _f(rows)
    for t in range(n):
        if t < 4 or t >= n - 128:
            assert np.array_equal(sel[t], raw[t]), t
        else:
            np.testing.assert_array_equal(sel[t], _unpack_page_token(pages, bt, t, bits_c))
    out, lse = oracle.attend(sel, np.zeros((2, 576), np.uint16), SCALE)
    np.testing.assert_allclose(out[0], sel[:, :512].mean(0), rtol=1e-12, atol=1e-12)
    assert abs(lse[0] - math.log(n)) < 1e-12


def test_empty_sequence():
    out, lse = oracle.attend(np.zeros((0, 576)), mi.queries(1, 1, 3)[0], SCALE)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


# ----------------------------------------------------------------- P6: brute force on tiny contexts
@pytest.mark.parametrize("bits_c", [4, 2])
def test_brute_force_tiny_contexts(bits_c):
    """N in 1..200 and 255..257: oracle == explicit-loop attention over page-decoded tokens."""
    rows_all = mi.rows(14, 0, 257)
    q = mi.queries(14, 1, 2)[0]
    cc, cr, meta = oracle.quantize(rows_all, bits_c)
    pages = np.zeros((8, oracle.page_bytes(bits_c)), np.uint8)
    bt = np.array([5, 2, 7, 0, 3], np.int32)
    oracle.place_pages(pages, bt, cc, cr, meta, bits_c)
    decoded = np.array([_unpack_page_token(pages, bt, t, bits_c) for t in range(257)])
    raw = _f(rows_all)
    for n in list(range(1, 201, 3)) + [132, 133, 134, 196, 197, 255, 256, 257]:
        K = np.array([raw[t] if (t < 4 or t >= n - 128) else decoded[t] for t in range(n)])
        ref_o, ref_l = _brute_attention(K, q, SCALE)
        out, lse = oracle.decode_sequence(rows_all[:n], q, SCALE, bits_c)
        np.testing.assert_allclose(out, ref_o, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(lse, ref_l, rtol=1e-12)


# ----------------------------------------------------------------- P7: split / merge identity
def test_split_merge_identity():
    """LSE merge of attention over any partition of tokens equals attention over all of them."""
    n = 1500
    rows = mi.rows(15, 0, n)
    q = mi.queries(15, 1, 3)[0]
    cc, cr, meta = oracle.quantize(rows, 2)
    sel = oracle.select(rows, cc, cr, meta, 2)
    full_o, full_l = oracle.attend(sel, q, SCALE)
    cuts = [0, 1, 64, 700, 701, 1436, n]
    parts = [oracle.attend(sel[a:b], q, SCALE) for a, b in zip(cuts[:-1], cuts[1:])]
    L = np.logaddexp.reduce(np.stack([p[1] for p in parts]), axis=0)
    o = sum(np.exp(p[1] - L)[:, None] * p[0] for p in parts)
    np.testing.assert_allclose(L, full_l, rtol=1e-13)
    np.testing.assert_allclose(o, full_o, rtol=1e-11, atol=1e-11)


def test_identical_tokens_closed_form():
    """All tokens equal: uniform weights, output = the row's content part, lse = score + ln N."""
    n = 900
    row = mi.rows(16, 0, 1)
    rows = np.repeat(row, n, axis=0)
    q = mi.queries(16, 1, 2)[0]
    out, lse = oracle.decode_sequence(rows, q, SCALE, 4)
    cc, cr, meta = oracle.quantize(rows, 4)
    sel = oracle.select(rows, cc, cr, meta, 4)
    # packed tokens dequantize to one value, BF16 tokens keep another: two-point closed form
    raw = _f(row)[0]
    deq = sel[500]
    n_bf = 4 + 128
    qf = _f(q)
    for h in range(2):
        s_raw, s_deq = SCALE * qf[h] @ raw, SCALE * qf[h] @ deq
        m = max(s_raw, s_deq)
        l = n_bf * math.exp(s_raw - m) + (n - n_bf) * math.exp(s_deq - m)
        ref = (n_bf * math.exp(s_raw - m) * raw[:512] + (n - n_bf) * math.exp(s_deq - m) * deq[:512]) / l
        np.testing.assert_allclose(out[h], ref, rtol=1e-11, atol=1e-11)
        assert abs(lse[h] - (m + math.log(l))) < 1e-11


# ----------------------------------------------------------------- O4: sink and recent-ring contents
# The writer keeps the bf16 rows of the first n_sink tokens and of the most recent n_recent tokens
# (onedev.kr review, "How it is used"), the ring row of position p being p mod n_recent.  The maps
# below were worked out by hand for each (N, n_recent) and are written as segments
# (first ring row, last ring row, position held by the first row); a segment's rows hold
# consecutive positions.
RING_MAPS = {
    (1, 1): [(0, 0, 0)],
    (4, 1): [(0, 0, 3)],
    (5, 1): [(0, 0, 4)],
    (131, 1): [(0, 0, 130)],
    (132, 1): [(0, 0, 131)],
    (133, 1): [(0, 0, 132)],
    (300, 1): [(0, 0, 299)],
    (1, 3): [(0, 0, 0)],
    (4, 3): [(0, 0, 3), (1, 2, 1)],                    # positions 1, 2, 3
    (5, 3): [(0, 1, 3), (2, 2, 2)],                    # positions 2, 3, 4
    (131, 3): [(0, 1, 129), (2, 2, 128)],              # positions 128, 129, 130
    (132, 3): [(0, 2, 129)],                           # positions 129, 130, 131
    (133, 3): [(0, 0, 132), (1, 2, 130)],              # positions 130, 131, 132
    (300, 3): [(0, 2, 297)],                           # positions 297, 298, 299
    (1, 128): [(0, 0, 0)],
    (4, 128): [(0, 3, 0)],
    (5, 128): [(0, 4, 0)],
    (131, 128): [(0, 2, 128), (3, 127, 3)],            # positions 3 .. 130, wrapped after 127
    (132, 128): [(0, 3, 128), (4, 127, 4)],            # positions 4 .. 131
    (133, 128): [(0, 4, 128), (5, 127, 5)],            # positions 5 .. 132
    (300, 128): [(0, 43, 256), (44, 127, 172)],        # positions 172 .. 299, wrapped after 255
}
SINK_MAPS = {1: [0], 4: [0, 1, 2, 3], 5: [0, 1, 2, 3], 131: [0, 1, 2, 3], 132: [0, 1, 2, 3],
             133: [0, 1, 2, 3], 300: [0, 1, 2, 3]}


@pytest.mark.parametrize("n,n_recent", sorted(RING_MAPS))
def test_bf16_buffers_hand_maps(n, n_recent):
    """The oracle's expected sink and ring rows (the reference for every writer byte test) equal
    the hand-written maps above: which positions are kept, and in which ring row each one sits."""
    rows = np.zeros((n, 576), np.uint16)
    rows[:, 0] = np.arange(n)                 # a row's position, readable from its first channel
    rows[:, 1] = 0x4000 + np.arange(n) % 7    # and some other content
    sink, ring = oracle.bf16_buffers(rows, n_sink=4, n_recent=n_recent)
    expect = {}
    for lo, hi, p0 in RING_MAPS[(n, n_recent)]:
        for k, slot in enumerate(range(lo, hi + 1)):
            expect[slot] = p0 + k
    assert {s: int(r[0]) for s, r in ring.items()} == expect
    for s, r in ring.items():
        assert np.array_equal(r, rows[expect[s]])
    assert {i: int(r[0]) for i, r in sink.items()} == {i: i for i in SINK_MAPS[n]}
    assert oracle.bf16_buffers(rows, n_sink=0, n_recent=n_recent)[0] == {}

"""Pins of the oracle's interleaved KV-cache write with FP8 quantisation
(CPU only).  The E4M3FN encoder is checked against the bit definition (round
trip over every code, ties to even at every midpoint), against torch's own
float8_e4m3fn conversion (a library routine used only as a check), and the
per-token quantisation against its error bound and two examples worked by
hand (one where multiplying by the inverse scale and dividing by the scale
give different codes, which pins the reading taken); the write against
placements stated by hand (slot 5 of a 2-shard pool is shard 1, row 2), a
write read back through the remap and the single-token closed form of the
attention, and a brute-force check that nothing else moves."""

import numpy as np
import pytest
import torch

import oracle

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def bf16_bits(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_encode_round_trips_every_code():
    vals = oracle.decode_e4m3fn(FINITE).astype(np.float32)
    np.testing.assert_array_equal(oracle.encode_e4m3fn(vals), FINITE)


def test_encode_ties_to_even_and_neighbours_of_midpoints():
    pos = [c for c in range(0x00, 0x7E)]             # adjacent positive pairs (c, c + 1)
    for c in pos:
        lo, hi = oracle.decode_e4m3fn(np.array([c, c + 1], dtype=np.uint8))
        mid = np.float32((lo + hi) / 2)               # exact in fp32
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.encode_e4m3fn([mid])[0] == even, hex(c)
        assert oracle.encode_e4m3fn([-mid])[0] == even | 0x80, hex(c)
        above = np.nextafter(mid, np.float32(np.inf), dtype=np.float32)
        below = np.nextafter(mid, np.float32(-np.inf), dtype=np.float32)
        assert oracle.encode_e4m3fn([above])[0] == c + 1
        assert oracle.encode_e4m3fn([below])[0] == c


def test_encode_matches_torch_conversion_in_range():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 1, 20000),
                        rng.normal(0, 2.0 ** -7, 20000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.encode_e4m3fn(x), ref)


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.encode_e4m3fn([449.0])
    with pytest.raises(ValueError):
        oracle.encode_e4m3fn([np.nan])


def test_quantize_row_scale_and_error_bound():
    rng = np.random.default_rng(6)
    for trial in range(50):
        x = (rng.normal(0, 1, 576) * 2.0 ** rng.uniform(-8, 8)).astype(np.float32)
        bits = bf16_bits(x)
        xv = oracle.decode_bf16(bits)
        codes, scale = oracle.quantize_row_e4m3(bits)
        assert scale.dtype == np.float32
        amax = np.float32(np.max(np.abs(xv)))
        assert scale == np.float32(amax / np.float32(448.0))
        # the largest magnitude maps to the largest code
        k = int(np.argmax(np.abs(xv)))
        assert codes[k] & 0x7F == 0x7E
        # dequantised values are within half an E4M3 step (plus the fp32
        # rounding of the quotient) of the inputs
        deq = oracle.decode_e4m3fn(codes) * np.float64(scale)
        qa = np.abs(xv) / np.float64(scale)               # magnitude on the E4M3 grid
        step = np.float64(scale) * np.where(
            qa < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(qa, 1e-300))) - 3))
        assert np.all(np.abs(deq - xv) <= 0.5 * step * (1 + 2.0 ** -20) + 2.0 ** -24 * np.abs(xv))
        assert np.all(np.signbit(deq[xv != 0]) == np.signbit(xv[xv != 0]))


def test_quantize_all_zero_row():
    codes, scale = oracle.quantize_row_e4m3(np.zeros(576, dtype=np.uint16))
    assert scale == np.float32(1.0) and not codes.any()


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_kv_write_places_every_slot_by_brute_force(n, kv):
    rng = np.random.default_rng(10 + n)
    rows = 40
    if kv == "bf16":
        pools = [rng.integers(0, 1 << 16, (rows, 576)).astype(np.uint16) for _ in range(n)]
        scales = [None] * n
    else:
        pools = [rng.integers(0, 0x7F, (rows, 576)).astype(np.uint8) for _ in range(n)]
        scales = [rng.uniform(0.1, 1, rows).astype(np.float32) for _ in range(n)]
    t = 25
    slots = rng.choice(n * rows, size=t, replace=False).astype(np.int32)
    slots[[3, 17]] = -1                                   # skipped tokens
    new = bf16_bits(rng.normal(0, 3, (t, 576)))
    out_p, out_s = oracle.kv_write(new, slots, n, pools, scales, kv)
    written = set()
    for i, g in enumerate(slots):
        if g < 0:
            continue
        r, row = g % n, g // n
        written.add((r, row))
        if kv == "bf16":
            np.testing.assert_array_equal(out_p[r][row], new[i])
        else:
            codes, sc = oracle.quantize_row_e4m3(new[i])
            np.testing.assert_array_equal(out_p[r][row], codes)
            assert out_s[r][row] == sc
    for r in range(n):
        for row in range(rows):
            if (r, row) not in written:
                np.testing.assert_array_equal(out_p[r][row], pools[r][row])
                if kv == "fp8":
                    assert out_s[r][row] == scales[r][row]


def _golden(name):
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        return json.load(f)


def _check_worked_example(ex):
    x = np.zeros(576, dtype=np.float32)
    x[:len(ex["values"])] = ex["values"]
    bits = bf16_bits(x)
    assert (oracle.decode_bf16(bits)[:len(ex["values"])] == np.array(ex["values"])).all()  # exact in bf16
    codes, scale = oracle.quantize_row_e4m3(bits)
    assert format(int(np.float32(scale).view(np.uint32)), "08x") == ex["scale_bits_hex"]
    np.testing.assert_array_equal(codes[:len(ex["codes"])], np.array(ex["codes"], dtype=np.uint8))
    assert (codes[len(ex["codes"]):] == ex["rest_code"]).all()


def test_quantize_matches_hand_worked_example():
    # tests/golden/kv_write_worked_example.json: codes derived by hand from the
    # E4M3FN bit definition (exact products, two ties to even, subnormals)
    _check_worked_example(_golden("kv_write_worked_example.json"))


def test_quantize_multiplies_by_the_inverse_scale():
    # tests/golden/kv_write_product_vs_division.json: amax 3.875, so neither
    # the scale nor its inverse is a power of two; x = 1.453125 times the fp32
    # inverse scale is exactly 168, a tie that goes to 0x72, while x divided
    # by the fp32 scale lands just above 168 and would give 0x73
    ex = _golden("kv_write_product_vs_division.json")
    _check_worked_example(ex)
    assert ex["codes"] != ex["codes_if_divided_by_scale"]


# Placements stated by hand: (shards, slot) -> (shard, row).  Interleave 1
# means consecutive slots go round the shards: with two shards slots 0, 2, 4
# are rows 0, 1, 2 of shard 0 and slots 1, 3, 5 rows 0, 1, 2 of shard 1.
HAND_PLACEMENT = {
    (2, 0): (0, 0), (2, 1): (1, 0), (2, 5): (1, 2), (2, 6): (0, 3), (2, 11): (1, 5),
    (3, 5): (2, 1), (3, 9): (0, 3), (3, 10): (1, 3),
    (4, 6): (2, 1), (4, 13): (1, 3), (4, 15): (3, 3),
}


def test_kv_write_hand_stated_placement():
    rows = 8
    for (n, g), (r_exp, row_exp) in HAND_PLACEMENT.items():
        pools = [np.zeros((rows, 576), dtype=np.uint16) for _ in range(n)]
        new = np.full((1, 576), 0x3F80, dtype=np.uint16)          # bf16 1.0 everywhere
        out_p, _ = oracle.kv_write(new, np.array([g], dtype=np.int32), n, pools, [None] * n, "bf16")
        hit = [(r, row) for r in range(n) for row in range(rows) if out_p[r][row].any()]
        assert hit == [(r_exp, row_exp)], (n, g, hit)


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_kv_write_then_read_back(kv):
    # A token written at slot 5 of a 2-shard cache is read back by the remap
    # (shard 1, local id 2, count 1; shard 0 empty) and by the attention of a
    # row that selects only that slot: with one token, O is its value and the
    # LSE is its logit.
    rng = np.random.default_rng(21)
    n, rows, sigma = 2, 6, 1.0 / np.sqrt(192.0)
    if kv == "bf16":
        pools = [rng.integers(0, 1 << 16, (rows, 576)).astype(np.uint16) & 0xBFFF for _ in range(n)]
        scales = [None] * n
    else:
        pools = [rng.integers(0, 0x7F, (rows, 576)).astype(np.uint8) for _ in range(n)]
        scales = [rng.uniform(0.1, 1, rows).astype(np.float32) for _ in range(n)]
    x = bf16_bits(rng.normal(0, 2, (1, 576)))
    out_p, out_s = oracle.kv_write(x, np.array([5], dtype=np.int32), n, pools, scales, kv)
    local, counts = oracle.remap_topk(np.array([[-1, 5, -1]], dtype=np.int32), n)
    assert counts.tolist() == [[0], [1]]
    assert local[1, 0].tolist() == [2, -1, -1] and local[0, 0].tolist() == [-1, -1, -1]
    if kv == "bf16":
        val = oracle.decode_bf16(x[0])
    else:
        codes, sc = oracle.quantize_row_e4m3(x[0])
        val = oracle.decode_e4m3fn(codes) * np.float64(sc)
    q = oracle.decode_bf16(bf16_bits(rng.normal(0, 1, (1, 3, 576))))
    o, lse = oracle.sparse_attn_shard(q, out_p[1], kv, out_s[1], local[1], counts[1], sigma)
    np.testing.assert_array_equal(o[0], np.broadcast_to(val[:512], (3, 512)))
    np.testing.assert_allclose(lse[0], sigma * (q[0] @ val), rtol=0, atol=1e-12)
    o0, lse0 = oracle.sparse_attn_shard(q, out_p[0], kv, out_s[0], local[0], counts[0], sigma)
    assert (o0 == 0).all() and (lse0 == -np.inf).all()

"""Pins of the oracle's interleaved KV-cache write with FP8 quantisation
(CPU only).  The E4M3FN encoder is checked against the bit definition (round
trip over every code, ties to even at every midpoint), against torch's own
float8_e4m3fn conversion (a library routine used only as a check), and the
per-token quantisation against its error bound; the write against a brute-force
placement: slot g lands in row g div N of shard g mod N and nothing else moves."""

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


def test_quantize_matches_hand_worked_example():
    # tests/golden/kv_write_worked_example.json: codes derived by hand from the
    # E4M3FN bit definition (exact products, two ties to even, subnormals)
    import json
    import os
    ex = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_write_worked_example.json")))
    x = np.zeros(576, dtype=np.float32)
    x[:len(ex["values"])] = ex["values"]
    bits = bf16_bits(x)
    assert (oracle.decode_bf16(bits)[:len(ex["values"])] == np.array(ex["values"])).all()  # exact in bf16
    codes, scale = oracle.quantize_row_e4m3(bits)
    assert format(int(np.float32(scale).view(np.uint32)), "08x") == ex["scale_bits_hex"]
    np.testing.assert_array_equal(codes[:len(ex["codes"])], np.array(ex["codes"], dtype=np.uint8))
    assert (codes[len(ex["codes"]):] == ex["rest_code"]).all()

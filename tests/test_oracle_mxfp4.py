"""Pins for the oracle's MXFP4 decoder against the OCP MX v1.0 e2m1 table (CPU only)."""
import os

import numpy as np
import pytest

from oracle import bf16_to_f64, mxfp4_dequant
from synthetic import f32_to_bf16_bits, quantise_mxfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _table():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_table.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                c, v = line.split()
                vals[int(c, 16)] = float(v)
    assert len(vals) == 16
    return vals


@pytest.mark.parametrize("scale_byte", [0, 1, 100, 121, 127, 128, 140, 254])
def test_every_code_every_position(scale_byte):
    tab = _table()
    # 32 k-values per block: byte j holds k=2j (low nibble) and k=2j+1 (high nibble)
    codes = np.arange(32) % 16
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)[None, :]
    deq = mxfp4_dequant(packed, np.array([[scale_byte]], np.uint8))[0]
    want = np.array([tab[c] for c in codes]) * 2.0 ** (scale_byte - 127)
    np.testing.assert_array_equal(deq, want)
    # -0.0 must stay a zero
    assert deq[8] == 0.0


def test_nibble_order_and_block_scales():
    # byte 0x71: k=0 -> code 1 (0.5), k=1 -> code 7 (6.0); second block scaled by 2^1
    packed = np.zeros((1, 32), np.uint8)
    packed[0, 0] = 0x71
    packed[0, 16] = 0x2A          # k=32 -> code 0xA (-1.0), k=33 -> code 2 (1.0)
    deq = mxfp4_dequant(packed, np.array([[127, 128]], np.uint8))[0]
    assert deq[0] == 0.5 and deq[1] == 6.0 and deq[32] == -2.0 and deq[33] == 2.0
    assert np.count_nonzero(deq) == 4


def test_quantise_dequantise_error_bound():
    # values round to the nearest e2m1 step: error <= half the local grid spacing
    # (0.25 * 2^X below 2, up to 1 * 2^X below 6); the shared-exponent rule
    # X = floor(log2 amax) - 2 puts the block maximum in [4, 8) * 2^X, so values above
    # 6 * 2^X saturate to 6 * 2^X (the specification's clamp)
    rng = np.random.default_rng(0)
    w = f32_to_bf16_bits(rng.standard_normal((64, 256)).astype(np.float32) * 0.02)
    q, s = quantise_mxfp4(w)
    deq = mxfp4_dequant(q, s)
    v = bf16_to_f64(w)
    X = (s.astype(np.float64) - 127).repeat(32, axis=1)
    step = np.where(np.abs(v) / 2 ** X >= 4, 2.0, np.where(np.abs(v) / 2 ** X >= 2, 1.0, 0.5))
    r = np.abs(v) / 2 ** X
    bound = np.where(r > 6, r - 6, 0.5 * step) * 2 ** X
    assert np.all(np.abs(deq - v) <= bound)
    assert np.all(np.abs(deq[r > 6]) == 6 * 2 ** X[r > 6])
    # the shared exponent keeps every block maximum below 8 * 2^X
    assert np.all(np.abs(v).reshape(64, 8, 32).max(2) / 2 ** (s.astype(np.float64) - 127) < 8)


def test_quantise_is_identity_on_representable_values():
    # dequantised values re-quantise to the same codes and scales
    rng = np.random.default_rng(1)
    w = f32_to_bf16_bits(rng.standard_normal((16, 128)).astype(np.float32) * 0.02)
    q, s = quantise_mxfp4(w)
    deq = mxfp4_dequant(q, s).astype(np.float32)
    q2, s2 = quantise_mxfp4(f32_to_bf16_bits(deq))
    np.testing.assert_array_equal(s2, s)
    np.testing.assert_array_equal(q2, q)


def test_dequant_exact_in_bf16():
    # every dequantised weight of an N(0, 0.02) tensor is exactly a bf16 value
    rng = np.random.default_rng(2)
    w = f32_to_bf16_bits(rng.standard_normal((32, 512)).astype(np.float32) * 0.02)
    deq = mxfp4_dequant(*quantise_mxfp4(w))
    np.testing.assert_array_equal(bf16_to_f64(f32_to_bf16_bits(deq.astype(np.float32))), deq)

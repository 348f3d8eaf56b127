"""Pins for the oracle's decoders and data layout (CPU only)."""
import os

import numpy as np
import torch

from oracle import (E2M1_TABLE, e2m1_decode, e4m3_decode, pack_nibbles,
                    quantize_ref, unpack_nibbles)
from tests.indep import e2m1_fraction, unpack_by_hand

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e2m1_table_matches_bit_fields():
    # 16-entry table vs the E2M1 bit-field formula (bias 1), two derivations
    for n in range(16):
        assert E2M1_TABLE[n] == float(e2m1_fraction(n)), n
        assert e2m1_decode(n) == float(e2m1_fraction(n))
    assert list(E2M1_TABLE[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_e4m3_decode_matches_torch_all_bytes():
    codes = np.arange(256)
    ours = e4m3_decode(codes)
    t = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn)
    ref = t.to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.all(both_nan | (ours == ref))
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    # signed zeros agree too
    assert np.array_equal(np.signbit(ours[~np.isnan(ours)]), np.signbit(ref[~np.isnan(ref)]))


def test_e4m3_landmarks():
    d = lambda b: float(e4m3_decode(b))  # noqa: E731
    assert d(0x38) == 1.0
    assert d(0x7E) == 448.0
    assert d(0x01) == 2.0 ** -9
    assert d(0x08) == 2.0 ** -6
    assert d(0x07) == 7 * 2.0 ** -9
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x80) == 0.0 and np.signbit(d(0x80))
    assert d(0xB8) == -1.0


def test_pack_order_low_nibble_first():
    rng = np.random.default_rng(1)
    nib = rng.integers(0, 16, size=(5, 64)).astype(np.uint8)
    q = pack_nibbles(nib)
    assert np.array_equal(unpack_by_hand(q), nib)
    assert np.array_equal(unpack_nibbles(q), nib)
    assert pack_nibbles(np.array([[0x3, 0xA]], dtype=np.uint8))[0, 0] == 0xA3


def _golden_workload():
    vals = {}
    with open(os.path.join(GOLDEN, "kernelindex_nvfp4_linear_workload.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                vals[k] = int(v)
    return vals


def test_layout_matches_page_workload_parameters():
    # in_features_half and sf_k printed on the page pin "two values per byte"
    # and "one scale per sf_vec_size = 16 elements" for the operand layout
    wl = _golden_workload()
    K = wl["in_features"]
    x = np.linspace(-3, 3, 2 * K, dtype=np.float32).reshape(2, K)
    q, s, g = quantize_ref(x)
    assert q.shape == (2, wl["in_features_half"])
    assert s.shape == (2, wl["sf_k"])
    assert K // wl["sf_vec_size"] == wl["sf_k"]
    assert wl["out_features"] == 8192

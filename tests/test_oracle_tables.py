"""Pins for the oracle's code tables and encoders (CPU only).

The oracle's E4M3 / E2M1 / bf16 decoders and its E4M3 encoder are checked
against the format definitions' fixed points and against torch's own float8
and bfloat16 conversions (library routines, run not read)."""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_fixed_points():
    t = oracle.e4m3_table()
    assert t.shape == (256,)
    assert t[0x00] == 0.0 and not math.copysign(1, t[0x00]) < 0
    assert t[0x80] == 0.0 and math.copysign(1, t[0x80]) < 0
    nan_codes = [c for c in range(256) if math.isnan(t[c])]
    assert nan_codes == [0x7F, 0xFF]
    assert t[0x7E] == 448.0
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert t[0x38] == 1.0
    assert t[0x20] == 0.125
    assert t[0x5F] == 30.0
    pos = t[0x00:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must be strictly increasing"
    for c in range(0x7F):
        assert t[c | 0x80] == -t[c]


def test_e4m3_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t = oracle.e4m3_table()
    both_nan = np.isnan(ref) & np.isnan(t)
    assert np.array_equal(np.isnan(ref), np.isnan(t))
    assert np.array_equal(ref[~both_nan], t[~both_nan])
    # signed zeros too
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(t[~both_nan]))


def test_e2m1_matches_ocp_values():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_values.txt"))
            if l.strip() and not l.startswith("#")]
    t = oracle.e2m1_table()
    for code, val in rows:
        v = float(val)
        assert t[int(code)] == v
        assert math.copysign(1, t[int(code)]) == math.copysign(1, v)


def test_bf16_decode_matches_torch_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    sample = np.concatenate([np.arange(0, 65536, 97), [0, 0x8000, 0x7F7F, 0x0001, 0x3F80]])
    for b in sample:
        v = oracle.bf16_value(int(b))
        r = ref[b]
        if math.isnan(r):
            assert math.isnan(v)
        else:
            assert v == r


def _encode_ref(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_round_trips_every_finite_code():
    t = oracle.e4m3_table()
    finite = [c for c in range(256) if not math.isnan(t[c])]
    vals = np.array([t[c] for c in finite], np.float32)
    enc = oracle.e4m3_encode(vals)
    assert list(enc) == finite


def test_e4m3_encode_matches_torch_rne_in_range():
    t = oracle.e4m3_table()
    pos = t[0:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2.0  # exact ties: must go to the even code
    rng = np.random.default_rng(5)
    rand = rng.uniform(-447.9, 447.9, 4000)
    small = rng.uniform(-0.02, 0.02, 2000)
    v = np.concatenate([mids, -mids, rand, small, np.nextafter(mids, 0), np.nextafter(mids, 1000)])
    v = v.astype(np.float32)
    v = v[np.abs(v) < 464.0]
    got = oracle.e4m3_encode(v)
    ref = _encode_ref(v)
    assert np.array_equal(got, ref)
    # ties: even mantissa (lowest code bit 0)
    tie_codes = oracle.e4m3_encode(mids.astype(np.float32))
    assert np.all(tie_codes % 2 == 0)


def test_e4m3_encode_saturates():
    v = np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e30, -600.0], np.float32)
    got = oracle.e4m3_encode(v)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]

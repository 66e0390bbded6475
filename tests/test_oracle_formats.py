"""Pins of the oracle's storage decoders against library routines and the
published FP4 table (no GPU)."""
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_all_codes_match_torch(orc):
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = codes.view(torch.bfloat16).double().numpy()
    got = np.array([orc.decode_bf16(c) for c in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    # signed zero kept
    assert math.copysign(1.0, orc.decode_bf16(0x8000)) == -1.0


def test_e4m3_all_codes_match_torch(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([orc.decode_e4m3(c) for c in range(256)])
    nan = np.isnan(ref)
    assert nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert orc.decode_e4m3(0x7E) == 448.0
    assert orc.decode_e4m3(0x01) == 2.0 ** -9


def test_e2m1_matches_published_table(orc):
    table = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            table[int(code)] = float(val)
    assert sorted(table) == list(range(16))
    for code, val in table.items():
        got = orc.decode_e2m1(code)
        assert got == val and math.copysign(1.0, got) == math.copysign(1.0, val), code


def test_fp4_products_exact_in_bf16(orc):
    """Every E2M1 value times every finite E4M3 scale is exactly a bfloat16,
    so dequantising to bf16 loses nothing."""
    e2 = np.array([orc.decode_e2m1(c) for c in range(16)])
    e4 = np.array([orc.decode_e4m3(c) for c in range(256)])
    e4 = e4[~np.isnan(e4)]
    prod = torch.tensor(np.outer(e2, e4), dtype=torch.float64)
    assert torch.equal(prod.to(torch.bfloat16).double(), prod)


def test_fp4_encoder_roundtrip(orc):
    """The input generator's FP4 encoder produces codes whose decoded values
    are within half a grid step of the drawn values (sanity of generation)."""
    import synth

    x = synth.normal((64, 32), seed=5)
    codes, scales = synth.fp4_encode(x)
    dec = np.zeros((64, 32))
    for r in range(64):
        for c in range(32):
            byte = int(codes[r, c // 2])
            nib = byte & 15 if c % 2 == 0 else byte >> 4
            dec[r, c] = orc.decode_e2m1(nib) * orc.decode_e4m3(int(scales[r, c // 16]))
    scale = np.array([[orc.decode_e4m3(int(s)) for s in row] for row in scales.numpy()])
    step = np.repeat(scale, 16, axis=1) * 1.0  # largest E2M1 gap is 2 (4 -> 6)
    assert np.all(np.abs(dec - x.numpy()) <= step + 1e-6)

"""Pins for the oracle's number-format decoders and its E4M3FN encoder.

Each decoder is checked exhaustively against a library conversion (numpy's
binary16, torch's bfloat16 and float8_e4m3fn) and against named points of the
format's definition; the encoder against torch's round-to-nearest-even cast
wherever that cast does not overflow, and against the saturation rule above.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from conftest import GOLDEN


def _same(a, b):
    return (math.isnan(a) and math.isnan(b)) or (a == b and math.copysign(1, a) == math.copysign(1, b))


def test_f16_decoder_exhaustive():
    codes = np.arange(65536, dtype=np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    for c in range(65536):
        assert _same(oracle.f16_to_f64(c), float(ref[c])), hex(c)


def test_bf16_decoder_exhaustive():
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = codes.view(torch.bfloat16).to(torch.float64).numpy()
    for c in range(65536):
        assert _same(oracle.bf16_to_f64(c), float(ref[c])), hex(c)


def test_e4m3_decoder_exhaustive_and_named_points():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        assert _same(oracle.e4m3_to_f64(c), float(ref[c])), hex(c)
    pts = json.load(open(os.path.join(GOLDEN, "e4m3fn_points.json")))["points"]
    for p in pts:
        got = oracle.e4m3_to_f64(int(p["code"], 16))
        want = float("nan") if p["value"] == "nan" else float(p["value"])
        assert _same(got, want), p


def _e4m3_grid():
    return sorted({oracle.e4m3_to_f64(c) for c in range(0x7F)})


def test_e4m3_encoder_matches_rne_cast():
    # every bf16 magnitude up to 464 (beyond which torch's cast gives NaN)
    b = torch.arange(0, 0x7F80, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
    b = b[b <= 464.0]
    # midpoints between consecutive E4M3 values and their fp32 neighbours
    g = np.asarray(_e4m3_grid(), dtype=np.float64)
    mids = ((g[1:] + g[:-1]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    x = torch.cat([b, torch.from_numpy(near), torch.tensor([2.0 ** -12, 2.0 ** -10, 1e-30, 0.0])])
    x = torch.cat([x, -x])
    want = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    xs = x.numpy()
    for i in range(xs.shape[0]):
        assert oracle.f32_to_e4m3(float(xs[i])) == int(want[i]), (float(xs[i]), hex(want[i]))


def test_e4m3_encoder_saturates():
    for v in [464.0001, 480.0, 500.0, 1e6, 3.0e38, float("inf")]:
        assert oracle.f32_to_e4m3(v) == 0x7E
        assert oracle.f32_to_e4m3(-v) == 0xFE
    assert oracle.f32_to_e4m3(float("nan")) == 0x7F


def test_e4m3_encoder_exact_on_grid():
    for c in range(0x7F):
        v = oracle.e4m3_to_f64(c)
        assert oracle.f32_to_e4m3(v) == c
        if c:
            assert oracle.f32_to_e4m3(-v) == 0x80 | c

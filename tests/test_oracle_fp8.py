"""Pins of the oracle's E4M3 codec against the format definition and torch's CPU cast."""
import json
import os

import numpy as np
import pytest
import torch

from oracle.fp8 import e4m3_decode, e4m3_encode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_e4m3_landmarks.json")


def _torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, np.uint8).copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy().astype(np.float64)


def _torch_encode(x32):
    t = torch.from_numpy(np.asarray(x32, np.float32).copy()).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_decode_landmarks_from_format_definition():
    g = json.load(open(GOLDEN))
    for item in g["decode"]:
        v = e4m3_decode(np.array([int(item["code"], 16)], np.uint8))[0]
        if item["value"] == "nan":
            assert np.isnan(v)
        else:
            assert v == item["value"]
            assert np.signbit(v) == np.signbit(item["value"])


def test_decode_all_256_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    ref = _torch_decode(codes)
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.all(both_nan | (ours == ref))
    assert np.isnan(ours).sum() == 2


def test_encode_landmarks_round_to_nearest_even():
    g = json.load(open(GOLDEN))
    for item in g["encode_round_to_nearest_even"]:
        c = e4m3_encode(np.array([item["x"]], np.float32))[0]
        assert c == int(item["code"], 16), item


def test_encode_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(e4m3_encode(vals), codes)


def test_encode_matches_torch_on_midpoints_and_neighbours():
    pos = e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)          # exact in fp32
    assert np.all(mids.astype(np.float64) == (pos[1:] + pos[:-1]) / 2)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    x = np.concatenate([near, -near, pos.astype(np.float32)])
    assert np.array_equal(e4m3_encode(x), _torch_encode(x))


def test_encode_matches_torch_on_random_values():
    rng = np.random.default_rng(11)
    mag = np.exp2(rng.uniform(-14, np.log2(464.0), size=400_000))
    x = (mag * rng.choice([-1.0, 1.0], size=mag.size)).astype(np.float32)
    x = x[np.abs(x) <= 464]
    assert np.array_equal(e4m3_encode(x), _torch_encode(x))


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        e4m3_encode(np.array([465.0], np.float32))
    with pytest.raises(ValueError):
        e4m3_encode(np.array([np.nan], np.float32))

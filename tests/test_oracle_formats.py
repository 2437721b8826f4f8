"""Pins for the oracle's storage decoders: torch's own dtype decoders and the OCP FP8 table."""
import os

import numpy as np
import torch

from oracle import formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_decoder_matches_torch_all_codes():
    codes = np.arange(1 << 16, dtype=np.uint16)
    ours = formats.bf16_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_decoder_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = formats.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all() and nan.sum() == 2
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3_decoder_matches_ocp_table():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "ocp_e4m3_codes.txt")) if l.strip() and not l.startswith("#")]
    codes = np.array([int(c, 16) for c, _ in rows], dtype=np.uint8)
    want = np.array([float(v) for _, v in rows])
    got = formats.e4m3_to_f64(codes)
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all()
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    # include exact ties (bit 15 set, lower bits clear) to exercise round-half-even
    ties = (rng.integers(0, 1 << 31, 5000, dtype=np.uint32) & np.uint32(0x7F7F0000)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32), np.zeros(1, np.float32)])
    x = x[np.isfinite(x) & ((np.abs(x) >= 2.0 ** -126) | (x == 0))]
    ours = formats.f64_to_bf16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e2m1_decoder_matches_ocp_table():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "ocp_e2m1_codes.txt")) if l.strip() and not l.startswith("#")]
    codes = np.array([int(c, 16) for c, _ in rows], dtype=np.uint8)
    want = np.array([float(v) for _, v in rows])
    assert len(codes) == 16
    got = formats.e2m1_to_f64(codes)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))
    # only the low nibble is read
    assert np.array_equal(formats.e2m1_to_f64(codes | np.uint8(0xF0)), want)


def test_e8m0_decoder_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = formats.e8m0_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 1 and nan[255] and np.isnan(ours[255])
    assert np.array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


def test_mxfp4_element_order_and_block_scales():
    # one 64-element row: byte i holds element 2i (low nibble) and 2i+1 (high nibble)
    packed = np.zeros((1, 32), dtype=np.uint8)
    packed[0, 0] = 0x21          # e0 = 0.5, e1 = 1.0
    packed[0, 15] = 0xF7         # e30 = 6, e31 = -6
    packed[0, 16] = 0x3C         # e32 = -2, e33 = 1.5
    scales = np.array([[127 - 3, 127 + 5]], dtype=np.uint8)
    v = formats.mxfp4_to_f64(packed, scales)
    assert v.shape == (1, 64)
    want = np.zeros(64)
    want[0], want[1], want[30], want[31] = 0.5 / 8, 1.0 / 8, 6.0 / 8, -6.0 / 8
    want[32], want[33] = -2.0 * 32, 1.5 * 32
    assert np.array_equal(v[0], want)


def test_mxfp4_value_set():
    # every element value is a signed E2M1 magnitude times a power of two from its block
    rng = np.random.default_rng(3)
    packed = rng.integers(0, 256, (50, 64), dtype=np.uint8)
    scales = rng.integers(100, 150, (50, 4), dtype=np.uint8)
    v = formats.mxfp4_to_f64(packed, scales)
    mags = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}
    for r in range(50):
        for d in range(128):
            x = abs(v[r, d]) / 2.0 ** (int(scales[r, d // 32]) - 127)
            assert x in mags

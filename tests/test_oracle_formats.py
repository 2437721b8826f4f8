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

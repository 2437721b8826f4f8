"""Pins of the KV-write oracle: the e4m3 encoder against the OCP code table, torch's own
e4m3 cast and exhaustive round trips; the key quantization against its error bound and
special cases; the scatter against its invariants."""
import os

import numpy as np
import torch

from oracle import formats as of, kvwrite as okw
from oracle import paging as opg

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ocp_e4m3_codes.txt")


def _golden():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            c, v = line.split()
            out.append((int(c, 16), float(v)))
    return out


def test_encoder_matches_ocp_table():
    for code, value in _golden():
        if np.isnan(value):
            continue
        assert of.f64_to_e4m3_codes(np.array([value]))[0] == code, (hex(code), value)
        if value > 0:
            assert of.f64_to_e4m3_codes(np.array([-value]))[0] == code | 0x80


def test_encoder_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(of.f64_to_e4m3_codes(of.e4m3_to_f64(codes)), codes)


def test_encoder_ties_go_to_even_and_saturate():
    pos = of.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    mid = (pos[:-1] + pos[1:]) / 2
    got = of.f64_to_e4m3_codes(mid)
    lo = np.arange(0x7E)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8))
    assert (of.f64_to_e4m3_codes(np.array([448.0 * (1 + 2.0 ** -20), 464.0, 1e6, -1e6])) == [0x7E, 0x7E, 0x7E, 0xFE]).all()


def test_encoder_matches_torch_cast_in_range():
    rng = np.random.default_rng(11)
    mag = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 200_000))
    x = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(of.f64_to_e4m3_codes(x.astype(np.float64)), ref)


def test_quantize_key_bound_and_extremes():
    rng = np.random.default_rng(5)
    for scale in (1e-3, 1.0, 37.0):
        k = (rng.standard_normal((64, 128)) * scale).astype(np.float32)
        for row in k:
            codes, sigma = okw.quantize_key(row)
            deq = of.e4m3_to_f64(codes) * float(sigma)
            # nearest e4m3: half a mantissa step (2^-4 relative) for normals, half the
            # subnormal step (2^-10) below 2^-6; sigma and k/sigma add float32 rounding
            bound = 2.0 ** -4 * np.abs(row) * (1 + 2.0 ** -20) + float(sigma) * 2.0 ** -10 * (1 + 2.0 ** -20)
            assert (np.abs(deq - row) <= bound).all()
            j = int(np.argmax(np.abs(row)))
            assert codes[j] & 0x7F == 0x7E                    # the largest |k| maps to +-448
            assert float(sigma) == float(np.float32(np.max(np.abs(row)) / np.float32(448)))


def test_quantize_key_zero_and_single_element():
    codes, sigma = okw.quantize_key(np.zeros(128, np.float32))
    assert sigma == 0 and not codes.any()
    k = np.zeros(128, np.float32)
    k[7] = -2.5
    codes, sigma = okw.quantize_key(k)
    assert codes[7] == 0xFE and not np.delete(codes, 7).any() and np.float32(sigma) == np.float32(2.5 / 448)


def test_kv_write_scatter_invariants():
    rng = np.random.default_rng(2)
    B, Sq, ps, P, D = 3, 4, 16, 6, 128
    rows = 512
    pt = rng.permutation(rows // ps)[: B * P].reshape(B, P).astype(np.int32)
    pt[2, 5] = -1                                            # a page that is not allocated
    seq_lens = np.array([37, 4, 96], dtype=np.int32)         # request 2 writes positions 92..95 -> page 5
    lat = rng.integers(0, 65535, (B, Sq, 576), dtype=np.uint16)
    keys = rng.standard_normal((B, Sq, D)).astype(np.float32)
    kv0 = rng.integers(0, 65535, (rows, 576), dtype=np.uint16)
    ic0 = rng.integers(0, 255, (rows, D), dtype=np.uint8)
    is0 = rng.standard_normal(rows).astype(np.float32)
    kv, ic, isc, err = okw.kv_write(lat, keys, seq_lens, pt, ps, kv0, ic0, is0)
    assert err == Sq                                          # request 2's four tokens
    written = set()
    for b in range(2):
        pos = np.arange(seq_lens[b] - Sq, seq_lens[b])
        r = opg.paged_rows(pt[b], pos, ps)
        written |= set(r.tolist())
        assert np.array_equal(kv[r], lat[b])
        for t in range(Sq):
            c, s = okw.quantize_key(keys[b, t])
            assert np.array_equal(ic[r[t]], c) and isc[r[t]] == s
    keep = np.array(sorted(set(range(rows)) - written))
    assert np.array_equal(kv[keep], kv0[keep]) and np.array_equal(ic[keep], ic0[keep])
    assert np.array_equal(isc[keep], is0[keep])

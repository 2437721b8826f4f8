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


# ----------------------------------------------------------------------------- MXFP4 keys
E2M1_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ocp_e2m1_codes.txt")


def _e2m1_table():
    rows = [l.split() for l in open(E2M1_GOLDEN) if l.strip() and not l.startswith("#")]
    return [(int(c, 16), float(v)) for c, v in rows]


def _nearest_e2m1(y):
    """Brute force over the OCP table: the nearest non-negative value, ties to the code with
    an even mantissa bit; the sign bit copied from y."""
    a = abs(float(y))                                # distances in float64
    best = min((abs(v - a), c & 1, c) for c, v in _e2m1_table() if c < 8)
    return best[2] | (8 if np.signbit(y) else 0)


def test_e2m1_rounding_matches_brute_force_nearest():
    vals = [v for c, v in _e2m1_table() if c < 8]
    mids = [(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])]
    grid = np.linspace(-8, 8, 4001)
    for y in list(vals) + mids + [-m for m in mids] + list(grid) + [6.5, 100.0, -1e9, -0.0, 1e-30]:
        assert okw.e2m1_round(np.float32(y)) == _nearest_e2m1(np.float32(y)), y


def test_e2m1_ties_and_saturation_by_hand():
    # ties go to the even mantissa: 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4
    cases = {0.25: 0x0, 0.75: 0x2, 1.25: 0x2, 1.75: 0x4, 2.5: 0x4, 3.5: 0x6, 5.0: 0x6, 5.5: 0x7, 7.0: 0x7,
             -0.1: 0x8, -3.0: 0xD, 0.3: 0x1}
    for y, code in cases.items():
        assert okw.e2m1_round(np.float32(y)) == code, y


def test_mxfp4_quantize_round_trips_representable_blocks():
    rng = np.random.default_rng(9)
    for _ in range(200):
        codes = rng.integers(0, 16, 128).astype(np.uint8)
        shared = rng.integers(-20, 20, 4)
        for j in range(4):                       # the block's largest magnitude is 4 or 6
            codes[32 * j + rng.integers(0, 32)] = rng.choice([0x6, 0x7, 0xE, 0xF])
        scales = (shared + 127).astype(np.uint8)
        packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
        k = of.mxfp4_to_f64(packed[None], scales[None])[0].astype(np.float32)
        p2, s2 = okw.quantize_key_mxfp4(k)
        assert np.array_equal(s2, scales)
        # -0 and +0 both decode to 0.0; compare values, and codes where the value is nonzero
        assert np.array_equal(of.mxfp4_to_f64(p2[None], s2[None])[0], k.astype(np.float64))
        nz = codes & 7 != 0
        got = np.empty(128, np.uint8)
        got[0::2], got[1::2] = p2 & 0xF, p2 >> 4
        assert np.array_equal(got[nz], codes[nz])


def test_mxfp4_quantize_error_bound_and_special_blocks():
    rng = np.random.default_rng(4)
    for scale in (1e-3, 1.0, 50.0):
        for row in (rng.standard_normal((100, 128)) * scale).astype(np.float32):
            p, s = okw.quantize_key_mxfp4(row)
            deq = of.mxfp4_to_f64(p[None], s[None])[0]
            X = np.repeat(2.0 ** (s.astype(np.float64) - 127), 32)
            y = np.abs(row) / X
            assert (y < 8).all()                     # floor(log2 amax) - 2 puts every |k| / X below 8
            spacing = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
            bound = np.where(y <= 6, spacing / 2, y - 6) * X
            assert (np.abs(deq - row) <= bound * (1 + 1e-12)).all()
    k = np.zeros(128, np.float32)
    k[40] = 2.0 ** -140                              # tiny block: scale code clamps at 0
    k[70] = 7.0                                      # saturating block: 7 / 2^0 -> 6
    p, s = okw.quantize_key_mxfp4(k)
    assert list(s) == [0, 0, 127, 0]
    deq = of.mxfp4_to_f64(p[None], s[None])[0]
    assert deq[40] == 0.0 and deq[70] == 6.0 and not np.delete(deq, [40, 70]).any()


def test_kv_write_mxfp4_cache_rows():
    rng = np.random.default_rng(6)
    B, Sq, ps, D = 2, 3, 16, 128
    rows = 256
    pt = rng.permutation(rows // ps)[: B * 4].reshape(B, 4).astype(np.int32)
    seq_lens = np.array([20, 64], dtype=np.int32)
    lat = rng.integers(0, 65535, (B, Sq, 576), dtype=np.uint16)
    keys = rng.standard_normal((B, Sq, D)).astype(np.float32)
    kv0 = rng.integers(0, 65535, (rows, 576), dtype=np.uint16)
    ic0 = rng.integers(0, 255, (rows, D // 2), dtype=np.uint8)
    is0 = rng.integers(0, 255, (rows, D // 32), dtype=np.uint8)
    kv, ic, isc, err = okw.kv_write(lat, keys, seq_lens, pt, ps, kv0, ic0, is0, cache="mxfp4")
    assert err == 0
    written = set()
    for b in range(B):
        r = opg.paged_rows(pt[b], np.arange(seq_lens[b] - Sq, seq_lens[b]), ps)
        written |= set(r.tolist())
        for t in range(Sq):
            p, s = okw.quantize_key_mxfp4(keys[b, t])
            assert np.array_equal(ic[r[t]], p) and np.array_equal(isc[r[t]], s)
    keep = np.array(sorted(set(range(rows)) - written))
    assert np.array_equal(ic[keep], ic0[keep]) and np.array_equal(isc[keep], is0[keep])

"""Pins of the oracle's encoder against facts the pages fix (CPU only).

Sources: "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV
Caches" §3.2 (bit-plane K cache: code, sign MSB, prefix = t-bit mid-rise
quantizer, t = 4 special case) and the Appendix A walkthrough on the
jaehun.me review page (channel 2 codes and sign-plane decode).

The checks here compute the expected values by routes other than the
oracle's: exact rational arithmetic (fractions) or integer arithmetic on the
fp16 grid, and the direct t-bit quantizer formula instead of the prefix route.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _codes_from_planes(planes, g, j, blk):
    words = [int(planes[g, j, p, blk]) for p in range(4)]
    return np.array([sum(((words[p] >> i) & 1) << (3 - p) for p in range(4)) for i in range(64)])


def _block(values, d=1):
    k = np.zeros((1, 64, d), dtype=np.float16)
    k[0, :len(values), 0] = np.asarray(values, dtype=np.float16)
    return k


def test_appendix_a_channel2_codes(golden_dir):
    gold = json.load(open(os.path.join(golden_dir, "appendix_a.json")))
    planes, scales, bad = oracle.encode(_block(gold["channel2_values"]))
    assert bad == 0
    codes = _codes_from_planes(planes, 0, 0, 0)
    assert list(codes[:6]) == gold["channel2_codes"]
    assert all(c == 8 for c in codes[6:])           # zeros -> code 8 (§3.2: code 8 is zero)
    a = oracle.f16_to_f64(int(scales[0, 0, 0]))
    assert a == gold["channel2_a"]
    assert a / 8 == gold["channel2_s"]


def test_appendix_a_sign_plane_decode(golden_dir):
    gold = json.load(open(os.path.join(golden_dir, "appendix_a.json")))
    planes, scales, _ = oracle.encode(_block(gold["channel2_values"]))
    dec = oracle.decode(planes, scales, 64, 1)[0, :6, 0]
    assert list(dec) == gold["channel2_sign_plane_decode"]


def test_msb_is_sign():
    """§3.2: the most significant bit is the sign (1 for k >= 0 cells)."""
    rng = np.random.default_rng(0)
    v = rng.standard_normal(64).astype(np.float16)
    planes, _, _ = oracle.encode(_block(v))
    w = int(planes[0, 0, 0, 0])
    for i in range(64):
        assert ((w >> i) & 1) == (1 if float(v[i]) >= 0 else 0)


def _all_f16_upto(a_bits):
    """Every finite fp16 value k with |k| <= a (as fp16 bits)."""
    mags = np.arange(0, a_bits + 1, dtype=np.uint16)
    vals = np.concatenate([mags, mags[1:] | np.uint16(0x8000)])
    return vals


def _units(bits):
    """fp16 bits -> exact integer multiples of 2^-24 (int64)."""
    bits = bits.astype(np.int64)
    e = (bits >> 10) & 0x1F
    m = bits & 0x3FF
    u = np.where(e == 0, m, (m | 0x400) << np.maximum(e - 1, 0))
    return np.where(bits & 0x8000, -u, u)


A_VALUES = [0x7BFF, 0x3C00, 0x3800, 0x4248, 0x6400, 0x0400, 0x0005, 0x0001, 0x2E66]


@pytest.mark.parametrize("a_bits", A_VALUES)
def test_prefix_is_t_bit_midrise_quantizer_exhaustive(a_bits):
    """§3.2: the first t planes dequantize to exactly the t-bit mid-rise
    quantizer of [-a, a) with cells of width 2a/2^t, for every fp16 k with
    |k| <= a (k = +a lands in the top cell)."""
    vals = _all_f16_upto(a_bits)
    per = 63
    nblk = -(-len(vals) // per)
    k = np.zeros((1, nblk * 64, 1), dtype=np.uint16)
    for b in range(nblk):
        chunk = vals[b * per:(b + 1) * per]
        k[0, b * 64, 0] = a_bits                   # token 0 carries the block max a
        k[0, b * 64 + 1:b * 64 + 1 + len(chunk), 0] = chunk
    planes, scales, bad = oracle.encode(k)
    assert bad == 0
    assert np.all(scales == a_bits)
    K = _units(k[0, :, 0])
    A = int(_units(np.array([a_bits], dtype=np.uint16))[0])
    for t in range(1, 5):
        dec = oracle.decode(planes, scales, nblk * 64, t)[0, :, 0]
        # Direct quantizer, integer arithmetic in units of 2^-24 * (2A / 2^t):
        #   m = floor(k / delta_t), delta_t = 2a / 2^t, clamped to the 2^t cells,
        #   value = (m + 1/2) * delta_t = (2m + 1) * A / 2^t  [units of 2^-24].
        m = np.floor_divide(K * (1 << t), 2 * A)
        m = np.clip(m, -(1 << (t - 1)), (1 << (t - 1)) - 1)
        expect_scaled = (2 * m + 1) * A                        # = value * 2^24 * 2^t
        got_scaled = dec * float(2 ** (24 + t))
        assert np.all(got_scaled == expect_scaled.astype(np.float64)), t


def test_full_depth_is_c_minus_8_plus_half_times_s():
    """§3.2: at t = 4 the value reduces to (c - 8 + 0.5) * s."""
    rng = np.random.default_rng(1)
    k = (rng.standard_normal((1, 64 * 8, 1)) * 3).astype(np.float16)
    planes, scales, _ = oracle.encode(k)
    dec = oracle.decode(planes, scales, 64 * 8, 4)[0, :, 0]
    for b in range(8):
        a = oracle.f16_to_f64(int(scales[0, 0, b]))
        codes = _codes_from_planes(planes, 0, 0, b)
        assert np.all(dec[b * 64:(b + 1) * 64] == (codes - 8 + 0.5) * (a / 8))


def test_floor_is_exact_against_fractions():
    """Codes equal clamp(floor(k / (a/8)) + 8, 0, 15) in exact rationals,
    including values sitting exactly on cell edges and one ulp either side."""
    rng = np.random.default_rng(2)
    cases = []
    for _ in range(200):
        a = np.float16(abs(rng.standard_normal()) * 10 ** rng.uniform(-4, 4))
        if not np.isfinite(a) or a == 0:
            continue
        s = Fraction(float(a)) / 8
        vals = [np.float16(float(a))]
        for m in range(-8, 9):
            edge = np.float16(float(m * s))
            vals += [edge, np.nextafter(edge, np.float16(np.inf)), np.nextafter(edge, np.float16(-np.inf))]
        vals += list(rng.uniform(-float(a), float(a), 20).astype(np.float16))
        vals = [v for v in vals if np.isfinite(v) and abs(float(v)) <= float(a)][:63]
        cases.append((a, vals))
    for a, vals in cases:
        k = np.zeros((1, 64, 1), dtype=np.float16)
        k[0, 0, 0] = a
        k[0, 1:1 + len(vals), 0] = vals
        planes, _, _ = oracle.encode(k)
        codes = _codes_from_planes(planes, 0, 0, 0)
        s = Fraction(float(a)) / 8
        for i, v in enumerate([a] + vals):
            q = Fraction(float(v)) / s
            expect = min(15, max(0, (q.numerator // q.denominator) + 8))
            assert codes[i] == expect, (float(a), float(v))


def test_zero_block_and_extremes():
    """All-zero block: a = 0 and every code 8 (value 0 at any depth).  k = +a ->
    15, k = -a -> 0, +-0 -> 8."""
    k = np.zeros((1, 128, 1), dtype=np.float16)
    k[0, 64, 0] = 2.0
    k[0, 65, 0] = -2.0
    k[0, 66, 0] = -0.0
    planes, scales, _ = oracle.encode(k)
    assert scales[0, 0, 0] == 0
    assert all(c == 8 for c in _codes_from_planes(planes, 0, 0, 0))
    for t in range(1, 5):
        assert np.all(oracle.decode(planes, scales, 128, t)[0, :64, 0] == 0.0)
    c1 = _codes_from_planes(planes, 0, 0, 1)
    assert c1[0] == 15 and c1[1] == 0 and c1[2] == 8 and c1[3] == 8


def test_nonfinite_blocks_are_counted():
    k = np.zeros((2, 128, 3), dtype=np.float16)
    k[0, 5, 1] = np.inf
    k[1, 70, 2] = np.nan
    _, _, bad = oracle.encode(k)
    assert bad == 2


def test_channel_major_layout_and_append():
    """Planes are [group][channel][plane][block] (§3.6: the first t planes of a
    channel form one contiguous run); encoding block by block into slots of a
    larger store equals encoding the whole sequence at once."""
    rng = np.random.default_rng(3)
    k = (rng.standard_normal((2, 64 * 5, 7)) * rng.uniform(0.1, 5, 7)).astype(np.float16)
    p_all, s_all, _ = oracle.encode(k)
    p = np.full((2, 7, 4, 9), 0xDEADBEEF, dtype=np.uint64)
    s = np.full((2, 7, 9), 0x1234, dtype=np.uint16)
    for b in range(5):
        oracle.encode(np.ascontiguousarray(k[:, b * 64:(b + 1) * 64]), nb_store=9,
                      block_offset=2 + b, planes=p, scales=s)
    assert np.array_equal(p[:, :, :, 2:7], p_all)
    assert np.array_equal(s[:, :, 2:7], s_all)
    assert np.all(p[:, :, :, :2] == 0xDEADBEEF) and np.all(p[:, :, :, 7:] == 0xDEADBEEF)
    # channel j of block b decodes from its own column only
    for j in range(7):
        kj = k.copy()
        kj[:, :, j] = 0
        pj, _, _ = oracle.encode(kj)
        others = [c for c in range(7) if c != j]
        assert np.array_equal(pj[:, others], p_all[:, others])


def test_store_is_68_bytes_per_token_per_head():
    """§3.2/§7: 4 planes of 64 bits plus one fp16 scale per 64-token block and
    channel = 68 bytes per token per KV head at d = 128."""
    k = np.zeros((1, 64, 128), dtype=np.float16)
    planes, scales, _ = oracle.encode(k)
    assert (planes.nbytes + scales.nbytes) / 64 == 68

"""Pins of the oracle's element formats and block conversion (CPU only).

Each check ties the oracle to something other than itself: values the format
definitions name, torch's own float8 casts, hand-worked blocks, an exhaustive
code round trip, invariants of Algorithm 1, and a brute-force rational search
over all codes of a format.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from mx_brute import FMT_BITS, Grid, brute_block, f32_bits

HERE = os.path.dirname(os.path.abspath(__file__))
FMTS = ["e4m3", "e5m2", "e2m3", "e3m2", "e2m1", "int8"]


def test_named_values(oracle):
    o = oracle
    # E2M1 positive codes are exactly {0, .5, 1, 1.5, 2, 3, 4, 6}
    assert [o.elem_value(o.E2M1, c) for c in range(8)] == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    # largest normals 448 / 57344 / 7.5 / 28 / 6 / 127/64
    assert o.elem_value(o.E4M3, 0x7E) == 448.0
    assert o.elem_value(o.E5M2, 0x7B) == 57344.0
    assert o.elem_value(o.E2M3, 0x1F) == 7.5
    assert o.elem_value(o.E3M2, 0x1F) == 28.0
    assert o.elem_value(o.E2M1, 0x7) == 6.0
    assert o.elem_value(o.INT8, 0x7F) == 127 / 64
    for f, mx in [(o.E4M3, 448), (o.E5M2, 57344), (o.E2M3, 7.5), (o.E3M2, 28), (o.E2M1, 6),
                  (o.INT8, 127 / 64)]:
        assert o.elem_maxnorm(f) == mx
    # 1.0 codes
    assert o.elem_value(o.E4M3, 0x38) == 1.0
    assert o.elem_value(o.E5M2, 0x3C) == 1.0
    assert o.elem_value(o.E2M3, 0x08) == 1.0
    assert o.elem_value(o.E3M2, 0x0C) == 1.0
    assert o.elem_value(o.INT8, 0x40) == 1.0
    # smallest subnormals and normals
    assert o.elem_value(o.E4M3, 0x01) == 2.0 ** -9 and o.elem_value(o.E4M3, 0x08) == 2.0 ** -6
    assert o.elem_value(o.E5M2, 0x01) == 2.0 ** -16 and o.elem_value(o.E5M2, 0x04) == 2.0 ** -14
    assert o.elem_value(o.E2M3, 0x01) == 0.125
    assert o.elem_value(o.E3M2, 0x01) == 0.0625 and o.elem_value(o.E3M2, 0x04) == 0.25
    assert o.elem_value(o.E2M1, 0x01) == 0.5
    # special codes
    assert math.isnan(o.elem_value(o.E4M3, 0x7F)) and math.isnan(o.elem_value(o.E4M3, 0xFF))
    assert o.elem_value(o.E5M2, 0x7C) == math.inf and o.elem_value(o.E5M2, 0xFC) == -math.inf
    for c in (0x7D, 0x7E, 0x7F):
        assert math.isnan(o.elem_value(o.E5M2, c))
    assert o.elem_value(o.INT8, 0x80) == -2.0 and o.elem_value(o.INT8, 0xFF) == -1 / 64
    # emax: the largest normal lies in binade 2^emax
    assert [o.elem_emax(f) for f in range(6)] == [8, 15, 2, 4, 2, 0]


def test_fp8_decode_matches_torch(oracle):
    """Every E4M3 / E5M2 code decodes as torch's OCP float8 types do."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    for fmt, dt in [(oracle.E4M3, torch.float8_e4m3fn), (oracle.E5M2, torch.float8_e5m2)]:
        ref = codes.view(dt).to(torch.float64).numpy()
        mine = np.array([oracle.elem_value(fmt, c) for c in range(256)])
        np.testing.assert_array_equal(np.isnan(mine), np.isnan(ref))
        ok = ~np.isnan(ref)
        np.testing.assert_array_equal(mine[ok], ref[ok])
        np.testing.assert_array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


@pytest.mark.parametrize("fmt", range(5))
def test_decode_structure(oracle, fmt):
    """Positive finite codes increase strictly in value; the sign bit negates."""
    nbits = FMT_BITS[fmt]
    half = 1 << (nbits - 1)
    vals = [oracle.elem_value(fmt, c) for c in range(half)]
    finite = [v for v in vals if math.isfinite(v)]
    assert all(b > a for a, b in zip(finite, finite[1:]))
    for c in range(half):
        v, n = vals[c], oracle.elem_value(fmt, c | half)
        if math.isnan(v):
            assert math.isnan(n)
        else:
            assert n == -v and math.copysign(1, n) == -1
    # number of finite positive values: all codes but the NaN / Inf ones
    expect = {0: half - 1, 1: half - 4}.get(fmt, half)
    assert len(finite) == expect


def test_hand_worked_blocks(oracle):
    fx = json.load(open(os.path.join(HERE, "golden", "hand_blocks.json")))
    for blk in fx["blocks"]:
        fmt = oracle.FORMATS[blk["fmt"]]
        v = np.zeros(32, np.float32)
        v[: len(blk["inputs"])] = [np.float32(float(s)) for s in blk["inputs"]]
        if blk["inputs"][:2] == ["0.0", "-0.0"]:
            v[1] = np.float32(-0.0)
        sc, codes = oracle.quantize_block(fmt, v)
        n = len(blk["codes"])
        assert sc == blk["scale"], blk
        assert list(codes[:n]) == blk["codes"], blk
        assert not codes[n:].any(), blk


@pytest.mark.parametrize("fmt", range(6))
def test_exhaustive_code_round_trip(oracle, fmt):
    """Every finite code c comes back from the block [maxnorm, value(c), 0...]
    with scale 127, and with scale 127+s when the block is scaled by 2^s."""
    o = oracle
    maxnorm = o.elem_maxnorm(fmt)
    codes = range(256) if fmt == o.INT8 else range(1 << FMT_BITS[fmt])
    for c in codes:
        if fmt == o.INT8 and c == 0x80:
            continue  # -2.0 decodes but saturation never produces it
        val = o.elem_value(fmt, c)
        if not math.isfinite(val):
            continue
        expect = c
        for s in (-100, -20, -1, 0, 1, 7, 50, 100):
            v = np.zeros(32, np.float32)
            v[0] = np.float32(maxnorm * 2.0 ** s)
            v[1] = np.float32(val * 2.0 ** s)
            if val == 0 and math.copysign(1, val) < 0:
                v[1] = np.float32(-0.0)
            if f32_bits(float(v[1])) & 0x7F800000 == 0 and val != 0:
                continue  # scaled value became fp32-subnormal
            sc, q = o.quantize_block(fmt, v)
            assert sc == 127 + s, (fmt, c, s)
            assert q[1] == expect, (fmt, hex(c), s, q[1])


@pytest.mark.parametrize("fmt", range(2))
def test_fp8_rne_matches_torch_cast(oracle, fmt):
    """With the scale fixed at 1 (block max in [2^emax, 2^(emax+1))), in-range
    elements are converted like torch's RNE float8 cast."""
    o = oracle
    rng = np.random.default_rng(1)
    dt = [torch.float8_e4m3fn, torch.float8_e5m2][fmt]
    maxnorm = o.elem_maxnorm(fmt)
    emax = o.elem_emax(fmt)
    for trial in range(200):
        v = np.zeros(32, np.float32)
        mag = np.exp2(rng.uniform(-18 if fmt == 0 else -26, emax + 0.99, size=32))
        v[:] = (mag * rng.choice([-1, 1], size=32)).astype(np.float32)
        v = np.clip(v, -maxnorm, maxnorm).astype(np.float32)
        v[0] = np.float32(2.0 ** emax)
        sc, q = o.quantize_block(fmt, v)
        assert sc == 127
        ref = torch.from_numpy(v).to(dt).view(torch.uint8).numpy()
        np.testing.assert_array_equal(q, ref)


def _random_blocks(rng, n):
    """Blocks of mixed character: wide dynamic range, ties, zeros, subnormals."""
    out = []
    for i in range(n):
        kind = i % 5
        if kind == 0:
            v = rng.standard_normal(32).astype(np.float32)
        elif kind == 1:
            v = (rng.standard_t(3, 32) * 2.0 ** rng.uniform(-40, 40)).astype(np.float32)
        elif kind == 2:  # dyadic values: many exact ties
            v = (rng.integers(-64, 64, 32) * 2.0 ** rng.integers(-8, 8)).astype(np.float32)
        elif kind == 3:  # huge spread within one block
            v = (rng.standard_normal(32) * np.exp2(rng.uniform(-60, 60, 32))).astype(np.float32)
        else:  # zeros and fp32 subnormals mixed in
            v = rng.standard_normal(32).astype(np.float32) * np.float32(2.0 ** rng.integers(-126, 100))
            m = rng.random(32)
            v[m < 0.2] = 0.0
            sub = (rng.integers(1, 1 << 23, 32).astype(np.uint32)).view(np.float32)
            v[m > 0.8] = sub[m > 0.8] * np.sign(rng.standard_normal(32))[m > 0.8]
        out.append(v)
    return out


@pytest.mark.parametrize("fmt", range(6))
def test_rne_matches_brute_force(oracle, fmt):
    """Scale and every element equal an exhaustive nearest-code search."""
    grid = Grid(oracle, fmt)
    rng = np.random.default_rng(100 + fmt)
    for v in _random_blocks(rng, 150):
        sc, q = oracle.quantize_block(fmt, v)
        bsc, bq = brute_block(grid, v)
        assert sc == bsc
        assert list(q) == bq


@pytest.mark.parametrize("fmt", range(6))
def test_algorithm1_invariants(oracle, fmt):
    o = oracle
    rng = np.random.default_rng(200 + fmt)
    emax, maxnorm = o.elem_emax(fmt), o.elem_maxnorm(fmt)
    for v in _random_blocks(rng, 150):
        sc, q = o.quantize_block(fmt, v)
        X = 2.0 ** (sc - 127)
        deq = np.array([o.elem_value(fmt, int(c)) for c in q]) * X
        vv = v.astype(np.float64)
        sub = (v.view(np.uint32) & 0x7F800000) == 0
        vv[sub] = 0.0
        amax = np.abs(vv).max()
        if amax == 0:
            assert sc == 0 and not np.any(deq)
            continue
        a_i = int(np.argmax(np.abs(vv)))
        # the block max lands in [2^emax, maxnorm] * X unless the scale hit 2^-127
        assert abs(deq[a_i]) <= maxnorm * X
        if sc > 0:
            assert abs(deq[a_i]) >= 2.0 ** emax * X
        # monotone in magnitude, sign-symmetric
        order = np.argsort(np.abs(vv), kind="stable")
        assert np.all(np.diff(np.abs(deq[order])) >= 0)
        sc2, q2 = o.quantize_block(fmt, -v)
        assert sc2 == sc
        deq2 = np.array([o.elem_value(fmt, int(c)) for c in q2]) * X
        np.testing.assert_array_equal(deq2, -deq)
        # error within half a grid step for elements below the max normal
        for i in range(32):
            a = abs(vv[i]) / X
            if a >= maxnorm or a == 0:
                continue
            if fmt == o.INT8:
                step = 2.0 ** -6
            else:
                emin = {0: -6, 1: -14, 2: 0, 3: -2, 4: 0}[fmt]
                mb = {0: 3, 1: 2, 2: 3, 3: 2, 4: 1}[fmt]
                step = 2.0 ** (max(math.floor(math.log2(a)), emin) - mb)
            assert abs(abs(deq[i]) / X - a) <= step / 2


@pytest.mark.parametrize("fmt", range(6))
def test_power_of_two_equivariance(oracle, fmt):
    rng = np.random.default_rng(300 + fmt)
    for _ in range(100):
        v = rng.standard_normal(32).astype(np.float32)
        sc, q = oracle.quantize_block(fmt, v)
        for s in (-60, -3, 5, 90):
            sc2, q2 = oracle.quantize_block(fmt, (v * np.float32(2.0 ** s)).astype(np.float32))
            assert sc2 == sc + s
            np.testing.assert_array_equal(q2, q)


def test_daz_and_special_blocks(oracle):
    o = oracle
    sub = np.array([1, 0x7FFFFF, 0x400000, 5], np.uint32).view(np.float32)
    # all-subnormal block -> zero block: scale 0, signed zero elements
    v = np.zeros(32, np.float32)
    v[:4] = sub * np.array([1, -1, 1, -1], np.float32)
    for fmt in range(6):
        sc, q = o.quantize_block(fmt, v)
        assert sc == 0
        if fmt == o.INT8:
            assert not q.any()
        else:
            sign = 1 << (FMT_BITS[fmt] - 1)
            assert list(q[:4]) == [0, sign, 0, sign] and not q[4:].any()
    # a subnormal next to a normal: zero even where V/X would be representable
    v = np.zeros(32, np.float32)
    v[0] = np.float32(2.0 ** -126)
    v[1] = sub[1]  # just below 2^-126
    sc, q = o.quantize_block(o.E4M3, v)
    # floor(log2 2^-126) - 8 = -134 is clamped to -127 -> code 0, X = 2^-127
    assert sc == 0
    # 2^-126 / 2^-127 = 2 -> 0x40; the subnormal would have been ~2 as well,
    # but it is set to zero first
    assert q[0] == 0x40 and q[1] == 0
    # Inf / NaN anywhere -> NaN scale; FP8 elements are the NaN code
    for bad in (np.inf, -np.inf, np.nan):
        v = np.ones(32, np.float32)
        v[7] = bad
        for fmt in range(6):
            sc, q = o.quantize_block(fmt, v)
            assert sc == 0xFF
            nan_code = 0x7F if fmt in (o.E4M3, o.E5M2) else 0
            assert (q == nan_code).all()

"""Pins of the oracle's number formats against definitions, hand-derived points and torch's casts.

CPU only. torch's CPU bfloat16 / float8_e4m3fn conversions are an independent
implementation present in the image; they are used where they are single
roundings (fp32 -> bf16, fp32 -> e4m3 for in-range values).
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import codecs


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _expr(s):
    return float(eval(s, {"__builtins__": {}}, {}))  # fixtures hold plain arithmetic only


# ---------------------------------------------------------------------------
# bfloat16
# ---------------------------------------------------------------------------

def test_bf16_golden_points(golden_dir):
    pts = _load(golden_dir, "bf16_points.json")["points"]
    for p in pts:
        got = int(codecs.f64_to_bf16_bits(np.array([_expr(p["x_expr"])]))[0])
        assert got == int(p["bits"], 16), p


def test_bf16_matches_torch_fp32_cast():
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 2 ** 32, size=400_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    # values whose rounding overflows are out of the oracle's domain
    f = f[np.abs(f.astype(np.float64)) < (2 - 2 ** -8) * 2.0 ** 127]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = codecs.f64_to_bf16_bits(f.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_roundtrip_all_finite_patterns():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = codecs.bf16_bits_to_f64(b)
    fin = np.isfinite(v)
    assert np.array_equal(codecs.f64_to_bf16_bits(v[fin]), b[fin])


def test_bf16_rejects_nonfinite():
    with pytest.raises(ValueError):
        codecs.f64_to_bf16_bits(np.array([np.nan]))


# ---------------------------------------------------------------------------
# E4M3
# ---------------------------------------------------------------------------

def test_e4m3_golden_points(golden_dir):
    for p in _load(golden_dir, "e4m3_points.json")["points"]:
        got = int(codecs.e4m3_encode(np.array([_expr(p["x_expr"])]))[0])
        assert got == int(p["code"], 16), p


def test_e4m3_decode_table_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3_decode(codes)
    theirs = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(theirs)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(ours[~nan], theirs[~nan])
    # sign of zero
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_e4m3_encode_inverts_decode_and_rounds_midpoints_to_even():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = codecs.e4m3_decode(codes)
    assert np.array_equal(codecs.e4m3_encode(vals), codes)
    # midpoints of consecutive non-negative finite codes round to the even code
    pos = np.arange(0, 0x7F, dtype=np.uint8)
    v = codecs.e4m3_decode(pos)
    mid = (v[:-1] + v[1:]) / 2
    enc = codecs.e4m3_encode(mid)
    lo, hi = pos[:-1], pos[1:]
    want = np.where(lo % 2 == 0, lo, hi)
    assert np.array_equal(enc, want)
    # just off the midpoint goes to the nearer code
    d = (v[1:] - v[:-1]) * 1e-6
    assert np.array_equal(codecs.e4m3_encode(mid - d), lo)
    assert np.array_equal(codecs.e4m3_encode(mid + d), hi)


def test_e4m3_matches_torch_on_all_bf16_in_range():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = codecs.bf16_bits_to_f64(b)
    for shift in (-12, -6, 0, 3):
        x = v * 2.0 ** shift
        ok = np.isfinite(x) & (np.abs(x) <= 448.0)
        x = x[ok]
        want = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codecs.e4m3_encode(x), want), shift


def test_e4m3_saturates():
    assert int(codecs.e4m3_encode(np.array([1e6]))[0]) == 0x7E
    assert int(codecs.e4m3_encode(np.array([-500.0]))[0]) == 0xFE


# ---------------------------------------------------------------------------
# E8M0 and the MXFP8 block quantizer
# ---------------------------------------------------------------------------

def test_e8m0_golden_points(golden_dir):
    for p in _load(golden_dir, "e8m0_points.json")["points"]:
        e = int(codecs.e8m0_exponent(np.array([_expr(p["amax_expr"])]))[0])
        assert e + 127 == p["byte"], p


def test_e8m0_brute_force_search():
    """Against a direct search of the definition over every candidate exponent."""
    rng = np.random.default_rng(5)
    b = rng.integers(0, 0x7F80, size=3000).astype(np.uint16)  # non-negative finite bf16
    amax = codecs.bf16_bits_to_f64(b)
    got = codecs.e8m0_exponent(amax)
    for a, e in zip(amax, got):
        cands = [k for k in range(-127, 128) if a <= 448.0 * 2.0 ** k]
        assert e == (cands[0] if a > 0 else -127)


def test_mxfp8_roundtrip_within_half_ulp():
    rng = np.random.default_rng(7)
    x = rng.normal(0, 1, size=(16, 256)) * np.exp(rng.normal(0, 3, size=(16, 1)))
    bits = codecs.f64_to_bf16_bits(x)
    codes, scales = codecs.mxfp8_quantize(bits)
    xv = codecs.bf16_bits_to_f64(bits)
    e = scales.astype(np.int64) - 127
    back = codecs.e4m3_decode(codes) * np.repeat(2.0 ** e, 32, axis=1)
    # spacing of E4M3 at each element's magnitude (in scaled units), then rescaled
    scaled = np.abs(xv) * np.repeat(2.0 ** -e, 32, axis=1)
    _, ex = np.frexp(np.maximum(scaled, 2.0 ** -6))
    ulp = np.ldexp(1.0, ex - 1 - 3) * np.repeat(2.0 ** e, 32, axis=1)
    assert np.all(np.abs(back - xv) <= 0.5 * ulp)
    # and the block maximum never saturates
    assert np.all(np.abs(xv).reshape(16, 8, 32).max(axis=2) <= 448.0 * 2.0 ** e)


def test_mxfp8_zero_block_and_layout():
    bits = np.zeros((2, 64), dtype=np.uint16)
    bits[1, 32:] = codecs.f64_to_bf16_bits(np.full(32, 3.0))
    codes, scales = codecs.mxfp8_quantize(bits)
    assert scales.shape == (2, 2)
    assert list(scales[0]) == [0, 0] and scales[1, 0] == 0
    assert scales[1, 1] == 127 - 7  # 3.0 <= 448 * 2**-7 = 3.5
    assert np.all(codes[1, 32:] == codecs.e4m3_encode(np.array([3.0 * 2 ** 7]))[0])


# ---------------------------------------------------------------------------
# the swizzled 128x4 scale layout
# ---------------------------------------------------------------------------

def _swizzle_ids(rows, blocks):
    """Swizzle the element ids r * blocks + b (as two byte planes) and decode them back;
    padding (fill 255 in the high plane) decodes to -1."""
    ids = np.arange(rows * blocks, dtype=np.int64).reshape(rows, blocks)
    assert rows * blocks < 255 * 256
    lo = codecs.mxfp8_scales_swizzled_128x4((ids & 0xFF).astype(np.uint8), fill=0)
    hi = codecs.mxfp8_scales_swizzled_128x4((ids >> 8).astype(np.uint8), fill=255)
    out = lo.astype(np.int64) | (hi.astype(np.int64) << 8)
    return np.where(hi == 255, -1, out)


def test_scale_swizzle_golden_offsets(golden_dir):
    g = _load(golden_dir, "scale_swizzle_128x4.json")
    got = _swizzle_ids(g["rows"], g["blocks"])
    assert got.size == g["total_bytes"]
    for p in g["points"]:
        assert got[p["offset"]] == p["row"] * g["blocks"] + p["block"], p
    for p in g["padding"]:
        assert got[p["offset"]] == -1, p


@pytest.mark.parametrize("rows,blocks", [(1, 1), (128, 4), (130, 6), (64, 33), (300, 201)])
def test_scale_swizzle_is_a_padded_permutation(rows, blocks):
    got = _swizzle_ids(rows, blocks)
    rp, bp = -(-rows // 128) * 128, -(-blocks // 4) * 4
    assert got.size == rp * bp
    real = got[got >= 0]
    assert np.array_equal(np.sort(real), np.arange(rows * blocks))  # each scale exactly once
    assert np.count_nonzero(got < 0) == rp * bp - rows * blocks


@pytest.mark.parametrize("rows,blocks", [(130, 6), (300, 201)])
def test_scale_swizzle_tiles_and_row_groups(rows, blocks):
    """Tile i (512 bytes, row-major over the padded tile grid) holds exactly its 128 x 4
    block; its 16-byte group b holds rows b, b+32, b+64, b+96, four consecutive blocks
    each."""
    got = _swizzle_ids(rows, blocks)
    bp = -(-blocks // 4) * 4
    kt = bp // 4
    for tile in range(got.size // 512):
        tr, tk = divmod(tile, kt)
        t = got[tile * 512:(tile + 1) * 512]
        for b in range(32):
            grp = t[16 * b:16 * b + 16]
            for a in range(4):
                r = 128 * tr + 32 * a + b
                for c in range(4):
                    k = 4 * tk + c
                    want = r * blocks + k if (r < rows and k < blocks) else -1
                    assert grp[4 * a + c] == want, (tile, b, a, c)

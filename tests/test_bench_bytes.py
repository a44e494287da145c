"""The bench's algorithmic-byte counts (host logic, CPU only): each formula against a count
written out tensor by tensor for the headline and the other calls."""

import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_headline_bytes_by_tensor():
    b = _bench()
    R, H, T, n = 32, 7168, 8, 4
    partials = T * R * H * 2
    streams_in = streams_out = R * n * H * 2
    coeffs = R * (n + n * n + n) * 4        # post, comb, pre
    norm_w = H * 2
    layer = R * H * 2
    e4m3 = R * H
    e8m0 = R * H // 32
    want = partials + streams_in + streams_out + coeffs + norm_w + layer + e4m3 + e8m0
    assert want == 8_052_736
    assert b.bytes_boundary(R, H, T, pre=True, mxfp8=True) == want
    assert b.bytes_boundary(R, H, T, pre=True, mxfp8=False) == want - e4m3 - e8m0
    assert b.bytes_boundary(R, H, T, pre=False) == partials + streams_in + streams_out + \
        R * (n + n * n) * 4


def test_other_calls_bytes_by_tensor():
    b = _bench()
    R, H, K, n, nc = 64, 7168, 8, 4, 24
    gathered = R * K * H * 2 + R * K * (4 + 4)   # expert rows, weights, indices
    want = gathered + R * H * 2 + 2 * R * n * H * 2 + R * (n + n * n + n) * 4 + H * 2 + \
        R * H * 2 + R * H + R * H // 32
    assert b.bytes_finalize(R, H, K, pre=True, mxfp8=True) == want == 17_012_736
    assert b.bytes_pre(R, H) == R * n * H * 2 + n * H * nc * 2 + (3 + nc) * 4 + R * nc * 4 \
        == 5_052_524
    assert b.bytes_mean(128, H) == 128 * n * H * 2 + 128 * H * 2
    assert b.bytes_floor(32, H, 8) == 32 * (8 * H * 2 + 2 * n * H * 2 + H * 2 + H + H // 32)

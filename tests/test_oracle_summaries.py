"""Pins for the oracle's summary construction (reading R-sum).

Checked against: exact closed forms (constant keys), the fp64 mean, and the
hand-derived rounding fixtures in tests/golden/summary_rounding.txt.
"""
import os

import numpy as np
import pytest

from hga_inputs import round_to_bf16
from oracle import hga_oracle as ora

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "summary_rounding.txt")


def _empty_sums(B, H, t_cap, d):
    return (np.zeros((B, H, t_cap // 8, d), np.float32), np.zeros((B, H, t_cap // 64, d), np.float32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_constant_keys_give_the_key(dtype):
    rng = np.random.default_rng(0)
    B, H, T, d = 2, 3, 256, 16
    base = rng.standard_normal((B, H, T // 64, 1, d)).astype(np.float32)
    if dtype == "bf16":
        base = round_to_bf16(base)
    k = np.broadcast_to(base, (B, H, T // 64, 64, d)).reshape(B, H, T, d).copy()
    gs, cs = _empty_sums(B, H, T, d)
    ora.build_summaries(k, 0, T, dtype, gs, cs)
    np.testing.assert_array_equal(cs, base[:, :, :, 0, :])
    np.testing.assert_array_equal(gs, np.repeat(base[:, :, :, 0, :], 8, axis=2))


def test_fp32_summaries_match_fp64_mean():
    rng = np.random.default_rng(1)
    B, H, T, d = 1, 2, 512, 64
    k = rng.standard_normal((B, H, T, d)).astype(np.float32) * 3 + 1
    gs, cs = _empty_sums(B, H, T, d)
    ora.build_summaries(k, 0, T, "f32", gs, cs)
    g64 = k.astype(np.float64).reshape(B, H, T // 8, 8, d).mean(axis=3)
    c64 = k.astype(np.float64).reshape(B, H, T // 64, 64, d).mean(axis=3)
    assert np.max(np.abs(gs - g64)) <= 1e-6 * (1 + np.max(np.abs(g64)))
    assert np.max(np.abs(cs - c64)) <= 1e-6 * (1 + np.max(np.abs(c64)))


def test_bf16_summaries_within_half_ulp_of_exact_mean():
    rng = np.random.default_rng(2)
    B, H, T, d = 1, 2, 512, 64
    k = round_to_bf16(rng.standard_normal((B, H, T, d)).astype(np.float32))
    gs, cs = _empty_sums(B, H, T, d)
    ora.build_summaries(k, 0, T, "bf16", gs, cs)
    g64 = k.astype(np.float64).reshape(B, H, T // 8, 8, d).mean(axis=3)
    c64 = k.astype(np.float64).reshape(B, H, T // 64, 64, d).mean(axis=3)
    for got, ref in ((gs, g64), (cs, c64)):
        np.testing.assert_array_equal(got, round_to_bf16(got))          # stored as bf16
        half_ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 8)
        assert np.all(np.abs(got - ref) <= half_ulp * 1.0001 + 1e-6 * np.abs(ref) + 1e-30)


def test_chunk_summary_is_mean_of_unrounded_group_means_fp32():
    # power-of-two scaling commutes with the pinned tree: chunk = tree(group sums)/64
    # equals tree(group means)/8 bit for bit in fp32.
    rng = np.random.default_rng(3)
    k = rng.standard_normal((1, 1, 128, 32)).astype(np.float32)
    gs, cs = _empty_sums(1, 1, 128, 32)
    ora.build_summaries(k, 0, 128, "f32", gs, cs)
    for c in range(2):
        g = [gs[0, 0, 8 * c + u] for u in range(8)]
        tree = ((g[0] + g[1]) + (g[2] + g[3])) + ((g[4] + g[5]) + (g[6] + g[7]))
        np.testing.assert_array_equal(cs[0, 0, c], tree * np.float32(0.125))


def test_partial_range_leaves_other_rows_untouched():
    rng = np.random.default_rng(4)
    k = round_to_bf16(rng.standard_normal((1, 1, 256, 16)).astype(np.float32))
    gs, cs = _empty_sums(1, 1, 256, 16)
    gs[:] = 7.0
    cs[:] = 7.0
    ora.build_summaries(k, 64, 192, "bf16", gs, cs)
    assert np.all(gs[0, 0, :8] == 7.0) and np.all(gs[0, 0, 24:] == 7.0)
    assert np.all(cs[0, 0, 0] == 7.0) and np.all(cs[0, 0, 3] == 7.0)
    assert not np.any(gs[0, 0, 8:24] == 7.0)


def _golden_cases():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split("->")
            parts = lhs.split()
            out.append((parts[0], [float(x) for x in parts[1:]], float(rhs)))
    return out


@pytest.mark.parametrize("kind,args,expected", _golden_cases())
def test_golden_rounding(kind, args, expected):
    d = 4
    if kind == "group":
        keys = np.array(args, np.float32)
        k = np.zeros((1, 1, 64, d), np.float32)
        k[0, 0, :8, :] = keys[:, None]
        gs, cs = _empty_sums(1, 1, 64, d)
        ora.build_summaries(k, 0, 64, "bf16", gs, cs)
        np.testing.assert_array_equal(gs[0, 0, 0], np.full(d, expected, np.float32))
    else:
        base, idx, val = args
        k = np.full((1, 1, 64, d), base, np.float32)
        k[0, 0, int(idx), :] = val
        gs, cs = _empty_sums(1, 1, 64, d)
        ora.build_summaries(k, 0, 64, "bf16", gs, cs)
        np.testing.assert_array_equal(cs[0, 0, 0], np.full(d, expected, np.float32))

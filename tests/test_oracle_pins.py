"""Pins of the CPU oracle against things other than itself: closed forms,
library routines, brute force, invariants, the one number the pages print
for the row layout, and a second independently written model.

All CPU-only (no GPU marker).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

import oracle
from tests import numpy_model as nm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def unpack_codes(packed_row: np.ndarray, dim: int, bits: int) -> np.ndarray:
    if bits == 8:
        return packed_row[:dim].astype(np.int64)
    if bits == 2:
        C = (dim + 3) // 4
        b = packed_row[:C].astype(np.int64)
        q = np.empty(4 * C, dtype=np.int64)
        for j in range(4):
            q[j::4] = (b >> (2 * j)) & 3
        return q[:dim]
    C = (dim + 1) // 2
    b = packed_row[:C].astype(np.int64)
    q = np.empty(2 * C, dtype=np.int64)
    q[0::2] = b & 0xF
    q[1::2] = b >> 4
    return q[:dim]


def unpack_params(packed_row: np.ndarray, dim: int, bits: int):
    C = (dim * bits + 7) // 8
    s16 = int(packed_row[C]) | (int(packed_row[C + 1]) << 8)
    b16 = int(packed_row[C + 2]) | (int(packed_row[C + 3]) << 8)
    sf = float(np.array(s16, np.uint16).view(np.float16))
    bf = float(np.array(b16, np.uint16).view(np.float16))
    return s16, b16, sf, bf


# ---------------------------------------------------------------------------
# binary16 conversion: against numpy's float16 (round to nearest even)
# ---------------------------------------------------------------------------

def test_f32_to_f16_matches_numpy_on_every_mantissa_of_boundary_exponents(oracle_lib):
    # every binary32 mantissa for exponents around the binary16 subnormal
    # range, its normal/subnormal boundary, 1.0, the overflow threshold, and
    # the special exponents; both signs
    exps = [0, 1] + list(range(100, 116)) + [126, 127] + [141, 142, 143, 144] + [254, 255]
    mant = np.arange(1 << 23, dtype=np.uint32)
    for e in exps:
        for sign in (0, 1):
            u = (np.uint32(sign << 31) | np.uint32(e << 23) | mant).astype(np.uint32)
            x = u.view(np.float32)
            ours = oracle.f32_to_f16_bits(x)
            ref = x.astype(np.float16).view(np.uint16)
            nan = np.isnan(x)
            assert np.array_equal(ours[~nan], ref[~nan]), "exponent %d sign %d" % (e, sign)
            assert np.all((ours[nan] & 0x7C00) == 0x7C00) and np.all((ours[nan] & 0x3FF) != 0)


def test_f32_to_f16_matches_numpy_on_random_patterns(oracle_lib):
    g = np.random.default_rng(7)
    u = g.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    keep = ~np.isnan(x)
    assert np.array_equal(oracle.f32_to_f16_bits(x)[keep], x[keep].astype(np.float16).view(np.uint16))


def test_f16_to_f32_exhaustive(oracle_lib):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_bits_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.all(np.isnan(ours[nan]))


# ---------------------------------------------------------------------------
# row layout: the one number the pages print for it
# ---------------------------------------------------------------------------

def test_row_bytes_reproduce_printed_size_ratio(oracle_lib):
    with open(os.path.join(GOLDEN, "size_ratio_d128.json")) as f:
        g = json.load(f)
    d, bits = g["dim"], g["bits"]
    x = np.random.default_rng(0).standard_normal((3, d)).astype(np.float32) * np.float32(0.02)
    packed = oracle.quantize_rowwise(x, bits)
    S = packed.shape[1]
    # unpadded row = codes + fp16 scale + fp16 bias
    C = (d * bits + 7) // 8
    unpadded = C + 4
    assert round(100.0 * unpadded / (4.0 * d), 2) == g["percent_of_fp32"]
    assert S % 16 == 0 and S >= unpadded and S - unpadded < 16
    assert np.all(packed[:, unpadded:] == 0)


@pytest.mark.parametrize("dim,bits,stride", [(16, 4, 16), (64, 4, 48), (128, 4, 80), (128, 8, 144),
                                             (1, 4, 16), (12, 8, 16), (13, 8, 32), (24, 4, 16),
                                             (25, 4, 32), (128, 2, 48), (48, 2, 16), (49, 2, 32),
                                             (5, 2, 16)])
def test_row_stride(oracle_lib, dim, bits, stride):
    assert oracle.row_stride(dim, bits) == stride


# ---------------------------------------------------------------------------
# range quantization: closed forms
# ---------------------------------------------------------------------------

def _grid_rows(g, n, dim, bits):
    """Rows x_i = b + k_i * s with s, b binary16 numbers of <= 3 significant
    bits and k containing 0 and Q: every step of the encoding is exact."""
    Q = (1 << bits) - 1
    rows, ks, ss, bs = [], [], [], []
    for _ in range(n):
        s = float(g.choice([1, 3, 5, 7])) * 2.0 ** int(g.integers(-14, -6))
        b = float(g.choice([-7, -5, -3, -1, 0, 1, 3, 5])) * 2.0 ** int(g.integers(-10, -2))
        k = g.integers(0, Q + 1, size=dim)
        if dim >= 2:
            k[g.integers(0, dim)] = 0
            j = g.integers(0, dim)
            while dim > 1 and k[j] == 0 and np.count_nonzero(k == 0) == 1:
                j = g.integers(0, dim)
            k[j] = Q
        x = (b + k.astype(np.float64) * s).astype(np.float32)
        assert np.array_equal(x.astype(np.float64), b + k * s)  # exactly representable
        rows.append(x)
        ks.append(k)
        ss.append(s)
        bs.append(b)
    return np.stack(rows), np.stack(ks), ss, bs


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("dim", [2, 7, 16, 64])
def test_grid_rows_round_trip_exactly(oracle_lib, bits, dim):
    g = np.random.default_rng(100 + dim + bits)
    x, k, ss, bs = _grid_rows(g, 40, dim, bits)
    packed = oracle.quantize_rowwise(x, bits)
    C = (dim * bits + 7) // 8
    for r in range(x.shape[0]):
        q = unpack_codes(packed[r], dim, bits)
        s16, b16, sf, bf = unpack_params(packed[r], dim, bits)
        assert sf == ss[r] and bf == bs[r]
        assert np.array_equal(q, k[r])
        # packing written out independently: low nibble holds the even element
        if bits == 4:
            kk = np.zeros(2 * C, dtype=np.int64)
            kk[:dim] = k[r]
            assert np.array_equal(packed[r, :C], (kk[0::2] | (kk[1::2] << 4)).astype(np.uint8))
        elif bits == 2:
            kk = np.zeros(4 * C, dtype=np.int64)
            kk[:dim] = k[r]
            assert np.array_equal(packed[r, :C], (kk[0::4] | (kk[1::4] << 2) | (kk[2::4] << 4) |
                                                  (kk[3::4] << 6)).astype(np.uint8))
        else:
            assert np.array_equal(packed[r, :C], k[r].astype(np.uint8))
    y = oracle.dequantize(packed, dim, bits)
    assert np.array_equal(y.view(np.uint32), x.view(np.uint32))


def test_constant_rows(oracle_lib):
    vals = np.array([0.0, -0.0, 1.0, -3.5, 0.1, 1e-6, -65504.0, 65504.0, 3e-8, 1234.567],
                    dtype=np.float32)
    for dim in (1, 5, 32):
        x = np.repeat(vals[:, None], dim, axis=1)
        packed = oracle.quantize_rowwise(x, 4)
        y = oracle.dequantize(packed, dim, 4)
        for r, c in enumerate(vals):
            s16, b16, sf, bf = unpack_params(packed[r], dim, 4)
            assert s16 == 0
            assert np.all(unpack_codes(packed[r], dim, 4) == 0)
            hc = np.float32(np.float16(c))
            assert bf == hc and b16 == int(np.array(np.float16(c + np.float32(0))).view(np.uint16))
            assert np.all(y[r] == hc)
            if abs(c) >= 2.0 ** -14:
                assert abs(float(c) - float(hc)) <= 2.0 ** -11 * abs(float(c))
        # +0 folding: a row of -0 stores +0 as its bias
        assert unpack_params(packed[1], dim, 4)[1] == 0


def _ulp32(v):
    v = np.abs(np.asarray(v, dtype=np.float32))
    return (np.nextafter(v, np.float32(np.inf)) - v).astype(np.float64)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("dim", [3, 16, 64, 128])
def test_range_error_bound_and_nearest_code(oracle_lib, bits, dim):
    """Each element lands on the grid point nearest to it (brute force over all
    Q+1 codes), and its error is at most half a step plus how far it lies
    outside the stored window [bf, bf + Q*sf]."""
    g = np.random.default_rng(5 + dim + bits)
    Q = (1 << bits) - 1
    x = (g.standard_normal((200, dim)) * 0.02).astype(np.float32)
    x[:20] *= np.float32(1000.0)
    packed = oracle.quantize_rowwise(x, bits)
    y = oracle.dequantize(packed, dim, bits).astype(np.float64)
    kk = np.arange(Q + 1, dtype=np.float64)
    for r in range(x.shape[0]):
        s16, b16, sf, bf = unpack_params(packed[r], dim, bits)
        lo, hi = float(x[r].min()), float(x[r].max())
        # the stored parameters are the fp16 roundings of the range's step and low end
        assert sf == float(np.float16(np.float32((np.float32(hi) - np.float32(lo)) / np.float32(Q))))
        assert bf == float(np.float16(np.float32(lo)))
        xr = x[r].astype(np.float64)
        grid = (sf * kk + bf).astype(np.float32).astype(np.float64)
        dist = np.abs(xr[:, None] - grid[None, :])
        q = unpack_codes(packed[r], dim, bits)
        chosen = dist[np.arange(dim), q]
        assert np.all(chosen <= dist.min(axis=1) + 4 * _ulp32(xr) + 4 * _ulp32(grid.max()))
        outside = np.maximum.reduce([np.zeros(dim), bf - xr, xr - (bf + Q * sf)])
        bound = sf / 2 * (1 + 1e-5) + outside + 2 * _ulp32(np.maximum(np.abs(xr), np.abs(y[r])))
        assert np.all(np.abs(xr - y[r]) <= bound)
        # the window edges move by at most the fp16 rounding of lo and of the step
        assert abs(lo - bf) <= 2.0 ** -11 * abs(lo) + 2.0 ** -25
        assert abs(hi - (bf + Q * sf)) <= 2.0 ** -11 * abs(lo) + Q * (2.0 ** -11 * sf + 2.0 ** -25) + 2 * _ulp32(hi)


def test_range_codes_are_permutation_equivariant_and_power_of_two_scaled(oracle_lib):
    g = np.random.default_rng(11)
    x = (g.standard_normal((100, 24)) * 0.05).astype(np.float32)
    p0 = oracle.quantize_rowwise(x, 4)
    perm = g.permutation(24)
    p1 = oracle.quantize_rowwise(x[:, perm], 4)
    x2 = (x * np.float32(8.0)).astype(np.float32)
    p2 = oracle.quantize_rowwise(x2, 4)
    for r in range(100):
        q0 = unpack_codes(p0[r], 24, 4)
        assert np.array_equal(unpack_codes(p1[r], 24, 4), q0[perm])
        assert unpack_params(p1[r], 24, 4)[:2] == unpack_params(p0[r], 24, 4)[:2]
        assert np.array_equal(unpack_codes(p2[r], 24, 4), q0)
        _, _, sf0, bf0 = unpack_params(p0[r], 24, 4)
        _, _, sf2, bf2 = unpack_params(p2[r], 24, 4)
        if sf0 >= 2.0 ** -14 and abs(bf0) >= 2.0 ** -14:  # both fp16-normal
            assert sf2 == 8 * sf0 and bf2 == 8 * bf0


def _expected_range_norm_l2(dim, Q, n=200000, seed=3):
    """Textbook uniform-quantization noise: interior elements carry an error
    uniform over one step s = R/Q (variance s^2/12); the two extremes are on
    the grid.  E[R^2] of the range of `dim` standard normals by sampling."""
    g = np.random.default_rng(seed)
    z = g.standard_normal((n // dim + 1, dim))
    R = z.max(axis=1) - z.min(axis=1)
    return math.sqrt((dim - 2) / dim * np.mean(R ** 2) / (12 * Q * Q))


@pytest.mark.parametrize("dim", [16, 64, 128])
def test_range_normalized_l2_matches_uniform_noise_model(oracle_lib, dim):
    g = np.random.default_rng(dim)
    x = (g.standard_normal((4000, dim)) * 0.02).astype(np.float32)
    packed = oracle.quantize_rowwise(x, 4)
    m = oracle.l2_error(x, packed, 4)
    exp = _expected_range_norm_l2(dim, 15)
    assert abs(m["mean_row"] / exp - 1) < 0.08, (m["mean_row"], exp)


def test_l2_error_against_numpy(oracle_lib):
    g = np.random.default_rng(2)
    x = (g.standard_normal((777, 40)) * 0.03).astype(np.float32)
    x[5] = 0.0
    packed = oracle.quantize_rowwise(x, 4)
    y = oracle.dequantize(packed, 40, 4).astype(np.float64)
    xd = x.astype(np.float64)
    en = np.linalg.norm(xd - y, axis=1)
    xn = np.linalg.norm(xd, axis=1)
    keep = xn > 0
    m = oracle.l2_error(x, packed, 4)
    assert m["rows"] == int(keep.sum()) == 776
    assert abs(m["mean_row"] - np.mean(en[keep] / xn[keep])) < 1e-12
    assert abs(m["frobenius"] - np.linalg.norm(xd - y) / np.linalg.norm(xd)) < 1e-12


# ---------------------------------------------------------------------------
# greedy search
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [2, 4, 8])
def test_greedy_with_zero_steps_is_range_encoding(oracle_lib, bits):
    g = np.random.default_rng(21)
    x = (g.standard_normal((300, 33)) * 0.02).astype(np.float32)
    a = oracle.quantize_rowwise(x, bits, oracle.RANGE)
    b, ij = oracle.quantize_rowwise(x, bits, oracle.GREEDY, n_bins=200, n_steps=0, return_window=True)
    assert np.array_equal(a, b) and np.all(ij == 0)


def _sse64(x, packed, dim, bits):
    y = oracle.dequantize(packed, dim, bits).astype(np.float64)
    return ((x.astype(np.float64) - y) ** 2).sum(axis=1)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("dim", [16, 64])
def test_greedy_never_worse_than_range(oracle_lib, bits, dim):
    g = np.random.default_rng(31 + dim)
    x = (g.standard_normal((400, dim)) * 0.02).astype(np.float32)
    mix = g.random((400, dim)) < 0.01
    x = np.where(mix, g.laplace(0, 0.2, size=(400, dim)).astype(np.float32), x)
    pr = oracle.quantize_rowwise(x, bits, oracle.RANGE)
    pg = oracle.quantize_rowwise(x, bits, oracle.GREEDY)
    # the kept window's fp32 row error never exceeds the range window's
    for r in range(400):
        assert oracle.row_sse(x[r], pg[r], bits) <= oracle.row_sse(x[r], pr[r], bits)
    sr, sg = _sse64(x, pr, dim, bits), _sse64(x, pg, dim, bits)
    assert np.all(sg <= sr * (1 + 1e-5) + 1e-12)
    if bits == 4:
        # and on Gaussian rows with rare heavy tails it helps on average
        assert sg.mean() < 0.9 * sr.mean()


def test_greedy_first_move_worked_by_hand(oracle_lib):
    """Row: a cluster 0.00, 0.01, ..., 0.14 and one value at 10 (d=16, INT4,
    200 bins, so one step is 0.05).  At the range window every cluster value
    gets code 0, error sum(x_k^2) ~= 0.1015.  Raising the low end one step puts
    the bias at fp16(0.05) with the cluster still on code 0, error
    sum((x_k - 0.05)^2) ~= 0.0340; lowering the high end instead leaves the
    cluster where it was and adds the outlier's clip error (~0.104).  So the
    walk must first raise the low end, and later steps (whose windows are
    still too wide to resolve the cluster) never beat that window.  The
    mirrored row must lower its high end first."""
    base = np.linspace(0.0, 0.14, 15, dtype=np.float32)
    up = np.concatenate([base, [np.float32(10.0)]]).astype(np.float32)
    down = (-up[::-1]).astype(np.float32)
    pu, ij_up = oracle.quantize_rowwise(up[None], 4, oracle.GREEDY, 200, 100, return_window=True)
    pd, ij_dn = oracle.quantize_rowwise(down[None], 4, oracle.GREEDY, 200, 100, return_window=True)
    assert tuple(ij_up[0]) == (1, 0)
    b = float(np.float16(0.05))
    hand = sum((float(v) - b) ** 2 for v in base)
    assert abs(float(oracle.row_sse(up, pu[0], 4)) / hand - 1) < 1e-3
    assert float(oracle.window_sse(up, 4, 200, 0, 1)) > 0.1
    assert ij_dn[0, 1] >= 1
    assert float(oracle.window_sse(down, 4, 200, 0, 1)) < 0.04 < float(oracle.window_sse(down, 4, 200, 1, 0))


def test_greedy_keeps_an_exactly_representable_row(oracle_lib):
    g = np.random.default_rng(41)
    x, _, _, _ = _grid_rows(g, 30, 16, 4)
    a = oracle.quantize_rowwise(x, 4, oracle.RANGE)
    b, ij = oracle.quantize_rowwise(x, 4, oracle.GREEDY, return_window=True)
    assert np.array_equal(a, b) and np.all(ij == 0)


def test_greedy_best_is_minimum_of_its_walk_and_bounded_by_lattice(oracle_lib):
    """Brute force over every window (i, j) with i + j <= K."""
    g = np.random.default_rng(51)
    K, Bn = 10, 16
    for _ in range(60):
        d = int(g.integers(2, 9))
        x = (g.standard_normal(d) * 0.05).astype(np.float32)
        _, ij = oracle.quantize_rowwise(x[None], 4, oracle.GREEDY, Bn, K, return_window=True)
        L = {(i, j): float(oracle.window_sse(x, 4, Bn, i, j)) for i in range(K + 1) for j in range(K + 1 - i)}
        best = L[(int(ij[0, 0]), int(ij[0, 1]))]
        assert min(L.values()) <= best <= L[(0, 0)]
        # walk the lattice: each move takes the lower neighbour (ties: high end)
        i = j = 0
        seen = [L[(0, 0)]]
        for _s in range(K):
            if L[(i + 1, j)] < L[(i, j + 1)]:
                i += 1
            else:
                j += 1
            seen.append(L[(i, j)])
        assert best == min(seen)


def test_oracle_matches_independent_numpy_model_bit_for_bit(oracle_lib):
    """Tiny rows through both the C oracle and the separately written numpy /
    exact-rounding model: packed bytes must agree exactly."""
    g = np.random.default_rng(61)
    n_cases = 0
    for d in (1, 2, 3, 4, 5, 8, 16):
        for bits in (2, 4, 8):
            for _ in range(12):
                scale = float(g.choice([1e-3, 0.02, 1.0, 300.0]))
                x = (g.standard_normal(d) * scale).astype(np.float32)
                if g.random() < 0.2:
                    x[g.integers(0, d)] = np.float32(-0.0)
                if g.random() < 0.1:
                    x[:] = x[0]
                Bn = int(g.integers(1, 17))
                K = int(g.integers(0, Bn))
                K = min(K, 12)
                for clip in ("range", "greedy"):
                    mode = oracle.RANGE if clip == "range" else oracle.GREEDY
                    ours = oracle.quantize_rowwise(x[None], bits, mode, Bn, K)[0]
                    ref = nm.encode(x, bits, clip, Bn, K)
                    assert np.array_equal(ours, ref), (d, bits, clip, Bn, K, x)
                    n_cases += 1
    assert n_cases == 7 * 3 * 12 * 2


def _tiny_row(g, d):
    """A tiny row of one of the value kinds the rules single out."""
    kind = int(g.integers(0, 9))
    scale = float(g.choice([1e-7, 1e-3, 0.02, 1.0, 300.0, 20000.0]))
    x = (g.standard_normal(d) * scale).astype(np.float32)
    if kind == 1:
        x[:] = x[0]                                            # constant
    elif kind == 2:
        x[g.random(d) < 0.5] = np.float32(-0.0)                # signed zeros
    elif kind == 3:
        x = np.where(g.random(d) < 0.5, -1.5, 2.25).astype(np.float32)   # two values
    elif kind == 4:
        x = (g.integers(-8, 8, size=d) * 0.125).astype(np.float32)       # grid values
    elif kind == 5:
        x = np.clip(x * 4.0, -65504, 65504).astype(np.float32)           # near the fp16 limit
    elif kind == 6:
        x = (g.standard_normal(d) * 1e-40).astype(np.float32)            # fp32 denormals
    elif kind == 7:
        x = g.laplace(0, 0.2, size=d).astype(np.float32)                  # heavy tails
    return np.clip(x, -65504, 65504).astype(np.float32)  # the rules take fp16-range values only


def test_oracle_matches_independent_numpy_model_on_ten_thousand_rows(oracle_lib):
    """10800 tiny rows (d in {1, 2, 3, 4, 8, 16}, INT2/4/8, range and greedy,
    greedy bins 1..16 and steps 0..min(bins - 1, 12)) through the C oracle and the
    independent numpy model: packed bytes identical for every row."""
    g = np.random.default_rng(62)
    n_cases = 0
    for d in (1, 2, 3, 4, 8, 16):
        for bits in (2, 4, 8):
            for _ in range(300):
                x = _tiny_row(g, d)
                Bn = int(g.integers(1, 17))
                K = int(g.integers(0, min(Bn, 13)))  # 0 <= K < Bn, K <= 12
                for clip in ("range", "greedy"):
                    mode = oracle.RANGE if clip == "range" else oracle.GREEDY
                    ours = oracle.quantize_rowwise(x[None], bits, mode, Bn, K)[0]
                    ref = nm.encode(x, bits, clip, Bn, K)
                    assert np.array_equal(ours, ref), (d, bits, clip, Bn, K, x)
                    n_cases += 1
    assert n_cases == 6 * 3 * 300 * 2 >= 10000


def test_oracle_rejects_values_outside_fp16_range(oracle_lib):
    x = np.zeros((2, 4), np.float32)
    x[1, 2] = np.float32(70000.0)
    with pytest.raises(oracle.OracleError):
        oracle.quantize_rowwise(x, 4)
    x[1, 2] = np.float32(np.nan)
    with pytest.raises(oracle.OracleError):
        oracle.quantize_rowwise(x, 4)


# ---------------------------------------------------------------------------
# pooled lookup: library routine and special cases
# ---------------------------------------------------------------------------

def _table(g, rows, dim, bits):
    x = (g.standard_normal((rows, dim)) * 0.05).astype(np.float32)
    return x, oracle.quantize_rowwise(x, bits)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("itype", [np.int32, np.int64])
def test_bag_matches_torch_embedding_bag(oracle_lib, bits, weighted, itype):
    import torch
    g = np.random.default_rng(71)
    dim, T, B = 20, 3, 17
    rows = [50, 1, 33]
    x, packed = _table(g, sum(rows), dim, bits)
    toff = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    lengths = g.integers(0, 6, size=T * B)
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(itype)
    idx = np.concatenate([g.integers(0, rows[gb // B], size=lengths[gb]) for gb in range(T * B)]).astype(itype)
    w = g.random(idx.size).astype(np.float32) if weighted else None
    out, absd, err = oracle.bag_forward(packed, toff, B, dim, bits, idx, offsets, w)
    assert err == 0
    y = torch.from_numpy(oracle.dequantize(packed, dim, bits).astype(np.float64))
    for t in range(T):
        sl = slice(int(offsets[t * B]), int(offsets[(t + 1) * B]))
        ids = torch.from_numpy(idx[sl].astype(np.int64) + toff[t])
        offs = torch.from_numpy((offsets[t * B:(t + 1) * B] - offsets[t * B]).astype(np.int64))
        psw = None if w is None else torch.from_numpy(w[sl].astype(np.float64))
        ref = torch.nn.functional.embedding_bag(ids, y, offs, mode="sum", per_sample_weights=psw).numpy()
        assert np.allclose(out[:, t, :], ref, rtol=1e-12, atol=1e-15)
        absref = torch.nn.functional.embedding_bag(
            ids, y.abs(), offs, mode="sum",
            per_sample_weights=None if psw is None else psw.abs()).numpy()
        assert np.allclose(absd[:, t, :], absref, rtol=1e-12, atol=1e-15)


def test_bag_one_hot_equals_dequantized_row_and_empty_is_zero(oracle_lib):
    g = np.random.default_rng(81)
    dim = 16
    x, packed = _table(g, 40, dim, 4)
    y = oracle.dequantize(packed, dim, 4)
    B = 40
    toff = np.array([0, 40], np.int64)
    idx = np.arange(40, dtype=np.int32)[::-1].copy()
    offsets = np.arange(41, dtype=np.int32)
    out, _, err = oracle.bag_forward(packed, toff, B, dim, 4, idx, offsets)
    assert err == 0 and np.array_equal(out[:, 0, :], y[::-1].astype(np.float64))
    offsets0 = np.zeros(41, np.int32)
    out0, _, err0 = oracle.bag_forward(packed, toff, B, dim, 4, idx, offsets0)
    assert err0 == 0 and np.all(out0 == 0) and not np.any(np.signbit(out0))


def test_bag_skips_and_counts_invalid_ids_and_offsets(oracle_lib):
    g = np.random.default_rng(91)
    dim, B = 8, 4
    rows = [10, 5]
    x, packed = _table(g, 15, dim, 4)
    toff = np.array([0, 10, 15], np.int64)
    # bags: t0: [0,3) [3,5) [5,5) [5,8) ; t1: [8,9) [9,12) [12,11)->bad [11,13)->bad neighbour
    idx = np.array([1, -1, 9, 10, 2, 0, 0, 3, 4, 5, 2, 1, 0], np.int64)
    offsets = np.array([0, 3, 5, 5, 8, 9, 12, 11, 13], np.int64)
    out, _, err = oracle.bag_forward(packed, toff, B, dim, 4, idx, offsets)
    y = oracle.dequantize(packed, dim, 4).astype(np.float64)
    # invalid: idx -1 (t0), idx 10 (t0, only 10 rows), idx 5 (t1, only 5 rows)
    # offsets: bag 6 = [12, 11) decreasing -> empty; bag 7 = [11, 13) valid
    assert err == 4
    assert np.array_equal(out[0, 0], y[1] + y[9])
    assert np.array_equal(out[1, 0], y[2])
    assert np.all(out[2, 0] == 0)
    assert np.array_equal(out[3, 0], y[0] + y[0] + y[3])
    assert np.array_equal(out[0, 1], y[10 + 4])
    assert np.array_equal(out[1, 1], y[10 + 2] + y[10 + 1])   # id 5 skipped
    assert np.all(out[2, 1] == 0)
    assert np.array_equal(out[3, 1], y[10 + 1] + y[10 + 0])
    # a table whose row range leaves the packed buffer: all its terms skipped
    out2, _, err2 = oracle.bag_forward(packed, np.array([0, 10, 16], np.int64), B, dim, 4, idx, offsets,
                                       total_rows=15)
    # table 0: two bad ids; table 1: six terms skipped plus the bad offsets
    assert np.all(out2[:, 1] == 0) and err2 == 2 + 6 + 1


def _walk_events(x, bits, Bn, K):
    """Count, along the greedy walk of the numpy model, the steps whose two
    candidates tie exactly and the steps that equal the best so far."""
    Q = (1 << bits) - 1
    xmin, xmax = nm.row_range(x)
    delta = (xmax - xmin) / np.float32(Bn)

    def L(i, j):
        lo = np.float32(nm.fma32(float(i), float(delta), float(xmin))) + np.float32(0.0)
        hi = np.float32(nm.fma32(-float(j), float(delta), float(xmax))) + np.float32(0.0)
        return nm.window_sse(x, lo, hi, Q)

    i = j = 0
    best = L(0, 0)
    ties = equal_best = 0
    for _ in range(K):
        la, lb = L(i + 1, j), L(i, j + 1)
        ties += int(la == lb)
        if la < lb:
            i, cur = i + 1, la
        else:
            j, cur = j + 1, lb
        equal_best += int(cur == best)
        best = min(best, cur)
    return ties, equal_best


def test_greedy_tie_rules_match_independent_model(oracle_lib):
    """Coarse rows (few distinct values, some below fp16 resolution) make the
    two candidates of a step tie exactly, or a later window equal the best
    one: there the tie rules (a tie moves the high end; only a strictly lower
    error replaces the best window) decide the result.  Both implementations
    must agree bit for bit on such rows."""
    g = np.random.default_rng(6)
    n_tie = n_eq = 0
    for trial in range(2500):
        d = int(g.integers(2, 9))
        Bn = int(g.integers(2, 33))
        K = min(Bn - 1, 12)
        bits = int(g.choice([4, 8]))
        kind = trial % 3
        if kind == 0:
            x = (g.integers(-3, 4, size=d) * 0.25).astype(np.float32)
        elif kind == 1:
            x = g.integers(0, 2, size=d).astype(np.float32)
        else:
            x = (g.integers(-1, 2, size=d) * 2.0 ** int(g.integers(-30, 3))).astype(np.float32)
        if x.min() == x.max():
            continue
        ties, eq = _walk_events(x, bits, Bn, K)
        if not (ties or eq):
            continue
        n_tie += ties > 0
        n_eq += eq > 0
        ours, ij = oracle.quantize_rowwise(x[None], bits, oracle.GREEDY, Bn, K, return_window=True)
        assert np.array_equal(ours[0], nm.encode(x, bits, "greedy", Bn, K)), (x, bits, Bn, K)
        assert tuple(ij[0]) == nm.greedy(x, bits, Bn, K)[2:], (x, bits, Bn, K)
    assert n_tie >= 50 and n_eq >= 50, (n_tie, n_eq)

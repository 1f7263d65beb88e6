"""A second, independent model of the row-wise quantizer, used only to pin
the C oracle.

It follows the same reading of the pages ("Post-Training 4-bit Quantization
on Embedding Tables", review page, "Proposed method": row-wise uniform
quantization, fp16 scale and bias, greedy search of the clipping thresholds
on the row's squared error) but is built from different primitives:

* binary32 operations are numpy float32 array/scalar operations (each
  correctly rounded, never contracted);
* fused multiply-adds are evaluated exactly (binary64 when an error-free
  check proves the sum exact, else ``fractions.Fraction``) and rounded once to
  binary32 by a rounding routine written here from the IEEE-754 format;
* binary16 rounding is numpy's float16 conversion;
* the row error is summed pairwise bottom-up (adjacent pairs, then adjacent
  pairs of those), which is the same tree as summing contiguous halves.

Slow; meant for rows of a few elements.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

F32 = np.float32


def _round_fraction_f32(a: Fraction, neg_zero: bool = False) -> np.float32:
    """Round an exact rational to the nearest binary32 (ties to even)."""
    if a == 0:
        return F32(-0.0) if neg_zero else F32(0.0)
    sign = -1 if a < 0 else 1
    a = abs(a)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    if r >= Fraction(2) ** 128:
        return F32(sign * np.inf)
    return F32(sign * float(r))


def fma32(a, b, c) -> np.ndarray:
    """Element-wise a*b + c with one rounding to binary32.  a*b must be exact
    in binary64 (true for the operand widths used here)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    a, b, c = np.broadcast_arrays(a, b, c)
    p = a * b
    s = p + c
    # TwoSum: s is the exact sum iff the recovered error term is zero
    bb = s - p
    err = (p - (s - bb)) + (c - bb)
    out = s.astype(np.float32)
    inexact = np.nonzero(err != 0)[0] if out.ndim else ([] if err == 0 else [None])
    if out.ndim == 0:
        if err != 0:
            return _round_fraction_f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))
        return F32(out)
    for k in inexact:
        out[k] = _round_fraction_f32(Fraction(float(a[k])) * Fraction(float(b[k])) + Fraction(float(c[k])))
    return out


def half(x) -> np.float32:
    return F32(np.float16(F32(x)))


def half_bits(x) -> int:
    return int(np.array(np.float16(F32(x))).view(np.uint16))


def pairwise(u: np.ndarray) -> np.float32:
    n = 1
    while n < u.size:
        n *= 2
    v = np.zeros(n, dtype=np.float32)
    v[:u.size] = u
    while v.size > 1:
        v = (v[0::2] + v[1::2]).astype(np.float32)
    return F32(v[0])


def row_range(x: np.ndarray):
    return F32(x.min()) + F32(0.0), F32(x.max()) + F32(0.0)


def params(lo, hi, Q):
    s = (F32(hi) - F32(lo)) / F32(Q)
    if not s > 0:
        s = F32(0.0)
    return half_bits(s), half_bits(lo), half(s), half(lo)


def codes(x, sf, bf, Q):
    if sf == 0:
        return np.zeros(x.size, dtype=np.int64)
    r = F32(1.0) / F32(sf)
    t = (x - F32(bf)).astype(np.float32) * r
    q = np.rint(t.astype(np.float32))
    return np.clip(q, 0, Q).astype(np.int64)


def dequant(q, sf, bf):
    return fma32(np.full(q.size, sf, np.float64), q.astype(np.float64), np.full(q.size, bf, np.float64))


def window_sse(x, lo, hi, Q):
    _, _, sf, bf = params(lo, hi, Q)
    q = codes(x, sf, bf, Q)
    y = dequant(q, sf, bf)
    e = (x - y).astype(np.float32)
    return pairwise((e * e).astype(np.float32))


def greedy(x, bits, n_bins, n_steps):
    """Returns (lo, hi, i, j) of the kept window."""
    Q = (1 << bits) - 1
    xmin, xmax = row_range(x)
    if xmax == xmin:
        return xmin, xmax, 0, 0
    delta = (xmax - xmin) / F32(n_bins)

    def lo_at(i):
        return F32(fma32(float(i), float(delta), float(xmin))) + F32(0.0)

    def hi_at(j):
        return F32(fma32(-float(j), float(delta), float(xmax))) + F32(0.0)

    i = j = 0
    best = window_sse(x, lo_at(0), hi_at(0), Q)
    bi = bj = 0
    for _ in range(n_steps):
        la = window_sse(x, lo_at(i + 1), hi_at(j), Q)
        lb = window_sse(x, lo_at(i), hi_at(j + 1), Q)
        if la < lb:
            i, cur = i + 1, la
        else:
            j, cur = j + 1, lb
        if cur < best:
            best, bi, bj = cur, i, j
    return lo_at(bi), hi_at(bj), bi, bj


def encode(x, bits, clip="range", n_bins=200, n_steps=100):
    """Packed row bytes (codes | s16 LE | b16 LE | zero pad to 16 B)."""
    x = np.asarray(x, dtype=np.float32)
    Q = (1 << bits) - 1
    if clip == "range":
        lo, hi = row_range(x)
    else:
        lo, hi, _, _ = greedy(x, bits, n_bins, n_steps)
    s16, b16, sf, bf = params(lo, hi, Q)
    q = codes(x, sf, bf, Q)
    return _pack(q, bits, s16, b16)


# ---- codebook rows: 16 levels from 1-D k-means (Lloyd), 4-bit codes ----

def codebook(x, n_iter=10):
    """(levels[16] float32, codes[d]) by the codebook rule: start at the
    row's uniform grid, n_iter rounds of nearest-level assignment (lowest
    index on ties) and member means (pairwise member sum / count), then the
    final assignment."""
    x = np.asarray(x, dtype=np.float32)
    lo, hi = row_range(x)
    delta = (F32(hi) - F32(lo)) / F32(15)
    c = np.array([fma32(F32(k), delta, lo) + F32(0.0) for k in range(16)], dtype=np.float32)

    def assign(c):
        dist = np.abs((x[:, None] - c[None, :]).astype(np.float32))
        return np.argmin(dist, axis=1)  # first minimum: lowest index on ties

    for _ in range(n_iter):
        a = assign(c)
        nxt = c.copy()
        for k in range(16):
            m = a == k
            if m.any():
                v = np.where(m, x, F32(0.0)).astype(np.float32)
                nxt[k] = F32(pairwise(v) / F32(int(m.sum()))) + F32(0.0)
        c = nxt
    return c, assign(c)


def encode_codebook(x, n_iter=10):
    """Packed codebook row bytes (16 levels fp32 LE | codes | zero pad to 16 B)."""
    x = np.asarray(x, dtype=np.float32)
    c, q = codebook(x, n_iter)
    d = x.size
    C = (d + 1) // 2
    S = (64 + C + 15) // 16 * 16
    row = np.zeros(S, dtype=np.uint8)
    row[:64] = np.frombuffer(c.astype("<f4").tobytes(), dtype=np.uint8)
    qq = np.zeros(2 * C, dtype=np.int64)
    qq[:d] = q
    row[64:64 + C] = (qq[0::2] | (qq[1::2] << 4)).astype(np.uint8)
    return row


# ---- quantizer baselines: symmetric, percentile clipping, ACIQ ----

def encode_symmetric(x, bits):
    """Symmetric row: s = max|x| / (2^(b-1) - 1) in fp16 (capped at
    65504 / 2^(b-1)), codes rint(x * (1/s)) clamped to +-(2^(b-1) - 1) and
    stored + 2^(b-1), bias -2^(b-1) s."""
    x = np.asarray(x, dtype=np.float32)
    H = 1 << (bits - 1)
    m = F32(np.max(np.abs(x)))
    sf = half(m / F32(H - 1))
    if sf > F32(65504.0 / H):
        sf = F32(65504.0 / H)
    s16 = half_bits(sf)
    b16 = half_bits(F32(-H) * sf)
    if sf == 0:
        q = np.zeros(x.size, dtype=np.int64)
    else:
        r = F32(1.0) / sf
        q = np.clip(np.rint((x * r).astype(np.float32)), -(H - 1), H - 1).astype(np.int64)
    return _pack(q + H, bits, s16, b16)


def _pack(codes, bits, s16, b16):
    """Row bytes: codes (8 / bits per byte, element i at bits
    bits * (i mod per) of byte i // per), fp16 scale and bias little-endian,
    zero padding to 16 bytes."""
    d = codes.size
    C = (d * bits + 7) // 8
    S = (C + 4 + 15) // 16 * 16
    row = np.zeros(S, dtype=np.uint8)
    per = 8 // bits
    qq = np.zeros(per * C, dtype=np.int64)
    qq[:d] = codes
    acc = np.zeros(C, dtype=np.int64)
    for j in range(per):
        acc |= qq[j::per] << (bits * j)
    row[:C] = acc.astype(np.uint8)
    row[C:C + 2] = [s16 & 0xFF, s16 >> 8]
    row[C + 2:C + 4] = [b16 & 0xFF, b16 >> 8]
    return row


def percentile_window(x, p):
    v = np.sort(np.asarray(x, dtype=np.float32), kind="stable")
    d = v.size

    def qnt(q):
        h = F32(d - 1) * F32(q)
        i = int(np.floor(h))
        if i >= d - 1:
            return F32(v[d - 1])
        f = F32(h - F32(i))
        return F32(fma32(float(f), float(F32(v[i + 1] - v[i])), float(v[i])))

    return qnt(F32(1.0) - F32(p)) + F32(0.0), qnt(p) + F32(0.0)


def aciq_window(x, bits, ratio):
    """ratio: the clip ratio a/b as a float32."""
    x = np.asarray(x, dtype=np.float32)
    mn, mx = row_range(x)
    mu = F32(pairwise(x) / F32(x.size))
    b = F32(pairwise(np.abs((x - mu).astype(np.float32))) / F32(x.size))
    a = F32(F32(ratio) * b)
    lo, hi = F32(mu - a), F32(mu + a)
    return max(lo, mn) + F32(0.0), min(hi, mx) + F32(0.0)


def encode_window(x, bits, lo, hi):
    x = np.asarray(x, dtype=np.float32)
    Q = (1 << bits) - 1
    s16, b16, sf, bf = params(lo, hi, Q)
    return _pack(codes(x, sf, bf, Q), bits, s16, b16)

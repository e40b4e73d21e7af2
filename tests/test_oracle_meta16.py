"""Pins of the oracle's bfloat16 metadata (meta_bits = 16): each statistic of
Algorithm 1 is rounded to a bfloat16 value where it is produced and used
from there on.  What fixes it:

* every stored statistic is a bfloat16 value;
* gamma_min is the binary32 run's value (a minimum of bfloat16 inputs);
  gamma_scale is the smallest bfloat16 >= max - min; mu is the nearest
  bfloat16 (ties to even) of the balanced-tree mean of the oracle's own X_norm,
  recomputed here; sigma is the smallest bfloat16 >= max |X_cent| of the
  oracle's own X_cent;
* Stage 1 / Stage 2 ranges still hold (X_norm in [0, 1], |X_final| <= 1) on
  the single page and every adversarial page;
* every full reconstruction lies within its code's cell around the level,
  scaled back with the stored (rounded) statistics, plus rounding.
"""
import math

import numpy as np
import pytest

import oracle
from progressive_kv_transfer_amd import kvgen


def bits(t):
    return kvgen.bf16_bits(t)


def f32_bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def is_bf16(a):
    return bool(np.all((f32_bits(a) & 0xFFFF) == 0))


def bf16_ceil(v):
    """Smallest bfloat16 >= v >= 0, by search over bfloat16 patterns."""
    u = int(np.float32(v).view(np.uint32))
    hi = u >> 16
    for cand in (hi, hi + 1):
        f = np.uint32(cand << 16).view(np.float32)
        if f >= np.float32(v):
            return np.float32(f)
    raise AssertionError(v)


def bf16_nearest(v):
    """Nearest bfloat16 of a binary32 value, ties to even, by comparing the
    two bracketing bfloat16 values exactly in binary64."""
    v = np.float32(v)
    u = int(v.view(np.uint32))
    lo = np.uint32((u >> 16) << 16).view(np.float32)
    hi = np.uint32(((u >> 16) + 1) << 16).view(np.float32)
    if lo == v:
        return lo
    dl, dh = abs(float(v) - float(lo)), abs(float(hi) - float(v))
    if dl != dh:
        return lo if dl < dh else hi
    return lo if ((u >> 16) & 1) == 0 else hi


def tree_mean(x):
    x = [np.float32(v) for v in x]
    while len(x) > 1:
        x = [np.float32(x[2 * i] + x[2 * i + 1]) for i in range(len(x) // 2)]
    return np.float32(x[0] / np.float32(32.0))


def pages():
    yield "single_k", bits(kvgen.CONFIGS["single_page"].make()[0])
    yield "single_v", bits(kvgen.CONFIGS["single_page"].make()[1])
    for name, t in sorted(kvgen.edge_pages().items()):
        yield name, bits(t)


@pytest.mark.parametrize("name,x", list(pages()))
def test_statistics_are_rounded_where_produced(name, x):
    r32 = oracle.quantize_block(x)
    r16 = oracle.quantize_block(x, meta_bits=16)
    for s in ("gamma_min", "gamma_scale", "mu", "sigma"):
        assert is_bf16(getattr(r16, s)), (name, s)
    assert np.array_equal(f32_bits(r16.gamma_min), f32_bits(r32.gamma_min))
    for c in range(x.shape[1]):
        assert r16.gamma_scale[c] == bf16_ceil(r32.gamma_scale[c]), (name, c)
        for j in range(8):
            xn = r16.xn[c, 32 * j:32 * j + 32]
            assert r16.mu[j, c] == bf16_nearest(tree_mean(xn)), (name, c, j)
            xc = r16.xcent[c, 32 * j:32 * j + 32]
            assert r16.sigma[j, c] == bf16_ceil(np.max(np.abs(xc))), (name, c, j)


@pytest.mark.parametrize("name,x", list(pages()))
def test_ranges_still_hold(name, x):
    r = oracle.quantize_block(x, meta_bits=16)
    assert np.all(r.xn >= 0.0) and np.all(r.xn <= 1.0), name
    assert np.all(np.abs(r.xfinal) <= 1.0), name


def _cell(alpha, cs):
    la = math.log1p(alpha)
    thr = [math.expm1((k - 0.5) / cs * la) / alpha for k in range(129)]
    thr[0] = 0.0
    lev = [math.expm1(k / cs * la) / alpha for k in range(128)]
    return thr, lev


def test_reconstruction_within_code_cell_with_stored_statistics():
    alpha, eps, cs = 255.0, 1e-6, 120.0
    thr, lev = _cell(alpha, cs)
    for name, x in pages():
        r = oracle.quantize_block(x, alpha=alpha, eps=eps, code_scale=cs, meta_bits=16)
        out = oracle.dequant_block(r, True, alpha=alpha, eps=eps, code_scale=cs)
        xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        xr = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        P, H = x.shape
        for c in range(H):
            d1 = float(r.gamma_scale[c]) + eps
            for t in range(P):
                d2 = float(r.sigma[t // 32, c]) + eps
                code = min(int(r.code_raw[c, t]), 120)
                hi = 1.0 if code >= 120 else thr[code + 1]
                dev = max(lev[code] - thr[code], hi - lev[code])
                ulp_bf16 = 2.0 ** (math.frexp(max(abs(xr[t, c]), 1e-38))[1] - 8)
                slack = 1e-6 * (abs(xf[t, c]) + abs(float(r.gamma_min[c])) + d1) + ulp_bf16
                assert abs(xf[t, c] - xr[t, c]) <= dev * d2 * d1 * (1 + 1e-5) + slack, \
                    (name, c, t)


def test_rejects_other_metadata_widths():
    x = bits(kvgen.CONFIGS["single_page"].make()[0])
    for m in (0, 8, 24, 64):
        with pytest.raises(ValueError):
            oracle.quantize_block(x, meta_bits=m)

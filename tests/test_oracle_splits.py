"""Pins of the oracle's other splits of the 8-bit code (a anchor bits,
b = 8 - a residual bits; the paper's Algorithm 1 Stage 4 is a = b = 4 with
the bias +7 = 2^(b-1) - 1).  What fixes them:

* the largest storable code is the largest I whose anchor magnitude
  (I + 2^(b-1) - 1) >> b fits an a-bit two's-complement field (brute force);
* exhaustively over every code and sign: the fields fit their widths,
  (V << b) - Q_res = I, the anchor's sign is S, the decoder inverts the
  split, and the anchor-only level V << b is the multiple of 2^b nearest to
  I (within (-2^(b-1), 2^(b-1)]);
* the stream layout: a Python bit reader over the packed bytes returns the
  fields that the split of the oracle's own codes (recomputed here in
  Python) gives, at bit w (2 i + e) of each (chunk, pair) run;
* with a >= 4 and the default code scale no code is clipped, so the full
  reconstruction equals the paper's 4 + 4 one bit for bit, and the
  anchor-only reconstruction of every split is within its cell (the codes
  sharing the anchor) around the level, scaled back, plus rounding.
"""
import math

import numpy as np
import pytest

import oracle
from progressive_kv_transfer_amd import kvgen

SPLITS = [3, 4, 5, 6]


def bits(t):
    return kvgen.bf16_bits(t)


def bf16_to_f32(u16):
    return (u16.astype(np.uint32) << 16).view(np.float32)


def sext(f, w):
    f &= (1 << w) - 1
    return f - (1 << w) if f >> (w - 1) else f


@pytest.mark.parametrize("a", SPLITS)
def test_code_max_is_the_largest_storable_code(a):
    b = 8 - a
    fits = [i for i in range(256) if (i + (1 << (b - 1)) - 1) >> b <= (1 << (a - 1)) - 1]
    assert oracle.code_max(a) == max(fits)
    assert oracle.code_max(4) == 120


@pytest.mark.parametrize("a", SPLITS)
def test_split_exhaustive(a):
    b = 8 - a
    for i in range(oracle.code_max(a) + 1):
        for s in (1, -1):
            v, q_res, q_anc = oracle.split(i, s, a)
            assert 0 <= v <= (1 << (a - 1)) - 1
            assert -(1 << (b - 1)) <= q_res <= (1 << (b - 1)) - 1
            assert -(1 << (a - 1)) <= q_anc <= (1 << (a - 1)) - 1
            assert (v << b) - q_res == i
            assert (q_anc < 0) == (s < 0)
            # anchor-only level: nearest multiple of 2^b
            assert -(1 << (b - 1)) < i - (v << b) <= (1 << (b - 1))
            mask_a, mask_b = (1 << a) - 1, (1 << b) - 1
            assert oracle.unsplit(q_anc & mask_a, q_res & mask_b, a) == (i, s)
            assert oracle.unsplit(q_anc & mask_a, None, a) == (v << b, s)
            if a == 4:
                assert (v, q_res, q_anc) == oracle.split(i, s)


def read_field(run, pos, w):
    val = int.from_bytes(bytes(run), "little")
    return (val >> pos) & ((1 << w) - 1)


@pytest.mark.parametrize("a", SPLITS)
def test_stream_layout(a):
    b = 8 - a
    x = bits(kvgen.CONFIGS["single_page"].make()[0])
    r = oracle.quantize_block(x, anchor_bits=a)
    P, H = x.shape
    C = 32
    imax = oracle.code_max(a)
    assert r.anchor.shape == (P // C, H // 2, C * a // 4)
    assert r.residual.shape == (P // C, H // 2, C * b // 4)
    for t in range(0, P, 7):
        j, i = divmod(t, C)
        for c in range(0, H, 5):
            code = min(int(r.code_raw[c, t]), imax)
            s = int(r.sign[c, t])
            v = (code + (1 << (b - 1)) - 1) >> b
            q_res = (v << b) - code
            q_anc = v if s > 0 else -v - 1
            k, e = divmod(c, 2)
            fa = read_field(r.anchor[j, k], a * (2 * i + e), a)
            fr = read_field(r.residual[j, k], b * (2 * i + e), b)
            assert sext(fa, a) == q_anc, (t, c)
            assert sext(fr, b) == q_res, (t, c)


@pytest.mark.parametrize("a", [5, 6])
def test_full_reconstruction_independent_of_split(a):
    """Codes up to 120 fit every split with a >= 4: the full code, and so the
    full reconstruction, is the same as with the paper's split."""
    for x in (bits(t) for t in kvgen.CONFIGS["single_page"].make()):
        r4 = oracle.quantize_block(x)
        ra = oracle.quantize_block(x, anchor_bits=a)
        assert np.array_equal(r4.code_raw, ra.code_raw)
        assert np.array_equal(oracle.dequant_block(r4, True), oracle.dequant_block(ra, True))
        assert np.array_equal(r4.mu, ra.mu) and np.array_equal(r4.sigma, ra.sigma)


def _thr_lev(alpha, code_scale):
    la = math.log1p(alpha)
    thr = [math.expm1((k - 0.5) / code_scale * la) / alpha for k in range(129)]
    thr[0] = 0.0
    lev = [math.expm1(k / code_scale * la) / alpha for k in range(128)]
    return thr, lev


@pytest.mark.parametrize("a", SPLITS)
def test_anchor_only_error_within_the_anchor_cell(a):
    """Anchor-only reconstruction of every element lies within the cell of
    codes that share its anchor (codes 2^b V - 2^(b-1) + 1 .. 2^b V +
    2^(b-1), clipped to the storable range) around the level of V << b,
    scaled back by (sigma + eps)(gamma_scale + eps), plus binary32 and bf16
    rounding; the scale is the split's largest code so nothing clips."""
    b = 8 - a
    alpha, eps = 255.0, 1e-6
    imax = oracle.code_max(a)
    cs = float(imax)
    thr, lev = _thr_lev(alpha, cs)
    for x in (bits(t) for t in kvgen.CONFIGS["single_page"].make()):
        r = oracle.quantize_block(x, alpha=alpha, eps=eps, code_scale=cs, anchor_bits=a)
        out = oracle.dequant_block(r, False, alpha=alpha, eps=eps, code_scale=cs)
        xf = bf16_to_f32(x).astype(np.float64)
        xr = bf16_to_f32(out).astype(np.float64)
        P, H = x.shape
        for c in range(H):
            d1 = float(r.gamma_scale[c]) + eps
            for t in range(P):
                d2 = float(r.sigma[t // 32, c]) + eps
                code = min(int(r.code_raw[c, t]), imax)
                v = (code + (1 << (b - 1)) - 1) >> b
                lo_code = max((v << b) - (1 << (b - 1)) + 1, 0)
                hi_code = min((v << b) + (1 << (b - 1)), imax)
                rec = lev[v << b]
                lo = thr[lo_code]
                hi = 1.0 if hi_code >= imax else thr[hi_code + 1]
                dev = max(rec - lo, hi - rec)
                ulp_bf16 = 2.0 ** (math.frexp(max(abs(xr[t, c]), 1e-38))[1] - 8)
                slack = 1e-6 * (abs(xf[t, c]) + abs(float(r.gamma_min[c])) + d1) + ulp_bf16
                assert abs(xf[t, c] - xr[t, c]) <= dev * d2 * d1 * (1 + 1e-5) + slack, (c, t)


def test_fewer_anchor_bits_coarser_draft():
    """The anchor-only error grows as anchor bits are taken away (mean
    squared error over a page at each split's own scale)."""
    x = bits(kvgen.CONFIGS["single_page"].make()[0])
    xf = bf16_to_f32(x).astype(np.float64)
    errs = []
    for a in SPLITS:
        cs = float(oracle.code_max(a))
        r = oracle.quantize_block(x, code_scale=cs, anchor_bits=a)
        xr = bf16_to_f32(oracle.dequant_block(r, False, code_scale=cs)).astype(np.float64)
        errs.append(float(np.mean((xf - xr) ** 2)))
    assert errs[0] > errs[1] > errs[2] > errs[3], errs


def test_rejects_bad_split():
    x = bits(kvgen.CONFIGS["single_page"].make()[0])
    for a, b in ((0, None), (1, None), (1, 0), (9, 0), (5, 4), (4, 5), (3, 3)):
        with pytest.raises(ValueError):
            oracle.quantize_block(x, anchor_bits=a, residual_bits=b)

"""CPU oracle for the Lynx hierarchical split-stream quantizer.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark are the only callers.  The GPU library never imports,
links or calls this package, and the two share no code.

The arithmetic lives in ``lynx_oracle.c`` (plain C, binary32 with one
rounding per operation, compander decision and attention in binary64); this
module only compiles it with gcc and marshals numpy arrays through ctypes.
It follows "Lynx: Progressive Speculative Quantization for accelerating KV
Transfer in Long-Context Inference", Section 4.1, Algorithm 1 and Eq. (3)-(4),
and the reading notes "Lynx 阅读笔记", section "具体算例" (worked example).

Pins of every function (tests/test_oracle_*.py) hold it to what the pages and
the mathematics fix; see the docstring of each wrapper for its pin.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lynx_oracle.c")

# Plain scalar build: no FMA contraction, no fast-math, SSE binary32.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-fno-unsafe-math-optimizations", "-Wall"]

# LYNX_ORACLE_SANITIZE=1 selects a separate build of the same source with
# AddressSanitizer and UndefinedBehaviorSanitizer (every report fatal), for
# running the CPU test suite under the sanitizers.  Python itself is not
# instrumented, so that run preloads the ASan runtime:
#   LD_PRELOAD=$(gcc -print-file-name=libasan.so) \
#   ASAN_OPTIONS=detect_leaks=0 LYNX_ORACLE_SANITIZE=1 \
#   python -m pytest tests -m "not gpu"
SANITIZE = os.environ.get("LYNX_ORACLE_SANITIZE", "") == "1"
SAN_FLAGS = ["-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-g"]
_LIB = os.path.join(_HERE, "liblynx_oracle_san.so" if SANITIZE else "liblynx_oracle.so")

_lock = threading.Lock()
_lib = None

P_DEFAULT, C_DEFAULT, H_DEFAULT = 256, 32, 128
# Top of the compander's code range: Eq. (3) prints 2^7 - 1 = 127, but a
# 4-bit anchor (Algorithm 1 Stage 4: magnitude (I + 7) >> 4 <= 7) carries
# codes up to 120 only; the compander is scaled to 120 so that every
# |X_final| in [0, 1] keeps its code (127 with the clip at 120 remains a
# parameter value).
CODE_SCALE = 120.0


def build(force: bool = True) -> str:
    """Compile lynx_oracle.c into liblynx_oracle.so with gcc."""
    if not force and os.path.exists(_LIB) and \
            os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", *CFLAGS, *(SAN_FLAGS if SANITIZE else []), "-o", tmp,
                           _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or \
                    os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            L = ctypes.CDLL(_LIB)
            i64, i32, f32, f64 = (ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                                  ctypes.c_double)
            vp = ctypes.c_void_p
            L.oracle_code.restype = i32
            L.oracle_code.argtypes = [f32, f32, f32]
            L.oracle_code_real.restype = f64
            L.oracle_code_real.argtypes = [f32, f32, f32]
            L.oracle_level.restype = f32
            L.oracle_level.argtypes = [i32, f32, f32]
            L.oracle_code_max.restype = i32
            L.oracle_code_max.argtypes = [i32, i32]
            L.oracle_split_bits.restype = None
            L.oracle_split_bits.argtypes = [i32, i32, i32, i32, ctypes.POINTER(i32),
                                            ctypes.POINTER(i32), ctypes.POINTER(i32)]
            L.oracle_unsplit_bits.restype = i32
            L.oracle_unsplit_bits.argtypes = [ctypes.c_uint, i32, ctypes.c_uint, i32, i32,
                                              ctypes.POINTER(i32)]
            L.oracle_quantize_block_bits.restype = i32
            L.oracle_quantize_block_bits.argtypes = [
                vp, i64, i32, i32, i32, f32, f32, f32, i32, i32, i32, vp, vp, vp, vp, vp,
                vp, vp, vp, vp, vp, vp]
            L.oracle_dequant_block_bits.restype = i32
            L.oracle_dequant_block_bits.argtypes = [
                vp, vp, vp, vp, vp, vp, i32, i32, i32, f32, f32, f32, i32, i32, vp, i64]
            L.oracle_quantize_bits.restype = i32
            L.oracle_quantize_bits.argtypes = [
                vp, i64, i64, i64, i64, i64, i32, i32, i32, f32, f32, f32, i32, i32, i32,
                i64, i64, i64, vp, vp, vp, vp, vp, vp]
            L.oracle_dequant_bits.restype = i32
            L.oracle_dequant_bits.argtypes = [
                vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32, i32,
                f32, f32, f32, i32, i32, i64, i64, i64, vp]
            L.oracle_spec_verify.restype = i32
            L.oracle_spec_verify.argtypes = [vp, vp, vp, vp, f64, i32, i32,
                                             ctypes.POINTER(i32), ctypes.POINTER(i32)]
            L.oracle_attention.restype = i32
            L.oracle_attention.argtypes = [
                vp, vp, vp, i32, i32, i32, i32, i64, f64, i32, i32, i32, vp]
            _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"] or a.ndim == 0
    return a.ctypes.data


# ---------------------------------------------------------------- scalars --

def code(x_abs: float, alpha: float = 255.0, code_scale: float = CODE_SCALE) -> int:
    """Round(Eq. (3)) of one binary32 magnitude, before the 120 clip."""
    return lib().oracle_code(x_abs, alpha, code_scale)


def code_real(x_abs: float, alpha: float = 255.0, code_scale: float = CODE_SCALE) -> float:
    """Y of Eq. (3) in binary64 (used to measure rounding margins)."""
    return lib().oracle_code_real(x_abs, alpha, code_scale)


def level(k: int, alpha: float = 255.0, code_scale: float = CODE_SCALE) -> float:
    """Reconstruction magnitude of code k (inverse of Eq. (3))."""
    return lib().oracle_level(k, alpha, code_scale)


def residual_width(anchor_bits: int, residual_bits: int | None) -> int:
    """Residual field width: 8 - a for a split of the 8-bit code unless given
    (0 = a single a-bit stream, the paper's Lynx-INT4 / Lynx-INT8)."""
    return 8 - anchor_bits if residual_bits is None else residual_bits


def code_max(anchor_bits: int = 4, residual_bits: int | None = None) -> int:
    """Largest code whose anchor magnitude fits an anchor_bits-bit anchor:
    2^7 - 2^(b-1) for a split (120 for the paper's 4 + 4), 2^(a-1) - 1 for
    a single stream."""
    return lib().oracle_code_max(anchor_bits, residual_width(anchor_bits, residual_bits))


def split(code_c: int, sign: int, anchor_bits: int = 4, residual_bits: int | None = None):
    """Algorithm 1 Stage 4 on one clipped code: returns (V_mag, Q_res, Q_anc)
    (the paper's 4 + 4 split by default)."""
    v, r, a = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    lib().oracle_split_bits(code_c, sign, anchor_bits,
                            residual_width(anchor_bits, residual_bits), ctypes.byref(v),
                            ctypes.byref(r), ctypes.byref(a))
    return v.value, r.value, a.value


def unsplit(anchor_field: int, residual_field: int | None, anchor_bits: int = 4,
            residual_bits: int | None = None):
    """Decoder side of Stage 4: (code, sign) from the anchor field (and the
    residual field for the full code)."""
    s = ctypes.c_int()
    c = lib().oracle_unsplit_bits(anchor_field, residual_field is not None,
                                  residual_field or 0, anchor_bits,
                                  residual_width(anchor_bits, residual_bits), ctypes.byref(s))
    return c, s.value


# ------------------------------------------------------------ page blocks --

class BlockResult:
    """Outputs of one oracle page block (plus optional intermediates)."""

    def __init__(self, H, P, C, anchor_bits=4, residual_bits=None):
        nch = P // C
        self.C, self.anchor_bits = C, anchor_bits
        self.residual_bits = residual_width(anchor_bits, residual_bits)
        # chunk-tiled streams: [chunk][channel pair][run of 2C w-bit fields]
        # (for w = 4: [chunk][channel pair][token of the chunk])
        self.anchor = np.zeros((nch, H // 2, C * anchor_bits // 4), np.uint8)
        self.residual = np.zeros((nch, H // 2, C * self.residual_bits // 4), np.uint8)
        self.gamma_min = np.zeros(H, np.float32)
        self.gamma_scale = np.zeros(H, np.float32)
        self.mu = np.zeros((nch, H), np.float32)
        self.sigma = np.zeros((nch, H), np.float32)
        self.xn = np.zeros((H, P), np.float32)
        self.xcent = np.zeros((H, P), np.float32)
        self.xfinal = np.zeros((H, P), np.float32)
        self.code_raw = np.zeros((H, P), np.int32)
        self.sign = np.zeros((H, P), np.int8)


def quantize_block(x_bf16: np.ndarray, alpha=255.0, eps=1e-6, code_scale=CODE_SCALE,
                   C=C_DEFAULT, anchor_bits=4, residual_bits=None,
                   meta_bits=32) -> BlockResult:
    """Quantize one page block given token-major as uint16 bf16 bits [P][H].
    meta_bits = 16: the statistics are rounded to bfloat16 where they are
    produced (their float32 arrays then hold bfloat16 values)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    P, H = x.shape
    r = BlockResult(H, P, C, anchor_bits, residual_bits)
    rc = lib().oracle_quantize_block_bits(
        _ptr(x), H, H, P, C, alpha, eps, code_scale, anchor_bits, r.residual_bits,
        meta_bits, _ptr(r.anchor), _ptr(r.residual) if r.residual_bits else None, _ptr(r.gamma_min), _ptr(r.gamma_scale), _ptr(r.mu),
        _ptr(r.sigma), _ptr(r.xn), _ptr(r.xcent), _ptr(r.xfinal),
        _ptr(r.code_raw), _ptr(r.sign))
    if rc:
        raise ValueError("oracle_quantize_block_bits rejected the block")
    return r


def dequant_block(r: BlockResult, full: bool, alpha=255.0, eps=1e-6,
                  code_scale=CODE_SCALE) -> np.ndarray:
    """Reconstruct a block from its codes: anchor-only or anchor + residual
    (a single stream has no residual: its anchor is the whole code)."""
    if full and not r.residual_bits:
        raise ValueError("a single-stream code has no residual")
    nch, Hh = r.anchor.shape[:2]
    C = r.C
    P, H = nch * C, Hh * 2
    out = np.zeros((P, H), np.uint16)
    rc = lib().oracle_dequant_block_bits(
        _ptr(r.anchor), _ptr(r.residual) if full else None, _ptr(r.gamma_min),
        _ptr(r.gamma_scale), _ptr(r.mu), _ptr(r.sigma), H, P, C, alpha, eps,
        code_scale, r.anchor_bits, r.residual_bits, _ptr(out), H)
    if rc:
        raise ValueError("oracle_dequant_block_bits rejected the block")
    return out


# ---------------------------------------------------------------- tensors --

class Codes:
    """Oracle outputs for a KV set of num_tensors [T][Ch] tensors."""

    def __init__(self, nblocks, H=H_DEFAULT, P=P_DEFAULT, C=C_DEFAULT, anchor_bits=4,
                 residual_bits=None):
        self.nblocks = nblocks
        self.anchor_bits = anchor_bits
        self.residual_bits = residual_width(anchor_bits, residual_bits)
        self.anchor = np.zeros((nblocks, P // C, H // 2, C * anchor_bits // 4), np.uint8)
        self.residual = np.zeros((nblocks, P // C, H // 2, C * self.residual_bits // 4),
                                 np.uint8)
        self.gamma_min = np.zeros((nblocks, H), np.float32)
        self.gamma_scale = np.zeros((nblocks, H), np.float32)
        self.mu = np.zeros((nblocks, P // C, H), np.float32)
        self.sigma = np.zeros((nblocks, P // C, H), np.float32)


def _ranges(n, parts):
    parts = max(1, min(parts, n))
    step = (n + parts - 1) // parts
    return [(b, min(n, b + step)) for b in range(0, n, step)]


def quantize(kv: np.ndarray, alpha=255.0, eps=1e-6, code_scale=CODE_SCALE,
             H=H_DEFAULT, P=P_DEFAULT, C=C_DEFAULT, threads=1,
             blocks: tuple[int, int] | None = None, anchor_bits=4,
             residual_bits=None, meta_bits=32) -> Codes:
    """Quantize kv (uint16 bf16 bits, shape [num_tensors, T, Ch]).

    ``blocks=(b0, b1)`` restricts the work (and the returned arrays) to page
    blocks b0..b1-1 of the global block order.  ``threads`` splits the block
    range over Python threads (the C call releases the GIL).
    """
    kv = np.ascontiguousarray(kv, dtype=np.uint16)
    nt, T, Ch = kv.shape
    nblocks = nt * (T // P) * (Ch // H)
    b0, b1 = blocks if blocks is not None else (0, nblocks)
    out = Codes(b1 - b0, H, P, C, anchor_bits, residual_bits)
    L = lib()

    def run(r):
        lo, hi = r
        rc = L.oracle_quantize_bits(
            _ptr(kv), nt, T * Ch, T, Ch, Ch, H, P, C, alpha, eps, code_scale,
            anchor_bits, out.residual_bits, meta_bits, lo, hi, b0, _ptr(out.anchor),
            _ptr(out.residual) if out.residual_bits else None,
            _ptr(out.gamma_min), _ptr(out.gamma_scale), _ptr(out.mu),
            _ptr(out.sigma))
        if rc:
            raise ValueError("oracle_quantize rejected the arguments")

    ranges = [(lo + b0, hi + b0) for lo, hi in _ranges(b1 - b0, threads)]
    if len(ranges) == 1:
        run(ranges[0])
    else:
        with ThreadPoolExecutor(len(ranges)) as ex:
            list(ex.map(run, ranges))
    return out


def dequant(codes: Codes, shape, full: bool, alpha=255.0, eps=1e-6,
            code_scale=CODE_SCALE, H=H_DEFAULT, P=P_DEFAULT, C=C_DEFAULT, threads=1,
            blocks: tuple[int, int] | None = None) -> np.ndarray:
    """Reconstruct bf16 bits [num_tensors, T, Ch] from codes.

    With ``blocks=(b0, b1)`` the codes hold blocks b0..b1-1 only and only
    those blocks of the output are written (the rest stays zero).
    """
    nt, T, Ch = shape
    nblocks = nt * (T // P) * (Ch // H)
    b0, b1 = blocks if blocks is not None else (0, nblocks)
    assert codes.nblocks == b1 - b0
    rbits = getattr(codes, "residual_bits", 8 - getattr(codes, "anchor_bits", 4))
    if full and not rbits:
        raise ValueError("a single-stream code has no residual")
    out = np.zeros((nt, T, Ch), np.uint16)
    L = lib()

    def run(r):
        lo, hi = r
        rc = L.oracle_dequant_bits(
            _ptr(codes.anchor), _ptr(codes.residual) if full else None,
            _ptr(codes.gamma_min), _ptr(codes.gamma_scale), _ptr(codes.mu),
            _ptr(codes.sigma), nt, T * Ch, T, Ch, Ch, H, P, C, alpha, eps,
            code_scale, getattr(codes, "anchor_bits", 4), rbits, lo, hi, b0, _ptr(out))
        if rc:
            raise ValueError("oracle_dequant rejected the arguments")

    ranges = [(lo + b0, hi + b0) for lo, hi in _ranges(b1 - b0, threads)]
    if len(ranges) == 1:
        run(ranges[0])
    else:
        with ThreadPoolExecutor(len(ranges)) as ex:
            list(ex.map(run, ranges))
    return out


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              causal_tail: bool, threads=1) -> np.ndarray:
    """softmax(q k^T * scale) v in binary64 over bf16 bits.

    q: [t_q, n_qh, d], k / v: [ctx, n_kvh, d] (uint16 bf16 bits).
    Returns float64 [t_q, n_qh, d].
    """
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    t_q, n_qh, d = q.shape
    ctx, n_kvh, _ = k.shape
    out = np.zeros((t_q, n_qh, d), np.float64)
    L = lib()

    def run(r):
        lo, hi = r
        rc = L.oracle_attention(_ptr(q), _ptr(k), _ptr(v), t_q, n_qh, n_kvh, d,
                                ctx, scale, int(causal_tail), lo, hi, _ptr(out))
        if rc:
            raise ValueError("oracle_attention rejected the arguments")

    ranges = _ranges(n_qh, threads)
    if len(ranges) == 1:
        run(ranges[0])
    else:
        with ThreadPoolExecutor(len(ranges)) as ex:
            list(ex.map(run, ranges))
    return out


def spec_verify(draft_logits: np.ndarray, target_logits: np.ndarray, tokens: np.ndarray,
                u_accept: np.ndarray, u_sample: float):
    """Speculative verification (accept prefix, correct at the first
    rejection): returns (n_accepted, next_token)."""
    d = np.ascontiguousarray(draft_logits, np.float32)
    t = np.ascontiguousarray(target_logits, np.float32)
    s = np.ascontiguousarray(tokens, np.int32)
    u = np.ascontiguousarray(u_accept, np.float64)
    T, V = d.shape
    assert t.shape == (T + 1, V) and s.shape == (T,) and u.shape == (T,)
    n, tok = ctypes.c_int(0), ctypes.c_int(0)
    rc = lib().oracle_spec_verify(_ptr(d), _ptr(t), _ptr(s), _ptr(u), float(u_sample), T, V,
                                  ctypes.byref(n), ctypes.byref(tok))
    if rc:
        raise ValueError("oracle_spec_verify rejected the arguments")
    return n.value, tok.value

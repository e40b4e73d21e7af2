"""Thin Python binding of liblynx.so (include/lynx.h).

Same names as the C ABI; this module only marshals torch tensors (device
memory) and the current torch stream into the C calls.  All arithmetic runs
in the library's HIP kernels.  If liblynx.so is missing or cannot be loaded
every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblynx.so")

PAGE_TOKENS = 256
CHUNK_TOKENS = 32
BLOCK_CHANNELS = 128
OUT_BF16, OUT_F32 = 0, 1  # lynx_decode_attn_dequant output element types
STATUS = {0: "LYNX_OK", -1: "LYNX_EINVAL", -2: "LYNX_ESHAPE", -3: "LYNX_EHIP",
          -4: "LYNX_ESCRATCH"}
ATTN_SCRATCH_BYTES = 24 << 20  # LYNX_ATTN_SCRATCH_BYTES


class LynxError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({text})")
        self.status = status


class lynx_params(ctypes.Structure):
    _fields_ = [("alpha", ctypes.c_float), ("eps", ctypes.c_float),
                ("code_scale", ctypes.c_float), ("page_tokens", ctypes.c_int32),
                ("chunk_tokens", ctypes.c_int32), ("block_channels", ctypes.c_int32),
                ("anchor_bits", ctypes.c_int32), ("residual_bits", ctypes.c_int32),
                ("meta_bits", ctypes.c_int32), ("layout", ctypes.c_int32)]


class lynx_kv_shape(ctypes.Structure):
    _fields_ = [("num_tensors", ctypes.c_int64), ("tensor_stride", ctypes.c_int64),
                ("num_tokens", ctypes.c_int64), ("num_channels", ctypes.c_int64),
                ("row_stride", ctypes.c_int64)]


class lynx_meta(ctypes.Structure):
    _fields_ = [("gamma_min", ctypes.c_void_p), ("gamma_scale", ctypes.c_void_p),
                ("mu", ctypes.c_void_p), ("sigma", ctypes.c_void_p)]


class lynx_codes(ctypes.Structure):
    _fields_ = [("anchor", ctypes.c_void_p), ("residual", ctypes.c_void_p),
                ("meta", lynx_meta)]


class lynx_transfer_times(ctypes.Structure):
    _fields_ = [(n, ctypes.c_float) for n in ("quantized", "anchor_arrived", "residual_arrived",
                                              "first_anchor_ready", "anchor_ready",
                                              "full_ready")]


TRANSFER_COPIES_ONLY = 1
LAYOUT_SEPARATE, LAYOUT_PACKED = 0, 1  # lynx_params.layout

# Every symbol include/lynx.h declares.
EXPORTS = ["lynx_default_params", "lynx_num_blocks", "lynx_stream_bytes",
           "lynx_field_stream_bytes",
           "lynx_gamma_floats", "lynx_chunk_floats", "lynx_anchor_block_bytes",
           "lynx_kv_bytes",
           "lynx_status_string", "lynx_compander_thresholds", "lynx_quantize_pages", "lynx_dequant_anchor",
           "lynx_dequant_full", "lynx_page_stats", "lynx_block_stats",
           "lynx_attn_workspace_bytes", "lynx_decode_attn_dequant",
           "lynx_decode_attn_dequant_noalloc",
           "lynx_split_stream_transfer", "lynx_codec_stream_create", "lynx_stream_destroy",
           "lynx_spec_verify_workspace_bytes", "lynx_spec_verify"]

_lib = None


def lib():
    """Load liblynx.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built: run "
                "`python -m progressive_kv_transfer_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        P = ctypes.POINTER
        L.lynx_default_params.argtypes = [P(lynx_params)]
        L.lynx_default_params.restype = None
        L.lynx_num_blocks.argtypes = [P(lynx_kv_shape)]
        L.lynx_num_blocks.restype = i64
        for f in ("lynx_stream_bytes", "lynx_gamma_floats", "lynx_chunk_floats"):
            getattr(L, f).argtypes = [P(lynx_kv_shape)]
            getattr(L, f).restype = ctypes.c_size_t
        L.lynx_anchor_block_bytes.argtypes = [P(lynx_params)]
        L.lynx_anchor_block_bytes.restype = ctypes.c_size_t
        L.lynx_field_stream_bytes.argtypes = [P(lynx_kv_shape), i32]
        L.lynx_field_stream_bytes.restype = ctypes.c_size_t
        L.lynx_kv_bytes.argtypes = [i64] * 5
        L.lynx_kv_bytes.restype = ctypes.c_uint64
        L.lynx_compander_thresholds.argtypes = [P(lynx_params), vp]
        L.lynx_compander_thresholds.restype = i32
        L.lynx_status_string.argtypes = [i32]
        L.lynx_status_string.restype = ctypes.c_char_p
        L.lynx_quantize_pages.argtypes = [vp, P(lynx_kv_shape), P(lynx_params), vp, vp,
                                          lynx_meta, vp]
        L.lynx_dequant_anchor.argtypes = [vp, lynx_meta, P(lynx_kv_shape), P(lynx_params),
                                          vp, vp]
        L.lynx_dequant_full.argtypes = [vp, vp, lynx_meta, P(lynx_kv_shape),
                                        P(lynx_params), vp, vp]
        L.lynx_page_stats.argtypes = [vp, P(lynx_kv_shape), P(lynx_params), vp, vp, vp]
        L.lynx_block_stats.argtypes = [vp, P(lynx_kv_shape), P(lynx_params), vp, vp, vp,
                                       vp, vp]
        L.lynx_attn_workspace_bytes.argtypes = [i32, i32, i32, i64]
        L.lynx_attn_workspace_bytes.restype = ctypes.c_size_t
        L.lynx_decode_attn_dequant.argtypes = [vp, i32, i32, vp, vp, lynx_meta, vp, vp,
                                               lynx_meta, i64, i32, i32, ctypes.c_float, i32,
                                               P(lynx_params), vp, i32, vp, ctypes.c_size_t,
                                               vp]
        L.lynx_decode_attn_dequant_noalloc.argtypes = [
            vp, i32, i32, vp, vp, lynx_meta, vp, vp, lynx_meta, i64, i32, i32,
            ctypes.c_float, i32, P(lynx_params), vp, i32, vp]
        L.lynx_split_stream_transfer.argtypes = [vp, P(lynx_kv_shape), P(lynx_params), i64,
                                                 lynx_codes, lynx_codes, lynx_codes, vp, vp,
                                                 i32, vp, vp, vp, vp, P(lynx_transfer_times)]
        L.lynx_codec_stream_create.argtypes = [i32, P(vp)]
        L.lynx_stream_destroy.argtypes = [vp]
        L.lynx_spec_verify_workspace_bytes.argtypes = [i32, i32]
        L.lynx_spec_verify_workspace_bytes.restype = ctypes.c_size_t
        L.lynx_spec_verify.argtypes = [vp, vp, vp, vp, ctypes.c_double, i32, i32, vp, vp,
                                       ctypes.c_size_t, vp]
        for f in ("lynx_quantize_pages", "lynx_dequant_anchor", "lynx_dequant_full",
                  "lynx_page_stats", "lynx_block_stats", "lynx_decode_attn_dequant",
                  "lynx_decode_attn_dequant_noalloc",
                  "lynx_split_stream_transfer", "lynx_spec_verify",
                  "lynx_codec_stream_create", "lynx_stream_destroy"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


def _check(fn, rc):
    if rc != 0:
        raise LynxError(fn, rc, lib().lynx_status_string(rc).decode())


def params(alpha=255.0, eps=1e-6, code_scale=120.0, anchor_bits=4,
           residual_bits=None, meta_bits=32, layout=LAYOUT_SEPARATE) -> lynx_params:
    """Method parameters; anchor_bits, residual_bits = widths of the anchor
    and residual fields: 4 + 4 is the paper's split, 3..6 + 8 - a the other
    splits of the 8-bit code (residual_bits None means 8 - anchor_bits), and
    residual_bits = 0 with anchor_bits 4 or 8 a single stream (the paper's
    Lynx-INT4 / Lynx-INT8, with code_scale 7 / 127); meta_bits = 16 keeps the
    metadata in bfloat16 (4 + 4 only); layout = LAYOUT_PACKED stores each
    block's anchor stream followed by its metadata in one record."""
    p = lynx_params()
    lib().lynx_default_params(ctypes.byref(p))
    p.alpha, p.eps, p.code_scale, p.anchor_bits = alpha, eps, code_scale, anchor_bits
    p.residual_bits = 8 - anchor_bits if residual_bits is None else residual_bits
    p.meta_bits = meta_bits
    p.layout = layout
    return p


def anchor_block_bytes(p: lynx_params | None = None) -> int:
    """Bytes per page block of the anchor-side buffer (the packed record
    with LAYOUT_PACKED)."""
    n = int(lib().lynx_anchor_block_bytes(ctypes.byref(p) if p else None))
    if n == 0:
        raise ValueError("anchor_block_bytes: invalid parameters")
    return n


def code_max(anchor_bits: int = 4, residual_bits: int | None = None) -> int:
    """Largest storable code: 128 - 2^(b - 1) for a split (120 for 4 + 4),
    2^(a - 1) - 1 for a single stream (b = 0)."""
    b = 8 - anchor_bits if residual_bits is None else residual_bits
    return (1 << (anchor_bits - 1)) - 1 if b == 0 else 128 - (1 << (b - 1))


def shape_of(kv: torch.Tensor) -> lynx_kv_shape:
    """lynx_kv_shape of a [num_tensors, T, Ch] (or [T, Ch]) tensor view."""
    if kv.dim() == 2:
        kv = kv.unsqueeze(0)
    if kv.dim() != 3 or kv.stride(2) != 1:
        raise ValueError("KV must be [num_tensors, tokens, channels] with unit channel stride")
    s = lynx_kv_shape()
    s.num_tensors, s.num_tokens, s.num_channels = kv.shape
    s.tensor_stride, s.row_stride = kv.stride(0), kv.stride(1)
    return s


def kv_bytes(k_factor, seq_len, hidden, layers, precision_bytes) -> int:
    """Eq. (1) of the paper through the library."""
    return lib().lynx_kv_bytes(k_factor, seq_len, hidden, layers, precision_bytes)


def compander_thresholds(p: lynx_params | None = None):
    """The 128 binary32 thresholds of lynx_compander_thresholds (host only)."""
    import numpy as np
    out = np.zeros(128, np.float32)
    _check("lynx_compander_thresholds", lib().lynx_compander_thresholds(
        ctypes.byref(p) if p else None, out.ctypes.data))
    return out


def num_blocks(shape: lynx_kv_shape) -> int:
    n = lib().lynx_num_blocks(ctypes.byref(shape))
    if n < 0:
        _check("lynx_num_blocks", int(n))
    return int(n)


@dataclass
class Codes:
    """Device buffers of one quantized KV set (layouts of include/lynx.h).
    With the packed layout `records` is the anchor-side buffer (one record
    of anchor stream + metadata per block) and `anchor` and the four
    metadata tensors are views into it."""
    anchor: torch.Tensor       # uint8 [nblocks, 8 chunks, 64 channel pairs, 32 tokens]
    residual: torch.Tensor     # uint8 [nblocks, 8, 64, 32]
    gamma_min: torch.Tensor    # float32 [nblocks, 128]
    gamma_scale: torch.Tensor  # float32 [nblocks, 128]
    mu: torch.Tensor           # float32 [nblocks, 8, 128]
    sigma: torch.Tensor        # float32 [nblocks, 8, 128]
    records: torch.Tensor | None = None  # uint8 [nblocks, record bytes] (packed)

    @property
    def packed(self) -> bool:
        return self.records is not None

    def anchor_ptr(self) -> int:
        return (self.records if self.packed else self.anchor).data_ptr()

    def meta(self) -> lynx_meta:
        m = lynx_meta()  # all NULL with the packed layout
        if not self.packed:
            m.gamma_min, m.gamma_scale = self.gamma_min.data_ptr(), self.gamma_scale.data_ptr()
            m.mu, m.sigma = self.mu.data_ptr(), self.sigma.data_ptr()
        return m

    def c_struct(self) -> lynx_codes:
        c = lynx_codes()
        c.anchor, c.residual = self.anchor_ptr(), self.residual.data_ptr()
        c.meta = self.meta()
        return c

    def tensors(self):
        return (self.anchor, self.residual, self.gamma_min, self.gamma_scale, self.mu,
                self.sigma)


def alloc_codes(nblocks: int, device, pin_memory: bool = False, anchor_bits: int = 4,
                residual_bits: int | None = None, meta_bits: int = 32,
                layout: int = LAYOUT_SEPARATE) -> Codes:
    """Code buffers for nblocks page blocks on `device`; on the CPU with
    pin_memory=True they are pinned host memory (a transfer's wire).  The
    streams hold [block][chunk][channel pair][run of 8 w bytes] with
    w = anchor_bits for the anchor, residual_bits (default 8 - anchor_bits)
    for the residual (for w = 4 the run is the pair's 32 tokens, one byte
    each); a single stream (residual_bits 0) has an empty residual; with
    meta_bits = 16 the metadata tensors are bfloat16."""
    b = 8 - anchor_bits if residual_bits is None else residual_bits
    u8 = dict(dtype=torch.uint8, device=device, pin_memory=pin_memory)
    f32 = dict(dtype=torch.bfloat16 if meta_bits == 16 else torch.float32, device=device,
               pin_memory=pin_memory)
    tile = (nblocks, PAGE_TOKENS // CHUNK_TOKENS, BLOCK_CHANNELS // 2)
    if layout == LAYOUT_PACKED:
        mdt = f32["dtype"]
        esz = 2 if meta_bits == 16 else 4
        sbytes = 4096 * anchor_bits
        rec = sbytes + 2304 * esz
        records = torch.empty((nblocks, rec), **u8)
        meta = records.view(mdt)  # [nblocks, rec / esz]
        m0 = sbytes // esz
        return Codes(records[:, :sbytes].view(tile + (8 * anchor_bits,)),
                     torch.empty(tile + (8 * b,), **u8),
                     meta[:, m0:m0 + 128], meta[:, m0 + 128:m0 + 256],
                     meta[:, m0 + 256:m0 + 1280].view(nblocks, 8, 128),
                     meta[:, m0 + 1280:m0 + 2304].view(nblocks, 8, 128), records)
    return Codes(torch.empty(tile + (8 * anchor_bits,), **u8),
                 torch.empty(tile + (8 * b,), **u8),
                 torch.empty((nblocks, BLOCK_CHANNELS), **f32),
                 torch.empty((nblocks, BLOCK_CHANNELS), **f32),
                 torch.empty((nblocks, PAGE_TOKENS // CHUNK_TOKENS, BLOCK_CHANNELS), **f32),
                 torch.empty((nblocks, PAGE_TOKENS // CHUNK_TOKENS, BLOCK_CHANNELS), **f32))


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _require_cuda(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("lynx calls take device tensors")


def _fields(p: lynx_params | None):
    """(anchor_bits, residual_bits, metadata dtype) of p (None = defaults)."""
    if p is None:
        return 4, 4, torch.float32
    return p.anchor_bits, p.residual_bits, \
        torch.bfloat16 if p.meta_bits == 16 else torch.float32


def _check_codes(fn: str, codes: Codes, nblocks: int, p: lynx_params | None = None,
                 residual: bool = True, device: bool = True):
    """The library writes and reads code buffers through bare pointers: make
    sure each one is a dense tensor of the right type that holds nblocks
    page blocks (on the device unless device=False: a transfer's wire may be
    pinned host memory)."""
    a, b, mdt = _fields(p)
    packed = p is not None and p.layout == LAYOUT_PACKED
    if packed != codes.packed:
        raise ValueError(f"{fn}: the code buffers' layout differs from the parameters' "
                         f"({'packed' if packed else 'separate'} expected)")
    if packed:
        need = [("records", codes.records, torch.uint8, nblocks * anchor_block_bytes(p))]
    else:
        need = [("anchor", codes.anchor, torch.uint8, nblocks * 4096 * a),
                ("gamma_min", codes.gamma_min, mdt, nblocks * BLOCK_CHANNELS),
                ("gamma_scale", codes.gamma_scale, mdt, nblocks * BLOCK_CHANNELS),
                ("mu", codes.mu, mdt, nblocks * 8 * BLOCK_CHANNELS),
                ("sigma", codes.sigma, mdt, nblocks * 8 * BLOCK_CHANNELS)]
    if residual and b:
        need.append(("residual", codes.residual, torch.uint8, nblocks * 4096 * b))
    for name, t, dt, n in need:
        if device and not t.is_cuda:
            raise ValueError(f"{fn}: {name} must be a device tensor")
        if t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"{fn}: {name} must be a contiguous {dt} tensor")
        if t.numel() < n:
            raise ValueError(f"{fn}: {name} holds {t.numel()} elements, "
                             f"{n} needed for {nblocks} page blocks")


def _check_kv(fn: str, name: str, t: torch.Tensor, shape: lynx_kv_shape):
    """A bf16 device tensor whose memory covers every element `shape` addresses."""
    if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous():
        raise ValueError(f"{fn}: {name} must be a contiguous bf16 device tensor")
    if shape.num_tensors > 0 and shape.num_tokens > 0 and shape.num_channels > 0:
        extent = ((shape.num_tensors - 1) * shape.tensor_stride +
                  (shape.num_tokens - 1) * shape.row_stride + shape.num_channels)
        if t.numel() < extent:
            raise ValueError(f"{fn}: {name} holds {t.numel()} elements, {extent} addressed")


def quantize_pages(kv: torch.Tensor, p: lynx_params | None = None,
                   out: Codes | None = None, stream=None) -> Codes:
    """lynx_quantize_pages on a bf16 [num_tensors, T, Ch] device tensor."""
    _require_cuda(kv)
    if kv.dtype != torch.bfloat16:
        raise ValueError("KV must be bfloat16")
    sh = shape_of(kv)
    nb = num_blocks(sh)
    codes = out if out is not None else alloc_codes(
        nb, kv.device, anchor_bits=p.anchor_bits if p else 4,
        residual_bits=p.residual_bits if p else 4, meta_bits=p.meta_bits if p else 32,
        layout=p.layout if p else LAYOUT_SEPARATE)
    _check_codes("quantize_pages", codes, nb, p)
    single = p is not None and p.residual_bits == 0
    _check("lynx_quantize_pages", lib().lynx_quantize_pages(
        kv.data_ptr(), ctypes.byref(sh), ctypes.byref(p) if p else None,
        codes.anchor_ptr(), None if single else codes.residual.data_ptr(), codes.meta(),
        _stream(stream)))
    return codes


def dequant_anchor(codes: Codes, out: torch.Tensor, p: lynx_params | None = None,
                   stream=None) -> torch.Tensor:
    """lynx_dequant_anchor into a bf16 [num_tensors, T, Ch] device tensor."""
    _require_cuda(out)
    if out.dtype != torch.bfloat16:
        raise ValueError("dequant_anchor: out must be bfloat16")
    sh = shape_of(out)
    _check_codes("dequant_anchor", codes, num_blocks(sh), p, residual=False)
    _check("lynx_dequant_anchor", lib().lynx_dequant_anchor(
        codes.anchor_ptr(), codes.meta(), ctypes.byref(sh),
        ctypes.byref(p) if p else None, out.data_ptr(), _stream(stream)))
    return out


def dequant_full(codes: Codes, out: torch.Tensor, p: lynx_params | None = None,
                 stream=None) -> torch.Tensor:
    """lynx_dequant_full into a bf16 [num_tensors, T, Ch] device tensor."""
    _require_cuda(out)
    if out.dtype != torch.bfloat16:
        raise ValueError("dequant_full: out must be bfloat16")
    sh = shape_of(out)
    _check_codes("dequant_full", codes, num_blocks(sh), p)
    _check("lynx_dequant_full", lib().lynx_dequant_full(
        codes.anchor_ptr(), codes.residual.data_ptr(), codes.meta(), ctypes.byref(sh),
        ctypes.byref(p) if p else None, out.data_ptr(), _stream(stream)))
    return out


def _blocks_of(sh: lynx_kv_shape) -> int:
    """Page blocks of a shape, computed here (no library call); shapes the
    library refuses count as 0 blocks and are left to its status code."""
    if min(sh.num_tensors, sh.num_tokens, sh.num_channels) < 0 or \
            sh.num_tokens % PAGE_TOKENS or sh.num_channels % BLOCK_CHANNELS:
        return 0
    return sh.num_tensors * (sh.num_tokens // PAGE_TOKENS) * (sh.num_channels // BLOCK_CHANNELS)


def _check_stats(fn: str, kv: torch.Tensor, arrays, p: lynx_params | None):
    """The statistics calls: a bf16 KV set and float32 arrays (binary32
    metadata only) of at least the listed element counts per page block, all
    on the device; checked before any library call (types and sizes first,
    then placement)."""
    if kv.dtype != torch.bfloat16:
        raise ValueError(f"{fn}: kv must be bfloat16")
    # the shape comes from the view's own strides, so it addresses only the
    # view's elements
    sh = shape_of(kv)
    if p is not None and p.meta_bits != 32:
        raise ValueError(f"{fn}: the statistics calls write binary32 metadata")
    nb = _blocks_of(sh)
    for name, t, per_block in arrays:
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{fn}: {name} must be a contiguous float32 tensor")
        if t.numel() < nb * per_block:
            raise ValueError(f"{fn}: {name} holds {t.numel()} elements, "
                             f"{nb * per_block} needed for {nb} page blocks")
    for name, t in [("kv", kv)] + [(n, t) for n, t, _ in arrays]:
        if not t.is_cuda:
            raise ValueError(f"{fn}: {name} must be a device tensor")
    return sh


def page_stats(kv: torch.Tensor, gamma_min: torch.Tensor, gamma_scale: torch.Tensor,
               p: lynx_params | None = None, stream=None):
    """lynx_page_stats (Stage 1 statistics only)."""
    sh = _check_stats("page_stats", kv, (("gamma_min", gamma_min, BLOCK_CHANNELS),
                                         ("gamma_scale", gamma_scale, BLOCK_CHANNELS)), p)
    _check("lynx_page_stats", lib().lynx_page_stats(
        kv.data_ptr(), ctypes.byref(sh), ctypes.byref(p) if p else None,
        gamma_min.data_ptr(), gamma_scale.data_ptr(), _stream(stream)))


def block_stats(kv: torch.Tensor, gamma_min: torch.Tensor, gamma_scale: torch.Tensor,
                mu: torch.Tensor, sigma: torch.Tensor, p: lynx_params | None = None,
                stream=None):
    """lynx_block_stats (Stage 2 statistics given Stage 1's)."""
    chunk = PAGE_TOKENS // CHUNK_TOKENS * BLOCK_CHANNELS
    sh = _check_stats("block_stats", kv, (("gamma_min", gamma_min, BLOCK_CHANNELS),
                                          ("gamma_scale", gamma_scale, BLOCK_CHANNELS),
                                          ("mu", mu, chunk), ("sigma", sigma, chunk)), p)
    _check("lynx_block_stats", lib().lynx_block_stats(
        kv.data_ptr(), ctypes.byref(sh), ctypes.byref(p) if p else None,
        gamma_min.data_ptr(), gamma_scale.data_ptr(), mu.data_ptr(), sigma.data_ptr(),
        _stream(stream)))


@dataclass
class CodeView:
    """One quantized tensor inside a Codes set: blocks [b0, b1) and whether the
    residual stream takes part (False = anchor-only reconstruction)."""
    codes: Codes
    b0: int
    b1: int
    full: bool = True

    def _ptr(self, t: torch.Tensor, per_block: int) -> int:
        return t.data_ptr() + self.b0 * per_block * t.element_size()

    def anchor(self) -> int:
        if self.codes.packed:
            return self._ptr(self.codes.records, self.codes.records[0].numel())
        return self._ptr(self.codes.anchor, self.codes.anchor[0].numel())

    def residual(self):
        return self._ptr(self.codes.residual, self.codes.residual[0].numel()) if self.full \
            else None

    def meta(self) -> lynx_meta:
        c = self.codes
        m = lynx_meta()
        if c.packed:
            return m  # all NULL: the metadata sits in the records
        m.gamma_min = self._ptr(c.gamma_min, c.gamma_min[0].numel())
        m.gamma_scale = self._ptr(c.gamma_scale, c.gamma_scale[0].numel())
        m.mu = self._ptr(c.mu, c.mu[0].numel())
        m.sigma = self._ptr(c.sigma, c.sigma[0].numel())
        return m


def attn_workspace_bytes(t_q: int, num_q_heads: int, num_kv_heads: int, ctx_len: int) -> int:
    return int(lib().lynx_attn_workspace_bytes(t_q, num_q_heads, num_kv_heads, ctx_len))


def decode_attn_dequant(q: torch.Tensor, k: CodeView, v: CodeView, ctx_len: int,
                        num_kv_heads: int, scale: float, causal_tail: bool = False,
                        p: lynx_params | None = None, out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, stream=None,
                        out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """lynx_decode_attn_dequant: q bf16 [t_q, num_q_heads, 128] on the device;
    k / v the code views of one [ctx_len, num_kv_heads * 128] tensor each;
    the output is bf16 or float32 (out_dtype, or the dtype of `out`)."""
    _require_cuda(q)
    if q.dtype != torch.bfloat16 or q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous bf16 [t_q, num_q_heads, head_dim] tensor")
    t_q, nqh, hd = q.shape
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if out.dtype not in (torch.bfloat16, torch.float32) or out.shape != q.shape \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 or float32 tensor shaped like q")
    code = OUT_F32 if out.dtype == torch.float32 else OUT_BF16
    if ctx_len > 0 and ctx_len % PAGE_TOKENS == 0 and num_kv_heads > 0:
        # (other sizes are refused by the library)
        nb = ctx_len // PAGE_TOKENS * num_kv_heads
        for name, view in (("k", k), ("v", v)):
            if not 0 <= view.b0 <= view.b1 or view.b1 - view.b0 != nb:
                raise ValueError(f"decode_attn_dequant: the {name} view must hold the {nb} "
                                 f"page blocks of a [{ctx_len}, {num_kv_heads} x 128] tensor")
            _check_codes("decode_attn_dequant", view.codes, view.b1, p, residual=view.full)
    _require_cuda(out)
    need = attn_workspace_bytes(t_q, nqh, num_kv_heads, ctx_len)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _require_cuda(workspace)
    if not workspace.is_contiguous():
        raise ValueError("decode_attn_dequant: workspace must be a contiguous device tensor")
    _check("lynx_decode_attn_dequant", lib().lynx_decode_attn_dequant(
        q.data_ptr(), t_q, nqh, k.anchor(), k.residual(), k.meta(), v.anchor(), v.residual(),
        v.meta(), ctx_len, num_kv_heads, hd, scale, int(causal_tail),
        ctypes.byref(p) if p else None, out.data_ptr(), code, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def decode_attn_dequant_noalloc(q: torch.Tensor, k: CodeView, v: CodeView, ctx_len: int,
                                num_kv_heads: int, scale: float, out: torch.Tensor,
                                causal_tail: bool = False, p: lynx_params | None = None,
                                stream=None) -> torch.Tensor:
    """lynx_decode_attn_dequant_noalloc: decode_attn_dequant with the split
    partials in the library's fixed device scratch.  Nothing is allocated,
    here or in the library: the caller passes `out` (bf16 or float32 shaped
    like q)."""
    _require_cuda(q, out)
    if q.dtype != torch.bfloat16 or q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous bf16 [t_q, num_q_heads, head_dim] tensor")
    t_q, nqh, hd = q.shape
    if out.dtype not in (torch.bfloat16, torch.float32) or out.shape != q.shape \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 or float32 tensor shaped like q")
    code = OUT_F32 if out.dtype == torch.float32 else OUT_BF16
    if ctx_len > 0 and ctx_len % PAGE_TOKENS == 0 and num_kv_heads > 0:
        nb = ctx_len // PAGE_TOKENS * num_kv_heads
        for name, view in (("k", k), ("v", v)):
            if not 0 <= view.b0 <= view.b1 or view.b1 - view.b0 != nb:
                raise ValueError(f"decode_attn_dequant_noalloc: the {name} view must hold the "
                                 f"{nb} page blocks of a [{ctx_len}, {num_kv_heads} x 128] "
                                 f"tensor")
            _check_codes("decode_attn_dequant_noalloc", view.codes, view.b1, p,
                         residual=view.full)
    _check("lynx_decode_attn_dequant_noalloc", lib().lynx_decode_attn_dequant_noalloc(
        q.data_ptr(), t_q, nqh, k.anchor(), k.residual(), k.meta(), v.anchor(), v.residual(),
        v.meta(), ctx_len, num_kv_heads, hd, scale, int(causal_tail),
        ctypes.byref(p) if p else None, out.data_ptr(), code, _stream(stream)))
    return out


class CodecStream:
    """lynx_codec_stream_create: a stream of the current device whose kernels
    leave `reserved_cus` compute units free (for the runtime's copy kernels
    during a transfer); `.stream` is the torch view of it.  Destroyed by
    close() or when the object goes away (after the caller has synchronized
    it)."""

    def __init__(self, reserved_cus: int = 16):
        h = ctypes.c_void_p()
        _check("lynx_codec_stream_create",
               lib().lynx_codec_stream_create(int(reserved_cus), ctypes.byref(h)))
        self.handle = h.value
        self.reserved_cus = int(reserved_cus)
        self.stream = torch.cuda.ExternalStream(self.handle)

    def close(self):
        if self.handle:
            self.stream.synchronize()
            h, self.handle = self.handle, None
            _check("lynx_stream_destroy", lib().lynx_stream_destroy(h))

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def split_stream_transfer(kv: torch.Tensor | None, shape: lynx_kv_shape, object_blocks: int,
                          tx: Codes, wire: Codes, rx: Codes,
                          kv_anchor: torch.Tensor | None = None,
                          kv_full: torch.Tensor | None = None, copies_only: bool = False,
                          p: lynx_params | None = None, streams=None) -> dict:
    """lynx_split_stream_transfer (blocking); returns the milestones in ms.
    streams: (sender, link_out, link_in, receiver), default four new streams
    of default priority."""
    nb = num_blocks(shape)
    for name, c in (("tx", tx), ("rx", rx)):
        _check_codes(f"split_stream_transfer ({name})", c, nb, p)
    _check_codes("split_stream_transfer (wire)", wire, nb, p, device=False)
    if not copies_only:
        for name, t in (("kv", kv), ("kv_anchor", kv_anchor), ("kv_full", kv_full)):
            if t is None:
                raise ValueError(f"split_stream_transfer: {name} is required")
            _check_kv("split_stream_transfer", name, t, shape)
    if streams is None:
        streams = tuple(torch.cuda.Stream() for _ in range(4))
    t = lynx_transfer_times()
    ptr = lambda x: None if x is None else x.data_ptr()
    _check("lynx_split_stream_transfer", lib().lynx_split_stream_transfer(
        ptr(kv), ctypes.byref(shape), ctypes.byref(p) if p else None, object_blocks,
        tx.c_struct(), wire.c_struct(), rx.c_struct(), ptr(kv_anchor), ptr(kv_full),
        TRANSFER_COPIES_ONLY if copies_only else 0,
        *(ctypes.c_void_p(s.cuda_stream) for s in streams), ctypes.byref(t)))
    return {n: float(getattr(t, n)) for n, _ in lynx_transfer_times._fields_}


def spec_verify_workspace_bytes(t_draft: int, vocab: int) -> int:
    return int(lib().lynx_spec_verify_workspace_bytes(t_draft, vocab))


def spec_verify(draft_logits: torch.Tensor, target_logits: torch.Tensor, tokens: torch.Tensor,
                u_accept: torch.Tensor, u_sample: float, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """lynx_spec_verify: float32 logits [T, V] / [T + 1, V], int32 tokens [T],
    float64 uniforms [T] on the device; returns int32 [2] (accepted drafts,
    next token) on the device."""
    _require_cuda(draft_logits, target_logits, tokens, u_accept)
    if target_logits.dim() != 2:
        raise ValueError("spec_verify: target_logits must be [T + 1, V]")
    t_draft, vocab = target_logits.shape[0] - 1, target_logits.shape[1]
    for x, dt in ((draft_logits, torch.float32), (target_logits, torch.float32),
                  (tokens, torch.int32), (u_accept, torch.float64)):
        if x.dtype != dt or not x.is_contiguous():
            raise ValueError("spec_verify: contiguous float32 logits, int32 tokens and "
                             "float64 uniforms expected")
    if draft_logits.numel() != t_draft * vocab or tokens.numel() != t_draft \
            or u_accept.numel() != t_draft:
        raise ValueError(f"spec_verify: draft_logits [{t_draft}, {vocab}], tokens and "
                         f"u_accept [{t_draft}] expected")
    if out is None:
        out = torch.empty(2, dtype=torch.int32, device=target_logits.device)
    _require_cuda(out)
    if out.dtype != torch.int32 or out.numel() < 2 or not out.is_contiguous():
        raise ValueError("spec_verify: out must be a contiguous int32 tensor of 2 elements")
    if workspace is None:
        workspace = torch.empty(max(spec_verify_workspace_bytes(t_draft, vocab), 16),
                                dtype=torch.uint8, device=target_logits.device)
    _require_cuda(workspace)
    if not workspace.is_contiguous():
        raise ValueError("spec_verify: workspace must be a contiguous device tensor")
    _check("lynx_spec_verify", lib().lynx_spec_verify(
        draft_logits.data_ptr(), target_logits.data_ptr(), tokens.data_ptr(),
        u_accept.data_ptr(), float(u_sample), t_draft, vocab, out.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out

"""CPU tests of the C ABI (no GPU): the library loads and exports every
symbol include/lynx.h declares, the host helpers, the compander threshold
table against the oracle's decision, and argument errors that are rejected
before any launch."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from progressive_kv_transfer_amd import lynx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lynx.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lynx_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_symbols()
    assert names == sorted(lynx.EXPORTS)
    L = lynx.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", lynx.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (lynx_[a-z0-9_]+)", out))
    assert set(names) <= exported


def test_kv_bytes_eq1_worked_example():
    """Eq. (1) with the paper's Qwen3-235B-A22B example (footnote 4):
    2 x 94 x 131072 x (4 x 128) x 2 bytes = 23.5 GiB."""
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden",
                                    "kv_size_qwen3_235b_128k.json")))
    n = lynx.kv_bytes(g["k_factor"], g["tokens"], g["kv_heads"] * g["head_dim"],
                      g["layers"], g["precision_bytes"])
    assert n == g["bytes"]
    assert n / 2**30 == g["printed_gb"]
    # Qwen-32B-shaped KV at 16K: 64 layers x 8 heads x 128 -> 4 GiB
    assert lynx.kv_bytes(2, 16384, 1024, 64, 2) == 2**32
    assert lynx.kv_bytes(1, 10, 10, 10, 2) == 2000  # MLA: K_factor 1
    assert lynx.kv_bytes(-1, 1, 1, 1, 1) == 0
    assert lynx.kv_bytes(2**40, 2**40, 1, 1, 1) == 0  # overflow


def test_size_helpers_and_metadata_overhead():
    """Stream and metadata sizes; the reading notes' metadata count of
    2304 scalars (9 KB fp32) per 128 x 256 page."""
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "metadata_overhead.json")))
    s = lynx.lynx_kv_shape(num_tensors=128, tensor_stride=16384 * 1024,
                           num_tokens=16384, num_channels=1024, row_stride=1024)
    L = lynx.lib()
    nb = lynx.num_blocks(s)
    assert nb == 128 * 64 * 8
    assert L.lynx_stream_bytes(ctypes.byref(s)) == nb * 16384
    per_block = (L.lynx_gamma_floats(ctypes.byref(s)) * 2 +
                 L.lynx_chunk_floats(ctypes.byref(s)) * 2) // nb
    assert per_block == g["scalars"]
    assert per_block * 4 == g["bytes_fp32"]


@pytest.mark.parametrize("alpha,code_scale", [(255.0, 127.0), (100.0, 127.0),
                                              (255.0, 120.0)])
def test_compander_thresholds_match_oracle_decision(alpha, code_scale):
    """Every threshold of the kernels' table is exactly the point where the
    oracle's Eq. (3) code steps: code(thr[k]) >= k > code(pred(thr[k]))."""
    thr = lynx.compander_thresholds(lynx.params(alpha=alpha, code_scale=code_scale))
    assert thr[0] == 0.0
    for k in range(1, 128):
        t = float(thr[k])
        if k > 120:
            assert np.isinf(t)
            continue
        if np.isinf(t):
            assert oracle.code(1.0, alpha, code_scale) < k
            continue
        prev = float(np.nextafter(np.float32(t), np.float32(0)))
        assert oracle.code(t, alpha, code_scale) >= k
        assert oracle.code(prev, alpha, code_scale) < k


def _shape(nt=1, T=256, Ch=128, rs=None, ts=None):
    rs = Ch if rs is None else rs
    ts = T * rs if ts is None else ts
    return lynx.lynx_kv_shape(num_tensors=nt, tensor_stride=ts, num_tokens=T,
                              num_channels=Ch, row_stride=rs)


FAKE = 1 << 20  # a 16-byte aligned non-null address; never dereferenced


def _meta(ptr=FAKE):
    m = lynx.lynx_meta()
    m.gamma_min = m.gamma_scale = m.mu = m.sigma = ptr
    return m


@pytest.mark.parametrize("case,expect", [
    ("tokens", -2), ("channels", -2), ("row_stride", -2), ("row_stride_small", -2),
    ("row_stride_huge", -2),
    ("tensor_stride", -2), ("negative", -1), ("alpha", -1), ("alpha_nan", -1),
    ("eps", -1), ("page", -1), ("chunk", -1), ("null_kv", -1), ("null_anchor", -1),
    ("misaligned", -2), ("code_scale", -1)])
def test_quantize_argument_errors(case, expect):
    """Every malformed call returns its status before launching anything."""
    L = lynx.lib()
    s = _shape()
    p = lynx.params()
    kv, anc, res, meta = FAKE, FAKE, FAKE, _meta()
    if case == "tokens":
        s = _shape(T=300)
    elif case == "channels":
        s = _shape(Ch=192)
    elif case == "row_stride":
        s = _shape(rs=132)
    elif case == "row_stride_small":
        s = _shape(rs=64)
    elif case == "row_stride_huge":
        # the first multiple of 8 above the 32-bit row addressing limit
        s = _shape(rs=4210752)
    elif case == "tensor_stride":
        s = _shape(nt=2, ts=1000)
    elif case == "negative":
        s = _shape(nt=-1)
    elif case == "alpha":
        p.alpha = 0.0
    elif case == "alpha_nan":
        p.alpha = float("nan")
    elif case == "eps":
        p.eps = 0.5
    elif case == "page":
        p.page_tokens = 128
    elif case == "chunk":
        p.chunk_tokens = 16
    elif case == "code_scale":
        p.code_scale = 200.0
    elif case == "null_kv":
        kv = None
    elif case == "null_anchor":
        anc = None
    elif case == "misaligned":
        kv = FAKE + 2
    rc = L.lynx_quantize_pages(kv, ctypes.byref(s), ctypes.byref(p), anc, res, meta, None)
    assert rc == expect
    assert L.lynx_status_string(rc).decode()


def test_dequant_and_stats_argument_errors():
    L = lynx.lib()
    s = _shape()
    p = lynx.params()
    assert L.lynx_dequant_full(FAKE, None, _meta(), ctypes.byref(s), None, FAKE, None) == -1
    assert L.lynx_dequant_anchor(None, _meta(), ctypes.byref(s), None, FAKE, None) == -1
    assert L.lynx_dequant_anchor(FAKE, _meta(None), ctypes.byref(s), None, FAKE, None) == -1
    assert L.lynx_dequant_anchor(FAKE, _meta(), ctypes.byref(_shape(T=100)), None, FAKE,
                                 None) == -2
    assert L.lynx_dequant_full(FAKE, FAKE + 8, _meta(), ctypes.byref(s), None, FAKE,
                               None) == -2
    assert L.lynx_page_stats(FAKE, ctypes.byref(s), ctypes.byref(p), None, FAKE, None) == -1
    assert L.lynx_block_stats(FAKE, ctypes.byref(s), None, FAKE, FAKE, None, FAKE,
                              None) == -1
    huge = _shape(rs=4210752)
    assert L.lynx_dequant_anchor(FAKE, _meta(), ctypes.byref(huge), None, FAKE, None) == -2
    assert L.lynx_page_stats(FAKE, ctypes.byref(huge), None, FAKE, FAKE, None) == -2
    assert L.lynx_num_blocks(ctypes.byref(huge)) == -2
    bad = lynx.params(eps=0.0)
    assert L.lynx_page_stats(FAKE, ctypes.byref(s), ctypes.byref(bad), FAKE, FAKE,
                             None) == -1


def test_empty_shapes_are_no_ops():
    """Zero tensors / tokens / channels: nothing to do, OK without touching
    any pointer."""
    L = lynx.lib()
    for s in (_shape(nt=0), _shape(T=0), _shape(Ch=0, rs=0)):
        assert L.lynx_quantize_pages(None, ctypes.byref(s), None, None, None, _meta(None),
                                     None) == 0
        assert L.lynx_dequant_anchor(None, _meta(None), ctypes.byref(s), None, None,
                                     None) == 0


def test_attention_workspace_sizes():
    """Split-KV workspace: partials of splits x KV heads x query rows x
    (2 + 128) floats.  Up to 16 rows per KV head (the decode kernel) the
    splits are runs of 32-token chunks, a multiple of 8, about 512
    workgroups in all; beyond 16 rows (the tile kernel) runs of 128-token
    steps."""
    ws = lynx.attn_workspace_bytes
    per = lambda nkvh, rows: nkvh * rows * 130 * 4
    # decode, 64 q-heads over 8 KV heads at 32K: 8 rows, 1024 chunks, 16 per split
    assert ws(1, 64, 8, 32768) == 64 * per(8, 8)
    # verify, 8 drafts x 32 q-heads over 4 KV heads at 128K: 64 rows, 8 steps per split
    assert ws(8, 32, 4, 131072) == 128 * per(4, 64)
    # small contexts: 32 chunks in splits of 8 chunks
    assert ws(3, 8, 4, 1024) == 4 * per(4, 6)
    assert ws(5, 8, 4, 1024) == 4 * per(4, 10)
    # 17 rows and more: the tile kernel's steps, one per split
    assert ws(3, 24, 4, 1024) == 8 * per(4, 18)
    # more than 64 rows per KV head: passes of floor(64 / g) query tokens,
    # the workspace of the first (largest) pass serves them all
    assert ws(9, 64, 8, 32768) == ws(8, 64, 8, 32768) == 64 * per(8, 64)  # 72 rows: 64 + 8
    assert ws(64, 64, 8, 131072) == ws(8, 64, 8, 131072)                  # 8 passes of 64
    assert ws(5, 32, 2, 1024) == ws(4, 32, 2, 1024)                       # g = 16: 64 + 16
    assert ws(1, 64, 1, 1024) == 8 * per(1, 64)                           # g = 64: one row a token
    # invalid plans report 0
    assert ws(1, 130, 2, 1024) == 0      # 65 query heads per KV head
    assert ws(1, 6, 4, 1024) == 0        # not grouped-query
    assert ws(1, 8, 8, 1000) == 0        # context not whole pages
    assert ws(0, 8, 8, 1024) == 0


@pytest.mark.parametrize("case,expect", [
    ("ok_shape_null_q", -1), ("group", -1), ("rows", -1), ("ctx", -2), ("head_dim", -1),
    ("scale", -1), ("workspace", -1), ("null_v_meta", -1), ("misaligned_k", -2),
    ("empty_ctx", -1), ("params", -1), ("out_dtype", -1)])
def test_attention_argument_errors(case, expect):
    """Malformed attention calls return their status before any launch."""
    L = lynx.lib()
    t_q, nqh, nkvh, ctx, hd, scale, causal = 1, 8, 2, 1024, 128, 0.088, 0
    q, kanc, kres, vanc, vres, kmeta, vmeta = FAKE, FAKE, FAKE, FAKE, FAKE, _meta(), _meta()
    wsb = 1 << 30
    p = lynx.params()
    odt = lynx.OUT_F32
    if case == "ok_shape_null_q":
        q = None
    elif case == "group":
        nqh = 7
    elif case == "rows":  # a group of more than 64 query heads per KV head
        nqh, nkvh = 130, 2
    elif case == "ctx":
        ctx = 1000
    elif case == "head_dim":
        hd = 64
    elif case == "scale":
        scale = float("nan")
    elif case == "workspace":
        wsb = 64
    elif case == "null_v_meta":
        vmeta = _meta(None)
    elif case == "misaligned_k":
        kanc = FAKE + 4
    elif case == "empty_ctx":
        ctx, causal = 0, 1
    elif case == "params":
        p.alpha = -1.0
    elif case == "out_dtype":
        odt = 2
    rc = L.lynx_decode_attn_dequant(q, t_q, nqh, kanc, kres, kmeta, vanc, vres, vmeta, ctx,
                                    nkvh, hd, scale, causal, ctypes.byref(p), FAKE, odt, FAKE,
                                    wsb, None)
    assert rc == expect


def _codes(ptr=FAKE):
    c = lynx.lynx_codes()
    c.anchor = c.residual = ptr
    c.meta = _meta(ptr)
    return c


def test_packed_layout_sizes_and_errors():
    """LYNX_LAYOUT_PACKED: records of 4096 a + 2304 meta_bits / 8 bytes per
    block (25600 for the paper's 4 + 4 split: 16 KiB anchor + 9 KiB
    scalars); metadata pointers must be NULL; the statistics calls refuse it;
    an unknown layout is refused."""
    L = lynx.lib()
    assert lynx.anchor_block_bytes() == 16384
    for a, mb, want in ((4, 32, 25600), (4, 16, 20992), (3, 32, 21504), (6, 32, 33792),
                        (5, 32, 29696)):
        assert lynx.anchor_block_bytes(lynx.params(anchor_bits=a, meta_bits=mb,
                                                   layout=lynx.LAYOUT_PACKED)) == want
        assert want % 16 == 0
    p = lynx.params(layout=lynx.LAYOUT_PACKED)
    s = _shape()
    # metadata pointers given with the packed layout
    assert L.lynx_quantize_pages(FAKE, ctypes.byref(s), ctypes.byref(p), FAKE, FAKE, _meta(),
                                 None) == -1
    assert L.lynx_dequant_anchor(FAKE, _meta(), ctypes.byref(s), ctypes.byref(p), FAKE,
                                 None) == -1
    assert L.lynx_page_stats(FAKE, ctypes.byref(s), ctypes.byref(p), FAKE, FAKE, None) == -1
    assert L.lynx_block_stats(FAKE, ctypes.byref(s), ctypes.byref(p), FAKE, FAKE, FAKE, FAKE,
                              None) == -1
    bad = lynx.params()
    bad.layout = 2
    assert L.lynx_quantize_pages(FAKE, ctypes.byref(s), ctypes.byref(bad), FAKE, FAKE,
                                 _meta(), None) == -1
    assert L.lynx_anchor_block_bytes(ctypes.byref(bad)) == 0


def test_noalloc_attention_refuses_beyond_its_scratch():
    """lynx_decode_attn_dequant_noalloc: partials of more than
    LYNX_ATTN_SCRATCH_BYTES are refused with LYNX_ESCRATCH before any
    launch; other argument errors as the workspace entry point."""
    L = lynx.lib()
    # 8 drafts x 8 query heads per KV head = 64 rows, 1024 KV heads: one split
    # of 64 partials of (2 + 128) floats per KV head
    need = lynx.attn_workspace_bytes(8, 8192, 1024, 256)
    assert need == 1024 * 64 * 130 * 4 > lynx.ATTN_SCRATCH_BYTES
    args = lambda t_q, nqh, nkvh, ctx: (FAKE, t_q, nqh, FAKE, FAKE, _meta(), FAKE, FAKE,
                                        _meta(), ctx, nkvh, 128, 0.088, 0, None, FAKE, 0, None)
    rc = L.lynx_decode_attn_dequant_noalloc(*args(8, 8192, 1024, 256))
    assert rc == -4 and "scratch" in L.lynx_status_string(rc).decode()
    assert L.lynx_decode_attn_dequant_noalloc(*args(1, 64, 8, 300)) == -2
    assert L.lynx_decode_attn_dequant_noalloc(*args(1, 130, 2, 256)) == -1  # g = 65
    a = list(args(1, 64, 8, 256))
    a[15] = None  # out
    assert L.lynx_decode_attn_dequant_noalloc(*a) == -1
    # every size the decode and verify workloads use fits
    assert lynx.attn_workspace_bytes(1, 64, 8, 32768) <= lynx.ATTN_SCRATCH_BYTES
    assert lynx.attn_workspace_bytes(8, 32, 4, 131072) <= lynx.ATTN_SCRATCH_BYTES


@pytest.mark.parametrize("case,expect", [
    ("object_blocks", -1), ("huge_objects", -1), ("flags", -1), ("null_wire", -1), ("misaligned_rx", -1),
    ("misaligned_kv", -2), ("null_out", -1), ("too_many_objects", -1), ("tokens", -2),
    ("params", -1)])
def test_transfer_argument_errors(case, expect):
    """Malformed transfers are rejected before any stream or event is used."""
    L = lynx.lib()
    s, p = _shape(), lynx.params()
    ob, flags = 1, 0
    kv, ka, kf = FAKE, FAKE, FAKE
    tx, wire, rx = _codes(), _codes(), _codes()
    if case == "object_blocks":
        ob = 0
    elif case == "huge_objects":
        ob = (1 << 22) + 1  # one launch per object: over the grid limit
    elif case == "flags":
        flags = 2
    elif case == "null_wire":
        wire = _codes(None)
    elif case == "misaligned_rx":
        rx.meta.mu = FAKE + 4
    elif case == "misaligned_kv":
        kv = FAKE + 2
    elif case == "null_out":
        kf = None
    elif case == "too_many_objects":
        s = _shape(nt=4097, T=256, ts=256 * 128)  # 4097 blocks, one object each
    elif case == "tokens":
        s = _shape(T=300)
    elif case == "params":
        p.eps = 1.0
    t = lynx.lynx_transfer_times()
    rc = L.lynx_split_stream_transfer(kv, ctypes.byref(s), ctypes.byref(p), ob, tx, wire, rx,
                                      ka, kf, flags, None, None, None, None, ctypes.byref(t))
    assert rc == expect


def test_transfer_empty_set_and_copies_only_needs_no_kv():
    L = lynx.lib()
    t = lynx.lynx_transfer_times()
    t.full_ready = 5.0
    for s in (_shape(nt=0), _shape(T=0)):
        assert L.lynx_split_stream_transfer(None, ctypes.byref(s), None, 4, _codes(), _codes(),
                                            _codes(), None, None, 1, None, None, None, None,
                                            ctypes.byref(t)) == 0
        assert t.full_ready == 0.0


def test_spec_verify_workspace_and_errors():
    L = lynx.lib()
    ws = lynx.spec_verify_workspace_bytes
    # 2T+1 rows x 75 chunks of 2048 tokens (max, sum), the chunk weight sums,
    # 8 slots for the decision
    assert ws(8, 151936) == (17 * 75 * 2 + 75 + 8) * 8
    assert ws(0, 1) == (2 + 1 + 8) * 8
    assert ws(65, 100) == 0 and ws(-1, 100) == 0 and ws(3, 0) == 0
    ok = dict(d=FAKE, t=FAKE, s=FAKE, u=FAKE, us=0.5, T=8, V=1000, out=FAKE, w=FAKE, wb=1 << 20)
    cases = [dict(T=65), dict(V=0), dict(us=1.0), dict(us=float("nan")), dict(t=None),
             dict(d=None), dict(out=None), dict(w=None), dict(wb=16), dict(u=FAKE + 4)]
    expect = [-1, -1, -1, -1, -1, -1, -1, -1, -1, -2]
    for c, e in zip(cases, expect):
        a = {**ok, **c}
        rc = L.lynx_spec_verify(a["d"], a["t"], a["s"], a["u"], a["us"], a["T"], a["V"],
                                a["out"], a["w"], a["wb"], None)
        assert rc == e, (c, rc)


def test_split_parameters_and_stream_sizes():
    """anchor_bits: default 4, 3..6 accepted by the codec calls, rejected by
    attention and the transfer; the compander clips at 128 - 2^(7 - a);
    field streams take 4096 x bits bytes per block."""
    L = lynx.lib()
    p = lynx.params()
    assert p.anchor_bits == 4
    sh = lynx.lynx_kv_shape(1, 256 * 128, 256, 128, 128)
    assert L.lynx_stream_bytes(ctypes.byref(sh)) == 16384
    for bits_ in range(1, 9):
        assert L.lynx_field_stream_bytes(ctypes.byref(sh), bits_) == 4096 * bits_
    assert L.lynx_field_stream_bytes(ctypes.byref(sh), 0) == 0
    assert L.lynx_field_stream_bytes(ctypes.byref(sh), 9) == 0
    thr = np.zeros(128, np.float32)
    for a, top in ((3, 112), (4, 120), (5, 124), (6, 126)):
        q = lynx.params(code_scale=127.0, anchor_bits=a)
        assert L.lynx_compander_thresholds(ctypes.byref(q), thr.ctypes.data) == 0
        assert np.isfinite(thr[top]) and np.all(np.isinf(thr[top + 1:])), a
        assert lynx.code_max(a) == top
    for a in (2, 7, 0):
        q = lynx.params(anchor_bits=a)
        assert L.lynx_compander_thresholds(ctypes.byref(q), thr.ctypes.data) == -1
        assert L.lynx_quantize_pages(FAKE, ctypes.byref(sh), ctypes.byref(q), FAKE, FAKE,
                                     lynx.lynx_meta(FAKE, FAKE, FAKE, FAKE), None) == -1
    q5 = lynx.params(anchor_bits=5)
    m = lynx.lynx_meta(FAKE, FAKE, FAKE, FAKE)
    assert L.lynx_decode_attn_dequant(FAKE, 1, 8, FAKE, FAKE, m, FAKE, FAKE, m, 256, 1, 128,
                                      0.1, 0, ctypes.byref(q5), FAKE, 0, FAKE, 1 << 20,
                                      None) == -1
    c = lynx.lynx_codes(FAKE, FAKE, m)
    t = lynx.lynx_transfer_times()
    assert L.lynx_split_stream_transfer(FAKE, ctypes.byref(sh), ctypes.byref(q5), 1, c, c, c,
                                        FAKE, FAKE, 0, None, None, None, None,
                                        ctypes.byref(t)) == -1


def test_single_stream_parameters():
    """residual_bits = 0 with anchor_bits 4 or 8 (Lynx-INT4 / Lynx-INT8) is
    accepted by the codec calls with no residual buffer; the compander tops
    out at 2^(a-1) - 1; a residual buffer, the residual phase, attention and
    the transfer are refused, and so are widths that are neither a split of
    the 8-bit code nor a built single stream."""
    L = lynx.lib()
    sh = lynx.lynx_kv_shape(1, 256 * 128, 256, 128, 128)
    m = lynx.lynx_meta(FAKE, FAKE, FAKE, FAKE)
    thr = np.zeros(128, np.float32)
    for a, cs in ((4, 7.0), (8, 127.0)):
        q = lynx.params(code_scale=cs, anchor_bits=a, residual_bits=0)
        assert q.residual_bits == 0
        assert L.lynx_compander_thresholds(ctypes.byref(q), thr.ctypes.data) == 0
        top = (1 << (a - 1)) - 1
        assert lynx.code_max(a, 0) == top
        assert np.isfinite(thr[top]) and np.all(np.isinf(thr[top + 1:])), a
        # a residual buffer for a single stream is an argument error
        assert L.lynx_quantize_pages(FAKE, ctypes.byref(sh), ctypes.byref(q), FAKE, FAKE, m,
                                     None) == -1
        assert L.lynx_dequant_full(FAKE, FAKE, m, ctypes.byref(sh), ctypes.byref(q), FAKE,
                                   None) == -1
        assert L.lynx_decode_attn_dequant(FAKE, 1, 8, FAKE, None, m, FAKE, None, m, 256, 1,
                                          128, 0.1, 0, ctypes.byref(q), FAKE, 0, FAKE,
                                          1 << 20, None) == -1
    # the paper's split needs its residual buffer
    q44 = lynx.params()
    assert L.lynx_quantize_pages(FAKE, ctypes.byref(sh), ctypes.byref(q44), FAKE, None, m,
                                 None) == -1
    for a, b in ((4, 5), (8, 4), (5, 0), (3, 0), (6, 0), (2, 6), (7, 1), (4, 3)):
        q = lynx.params(anchor_bits=a, residual_bits=b)
        assert L.lynx_compander_thresholds(ctypes.byref(q), thr.ctypes.data) == -1, (a, b)
        assert L.lynx_quantize_pages(FAKE, ctypes.byref(sh), ctypes.byref(q), FAKE, FAKE, m,
                                     None) == -1, (a, b)


def test_bf16_metadata_parameters():
    """meta_bits: 32 by default, 16 accepted by the codec calls for the 4 + 4
    split only, refused by the statistics calls, attention and the
    transfer, and any other width refused."""
    L = lynx.lib()
    sh = lynx.lynx_kv_shape(1, 256 * 128, 256, 128, 128)
    m = lynx.lynx_meta(FAKE, FAKE, FAKE, FAKE)
    thr = np.zeros(128, np.float32)
    assert lynx.params().meta_bits == 32
    q16 = lynx.params(meta_bits=16)
    assert L.lynx_compander_thresholds(ctypes.byref(q16), thr.ctypes.data) == 0
    for bad in (lynx.params(meta_bits=8), lynx.params(meta_bits=64),
                lynx.params(meta_bits=16, anchor_bits=5),
                lynx.params(meta_bits=16, code_scale=127.0, anchor_bits=8, residual_bits=0)):
        assert L.lynx_compander_thresholds(ctypes.byref(bad), thr.ctypes.data) == -1
        assert L.lynx_quantize_pages(FAKE, ctypes.byref(sh), ctypes.byref(bad), FAKE, FAKE, m,
                                     None) == -1
    assert L.lynx_page_stats(FAKE, ctypes.byref(sh), ctypes.byref(q16), FAKE, FAKE,
                             None) == -1
    assert L.lynx_block_stats(FAKE, ctypes.byref(sh), ctypes.byref(q16), FAKE, FAKE, FAKE,
                              FAKE, None) == -1
    assert L.lynx_decode_attn_dequant(FAKE, 1, 8, FAKE, FAKE, m, FAKE, FAKE, m, 256, 1, 128,
                                      0.1, 0, ctypes.byref(q16), FAKE, 0, FAKE, 1 << 20,
                                      None) == -1
    c = lynx.lynx_codes(FAKE, FAKE, m)
    t = lynx.lynx_transfer_times()
    assert L.lynx_split_stream_transfer(FAKE, ctypes.byref(sh), ctypes.byref(q16), 1, c, c, c,
                                        FAKE, FAKE, 0, None, None, None, None,
                                        ctypes.byref(t)) == -1


def test_table_cache_is_bounded_and_stable():
    """More parameter sets than the table cache holds: the tables are
    rebuilt after eviction and come out identical (host only)."""
    first = lynx.compander_thresholds(lynx.params(alpha=255.0))
    seen = {}
    for i in range(150):
        a = 10.0 + 7.25 * i
        seen[a] = lynx.compander_thresholds(lynx.params(alpha=a))
    again = lynx.compander_thresholds(lynx.params(alpha=255.0))
    assert np.array_equal(first.view(np.uint32), again.view(np.uint32))
    for a in (10.0, 10.0 + 7.25 * 149):
        assert np.array_equal(seen[a].view(np.uint32),
                              lynx.compander_thresholds(lynx.params(alpha=a)).view(np.uint32))


def test_codec_stream_argument_errors():
    """lynx_codec_stream_create / lynx_stream_destroy refuse a NULL output,
    a negative reserve and a NULL stream before any HIP call."""
    L = lynx.lib()
    h = ctypes.c_void_p()
    assert L.lynx_codec_stream_create(16, None) == -1
    assert L.lynx_codec_stream_create(-1, ctypes.byref(h)) == -1
    assert h.value is None
    assert L.lynx_stream_destroy(None) == -1

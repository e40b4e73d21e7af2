"""Compression error of attention outputs (vNMSE), the paper's Table 3
measure E(||o - o_hat||^2 / ||o_hat||^2), on synthetic KV.

o_hat: binary64 attention (oracle) over the uncompressed bf16 K, V.
o:     Lynx (anchor + residual codes) and its draft (anchor codes alone)
       from the fused GPU kernel (binary32 output); the paper's Lynx-INT8 and
       Lynx-INT4 configurations (Algorithm 1 into one 8-bit or 4-bit stream,
       code scale 127 / 7) rebuilt by the GPU dequant, attention by the
       oracle; uniform INT8 / INT4 baselines: per token and head (128
       channels) asymmetric min-max quantization with round to nearest,
       rebuilt to bf16, attention by the oracle.

The paper's numbers (LLaMA 8B on MMLU) cannot be reproduced without the
model; what is checked is the ordering it reports (Lynx < INT8 < Lynx-INT4 <
INT4, with both the 4-bit stream and the split's anchor as the 4-bit Lynx)
on the outlier-bearing decode workload, and Lynx < INT8 without outliers
(there the 4-bit anchor alone is about as coarse as uniform INT4, 0.42
against 0.40 in an oracle run).  The values are printed for the record.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from progressive_kv_transfer_amd import kvgen, lynx

pytestmark = pytest.mark.gpu
DEV = "cuda"


def uniform_baseline(x_bits: np.ndarray, bits: int) -> np.ndarray:
    """Per token and 128-channel head: x_hat = round((x - min) / s) s + min,
    s = (max - min) / (2^bits - 1); returned as bf16 bits."""
    x = (x_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    t, ch = x.shape
    g = x.reshape(t, ch // 128, 128)
    lo, hi = g.min(axis=2, keepdims=True), g.max(axis=2, keepdims=True)
    s = (hi - lo) / (2 ** bits - 1)
    s = np.where(s > 0, s, 1.0)
    xh = (np.round((g - lo) / s) * s + lo).reshape(t, ch)
    return kvgen.bf16_bits(torch.from_numpy(xh.astype(np.float32)).to(torch.bfloat16))


def vnmse(o: np.ndarray, ref: np.ndarray) -> float:
    o = o.reshape(-1, o.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    return float(np.mean(np.sum((o - ref) ** 2, axis=1) / np.sum(ref ** 2, axis=1)))


def measure(name: str, n_q: int = 4):
    cfg = kvgen.CONFIGS[name]
    kv = cfg.make(DEV)  # [2, ctx, n_kvh * 128]: K, V
    ctx, ch = kv.shape[1], kv.shape[2]
    n_kvh, n_qh = ch // 128, 64
    scale = 1.0 / math.sqrt(128.0)
    codes = lynx.quantize_pages(kv)
    nb = codes.anchor.shape[0]
    xb = kvgen.bf16_bits(kv)
    res = {"lynx": [], "lynx_anchor": [], "lynx_int8": [], "lynx_int4": [], "int8": [],
           "int4": []}
    single = {}
    for key, a, cs in (("lynx_int8", 8, 127.0), ("lynx_int4", 4, 7.0)):
        p = lynx.params(code_scale=cs, anchor_bits=a, residual_bits=0)
        out = torch.empty_like(kv)
        lynx.dequant_anchor(lynx.quantize_pages(kv, p), out, p)
        torch.cuda.synchronize()
        ob = kvgen.bf16_bits(out)
        single[key] = (ob[0].reshape(ctx, n_kvh, 128), ob[1].reshape(ctx, n_kvh, 128))
        del out
    base = {b: [uniform_baseline(xb[i], b).reshape(ctx, n_kvh, 128) for i in range(2)]
            for b in (8, 4)}
    k_exact, v_exact = xb[0].reshape(ctx, n_kvh, 128), xb[1].reshape(ctx, n_kvh, 128)
    for s in range(n_q):
        q = kvgen.queries(5000 + s, 1, n_qh, device=DEV)
        qb = kvgen.bf16_bits(q)
        ref = oracle.attention(qb, k_exact, v_exact, scale, False, threads=16)
        for key, full in (("lynx", True), ("lynx_anchor", False)):
            o = lynx.decode_attn_dequant(q, lynx.CodeView(codes, 0, nb // 2, full),
                                         lynx.CodeView(codes, nb // 2, nb, full), ctx, n_kvh,
                                         scale, out_dtype=torch.float32)
            res[key].append(vnmse(o.cpu().double().numpy(), ref))
        for b in (8, 4):
            o = oracle.attention(qb, base[b][0], base[b][1], scale, False, threads=16)
            res[f"int{b}"].append(vnmse(o, ref))
        for key, (kh, vh) in single.items():
            res[key].append(vnmse(oracle.attention(qb, kh, vh, scale, False, threads=16), ref))
    out = {k: float(np.mean(v)) for k, v in res.items()}
    print(f"[gpu-vnmse] {name}: " + ", ".join(f"{k} {v:.3g}" for k, v in out.items()),
          flush=True)
    return out


def test_vnmse_ordering_with_outliers():
    r = measure("decode_attn_32k")
    assert r["lynx"] < r["int8"] < r["lynx_anchor"] < r["int4"]
    assert r["int8"] < r["lynx_int4"] < r["int4"]
    assert r["lynx"] < 5e-3 and r["lynx_int8"] < 5e-3


def test_vnmse_without_outliers():
    r = measure("decode_attn_32k_plain")
    assert r["lynx"] < r["int8"]
    assert r["lynx"] < 5e-3 and r["lynx_int8"] < 5e-3
    assert r["lynx_anchor"] < 1.0 and r["lynx_int4"] < 1.0


def test_vnmse_of_the_splits():
    """The other splits of the 8-bit code (anchor bits a = 3, 5, 6 beside the
    paper's 4), each at its own code range: the attention error of the
    draft (anchor alone) shrinks as anchor bits are added; the full 8-bit
    code keeps its small error for every split.  K^, V^ from
    the GPU dequant, attention by the oracle in binary64; values printed for
    the record."""
    cfg = kvgen.CONFIGS["decode_attn_32k"]
    kv = cfg.make(DEV)
    ctx, ch = kv.shape[1], kv.shape[2]
    n_kvh, n_qh = ch // 128, 64
    scale = 1.0 / math.sqrt(128.0)
    xb = kvgen.bf16_bits(kv)
    k_exact, v_exact = xb[0].reshape(ctx, n_kvh, 128), xb[1].reshape(ctx, n_kvh, 128)
    qs = [kvgen.bf16_bits(kvgen.queries(5100 + s, 1, n_qh, device=DEV)) for s in range(2)]
    refs = [oracle.attention(q, k_exact, v_exact, scale, False, threads=16) for q in qs]
    res = {}
    for a in (3, 4, 5, 6):
        p = lynx.params(code_scale=float(lynx.code_max(a)), anchor_bits=a)
        codes = lynx.quantize_pages(kv, p)
        out = torch.empty_like(kv)
        for full in (False, True):
            (lynx.dequant_full if full else lynx.dequant_anchor)(codes, out, p)
            torch.cuda.synchronize()
            ob = kvgen.bf16_bits(out)
            kh, vh = ob[0].reshape(ctx, n_kvh, 128), ob[1].reshape(ctx, n_kvh, 128)
            res[(a, full)] = float(np.mean([
                vnmse(oracle.attention(q, kh, vh, scale, False, threads=16), r)
                for q, r in zip(qs, refs)]))
    print("[gpu-vnmse] splits (anchor-only, full): " + ", ".join(
        f"{a}+{8 - a} {res[(a, False)]:.3g} {res[(a, True)]:.3g}" for a in (3, 4, 5, 6)),
        flush=True)
    drafts = [res[(a, False)] for a in (3, 4, 5, 6)]
    assert drafts[0] > drafts[1] > drafts[2] > drafts[3]
    for a in (3, 4, 5, 6):
        assert res[(a, True)] < 5e-3


def test_vnmse_bf16_metadata():
    """The paper's split with bfloat16 metadata against binary32 metadata,
    on the decode workload without outlier channels (4 queries): with
    outliers the softmax of many heads is nearly one-hot and a head's error
    jumps whenever its top token changes, so per-query values there swing
    by more than 10x between formats of equal reconstruction error (oracle
    runs); here they agree within a small factor.  K^, V^ from the GPU
    dequant, attention by the oracle in binary64."""
    cfg = kvgen.CONFIGS["decode_attn_32k_plain"]
    kv = cfg.make(DEV)
    ctx, ch = kv.shape[1], kv.shape[2]
    n_kvh, n_qh = ch // 128, 64
    scale = 1.0 / math.sqrt(128.0)
    xb = kvgen.bf16_bits(kv)
    k_exact, v_exact = xb[0].reshape(ctx, n_kvh, 128), xb[1].reshape(ctx, n_kvh, 128)
    qs = [kvgen.bf16_bits(kvgen.queries(5200 + s, 1, n_qh, device=DEV)) for s in range(4)]
    refs = [oracle.attention(q, k_exact, v_exact, scale, False, threads=16) for q in qs]
    res = {}
    for mb in (32, 16):
        p = lynx.params(meta_bits=mb)
        codes = lynx.quantize_pages(kv, p)
        out = torch.empty_like(kv)
        for full in (False, True):
            (lynx.dequant_full if full else lynx.dequant_anchor)(codes, out, p)
            torch.cuda.synchronize()
            ob = kvgen.bf16_bits(out)
            kh, vh = ob[0].reshape(ctx, n_kvh, 128), ob[1].reshape(ctx, n_kvh, 128)
            res[(mb, full)] = float(np.mean([
                vnmse(oracle.attention(q, kh, vh, scale, False, threads=16), r)
                for q, r in zip(qs, refs)]))
    print("[gpu-vnmse] metadata (anchor-only, full): " + ", ".join(
        f"{mb}-bit {res[(mb, False)]:.3g} {res[(mb, True)]:.3g}" for mb in (32, 16)), flush=True)
    assert res[(16, True)] < 5e-3
    assert res[(16, True)] < 3.0 * res[(32, True)]
    assert res[(16, False)] < 1.5 * res[(32, False)]

"""GPU parity of the other splits of the 8-bit code (anchor_bits a = 3, 5,
6 beside the paper's 4): quantize (anchor and residual bit streams,
metadata) and both reconstructions against the oracle, bit for bit, on the
single-page workload, the adversarial pages, a strided multi-block set and
sampled blocks of the Qwen-32B-shaped set; at each split's own code range
(nothing clipped) and at the default 120 (clipped at 112 for a = 3)."""
import numpy as np
import pytest
import torch

import oracle
from progressive_kv_transfer_amd import kvgen, lynx

pytestmark = pytest.mark.gpu
DEV = "cuda"


def bits(t):
    return kvgen.bf16_bits(t)


def host(t):
    return t.detach().cpu().numpy()


def announce(msg):
    print(f"[gpu-splits] {msg}", flush=True)


def check(kv, a, code_scale, alpha=255.0):
    p = lynx.params(alpha=alpha, code_scale=code_scale, anchor_bits=a)
    codes = lynx.quantize_pages(kv, p)
    out_a = torch.empty_like(kv)
    out_f = torch.empty_like(kv)
    lynx.dequant_anchor(codes, out_a, p)
    lynx.dequant_full(codes, out_f, p)
    torch.cuda.synchronize()
    xb = bits(kv.contiguous())
    ref = oracle.quantize(xb, alpha=alpha, code_scale=code_scale, threads=8, anchor_bits=a)
    nb = ref.nblocks
    np.testing.assert_array_equal(host(codes.anchor).reshape(nb, -1), ref.anchor.reshape(nb, -1))
    np.testing.assert_array_equal(host(codes.residual).reshape(nb, -1),
                                  ref.residual.reshape(nb, -1))
    for name in ("gamma_min", "gamma_scale", "mu", "sigma"):
        assert np.array_equal(host(getattr(codes, name)).view(np.uint32),
                              getattr(ref, name).view(np.uint32)), name
    np.testing.assert_array_equal(
        bits(out_a), oracle.dequant(ref, xb.shape, False, alpha=alpha, code_scale=code_scale,
                                    threads=8))
    np.testing.assert_array_equal(
        bits(out_f), oracle.dequant(ref, xb.shape, True, alpha=alpha, code_scale=code_scale,
                                    threads=8))
    return codes


@pytest.mark.parametrize("a", [3, 4, 5, 6])
def test_single_page_and_edge_pages(a):
    for cs in sorted({float(lynx.code_max(a)), 120.0}):
        announce(f"a={a} code_scale={cs} single page")
        check(kvgen.CONFIGS["single_page"].make(DEV), a, cs)
        pages = kvgen.edge_pages()
        announce(f"a={a} code_scale={cs} edge pages")
        check(torch.stack([pages[n] for n in sorted(pages)]).to(DEV), a, cs)


@pytest.mark.parametrize("a", [3, 5, 6])
def test_strided_set_and_stream_sizes(a):
    """3 tensors x 5 pages x 3 heads in padded rows: stream sizes follow
    lynx_field_stream_bytes and the padding of the outputs is untouched."""
    nt, T, Ch = 3, 256 * 5, 128 * 3
    big = torch.empty((nt, T + 64, Ch + 24), dtype=torch.bfloat16, device=DEV)
    for i in range(nt):
        big[i, :T, :Ch] = kvgen.kv_tensor(500 + i, T, Ch, [5, 140, 300], True, DEV)
    kv = big[:, :T, :Ch]
    announce(f"a={a} strided {nt}x{T}x{Ch}")
    sh = lynx.shape_of(kv)
    L = lynx.lib()
    assert L.lynx_field_stream_bytes(sh, a) == 45 * 4096 * a
    assert L.lynx_field_stream_bytes(sh, 8 - a) == 45 * 4096 * (8 - a)
    p = lynx.params(code_scale=float(lynx.code_max(a)), anchor_bits=a)
    codes = lynx.quantize_pages(kv, p)
    assert codes.anchor.numel() == 45 * 4096 * a
    outbig = torch.full_like(big, 7.0)
    lynx.dequant_full(codes, outbig[:, :T, :Ch], p)
    torch.cuda.synchronize()
    xb = bits(kv.contiguous())
    ref = oracle.quantize(xb, code_scale=p.code_scale, threads=8, anchor_bits=a)
    np.testing.assert_array_equal(host(codes.anchor).reshape(45, -1), ref.anchor.reshape(45, -1))
    np.testing.assert_array_equal(
        bits(outbig[:, :T, :Ch].contiguous()),
        oracle.dequant(ref, xb.shape, True, code_scale=p.code_scale, threads=8))
    pad = torch.ones_like(outbig, dtype=torch.bool)
    pad[:, :T, :Ch] = False
    assert bool((outbig[pad] == 7.0).all())


@pytest.mark.parametrize("a", [3, 5, 6])
def test_qwen32b_16k_two_layers(a):
    """Every block of two layers (K, V) of the Qwen-32B-shaped set."""
    cfg = kvgen.CONFIGS["qwen32b_16k"]
    kv = cfg.make(DEV, tensors=[0, 1, cfg.num_tensors - 2, cfg.num_tensors - 1])
    announce(f"a={a} qwen32b_16k layers 0 and 63 {tuple(kv.shape)}")
    check(kv, a, float(lynx.code_max(a)))

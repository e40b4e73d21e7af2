"""GPU parity of bfloat16 metadata (meta_bits = 16, the 4 + 4 split): the
codes, the four bfloat16 metadata arrays and both reconstructions against
the oracle, bit for bit, on the single-page workload, the adversarial
pages, alpha = 100, a strided multi-block set and two layers of the
Qwen-32B-shaped set."""
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
    print(f"[gpu-meta16] {msg}", flush=True)


def check(kv, alpha=255.0, code_scale=120.0):
    p = lynx.params(alpha=alpha, code_scale=code_scale, meta_bits=16)
    codes = lynx.quantize_pages(kv, p)
    assert codes.gamma_min.dtype == torch.bfloat16 and codes.mu.dtype == torch.bfloat16
    out_a = torch.empty_like(kv)
    out_f = torch.empty_like(kv)
    lynx.dequant_anchor(codes, out_a, p)
    lynx.dequant_full(codes, out_f, p)
    torch.cuda.synchronize()
    xb = bits(kv.contiguous())
    ref = oracle.quantize(xb, alpha=alpha, code_scale=code_scale, threads=8, meta_bits=16)
    nb = ref.nblocks
    np.testing.assert_array_equal(host(codes.anchor).reshape(nb, -1), ref.anchor.reshape(nb, -1))
    np.testing.assert_array_equal(host(codes.residual).reshape(nb, -1),
                                  ref.residual.reshape(nb, -1))
    for name in ("gamma_min", "gamma_scale", "mu", "sigma"):
        got = host(getattr(codes, name).float())
        want = getattr(ref, name)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), name
    np.testing.assert_array_equal(
        bits(out_a), oracle.dequant(ref, xb.shape, False, alpha=alpha, code_scale=code_scale,
                                    threads=8))
    np.testing.assert_array_equal(
        bits(out_f), oracle.dequant(ref, xb.shape, True, alpha=alpha, code_scale=code_scale,
                                    threads=8))
    return codes


def test_single_page_edge_pages_and_alpha():
    announce("single page")
    check(kvgen.CONFIGS["single_page"].make(DEV))
    pages = kvgen.edge_pages()
    announce("edge pages")
    check(torch.stack([pages[n] for n in sorted(pages)]).to(DEV))
    announce("alpha=100, code_scale=127")
    check(kvgen.CONFIGS["single_page"].make(DEV), alpha=100.0, code_scale=127.0)


def test_strided_set():
    nt, T, Ch = 3, 256 * 5, 128 * 3
    big = torch.empty((nt, T + 64, Ch + 24), dtype=torch.bfloat16, device=DEV)
    for i in range(nt):
        big[i, :T, :Ch] = kvgen.kv_tensor(900 + i, T, Ch, [5, 140, 300], True, DEV)
    announce(f"strided {nt}x{T}x{Ch}")
    check(big[:, :T, :Ch])


def test_qwen32b_16k_two_layers():
    cfg = kvgen.CONFIGS["qwen32b_16k"]
    kv = cfg.make(DEV, tensors=[0, 1, cfg.num_tensors - 2, cfg.num_tensors - 1])
    announce(f"qwen32b_16k layers 0 and 63 {tuple(kv.shape)}")
    check(kv)

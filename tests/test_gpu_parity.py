"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: anchor and residual bytes identical; metadata identical bit for bit
(binary32 patterns, so a zero statistic must carry the same sign as the
oracle's canonical +0); reconstructed bf16 bits
identical for the anchor-only and the full dequant.  Cases: the single-page
workload, adversarial pages, strided multi-block sets, other parameters,
the separately launched statistics kernels, determinism, and the two
full-size KV workloads: every page block of the Qwen-32B-shaped set at 16K;
every block of four layers plus a seeded 1% sample of all blocks of the
Qwen3-235B-A22B-shaped set at 128K.
"""
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


def same_bits(a, b):
    """Arrays equal bit for bit (float32 compared as their uint32 patterns)."""
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    if a.dtype == np.float32 and b.dtype == np.float32:
        a, b = a.view(np.uint32), b.view(np.uint32)
    return a.shape == b.shape and np.array_equal(a, b)


def announce(msg):
    print(f"[gpu-parity] {msg}", flush=True)


def run_gpu(kv, p=None):
    """quantize + anchor dequant + full dequant on the device."""
    codes = lynx.quantize_pages(kv, p)
    out_a = torch.empty_like(kv)
    out_f = torch.empty_like(kv)
    lynx.dequant_anchor(codes, out_a, p)
    lynx.dequant_full(codes, out_f, p)
    torch.cuda.synchronize()
    return codes, out_a, out_f


def assert_codes_equal(gpu: lynx.Codes, ref: oracle.Codes, sel=slice(None)):
    np.testing.assert_array_equal(host(gpu.anchor[sel]), ref.anchor)
    np.testing.assert_array_equal(host(gpu.residual[sel]), ref.residual)
    for name in ("gamma_min", "gamma_scale", "mu", "sigma"):
        g = host(getattr(gpu, name)[sel])
        r = getattr(ref, name)
        assert same_bits(g, r), name


def full_check(kv, alpha=255.0, eps=1e-6, code_scale=120.0):
    p = lynx.params(alpha=alpha, eps=eps, code_scale=code_scale)
    codes, out_a, out_f = run_gpu(kv, p)
    xb = bits(kv.contiguous())
    ref = oracle.quantize(xb, alpha=alpha, eps=eps, code_scale=code_scale, threads=8)
    assert_codes_equal(codes, ref)
    ra = oracle.dequant(ref, xb.shape, False, alpha=alpha, eps=eps, code_scale=code_scale,
                        threads=8)
    rf = oracle.dequant(ref, xb.shape, True, alpha=alpha, eps=eps, code_scale=code_scale,
                        threads=8)
    np.testing.assert_array_equal(bits(out_a), ra)
    np.testing.assert_array_equal(bits(out_f), rf)
    return codes


def test_single_page_kv():
    """The single-page workload: one K and one V block (3 outlier channels,
    one burst), all outputs exact."""
    announce("single_page K,V")
    kv = kvgen.CONFIGS["single_page"].make(DEV)
    full_check(kv)


def test_edge_pages():
    """Adversarial pages: constant channels / chunks, spikes, two-valued
    chunks, signed zeros, bf16 subnormals, huge dynamic range, 1e38
    magnitudes, all-negative, all-zero."""
    pages = kvgen.edge_pages()
    names = sorted(pages)
    announce(f"edge pages {names}")
    kv = torch.stack([pages[n] for n in names]).to(DEV)
    full_check(kv)


def test_non_finite_values_stay_in_their_block():
    """NaN and +-Inf in three of eight page blocks (outputs unspecified
    there): every launch completes and the other blocks' codes, metadata and
    reconstructions equal the oracle's on the clean set bit for bit (page
    blocks are independent; the compander clamps every magnitude into its
    table)."""
    announce("non-finite values in blocks 0, 3, 5 of 8")
    clean = torch.stack([kvgen.kv_tensor(610 + i, 512, 256, [7], True, DEV)
                         for i in range(2)])
    kv = clean.clone()
    kv[0, 5, 3] = float("nan")                    # block 0: tensor 0, page 0, head 0
    kv[0, 256 + 17, 128 + 9] = float("inf")       # block 3: tensor 0, page 1, head 1
    kv[1, 40:72, 128 + 100] = float("-inf")       # block 5: tensor 1, page 0, head 1
    kv[1, 44, 128 + 3] = float("nan")
    codes, out_a, out_f = run_gpu(kv)
    xb = bits(clean)
    ref = oracle.quantize(xb, threads=8)
    keep = [1, 2, 4, 6, 7]
    nb = 8
    for name in ("anchor", "residual", "gamma_min", "gamma_scale", "mu", "sigma"):
        g = host(getattr(codes, name)).reshape(nb, -1)[keep]
        r = np.asarray(getattr(ref, name)).reshape(nb, -1)[keep]
        assert same_bits(g, r), name
    for full, out in ((False, out_a), (True, out_f)):
        rd = oracle.dequant(ref, xb.shape, full, threads=8)
        got = bits(out)
        for b in keep:
            t, rest = divmod(b, 4)
            page, head = divmod(rest, 2)
            rows = slice(256 * page, 256 * page + 256)
            cols = slice(128 * head, 128 * head + 128)
            np.testing.assert_array_equal(got[t, rows, cols], rd[t, rows, cols])


def test_strided_multi_block_set():
    """3 tensors x 5 pages x 3 heads inside padded rows and tensors; the
    padding of the dequant outputs is left untouched."""
    announce("strided 3x1280x384 in padded buffers")
    nt, T, Ch = 3, 256 * 5, 128 * 3
    big = torch.empty((nt, T + 64, Ch + 24), dtype=torch.bfloat16, device=DEV)
    for i in range(nt):
        big[i, :T, :Ch] = kvgen.kv_tensor(300 + i, T, Ch, [5, 140, 300], True, DEV)
    kv = big[:, :T, :Ch]
    assert kv.stride(1) == Ch + 24
    p = lynx.params()
    codes = lynx.quantize_pages(kv, p)
    outbig = torch.full_like(big, 7.0)
    out = outbig[:, :T, :Ch]
    lynx.dequant_full(codes, out, p)
    torch.cuda.synchronize()
    xb = bits(kv.contiguous())
    ref = oracle.quantize(xb, threads=8)
    assert_codes_equal(codes, ref)
    np.testing.assert_array_equal(bits(out.contiguous()),
                                  oracle.dequant(ref, xb.shape, True, threads=8))
    pad = torch.ones_like(outbig, dtype=torch.bool)
    pad[:, :T, :Ch] = False
    assert bool((outbig[pad] == 7.0).all())


@pytest.mark.parametrize("alpha,eps,code_scale", [(100.0, 1e-6, 127.0),
                                                  # Eq. (3)'s printed 127, clip at 120
                                                  (255.0, 1e-6, 127.0),
                                                  (255.0, 2.0 ** -20, 127.0),
                                                  (8.0, 1e-3, 127.0),
                                                  # thresholds over > 16 octaves: the
                                                  # compander falls back to coarser buckets
                                                  (1e6, 1e-6, 127.0),
                                                  (1e12, 1e-6, 127.0)])
def test_parameter_variants(alpha, eps, code_scale):
    announce(f"params alpha={alpha} eps={eps} code_scale={code_scale}")
    kv = torch.stack([kvgen.kv_tensor(400 + i, 512, 256, [7, 200], True, DEV)
                      for i in range(2)])
    full_check(kv, alpha, eps, code_scale)


def test_stats_kernels_match_fused():
    """lynx_page_stats and lynx_block_stats give the fused kernel's
    metadata (and hence the oracle's)."""
    announce("stats kernels")
    kv = torch.stack([kvgen.kv_tensor(500 + i, 1024, 256, [9], True, DEV) for i in range(2)])
    codes = lynx.quantize_pages(kv)
    nb = codes.gamma_min.shape[0]
    gmin = torch.empty((nb, 128), device=DEV)
    gsc = torch.empty((nb, 128), device=DEV)
    mu = torch.empty((nb, 8, 128), device=DEV)
    sg = torch.empty((nb, 8, 128), device=DEV)
    lynx.page_stats(kv, gmin, gsc)
    lynx.block_stats(kv, gmin, gsc, mu, sg)
    torch.cuda.synchronize()
    for a, b in ((gmin, codes.gamma_min), (gsc, codes.gamma_scale), (mu, codes.mu),
                 (sg, codes.sigma)):
        assert same_bits(host(a), host(b))
    ref = oracle.quantize(bits(kv), threads=8)
    assert same_bits(host(mu), ref.mu) and same_bits(host(gsc), ref.gamma_scale)
    assert same_bits(host(gmin), ref.gamma_min) and same_bits(host(sg), ref.sigma)


def test_determinism():
    announce("determinism")
    kv = torch.stack([kvgen.kv_tensor(600 + i, 2048, 1024, [1, 500], True, DEV)
                      for i in range(2)])
    c1, a1, f1 = run_gpu(kv)
    c2, a2, f2 = run_gpu(kv)
    for n in ("anchor", "residual", "gamma_min", "gamma_scale", "mu", "sigma"):
        assert torch.equal(getattr(c1, n), getattr(c2, n)), n
    assert torch.equal(a1.view(torch.int16), a2.view(torch.int16))
    assert torch.equal(f1.view(torch.int16), f2.view(torch.int16))


def _block_region(b, pages, heads):
    head = b % heads
    page = (b // heads) % pages
    tensor = b // (heads * pages)
    return tensor, slice(page * 256, page * 256 + 256), slice(head * 128, head * 128 + 128)


def test_qwen32b_16k_every_block():
    """The whole Qwen-32B-shaped set (64 layers x K,V x 16384 x 1024, 65536
    page blocks, 4 GiB bf16): every block's codes, metadata and both
    reconstructions equal to the oracle's (16 host threads)."""
    cfg = kvgen.CONFIGS["qwen32b_16k"]
    announce(f"{cfg.name}: generating {cfg.num_tensors} x {cfg.num_tokens} x "
             f"{cfg.num_channels} on the device")
    kv = cfg.make(DEV)
    announce(f"{cfg.name}: quantize + dequant on the device")
    codes, out_a, out_f = run_gpu(kv)
    xb = bits(kv)
    del kv
    announce(f"{cfg.name}: oracle on every one of the {xb.size // 32768} blocks")
    ref = oracle.quantize(xb, threads=16)
    assert_codes_equal(codes, ref)
    del codes
    for out, full in ((out_a, False), (out_f, True)):
        np.testing.assert_array_equal(bits(out), oracle.dequant(ref, xb.shape, full, threads=16))
    del out_a, out_f
    torch.cuda.empty_cache()


def test_qwen3_235b_128k_four_layers_and_sample():
    """The Qwen3-235B-A22B-shaped set (94 layers x K,V x 131072 x 512, 23.5
    GiB bf16, 385024 blocks) on the device: every block of layers 0, 31, 62
    and 93 against the oracle, and a seeded 1% sample of all blocks against
    the oracle's block routine."""
    cfg = kvgen.CONFIGS["qwen3_235b_128k"]
    announce(f"{cfg.name}: generating {cfg.num_tensors} x {cfg.num_tokens} x "
             f"{cfg.num_channels} on the device")
    kv = cfg.make(DEV)
    announce(f"{cfg.name}: quantize + dequant on the device")
    codes, out_a, out_f = run_gpu(kv)
    pages, heads = cfg.num_tokens // 256, cfg.num_channels // 128
    per_tensor = pages * heads
    layers = [0, 31, 62, 93]
    tensors = [2 * l + kv_ for l in layers for kv_ in (0, 1)]
    announce(f"{cfg.name}: every block of layers {layers}")
    for t in tensors:
        xb = bits(kv[t:t + 1])
        ref = oracle.quantize(xb, threads=16)
        assert_codes_equal(codes, ref, slice(t * per_tensor, (t + 1) * per_tensor))
        for out, full in ((out_a, False), (out_f, True)):
            np.testing.assert_array_equal(bits(out[t:t + 1]),
                                          oracle.dequant(ref, xb.shape, full, threads=16))
    nb = cfg.num_tensors * per_tensor
    rng = np.random.default_rng(12)
    sample = sorted(set([0, 1, nb - 1] + list(rng.choice(nb, nb // 100, replace=False))))
    announce(f"{cfg.name}: sampled {len(sample)} of {nb} blocks")
    for b in sample:
        t, rows, cols = _block_region(b, pages, heads)
        xb = bits(kv[t, rows, cols])
        r = oracle.quantize_block(xb)
        np.testing.assert_array_equal(host(codes.anchor[b]), r.anchor)
        np.testing.assert_array_equal(host(codes.residual[b]), r.residual)
        for name in ("gamma_min", "gamma_scale", "mu", "sigma"):
            assert same_bits(host(getattr(codes, name)[b]), getattr(r, name)), (b, name)
        np.testing.assert_array_equal(bits(out_a[t, rows, cols]), oracle.dequant_block(r, False))
        np.testing.assert_array_equal(bits(out_f[t, rows, cols]), oracle.dequant_block(r, True))
    del kv, codes, out_a, out_f
    torch.cuda.empty_cache()

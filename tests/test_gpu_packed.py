"""The packed code layout (the paper's transmission buffer: every page
block's anchor stream followed immediately by its scalars; Section 4.2,
prefill workflow step 3, and Section 5, "Compression Kernel") on the GPU
against the CPU oracle: the expected record buffer is assembled from the
oracle's outputs in the documented order (anchor stream, gamma_min,
gamma_scale, mu, sigma) and compared byte for byte; both reconstructions,
attention and the split-stream transfer run on packed codes and give the
oracle's results (attention: the separate layout's output bit for bit)."""
import numpy as np
import pytest
import torch

import oracle
from progressive_kv_transfer_amd import kvgen, lynx

pytestmark = pytest.mark.gpu
DEV = "cuda"


def announce(msg):
    print(f"[gpu-packed] {msg}", flush=True)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.uint8).numpy()


def expected_records(ref: oracle.Codes, meta_bits: int = 32) -> np.ndarray:
    """[nblocks, record bytes]: per block the anchor stream, then gamma_min,
    gamma_scale, mu, sigma (binary32, or the bfloat16 patterns: the upper
    halves of the oracle's binary32 values, which are bfloat16 values)."""
    nb = ref.nblocks
    parts = [np.ascontiguousarray(ref.anchor).reshape(nb, -1)]
    for name in ("gamma_min", "gamma_scale", "mu", "sigma"):
        a = np.ascontiguousarray(getattr(ref, name), np.float32).reshape(nb, -1)
        if meta_bits == 16:
            a = (a.view(np.uint32) >> 16).astype(np.uint16)
        parts.append(a.view(np.uint8).reshape(nb, -1))
    return np.concatenate(parts, axis=1)


def kv_set(seed=900):
    return torch.stack([kvgen.kv_tensor(seed + i, 1024, 512, [5, 300], True, DEV)
                        for i in range(2)])


@pytest.mark.parametrize("anchor_bits,meta_bits", [(4, 32), (4, 16), (3, 32), (6, 32)])
def test_packed_quantize_and_dequant(anchor_bits, meta_bits):
    announce(f"packed quantize a={anchor_bits} meta_bits={meta_bits}")
    kv = kv_set()
    p = lynx.params(anchor_bits=anchor_bits, meta_bits=meta_bits, layout=lynx.LAYOUT_PACKED)
    assert lynx.anchor_block_bytes(p) == 4096 * anchor_bits + 2304 * meta_bits // 8
    codes = lynx.quantize_pages(kv, p)
    assert codes.packed
    out_a, out_f = torch.empty_like(kv), torch.empty_like(kv)
    lynx.dequant_anchor(codes, out_a, p)
    lynx.dequant_full(codes, out_f, p)
    torch.cuda.synchronize()
    xb = kvgen.bf16_bits(kv)
    ref = oracle.quantize(xb, threads=8, anchor_bits=anchor_bits, meta_bits=meta_bits)
    want = expected_records(ref, meta_bits)
    assert np.array_equal(u8(codes.records), want)
    assert np.array_equal(u8(codes.residual).reshape(ref.nblocks, -1),
                          np.ascontiguousarray(ref.residual).reshape(ref.nblocks, -1))
    np.testing.assert_array_equal(kvgen.bf16_bits(out_a),
                                  oracle.dequant(ref, xb.shape, False, threads=8))
    np.testing.assert_array_equal(kvgen.bf16_bits(out_f),
                                  oracle.dequant(ref, xb.shape, True, threads=8))


def test_packed_attention_equals_separate():
    """Decode and verification attention on packed K / V codes: the output of
    the separate layout's codes bit for bit (same kernels, other strides)."""
    announce("attention packed vs separate")
    ctx, nkvh = 2048, 2
    kv = torch.stack([kvgen.kv_tensor(910 + i, ctx, nkvh * 128, [3], True, DEV) for i in range(2)])
    nb = ctx // 256 * nkvh
    ps = lynx.params()
    pp = lynx.params(layout=lynx.LAYOUT_PACKED)
    cs, cp = lynx.quantize_pages(kv, ps), lynx.quantize_pages(kv, pp)
    for t_q, nqh, full, causal in ((1, 16, False, False), (1, 16, True, False), (8, 8, True, True)):
        q = kvgen.queries(911, t_q, nqh, device=DEV)
        o_s = lynx.decode_attn_dequant(q, lynx.CodeView(cs, 0, nb, full),
                                       lynx.CodeView(cs, nb, 2 * nb, full), ctx, nkvh,
                                       128 ** -0.5, causal, ps, out_dtype=torch.float32)
        o_p = lynx.decode_attn_dequant(q, lynx.CodeView(cp, 0, nb, full),
                                       lynx.CodeView(cp, nb, 2 * nb, full), ctx, nkvh,
                                       128 ** -0.5, causal, pp, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(o_s.view(torch.int32), o_p.view(torch.int32)), (t_q, full, causal)


@pytest.mark.parametrize("object_blocks", [1, 5, 16, 100])
def test_packed_transfer_matches_oracle(object_blocks):
    """The split-stream transfer on packed codes: one copy per hop for each
    object's anchor + metadata records and one for its residual; tx, wire
    and rx equal the oracle's assembled records byte for byte, the caches
    rebuilt on the receiver equal the oracle's reconstructions bit for bit."""
    announce(f"packed transfer object_blocks={object_blocks}")
    kv = kv_set(920)
    shape = lynx.shape_of(kv)
    nb = lynx.num_blocks(shape)
    p = lynx.params(layout=lynx.LAYOUT_PACKED)
    tx = lynx.alloc_codes(nb, DEV, layout=lynx.LAYOUT_PACKED)
    rx = lynx.alloc_codes(nb, DEV, layout=lynx.LAYOUT_PACKED)
    wire = lynx.alloc_codes(nb, "cpu", pin_memory=True, layout=lynx.LAYOUT_PACKED)
    for c in (tx, rx, wire):
        c.records.fill_(0x5a)
        c.residual.fill_(0x5a)
    out_a, out_f = torch.full_like(kv, 7.0), torch.full_like(kv, 7.0)
    torch.cuda.synchronize()
    times = lynx.split_stream_transfer(kv, shape, object_blocks, tx, wire, rx, out_a, out_f, p=p)
    xb = kvgen.bf16_bits(kv)
    ref = oracle.quantize(xb, threads=8)
    want = expected_records(ref)
    for where, c in (("tx", tx), ("wire", wire), ("rx", rx)):
        assert np.array_equal(u8(c.records), want), where
        assert np.array_equal(u8(c.residual).reshape(nb, -1),
                              np.ascontiguousarray(ref.residual).reshape(nb, -1)), where
    np.testing.assert_array_equal(kvgen.bf16_bits(out_a),
                                  oracle.dequant(ref, xb.shape, False, threads=8))
    np.testing.assert_array_equal(kvgen.bf16_bits(out_f),
                                  oracle.dequant(ref, xb.shape, True, threads=8))
    assert times["anchor_arrived"] <= times["residual_arrived"] + 1e-3

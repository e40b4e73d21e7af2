"""GPU checks of the split-stream transfer (lynx_split_stream_transfer): the
codes that arrive, and the caches rebuilt from them, are bit-identical to
quantizing and rebuilding in place; the milestones come in the order the
protocol imposes."""
import pytest
import torch

from progressive_kv_transfer_amd import kvgen, lynx

pytestmark = pytest.mark.gpu
DEV = "cuda"


def announce(msg):
    print(f"[gpu-transfer] {msg}", flush=True)


def same_codes(a: lynx.Codes, b: lynx.Codes):
    for x, y in zip(a.tensors(), b.tensors()):
        assert torch.equal(x.cpu().view(torch.uint8), y.cpu().view(torch.uint8))


@pytest.mark.parametrize("object_blocks", [1, 7, 64, 1000])
def test_transfer_round_trip(object_blocks):
    """2 tensors x 2048 tokens x 512 channels = 64 page blocks, objects of
    1, 7 (ragged last object), 64 and more than all blocks."""
    announce(f"round trip object_blocks={object_blocks}")
    kv = torch.stack([kvgen.kv_tensor(800 + i, 2048, 512, [5, 300], True, DEV)
                      for i in range(2)])
    shape = lynx.shape_of(kv)
    nb = lynx.num_blocks(shape)
    ref = lynx.quantize_pages(kv)
    ref_a = torch.empty_like(kv)
    ref_f = torch.empty_like(kv)
    lynx.dequant_anchor(ref, ref_a)
    lynx.dequant_full(ref, ref_f)
    tx, rx = lynx.alloc_codes(nb, DEV), lynx.alloc_codes(nb, DEV)
    wire = lynx.alloc_codes(nb, "cpu", pin_memory=True)
    for c in (tx, rx):
        for t in c.tensors():
            t.fill_(0)
    out_a = torch.full_like(kv, 7.0)
    out_f = torch.full_like(kv, 7.0)
    torch.cuda.synchronize()
    times = lynx.split_stream_transfer(kv, shape, object_blocks, tx, wire, rx, out_a, out_f)
    same_codes(tx, ref)
    same_codes(rx, ref)
    assert torch.equal(wire.anchor, ref.anchor.cpu())
    assert torch.equal(out_a.view(torch.int16), ref_a.view(torch.int16))
    assert torch.equal(out_f.view(torch.int16), ref_f.view(torch.int16))
    t = times
    assert 0.0 < t["quantized"] <= t["anchor_arrived"] + 1e-3
    assert t["anchor_arrived"] <= t["residual_arrived"] + 1e-3
    assert t["first_anchor_ready"] <= t["anchor_ready"] + 1e-3
    assert t["anchor_arrived"] <= t["anchor_ready"] + 1e-3
    assert t["residual_arrived"] <= t["full_ready"] + 1e-3
    assert t["anchor_ready"] <= t["full_ready"] + 1e-3


def test_transfer_copies_only():
    """The link alone moves existing codes and touches no cache."""
    announce("copies only")
    kv = kvgen.kv_tensor(810, 1024, 256, [], True, DEV)[None]
    shape = lynx.shape_of(kv)
    nb = lynx.num_blocks(shape)
    tx = lynx.quantize_pages(kv)
    rx = lynx.alloc_codes(nb, DEV)
    wire = lynx.alloc_codes(nb, "cpu", pin_memory=True)
    times = lynx.split_stream_transfer(None, shape, 3, tx, wire, rx, copies_only=True)
    same_codes(rx, tx)
    assert times["quantized"] >= 0.0 and times["full_ready"] >= times["residual_arrived"] - 1e-3

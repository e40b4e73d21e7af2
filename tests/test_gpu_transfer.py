"""GPU checks of the split-stream transfer (lynx_split_stream_transfer)
against the CPU oracle: the codes on every hop (tx on the sender, the wire,
rx on the receiver) equal the oracle's Algorithm 1 outputs byte for byte and
bit for bit, and the caches rebuilt from them equal the oracle's anchor-only
and full reconstructions (the paper's Section 4.2, Figure 7(a)-(c): Q_anc
and the metadata first, then Q_res, then the two rebuilds); the milestones
come in the order the protocol imposes."""
import numpy as np
import pytest
import torch

import oracle
from progressive_kv_transfer_amd import kvgen, lynx

pytestmark = pytest.mark.gpu
DEV = "cuda"


def announce(msg):
    print(f"[gpu-transfer] {msg}", flush=True)


def u8(t: torch.Tensor) -> np.ndarray:
    """Bytes of a code tensor (device or host), as numpy uint8."""
    return t.detach().contiguous().cpu().view(torch.uint8).numpy().reshape(-1)


def assert_codes_match_oracle(got: lynx.Codes, ref: oracle.Codes, where: str):
    for name in ("anchor", "residual", "gamma_min", "gamma_scale", "mu", "sigma"):
        want = np.ascontiguousarray(getattr(ref, name)).view(np.uint8).reshape(-1)
        assert np.array_equal(u8(getattr(got, name)), want), f"{where}: {name}"


def oracle_set(kv: torch.Tensor):
    """Oracle codes and both reconstructions of a device KV set."""
    xb = kvgen.bf16_bits(kv)
    ref = oracle.quantize(xb, threads=8)
    ra = oracle.dequant(ref, xb.shape, False, threads=8)
    rf = oracle.dequant(ref, xb.shape, True, threads=8)
    return ref, ra, rf


@pytest.fixture(scope="module")
def kv_set():
    """2 tensors x 2048 tokens x 512 channels = 64 page blocks (32 per
    tensor), with outlier channels and bursts."""
    kv = torch.stack([kvgen.kv_tensor(800 + i, 2048, 512, [5, 300], True, DEV)
                      for i in range(2)])
    return kv, oracle_set(kv)


@pytest.mark.parametrize("object_blocks", [1, 3, 7, 13, 64, 1000])
def test_transfer_matches_oracle(kv_set, object_blocks):
    """Objects of 1 block, of 3, 7 and 13 blocks (ragged last object;
    objects that start mid-tensor and straddle the tensor boundary, so most
    launches start at a block offset that is not a tensor start), all 64
    blocks in one object, and more than all blocks."""
    kv, (ref, ra, rf) = kv_set
    announce(f"transfer vs oracle object_blocks={object_blocks}")
    shape = lynx.shape_of(kv)
    nb = lynx.num_blocks(shape)
    assert nb == ref.nblocks == 64
    tx, rx = lynx.alloc_codes(nb, DEV), lynx.alloc_codes(nb, DEV)
    wire = lynx.alloc_codes(nb, "cpu", pin_memory=True)
    for c in (tx, rx, wire):
        for t in c.tensors():
            t.fill_(0x55 if t.dtype == torch.uint8 else 3.0)
    out_a = torch.full_like(kv, 7.0)
    out_f = torch.full_like(kv, 7.0)
    torch.cuda.synchronize()
    times = lynx.split_stream_transfer(kv, shape, object_blocks, tx, wire, rx, out_a, out_f)
    for where, c in (("tx", tx), ("wire", wire), ("rx", rx)):
        assert_codes_match_oracle(c, ref, where)
    np.testing.assert_array_equal(kvgen.bf16_bits(out_a), ra)
    np.testing.assert_array_equal(kvgen.bf16_bits(out_f), rf)
    t = times
    assert 0.0 < t["quantized"] <= t["anchor_arrived"] + 1e-3
    assert t["anchor_arrived"] <= t["residual_arrived"] + 1e-3
    assert t["first_anchor_ready"] <= t["anchor_ready"] + 1e-3
    assert t["anchor_arrived"] <= t["anchor_ready"] + 1e-3
    assert t["residual_arrived"] <= t["full_ready"] + 1e-3
    assert t["anchor_ready"] <= t["full_ready"] + 1e-3


def test_transfer_copies_only():
    """The link alone moves the oracle's codes unchanged (wire and rx equal
    the oracle byte for byte) and touches no cache."""
    announce("copies only")
    kv = kvgen.kv_tensor(810, 1024, 256, [], True, DEV)[None]
    shape = lynx.shape_of(kv)
    nb = lynx.num_blocks(shape)
    ref, _, _ = oracle_set(kv)
    tx = lynx.alloc_codes(nb, DEV)
    for name in ("anchor", "residual", "gamma_min", "gamma_scale", "mu", "sigma"):
        getattr(tx, name).copy_(torch.from_numpy(np.ascontiguousarray(getattr(ref, name))))
    rx = lynx.alloc_codes(nb, DEV)
    wire = lynx.alloc_codes(nb, "cpu", pin_memory=True)
    times = lynx.split_stream_transfer(None, shape, 3, tx, wire, rx, copies_only=True)
    for where, c in (("wire", wire), ("rx", rx)):
        assert_codes_match_oracle(c, ref, where)
    assert times["quantized"] >= 0.0 and times["full_ready"] >= times["residual_arrived"] - 1e-3


@pytest.mark.parametrize("reserved", [8, 16, 32, 64, 0])
def test_transfer_on_codec_streams_matches_oracle(kv_set, reserved):
    """Sender and receiver on lynx_codec_stream_create streams (kernels kept
    off `reserved` compute units; 0 = a plain stream): the codes on every hop
    and both rebuilds still equal the oracle's."""
    kv, (ref, ra, rf) = kv_set
    announce(f"transfer on codec streams reserved={reserved}")
    shape = lynx.shape_of(kv)
    nb = lynx.num_blocks(shape)
    tx, rx = lynx.alloc_codes(nb, DEV), lynx.alloc_codes(nb, DEV)
    wire = lynx.alloc_codes(nb, "cpu", pin_memory=True)
    out_a = torch.full_like(kv, 7.0)
    out_f = torch.full_like(kv, 7.0)
    sender, receiver = lynx.CodecStream(reserved), lynx.CodecStream(reserved)
    torch.cuda.synchronize()
    streams = (sender.stream, torch.cuda.Stream(), torch.cuda.Stream(), receiver.stream)
    lynx.split_stream_transfer(kv, shape, 7, tx, wire, rx, out_a, out_f, streams=streams)
    sender.close()
    receiver.close()
    for where, c in (("tx", tx), ("wire", wire), ("rx", rx)):
        assert_codes_match_oracle(c, ref, where)
    np.testing.assert_array_equal(kvgen.bf16_bits(out_a), ra)
    np.testing.assert_array_equal(kvgen.bf16_bits(out_f), rf)


def test_codec_stream_errors():
    """A reserve of every compute unit (or more) and a negative reserve are
    refused before any stream is made."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    for bad in (ncu, ncu + 5, -1):
        with pytest.raises(lynx.LynxError):
            lynx.CodecStream(bad)

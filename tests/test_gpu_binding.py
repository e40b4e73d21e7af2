"""GPU-side checks of the Python binding: device calls refuse host (CPU)
output, workspace and metadata tensors with a ValueError before anything is
launched (the C ABI takes bare pointers, so a host address would be written
by a kernel)."""
import pytest
import torch

from progressive_kv_transfer_amd import kvgen, lynx

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _attn_set():
    kv = torch.stack([kvgen.kv_tensor(700 + i, 512, 128, [3], True, DEV) for i in range(2)])
    codes = lynx.quantize_pages(kv)
    q = kvgen.queries(701, 1, 8, device=DEV)
    return q, lynx.CodeView(codes, 0, 2), lynx.CodeView(codes, 2, 4)


def test_attention_refuses_host_out_and_workspace():
    print("[gpu-binding] attention host buffers", flush=True)
    q, k, v = _attn_set()
    with pytest.raises(ValueError):
        lynx.decode_attn_dequant(q, k, v, 512, 1, 128 ** -0.5,
                                 out=torch.empty(q.shape, dtype=torch.bfloat16))
    need = lynx.attn_workspace_bytes(1, 8, 1, 512)
    with pytest.raises(ValueError):
        lynx.decode_attn_dequant(q, k, v, 512, 1, 128 ** -0.5,
                                 workspace=torch.empty(need, dtype=torch.uint8))
    # the same call with device buffers runs
    out = lynx.decode_attn_dequant(q, k, v, 512, 1, 128 ** -0.5)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())


def test_stats_refuse_host_or_short_metadata():
    print("[gpu-binding] statistics buffers", flush=True)
    kv = kvgen.kv_tensor(702, 512, 256, [], True, DEV)[None]
    nb = 4
    with pytest.raises(ValueError):
        lynx.page_stats(kv, torch.empty((nb, 128)), torch.empty((nb, 128), device=DEV))
    with pytest.raises(ValueError):
        lynx.page_stats(kv, torch.empty((nb, 128), device=DEV),
                        torch.empty((nb - 1, 128), device=DEV))
    with pytest.raises(ValueError):
        lynx.block_stats(kv, torch.empty((nb, 128), device=DEV),
                         torch.empty((nb, 128), device=DEV),
                         torch.empty((nb, 8, 128), device=DEV, dtype=torch.float64),
                         torch.empty((nb, 8, 128), device=DEV))


def test_spec_verify_refuses_host_workspace():
    print("[gpu-binding] verification workspace", flush=True)
    draft, target, tokens, u, us = kvgen.verify_inputs(703, 4, 1000, 0.3)
    ws = torch.empty(lynx.spec_verify_workspace_bytes(4, 1000), dtype=torch.uint8)
    with pytest.raises(ValueError):
        lynx.spec_verify(draft.to(DEV), target.to(DEV), tokens.to(DEV), u.to(DEV), us,
                         workspace=ws)

"""The allocation-free attention entry point, lynx_decode_attn_dequant_noalloc
(split partials in the library's fixed device scratch), called through the
C ABI and compared bit for bit with lynx_decode_attn_dequant (partials in a
caller's workspace) on consecutive calls: a verification-shaped call, then a
smaller decode call (the scratch keeps the first call's partials, which the
second must not read), then the first call again."""
import pytest
import torch

from progressive_kv_transfer_amd import kvgen, lynx

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(seed, t_q, nqh, nkvh, ctx, full, causal, out_dtype):
    kv = torch.stack([kvgen.kv_tensor(seed + i, ctx, nkvh * 128, [5], True, DEV)
                      for i in range(2)])
    codes = lynx.quantize_pages(kv)
    nb = ctx // 256 * nkvh
    k = lynx.CodeView(codes, 0, nb, full)
    v = lynx.CodeView(codes, nb, 2 * nb, full)
    q = kvgen.queries(seed + 7, t_q, nqh, device=DEV)
    return q, k, v, ctx, nkvh, causal, out_dtype


def _compare(case, label):
    q, k, v, ctx, nkvh, causal, out_dtype = case
    print(f"[no-alloc] {label}: t_q={q.shape[0]} q_heads={q.shape[1]} kv_heads={nkvh} "
          f"ctx={ctx} full={k.full} causal={causal}", flush=True)
    need = lynx.attn_workspace_bytes(q.shape[0], q.shape[1], nkvh, ctx)
    assert 0 < need <= lynx.ATTN_SCRATCH_BYTES
    ref = lynx.decode_attn_dequant(q, k, v, ctx, nkvh, 128 ** -0.5, causal,
                                   out_dtype=out_dtype)
    out = torch.full(q.shape, 3.0, dtype=out_dtype, device=DEV)
    lynx.decode_attn_dequant_noalloc(q, k, v, ctx, nkvh, 128 ** -0.5, out, causal)
    torch.cuda.synchronize()
    view = torch.int32 if out_dtype == torch.float32 else torch.int16
    assert torch.equal(out.view(view), ref.view(view)), label


def test_noalloc_matches_workspace_entry_point():
    big = _case(9100, 8, 32, 4, 16384, True, True, torch.float32)
    small = _case(9200, 1, 16, 2, 1024, False, False, torch.bfloat16)
    _compare(big, "call 1 (verification shape)")
    _compare(small, "call 2 (smaller decode)")
    _compare(big, "call 3 (first shape again)")

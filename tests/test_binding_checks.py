"""CPU tests of the Python binding's own checks (no GPU): the statistics
calls refuse wrongly typed or too small metadata arrays, a non-bf16 KV set
and host tensors with a ValueError before the library is touched (the C ABI
sees bare pointers, so a short or misplaced buffer would be written past its
end or through a host address)."""
import pytest
import torch

from progressive_kv_transfer_amd import lynx


@pytest.fixture
def no_library(monkeypatch):
    """Any library call fails the test."""
    def boom():
        raise AssertionError("the library was called before the checks")
    monkeypatch.setattr(lynx, "lib", boom)


def _stats_args(nb_tokens=512, ch=256):
    kv = torch.zeros((1, nb_tokens, ch), dtype=torch.bfloat16)
    nb = (nb_tokens // 256) * (ch // 128)
    return kv, nb


@pytest.mark.parametrize("case,msg", [
    ("kv_dtype", "bfloat16"), ("gmin_dtype", "float32"), ("gscale_short", "needed"),
    ("host", "device")])
def test_page_stats_refuses_before_any_call(no_library, case, msg):
    kv, nb = _stats_args()
    gmin = torch.zeros((nb, 128))
    gsc = torch.zeros((nb, 128))
    if case == "kv_dtype":
        kv = kv.float()
    elif case == "gmin_dtype":
        gmin = gmin.double()
    elif case == "gscale_short":
        gsc = torch.zeros((nb - 1, 128))
    with pytest.raises(ValueError, match=msg):
        lynx.page_stats(kv, gmin, gsc)


@pytest.mark.parametrize("case,msg", [
    ("mu_short", "needed"), ("sigma_dtype", "float32"), ("sigma_strided", "contiguous"),
    ("meta16", "binary32"), ("host", "device")])
def test_block_stats_refuses_before_any_call(no_library, case, msg):
    kv, nb = _stats_args()
    gmin, gsc = torch.zeros((nb, 128)), torch.zeros((nb, 128))
    mu, sg = torch.zeros((nb, 8, 128)), torch.zeros((nb, 8, 128))
    p = None
    if case == "mu_short":
        mu = torch.zeros((nb, 7, 128))
    elif case == "sigma_dtype":
        sg = sg.half()
    elif case == "sigma_strided":
        sg = torch.zeros((nb, 8, 256))[:, :, ::2]
    elif case == "meta16":
        p = lynx.lynx_params()
        p.meta_bits = 16
    with pytest.raises(ValueError, match=msg):
        lynx.block_stats(kv, gmin, gsc, mu, sg, p)


def test_block_count_without_the_library(no_library):
    s = lynx.shape_of(torch.zeros((3, 1024, 384), dtype=torch.bfloat16))
    assert lynx._blocks_of(s) == 3 * 4 * 3
    s.num_tokens = 300
    assert lynx._blocks_of(s) == 0

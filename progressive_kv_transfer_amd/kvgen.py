"""Seeded synthetic KV and query generators.

This module produces inputs only; it holds none of the quantizer's arithmetic
and imports neither the GPU binding nor the CPU oracle, so both sides can be
fed the same bytes.

Value structure follows what the Lynx paper shows of real KV caches
("Lynx: Progressive Speculative Quantization for accelerating KV Transfer in
Long-Context Inference", Section 2.3 and Figure 4: a few channels hold values
up to 100x larger than the rest, as horizontal stripes; Section 3.2 and
Figure 5: after per-channel normalisation the values are Laplacian-like,
about half of them inside the middle 17% of the range):

  per channel c : offset o_c ~ U(-2, 2), scale s_c = exp(N(0, 0.5^2)),
                  both fixed over all tokens;
  element       : x[t, c] = o_c + s_c * Laplace(0, 1);
  outliers      : the whole value of a seeded set of channels is x100
                  (1% of the channels of a tensor, at least one per
                  128-channel head when requested per head);
  bursts        : per 256-token x 128-channel page block, one seeded
                  non-outlier channel gets x20 on 32 consecutive tokens whose
                  start is seeded and never a multiple of 32;
  cast          : bfloat16, round-to-nearest-even.

Everything is drawn from torch.Generator streams seeded per tensor, on the
device the caller names, so a given (seed, device) is reproducible.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

PAGE = 256
HEAD = 128
CHUNK = 32


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def outlier_channels(num_channels: int, count: int, seed: int) -> list[int]:
    """A seeded set of `count` distinct channels (host-side, device-free)."""
    g = torch.Generator()
    g.manual_seed(int(seed))
    perm = torch.randperm(num_channels, generator=g)
    return sorted(int(c) for c in perm[:count])


def outlier_channels_per_head(num_channels: int, per_head: int,
                              seed: int) -> list[int]:
    """`per_head` seeded outlier channels inside every 128-channel head."""
    out = []
    for h in range(num_channels // HEAD):
        out += [h * HEAD + c for c in outlier_channels(HEAD, per_head,
                                                        seed * 7919 + h)]
    return out


def kv_tensor(seed: int, num_tokens: int, num_channels: int,
              outliers: list[int], bursts: bool = True, device="cpu",
              out: torch.Tensor | None = None) -> torch.Tensor:
    """One token-major [num_tokens][num_channels] bf16 KV tensor."""
    g = _gen(seed, device)
    T, Ch = num_tokens, num_channels
    off = torch.rand(Ch, generator=g, device=device) * 4.0 - 2.0
    scale = torch.exp(torch.randn(Ch, generator=g, device=device) * 0.5)
    lap = torch.empty((T, Ch), device=device).exponential_(1.0, generator=g)
    neg = torch.rand((T, Ch), generator=g, device=device) < 0.5
    lap = torch.where(neg, -lap, lap)
    x = off + scale * lap
    del lap, neg
    if outliers:
        x[:, torch.tensor(outliers, device=device)] *= 100.0
    if bursts and T >= PAGE and Ch >= HEAD:
        pages, heads = T // PAGE, Ch // HEAD
        nb = pages * heads
        mask = torch.zeros(Ch, dtype=torch.bool)
        if outliers:
            mask[torch.tensor(outliers)] = True
        # Seeded channel inside the head, redrawn until it is not an outlier.
        ch_in = torch.randint(0, HEAD, (nb,), generator=g, device=device).cpu()
        head_of = torch.arange(nb) % heads
        ch = head_of * HEAD + ch_in
        for _ in range(64):
            bad = mask[ch]
            if not bool(bad.any()):
                break
            ch = torch.where(bad, head_of * HEAD + (ch_in + 1) % HEAD, ch)
            ch_in = torch.where(bad, (ch_in + 1) % HEAD, ch_in)
        # Start within the page, 0..224, never a multiple of the chunk.
        st = torch.randint(0, PAGE - CHUNK + 1 - (PAGE // CHUNK), (nb,),
                           generator=g, device=device).cpu()
        st = st + st // (CHUNK - 1) + 1  # skip multiples of 32
        page_of = torch.arange(nb) // heads
        rows = (page_of * PAGE + st)[:, None] + torch.arange(CHUNK)[None, :]
        cols = ch[:, None].expand(-1, CHUNK)
        rows, cols = rows.reshape(-1).to(device), cols.reshape(-1).to(device)
        x[rows, cols] *= 20.0
    xb = x.to(torch.bfloat16)
    if out is not None:
        out.copy_(xb)
        return out
    return xb


@dataclass
class KVConfig:
    """Shape and generator recipe of one workload."""
    name: str
    layers: int
    num_tokens: int
    num_channels: int
    seed_base: int
    outlier_count: int = 0          # 1%-of-channels set shared by all layers
    outlier_per_head: int = 0       # or per-head outliers
    outlier_seed: int = 0

    @property
    def num_tensors(self) -> int:
        return 2 * self.layers

    @property
    def num_elements(self) -> int:
        return self.num_tensors * self.num_tokens * self.num_channels

    def outliers(self) -> list[int]:
        if self.outlier_per_head:
            return outlier_channels_per_head(self.num_channels,
                                             self.outlier_per_head,
                                             self.outlier_seed)
        if self.outlier_count:
            return outlier_channels(self.num_channels, self.outlier_count,
                                    self.outlier_seed)
        return []

    def seed(self, tensor: int) -> int:
        """Seed of tensor index 2*layer + kv (kv = 0 for K, 1 for V)."""
        return self.seed_base + tensor

    def tensor(self, tensor: int, device="cpu", out=None) -> torch.Tensor:
        return kv_tensor(self.seed(tensor), self.num_tokens,
                         self.num_channels, self.outliers(), True, device, out)

    def make(self, device="cpu", tensors: list[int] | None = None) -> torch.Tensor:
        """[n, T, Ch] bf16 for the listed tensor indices (default: all)."""
        idx = list(range(self.num_tensors)) if tensors is None else tensors
        out = torch.empty((len(idx), self.num_tokens, self.num_channels),
                          dtype=torch.bfloat16, device=device)
        for i, t in enumerate(idx):
            self.tensor(t, device, out[i])
        return out


# The workloads: a single page (K and V), a Qwen-32B-shaped KV set at 16K
# context (64 layers, 8 KV heads of 128), a Qwen3-235B-A22B-shaped KV set at
# 128K context (94 layers, 4 KV heads of 128), and the KV of the two
# attention workloads.
CONFIGS = {
    "single_page": KVConfig("single_page", 1, 256, 128, 1,
                            outlier_per_head=3, outlier_seed=11),
    "qwen32b_16k": KVConfig("qwen32b_16k", 64, 16384, 1024, 1000,
                            outlier_count=10, outlier_seed=1001),
    "qwen3_235b_128k": KVConfig("qwen3_235b_128k", 94, 131072, 512, 2000,
                                outlier_count=5, outlier_seed=2001),
    "decode_attn_32k": KVConfig("decode_attn_32k", 1, 32768, 1024, 3100,
                                outlier_per_head=3, outlier_seed=3001),
    "decode_attn_32k_plain": KVConfig("decode_attn_32k_plain", 1, 32768, 1024,
                                      3200),
    "verify_attn_128k": KVConfig("verify_attn_128k", 1, 131072, 512, 4100,
                                 outlier_count=5, outlier_seed=4001),
}


def queries(seed: int, t_q: int, num_q_heads: int, head_dim: int = HEAD,
            device="cpu") -> torch.Tensor:
    """q ~ N(0, 1) as bf16, shape [t_q][num_q_heads][head_dim]."""
    g = _gen(seed, device)
    return torch.randn((t_q, num_q_heads, head_dim), generator=g,
                       device=device).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor):
    """Host numpy uint16 view of a bf16 tensor's bits."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view("uint16")


def _bf16_from_f32(a) -> torch.Tensor:
    return torch.as_tensor(a, dtype=torch.float32).to(torch.bfloat16)


def edge_pages(seed: int = 7) -> dict[str, torch.Tensor]:
    """Adversarial single page blocks [256][128] bf16 (host tensors).

    constant_channels : every channel constant (codes all 0);
    constant_chunks   : every 32-token chunk constant, channels still vary;
    spike             : Laplacian page with one huge element;
    two_valued        : every chunk holds two values, 16 of each;
    signed_zeros      : +0 / -0 mixed with a few small values;
    subnormals        : bf16 subnormal magnitudes (~1e-39);
    huge_range        : 1e30 and 1e-30 in the same channel;
    large_same_sign   : magnitudes up to 1e38, all positive;
    all_negative      : strictly negative Laplacian page;
    zeros             : all +0;
    mixed_sign_zeros  : every value +0 or -0: channels whose first token is
                        -0 and the rest +0, all -0 channels, channels with
                        whole -0 chunks among +0 chunks, and channels with
                        scattered -0 plus one small positive value.
    """
    g = torch.Generator()
    g.manual_seed(int(seed))
    P, H = PAGE, HEAD
    lap = torch.empty((P, H)).exponential_(1.0, generator=g)
    lap = torch.where(torch.rand((P, H), generator=g) < 0.5, -lap, lap)
    out = {}
    out["constant_channels"] = _bf16_from_f32(
        (torch.randn(H, generator=g) * 3.0)[None, :].expand(P, H).clone())
    cc = torch.randn((P // CHUNK, H), generator=g) * 2.0
    out["constant_chunks"] = _bf16_from_f32(cc.repeat_interleave(CHUNK, 0))
    sp = lap.clone()
    sp[77, 5] = 5.0e4
    sp[200, 100] = -3.0e3
    out["spike"] = _bf16_from_f32(sp)
    t = torch.arange(P)[:, None]
    c = torch.arange(H)[None, :]
    bit = (t >> (c % 5)) & 1
    out["two_valued"] = _bf16_from_f32(torch.where(bit == 1, 1.5 + 0.01 * c,
                                                   -0.75 - 0.02 * c))
    z = torch.zeros((P, H))
    z[torch.rand((P, H), generator=g) < 0.5] = -0.0
    few = torch.rand((P, H), generator=g) < 0.05
    z = torch.where(few, lap * 1e-3, z)
    out["signed_zeros"] = _bf16_from_f32(z)
    out["subnormals"] = _bf16_from_f32(lap * 1e-39)
    hr = torch.where(torch.rand((P, H), generator=g) < 0.5,
                     torch.full((P, H), 1e30), torch.full((P, H), 1e-30))
    out["huge_range"] = _bf16_from_f32(hr * torch.sign(lap))
    out["large_same_sign"] = _bf16_from_f32(lap.abs() * 2.0e37 + 1.0e30)
    out["all_negative"] = _bf16_from_f32(-(lap.abs() + 0.01))
    out["zeros"] = _bf16_from_f32(torch.zeros((P, H)))
    mz = torch.zeros((P, H))
    mz[0, 0:32] = -0.0
    mz[:, 32:64] = -0.0
    chunk_odd = ((torch.arange(P) // CHUNK) % 2 == 1)[:, None]
    mz[:, 64:96] = torch.where(chunk_odd, torch.tensor(-0.0), torch.tensor(0.0))
    mz[:, 96:128] = torch.where(torch.rand((P, 32), generator=g) < 0.5,
                                torch.tensor(-0.0), torch.tensor(0.0))
    mz[100, 96:128] = 2.0e-3
    out["mixed_sign_zeros"] = _bf16_from_f32(mz)
    return out


def verify_inputs(seed: int, t_draft: int, vocab: int, noise: float = 0.3,
                  logit_scale: float = 2.5):
    """Synthetic inputs of one speculative verification (host tensors):
    target logits [t_draft + 1][vocab] ~ N(0, logit_scale^2), draft logits =
    the first t_draft target rows + N(0, noise^2) (the draft model's
    approximation), draft tokens drawn from softmax(draft rows), uniforms
    u_accept [t_draft] and u_sample (float64)."""
    g = torch.Generator().manual_seed(seed)
    target = torch.randn((t_draft + 1, vocab), generator=g) * logit_scale
    draft = target[:t_draft] + torch.randn((t_draft, vocab), generator=g) * noise
    if t_draft:
        tokens = torch.multinomial(torch.softmax(draft.double(), dim=1), 1,
                                   generator=g)[:, 0].to(torch.int32)
    else:
        tokens = torch.zeros(0, dtype=torch.int32)
    u_accept = torch.rand(t_draft, dtype=torch.float64, generator=g)
    u_sample = float(torch.rand(1, dtype=torch.float64, generator=g))
    return draft.contiguous(), target.contiguous(), tokens, u_accept, u_sample


# Speculative verification workload: 8 drafts over a Qwen3-sized vocabulary.
VERIFY_T, VERIFY_VOCAB = 8, 151936

"""GPU parity of the speculative verification (lynx_spec_verify) with the
oracle: the accepted count and the next token must be equal.  Both sides
take the decisions in binary64; a case whose acceptance ratio or inverse-CDF
target lies within 1e-12 (relative) of a threshold would be reported, and
the seeds used here have none."""
import numpy as np
import pytest
import torch

import oracle
from progressive_kv_transfer_amd import kvgen, lynx

pytestmark = pytest.mark.gpu
DEV = "cuda"


def announce(msg):
    print(f"[gpu-verify] {msg}", flush=True)


def run_gpu(draft, target, tokens, u, us):
    out = lynx.spec_verify(draft.to(DEV), target.to(DEV), tokens.to(DEV), u.to(DEV), us)
    torch.cuda.synchronize()
    k, tok = out.cpu().tolist()
    return k, tok


def run_oracle(draft, target, tokens, u, us):
    return oracle.spec_verify(draft.numpy(), target.numpy(), tokens.numpy(), u.numpy(), us)


CASES = [(t, v, noise) for t in (0, 1, 3, 8) for v in (1, 7, 2048, 2049, 50000)
         for noise in (0.0, 0.3, 2.0)] + [(64, 1000, 0.5), (8, kvgen.VERIFY_VOCAB, 0.3),
                                          (8, kvgen.VERIFY_VOCAB, 1.5), (3, 8192, 0.3),
                                          (5, 600000, 0.5)]


@pytest.mark.parametrize("t_draft,vocab,noise", CASES)
def test_verify_matches_oracle(t_draft, vocab, noise):
    announce(f"T={t_draft} V={vocab} noise={noise}")
    for seed in range(3):
        inp = kvgen.verify_inputs(9000 + 31 * seed + t_draft, t_draft, vocab, noise)
        g = run_gpu(*inp)
        o = run_oracle(*inp)
        assert g == o, (seed, g, o)
        if noise == 0.0:
            assert g[0] == t_draft  # identical distributions accept every draft


def test_verify_acceptance_rate_tracks_the_approximation():
    """Over many seeds, closer drafts are accepted more often (sanity of the
    whole path at the Qwen-sized vocabulary)."""
    rates = []
    for noise in (0.1, 1.0):
        acc = 0
        for seed in range(20):
            acc += run_gpu(*kvgen.verify_inputs(9500 + seed, 8, kvgen.VERIFY_VOCAB, noise))[0]
        rates.append(acc / (20 * 8))
    announce(f"acceptance rate noise 0.1: {rates[0]:.3f}, noise 1.0: {rates[1]:.3f}")
    assert rates[0] > rates[1]


def test_invalid_draft_token_is_rejected():
    draft, target, tokens, u, us = kvgen.verify_inputs(9600, 4, 300, 0.0)
    tokens[2] = 300  # out of range: rejected at position 2 without a read
    k, tok = run_gpu(draft, target, tokens, u, us)
    assert k == 2
    # the correction at position 2 draws from max(0, p - q) of identical
    # draft and target rows (noise 0): no token carries weight, and the
    # library's contract for a correction without mass is token -1
    assert torch.equal(draft[2], target[2])
    assert tok == -1

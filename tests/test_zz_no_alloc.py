"""The allocation-free decode entry point (tg_decode_attention_noalloc): its
split-KV partials live in the library's static per-device scratch. Through the
C ABI, two calls in a row (the second smaller, so it runs over the first
call's leftover scratch) must equal tg_decode_attention with a caller
workspace (same kernels, same split plan: bit for bit, which is inside the
bf16 bar of the decode parity tests)."""

import numpy as np
import pytest
import torch

import learned_token_pruning_layer_amd as tg
from synthetic import make_attention_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(segs, hq, hkv, d, seed):
    rows = max(st + ln for st, ln, _ in segs)
    a = make_attention_inputs([rows], hq, hkv, d, seed=seed, dtype=torch.bfloat16)
    r = sum(nn for _, _, nn in segs)
    q = torch.randn((r, hq, d), generator=torch.Generator().manual_seed(seed + 1)).to(torch.bfloat16)
    return [t.to(DEV) for t in (q, a["k"], a["v"], a["bias"], a["pos"], a["gain"])]


def test_noalloc_decode_matches_workspace_entry_point_twice():
    print("[case] decode without allocation: a large call, then a smaller one, against tg_decode_attention",
          flush=True)
    cases = [([(0, 9152, 1), (9152, 5000, 2), (14152, 700, 3)], 16, 8, 128, 21),
             ([(0, 300, 1), (300, 41, 2)], 16, 8, 128, 22)]
    for segs, hq, hkv, d, seed in cases:
        q, k, v, bias, pos, gain = _inputs(segs, hq, hkv, d, seed)
        want, want_lse = tg.tg_decode_attention(q, k, v, bias, pos, segs, gain, 1.2, want_lse=True)
        out = torch.full_like(want, float("nan"))
        lse = torch.full_like(want_lse, float("nan"))
        got, got_lse = tg.tg_decode_attention_noalloc(q, k, v, bias, pos, segs, gain, 1.2, out=out, want_lse=True,
                                                      lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(got, want) and torch.equal(got_lse, want_lse)
        diff = (got.float() - want.float()).abs().max(dim=-1).values
        scale = want.float().abs().max(dim=-1).values
        assert bool((diff <= 2e-2 * scale).all())

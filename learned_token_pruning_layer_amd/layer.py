"""One gated-prefill layer as four C-ABI calls on one stream.

gate score -> top-K select -> compaction -> token-gated attention (one
attention call per above-gate layer that shares the kept set). Every buffer
is allocated once, up front, so a step enqueues exactly the four kernels
(plus one attention launch per extra layer) and never synchronises.
"""

from __future__ import annotations

from typing import List, Optional, Sequence

import torch

from ._lib import tg_compact, tg_gate_score, tg_gated_attention, tg_kept_rows, tg_select_topk


class GatedPrefillLayer:
    """Preallocated pruned-prefill layer.

    x [N, d] residual at the gate layer; w1 [H, d], w2 [H] (b1 [H] optional)
    gate weights; prompts: packed prompt descriptors; layers: objects with
    q [N, hq*D], k/v [N, hkv*D], gain [hq] fp32 and tau (one per above-gate
    layer sharing this kept set); pos [N] int32 or None (row - start).
    """

    def __init__(self, x: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, prompts: Sequence,
                 layers: Sequence, hq: int, hkv: int, head_dim: int, b1: Optional[torch.Tensor] = None,
                 b2: float = 0.0, pos: Optional[torch.Tensor] = None, gather_hidden: bool = True,
                 want_lse: bool = False):
        self.x, self.w1, self.w2, self.b1, self.b2 = x, w1, w2, b1, float(b2)
        self.prompts = list(prompts)
        self.layers = list(layers)
        self.hq, self.hkv, self.head_dim = hq, hkv, head_dim
        self.pos = pos
        self.want_lse = want_lse
        dev = x.device
        n = x.shape[0]
        self.m = tg_kept_rows(self.prompts)
        m = self.m
        self.scores = torch.empty(n, dtype=torch.float32, device=dev)
        self.kept = torch.empty(m, dtype=torch.int32, device=dev)
        self.pos_kept = torch.empty(m, dtype=torch.int32, device=dev)
        self.bias_kept = torch.empty(m, dtype=torch.float32, device=dev)
        srcs: List[torch.Tensor] = []
        self.hidden_kept = None
        if gather_hidden:
            self.hidden_kept = torch.empty((m, x.shape[1]), dtype=x.dtype, device=dev)
            srcs.append(x)
        self.qkv_kept = []
        self.outs = []
        self.lses = []
        for lay in self.layers:
            qk = torch.empty((m, hq * head_dim), dtype=lay.q.dtype, device=dev)
            kk = torch.empty((m, hkv * head_dim), dtype=lay.k.dtype, device=dev)
            vk = torch.empty((m, hkv * head_dim), dtype=lay.v.dtype, device=dev)
            self.qkv_kept.append((qk, kk, vk))
            srcs += [lay.q, lay.k, lay.v]
            self.outs.append(torch.empty((m, hq, head_dim), dtype=lay.q.dtype, device=dev))
            self.lses.append(torch.empty((hq, m), dtype=torch.float32, device=dev) if want_lse else None)
        self.srcs = srcs
        self.dsts = ([self.hidden_kept] if gather_hidden else []) + [t for trip in self.qkv_kept for t in trip]

    # The four steps, individually callable (the bench times each).
    def gate(self, stream=None):
        tg_gate_score(self.x, self.w1, self.w2, self.b1, self.b2, scores=self.scores, stream=stream)

    def select(self, stream=None):
        tg_select_topk(self.scores, self.prompts, kept_idx=self.kept, stream=stream)

    def compact(self, stream=None):
        tg_compact(self.kept, self.prompts, self.srcs, pos=self.pos, scores=self.scores, outs=self.dsts,
                   pos_kept=self.pos_kept, bias_kept=self.bias_kept, stream=stream)

    def attention(self, i: int = 0, stream=None):
        lay = self.layers[i]
        qk, kk, vk = self.qkv_kept[i]
        m, hq, hkv, dh = self.m, self.hq, self.hkv, self.head_dim
        tg_gated_attention(qk.view(m, hq, dh), kk.view(m, hkv, dh), vk.view(m, hkv, dh), self.bias_kept,
                           self.pos_kept, self.prompts, lay.gain, lay.tau, out=self.outs[i],
                           want_lse=self.want_lse, lse=self.lses[i], stream=stream)

    def run(self, stream=None):
        """One whole step: all four steps, every layer's attention."""
        self.gate(stream)
        self.select(stream)
        self.compact(stream)
        for i in range(len(self.layers)):
            self.attention(i, stream)

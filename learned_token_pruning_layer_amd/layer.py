"""One gated-prefill layer as four C-ABI calls on one stream.

gate score -> top-K select -> compaction -> token-gated attention (one
attention call per above-gate layer that shares the kept set). Every buffer
is allocated once, up front, so a step enqueues exactly the four kernels
(plus one attention launch per extra layer) and never synchronises.
"""

from __future__ import annotations

from typing import List, Optional, Sequence

import torch

import ctypes
import math

from ._lib import TG_BF16, TG_F32, TgGather, _check, load, seq_array, tg_kept_rows


def _dense_rows(t: torch.Tensor) -> bool:
    """Each row (index over dim 0) is one dense block: the inner dimensions
    are laid out contiguously; the row stride itself may be larger."""
    exp = 1
    for size, stride in zip(reversed(t.shape[1:]), reversed(t.stride()[1:])):
        if size != 1 and stride != exp:
            return False
        exp *= size
    return t.stride(0) >= exp or t.shape[0] <= 1


def _validate(x, w1, w2, b1, layers, hq, hkv, head_dim, pos):
    if not x.is_cuda or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [N, d] GPU tensor")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"x: unsupported dtype {x.dtype}")
    n, d = x.shape
    dev = x.device
    for t, nm in ((w1, "w1"), (w2, "w2")) + (((b1, "b1"),) if b1 is not None else ()):
        if t.device != dev or t.dtype != x.dtype or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous tensor of x's dtype on x's device")
    h = w1.shape[0]
    if tuple(w1.shape) != (h, d) or w2.numel() != h or (b1 is not None and b1.numel() != h):
        raise ValueError("w1 must be [H, d], w2 and b1 [H]")
    if hq <= 0 or hkv <= 0 or hq % hkv:
        raise ValueError("hq must be a positive multiple of hkv")
    for li, lay in enumerate(layers):
        for nm, heads in (("q", hq), ("k", hkv), ("v", hkv)):
            t = getattr(lay, nm)
            if t.device != dev or t.dtype != x.dtype:
                raise ValueError(f"layer {li} {nm}: must be on x's device with x's dtype")
            if t.dim() < 2 or t.shape[0] != n or math.prod(t.shape[1:]) != heads * head_dim:
                raise ValueError(f"layer {li} {nm}: expected {n} rows of {heads}x{head_dim}, got {tuple(t.shape)}")
            if not _dense_rows(t):
                raise ValueError(f"layer {li} {nm}: each row must be dense (inner dimensions contiguous)")
        g = lay.gain
        if g.device != dev or g.dtype != torch.float32 or g.numel() != hq or not g.is_contiguous():
            raise ValueError(f"layer {li} gain: must be a contiguous fp32 [hq] tensor on x's device")
    if pos is not None and (pos.device != dev or pos.dtype != torch.int32 or pos.numel() != n
                            or not pos.is_contiguous()):
        raise ValueError("pos must be a contiguous int32 [N] tensor on x's device")


class GatedPrefillLayer:
    """Preallocated pruned-prefill layer.

    x [N, d] residual at the gate layer (contiguous); w1 [H, d], w2 [H]
    (b1 [H] optional) gate weights of x's dtype; prompts: packed prompt
    descriptors; layers: objects with q [N, hq*D], k/v [N, hkv*D] (or
    [N, heads, D]), gain [hq] fp32 and tau (one per above-gate layer sharing
    this kept set); pos [N] int32 or None (row - start). A layer tensor may
    be a row-strided view (q, k, v sliced from one fused projection): its
    rows are gathered with its own row stride, as long as each row is dense.
    Every tensor is checked here (device, dtype, shape, layout), so a step
    cannot gather from a wrongly laid out buffer.
    """

    def __init__(self, x: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, prompts: Sequence,
                 layers: Sequence, hq: int, hkv: int, head_dim: int, b1: Optional[torch.Tensor] = None,
                 b2: float = 0.0, pos: Optional[torch.Tensor] = None, gather_hidden: bool = True,
                 want_lse: bool = False):
        _validate(x, w1, w2, b1, layers, hq, hkv, head_dim, pos)
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
        self._prepare()

    def _prepare(self):
        """Marshal every C-ABI argument once, so a step is four plain calls."""
        lib = self._lib = load()
        dt = TG_F32 if self.x.dtype == torch.float32 else TG_BF16
        n, d = self.x.shape
        h = self.w1.shape[0]
        self._seqs = seq_array(self.prompts)
        ns = len(self.prompts)
        self._gate_args = (dt, self.x.data_ptr(), n, d, self.w1.data_ptr(),
                           None if self.b1 is None else self.b1.data_ptr(), h, self.w2.data_ptr(),
                           ctypes.c_float(self.b2), self.scores.data_ptr())
        sel_ws = lib.tg_select_workspace_bytes(self._seqs, ns)
        self.sel_ws = (torch.empty(sel_ws, dtype=torch.uint8, device=self.x.device) if sel_ws else None)
        self._sel_args = (self.scores.data_ptr(), self._seqs, ns, self.kept.data_ptr(),
                          None if self.sel_ws is None else self.sel_ws.data_ptr(), sel_ws)
        garr = (TgGather * max(1, len(self.srcs)))()
        for i, (src, dst) in enumerate(zip(self.srcs, self.dsts)):
            rb = int(math.prod(src.shape[1:])) * src.element_size()
            garr[i] = TgGather(src.data_ptr(), dst.data_ptr(), rb, src.stride(0) * src.element_size(), rb)
        self._garr = garr
        self._comp_args = (self.kept.data_ptr(), self.m, self._seqs, ns, garr, len(self.srcs),
                           None if self.pos is None else self.pos.data_ptr(), self.pos_kept.data_ptr(),
                           self.scores.data_ptr(), self.bias_kept.data_ptr())
        self._attn_args = []
        for i, lay in enumerate(self.layers):
            qk, kk, vk = self.qkv_kept[i]
            lse = self.lses[i]
            self._attn_args.append((dt, qk.data_ptr(), kk.data_ptr(), vk.data_ptr(), self.bias_kept.data_ptr(),
                                    self.pos_kept.data_ptr(), self._seqs, ns, self.hq, self.hkv, self.head_dim,
                                    lay.gain.data_ptr(), ctypes.c_float(lay.tau), self.outs[i].data_ptr(),
                                    None if lse is None else lse.data_ptr()))

    @staticmethod
    def _stream(stream):
        if stream is None:
            return torch.cuda.current_stream().cuda_stream
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)

    # The four steps, individually callable (the bench times each).
    def gate(self, stream=None):
        _check(self._lib.tg_gate_score(*self._gate_args, self._stream(stream)))

    def select(self, stream=None):
        _check(self._lib.tg_select_topk(*self._sel_args, self._stream(stream)))

    def compact(self, stream=None):
        _check(self._lib.tg_compact(*self._comp_args, self._stream(stream)))

    def attention(self, i: int = 0, stream=None):
        _check(self._lib.tg_gated_attention(*self._attn_args[i], self._stream(stream)))

    def run(self, stream=None):
        """One whole step: all four steps, every layer's attention."""
        st = self._stream(stream)
        lib = self._lib
        _check(lib.tg_gate_score(*self._gate_args, st))
        _check(lib.tg_select_topk(*self._sel_args, st))
        _check(lib.tg_compact(*self._comp_args, st))
        for args in self._attn_args:
            _check(lib.tg_gated_attention(*args, st))

"""Seeded synthetic inputs for the TokenGate pruned-prefill layer.

This module only draws inputs. It holds none of the method's arithmetic
(no gate, no selection, no compaction, no attention): the HIP path and the
fp64 oracle both consume what it returns, so neither imports the other.

Workloads (shapes follow the configurations the layer is measured on):

  tiny      N=512 (448 doc + 64 query), d=256, gate 256->64->1, fp32,
            4 Q heads / 2 KV heads, head_dim 64, keep 112 doc rows.
  qwen16k   N=16384 (16000 doc + 384 query), d=2048, gate 2048->256->1,
            16 Q / 8 KV heads, head_dim 128, bf16, keep 2000 doc rows,
            16 planted rows.
  sweep32k  N=32768 (32256 doc + 512 query), same shapes, budgets of
            {5,10,25,50,100}% of the document.
  long128k  N=131072 (130048 doc + 1024 query), keep 8128 (6.25%),
            one planted row per 8192 doc rows.
  ragged    8 prompts, lengths uniform in [4096, 65536], 256-row query
            tail each, per-prompt budgets uniform in [10%, 40%], 4 stacked
            above-gate layers sharing one kept set.

Recipe (also stated in the design notes): the residual x is N(0,1); gate
weights are N(0, 1/fan_in); planted rows get 4*sqrt(d)*u added, with u a
random unit vector that is also the gate's first hidden row (and that
hidden unit's output weight is +1/sqrt(H)), so that planted rows score far
above the rest; Q/K/V are projections of the (rounded) residual by
N(0, 1/d) weights; per-head gains are U(0.5, 2); tau = 1.2.

Structural draws (lengths, budgets, planted rows) use NumPy's PCG64 seeded
by the workload; bulk tensors use a torch generator on the target device
seeded from the same seed, so every input is reproducible on its device.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, NamedTuple, Optional

import numpy as np
import torch


class Prompt(NamedTuple):
    """One packed prompt: rows [start, start+length) of the packed input.

    The prunable document span is rows [start+doc_begin, start+doc_end);
    every other row of the prompt (the query tail) is always kept.
    k_doc is the number of document rows to keep.
    """

    start: int
    length: int
    doc_begin: int
    doc_end: int
    k_doc: int

    @property
    def n_doc(self) -> int:
        return self.doc_end - self.doc_begin

    @property
    def n_kept(self) -> int:
        return self.k_doc + (self.length - self.n_doc)


def doc_budget(frac: float, n_doc: int) -> int:
    """Number of document rows kept at fraction `frac` of the document
    (floor of the product, clamped to [0, n_doc])."""
    return max(0, min(n_doc, int(math.floor(frac * n_doc + 1e-9))))


WORKLOADS = {
    "tiny": dict(n=512, n_query=64, d=256, h=64, hq=4, hkv=2, head_dim=64,
                 k_doc=112, dtype=torch.float32, planted_every=None, n_planted=0),
    "qwen16k": dict(n=16384, n_query=384, d=2048, h=256, hq=16, hkv=8, head_dim=128,
                    k_doc=2000, dtype=torch.bfloat16, planted_every=None, n_planted=16),
    "sweep32k": dict(n=32768, n_query=512, d=2048, h=256, hq=16, hkv=8, head_dim=128,
                     k_doc=None, dtype=torch.bfloat16, planted_every=None, n_planted=16),
    "long128k": dict(n=131072, n_query=1024, d=2048, h=256, hq=16, hkv=8, head_dim=128,
                     k_doc=8128, dtype=torch.bfloat16, planted_every=8192, n_planted=None),
}
SWEEP_FRACTIONS = (0.05, 0.10, 0.25, 0.50, 1.00)
TAU = 1.2


@dataclass
class Layer:
    """Inputs of one above-gate attention layer: full-length Q/K/V rows
    (row-major [N, heads*head_dim]) and the per-head gains."""

    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    gain: torch.Tensor  # [hq] fp32
    tau: float = TAU


@dataclass
class LayerInputs:
    name: str
    prompts: List[Prompt]
    x: torch.Tensor          # [N, d] residual at the gate layer
    w1: torch.Tensor         # [H, d] (nn.Linear layout)
    w2: torch.Tensor         # [H]
    b1: Optional[torch.Tensor]
    b2: float
    layers: List[Layer]
    hq: int
    hkv: int
    head_dim: int
    planted: np.ndarray      # absolute row ids of planted rows
    pos: Optional[torch.Tensor] = None   # [N] int32 original positions, None = row - start
    meta: dict = field(default_factory=dict)

    @property
    def n_rows(self) -> int:
        return int(self.x.shape[0])


def _torch_gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, std, gen, device, dtype=torch.float32):
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def _uniform(shape, lo, hi, gen, device):
    t = torch.rand(shape, generator=gen, device=device, dtype=torch.float32)
    return t.mul_(hi - lo).add_(lo)


def _planted_rows(rng: np.random.Generator, prompts: List[Prompt], n_planted_fixed, every):
    rows = []
    for p in prompts:
        n_doc = p.n_doc
        if n_planted_fixed is not None:
            cnt = n_planted_fixed
        elif every is not None:
            cnt = max(1, int(round(n_doc / every)))
        else:
            cnt = 0
        cnt = min(cnt, n_doc)
        if cnt:
            sel = rng.choice(n_doc, size=cnt, replace=False)
            rows.extend(int(p.start + p.doc_begin + r) for r in np.sort(sel))
    return np.asarray(rows, dtype=np.int64)


def _make_weights_and_x(rng, gen, device, n, d, h, dtype, planted):
    # Residual stream x ~ N(0, 1).
    x = _normal((n, d), 1.0, gen, device)
    # Gate weights N(0, 1/fan_in); biases are absent (zero).
    w1 = _normal((h, d), 1.0 / math.sqrt(d), gen, device)
    w2 = _normal((h,), 1.0 / math.sqrt(h), gen, device)
    if len(planted):
        u = torch.randn((d,), generator=gen, device=device, dtype=torch.float32)
        u = u / torch.linalg.vector_norm(u)
        idx = torch.as_tensor(planted, device=device)
        x[idx] += (4.0 * math.sqrt(d)) * u
        w1[0] = u
        w2[0] = 1.0 / math.sqrt(h)
    return x.to(dtype), w1.to(dtype), w2.to(dtype)


def _make_layer(gen, device, x_rounded, d, hq, hkv, head_dim, dtype):
    """Project the (rounded) residual into Q/K/V with N(0, 1/d) weights.
    Plain model code that produces attention inputs; done in fp32 and
    rounded once to the storage type."""
    xf = x_rounded.to(torch.float32)
    std = 1.0 / math.sqrt(d)
    outs = []
    for heads in (hq, hkv, hkv):
        w = _normal((heads * head_dim, d), std, gen, device)
        outs.append((xf @ w.t()).to(dtype).contiguous())
        del w
    gain = _uniform((hq,), 0.5, 2.0, gen, device)
    return Layer(q=outs[0], k=outs[1], v=outs[2], gain=gain, tau=TAU)


def single_prompt(n: int, n_query: int, k_doc: int) -> List[Prompt]:
    return [Prompt(0, n, 0, n - n_query, k_doc)]


def make_workload(name: str, device="cpu", seed: Optional[int] = None,
                  k_doc: Optional[int] = None, with_layers: bool = True,
                  n_layers: int = 1) -> LayerInputs:
    """Build the named workload on `device`.

    `k_doc` overrides the document budget (the sweep uses this); the
    default budget is the workload's own (sweep32k defaults to 25%).
    """
    if name == "ragged":
        return make_ragged(device=device, seed=seed, with_layers=with_layers)
    cfg = WORKLOADS[name]
    seed = {"tiny": 0, "qwen16k": 1, "sweep32k": 2, "long128k": 3}[name] if seed is None else seed
    n, nq = cfg["n"], cfg["n_query"]
    n_doc = n - nq
    if k_doc is None:
        k_doc = cfg["k_doc"] if cfg["k_doc"] is not None else doc_budget(0.25, n_doc)
    prompts = single_prompt(n, nq, k_doc)
    rng = np.random.Generator(np.random.PCG64(seed))
    gen = _torch_gen(device, seed)
    planted = _planted_rows(rng, prompts, cfg["n_planted"], cfg["planted_every"])
    x, w1, w2 = _make_weights_and_x(rng, gen, device, n, cfg["d"], cfg["h"], cfg["dtype"], planted)
    layers = []
    if with_layers:
        for _ in range(n_layers):
            layers.append(_make_layer(gen, device, x, cfg["d"], cfg["hq"], cfg["hkv"],
                                      cfg["head_dim"], cfg["dtype"]))
    return LayerInputs(name=name, prompts=prompts, x=x, w1=w1, w2=w2, b1=None, b2=0.0,
                       layers=layers, hq=cfg["hq"], hkv=cfg["hkv"], head_dim=cfg["head_dim"],
                       planted=planted, meta=dict(seed=seed, d=cfg["d"], h=cfg["h"]))


def ragged_prompts(seed: int = 4, n_prompts: int = 8, lo: int = 4096, hi: int = 65536,
                   n_query: int = 256, frac_lo: float = 0.10, frac_hi: float = 0.40) -> List[Prompt]:
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(lo, hi, size=n_prompts, endpoint=True)
    fracs = rng.uniform(frac_lo, frac_hi, size=n_prompts)
    prompts, start = [], 0
    for ln, fr in zip(lens.tolist(), fracs.tolist()):
        n_doc = ln - n_query
        prompts.append(Prompt(start, ln, 0, n_doc, doc_budget(fr, n_doc)))
        start += ln
    return prompts


def make_ragged(device="cpu", seed: Optional[int] = None, with_layers: bool = True,
                n_layers: int = 4, prompts: Optional[List[Prompt]] = None) -> LayerInputs:
    """8 packed prompts feeding `n_layers` stacked above-gate layers with
    qwen16k shapes; one gate and one select cover all prompts."""
    seed = 4 if seed is None else seed
    prompts = ragged_prompts(seed) if prompts is None else prompts
    n = prompts[-1].start + prompts[-1].length
    d, h, hq, hkv, hd = 2048, 256, 16, 8, 128
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    gen = _torch_gen(device, seed)
    planted = _planted_rows(rng, prompts, None, 8192)
    x, w1, w2 = _make_weights_and_x(rng, gen, device, n, d, h, torch.bfloat16, planted)
    layers = []
    if with_layers:
        for _ in range(n_layers):
            layers.append(_make_layer(gen, device, x, d, hq, hkv, hd, torch.bfloat16))
    return LayerInputs(name="ragged", prompts=prompts, x=x, w1=w1, w2=w2, b1=None, b2=0.0,
                       layers=layers, hq=hq, hkv=hkv, head_dim=hd, planted=planted,
                       meta=dict(seed=seed, d=d, h=h))


# ---------------------------------------------------------------------------
# Stage-level inputs: each stage can be fed identical synthetic inputs on
# both sides, independent of the previous stage's output.
# ---------------------------------------------------------------------------

def make_scores(n: int, seed: int, kind: str = "normal", device="cpu") -> torch.Tensor:
    """fp32 gate-score-like vectors.

    kind: "normal"  N(0,1)
          "ties"    N(0,1) quantised to multiples of 1/8 (many exact ties)
          "few"     values from {-1, 0, 1} (massive ties)
          "signed0" half +0.0, half -0.0 and a few ones (sign-of-zero ties)
          "wide"    N(0,1) * 10**U(-30, 30) (spans the exponent range)
    """
    gen = _torch_gen("cpu", seed)
    if kind == "normal":
        s = torch.randn(n, generator=gen)
    elif kind == "ties":
        s = torch.round(torch.randn(n, generator=gen) * 8) / 8
    elif kind == "few":
        s = torch.randint(-1, 2, (n,), generator=gen).to(torch.float32)
    elif kind == "signed0":
        s = torch.zeros(n)
        neg = torch.rand(n, generator=gen) < 0.5
        s[neg] = -0.0
        ones = torch.rand(n, generator=gen) < 0.05
        s[ones] = 1.0
    elif kind == "wide":
        e = torch.rand(n, generator=gen, dtype=torch.float64) * 60 - 30
        s = (torch.randn(n, generator=gen, dtype=torch.float64) * torch.pow(10.0, e)).to(torch.float32)
    else:
        raise ValueError(kind)
    return s.to(torch.float32).to(device)


def make_attention_inputs(seg_lens: List[int], hq: int, hkv: int, head_dim: int, seed: int,
                          dtype=torch.bfloat16, device="cpu", n_query_tail: int = 0,
                          pos_ties: bool = False, qk_std: float = 1.0) -> dict:
    """Kept-row attention inputs for packed segments of the given lengths.

    Q/K/V ~ N(0, qk_std^2) rounded to `dtype`; bias is a non-positive
    log-weight drawn as -|N(0, 1.5^2)| for document rows and exactly 0 for
    the last `n_query_tail` rows of each segment; positions are strictly
    increasing within a segment (random gaps), or non-decreasing with
    repeats when pos_ties is set; gains are U(0.5, 2); tau = 1.2.
    """
    m = int(sum(seg_lens))
    gen = _torch_gen("cpu", seed)
    q = (torch.randn((m, hq, head_dim), generator=gen) * qk_std).to(dtype)
    k = (torch.randn((m, hkv, head_dim), generator=gen) * qk_std).to(dtype)
    v = torch.randn((m, hkv, head_dim), generator=gen).to(dtype)
    bias = -(torch.randn((m,), generator=gen) * 1.5).abs()
    pos = torch.empty((m,), dtype=torch.int32)
    off = 0
    for ln in seg_lens:
        if ln:
            if pos_ties:
                gaps = torch.randint(0, 2, (ln,), generator=gen)
            else:
                gaps = torch.randint(1, 9, (ln,), generator=gen)
            gaps[0] = torch.randint(0, 5, (1,), generator=gen)[0]
            pos[off:off + ln] = torch.cumsum(gaps, 0).to(torch.int32)
            tail = min(n_query_tail, ln)
            if tail:
                bias[off + ln - tail: off + ln] = 0.0
        off += ln
    gain = torch.rand((hq,), generator=gen) * 1.5 + 0.5
    return dict(q=q.to(device), k=k.to(device), v=v.to(device), bias=bias.to(device),
                pos=pos.to(device), gain=gain.to(device), tau=TAU, seg_lens=list(seg_lens))


def make_dense_layer(d: int, hq: int, hkv: int, head_dim: int, d_ff: int, seed: int,
                     dtype=torch.bfloat16, device="cpu") -> dict:
    """Weights of one above-gate decoder layer (Qwen3 layout: RMSNorm, fused
    QKV projection, per-head Q/K RMSNorm, output projection, RMSNorm, SwiGLU
    MLP), all nn.Linear [out, in]: projections N(0, 1/fan_in), norm weights
    1 + N(0, 0.1^2), gains U(0.5, 2); tau 1.2, eps 1e-6, rope theta 1e6."""
    gen = _torch_gen("cpu", seed)

    def lin(n_out, n_in):
        return (torch.randn((n_out, n_in), generator=gen) / math.sqrt(n_in)).to(dtype).to(device)

    def norm_w(n):
        return (1.0 + 0.1 * torch.randn((n,), generator=gen)).to(dtype).to(device)

    w = dict(ln1=norm_w(d), wqkv=lin((hq + 2 * hkv) * head_dim, d), q_norm=norm_w(head_dim),
             k_norm=norm_w(head_dim), wo=lin(d, hq * head_dim), ln2=norm_w(d), w_gate=lin(d_ff, d),
             w_up=lin(d_ff, d), w_down=lin(d, d_ff))
    w["gain"] = (torch.rand((hq,), generator=gen) * 1.5 + 0.5).to(device)
    w.update(tau=TAU, eps=1e-6, theta=1.0e6)
    return w


def make_kept_hidden(seg_lens: List[int], d: int, seed: int, dtype=torch.bfloat16, device="cpu",
                     n_query_tail: int = 0) -> dict:
    """Kept rows entering an above-gate layer: hidden states N(0, 1), original
    positions strictly increasing within each segment (random gaps 1..8),
    bias -|N(0, 1.5^2)| for document rows and 0 for the last n_query_tail rows
    of each segment."""
    m = int(sum(seg_lens))
    gen = _torch_gen("cpu", seed)
    h = torch.randn((m, d), generator=gen).to(dtype)
    bias = -(torch.randn((m,), generator=gen) * 1.5).abs()
    pos = torch.empty((m,), dtype=torch.int32)
    off = 0
    for ln in seg_lens:
        if ln:
            gaps = torch.randint(1, 9, (ln,), generator=gen)
            gaps[0] = torch.randint(0, 5, (1,), generator=gen)[0]
            pos[off:off + ln] = torch.cumsum(gaps, 0).to(torch.int32)
            tail = min(n_query_tail, ln)
            if tail:
                bias[off + ln - tail: off + ln] = 0.0
        off += ln
    return dict(h=h.to(device), pos=pos.to(device), bias=bias.to(device), seg_lens=list(seg_lens))


def make_delta_inputs(seg_lens: List[int], n_heads: int, dk: int, dv: int, seed: int, dtype=torch.bfloat16,
                      device="cpu") -> dict:
    """Kept-row inputs of a Gated-DeltaNet token mixer: q and k L2-normalised per
    head (then rounded to dtype), v ~ N(0, 1), decay alpha ~ U(0.9, 1) given as
    g = log(alpha), beta ~ U(0.05, 0.95), both fp32 [M, H]."""
    m = int(sum(seg_lens))
    gen = _torch_gen("cpu", seed)
    q = torch.randn((m, n_heads, dk), generator=gen)
    k = torch.randn((m, n_heads, dk), generator=gen)
    q = q / torch.linalg.vector_norm(q, dim=-1, keepdim=True)
    k = k / torch.linalg.vector_norm(k, dim=-1, keepdim=True)
    v = torch.randn((m, n_heads, dv), generator=gen)
    g = torch.log(torch.rand((m, n_heads), generator=gen) * 0.1 + 0.9)
    beta = torch.rand((m, n_heads), generator=gen) * 0.9 + 0.05
    return dict(q=q.to(dtype).to(device), k=k.to(dtype).to(device), v=v.to(dtype).to(device), g=g.to(device),
                beta=beta.to(device), seg_lens=list(seg_lens))

"""GPU parity on seeded random prompt tables: the whole pruned-prefill layer
(gate, select, compaction, attention) through the C ABI against the fp64
oracle, over prompt tables no hand-written case covers; then the backward of
the attention, the gate MLP's backward, decode over the pruned cache, the
above-gate decoder layer and the gated delta rule on random tables of their
own.

Each seed draws one to five packed prompts with rows before the document
(sometimes none), a document of 0 to ~1400 rows, a question of 1 to 160
rows and a budget anywhere in [0, n_doc] (both ends included often), one of
the gate / head shapes below (MFMA and plain gate paths, head_dim 64 and
128, GQA ratios 1, 2, 3, 8, bf16 and fp32), with or without gate biases and
with or without an explicit non-decreasing position array that repeats
and skips positions. Bars as in the other parity tests: selection,
gathers and positions bit-exact on the GPU's own scores; gate scores and
attention within the dtype's bar of the oracle; bias within 1e-6 relative.
The other calls use the bars of their hand-written tests (check_backward,
check_gate_backward, check_decode, check_dense_layer, check_delta_scan).
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import learned_token_pruning_layer_amd as tg
from synthetic import Prompt
from tests.test_gpu_parity import (check_backward, check_decode, check_delta_scan, check_dense_layer,
                                   check_gate_backward)

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (dtype, d_model, d_hidden, hq, hkv, head_dim)
SHAPES = [
    (torch.bfloat16, 256, 128, 4, 2, 64),
    (torch.bfloat16, 512, 192, 8, 1, 128),
    (torch.bfloat16, 320, 48, 6, 3, 128),    # d_hidden 48: the plain gate path
    (torch.float32, 192, 64, 4, 4, 64),
    (torch.bfloat16, 2048, 256, 16, 8, 128),
    (torch.bfloat16, 256, 256, 2, 2, 64),
]


def note(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().float().cpu().double().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().double().numpy()


def random_table(rng, max_prompts):
    prompts, start = [], 0
    for _ in range(int(rng.integers(1, max_prompts + 1))):
        pre = 0 if rng.random() < 0.5 else int(rng.integers(1, 64))
        r = rng.random()
        n_doc = 0 if r < 0.1 else (int(rng.integers(1, 40)) if r < 0.3 else int(rng.integers(100, 1400)))
        nq = int(rng.integers(1, 161))
        r = rng.random()
        k_doc = 0 if r < 0.15 else (n_doc if r < 0.3 else int(rng.integers(0, n_doc + 1)))
        prompts.append(Prompt(start, pre + n_doc + nq, pre, pre + n_doc, k_doc))
        start += pre + n_doc + nq
    return prompts


def random_positions(rng, prompts):
    pos = np.empty(prompts[-1].start + prompts[-1].length, dtype=np.int32)
    for p in prompts:
        steps = rng.choice([0, 1, 1, 1, 2, 5], size=p.length)
        steps[0] = int(rng.integers(0, 3))
        pos[p.start:p.start + p.length] = np.cumsum(steps)
    return pos


@pytest.mark.parametrize("seed", range(len(SHAPES) * 5))
def test_end_to_end_random_table(seed):
    dt, d, h, hq, hkv, hd = SHAPES[seed % len(SHAPES)]
    rng = np.random.default_rng(7000 + seed)
    prompts = random_table(rng, 3 if d >= 2048 else 5)
    n = prompts[-1].start + prompts[-1].length
    with_b = bool(rng.random() < 0.5)
    with_pos = bool(rng.random() < 0.5)
    note(f"random table seed={seed}: {dt} d={d} H={h} hq={hq} hkv={hkv} D={hd} N={n} "
         f"prompts={[(p.doc_begin, p.n_doc, p.length - p.doc_end, p.k_doc) for p in prompts]} "
         f"biases={with_b} pos={with_pos}")
    g = torch.Generator().manual_seed(7000 + seed)
    x = torch.randn(n, d, generator=g)
    w1 = torch.randn(h, d, generator=g) / d ** 0.5
    w2 = torch.randn(h, generator=g) / h ** 0.5
    b1 = torch.randn(h, generator=g) * 0.1 if with_b else None
    b2 = float(rng.normal()) if with_b else 0.0
    q = torch.randn(n, hq * hd, generator=g)
    k = torch.randn(n, hkv * hd, generator=g)
    v = torch.randn(n, hkv * hd, generator=g)
    gain = torch.rand(hq, generator=g) * 1.5 + 0.5
    tau = float(rng.uniform(0.6, 1.8))
    pos = random_positions(rng, prompts) if with_pos else None
    cast = [t.to(dt) if t is not None else None for t in (x, w1, w2, b1, q, k, v)]
    x, w1, w2, b1, q, k, v = cast
    layer_in = type("L", (), dict(q=q.to(DEV), k=k.to(DEV), v=v.to(DEV), gain=gain.to(DEV), tau=tau))
    lay = tg.GatedPrefillLayer(x.to(DEV), w1.to(DEV), w2.to(DEV), prompts, [layer_in], hq, hkv, hd,
                               b1=None if b1 is None else b1.to(DEV), b2=b2,
                               pos=None if pos is None else torch.as_tensor(pos, device=DEV))
    lay.run()
    torch.cuda.synchronize()

    # gate
    s_ref = oracle.gate_scores(x, w1, w2, b1, b2)
    s_gpu = lay.scores.cpu().numpy()
    bar = 2e-2 * np.abs(s_ref).max() if dt == torch.bfloat16 else 1e-4
    assert np.abs(s_gpu.astype(np.float64) - s_ref).max() <= bar
    # select, on the GPU's own scores
    kept = lay.kept.cpu().numpy().astype(np.int64)
    assert np.array_equal(kept, oracle.select_topk(s_gpu, prompts))
    assert len(kept) == sum(p.n_kept for p in prompts)
    # compaction
    (hk, qk, kk, vk), pk, bk = oracle.compact(kept, prompts, (x, q, k, v), s_gpu, pos)
    assert torch.equal(lay.hidden_kept.cpu(), hk)
    for got, ref in zip(lay.qkv_kept[0], (qk, kk, vk)):
        assert torch.equal(got.cpu(), ref)
    assert np.array_equal(lay.pos_kept.cpu().numpy().astype(np.int64), np.asarray(pk, dtype=np.int64))
    b = f64(lay.bias_kept)
    assert np.all(np.abs(b - bk) <= 1e-6 * np.maximum(1.0, np.abs(bk)))
    # attention
    m = len(kept)
    if m == 0:
        return
    rows = None if m <= 1500 else np.sort(rng.choice(m, 256, replace=False))
    o, _ = oracle.gated_attention(qk.view(m, hq, hd), kk.view(m, hkv, hd), vk.view(m, hkv, hd), bk, pk,
                                  [p.n_kept for p in prompts], hq, hkv, gain, tau, rows=rows)
    got = f64(lay.outs[0])
    if rows is not None:
        got, o = got[rows], o[rows]
    if dt == torch.bfloat16:
        err = np.abs(got - o).max(axis=-1)
        assert np.all(err <= 2e-2 * np.abs(o).max(axis=-1))
    else:
        assert np.abs(got - o).max() <= 1e-4


# (hq, hkv, head_dim) for the backward and decode tables
HEADS = [(16, 8, 128), (4, 2, 64), (6, 3, 128), (8, 1, 64), (4, 4, 128)]


@pytest.mark.parametrize("seed", range(10))
def test_backward_random_table(seed):
    """One to four prompts of 1-899 kept rows, a question tail of 1-60 rows, random
    temperature, with or without repeated positions."""
    hq, hkv, d = HEADS[seed % len(HEADS)]
    rng = np.random.default_rng(8000 + seed)
    lens = [int(x) for x in rng.integers(1, 900, size=int(rng.integers(1, 5)))]
    ties = bool(rng.random() < 0.5)
    tau = float(rng.uniform(0.6, 1.6))
    tail = int(rng.integers(1, 61))
    note(f"backward random table seed={seed}: hq={hq} hkv={hkv} D={d} lens={lens} ties={ties} "
         f"tau={tau:.3f} tail={tail}")
    check_backward(lens, hq, hkv, d, seed=8000 + seed, pos_ties=ties, tau=tau, tail=tail)


@pytest.mark.parametrize("seed", range(10))
def test_decode_random_table(seed):
    """One to forty cached sequences of 1-2999 rows with gaps between them, 1 to
    8/G new tokens each, random temperature, with or without repeated positions;
    bf16, and fp32 for every fifth seed."""
    hq, hkv, d = HEADS[seed % len(HEADS)]
    rng = np.random.default_rng(9000 + seed)
    g = hq // hkv
    segs, st = [], int(rng.integers(0, 5))
    for _ in range(int(rng.integers(1, 41))):
        ln = int(rng.integers(1, 3000))
        nn = int(min(ln, rng.integers(1, 8 // g + 1)))
        segs.append((st, ln, nn))
        st += ln + int(rng.integers(0, 3))
    dt = torch.float32 if seed % 5 == 4 else torch.bfloat16
    ties = bool(rng.random() < 0.5)
    tau = float(rng.uniform(0.6, 1.6))
    note(f"decode random table seed={seed}: {dt} hq={hq} hkv={hkv} D={d} {len(segs)} sequences, "
         f"{sum(s[1] for s in segs)} cached rows, {sum(s[2] for s in segs)} new, ties={ties} tau={tau:.3f}")
    check_decode(segs, hq, hkv, d, seed=9000 + seed, dtype=dt, pos_ties=ties, tau=tau)


# (d_model, hq, hkv, head_dim, d_ff) of the above-gate decoder layer
DENSE = [(256, 4, 2, 64, 384), (512, 8, 4, 128, 1024), (384, 6, 3, 64, 448), (256, 2, 2, 128, 192),
         (640, 10, 2, 64, 704)]


@pytest.mark.parametrize("seed", range(5))
def test_dense_layer_random_table(seed):
    """One to four prompts of 1-699 kept rows, positions starting at 0 or far out."""
    d, hq, hkv, dh, d_ff = DENSE[seed]
    rng = np.random.default_rng(9500 + seed)
    segs = [int(x) for x in rng.integers(1, 700, size=int(rng.integers(1, 5)))]
    pos_offset = 0 if rng.random() < 0.5 else int(rng.integers(1, 100000))
    note(f"dense layer random table seed={seed}: d={d} hq={hq} hkv={hkv} D={dh} d_ff={d_ff} "
         f"segs={segs} pos_offset={pos_offset}")
    check_dense_layer(segs, d, hq, hkv, dh, d_ff, seed=9500 + seed, pos_offset=pos_offset)


@pytest.mark.parametrize("seed", range(5))
def test_delta_scan_random_table(seed):
    """One to five prompts of 1-499 kept rows, 1-8 heads, with or without initial
    states (prompts without rows have a test of their own)."""
    rng = np.random.default_rng(9700 + seed)
    segs = [int(x) for x in rng.integers(1, 500, size=int(rng.integers(1, 6)))]
    nh = int(rng.choice([1, 2, 4, 8]))
    with_state = bool(rng.random() < 0.5)
    note(f"delta scan random table seed={seed}: segs={segs} heads={nh} state={with_state}")
    check_delta_scan(segs, nh, seed=9700 + seed, with_state=with_state)


@pytest.mark.parametrize("seed", range(6))
def test_gate_backward_random_table(seed):
    """1-3000 rows, d a multiple of 64 up to 1024, every built d_hidden, a random
    row list (sometimes empty or every row), with or without b1 and dx."""
    rng = np.random.default_rng(9900 + seed)
    n = int(rng.integers(1, 3001))
    d = 64 * int(rng.integers(1, 17))
    h = int(rng.choice([64, 128, 192, 256]))
    r = rng.random()
    n_list = 0 if r < 0.15 else (n if r < 0.3 else int(rng.integers(1, n + 1)))
    with_b1 = bool(rng.random() < 0.5)
    with_dx = bool(rng.random() < 0.7)
    note(f"gate backward random table seed={seed}: n={n} d={d} H={h} listed={n_list} b1={with_b1} dx={with_dx}")
    check_gate_backward(n, d, h, n_list, seed=9900 + seed, with_b1=with_b1, with_dx=with_dx)

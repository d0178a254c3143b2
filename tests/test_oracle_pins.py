"""Pins for the fp64 oracle, independent of the oracle itself (CPU only).

Every oracle function is checked against at least one of: hand-derived
closed forms (tests/golden/hand_cases.json), pure-Python brute force on
tiny inputs (tests/brute.py), exhaustive enumeration, invariants the pages
fix, and library routines the operation reduces to (torch CPU fp64
nn.functional.linear/silu/logsigmoid/scaled_dot_product_attention).
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synthetic import Prompt, make_attention_inputs, make_scores, make_workload
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")
_MATH = {k: getattr(math, k) for k in ("log", "exp", "sqrt", "pi")}


def ev(x):
    """Evaluate a closed-form expression string (math names only)."""
    if x is None:
        return None
    if isinstance(x, (int, float)):
        return float(x)
    if isinstance(x, list):
        return [ev(e) for e in x]
    return float(eval(x, {"__builtins__": {}}, _MATH))


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------- gate ----

def test_gate_golden(golden):
    for case in golden["gate"]:
        x = np.array(ev(case["x"]))
        w1 = np.array(ev(case["w1"]))
        w2 = np.array(ev(case["w2"]))
        b1 = None if case["b1"] is None else np.array(ev(case["b1"]))
        got = oracle.gate_scores(x, w1, w2, b1, ev(case["b2"]))
        np.testing.assert_allclose(got, ev(case["expected"]), rtol=1e-15, atol=1e-15,
                                   err_msg=case["name"])


@pytest.mark.parametrize("seed", range(4))
def test_gate_vs_bruteforce(seed):
    rng = np.random.default_rng(seed)
    n, d, h = 7, 13, 5
    x = rng.normal(size=(n, d)) * 2
    w1 = rng.normal(size=(h, d))
    w2 = rng.normal(size=h)
    b1 = rng.normal(size=h)
    got = oracle.gate_scores(x, w1, w2, b1, 0.7)
    ref = brute.gate(x.tolist(), w1.tolist(), w2.tolist(), b1.tolist(), 0.7)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_gate_vs_torch_library():
    g = torch.Generator().manual_seed(5)
    n, d, h = 300, 96, 40
    x = torch.randn(n, d, generator=g, dtype=torch.float64)
    w1 = torch.randn(h, d, generator=g, dtype=torch.float64) / math.sqrt(d)
    b1 = torch.randn(h, generator=g, dtype=torch.float64)
    w2 = torch.randn(1, h, generator=g, dtype=torch.float64)
    ref = F.linear(F.silu(F.linear(x, w1, b1)), w2, torch.tensor([-0.3], dtype=torch.float64))[:, 0]
    got = oracle.gate_scores(x.numpy(), w1.numpy(), w2.numpy()[0], b1.numpy(), -0.3, block_rows=64)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_gate_one_hot_reduces_to_silu():
    rng = np.random.default_rng(0)
    n, d, h = 50, 8, 3
    x = rng.normal(size=(n, d)) * 5
    w1 = np.zeros((h, d))
    w1[0, 6] = 1.0
    w1[1, 2] = 1.0
    w2 = np.array([1.0, 0.0, 0.0])
    s = oracle.gate_scores(x, w1, w2)
    z = x[:, 6]
    np.testing.assert_allclose(s, z / (1 + np.exp(-z)), rtol=1e-14, atol=1e-14)


def test_planted_rows_score_top():
    """The synthetic 16k workload plants 16 rows along the gate's first
    hidden direction; the oracle gate must rank them all in the top 16 and
    the selector must keep them."""
    w = make_workload("qwen16k", with_layers=False)
    s = oracle.gate_scores(w.x, w.w1, w.w2)
    top16 = np.argsort(-s, kind="stable")[:16]
    assert set(top16.tolist()) == set(w.planted.tolist())
    kept = oracle.select_topk(s.astype(np.float32), w.prompts)
    assert set(w.planted.tolist()) <= set(kept.tolist())


# -------------------------------------------------------------- select ----

def test_select_golden(golden):
    for case in golden["select"]:
        prompts = [Prompt(*p) for p in case["prompts"]]
        got = oracle.select_topk(np.array(case["scores"], dtype=np.float64), prompts)
        assert got.tolist() == case["expected"], case["name"]


def _spans(n):
    yield 0, n
    if n >= 3:
        yield 1, n - 1
        yield 0, n - 2
        yield 2, n


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_select_exhaustive_small(n):
    """Every score vector in {0,1,2}^n, several document spans, every k."""
    for vals in itertools.product((0.0, 1.0, 2.0), repeat=n):
        s = np.array(vals)
        for db, de in _spans(n):
            for k in range(de - db + 1):
                prompts = [Prompt(0, n, db, de, k)]
                assert oracle.select_topk(s, prompts).tolist() == brute.select(s.tolist(), prompts)


def test_select_exhaustive_nan_and_signed_zero():
    """NaN ranks below every number; -0 and +0 tie (lower row wins)."""
    vals = (float("nan"), -0.0, 0.0, 1.0, -float("inf"))
    n = 5
    for tup in itertools.product(vals, repeat=n):
        s = np.array(tup)
        for k in range(n + 1):
            prompts = [Prompt(0, n, 0, n, k)]
            assert oracle.select_topk(s, prompts).tolist() == brute.select(s.tolist(), prompts)


def test_select_multi_prompt_bruteforce():
    rng = np.random.default_rng(3)
    for trial in range(200):
        prompts, start = [], 0
        for _ in range(rng.integers(1, 5)):
            ln = int(rng.integers(0, 9))
            db = int(rng.integers(0, ln + 1))
            de = int(rng.integers(db, ln + 1))
            prompts.append(Prompt(start, ln, db, de, int(rng.integers(0, de - db + 1))))
            start += ln
        s = rng.integers(-2, 3, size=start).astype(np.float64)
        assert oracle.select_topk(s, prompts).tolist() == brute.select(s.tolist(), prompts)


@pytest.mark.parametrize("kind", ["normal", "ties", "few", "signed0", "wide"])
def test_select_invariants(kind):
    s = make_scores(5000, seed=11, kind=kind).numpy()
    prompts = [Prompt(0, 3000, 100, 2900, 700), Prompt(3000, 2000, 0, 1744, 1000)]
    kept = oracle.select_topk(s, prompts)
    assert len(kept) == oracle.kept_rows(prompts)
    assert np.all(np.diff(kept) > 0)
    ks = set(kept.tolist())
    for p in prompts:
        rows = range(p.start, p.start + p.length)
        doc = range(p.start + p.doc_begin, p.start + p.doc_end)
        # the question (every non-document row) survives
        assert all(r in ks for r in rows if r not in doc)
        kd = [r for r in doc if r in ks]
        dropped = [r for r in doc if r not in ks]
        assert len(kd) == p.k_doc
        if kd and dropped:
            lo = min(s[r] for r in kd)
            hi = max(s[r] for r in dropped)
            assert lo >= hi
            # ties at the threshold go to the lower row ids
            if lo == hi:
                assert max(r for r in kd if s[r] == lo) < min(r for r in dropped if s[r] == hi)


def test_select_budget_extremes():
    s = make_scores(1000, seed=1).numpy()
    full = [Prompt(0, 1000, 0, 900, 900)]
    assert oracle.select_topk(s, full).tolist() == list(range(1000))
    none = [Prompt(0, 1000, 0, 900, 0)]
    assert oracle.select_topk(s, none).tolist() == list(range(900, 1000))
    with pytest.raises(ValueError):
        oracle.select_topk(s, [Prompt(0, 1000, 0, 900, 901)])


# ------------------------------------------------------------- compact ----

def test_logsigmoid_golden(golden):
    for case in golden["logsigmoid"]:
        assert oracle.logsigmoid(ev(case["s"])) == pytest.approx(ev(case["expected"]), rel=1e-15, abs=1e-15)


def test_logsigmoid_vs_library_and_asymptotes():
    s = np.concatenate([np.linspace(-60, 60, 2001), [-745.0, 700.0]])
    ref = F.logsigmoid(torch.tensor(s, dtype=torch.float64)).numpy()
    np.testing.assert_allclose(oracle.logsigmoid(s), ref, rtol=1e-14, atol=1e-300)
    # log sigmoid(s) -> -e^{-s} for large s, -> s for very negative s
    assert oracle.logsigmoid(40.0) == pytest.approx(-math.exp(-40.0), rel=1e-12)
    assert oracle.logsigmoid(-40.0) == pytest.approx(-40.0 - math.exp(-40.0), rel=1e-15)
    # independent form -log(1 + e^{-s}) where it does not overflow
    t = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(oracle.logsigmoid(t), -np.log(1 + np.exp(-t)), rtol=1e-13, atol=4e-16)


def test_compact_gather_pos_bias():
    rng = np.random.default_rng(2)
    prompts = [Prompt(0, 10, 2, 8, 3), Prompt(10, 6, 0, 4, 1)]
    s = rng.normal(size=16)
    kept = oracle.select_topk(s, prompts)
    t1 = rng.normal(size=(16, 5))
    t2 = np.arange(16 * 3).reshape(16, 3)
    (g1, g2), pk, bias = oracle.compact(kept, prompts, (t1, t2), s)
    for m, r in enumerate(kept):
        assert np.array_equal(g1[m], t1[r]) and np.array_equal(g2[m], t2[r])
        p = prompts[0] if r < 10 else prompts[1]
        assert pk[m] == r - p.start
        in_doc = p.start + p.doc_begin <= r < p.start + p.doc_end
        # query rows carry no bias; document rows carry log sigmoid(score)
        expect = math.log(1.0 / (1.0 + math.exp(-s[r]))) if in_doc else 0.0
        assert bias[m] == pytest.approx(expect, rel=1e-13, abs=0)
    pos = rng.integers(0, 100000, size=16)
    _, pk2, _ = oracle.compact(kept, prompts, (), s, pos)
    assert pk2.tolist() == pos[kept].tolist()


def test_compact_full_budget_is_identity():
    s = make_scores(200, seed=4).numpy()
    prompts = [Prompt(0, 200, 0, 180, 180)]
    kept = oracle.select_topk(s, prompts)
    x = np.random.default_rng(0).normal(size=(200, 4))
    (g,), pk, _ = oracle.compact(kept, prompts, (x,), s)
    assert np.array_equal(g, x) and pk.tolist() == list(range(200))


# ----------------------------------------------------------- attention ----

def test_attention_golden(golden):
    for case in golden["attention"]:
        q = np.array(ev(case["q"]))
        k = np.array(ev(case["k"]))
        v = np.array(ev(case["v"]))
        sc = case["scores"]
        prompts = [Prompt(0, len(sc), 0, sum(1 for e in sc if e is not None), 0)]
        bias = np.array([0.0 if e is None else oracle.logsigmoid(ev(e)) for e in sc])
        o, lse = oracle.gated_attention(q, k, v, bias, np.array(case["pos"]), [len(sc)],
                                        case["hq"], case["hkv"], np.array(ev(case["gain"])),
                                        ev(case["tau"]))
        np.testing.assert_allclose(o, ev(case["expected_o"]), rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(lse, ev(case["expected_lse"]), rtol=1e-14, atol=1e-14)
        del prompts


@pytest.mark.parametrize("hq,hkv", [(4, 2), (3, 3), (8, 2)])
def test_attention_reduces_to_sdpa(hq, hkv):
    """Full budget and zero gain: plain causal GQA attention (torch SDPA,
    fp64, K/V heads repeated for each query-head group)."""
    d, m, tau = 16, 70, 1.2
    a = make_attention_inputs([m], hq, hkv, d, seed=7, dtype=torch.float64)
    pos = np.arange(m)
    o, lse = oracle.gated_attention(a["q"], a["k"], a["v"], a["bias"], pos, [m], hq, hkv,
                                    np.zeros(hq), tau)
    q = a["q"].permute(1, 0, 2)[None]
    k = a["k"].permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    v = a["v"].permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    ref = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=1.0 / (math.sqrt(d) * tau))
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_attention_with_bias_vs_sdpa_float_mask():
    """Nonzero gain: SDPA with an additive float mask gain[h]*bias[j] on
    visible keys and -inf elsewhere (positions with repeats)."""
    hq, hkv, d, m, tau = 4, 2, 8, 41, 0.7
    a = make_attention_inputs([m], hq, hkv, d, seed=9, dtype=torch.float64, pos_ties=True,
                              n_query_tail=5)
    pos = a["pos"].numpy()
    o, _ = oracle.gated_attention(a["q"], a["k"], a["v"], a["bias"], pos, [m], hq, hkv,
                                  a["gain"], tau)
    vis = torch.tensor(pos[None, :] <= pos[:, None])
    mask = torch.where(vis[None], a["gain"].double()[:, None, None] * a["bias"][None, None, :],
                       torch.tensor(-math.inf, dtype=torch.float64))
    q = a["q"].permute(1, 0, 2)[None]
    k = a["k"].permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    v = a["v"].permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    ref = F.scaled_dot_product_attention(q, k, v, attn_mask=mask[None], scale=1.0 / (math.sqrt(d) * tau))
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_attention_vs_multiplicative_bruteforce():
    """exp(l_ij) = exp(q.k/(sqrt(D) tau)) * sigmoid(s_j)^g: the additive
    log-sigmoid bias is the multiplicative re-weighting of each key."""
    seg = [9, 1, 6]
    hq, hkv, d = 4, 2, 4
    a = make_attention_inputs(seg, hq, hkv, d, seed=13, dtype=torch.float64, pos_ties=True)
    m = sum(seg)
    rng = np.random.default_rng(0)
    s = rng.normal(size=m) * 3
    is_doc = rng.random(m) < 0.7
    bias = np.where(is_doc, oracle.logsigmoid(s), 0.0)
    pos = a["pos"].numpy()
    gain = a["gain"].numpy()
    o, lse = oracle.gated_attention(a["q"], a["k"], a["v"], bias, pos, seg, hq, hkv, gain, 1.2)
    ob, lb = brute.attention_multiplicative(a["q"].tolist(), a["k"].tolist(), a["v"].tolist(),
                                            s.tolist(), is_doc.tolist(), pos.tolist(), seg, hq, hkv,
                                            gain.tolist(), 1.2)
    np.testing.assert_allclose(o, ob, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, lb, rtol=1e-11, atol=1e-12)


def test_attention_closed_forms():
    hq, hkv, d = 4, 2, 8
    seg = [30, 17]
    a = make_attention_inputs(seg, hq, hkv, d, seed=21, dtype=torch.float64)
    m = sum(seg)
    pos = a["pos"].numpy()
    # V = 1 => O = 1 (softmax rows sum to one)
    ones = np.ones((m, hkv, d))
    o1, _ = oracle.gated_attention(a["q"], a["k"], ones, a["bias"], pos, seg, hq, hkv, a["gain"], 1.2)
    np.testing.assert_allclose(o1, 1.0, rtol=0, atol=1e-14)
    # the first row of each segment sees only itself
    o, lse = oracle.gated_attention(a["q"], a["k"], a["v"], a["bias"], pos, seg, hq, hkv, a["gain"], 1.2)
    vv = a["v"].numpy()
    for off in (0, seg[0]):
        for h in range(hq):
            np.testing.assert_allclose(o[off, h], vv[off, (h * hkv) // hq], rtol=1e-14)
    # equal keys: weights are sigmoid(s)^g, independent of q and of tau
    kk = np.repeat(a["k"].numpy()[:1], m, axis=0)
    s = np.random.default_rng(1).normal(size=m)
    bias = oracle.logsigmoid(s)
    for tau in (0.5, 3.0):
        o2, _ = oracle.gated_attention(a["q"], kk, vv, bias, pos, seg, hq, hkv, a["gain"], tau)
        i = seg[0] - 1
        for h in range(hq):
            w = (1.0 / (1.0 + np.exp(-s[:seg[0]]))) ** float(a["gain"][h])
            ref = (w[:, None] * vv[:seg[0], (h * hkv) // hq]).sum(0) / w.sum()
            np.testing.assert_allclose(o2[i, h], ref, rtol=1e-12)


def test_attention_sampled_rows_match_full():
    hq, hkv, d = 2, 1, 8
    a = make_attention_inputs([50], hq, hkv, d, seed=3, dtype=torch.float64)
    pos = a["pos"].numpy()
    full, lf = oracle.gated_attention(a["q"], a["k"], a["v"], a["bias"], pos, [50], hq, hkv, a["gain"], 1.2)
    rows = np.array([0, 7, 49])
    part, lp = oracle.gated_attention(a["q"], a["k"], a["v"], a["bias"], pos, [50], hq, hkv, a["gain"], 1.2,
                                      rows=rows)
    np.testing.assert_array_equal(part[rows], full[rows])
    assert np.isnan(part[1]).all()


# -------------------------------------------------------------- backward ----

def _bwd_case(seed, seg, hq, hkv, d, pos_ties=True):
    m = sum(seg)
    a = make_attention_inputs(seg, hq, hkv, d, seed=seed, dtype=torch.float64, pos_ties=pos_ties, n_query_tail=2)
    gd = torch.Generator().manual_seed(seed + 3)
    d_out = torch.randn((m, hq, d), generator=gd, dtype=torch.float64).numpy()
    return (a["q"].numpy(), a["k"].numpy(), a["v"].numpy(), a["bias"].numpy().astype(np.float64),
            a["pos"].numpy(), a["gain"].numpy().astype(np.float64), d_out)


@pytest.mark.parametrize("hq,hkv", [(2, 1), (4, 2), (3, 3)])
def test_attention_backward_vs_finite_differences(hq, hkv):
    """Every gradient against central differences of the (pinned) forward:
    L = sum(d_out * o)."""
    seg, d, tau = [5, 3], 3, 0.8
    q, k, v, b, pos, g, do = _bwd_case(31 + hq, seg, hq, hkv, d)
    grads = oracle.gated_attention_backward(q, k, v, b, pos, seg, hq, hkv, g, tau, do)

    def loss(q_, k_, v_, b_, g_, t_):
        o, _ = oracle.gated_attention(q_, k_, v_, b_, pos, seg, hq, hkv, g_, t_)
        return float((o * do).sum())

    eps = 1e-6
    for name, arr in (("dq", q), ("dk", k), ("dv", v), ("dbias", b), ("dgain", g)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += eps
            minus[idx] -= eps
            args = {"dq": (plus, k, v, b, g), "dk": (q, plus, v, b, g), "dv": (q, k, plus, b, g),
                    "dbias": (q, k, v, plus, g), "dgain": (q, k, v, b, plus)}
            ap = args[name]
            am = {"dq": (minus, k, v, b, g), "dk": (q, minus, v, b, g), "dv": (q, k, minus, b, g),
                  "dbias": (q, k, v, minus, g), "dgain": (q, k, v, b, minus)}[name]
            num[idx] = (loss(*ap, tau) - loss(*am, tau)) / (2 * eps)
        np.testing.assert_allclose(grads[name], num, rtol=1e-6, atol=1e-8, err_msg=name)
    num_tau = (loss(q, k, v, b, g, tau + eps) - loss(q, k, v, b, g, tau - eps)) / (2 * eps)
    np.testing.assert_allclose(grads["dtau"], num_tau, rtol=1e-6, atol=1e-8)


def test_attention_backward_vs_torch_autograd():
    """torch autograd (fp64, CPU) through SDPA with an additive float mask
    gain[h] * bias[j] built from leaf tensors: dq, dk, dv, dbias, dgain."""
    hq, hkv, d, m, tau = 4, 2, 16, 37, 1.3
    q, k, v, b, pos, g, do = _bwd_case(41, [m], hq, hkv, d)
    grads = oracle.gated_attention_backward(q, k, v, b, pos, [m], hq, hkv, g, tau, do)
    tq, tk, tv = (torch.from_numpy(x).clone().requires_grad_() for x in (q, k, v))
    tb, tg_ = torch.from_numpy(b).clone().requires_grad_(), torch.from_numpy(g).clone().requires_grad_()
    vis = torch.from_numpy(pos[None, :] <= pos[:, None])
    mask = torch.where(vis[None], tg_[:, None, None] * tb[None, None, :], torch.tensor(-math.inf, dtype=torch.float64))
    kk = tk.permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    vv = tv.permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    o = F.scaled_dot_product_attention(tq.permute(1, 0, 2)[None], kk, vv, attn_mask=mask[None],
                                       scale=1.0 / (math.sqrt(d) * tau))
    (o[0].permute(1, 0, 2) * torch.from_numpy(do)).sum().backward()
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv), ("dbias", tb), ("dgain", tg_)):
        np.testing.assert_allclose(grads[name], t.grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)


def test_attention_backward_invariants():
    """Softmax rows: sum_j ds_ij = 0, so the bias gradient sums to zero over each
    segment; zero gain gives zero bias gradient; d_out = 0 gives all zeros."""
    seg, hq, hkv, d = [20, 9, 1], 4, 2, 8
    q, k, v, b, pos, g, do = _bwd_case(51, seg, hq, hkv, d)
    gr = oracle.gated_attention_backward(q, k, v, b, pos, seg, hq, hkv, g, 1.2, do)
    off = 0
    for ln in seg:
        assert abs(gr["dbias"][off:off + ln].sum()) < 1e-12
        off += ln
    gr0 = oracle.gated_attention_backward(q, k, v, b, pos, seg, hq, hkv, np.zeros(hq), 1.2, do)
    np.testing.assert_allclose(gr0["dbias"], 0.0, atol=1e-15)
    grz = oracle.gated_attention_backward(q, k, v, b, pos, seg, hq, hkv, g, 1.2, np.zeros_like(do))
    for key in ("dq", "dk", "dv", "dbias", "dgain"):
        assert not np.any(grz[key])
    # a one-row segment: o = v, so dv = d_out summed over the group and every ds is 0
    i = seg[0] + seg[1]
    for h in range(hq):
        assert np.abs(gr["dq"][i, h]).max() < 1e-14  # ds = p (dp - do.o) = 1 * (do.v - do.v)
    np.testing.assert_allclose(gr["dv"][i, 0], do[i, 0] + do[i, 1], rtol=1e-14)


def test_attention_backward_given_forward_output():
    """The row term taken from a given forward output o: the exact output (from the
    pinned forward) reproduces the default gradients; a change of o orthogonal to
    d_out changes nothing; a change beta_i d_out_i / |d_out_i|^2 moves each row term
    do_i . o_i by beta_i, so sum_j ds_ij = -beta_i: the bias gradient of each segment
    sums to -sum_h g_h sum_i beta_ih, and dv (no row term) stays as it was."""
    seg, hq, hkv, d, tau = [11, 6], 4, 2, 8, 0.9
    q, k, v, b, pos, g, do = _bwd_case(57, seg, hq, hkv, d)
    o_exact, _ = oracle.gated_attention(q, k, v, b, pos, seg, hq, hkv, g, tau)
    ref = oracle.gated_attention_backward(q, k, v, b, pos, seg, hq, hkv, g, tau, do)
    same = oracle.gated_attention_backward(q, k, v, b, pos, seg, hq, hkv, g, tau, do, o=o_exact)
    for key in ("dq", "dk", "dv", "dbias", "dgain", "dtau"):
        np.testing.assert_allclose(same[key], ref[key], rtol=1e-10, atol=1e-13, err_msg=key)
    rng = np.random.default_rng(5)
    w = rng.standard_normal(do.shape)
    w -= ((w * do).sum(-1, keepdims=True) / (do * do).sum(-1, keepdims=True)) * do
    orth = oracle.gated_attention_backward(q, k, v, b, pos, seg, hq, hkv, g, tau, do, o=o_exact + w)
    for key in ("dq", "dk", "dv", "dbias", "dgain", "dtau"):
        np.testing.assert_allclose(orth[key], ref[key], rtol=1e-10, atol=1e-12, err_msg=key)
    beta = rng.standard_normal(do.shape[:2])
    shift = o_exact + beta[..., None] * do / (do * do).sum(-1, keepdims=True)
    sh = oracle.gated_attention_backward(q, k, v, b, pos, seg, hq, hkv, g, tau, do, o=shift)
    np.testing.assert_allclose(sh["dv"], ref["dv"], rtol=1e-12, atol=1e-14)
    off = 0
    for ln in seg:
        want = -(g[None, :] * beta[off:off + ln]).sum()
        assert abs(sh["dbias"][off:off + ln].sum() - want) < 1e-10 * max(1.0, abs(want))
        off += ln
    # the magnitudes returned for tolerances bound the sums they describe
    assert abs(ref["dtau"]) <= ref["dtau_abs"] <= ref["dtau_mag"] * (1 + 1e-12)
    assert np.all(np.abs(ref["dgain"]) <= ref["dgain_abs"] * (1 + 1e-12))


def test_score_grad_chain():
    """d(score) = d(bias) * d logsigmoid(s)/ds for kept document rows (central
    differences of the pinned logsigmoid), 0 for question and pruned rows."""
    prompts = [Prompt(0, 12, 2, 9, 4), Prompt(12, 6, 0, 4, 2)]
    s = np.random.default_rng(3).normal(size=18) * 3
    kept = oracle.select_topk(s, prompts)
    db = np.random.default_rng(4).normal(size=len(kept))
    ds = oracle.score_grad(db, s, kept, prompts)
    eps = 1e-6
    for m, r in enumerate(kept):
        p = prompts[0] if r < 12 else prompts[1]
        doc = p.start + p.doc_begin <= r < p.start + p.doc_end
        want = db[m] * (oracle.logsigmoid(s[r] + eps) - oracle.logsigmoid(s[r] - eps)) / (2 * eps) if doc else 0.0
        assert abs(ds[r] - want) < 1e-8
    pruned = np.setdiff1d(np.arange(18), kept)
    assert not np.any(ds[pruned])


def _gate_bwd_case(seed, n=9, d=6, h=4):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(n, d)), rng.normal(size=(h, d)) / np.sqrt(d), rng.normal(size=h) / np.sqrt(h),
            rng.normal(size=h) * 0.3, rng.normal(size=n))


def test_gate_backward_vs_finite_differences():
    """Every gradient of L = sum_r ds_r s_r against central differences of the
    pinned forward (gate_scores), on a tiny gate with biases and a row list."""
    x, w1, w2, b1, ds = _gate_bwd_case(5)
    rows = np.array([7, 1, 4, 8])
    dsm = np.zeros_like(ds)
    dsm[rows] = ds[rows]  # rows outside the list count as d_scores = 0

    def loss(x_=x, w1_=w1, w2_=w2, b1_=b1, b2=0.25):
        return float(dsm @ oracle.gate_scores(x_, w1_, w2_, b1_, b2))

    g = oracle.gate_backward(x, w1, w2, ds, rows=rows, b1=b1)
    eps = 1e-6

    def fd(name, arr, idx):
        a = arr.copy()
        a[idx] += eps
        up = loss(**{name: a})
        a[idx] -= 2 * eps
        return (up - loss(**{name: a})) / (2 * eps)

    for idx in [(0, 0), (2, 5), (3, 1)]:
        assert abs(g["dw1"][idx] - fd("w1_", w1, idx)) < 1e-7
    for i in range(4):
        assert abs(g["db1"][i] - fd("b1_", b1, i)) < 1e-7
        assert abs(g["dw2"][i] - fd("w2_", w2, i)) < 1e-7
    for m, r in enumerate(rows):
        for c in (0, 3, 5):
            assert abs(g["dx"][m, c] - fd("x_", x, (r, c))) < 1e-7
    assert abs(g["db2"] - (loss(b2=0.25 + eps) - loss(b2=0.25 - eps)) / (2 * eps)) < 1e-7


def test_gate_backward_vs_torch_autograd():
    """The same gradients from torch autograd through a gate written with
    torch ops (not the oracle), all rows listed."""
    x, w1, w2, b1, ds = _gate_bwd_case(6, n=11, d=8, h=5)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in
         dict(x=x, w1=w1, w2=w2, b1=b1).items()}
    b2 = torch.tensor(0.5, dtype=torch.float64, requires_grad=True)
    s = torch.nn.functional.silu(t["x"] @ t["w1"].T + t["b1"]) @ t["w2"] + b2
    (s * torch.tensor(ds)).sum().backward()
    g = oracle.gate_backward(x, w1, w2, ds, b1=b1)
    for mine, ref in (("dx", t["x"]), ("dw1", t["w1"]), ("db1", t["b1"]), ("dw2", t["w2"])):
        np.testing.assert_allclose(g[mine], ref.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert abs(g["db2"] - b2.grad.item()) < 1e-12


def test_gate_backward_invariants():
    """Zero w2 blocks every gradient but dw2 and db2; unlisted rows change
    nothing; the gradients are linear in d_scores."""
    x, w1, w2, b1, ds = _gate_bwd_case(7)
    g0 = oracle.gate_backward(x, w1, np.zeros_like(w2), ds, b1=b1)
    assert not np.any(g0["dw1"]) and not np.any(g0["db1"]) and not np.any(g0["dx"])
    rows = np.array([2, 3, 6])
    ds2 = ds.copy()
    ds2[[0, 1, 4]] = 99.0  # rows outside the list
    ga, gb = (oracle.gate_backward(x, w1, w2, d, rows=rows, b1=b1) for d in (ds, ds2))
    for k in ("dx", "dw1", "db1", "dw2"):
        np.testing.assert_array_equal(ga[k], gb[k])
    g2 = oracle.gate_backward(x, w1, w2, 2.0 * ds, b1=b1)
    g1 = oracle.gate_backward(x, w1, w2, ds, b1=b1)
    for k in ("dx", "dw1", "db1", "dw2"):
        np.testing.assert_allclose(g2[k], 2.0 * g1[k], rtol=1e-14, atol=1e-14)


# ----------------------------------------------------- full above-gate layer ----

def test_rms_norm_vs_library_and_closed_form():
    """RMSNorm against torch's own rms_norm, and a constant row c against
    c / sqrt(c^2 + eps) * w."""
    rng = np.random.default_rng(11)
    x, w = rng.normal(size=(7, 24)), rng.normal(size=24)
    ref = torch.nn.functional.rms_norm(torch.tensor(x), (24,), torch.tensor(w), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rms_norm(x, w, 1e-6), ref, rtol=1e-12, atol=1e-12)
    c = np.full((1, 24), -3.0)
    np.testing.assert_allclose(oracle.rms_norm(c, w, 0.5), -3.0 / np.sqrt(9.5) * w[None, :], rtol=1e-14)


def test_rope_vs_complex_bruteforce_and_invariants():
    """Rotary embedding against a pure-Python complex rotation of each (i, i + D/2)
    pair by e^{i pos theta^(-2i/D)}; position 0 is the identity; norms are kept; the
    product of a rotated query and key depends only on the position difference."""
    rng = np.random.default_rng(12)
    m, heads, dh, theta = 5, 3, 8, 1.0e4
    x = rng.normal(size=(m, heads, dh))
    pos = np.array([0, 3, 17, 250, 40000])
    got = oracle.rope(x, pos, theta)
    for r in range(m):
        for hh in range(heads):
            for i in range(dh // 2):
                z = complex(x[r, hh, i], x[r, hh, i + dh // 2])
                z *= complex(math.cos(pos[r] * theta ** (-2 * i / dh)), math.sin(pos[r] * theta ** (-2 * i / dh)))
                assert abs(got[r, hh, i] - z.real) < 1e-12 and abs(got[r, hh, i + dh // 2] - z.imag) < 1e-12
    np.testing.assert_allclose(got[0], x[0], rtol=0, atol=0)
    np.testing.assert_allclose(np.linalg.norm(got, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    q, k = rng.normal(size=(1, 1, dh)), rng.normal(size=(1, 1, dh))
    d1 = (oracle.rope(q, [100], theta) * oracle.rope(k, [60], theta)).sum()
    d2 = (oracle.rope(q, [1040], theta) * oracle.rope(k, [1000], theta)).sum()
    assert abs(d1 - d2) < 1e-12


def _dense_case(seed, segs=(30, 1, 17), d=64, hq=4, hkv=2, dh=16, d_ff=96):
    from synthetic import make_dense_layer, make_kept_hidden
    w = make_dense_layer(d, hq, hkv, dh, d_ff, seed=seed, dtype=torch.float64)
    x = make_kept_hidden(list(segs), d, seed=seed + 1, dtype=torch.float64, n_query_tail=3)
    return w, x


def test_dense_layer_vs_torch_reference():
    """The layer against the same layer written with torch ops in fp64: torch's
    rms_norm, rotary embedding through complex multiplication of (i, i + D/2) pairs,
    SDPA with an additive float mask for the token-gated attention, torch's silu."""
    hq, hkv, dh = 4, 2, 16
    w, x = _dense_case(21)
    got = oracle.dense_layer(x["h"], x["pos"], x["bias"], x["seg_lens"], w, hq, hkv, dh)
    F = torch.nn.functional
    h = x["h"]
    m, d = h.shape
    eps = w["eps"]

    def rot(t):  # [m, heads, dh]
        half = dh // 2
        inv = torch.tensor(w["theta"], dtype=torch.float64) ** (-2.0 * torch.arange(half, dtype=torch.float64) / dh)
        ang = x["pos"].double()[:, None] * inv[None, :]
        z = torch.complex(t[..., :half], t[..., half:]) * torch.polar(torch.ones_like(ang), ang)[:, None, :]
        return torch.cat([z.real, z.imag], dim=-1)

    a = F.rms_norm(h, (d,), w["ln1"], eps=eps)
    qkv = a @ w["wqkv"].T
    q = rot(F.rms_norm(qkv[:, :hq * dh].reshape(m, hq, dh), (dh,), w["q_norm"], eps=eps))
    k = rot(F.rms_norm(qkv[:, hq * dh:(hq + hkv) * dh].reshape(m, hkv, dh), (dh,), w["k_norm"], eps=eps))
    v = qkv[:, (hq + hkv) * dh:].reshape(m, hkv, dh)
    o = torch.empty(m, hq, dh, dtype=torch.float64)
    off = 0
    for ln in x["seg_lens"]:
        sl = slice(off, off + ln)
        p = x["pos"][sl]
        for hh in range(hq):
            kv = hh // (hq // hkv)
            mask = torch.where(p[None, :] <= p[:, None], w["gain"][hh].double() * x["bias"][sl].double()[None, :],
                               torch.tensor(-math.inf, dtype=torch.float64))
            o[sl, hh] = F.scaled_dot_product_attention(q[None, None, sl, hh], k[None, None, sl, kv], v[None, None, sl, kv],
                                                       attn_mask=mask[None, None], scale=1.0 / (math.sqrt(dh) * w["tau"]))[0, 0]
        off += ln
    h2 = h + o.reshape(m, hq * dh) @ w["wo"].T
    a2 = F.rms_norm(h2, (d,), w["ln2"], eps=eps)
    out = h2 + (F.silu(a2 @ w["w_gate"].T) * (a2 @ w["w_up"].T)) @ w["w_down"].T
    np.testing.assert_allclose(got["q"], q.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["out"], out.numpy(), rtol=1e-10, atol=1e-11)


def test_dense_layer_residual_only_without_output_projections():
    """With zero output and down projections the layer returns its input."""
    hq, hkv, dh = 4, 2, 16
    w, x = _dense_case(22)
    w["wo"] = torch.zeros_like(w["wo"])
    w["w_down"] = torch.zeros_like(w["w_down"])
    got = oracle.dense_layer(x["h"], x["pos"], x["bias"], x["seg_lens"], w, hq, hkv, dh)
    np.testing.assert_array_equal(got["out"], x["h"].numpy())


# ------------------------------------------------------ gated delta rule ----

def test_delta_scan_vs_explicit_products():
    """Against the definition with the transition matrix written out:
    S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T, in pure Python lists."""
    rng = np.random.default_rng(41)
    segs, nh, dk, dv = [4, 3], 2, 3, 2
    m = sum(segs)
    q, k, v = rng.normal(size=(m, nh, dk)), rng.normal(size=(m, nh, dk)), rng.normal(size=(m, nh, dv))
    g, beta = np.log(rng.uniform(0.5, 1.0, size=(m, nh))), rng.uniform(0.0, 1.0, size=(m, nh))
    s0 = rng.normal(size=(2, nh, dv, dk))
    o, st = oracle.gated_delta_scan(q, k, v, g, beta, segs, state0=s0)
    off = 0
    for p, ln in enumerate(segs):
        for h in range(nh):
            sm = [[s0[p, h, i, j] for j in range(dk)] for i in range(dv)]
            for t in range(off, off + ln):
                a, b = math.exp(g[t, h]), beta[t, h]
                tr = [[(1.0 if i == j else 0.0) - b * k[t, h, i] * k[t, h, j] for j in range(dk)] for i in range(dk)]
                sm = [[a * sum(sm[i][r] * tr[r][j] for r in range(dk)) + b * v[t, h, i] * k[t, h, j]
                       for j in range(dk)] for i in range(dv)]
                for i in range(dv):
                    assert abs(o[t, h, i] - sum(sm[i][j] * q[t, h, j] for j in range(dk))) < 1e-12
            np.testing.assert_allclose(st[p, h], np.array(sm), rtol=1e-12, atol=1e-12)
        off += ln


def test_delta_scan_closed_forms():
    """beta = 0: the state only decays, o_t = exp(sum of g so far) S_0 q_t. Orthonormal keys
    with no decay and beta = 1: the delta rule stores each value exactly, so the final
    state maps key i to value i. One dimension: s_t = a (1 - b k^2) s + b v k."""
    rng = np.random.default_rng(42)
    nh, dk, dv, m = 1, 4, 3, 5
    q, k, v = rng.normal(size=(m, nh, dk)), rng.normal(size=(m, nh, dk)), rng.normal(size=(m, nh, dv))
    g = np.log(rng.uniform(0.6, 1.0, size=(m, nh)))
    s0 = rng.normal(size=(1, nh, dv, dk))
    o, _ = oracle.gated_delta_scan(q, k, v, g, np.zeros((m, nh)), [m], state0=s0)
    for t in range(m):
        np.testing.assert_allclose(o[t, 0], math.exp(g[: t + 1, 0].sum()) * s0[0, 0] @ q[t, 0], rtol=1e-12)
    basis = np.linalg.qr(rng.normal(size=(dk, dk)))[0].T  # orthonormal rows
    kk = basis[:, None, :]
    _, st = oracle.gated_delta_scan(kk, kk, v[:4], np.zeros((4, 1)), np.ones((4, 1)), [4])
    for i in range(4):
        np.testing.assert_allclose(st[0, 0] @ basis[i], v[i, 0], rtol=1e-12, atol=1e-12)
    q1, k1, v1 = rng.normal(size=(m, 1, 1)), rng.normal(size=(m, 1, 1)), rng.normal(size=(m, 1, 1))
    b1 = rng.uniform(0, 1, size=(m, 1))
    o1, _ = oracle.gated_delta_scan(q1, k1, v1, g, b1, [m])
    sv = 0.0
    for t in range(m):
        sv = math.exp(g[t, 0]) * (1 - b1[t, 0] * k1[t, 0, 0] ** 2) * sv + b1[t, 0] * v1[t, 0, 0] * k1[t, 0, 0]
        assert abs(o1[t, 0, 0] - sv * q1[t, 0, 0]) < 1e-12


def test_delta_scan_state_carries_across_calls():
    """A prompt split in two calls, the second starting from the first's final state,
    gives the outputs and final state of one call."""
    from synthetic import make_delta_inputs
    a = make_delta_inputs([20], 2, 8, 6, seed=43, dtype=torch.float64)
    full_o, full_s = oracle.gated_delta_scan(a["q"], a["k"], a["v"], a["g"], a["beta"], [20])
    o1, s1 = oracle.gated_delta_scan(a["q"][:7], a["k"][:7], a["v"][:7], a["g"][:7], a["beta"][:7], [7])
    o2, s2 = oracle.gated_delta_scan(a["q"][7:], a["k"][7:], a["v"][7:], a["g"][7:], a["beta"][7:], [13], state0=s1)
    np.testing.assert_allclose(np.concatenate([o1, o2]), full_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s2, full_s, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- decode ----

def _decode_case(seed, segs, hq, hkv, d, n_new_max=3, pos_ties=False):
    """Cache rows for `segs` (start, length, n_new) plus the new tokens' queries."""
    m = max(st + ln for st, ln, _ in segs)
    a = make_attention_inputs([m], hq, hkv, d, seed=seed, dtype=torch.float64, pos_ties=pos_ties)
    pos = np.zeros(m, dtype=np.int64)
    for st, ln, nn in segs:  # positions restart per sequence; new rows get bias 0
        pos[st:st + ln] = a["pos"].numpy()[:ln]
    bias = a["bias"].numpy().astype(np.float64)
    for st, ln, nn in segs:
        bias[st + ln - nn:st + ln] = 0.0
    r = sum(nn for _, _, nn in segs)
    q_new = torch.randn((r, hq, d), generator=torch.Generator().manual_seed(seed + 1), dtype=torch.float64)
    return q_new.numpy(), a["k"].numpy(), a["v"].numpy(), bias, pos, a["gain"].numpy().astype(np.float64)


@pytest.mark.parametrize("hq,hkv", [(4, 2), (3, 1), (2, 2)])
def test_decode_vs_bruteforce(hq, hkv):
    segs = [(0, 9, 1), (9, 5, 2), (14, 1, 1), (15, 7, 3)]
    q, k, v, b, pos, g = _decode_case(5, segs, hq, hkv, 4, pos_ties=True)
    o, lse = oracle.decode_attention(q, k, v, b, pos, segs, hq, hkv, g, 0.9)
    ob, lb = brute.decode_attention(q.tolist(), k.tolist(), v.tolist(), b.tolist(), pos.tolist(), segs,
                                    hq, hkv, g.tolist(), 0.9)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=1e-12, atol=1e-13)


def test_decode_vs_sdpa_library():
    """Each new token against its visible cache rows: torch SDPA (fp64) with
    the additive float mask gain[h]*bias[j] and -inf on invisible rows."""
    hq, hkv, d, tau = 4, 2, 16, 1.3
    segs = [(0, 40, 2), (40, 25, 1)]
    q, k, v, b, pos, g = _decode_case(11, segs, hq, hkv, d)
    o, _ = oracle.decode_attention(q, k, v, b, pos, segs, hq, hkv, g, tau)
    r = 0
    for st, ln, nn in segs:
        kk = torch.from_numpy(k[st:st + ln]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
        vv = torch.from_numpy(v[st:st + ln]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
        for t in range(nn):
            i = st + ln - nn + t
            vis = torch.from_numpy(pos[st:st + ln] <= pos[i])
            mask = torch.where(vis[None, None, :], torch.from_numpy(g)[:, None, None] * torch.from_numpy(b[st:st + ln])[None, None, :],
                               torch.tensor(-math.inf, dtype=torch.float64))
            qq = torch.from_numpy(q[r]).reshape(hq, 1, d)[None]
            ref = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask[None], scale=1.0 / (math.sqrt(d) * tau))
            np.testing.assert_allclose(o[r], ref[0, :, 0, :].numpy(), rtol=1e-12, atol=1e-12)
            r += 1


def test_decode_closed_forms():
    hq, hkv, d = 4, 2, 8
    segs = [(0, 30, 1), (30, 1, 1), (31, 12, 2)]
    q, k, v, b, pos, g = _decode_case(17, segs, hq, hkv, d)
    # V = 1 => O = 1
    o1, _ = oracle.decode_attention(q, k, np.ones_like(v), b, pos, segs, hq, hkv, g, 1.2)
    np.testing.assert_allclose(o1, 1.0, rtol=0, atol=1e-14)
    # a one-row cache: the new token sees only itself
    o, lse = oracle.decode_attention(q, k, v, b, pos, segs, hq, hkv, g, 1.2)
    for h in range(hq):
        np.testing.assert_allclose(o[1, h], v[30, (h * hkv) // hq], rtol=1e-14)
    # equal keys: weights exp(gain[h] * bias[j]), independent of q and tau
    kk = np.repeat(k[:1], k.shape[0], axis=0)
    for tau in (0.4, 5.0):
        o2, _ = oracle.decode_attention(q, kk, v, b, pos, segs, hq, hkv, g, tau)
        for h in range(hq):
            w = np.exp(g[h] * b[0:30])
            ref = (w[:, None] * v[0:30, (h * hkv) // hq]).sum(0) / w.sum()
            np.testing.assert_allclose(o2[0, h], ref, rtol=1e-12)


def test_decode_equals_prefill_last_rows():
    """Two independent routes to the same numbers: the new tokens' rows of a
    prefill over the cache (its queries filled in) equal the decode."""
    hq, hkv, d = 4, 2, 8
    segs = [(0, 21, 3), (21, 13, 1)]
    q, k, v, b, pos, g = _decode_case(23, segs, hq, hkv, d, pos_ties=True)
    m = 34
    qfull = np.zeros((m, hq, d))
    rows = []
    r = 0
    for st, ln, nn in segs:
        for t in range(nn):
            qfull[st + ln - nn + t] = q[r]
            rows.append(st + ln - nn + t)
            r += 1
    o, lse = oracle.decode_attention(q, k, v, b, pos, segs, hq, hkv, g, 1.1)
    of, lf = oracle.gated_attention(qfull, k, v, b, pos, [21, 13], hq, hkv, g, 1.1, rows=np.array(rows))
    np.testing.assert_allclose(o, of[rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lf[:, rows], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------- end to end ----

def test_tiny_layer_end_to_end_invariants():
    w = make_workload("tiny")
    lay = w.layers[0]
    res = oracle.gated_prefill(w.x, w.w1, w.w2, w.prompts, [lay], hq=w.hq, hkv=w.hkv,
                               head_dim=w.head_dim, decision_dtype=np.float32)
    kept = res["kept"]
    p = w.prompts[0]
    assert len(kept) == p.k_doc + (p.length - p.n_doc) == 176
    assert set(range(448, 512)) <= set(kept.tolist())
    o, lse = res["attn"][0]
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    # the kept set is the top-112 document rows by score
    s = res["scores"]
    kd = kept[kept < 448]
    assert np.min(s[kd]) >= np.max(np.delete(s[:448], kd))

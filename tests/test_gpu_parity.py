"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Each stage gets identical seeded synthetic inputs on both sides (the
oracle never sees a GPU output). Bars:
  select, compaction gathers, positions: bit-exact;
  fp32 scores and outputs: |diff| <= 1e-4;
  bf16 attention outputs: per (row, head) max|diff| <= 2e-2 * max|O_ref|;
  bf16 gate scores: |diff| <= 2e-2 * max|s_ref| over the prompt;
  bias: |diff| <= 1e-6 * max(1, |b|).
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import learned_token_pruning_layer_amd as tg
from learned_token_pruning_layer_amd._lib import seq_array
from synthetic import (Prompt, doc_budget, make_attention_inputs, make_ragged, make_scores,
                       make_workload, ragged_prompts)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def note(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().float().cpu().double().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().double().numpy()


def assert_rowmax_close(got, ref, rel=2e-2):
    """bf16 bar: per (row, head), max |got-ref| <= rel * max |ref|."""
    err = np.abs(got - ref).max(axis=-1)
    scale = np.abs(ref).max(axis=-1)
    bad = err > rel * scale
    assert not bad.any(), f"{bad.sum()} (row, head) pairs over the bar; worst ratio {np.max(err / np.maximum(scale, 1e-30)):.3e}"
    return float(np.max(err / np.maximum(scale, 1e-30)))


# ------------------------------------------------------------------ gate ----

def test_gate_fp32_tiny():
    note("gate fp32 tiny (N=512, d=256, H=64)")
    w = make_workload("tiny", device=DEV, with_layers=False)
    s = tg.tg_gate_score(w.x, w.w1, w.w2)
    ref = oracle.gate_scores(w.x.cpu(), w.w1.cpu(), w.w2.cpu())
    assert np.abs(f64(s) - ref).max() <= 1e-4


@pytest.mark.parametrize("n,d,h,with_b1", [(1000, 2048, 256, False), (65, 512, 128, True),
                                           (1, 2048, 256, True), (77, 320, 256, True), (300, 1088, 128, False),
                                           (200, 192, 64, False), (130, 100, 24, True), (70, 64, 256, True),
                                           (32769, 192, 256, True), (40001, 2048, 256, False),
                                           (33001, 128, 128, True), (1000, 2048, 192, True), (129, 1024, 192, False),
                                           (300, 512, 64, False), (40000, 256, 64, True)])
def test_gate_bf16(n, d, h, with_b1):
    note(f"gate bf16 n={n} d={d} h={h} b1={with_b1}")
    g = torch.Generator(device=DEV).manual_seed(n + d + h)
    x = torch.randn(n, d, generator=g, device=DEV).to(torch.bfloat16)
    w1 = (torch.randn(h, d, generator=g, device=DEV) / math.sqrt(d)).to(torch.bfloat16)
    w2 = (torch.randn(h, generator=g, device=DEV) / math.sqrt(h)).to(torch.bfloat16)
    b1 = (torch.randn(h, generator=g, device=DEV) * 0.5).to(torch.bfloat16) if with_b1 else None
    s = tg.tg_gate_score(x, w1, w2, b1, b2=0.375)
    ref = oracle.gate_scores(x.cpu(), w1.cpu(), w2.cpu(), None if b1 is None else b1.cpu(), 0.375)
    err = np.abs(f64(s) - ref)
    assert err.max() <= 2e-2 * np.abs(ref).max()
    # fp32 accumulation of exact bf16 products: far inside the bar
    assert err.max() <= 1e-3 * max(1.0, np.abs(ref).max())


def test_gate_bf16_qwen16k_sampled():
    note("gate bf16 qwen16k full size, 1024 sampled rows + planted rows")
    w = make_workload("qwen16k", device=DEV, with_layers=False)
    s = f64(tg.tg_gate_score(w.x, w.w1, w.w2))
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([rng.choice(w.n_rows, 1024, replace=False), w.planted, [w.n_rows - 1]]))
    ref = oracle.gate_scores(w.x[torch.as_tensor(rows, device=DEV)].cpu(), w.w1.cpu(), w.w2.cpu())
    assert np.abs(s[rows] - ref).max() <= 2e-2 * np.abs(ref).max()
    # planted rows rank first
    assert set(np.argsort(-s, kind="stable")[:16].tolist()) == set(w.planted.tolist())


# ---------------------------------------------------------------- select ----

def check_select(scores, prompts):
    got = tg.tg_select_topk(scores.to(DEV), prompts).cpu().numpy()
    ref = oracle.select_topk(scores.cpu().numpy(), prompts)
    assert got.dtype == np.int32
    assert np.array_equal(got.astype(np.int64), ref), "kept index set or order differs"


@pytest.mark.parametrize("kind", ["normal", "ties", "few", "signed0", "wide"])
def test_select_single_prompt(kind):
    note(f"select 16384 rows kind={kind}")
    s = make_scores(16384, seed=3, kind=kind)
    for k in (0, 1, 2, 1000, 2000, 15999, 16000):
        check_select(s, [Prompt(0, 16384, 0, 16000, k)])


def test_select_slice_edges():
    # A prompt of up to 32768 rows is ranked in 16 slices (1024 or 2048 rows,
    # one per workgroup): document edges on slice boundaries, runs of tied
    # keys crossing many slices, last slices of one row, and prompts at
    # unaligned offsets in one batch.
    note("select slices: document edges on slice boundaries, ties across slices, one-row last slices")
    s = make_scores(16384, seed=70, kind="few")
    doc = s[1024:15360]
    n1, n0 = int((doc == 1.0).sum()), int((doc == 0.0).sum())
    for k in (1, n1 - 1, n1, n1 + 1, n1 + n0 // 2, n1 + n0, 14335):
        check_select(s, [Prompt(0, 16384, 1024, 15360, k)])
    s = make_scores(4097, seed=71, kind="ties")
    for k in (1, 2048, 4096):
        check_select(s, [Prompt(0, 4097, 0, 4097, k)])
    s = make_scores(32768, seed=72, kind="few")
    for k in (3, 12000, 28671):
        check_select(s, [Prompt(0, 32768, 2048, 30720, k)])
    s = make_scores(60000, seed=73, kind="ties")
    check_select(s, [Prompt(7, 2049, 1, 2048, 1000), Prompt(2056, 1025, 1024, 1025, 1),
                     Prompt(3081, 20000, 3000, 19000, 4321), Prompt(23081, 32767, 0, 32767, 32766)])


def test_select_nan_inf_and_spans():
    note("select NaN/inf, inner document span")
    s = make_scores(5000, seed=5)
    s[::7] = float("nan")
    s[3::11] = float("inf")
    s[5::13] = -float("inf")
    s[10:20] = -0.0
    s[20:30] = 0.0
    # 480 of the 4000 document rows stay NaN (they rank last): budgets above
    # 3520 put the threshold among the NaN rows (key 0).
    for k in (0, 17, 1000, 2500, 3519, 3520, 3521, 3700, 3999, 4000):
        check_select(s, [Prompt(0, 5000, 300, 4300, k)])


@pytest.mark.parametrize("n", [16384, 16385, 32768, 32769])
def test_select_path_boundaries(n):
    # Prompt lengths at the edges of the 16-row and 32-row register paths
    # and the multi-workgroup path; a NaN-heavy document puts some thresholds at
    # key 0, where rows outside the document share the digit.
    note(f"select boundary prompt of {n} rows")
    s = make_scores(n, seed=40 + n % 7, kind="ties")
    s[1::9] = float("nan")
    n_doc = n - 150
    nan_doc = int(torch.isnan(s[100:n - 50]).sum())
    for k in (1, n_doc // 3, n_doc - nan_doc - 1, n_doc - nan_doc, n_doc - nan_doc // 2, n_doc - 1):
        check_select(s, [Prompt(0, n, 100, n - 50, k)])


def test_select_multi_prompt_edges():
    note("select multi-prompt: empty prompt, all-question prompt, tiny prompts")
    s = make_scores(7000, seed=8, kind="ties")
    prompts = [Prompt(0, 1, 0, 1, 1), Prompt(1, 0, 0, 0, 0), Prompt(1, 300, 0, 0, 0),
               Prompt(301, 2500, 100, 2400, 123), Prompt(2801, 3, 1, 2, 0), Prompt(2804, 4196, 0, 4000, 4000),
               Prompt(7000, 0, 0, 0, 0)]
    check_select(s, prompts)


def test_select_exhaustive_tiny_on_gpu():
    note("select exhaustive {0,1,2}^5 with every budget (batched as prompts)")
    import itertools
    vals = [np.array(v, dtype=np.float32) for v in itertools.product((0.0, 1.0, 2.0), repeat=5)]
    for k in range(6):
        batch = vals[:60]
        for i0 in range(0, len(vals), 60):
            batch = vals[i0:i0 + 60]
            s = torch.from_numpy(np.concatenate(batch))
            prompts = [Prompt(5 * i, 5, 0, 5, k) for i in range(len(batch))]
            check_select(s, prompts)


def test_select_long128k_and_ragged():
    note("select 131072 rows (keep 8128) and 8 ragged prompts")
    s = make_scores(131072, seed=12)
    check_select(s, [Prompt(0, 131072, 0, 130048, 8128)])
    prompts = ragged_prompts()
    n = prompts[-1].start + prompts[-1].length
    check_select(make_scores(n, seed=13, kind="ties"), prompts)


def test_select_multi_workgroup_path():
    # Prompts above 32768 rows: chunks of 16384 rows meet in a workspace.
    # Ties, NaN thresholds (key 0), chunk-boundary lengths, a small document
    # inside a long prompt, keep-none / keep-all, and long prompts mixed with
    # short ones in one call.
    note("select multi-workgroup: ties, NaN thresholds, chunk edges, mixed batch")
    s = make_scores(49153, seed=60, kind="ties")
    s[2::5] = float("nan")
    n_doc = 49153 - 200
    nan_doc = int(torch.isnan(s[150:49103]).sum())
    for k in (0, 1, 7777, n_doc - nan_doc - 1, n_doc - nan_doc, n_doc - nan_doc + 1, n_doc - 1, n_doc):
        check_select(s, [Prompt(0, 49153, 150, 49103, k)])
    for n in (32770, 49152, 65536, 65537):
        check_select(make_scores(n, seed=n, kind="few"), [Prompt(0, n, 0, n - 1, n // 3)])
    s = make_scores(200000, seed=61, kind="signed0")
    check_select(s, [Prompt(3, 70000, 30000, 30100, 50)])
    prompts = [Prompt(0, 100, 0, 50, 10), Prompt(100, 40000, 0, 38000, 3000), Prompt(40100, 16384, 0, 16000, 10),
               Prompt(56500, 98304, 1000, 98000, 70000), Prompt(154804, 32768, 0, 32000, 5),
               Prompt(187572, 0, 0, 0, 0), Prompt(187572, 12000, 0, 0, 0)]
    check_select(make_scores(199572, seed=62, kind="ties"), prompts)


def test_select_workspace_reuse_and_2p24():
    # A caller-provided workspace holding garbage, reused across calls with
    # different tables; then one prompt of 2^24 rows (1024 chunks).
    note("select workspace reuse; one prompt of 2^24 rows")
    lib = tg.load()
    p1 = [Prompt(0, 90000, 0, 89000, 4444)]
    p2 = [Prompt(0, 40000, 10, 39990, 39000), Prompt(40000, 50000, 0, 50000, 1)]
    need = max(lib.tg_select_workspace_bytes(seq_array(p), len(p)) for p in (p1, p2))
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV)
    s = make_scores(90000, seed=63, kind="ties")
    for p in (p1, p2, p1):
        got = tg.tg_select_topk(s.to(DEV), p, workspace=ws).cpu().numpy()
        assert np.array_equal(got.astype(np.int64), oracle.select_topk(s.numpy(), p))
    n = 1 << 24
    check_select(make_scores(n, seed=64), [Prompt(0, n, 0, n - 4096, 1 << 20)])


# --------------------------------------------------------------- compact ----

@pytest.mark.parametrize("n_tensors", [5, 0])
def test_compact_bit_exact_and_bias(n_tensors):
    note(f"compact: {n_tensors} tensors, positions, bias")
    prompts = [Prompt(0, 3000, 50, 2900, 400), Prompt(3000, 1000, 0, 744, 100), Prompt(4000, 64, 0, 0, 0)]
    n = 4064
    s = make_scores(n, seed=21) * 4
    kept = torch.from_numpy(oracle.select_topk(s.numpy(), prompts).astype(np.int32))
    g = torch.Generator(device=DEV).manual_seed(1)
    ts = [torch.randn(n, 2048, generator=g, device=DEV).to(torch.bfloat16),
          torch.randn(n, 16, 128, generator=g, device=DEV).to(torch.bfloat16),
          torch.randn(n, 8, 128, generator=g, device=DEV).to(torch.bfloat16),
          torch.randn(n, 4, generator=g, device=DEV),
          torch.randint(-2**31, 2**31 - 1, (n, 12), generator=g, device=DEV, dtype=torch.int32)][:n_tensors]
    pos = torch.randint(0, 10**6, (n,), generator=g, device=DEV, dtype=torch.int32)
    kd = kept.to(DEV)
    for use_pos in (False, True):
        outs, pk, bias = tg.tg_compact(kd, prompts, ts, pos=pos if use_pos else None, scores=s.to(DEV))
        (r_ts), r_pos, r_bias = oracle.compact(kept.numpy().astype(np.int64), prompts,
                                               [t.cpu() for t in ts], s.numpy(),
                                               pos.cpu().numpy() if use_pos else None)
        for o, r in zip(outs, r_ts):
            assert torch.equal(o.cpu(), r)
        assert np.array_equal(pk.cpu().numpy().astype(np.int64), r_pos)
        b = bias.cpu().double().numpy()
        assert np.all(np.abs(b - r_bias) <= 1e-6 * np.maximum(1.0, np.abs(r_bias)))
        assert np.all(b[np.asarray(r_bias) == 0.0] == 0.0)


def test_compact_full_budget_identity():
    note("compact at 100% budget is the identity")
    n = 1000
    prompts = [Prompt(0, n, 0, 900, 900)]
    kept = tg.tg_select_topk(make_scores(n, seed=2).to(DEV), prompts)
    x = torch.randn(n, 256, device=DEV)
    (xk,), pk, _ = tg.tg_compact(kept, prompts, [x])
    assert torch.equal(xk, x) and torch.equal(pk.cpu(), torch.arange(n, dtype=torch.int32))


# ------------------------------------------------------------- attention ----

def run_attention(a, hq, hkv, tau=1.2, want_lse=True):
    segs = a["seg_lens"]
    prompts, st = [], 0
    for ln in segs:
        prompts.append(Prompt(st, ln, 0, 0, 0))
        st += ln
    return tg.tg_gated_attention(a["q"].to(DEV), a["k"].to(DEV), a["v"].to(DEV), a["bias"].to(DEV),
                                 a["pos"].to(DEV), prompts, a["gain"].to(DEV), tau, want_lse=want_lse)


def ref_attention(a, hq, hkv, tau=1.2, rows=None):
    return oracle.gated_attention(a["q"], a["k"], a["v"], a["bias"], a["pos"].numpy(), a["seg_lens"],
                                  hq, hkv, a["gain"], tau, rows=rows)


@pytest.mark.parametrize("segs,hq,hkv,d", [([176], 4, 2, 64), ([1, 40, 100, 33], 4, 2, 64),
                                           ([130], 3, 1, 128), ([97], 8, 2, 64)])
def test_attention_fp32(segs, hq, hkv, d):
    note(f"attention fp32 segs={segs} hq={hq} hkv={hkv} d={d}")
    a = make_attention_inputs(segs, hq, hkv, d, seed=sum(segs), dtype=torch.float32, n_query_tail=7)
    o, lse = run_attention(a, hq, hkv)
    ro, rl = ref_attention(a, hq, hkv)
    assert np.abs(f64(o) - ro).max() <= 1e-4
    assert np.abs(f64(lse) - rl).max() <= 1e-4


BF16_CASES = [
    ([2384], 16, 8, 128, False),          # the 16k layer's kept set
    ([1200, 1000, 300], 16, 8, 128, False),  # 640 work items over three prompts
    ([1, 31, 64, 65, 200], 16, 8, 128, False),
    ([300, 129], 16, 8, 128, True),       # repeated positions
    ([257], 8, 8, 128, False),            # no GQA (G = 1)
    ([190], 16, 4, 128, False),           # G = 4
    ([150, 77], 12, 4, 64, False),        # G = 3, head_dim 64
    ([500], 4, 2, 64, True),
]


# A call whose longest prompt keeps at least 4096 rows runs the long-prompt
# kernel shape (two 32-row slabs share every K/V tile, no key split) for all
# of its prompts; these cases put ragged short prompts, repeated positions,
# every head ratio and D = 64 through that shape.
LONG_SHAPE_CASES = [
    ([4100, 1, 31, 65, 200], 16, 8, 128, False),
    ([4097, 129], 16, 8, 128, True),
    ([4160], 8, 8, 128, False),           # G = 1
    ([4150, 77], 12, 4, 64, False),       # G = 3, head_dim 64
    ([4096, 63], 16, 4, 128, False),      # G = 4
    ([4133], 4, 2, 64, True),
]


def attention_rows_sample(segs, seed, n_rand=192):
    """Every row of prompts under 300 rows; for longer ones, random rows plus the
    edges of the 32/64-row query blocks and 32-key tiles around a few places."""
    rng = np.random.default_rng(seed)
    rows, off = [], 0
    for ln in segs:
        if ln < 300:
            rows.append(np.arange(off, off + ln))
        else:
            edges = [e + d for e in (0, 32, 64, 128, ln // 2 // 64 * 64, ln - ln % 64, ln - 64) for d in (-1, 0, 1)]
            edges = [off + e for e in edges if 0 <= e < ln] + [off + ln - 1]
            rows.append(np.concatenate([off + rng.choice(ln, n_rand, replace=False), edges]))
        off += ln
    return np.unique(np.concatenate(rows))


@pytest.mark.parametrize("segs,hq,hkv,d,ties", BF16_CASES + LONG_SHAPE_CASES)
def test_attention_bf16(segs, hq, hkv, d, ties):
    note(f"attention bf16 segs={segs} hq={hq} hkv={hkv} d={d} ties={ties}")
    a = make_attention_inputs(segs, hq, hkv, d, seed=len(segs) * 7 + hq + sum(segs) % 97, dtype=torch.bfloat16,
                              n_query_tail=16, pos_ties=ties)
    o, lse = run_attention(a, hq, hkv)
    rows = attention_rows_sample(segs, seed=hq + d) if sum(segs) > 3000 else None
    ro, rl = ref_attention(a, hq, hkv, rows=rows)
    sel = np.arange(sum(segs)) if rows is None else rows
    worst = assert_rowmax_close(f64(o)[sel], ro[sel])
    note(f"  worst rel-to-row-max error {worst:.2e} over {len(sel)} rows")
    assert np.abs(f64(lse)[:, sel] - rl[:, sel]).max() <= 2e-2 * max(1.0, np.abs(rl[:, sel]).max())


def test_attention_bf16_sharp_logits():
    note("attention bf16 with large logits (online softmax rescaling)")
    a = make_attention_inputs([700], 16, 8, 128, seed=99, dtype=torch.bfloat16, qk_std=3.0)
    o, _ = run_attention(a, 16, 8, tau=0.5)
    ro, _ = ref_attention(a, 16, 8, tau=0.5)
    assert_rowmax_close(f64(o), ro)


def test_attention_ones_and_first_row():
    note("attention closed forms: V=1 gives 1; a prompt's first row returns its own V")
    a = make_attention_inputs([333, 64], 16, 8, 128, seed=5, dtype=torch.bfloat16)
    a1 = dict(a)
    a1["v"] = torch.ones_like(a["v"])
    o, _ = run_attention(a1, 16, 8)
    assert np.abs(f64(o) - 1.0).max() <= 1e-2
    o, _ = run_attention(a, 16, 8)
    for off in (0, 333):
        for h in range(16):
            assert torch.equal(o[off, h].cpu(), a["v"][off, h // 2])


def test_attention_reduces_to_sdpa_full_budget_zero_gain():
    note("attention at full budget with zero gain equals causal SDPA (fp32 CPU)")
    m, hq, hkv, d = 600, 16, 8, 128
    a = make_attention_inputs([m], hq, hkv, d, seed=17, dtype=torch.bfloat16)
    a["pos"] = torch.arange(m, dtype=torch.int32)
    a["gain"] = torch.zeros(hq)
    o, _ = run_attention(a, hq, hkv, tau=1.0)
    q = a["q"].float().permute(1, 0, 2)[None]
    k = a["k"].float().permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None].contiguous()
    v = a["v"].float().permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None].contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=1 / math.sqrt(d))
    assert_rowmax_close(f64(o), ref[0].permute(1, 0, 2).double().numpy())


@pytest.mark.parametrize("m", [9152, 17000], ids=["long-shape", "xl-shape"])
def test_attention_bf16_long_sampled(m):
    note(f"attention bf16 long kept set (M={m}), 128 sampled query rows")
    a = make_attention_inputs([m], 16, 8, 128, seed=31, dtype=torch.bfloat16, n_query_tail=1024)
    o, lse = run_attention(a, 16, 8)
    rows = np.unique(np.concatenate([np.random.default_rng(1).choice(m, 120, replace=False),
                                     [0, 1, 63, 64, m - 1]]))
    ro, rl = ref_attention(a, 16, 8, rows=rows)
    assert_rowmax_close(f64(o)[rows], ro[rows])


@pytest.mark.parametrize("segs", [[1000, 23], [2384], [1200, 1000, 300], [4200, 23, 1], [16500, 23, 1]],
                         ids=["short-shape", "short-shape-600-items", "short-shape-640-items-ragged", "long-shape",
                              "xl-shape"])
def test_attention_deterministic_and_fully_written(segs):
    note(f"attention determinism and poisoned-output check, prompts {segs}")
    a = make_attention_inputs(segs, 16, 8, 128, seed=3, dtype=torch.bfloat16)
    prompts, st = [], 0
    for ln in segs:
        prompts.append(Prompt(st, ln, 0, 0, 0))
        st += ln
    m = sum(segs)
    args = [a[n].to(DEV) for n in ("q", "k", "v", "bias", "pos")]
    out1 = torch.full_like(args[0], float("nan"))
    lse1 = torch.full((16, m), float("nan"), device=DEV)
    tg.tg_gated_attention(*args, prompts, a["gain"].to(DEV), 1.2, out=out1, want_lse=True, lse=lse1)
    out2, lse2 = tg.tg_gated_attention(*args, prompts, a["gain"].to(DEV), 1.2, want_lse=True)
    assert not torch.isnan(out1).any() and not torch.isnan(lse1).any()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


# ------------------------------------------------------------ end to end ----

def run_layer(w, layers=None):
    lay = tg.GatedPrefillLayer(w.x, w.w1, w.w2, w.prompts, w.layers if layers is None else layers,
                               w.hq, w.hkv, w.head_dim, want_lse=True)
    lay.run()
    torch.cuda.synchronize()
    return lay


def test_end_to_end_tiny_fp32():
    note("end to end: tiny fp32 layer (N=512, keep 112 + 64 query)")
    w = make_workload("tiny", device=DEV)
    lay = run_layer(w)
    wl = w.layers[0]
    ref = oracle.gated_prefill(w.x.cpu(), w.w1.cpu(), w.w2.cpu(), w.prompts,
                               [type("L", (), dict(q=wl.q.cpu(), k=wl.k.cpu(), v=wl.v.cpu(), gain=wl.gain.cpu(), tau=wl.tau))],
                               hq=w.hq, hkv=w.hkv, head_dim=w.head_dim, decision_dtype=np.float32)
    assert np.abs(f64(lay.scores) - ref["scores"]).max() <= 1e-4
    # the decision is taken on fp32 scores on both sides
    ref_kept_gpu_scores = oracle.select_topk(lay.scores.cpu().numpy(), w.prompts)
    assert np.array_equal(lay.kept.cpu().numpy().astype(np.int64), ref_kept_gpu_scores)
    assert np.array_equal(lay.kept.cpu().numpy().astype(np.int64), ref["kept"])
    assert np.array_equal(lay.pos_kept.cpu().numpy(), ref["pos_kept"])
    assert np.abs(f64(lay.bias_kept) - ref["bias"]).max() <= 1e-4
    o, lse = ref["attn"][0]
    assert np.abs(f64(lay.outs[0]) - o).max() <= 1e-4
    assert torch.equal(lay.hidden_kept.cpu(), w.x.cpu()[torch.as_tensor(ref["kept"])])


def test_end_to_end_qwen16k():
    note("end to end: qwen16k bf16 layer (N=16384, keep 2000 + 384 query)")
    w = make_workload("qwen16k", device=DEV)
    lay = run_layer(w)
    wl = w.layers[0]
    s_ref = oracle.gate_scores(w.x.cpu(), w.w1.cpu(), w.w2.cpu())
    s_gpu = f64(lay.scores)
    assert np.abs(s_gpu - s_ref).max() <= 2e-2 * np.abs(s_ref).max()
    kept = lay.kept.cpu().numpy().astype(np.int64)
    ref_kept = oracle.select_topk(s_ref.astype(np.float32), w.prompts)
    flipped = np.array(sorted(set(kept.tolist()) ^ set(ref_kept.tolist())), dtype=np.int64)
    note(f"  threshold flips vs fp64-gate selection: {len(flipped)}")
    # A row can only change sides if its score is near the threshold: the k-th
    # largest score moves by at most max|ds| (order statistics are 1-Lipschitz),
    # so a flipped row's fp64 score lies within 2 max|ds| of the fp64 threshold.
    p0 = w.prompts[0]
    doc = np.arange(p0.start + p0.doc_begin, p0.start + p0.doc_end)
    d_max = np.abs(s_gpu[doc] - s_ref[doc]).max()
    thr = np.sort(s_ref[doc].astype(np.float32).astype(np.float64))[::-1][p0.k_doc - 1]
    if len(flipped):
        assert np.all(np.abs(s_ref[flipped] - thr) <= 2 * d_max + 1e-7), (flipped, s_ref[flipped], thr, d_max)
    # identical scores give identical selection
    assert np.array_equal(kept, oracle.select_topk(lay.scores.cpu().numpy(), w.prompts))
    assert set(w.planted.tolist()) <= set(kept.tolist())
    assert set(range(16000, 16384)) <= set(kept.tolist())
    # attention against the oracle on the GPU's kept set (same compaction)
    (qk, kk, vk), pk, bk = oracle.compact(kept, w.prompts, (wl.q.cpu(), wl.k.cpu(), wl.v.cpu()),
                                          s_ref, None)
    assert torch.equal(lay.qkv_kept[0][0].cpu(), qk) and torch.equal(lay.qkv_kept[0][2].cpu(), vk)
    assert np.array_equal(lay.pos_kept.cpu().numpy(), pk)
    m = len(kept)
    o, _ = oracle.gated_attention(qk.view(m, 16, 128), kk.view(m, 8, 128), vk.view(m, 8, 128), bk, pk,
                                  [m], 16, 8, wl.gain.cpu(), wl.tau)
    assert_rowmax_close(f64(lay.outs[0]), o)


def test_end_to_end_sweep32k_full_budget_is_unpruned():
    note("sweep32k at 100% budget and zero gain: equals unpruned causal attention")
    w = make_workload("sweep32k", device=DEV, k_doc=doc_budget(1.0, 32256))
    wl = w.layers[0]
    wl.gain = torch.zeros_like(wl.gain)
    lay = run_layer(w)
    assert torch.equal(lay.kept.cpu(), torch.arange(32768, dtype=torch.int32))
    n = 32768
    # 64 random rows plus the edges of the 32-row query blocks and 32-key tiles
    edges = [0, 1, 31, 32, 33, 63, 64, 65, 4095, 4096, 16383, 16384, 32735, 32736, 32766, 32767]
    rows = np.unique(np.concatenate([np.random.default_rng(3).choice(n, 64, replace=False), edges]))
    o, _ = oracle.gated_attention(wl.q.cpu().view(n, 16, 128), wl.k.cpu().view(n, 8, 128),
                                  wl.v.cpu().view(n, 8, 128), np.zeros(n), np.arange(n), [n], 16, 8,
                                  np.zeros(16), wl.tau, rows=rows)
    assert_rowmax_close(f64(lay.outs[0])[rows], o[rows])


def check_layer_sampled(w, n_attn_rows=64, seed=0):
    """Whole layer on the GPU against the oracle: the selection exactly (the
    decision taken on the GPU's fp32 scores on both sides), the gate on every
    kept row, the compaction bit-exactly, attention on sampled kept rows."""
    lay = run_layer(w)
    kept = lay.kept.cpu().numpy().astype(np.int64)
    assert np.array_equal(kept, oracle.select_topk(lay.scores.cpu().numpy(), w.prompts))
    ks = set(kept.tolist())
    assert set(w.planted.tolist()) <= ks
    for p in w.prompts:  # the question is never pruned
        assert set(range(p.start + p.doc_end, p.start + p.length)) <= ks
    s_kept = oracle.gate_scores(w.x[torch.as_tensor(kept, device=DEV)].cpu(), w.w1.cpu(), w.w2.cpu())
    smax = np.abs(s_kept).max()
    assert np.abs(f64(lay.scores)[kept] - s_kept).max() <= 2e-2 * smax
    scores = np.full(w.n_rows, np.nan)
    scores[kept] = s_kept
    wl = w.layers[0]
    (qk, kk, vk), pk, bk = oracle.compact(kept, w.prompts, (wl.q.cpu(), wl.k.cpu(), wl.v.cpu()), scores)
    for got, ref in zip(lay.qkv_kept[0], (qk, kk, vk)):
        assert torch.equal(got.cpu(), ref)
    assert torch.equal(lay.hidden_kept.cpu(), w.x.cpu()[torch.as_tensor(kept)])
    assert np.array_equal(lay.pos_kept.cpu().numpy(), pk)
    # log-sigmoid is 1-Lipschitz: the bias can differ by at most the score difference
    assert np.abs(f64(lay.bias_kept) - bk).max() <= 2e-2 * smax
    m = len(kept)
    rows = np.unique(np.concatenate([np.random.default_rng(seed).choice(m, n_attn_rows, replace=False), [0, m - 1]]))
    hq, hkv, dh = w.hq, w.hkv, w.head_dim
    o, _ = oracle.gated_attention(qk.view(m, hq, dh), kk.view(m, hkv, dh), vk.view(m, hkv, dh), bk, pk,
                                  [p.n_kept for p in w.prompts], hq, hkv, wl.gain.cpu(), wl.tau, rows=rows)
    assert_rowmax_close(f64(lay.outs[0])[rows], o[rows])


@pytest.mark.parametrize("frac", [0.05, 0.10, 0.25, 0.50])
def test_end_to_end_sweep32k_budgets(frac):
    note(f"end to end: sweep32k at a {frac:.0%} document budget (sampled attention rows)")
    w = make_workload("sweep32k", device=DEV, k_doc=doc_budget(frac, 32256))
    check_layer_sampled(w)


def test_end_to_end_long128k_sampled():
    note("end to end: long128k (N=131072, keep 8128 + 1024 query), sampled attention rows")
    w = make_workload("long128k", device=DEV)
    check_layer_sampled(w)


def test_end_to_end_ragged_four_layers():
    """8 ragged prompts feeding 4 above-gate layers: one gate, select and compaction
    (13 gathered tensors: the hidden states and every layer's Q, K, V), then one
    attention call per layer. The selection is checked exactly on the GPU's scores,
    the compaction against the oracle's own gathers of the original tensors
    (bit-exact; bias from the same scores within 1e-6 relative), and each layer's
    attention on sampled rows against the oracle fed the oracle's compacted tensors."""
    note("end to end: ragged 8 prompts, 4 above-gate layers (13 gathered tensors, sampled rows)")
    prompts = [Prompt(p.start, p.length, p.doc_begin, p.doc_end, p.k_doc) for p in ragged_prompts()]
    w = make_ragged(device=DEV)
    lay = run_layer(w)
    kept = lay.kept.cpu().numpy().astype(np.int64)
    s_gpu = lay.scores.cpu().numpy()
    assert np.array_equal(kept, oracle.select_topk(s_gpu, prompts))
    s_ref_rows = np.random.default_rng(0).choice(w.n_rows, 512, replace=False)
    s_ref = oracle.gate_scores(w.x[torch.as_tensor(s_ref_rows, device=DEV)].cpu(), w.w1.cpu(), w.w2.cpu())
    assert np.abs(s_gpu[s_ref_rows] - s_ref).max() <= 2e-2 * np.abs(s_ref).max()
    (hk,), pk, bk = oracle.compact(kept, prompts, (w.x.cpu(),), s_gpu)
    assert torch.equal(lay.hidden_kept.cpu(), hk)
    assert np.array_equal(lay.pos_kept.cpu().numpy().astype(np.int64), pk)
    b = f64(lay.bias_kept)
    assert np.all(np.abs(b - bk) <= 1e-6 * np.maximum(1.0, np.abs(bk)))
    assert np.all(b[bk == 0.0] == 0.0)
    del hk
    seg = [p.n_kept for p in prompts]
    m = len(kept)
    rows = np.random.default_rng(2).choice(m, 64, replace=False)
    for i, wl in enumerate(w.layers):
        (qk, kk, vk), _, _ = oracle.compact(kept, prompts, (wl.q.cpu(), wl.k.cpu(), wl.v.cpu()))
        for got, ref in zip(lay.qkv_kept[i], (qk, kk, vk)):
            assert torch.equal(got.cpu(), ref)
        o, _ = oracle.gated_attention(qk.view(m, 16, 128), kk.view(m, 8, 128), vk.view(m, 8, 128), bk, pk,
                                      seg, 16, 8, wl.gain.cpu(), wl.tau, rows=rows)
        assert_rowmax_close(f64(lay.outs[i])[rows], o[rows])
        del qk, kk, vk


def test_end_to_end_long128k_unpruned_sampled():
    """The long128k prompt with every document row kept (the unpruned comparison
    run): the kept set is every row, the compaction the identity, and the attention
    over all 131072 rows matches the oracle on 64 sampled query rows plus block
    edges."""
    note("end to end: long128k with every row kept (attention over 131072 rows), sampled rows")
    w = make_workload("long128k", device=DEV)
    p0 = w.prompts[0]
    w.prompts = [p0._replace(k_doc=p0.n_doc)]
    lay = run_layer(w)
    n = w.n_rows
    assert torch.equal(lay.kept.cpu(), torch.arange(n, dtype=torch.int32))
    s_gpu = lay.scores.cpu().numpy()
    _, pk, bk = oracle.compact(np.arange(n), w.prompts, (), s_gpu)
    assert np.array_equal(lay.pos_kept.cpu().numpy().astype(np.int64), pk)
    assert np.all(np.abs(f64(lay.bias_kept) - bk) <= 1e-6 * np.maximum(1.0, np.abs(bk)))
    wl = w.layers[0]
    for got, src in zip(lay.qkv_kept[0], (wl.q, wl.k, wl.v)):
        assert torch.equal(got, src)
    edges = [0, 1, 31, 32, 8191, 8192, 65535, 65536, 130047, 130048, n - 33, n - 32, n - 1]
    rows = np.unique(np.concatenate([np.random.default_rng(4).choice(n, 64, replace=False), edges]))
    rt = torch.as_tensor(rows)
    o, _ = oracle.gated_attention(wl.q.cpu().view(n, 16, 128), wl.k.cpu().view(n, 8, 128),
                                  wl.v.cpu().view(n, 8, 128), bk, pk, [n], 16, 8, wl.gain.cpu(), wl.tau, rows=rows)
    assert_rowmax_close(f64(lay.outs[0][rt.to(DEV)]), o[rows])


# ---------------------------------------------------------------- decode ----

def decode_inputs(segs, hq, hkv, d, seed, dtype=torch.bfloat16, pos_ties=False):
    """A KV cache holding `segs` (start, len, n_new); the new rows carry bias 0."""
    rows = max(st + ln for st, ln, _ in segs)
    a = make_attention_inputs([rows], hq, hkv, d, seed=seed, dtype=dtype, pos_ties=pos_ties)
    pos = torch.zeros(rows, dtype=torch.int32)
    bias = a["bias"].clone()
    for st, ln, nn in segs:
        pos[st:st + ln] = a["pos"][:ln]
        bias[st + ln - nn:st + ln] = 0.0
    r = sum(nn for _, _, nn in segs)
    gq = torch.Generator().manual_seed(seed + 7)
    q_new = torch.randn((r, hq, d), generator=gq).to(dtype)
    return q_new, a["k"], a["v"], bias, pos, a["gain"]


def check_decode(segs, hq, hkv, d, seed, dtype=torch.bfloat16, pos_ties=False, tau=1.2):
    q, k, v, bias, pos, gain = decode_inputs(segs, hq, hkv, d, seed, dtype, pos_ties)
    out, lse = tg.tg_decode_attention(q.to(DEV), k.to(DEV), v.to(DEV), bias.to(DEV), pos.to(DEV), segs,
                                      gain.to(DEV), tau, want_lse=True)
    ref, ref_lse = oracle.decode_attention(f64(q), f64(k), f64(v), f64(bias), pos.numpy(), segs, hq, hkv,
                                           f64(gain), tau)
    got = f64(out)
    if dtype == torch.bfloat16:
        assert_rowmax_close(got, ref)
    else:
        assert np.abs(got - ref).max() <= 1e-4
    assert np.abs(f64(lse) - ref_lse).max() <= 1e-3 * max(1.0, np.abs(ref_lse).max())
    return out


def test_decode_qwen_shapes_single_and_ragged():
    note("decode bf16 16/8 heads D=128: one 9152-row cache, then ragged caches with 1..4 new tokens")
    check_decode([(0, 9152, 1)], 16, 8, 128, seed=1)
    check_decode([(0, 1, 1), (1, 33, 2), (34, 1000, 3), (1034, 5000, 4), (6034, 77, 1)], 16, 8, 128, seed=2)


@pytest.mark.parametrize("hq,hkv,d", [(8, 8, 128), (16, 4, 64), (8, 1, 64), (6, 3, 128)])
def test_decode_head_ratios(hq, hkv, d):
    note(f"decode bf16 hq={hq} hkv={hkv} D={d}")
    n_new = max(1, 8 // (hq // hkv))
    check_decode([(5, 700, n_new), (900, 64, 1), (964, 1, 1)], hq, hkv, d, seed=hq + d)


def test_decode_position_ties_and_fp32():
    note("decode: repeated positions (bf16), fp32 tiny shapes")
    check_decode([(0, 513, 3), (513, 40, 2)], 4, 2, 64, seed=5, pos_ties=True)
    check_decode([(0, 176, 1), (176, 90, 2)], 4, 2, 64, seed=6, dtype=torch.float32)
    check_decode([(0, 300, 2)], 4, 4, 128, seed=7, dtype=torch.float32)


def test_decode_many_sequences():
    """300 sequences in one call (five launch groups of at most 64 sharing one
    workspace): ragged caches of 1..400 rows with 1..4 new tokens each."""
    note("decode bf16 16/8 heads D=128 over 300 sequences")
    rng = np.random.default_rng(8)
    segs, st = [], 0
    for i in range(300):
        ln = int(rng.integers(1, 401))
        nn = int(min(ln, rng.integers(1, 5)))
        segs.append((st, ln, nn))
        st += ln + int(rng.integers(0, 3))  # gaps between caches are allowed
    out = check_decode(segs, 16, 8, 128, seed=12)
    assert not torch.isnan(out).any()


def test_check_positions():
    """tg_check_positions counts exactly the kept rows whose position is below the
    previous kept row's inside a prompt; a decrease across a prompt boundary is fine."""
    note("position check: valid positions, planted decreases, boundary between prompts")
    prompts = [Prompt(0, 3000, 50, 2900, 400), Prompt(3000, 1000, 0, 744, 100), Prompt(4000, 64, 0, 0, 0)]
    s = make_scores(4064, seed=31).to(DEV)
    kept = tg.tg_select_topk(s, prompts)
    _, pk, _ = tg.tg_compact(kept, prompts, [])
    assert int(tg.tg_check_positions(pk, prompts)[0]) == 0  # positions restart per prompt: no violation
    bad = pk.clone()
    m = bad.numel()
    idx = torch.tensor([5, 77, 500, m - 1], device=DEV)
    bad[idx] = -7  # each planted row now sits below its predecessor
    assert int(tg.tg_check_positions(bad, prompts)[0]) == 4
    ties = pk.clone()
    off = 0
    for p in prompts:  # each prompt's positions shifted by one row: every one repeated once
        n = p.n_kept
        if n > 1:
            ties[off + 1:off + n] = pk[off:off + n - 1].clone()
        off += n
    assert int(tg.tg_check_positions(ties, prompts)[0]) == 0  # repeated positions are allowed


def test_decode_deterministic_and_matches_prefill_rows():
    note("decode: bitwise repeatable; equals the prefill kernel's last rows within the bf16 bar")
    segs = [(0, 2384, 1), (2384, 1500, 2)]
    o1 = check_decode(segs, 16, 8, 128, seed=11)
    o2 = check_decode(segs, 16, 8, 128, seed=11)
    assert torch.equal(o1, o2)
    # the prefill kernel over the same cache, its queries filled in for the new rows
    q, k, v, bias, pos, gain = decode_inputs(segs, 16, 8, 128, seed=11)
    qfull = torch.zeros((3884, 16, 128), dtype=torch.bfloat16)
    qfull[2383] = q[0]
    qfull[3882:3884] = q[1:3]
    prompts = [Prompt(0, 2384, 0, 0, 0), Prompt(2384, 1500, 0, 0, 0)]
    pre, _ = tg.tg_gated_attention(qfull.to(DEV), k.to(DEV), v.to(DEV), bias.to(DEV), pos.to(DEV), prompts,
                                   gain.to(DEV), 1.2)
    rows = [2383, 3882, 3883]
    assert_rowmax_close(f64(o1), f64(pre[rows]), rel=2e-2)


# -------------------------------------------------------------- backward ----

def assert_slice_close(got, ref, rel=2e-2, what=""):
    """Gradient bar: per head slice [:, h, :], max |got - ref| <= rel * max |ref| of that
    slice (bf16 operands of the MFMAs: P, dS and dO round to 8 bits; gradients of rows that
    see little attention are sums with cancellation, so the slice maximum sets the scale)."""
    for h in range(ref.shape[1]):
        err = np.abs(got[:, h] - ref[:, h]).max()
        scale = np.abs(ref[:, h]).max()
        assert err <= rel * scale, f"{what} head {h}: max err {err:.3e} > {rel} * {scale:.3e}"


def check_backward(lens, hq, hkv, d, seed, pos_ties=False, tau=1.2, tail=20, qk_std=1.0, dout_from_v=0.0):
    """Backward against the oracle, which takes the row term d_out_i . o_i from the
    forward output handed to the backward (the GPU's bf16 `out`, an input of the call).
    Bars: dq, dk, dv per head slice (assert_slice_close); dbias within 2e-2 of its max;
    dgain per head within 2e-2 of that head's |dgain| (+1e-5 of the head's summed term
    magnitudes, for a head whose sum cancels to ~0); dtau within 2e-2 of |dtau| and
    within 1e-5 of dtau_mag. Error model of the scalar sums: each term dS_ij * x is
    formed in fp32 from fp32 S, P and dP (exact bf16 products, fp32 accumulation over D;
    p = exp2 of an argument with ~1e-6 absolute error), so it carries a relative error of
    ~1e-6 that cannot cancel, bounded by ~1e-6 of the summed magnitudes; the fp32 sums
    add ~1e-7 of them."""
    a = make_attention_inputs(lens, hq, hkv, d, seed=seed, dtype=torch.bfloat16, pos_ties=pos_ties,
                              n_query_tail=tail, qk_std=qk_std)
    ps, st = [], 0
    for ln in lens:
        ps.append(Prompt(st, ln, 0, 0, 0))
        st += ln
    dv_ = {k: (x.to(DEV) if hasattr(x, "to") else x) for k, x in a.items()}
    out, lse = tg.tg_gated_attention(dv_["q"], dv_["k"], dv_["v"], dv_["bias"], dv_["pos"], ps, dv_["gain"], tau,
                                     want_lse=True)
    dout = torch.randn(out.shape, generator=torch.Generator().manual_seed(seed + 1))
    if dout_from_v:
        # d_out correlated with the values: the row terms no longer cancel dtau's sum
        grp = hq // hkv
        dout = dout + dout_from_v * a["v"].float().repeat_interleave(grp, dim=1)
    dout = dout.to(torch.bfloat16)
    g = tg.tg_gated_attention_backward(dv_["q"], dv_["k"], dv_["v"], dv_["bias"], dv_["pos"], ps, dv_["gain"], tau,
                                       out, lse, dout.to(DEV))
    ref = oracle.gated_attention_backward(f64(a["q"]), f64(a["k"]), f64(a["v"]), f64(a["bias"]), a["pos"].numpy(),
                                          lens, hq, hkv, f64(a["gain"]), tau, f64(dout), o=f64(out))
    for key in ("dq", "dk", "dv"):
        assert_slice_close(f64(g[key]), ref[key], what=key)
    err = np.abs(f64(g["dbias"]) - ref["dbias"]).max()
    assert err <= 2e-2 * np.abs(ref["dbias"]).max(), f"dbias: {err:.3e}"
    dg_err = np.abs(f64(g["dgain"]) - ref["dgain"])
    dg_bar = 2e-2 * np.abs(ref["dgain"]) + 1e-5 * ref["dgain_abs"]
    note(f"  dgain worst err/|dgain_h| {np.max(dg_err / np.maximum(np.abs(ref['dgain']), 1e-30)):.2e}")
    assert np.all(dg_err <= dg_bar), f"dgain: err {dg_err} vs bar {dg_bar}"
    dt_err = abs(float(g["dtau"][0]) - ref["dtau"])
    note(f"  dtau {ref['dtau']:.6g} gpu {float(g['dtau'][0]):.6g} err/|dtau| {dt_err / abs(ref['dtau']):.2e} "
         f"err/dtau_mag {dt_err / ref['dtau_mag']:.2e} (dtau_mag/|dtau| {ref['dtau_mag'] / abs(ref['dtau']):.0f})")
    assert dt_err <= 2e-2 * abs(ref["dtau"]), f"dtau: {dt_err:.3e} vs {ref['dtau']:.3e}"
    assert dt_err <= 1e-5 * ref["dtau_mag"], f"dtau: {dt_err:.3e} vs mag {ref['dtau_mag']:.3e}"
    return g


def test_backward_qwen_shapes():
    note("backward bf16 16/8 heads D=128: one 2384-row prompt; ragged prompts with a one-row prompt")
    check_backward([2384], 16, 8, 128, seed=71)
    check_backward([700, 33, 1, 95], 16, 8, 128, seed=72)


@pytest.mark.parametrize("hq,hkv,d", [(4, 4, 64), (8, 2, 64), (6, 3, 128)])
def test_backward_head_ratios_and_ties(hq, hkv, d):
    note(f"backward bf16 hq={hq} hkv={hkv} D={d}, repeated positions")
    check_backward([300, 129], hq, hkv, d, seed=hq * 7 + d, pos_ties=True)


def test_backward_little_cancellation():
    note("backward bf16 16/8 heads D=128: sharp logits and d_out correlated with v (dtau's terms add up)")
    check_backward([900, 300], 16, 8, 128, seed=74, qk_std=2.0, tau=0.7, dout_from_v=1.0)


def test_backward_without_the_split():
    note("backward bf16 16/8 heads D=128, one 4200-row prompt (enough blocks that items are not split)")
    check_backward([4200], 16, 8, 128, seed=73)


def test_backward_deterministic():
    note("backward: bitwise repeatable")
    g1 = check_backward([1000], 16, 8, 128, seed=81)
    g2 = check_backward([1000], 16, 8, 128, seed=81)
    for key in g1:
        assert torch.equal(g1[key], g2[key]), key


def test_score_grad_chain_on_gpu():
    note("score gradient: d_bias * sigmoid(-s) on kept document rows, 0 elsewhere (bit-exact zeros)")
    prompts = [Prompt(0, 3000, 50, 2900, 400), Prompt(3000, 1000, 0, 744, 100), Prompt(4000, 64, 0, 0, 0)]
    s = make_scores(4064, seed=91) * 6
    kept = torch.from_numpy(oracle.select_topk(s.numpy(), prompts).astype(np.int32))
    db = torch.randn(len(kept), generator=torch.Generator().manual_seed(92))
    got = tg.tg_score_grad(db.to(DEV), s.to(DEV), kept.to(DEV), prompts).cpu().double().numpy()
    ref = oracle.score_grad(db.double().numpy(), s.numpy(), kept.numpy(), prompts)
    zero = ref == 0.0
    assert np.all(got[zero] == 0.0)
    np.testing.assert_allclose(got[~zero], ref[~zero], rtol=2e-6, atol=0)


# --------------------------------------------------------- gate backward ----

def check_gate_backward(n, d, h, n_list, seed, with_b1=True, with_dx=True):
    """Gate MLP backward over a row list (every row when n_list == n) against the oracle.
    Bars: dW1 and dx within 2e-2 of their maxima (dz enters the MFMAs in bf16); dw2, db1,
    db2 (fp32 sums of fp32 terms) within 1e-3 of their maxima; unlisted rows of dx
    untouched, bit for bit."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, d, generator=g).to(torch.bfloat16)
    w1 = (torch.randn(h, d, generator=g) / math.sqrt(d)).to(torch.bfloat16)
    w2 = (torch.randn(h, generator=g) / math.sqrt(h)).to(torch.bfloat16)
    b1 = (torch.randn(h, generator=g) * 0.5).to(torch.bfloat16) if with_b1 else None
    ds = torch.randn(n, generator=g)  # unlisted rows carry junk that must be ignored
    if n_list < n:
        rows = torch.randperm(n, generator=g)[:n_list].sort().values.to(torch.int32)
        rows_np = rows.numpy().astype(np.int64)
    else:
        rows, rows_np = None, np.arange(n)
    dx0 = torch.randn(n, d, generator=g) * 0.1
    dxd = dx0.to(DEV) if with_dx else None
    got = tg.tg_gate_backward(x.to(DEV), w1.to(DEV), w2.to(DEV), ds.to(DEV),
                              rows=None if rows is None else rows.to(DEV),
                              b1=None if b1 is None else b1.to(DEV), d_x=dxd)
    ref = oracle.gate_backward(f64(x), f64(w1), f64(w2), ds.double().numpy(), rows=rows_np,
                               b1=None if b1 is None else f64(b1))
    if n_list == 0:
        for k in ("dw1", "db1", "dw2", "db2"):
            assert not torch.any(got[k]), k
    else:
        for k, rel in (("dw1", 2e-2), ("dw2", 1e-3), ("db1", 1e-3)):
            err = np.abs(f64(got[k]) - ref[k]).max()
            assert err <= rel * np.abs(ref[k]).max(), f"{k}: {err:.3e} vs max {np.abs(ref[k]).max():.3e}"
        assert abs(float(got["db2"][0]) - ref["db2"]) <= 1e-5 * np.abs(ds.numpy()[rows_np]).sum()
    if with_dx:
        dxg = got["dx"].cpu()
        listed = np.zeros(n, dtype=bool)
        listed[rows_np] = True
        assert torch.equal(dxg[~torch.from_numpy(listed)], dx0[~torch.from_numpy(listed)])
        if n_list:
            delta = dxg[torch.from_numpy(rows_np)].double().numpy() - dx0[torch.from_numpy(rows_np)].double().numpy()
            err = np.abs(delta - ref["dx"]).max()
            assert err <= 2e-2 * np.abs(ref["dx"]).max(), f"dx: {err:.3e}"
    return got


def test_gate_backward_qwen16k_kept_rows():
    note("gate backward bf16 N=16384 d=2048 H=256 over 2384 listed rows, b1, dx accumulated")
    check_gate_backward(16384, 2048, 256, 2384, seed=101)


@pytest.mark.parametrize("n,d,h,n_list,with_b1", [(1000, 192, 64, 77, False), (300, 320, 128, 300, True),
                                                  (513, 64, 192, 1, True), (700, 2048, 256, 700, False),
                                                  (64, 128, 64, 0, True)])
def test_gate_backward_shapes(n, d, h, n_list, with_b1):
    note(f"gate backward bf16 n={n} d={d} H={h} listed={n_list} b1={with_b1}")
    check_gate_backward(n, d, h, n_list, seed=n + d + h + n_list, with_b1=with_b1)


def test_gate_backward_without_dx_and_deterministic():
    note("gate backward: no dx; bitwise repeatable")
    a = check_gate_backward(2000, 512, 128, 333, seed=7, with_dx=False)
    b = check_gate_backward(2000, 512, 128, 333, seed=7, with_dx=False)
    for k in a:
        assert torch.equal(a[k], b[k]), k


# ------------------------------------------------------- full above-gate layer ----

# (3000, 128, 8192) runs every epilogue on the 256 x 256 tiles with a ragged
# last row tile; the other cases run on 256 x 128 tiles, or on 128 x 128 for
# outputs that are not a multiple of 256 (store and residual at n = 128, 384).
@pytest.mark.parametrize("m,k,n", [(1, 64, 128), (77, 2048, 384), (300, 128, 4096), (2384, 2048, 256),
                                   (3000, 128, 8192)])
def test_linear_epilogues(m, k, n):
    """tg_linear against the oracle's linear / swiglu: store, residual add, SwiGLU.
    Bar: per row, max |err| <= 1e-2 * max |ref| (fp32 sums of exact bf16 products, one
    bf16 rounding of the result; SwiGLU: two such sums and an fp32 SiLU)."""
    note(f"linear m={m} k={k} n={n}: store, residual, swiglu")
    g = torch.Generator().manual_seed(m + k + n)
    x = torch.randn(m, k, generator=g).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g) / math.sqrt(k)).to(torch.bfloat16)
    wu = (torch.randn(n, k, generator=g) / math.sqrt(k)).to(torch.bfloat16)
    r = torch.randn(m, n, generator=g).to(torch.bfloat16)
    xd, wd, wud, rd = x.to(DEV), w.to(DEV), wu.to(DEV), r.to(DEV)
    assert_rowmax_close(f64(tg.tg_linear(xd, wd)), oracle.linear(f64(x), f64(w)), rel=1e-2)
    assert_rowmax_close(f64(tg.tg_linear(xd, wd, residual=rd)), oracle.linear(f64(x), f64(w), f64(r)), rel=1e-2)
    assert_rowmax_close(f64(tg.tg_linear(xd, wd, w_up=wud)), oracle.swiglu(f64(x), f64(w), f64(wu)), rel=1e-2)


def check_dense_layer(segs, d, hq, hkv, dh, d_ff, seed, pos_offset=0):
    from synthetic import make_dense_layer, make_kept_hidden
    w = make_dense_layer(d, hq, hkv, dh, d_ff, seed=seed)
    x = make_kept_hidden(list(segs), d, seed=seed + 1, n_query_tail=16)
    pos = x["pos"] + pos_offset
    ps, st = [], 0
    for ln in segs:
        ps.append(Prompt(st, ln, 0, 0, 0))
        st += ln
    wd = {kk: (t.to(DEV) if hasattr(t, "to") else t) for kk, t in w.items()}
    out, kc, vc = tg.tg_dense_layer(x["h"].to(DEV), x["bias"].to(DEV), pos.to(DEV), ps, wd, hq, hkv, dh,
                                    want_kv=True)
    ref = oracle.dense_layer(x["h"], pos, x["bias"], list(segs), w, hq, hkv, dh)
    # bf16 storage between the steps: per (row, head) and per row against the row maximum
    rk = assert_rowmax_close(f64(kc), ref["k"])
    rv = assert_rowmax_close(f64(vc), ref["v"])
    ro = assert_rowmax_close(f64(out), ref["out"])
    return out, (rk, rv, ro)


def test_dense_layer_small_ragged():
    note("dense layer d=256 hq=4 hkv=2 D=64 d_ff=384, prompts 100 + 1 + 37")
    check_dense_layer([100, 1, 37], 256, 4, 2, 64, 384, seed=31)


def test_dense_layer_qwen_shapes_far_positions():
    note("dense layer Qwen3-1.7B shapes (d=2048, 16/8 heads, D=128, d_ff=6144), 600 kept rows at positions ~120k")
    check_dense_layer([500, 100], 2048, 16, 8, 128, 6144, seed=32, pos_offset=120000)


def test_dense_layer_deterministic():
    note("dense layer: bitwise repeatable")
    a, _ = check_dense_layer([300], 512, 8, 4, 128, 1024, seed=33)
    b, _ = check_dense_layer([300], 512, 8, 4, 128, 1024, seed=33)
    assert torch.equal(a, b)


# -------------------------------------------------------- gated delta rule ----

def check_delta_scan(segs, nh, seed, with_state=True):
    """Bars: outputs per (row, head) within 2e-2 of their maximum over the row's dv values,
    final states per (prompt, head) within 2e-2 of their maximum (bf16 operands of the
    chunk products: the state copy, Y, P and W round to 8 bits; the state itself is kept
    in fp32)."""
    from synthetic import make_delta_inputs
    a = make_delta_inputs(list(segs), nh, 128, 128, seed=seed)
    s0 = (torch.randn(len(segs), nh, 128, 128, generator=torch.Generator().manual_seed(seed + 1)) * 0.05
          if with_state else None)
    ps, st = [], 0
    for ln in segs:
        ps.append(Prompt(st, ln, 0, 0, 0))
        st += ln
    out, fs = tg.tg_gated_delta_scan(a["q"].to(DEV), a["k"].to(DEV), a["v"].to(DEV), a["g"].to(DEV),
                                     a["beta"].to(DEV), ps, state_in=None if s0 is None else s0.to(DEV),
                                     want_state=True)
    ref_o, ref_s = oracle.gated_delta_scan(f64(a["q"]), f64(a["k"]), f64(a["v"]), a["g"].double().numpy(),
                                           a["beta"].double().numpy(), list(segs),
                                           state0=None if s0 is None else s0.double().numpy())
    r1 = assert_rowmax_close(f64(out), ref_o)
    got_s = fs.cpu().double().numpy()
    for p in range(len(segs)):
        for h in range(nh):
            err = np.abs(got_s[p, h] - ref_s[p, h]).max()
            assert err <= 2e-2 * np.abs(ref_s[p, h]).max() + 1e-6, f"state {p},{h}: {err:.3e}"
    return out, fs


def test_delta_scan_ragged_prompts_with_state():
    note("gated delta rule: prompts of 200, 1, 77 and 64 kept rows, 4 heads, initial states")
    check_delta_scan([200, 1, 77, 64], 4, seed=51)


def test_delta_scan_16k_kept_rows():
    note("gated delta rule: 2384 kept rows, 16 heads, zero initial state")
    check_delta_scan([2384], 16, seed=52, with_state=False)


def test_delta_scan_deterministic():
    note("gated delta rule: bitwise repeatable")
    a = check_delta_scan([300, 50], 2, seed=53)
    b = check_delta_scan([300, 50], 2, seed=53)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_delta_scan_empty_prompts_pass_state_through():
    """A prompt with no kept rows leaves its state as given; the others run as usual."""
    note("gated delta rule: prompts of 0, 70 and 0 kept rows with initial states")
    from synthetic import make_delta_inputs
    a = make_delta_inputs([70], 2, 128, 128, seed=61)
    s0 = torch.randn(3, 2, 128, 128, generator=torch.Generator().manual_seed(62)) * 0.05
    ps = [Prompt(0, 0, 0, 0, 0), Prompt(0, 70, 0, 0, 0), Prompt(70, 0, 0, 0, 0)]
    out, fs = tg.tg_gated_delta_scan(a["q"].to(DEV), a["k"].to(DEV), a["v"].to(DEV), a["g"].to(DEV),
                                     a["beta"].to(DEV), ps, state_in=s0.to(DEV), want_state=True)
    ref_o, ref_s = oracle.gated_delta_scan(f64(a["q"]), f64(a["k"]), f64(a["v"]), a["g"].double().numpy(),
                                           a["beta"].double().numpy(), [0, 70, 0], state0=s0.double().numpy())
    assert_rowmax_close(f64(out), ref_o)
    got = fs.cpu()
    assert torch.equal(got[0], s0[0]) and torch.equal(got[2], s0[2])
    np.testing.assert_allclose(got[1].double().numpy(), ref_s[1], atol=2e-2 * np.abs(ref_s[1]).max())


def test_dense_layer_16k_kept_rows():
    note("dense layer at the 16k layer's size: 2384 kept rows, Qwen3-1.7B shapes, d_ff 6144")
    check_dense_layer([2384], 2048, 16, 8, 128, 6144, seed=34)


def test_layer_gathers_row_strided_views():
    """q, k, v given as column slices of one fused projection (row stride larger than
    the row): the layer gathers each with its own row stride and gives bit-for-bit
    the result of contiguous copies."""
    note("layer over q/k/v sliced from one fused [N, (hq+2hkv)D] projection")
    w = make_workload("tiny", device=DEV)
    wl = w.layers[0]
    fused = torch.cat([wl.q, wl.k, wl.v], dim=1)
    dq, dk = w.hq * w.head_dim, w.hkv * w.head_dim

    class View:
        q, k, v = fused[:, :dq], fused[:, dq:dq + dk], fused[:, dq + dk:]
        gain, tau = wl.gain, wl.tau

    assert View.q.stride(0) == fused.shape[1] and not View.q.is_contiguous()
    a = run_layer(w, layers=[View])
    b = run_layer(w)
    for x, y in zip(a.qkv_kept[0], b.qkv_kept[0]):
        assert torch.equal(x, y)
    assert torch.equal(a.outs[0], b.outs[0])
    with pytest.raises(ValueError):
        class Bad:
            q, k, v = fused[:, :dq].t(), wl.k, wl.v
            gain, tau = wl.gain, wl.tau
        tg.GatedPrefillLayer(w.x, w.w1, w.w2, w.prompts, [Bad], w.hq, w.hkv, w.head_dim)

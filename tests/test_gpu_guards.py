"""Out-of-bounds and unwritten-output checks for every output of every call.

Each output lives inside a larger device buffer with 1 KiB guard regions
before and after it. The whole buffer is filled with one byte pattern, the
call runs, and then the same is done with a second pattern. The guards must
keep their pattern (no write outside the output), and the two runs must give
bit-identical outputs (an element the call never writes would keep the
pattern and differ between the runs). Outputs a call adds to (the gate
backward's dx) are checked for their guards and against a plain run instead.
"""

import math

import numpy as np
import pytest
import torch

import learned_token_pruning_layer_amd as tg
from synthetic import Prompt, make_attention_inputs, make_scores

pytestmark = pytest.mark.gpu
DEV = "cuda"
GUARD = 1024
PATTERNS = (0xA5, 0x5A)


def note(msg):
    print(f"[case] {msg}", flush=True)


class Guarded:
    """A device tensor of `shape` and `dtype` inside a buffer with GUARD bytes on each side."""

    def __init__(self, shape, dtype):
        esz = torch.empty((), dtype=dtype).element_size()
        nbytes = int(math.prod(shape)) * esz
        self.raw = torch.empty(2 * GUARD + nbytes, dtype=torch.uint8, device=DEV)
        self.t = self.raw[GUARD:GUARD + nbytes].view(dtype).view(shape)

    def fill(self, byte):
        self.raw.fill_(byte)

    def guards_intact(self, byte):
        return bool((self.raw[:GUARD] == byte).all()) and bool((self.raw[-GUARD:] == byte).all())


def run_guarded(call, outs):
    """call(outs) twice, once per fill pattern; returns the outputs of the first run.
    outs: dict name -> Guarded."""
    results = []
    for byte in PATTERNS:
        for g in outs.values():
            g.fill(byte)
        call({k: g.t for k, g in outs.items()})
        torch.cuda.synchronize()
        for k, g in outs.items():
            assert g.guards_intact(byte), f"{k}: a write landed outside the output (pattern {byte:#x})"
        results.append({k: g.t.clone() for k, g in outs.items()})
    for k in outs:
        a, b = results[0][k].view(torch.uint8), results[1][k].view(torch.uint8)
        assert torch.equal(a, b), f"{k}: {int((a != b).sum())} bytes left unwritten (they kept the fill pattern)"
    return results[0]


def test_guard_gate_score():
    note("guards: gate scores (bf16 MFMA path at every built hidden size, ragged tails; fp32 path)")
    g = torch.Generator(device=DEV).manual_seed(1)
    for n, d, h, dt in ((1000, 2048, 256, torch.bfloat16), (33000, 256, 256, torch.bfloat16),
                        (1001, 512, 192, torch.bfloat16), (129, 512, 128, torch.bfloat16),
                        (300, 256, 64, torch.bfloat16), (77, 256, 64, torch.float32)):
        x = torch.randn(n, d, generator=g, device=DEV).to(dt)
        w1 = (torch.randn(h, d, generator=g, device=DEV) / math.sqrt(d)).to(dt)
        w2 = (torch.randn(h, generator=g, device=DEV) / math.sqrt(h)).to(dt)
        run_guarded(lambda o: tg.tg_gate_score(x, w1, w2, scores=o["s"]), {"s": Guarded((n,), torch.float32)})


def test_guard_select_single_and_multi_workgroup():
    note("guards: select (one-workgroup prompts and a prompt above 32768 rows)")
    for prompts, n in (([Prompt(0, 3000, 50, 2900, 400), Prompt(3000, 1000, 0, 744, 100), Prompt(4000, 64, 0, 0, 0)],
                        4064),
                       ([Prompt(0, 40000, 100, 39900, 5000), Prompt(40000, 300, 0, 200, 7)], 40300)):
        s = make_scores(n, seed=n).to(DEV)
        m = tg.tg_kept_rows(prompts)
        run_guarded(lambda o: tg.tg_select_topk(s, prompts, kept_idx=o["kept"]), {"kept": Guarded((m,), torch.int32)})


def test_guard_compact():
    note("guards: compaction (two gathered tensors, positions, bias)")
    prompts = [Prompt(0, 3000, 50, 2900, 400), Prompt(3000, 1000, 0, 744, 100), Prompt(4000, 64, 0, 0, 0)]
    n = 4064
    s = make_scores(n, seed=21).to(DEV)
    kept = tg.tg_select_topk(s, prompts)
    m = kept.numel()
    g = torch.Generator(device=DEV).manual_seed(2)
    a = torch.randn(n, 2048, generator=g, device=DEV).to(torch.bfloat16)
    b = torch.randn(n, 8, 128, generator=g, device=DEV).to(torch.bfloat16)
    outs = {"a": Guarded((m, 2048), torch.bfloat16), "b": Guarded((m, 8, 128), torch.bfloat16),
            "pos": Guarded((m,), torch.int32), "bias": Guarded((m,), torch.float32)}
    run_guarded(lambda o: tg.tg_compact(kept, prompts, [a, b], scores=s, outs=[o["a"], o["b"]], pos_kept=o["pos"],
                                        bias_kept=o["bias"]), outs)


@pytest.mark.parametrize("dt,segs", [(torch.bfloat16, [1000, 23, 1]), (torch.float32, [1000, 23, 1]),
                                     (torch.bfloat16, [4200, 23, 1]), (torch.bfloat16, [16400, 23, 1])],
                         ids=["bf16-short", "fp32", "bf16-long", "bf16-xl"])
def test_guard_attention(dt, segs):
    note(f"guards: token-gated attention ({dt}, prompts {segs}), output and lse")
    hq, hkv, d = 16, 8, 128
    a = make_attention_inputs(segs, hq, hkv, d, seed=3, dtype=dt, n_query_tail=8)
    prompts, st = [], 0
    for ln in segs:
        prompts.append(Prompt(st, ln, 0, 0, 0))
        st += ln
    m = sum(segs)
    args = [a[k].to(DEV) for k in ("q", "k", "v", "bias", "pos")]
    outs = {"o": Guarded((m, hq, d), dt), "lse": Guarded((hq, m), torch.float32)}
    run_guarded(lambda o: tg.tg_gated_attention(*args, prompts, a["gain"].to(DEV), 1.2, out=o["o"], want_lse=True,
                                                lse=o["lse"]), outs)


def test_guard_decode():
    note("guards: decode (ragged caches, 1-3 new tokens), output and lse")
    segs, hq, hkv, d = [(0, 700, 3), (700, 33, 1), (733, 2000, 2)], 16, 8, 128
    rows = 2733
    a = make_attention_inputs([rows], hq, hkv, d, seed=4, dtype=torch.bfloat16)
    r = sum(nn for _, _, nn in segs)
    q = torch.randn((r, hq, d), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(DEV)
    outs = {"o": Guarded((r, hq, d), torch.bfloat16), "lse": Guarded((hq, r), torch.float32)}
    run_guarded(lambda o: tg.tg_decode_attention(q, a["k"].to(DEV), a["v"].to(DEV), a["bias"].to(DEV),
                                                 a["pos"].to(DEV), segs, a["gain"].to(DEV), 1.2, out=o["o"],
                                                 want_lse=True, lse=o["lse"]), outs)


def test_guard_attention_backward_and_score_grad():
    note("guards: attention backward (dq, dk, dv, dbias, dgain, dtau) and the score gradient")
    segs, hq, hkv, d = [700, 33, 1], 16, 8, 128
    a = make_attention_inputs(segs, hq, hkv, d, seed=6, dtype=torch.bfloat16, n_query_tail=8)
    prompts, st = [], 0
    for ln in segs:
        prompts.append(Prompt(st, ln, 0, 0, 0))
        st += ln
    m = sum(segs)
    dv_ = {k: a[k].to(DEV) for k in ("q", "k", "v", "bias", "pos", "gain")}
    out, lse = tg.tg_gated_attention(dv_["q"], dv_["k"], dv_["v"], dv_["bias"], dv_["pos"], prompts, dv_["gain"],
                                     1.2, want_lse=True)
    dout = torch.randn(out.shape, generator=torch.Generator().manual_seed(7)).to(torch.bfloat16).to(DEV)
    f32 = torch.float32
    outs = {"dq": Guarded((m, hq, d), f32), "dk": Guarded((m, hkv, d), f32), "dv": Guarded((m, hkv, d), f32),
            "dbias": Guarded((m,), f32), "dgain": Guarded((hq,), f32), "dtau": Guarded((1,), f32)}
    run_guarded(lambda o: tg.tg_gated_attention_backward(dv_["q"], dv_["k"], dv_["v"], dv_["bias"], dv_["pos"],
                                                         prompts, dv_["gain"], 1.2, out, lse, dout, grads=o), outs)
    sp = [Prompt(0, 3000, 50, 2900, 400), Prompt(3000, 1000, 0, 744, 100)]
    s = make_scores(4000, seed=8).to(DEV)
    kept = tg.tg_select_topk(s, sp)
    db = torch.randn(kept.numel(), generator=torch.Generator().manual_seed(9)).to(DEV)
    run_guarded(lambda o: tg.tg_score_grad(db, s, kept, sp, d_scores=o["ds"]), {"ds": Guarded((4000,), f32)})


def test_guard_gate_backward():
    note("guards: gate backward (dW1, db1, dw2, db2; dx is added to)")
    n, d, h = 2000, 512, 128
    g = torch.Generator().manual_seed(10)
    x = torch.randn(n, d, generator=g).to(torch.bfloat16).to(DEV)
    w1 = (torch.randn(h, d, generator=g) / math.sqrt(d)).to(torch.bfloat16).to(DEV)
    w2 = (torch.randn(h, generator=g) / math.sqrt(h)).to(torch.bfloat16).to(DEV)
    ds = torch.randn(n, generator=g).to(DEV)
    rows = torch.randperm(n, generator=g)[:333].sort().values.to(torch.int32).to(DEV)
    f32 = torch.float32
    outs = {"dw1": Guarded((h, d), f32), "db1": Guarded((h,), f32), "dw2": Guarded((h,), f32),
            "db2": Guarded((1,), f32)}
    run_guarded(lambda o: tg.tg_gate_backward(x, w1, w2, ds, rows=rows, grads=o), outs)
    # dx is accumulated into: guards around it, result equal to a plain buffer's
    dx0 = torch.randn(n, d, generator=g).to(DEV)
    gdx = Guarded((n, d), f32)
    gdx.fill(0xA5)
    gdx.t.copy_(dx0)
    tg.tg_gate_backward(x, w1, w2, ds, rows=rows, d_x=gdx.t)
    plain = dx0.clone()
    tg.tg_gate_backward(x, w1, w2, ds, rows=rows, d_x=plain)
    torch.cuda.synchronize()
    assert gdx.guards_intact(0xA5)
    assert torch.equal(gdx.t, plain)


def test_guard_linear_and_dense_layer():
    note("guards: linear (three epilogues) and the full above-gate layer (out, K, V)")
    from synthetic import make_dense_layer, make_kept_hidden
    g = torch.Generator().manual_seed(11)
    m, k, n = 300, 256, 384
    x = torch.randn(m, k, generator=g).to(torch.bfloat16).to(DEV)
    w = (torch.randn(n, k, generator=g) / 16).to(torch.bfloat16).to(DEV)
    wu = (torch.randn(n, k, generator=g) / 16).to(torch.bfloat16).to(DEV)
    r = torch.randn(m, n, generator=g).to(torch.bfloat16).to(DEV)
    for kw in ({}, {"residual": r}, {"w_up": wu}):
        run_guarded(lambda o: tg.tg_linear(x, w, out=o["o"], **kw), {"o": Guarded((m, n), torch.bfloat16)})
    segs, d, hq, hkv, dh, d_ff = [100, 1, 37], 256, 4, 2, 64, 384
    wts = {kk: (t.to(DEV) if hasattr(t, "to") else t) for kk, t in make_dense_layer(d, hq, hkv, dh, d_ff, seed=12).items()}
    xh = make_kept_hidden(segs, d, seed=13, n_query_tail=16)
    prompts, st = [], 0
    for ln in segs:
        prompts.append(Prompt(st, ln, 0, 0, 0))
        st += ln
    mm = sum(segs)
    outs = {"o": Guarded((mm, d), torch.bfloat16), "k": Guarded((mm, hkv, dh), torch.bfloat16),
            "v": Guarded((mm, hkv, dh), torch.bfloat16)}
    run_guarded(lambda o: tg.tg_dense_layer(xh["h"].to(DEV), xh["bias"].to(DEV), xh["pos"].to(DEV), prompts, wts, hq,
                                            hkv, dh, out=o["o"], want_kv=True, k_out=o["k"], v_out=o["v"]), outs)


def test_guard_delta_scan():
    note("guards: gated delta rule (out, final states; an empty prompt in the batch)")
    from synthetic import make_delta_inputs
    segs, nh = [200, 0, 77], 2
    a = make_delta_inputs([277], nh, 128, 128, seed=14)
    prompts = [Prompt(0, 200, 0, 0, 0), Prompt(200, 0, 0, 0, 0), Prompt(200, 77, 0, 0, 0)]
    s0 = (torch.randn(3, nh, 128, 128, generator=torch.Generator().manual_seed(15)) * 0.05).to(DEV)
    outs = {"o": Guarded((277, nh, 128), torch.bfloat16), "s": Guarded((3, nh, 128, 128), torch.float32)}
    run_guarded(lambda o: tg.tg_gated_delta_scan(a["q"].to(DEV), a["k"].to(DEV), a["v"].to(DEV), a["g"].to(DEV),
                                                 a["beta"].to(DEV), prompts, state_in=s0, want_state=True,
                                                 out=o["o"], state_out=o["s"]), outs)

"""Benchmark of the TokenGate pruned-prefill layer on one MI355X.

A step is one pass of the whole layer over one batch: gate score -> top-K
select -> compaction -> token-gated attention, four C-ABI calls on one
stream, inputs already resident in HBM. The workload is the 16k
Qwen3-1.7B-shaped layer: N=16384 rows (16000 document + 384 question),
d_model 2048, gate 2048->256->1, keep 2000 document rows (12.5%), 16 query /
8 KV heads, head_dim 128, bf16, 16 planted rows.

Prints ONE JSON line. `value` is the layer latency in ms (lower is better);
attention TFLOP/s and its fraction of the bf16 MFMA peak ride along, with a
per-kernel breakdown, a roofline entry for the dominant kernel and the fp64
oracle timed on the host cores as a reported CPU baseline.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "gated-prefill layer ms + attn TFLOP/s (% MFMA peak) at 16k, keep 12.5%"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    ap.add_argument("--cpu-budget-s", type=float, default=30.0)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the extra measurements (re-measured peaks, percentiles, cold runs, large select)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (the scale reference for --pmc byte counters)")
    ap.add_argument("--workload", default="qwen16k", choices=("qwen16k", "long128k"),
                    help="the layer the timed steps run (qwen16k is the reported metric; long128k serves "
                         "profiling runs of the 128k layer)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="CPU only: turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a "
                         "--calibrate-copy run into profiles/traffic_qwen16k.json and exit")
    return ap.parse_args()


def algorithmic_work(w, m):
    """Algorithmic bytes / flops of one launch of each kernel at this workload."""
    n, d = w.x.shape
    h = w.w1.shape[0]
    hq, hkv, dh = w.hq, w.hkv, w.head_dim
    p = w.prompts[0]
    # gate: read X once, W1 once, write one fp32 score per row
    gate_bytes = n * d * 2 + h * d * 2 + h * 2 + n * 4
    gate_flops = n * (2 * d * h + 4 * h)
    # select: read each document score once, write one int32 per kept row
    sel_bytes = p.n_doc * 4 + m * 4
    # compact: read + write every gathered row (hidden, Q, K, V), index read,
    # score read, position and bias writes
    row = (d + (hq + 2 * hkv) * dh) * 2
    comp_bytes = m * (2 * row + 4 + 4 + 4 + 4)
    # attention: 4*D*Hq flop per visible (query, key) pair, causal incl. diagonal
    pairs = m * (m + 1) // 2
    attn_flops = 4 * dh * hq * pairs
    return dict(gate=dict(bytes=gate_bytes, flops=gate_flops), select=dict(bytes=sel_bytes),
                compact=dict(bytes=comp_bytes), attention=dict(flops=attn_flops))


def source_hash(rel):
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


KERNEL_SOURCES = {
    "gate": "learned_token_pruning_layer_amd/csrc/gate_score.hip",
    "select": "learned_token_pruning_layer_amd/csrc/select_topk.hip",
    "compact": "learned_token_pruning_layer_amd/csrc/compact.hip",
    "attention": "learned_token_pruning_layer_amd/csrc/gated_attention.hip",
}


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic_qwen16k.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec or rec.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


WORKLOAD_TEXT = {
    "qwen16k": "qwen16k: one pruned-prefill layer, N=16384 (16000 doc + 384 query), keep 2000 doc rows (12.5%), "
               "d_model 2048, gate 2048->256->1, 16 Q / 8 KV heads, head_dim 128, 16 planted rows",
    "long128k": "long128k: one pruned-prefill layer, N=131072 (130048 doc + 1024 query), keep 8128 doc rows "
                "(6.25%), d_model 2048, gate 2048->256->1, 16 Q / 8 KV heads, head_dim 128, planted rows 1 per 8192",
}

COPY_BYTES = 256 << 20
KERNEL_NAMES = {"gate": "gate_mfma_kernel", "select": "select_kernel", "compact": "compact_kernel",
                "attention": "attn_bf16_kernel"}


def traffic_summary(fetch_csv, write_csv):
    """Per-launch HBM-side bytes of each kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by what the same counter reads for a plain copy of
    COPY_BYTES (which reads and writes exactly that many bytes)."""
    import csv

    def load(path, counter):
        per = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return per

    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        per = load(path, counter)
        copies = [v for k, vals in per.items() if "copy" in k.lower() for v in vals if v > COPY_BYTES / 2]
        if not copies:
            raise SystemExit(f"no copy kernel of ~{COPY_BYTES} bytes found in {path}")
        scale = COPY_BYTES / (sum(copies) / len(copies))
        for key, pat in KERNEL_NAMES.items():
            vals = [v for k, vs in per.items() if pat in k for v in vs]
            if vals:
                rec = out.setdefault(key, {})
                rec[counter.lower() + "_bytes"] = sum(vals) / len(vals) * scale
                rec[counter.lower() + "_scale"] = scale
    for key, rec in out.items():
        rec["hbm_bytes_per_launch"] = rec.get("fetch_size_bytes", 0.0) + rec.get("write_size_bytes", 0.0)
        rec["source_sha256_16"] = source_hash(KERNEL_SOURCES[key])
    dst = os.path.join(ROOT, "profiles", "traffic_qwen16k.json")
    with open(dst, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print(json.dumps(out, indent=1, sort_keys=True))


class Evictor:
    """Evicts the caches before a cold step: a 1 GiB device write (the 256 MB
    Infinity Cache and the L2s then hold none of the layer's inputs), and, with
    read=True, a 1 GiB read after it, which replaces the write's dirty lines
    with clean ones, so the timed kernels do not also pay for writing back
    the eviction buffer."""

    def __init__(self, torch, dev, read=True):
        self.torch = torch
        self.wbuf = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        self.rbuf = torch.ones(1 << 28, dtype=torch.float32, device=dev) if read else None
        self.acc = torch.zeros(1, dtype=torch.float32, device=dev)

    def __call__(self):
        self.wbuf.fill_(3.0)
        if self.rbuf is not None:
            self.acc.add_(self.rbuf.sum())


def kernel_times(torch, layer, reps, evict=None):
    """Median per-kernel durations (us) of the four steps, HIP events around each
    launch on the layer's stream. With evict (an Evictor), the caches are
    evicted before every step, so each kernel reads its inputs from HBM (the
    writes of the step's earlier kernels stay cached)."""
    stream = torch.cuda.current_stream()
    names = ["gate", "select", "compact", "attention"]
    samples = {k: [] for k in names}
    for _ in range(reps):
        if evict is not None:
            evict()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        ev[0].record(stream)
        layer.gate()
        ev[1].record(stream)
        layer.select()
        ev[2].record(stream)
        layer.compact()
        ev[3].record(stream)
        layer.attention(0)
        ev[4].record(stream)
        torch.cuda.synchronize()
        for i, k in enumerate(names):
            samples[k].append(ev[i].elapsed_time(ev[i + 1]) * 1e3)
    return {k: round(sorted(v)[len(v) // 2], 2) for k, v in samples.items()}


def rooflines_of(work, us, cache):
    """Roofline fractions of the kernels from their algorithmic work and times."""
    out = {}
    for k in ("gate", "compact", "select"):
        ach = work[k]["bytes"] / (us[k] * 1e-6) / 1e9
        out[k] = dict(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                      frac=round(ach / PEAK_HBM_GBS, 4), cache=cache)
    ach = work["attention"]["flops"] / (us["attention"] * 1e-6) / 1e12
    out["attention"] = dict(bound="mfma", achieved=round(ach, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                            frac=round(ach / PEAK_BF16_TFLOPS, 4), cache=cache)
    return out


def cpu_baseline(w, budget_s, gpu_layer=None):
    """The fp64 oracle, untuned, on the host cores: one whole layer if it
    fits the budget, else the gate + select + compaction in full and the
    attention on an evenly spaced sample of query rows, scaled by the
    number of visible (query, key) pairs."""
    import numpy as np
    import oracle

    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = ", ".join(sorted({f"{i.get('internal_api', '?')} {i.get('version', '')}".strip() for i in info})) or blas
    except Exception:
        threads = os.cpu_count() or 1
    lay = w.layers[0]
    x, w1, w2 = w.x.cpu(), w.w1.cpu(), w.w2.cpu()
    q, k, v, gain = lay.q.cpu(), lay.k.cpu(), lay.v.cpu(), lay.gain.cpu()
    hq, hkv, dh = w.hq, w.hkv, w.head_dim
    t0 = time.perf_counter()
    s = oracle.gate_scores(x, w1, w2)
    kept = oracle.select_topk(s.astype(np.float32), w.prompts)
    (qk, kk, vk), pk, bk = oracle.compact(kept, w.prompts, (q, k, v), s)
    t_front = time.perf_counter() - t0
    parity = None
    if gpu_layer is not None:
        # The selection the GPU made from its own scores against the one the
        # fp64 gate implies: rows near the threshold may change sides (the
        # scores differ by the fp32 accumulation of the bf16 products).
        gk = set(gpu_layer.kept.cpu().numpy().tolist())
        gs = gpu_layer.scores.cpu().double().numpy()
        parity = {"kept_flips_vs_fp64_gate": len(gk ^ set(kept.tolist())),
                  "max_abs_score_diff": float(np.abs(gs - s).max()),
                  "max_abs_score": float(np.abs(s).max())}
    m = len(kept)
    qk, kk, vk = qk.view(m, hq, dh), kk.view(m, hkv, dh), vk.view(m, hkv, dh)
    # probe the attention cost on a small sample to size the run
    probe = np.linspace(0, m - 1, 64).astype(np.int64)
    t1 = time.perf_counter()
    oracle.gated_attention(qk, kk, vk, bk, pk, [m], hq, hkv, gain, lay.tau, rows=probe)
    t_probe = time.perf_counter() - t1
    pairs_probe = float(np.sum(probe + 1))
    pairs_all = m * (m + 1) / 2
    est_full = t_probe * pairs_all / pairs_probe
    if t_front + est_full <= budget_s:
        t1 = time.perf_counter()
        oracle.gated_attention(qk, kk, vk, bk, pk, [m], hq, hkv, gain, lay.tau)
        t_attn = time.perf_counter() - t1
        sample = f"one whole layer: gate over {w.n_rows} rows, select, compaction, attention over all {m} kept rows"
    else:
        nrow = max(64, int(m * budget_s / max(est_full, 1e-9) * 0.5))
        rows = np.linspace(0, m - 1, min(nrow, m)).astype(np.int64)
        t1 = time.perf_counter()
        oracle.gated_attention(qk, kk, vk, bk, pk, [m], hq, hkv, gain, lay.tau, rows=rows)
        t_attn = (time.perf_counter() - t1) * pairs_all / float(np.sum(rows + 1))
        sample = (f"gate over {w.n_rows} rows, select and compaction in full; attention on {len(rows)} "
                  f"evenly spaced query rows of {m}, scaled by visible (query, key) pairs")
    total_ms = (t_front + t_attn) * 1e3
    return dict(value=round(total_ms, 3), unit="ms", cores=int(threads), kind="oracle", sample=sample,
                split_ms=dict(gate_select_compact=round(t_front * 1e3, 3), attention=round(t_attn * 1e3, 3)),
                blas=blas, host_cpus=len(os.sched_getaffinity(0))), parity


def measure_extras(torch, tg, layer, w, steps, dev):
    """Measurements beside the contract line: the box's own GEMM and copy
    peaks, per-step percentiles, the layer with the Infinity Cache evicted
    before every step, and select on one prompt of 2^24 rows."""
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            ts.append((a, b))
        torch.cuda.synchronize()
        return sorted(x.elapsed_time(y) * 1e3 for x, y in ts)  # us

    def pct(v, q):
        return v[min(len(v) - 1, int(q * len(v)))]

    out = {}
    # Peaks measured here: a large bf16 GEMM (hipBLASLt through torch) and a 1 GiB copy.
    g = torch.Generator(device=dev).manual_seed(0)
    a = torch.randn(8192, 8192, generator=g, device=dev).to(torch.bfloat16)
    b = torch.randn(8192, 8192, generator=g, device=dev).to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    t = timed(lambda: torch.matmul(a, b), 10)
    gemm_tflops = 2 * 8192 ** 3 / (pct(t, 0.5) * 1e-6) / 1e12
    del a, b
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)  # 1 GiB
    dst = torch.empty_like(src)
    dst.copy_(src)
    t = timed(lambda: dst.copy_(src), 10)
    copy_gbs = 2 * src.numel() * 4 / (pct(t, 0.5) * 1e-6) / 1e9
    out["measured_peaks"] = {"bf16_gemm_8192_tflops": round(gemm_tflops, 1),
                             "device_copy_1gib_gbs_read_plus_write": round(copy_gbs, 1)}
    # Per-step percentiles (warm) and the layer with the Infinity Cache evicted first.
    t = timed(layer.run, steps)
    out["layer_us_warm"] = {"p10": round(pct(t, 0.1), 2), "p50": round(pct(t, 0.5), 2), "p90": round(pct(t, 0.9), 2)}
    del src, dst
    torch.cuda.empty_cache()
    work = algorithmic_work(w, layer.m)
    ev_read, ev_write = Evictor(torch, dev, read=True), Evictor(torch, dev, read=False)
    for name, evict, note in (
            ("cold", ev_read, "a 1 GiB device write, then a 1 GiB read, before each step: no cache holds the "
                              "layer's inputs, and the eviction leaves no dirty lines to write back"),
            ("cold_write_evicted", ev_write, "a 1 GiB device write before each step; its dirty lines are "
                                             "written back while the step runs")):
        cold = []
        for _ in range(20):
            evict()
            cold += timed(layer.run, 1)
        cold.sort()
        out[f"layer_us_{name}"] = {"p10": round(pct(cold, 0.1), 2), "p50": round(pct(cold, 0.5), 2),
                                   "p90": round(pct(cold, 0.9), 2), "note": note}
        # Per-kernel times with the caches evicted before every step.
        kc = kernel_times(torch, layer, 20, evict=evict)
        out[f"kernels_us_{name}"] = kc
        out[f"kernel_rooflines_{name}"] = rooflines_of(work, kc, name)
    del ev_read, ev_write
    # Decode after this prefill: one new token over the kept K/V cache.
    out["decode_qwen16k"] = measure_decode(torch, tg, layer, timed, pct)
    # Backward of this layer's token-gated attention (the gradient path to the gate).
    out["backward_qwen16k"] = measure_backward(torch, tg, layer, timed, pct)
    # ... and on through the score chain into the gate MLP's weights.
    out["gate_backward_qwen16k"] = measure_gate_backward(torch, tg, layer, timed, pct)
    # The full above-gate decoder layer over the kept rows, against the same layer over all rows.
    out["dense_layer_qwen16k"] = measure_dense_layer(torch, tg, layer, w, timed, pct)
    # The gated delta rule of a Gated-DeltaNet layer over the kept rows, against all rows.
    out["delta_scan_qwen16k"] = measure_delta_scan(torch, tg, layer, timed, pct)
    # Select on one prompt of 2^24 document rows: the multi-workgroup path
    # (1024 chunks of 16384 rows), arguments marshalled once outside the
    # timed region.
    from synthetic import Prompt, make_scores
    from learned_token_pruning_layer_amd._lib import seq_array
    nbig = 1 << 24
    sc = make_scores(nbig, seed=7, device=dev)
    prompts = [Prompt(0, nbig, 0, nbig, nbig // 8)]
    kept = torch.empty(tg.tg_kept_rows(prompts), dtype=torch.int32, device=dev)
    lib = tg.load()
    sa = seq_array(prompts)
    wsb = lib.tg_select_workspace_bytes(sa, 1)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    args = (sc.data_ptr(), sa, 1, kept.data_ptr(), ws.data_ptr(), wsb, stream.cuda_stream)

    def sel_big():
        if lib.tg_select_topk(*args) != 0:
            raise RuntimeError(lib.tg_last_error().decode())

    sel_big()
    t = timed(sel_big, 20)
    sel_bytes = nbig * 4 + kept.numel() * 4
    out["select_2p24_keys"] = {"us": round(pct(t, 0.5), 1),
                               "algorithmic_gb_s": round(sel_bytes / (pct(t, 0.5) * 1e-6) / 1e9, 1),
                               "note": "one prompt of 2^24 document rows, keep 1/8; chunks of 16384 rows, "
                                       "one workgroup each, reading the scores three times (first-digit "
                                       "histogram, candidate lists, placement); the other two digits and "
                                       "the counts run over the candidate lists"}
    del sc, kept, ws
    out["configs"] = measure_configs(torch, tg, dev, timed, pct)
    return out


def measure_decode(torch, tg, lay, timed, pct, reps=50):
    """One decode step per prompt over the layer's KV cache: the kept K/V
    rows of the pruned prefill with one new token appended (bias 0, next
    position). Algorithmic bytes: every cached K and V row once per KV head,
    plus its bias and position."""
    from learned_token_pruning_layer_amd._lib import kv_seq_array
    _, kk, vk = lay.qkv_kept[0]
    hq, hkv, dh = lay.hq, lay.hkv, lay.head_dim
    dev = kk.device
    segs, rows, off = [], [], 0
    for p in lay.prompts:
        n = p.k_doc + p.length - (p.doc_end - p.doc_begin)
        rows.append((off, n))
        off += n
    total = off + len(rows)
    k = torch.empty((total, hkv, dh), dtype=kk.dtype, device=dev)
    v = torch.empty_like(k)
    bias = torch.zeros(total, dtype=torch.float32, device=dev)
    pos = torch.empty(total, dtype=torch.int32, device=dev)
    g = torch.Generator(device=dev).manual_seed(5)
    dst = 0
    for (src, n) in rows:  # cache of this prompt, then its new token
        k[dst:dst + n] = kk[src:src + n].view(n, hkv, dh)
        v[dst:dst + n] = vk[src:src + n].view(n, hkv, dh)
        bias[dst:dst + n] = lay.bias_kept[src:src + n]
        pos[dst:dst + n] = lay.pos_kept[src:src + n]
        k[dst + n] = torch.randn((hkv, dh), generator=g, device=dev).to(kk.dtype)
        v[dst + n] = torch.randn((hkv, dh), generator=g, device=dev).to(kk.dtype)
        pos[dst + n] = pos[dst + n - 1] + 1
        segs.append((dst, n + 1, 1))
        dst += n + 1
    q = torch.randn((len(segs), hq, dh), generator=g, device=dev).to(kk.dtype)
    out = torch.empty_like(q)
    lib = tg.load()
    sa = kv_seq_array(segs)
    wsb = lib.tg_decode_workspace_bytes(sa, len(segs), hq, hkv, dh)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    gain = lay.layers[0].gain
    st = torch.cuda.current_stream().cuda_stream
    args = (1 if kk.dtype == torch.bfloat16 else 0, q.data_ptr(), k.data_ptr(), v.data_ptr(), bias.data_ptr(),
            pos.data_ptr(), sa, len(segs), hq, hkv, dh, gain.data_ptr(), float(lay.layers[0].tau),
            out.data_ptr(), None, ws.data_ptr(), wsb, st)

    def call():
        if lib.tg_decode_attention(*args) != 0:
            raise RuntimeError(lib.tg_last_error().decode())

    call()
    us = pct(timed(call, reps), 0.5)
    byts = total * hkv * dh * k.element_size() * 2 + total * 8
    return {"cache_rows": total, "us": round(us, 2), "algorithmic_gb_s": round(byts / (us * 1e-6) / 1e9, 1),
            "frac_hbm_peak": round(byts / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}


def measure_backward(torch, tg, lay, timed, pct, reps=20):
    """Backward of the layer's token-gated attention over its kept rows (the
    forward's output and lse, a random upstream gradient). Algorithmic work:
    five products of 2*D*Hq flop per visible pair (S, dP, dV, dK, dQ), 2.5x
    the forward's."""
    from learned_token_pruning_layer_amd._lib import seq_array
    qk, kk, vk = lay.qkv_kept[0]
    hq, hkv, dh, m = lay.hq, lay.hkv, lay.head_dim, lay.m
    q3, k3, v3 = qk.view(m, hq, dh), kk.view(m, hkv, dh), vk.view(m, hkv, dh)
    lay_l = lay.layers[0]
    out, lse = tg.tg_gated_attention(q3, k3, v3, lay.bias_kept, lay.pos_kept, lay.prompts, lay_l.gain, lay_l.tau,
                                     want_lse=True)
    g = torch.Generator(device=q3.device).manual_seed(11)
    dout = torch.randn(out.shape, generator=g, device=q3.device).to(torch.bfloat16)
    lib = tg.load()
    sa = seq_array(lay.prompts)
    wsb = lib.tg_attention_backward_workspace_bytes(sa, len(lay.prompts), hq, hkv, dh)
    ws = torch.empty(wsb, dtype=torch.uint8, device=q3.device)
    f32 = torch.float32
    dq = torch.empty((m, hq, dh), dtype=f32, device=q3.device)
    dk = torch.empty((m, hkv, dh), dtype=f32, device=q3.device)
    dv = torch.empty_like(dk)
    db = torch.empty(m, dtype=f32, device=q3.device)
    dg = torch.empty(hq, dtype=f32, device=q3.device)
    dt = torch.empty(1, dtype=f32, device=q3.device)
    st = torch.cuda.current_stream().cuda_stream
    args = (1, q3.data_ptr(), k3.data_ptr(), v3.data_ptr(), lay.bias_kept.data_ptr(), lay.pos_kept.data_ptr(), sa,
            len(lay.prompts), hq, hkv, dh, lay_l.gain.data_ptr(), float(lay_l.tau), out.data_ptr(), lse.data_ptr(),
            dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), db.data_ptr(), dg.data_ptr(),
            dt.data_ptr(), ws.data_ptr(), wsb, st)

    def call():
        if lib.tg_gated_attention_backward(*args) != 0:
            raise RuntimeError(lib.tg_last_error().decode())

    call()
    us = pct(timed(call, reps), 0.5)
    pairs = sum((p.k_doc + p.length - (p.doc_end - p.doc_begin)) * (p.k_doc + p.length - (p.doc_end - p.doc_begin) + 1)
                // 2 for p in lay.prompts)
    fl = 5 * 2 * dh * hq * pairs
    return {"kept_rows": m, "us": round(us, 1), "algorithmic_tflops": round(fl / (us * 1e-6) / 1e12, 1),
            "frac_bf16_peak": round(fl / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def measure_gate_backward(torch, tg, lay, timed, pct, reps=20):
    """Backward of the gate MLP over the layer's kept rows: the score gradient of
    a random bias gradient (sigmoid(-s) on kept document rows), then dW1, db1,
    dw2, db2 and dx (added to an fp32 [N, d] buffer). Algorithmic work: three
    products of 2*M*d*H flop (recomputed pre-activation, dx, dW1)."""
    from learned_token_pruning_layer_amd._lib import seq_array
    n, d = lay.x.shape
    h = lay.w1.shape[0]
    m = lay.m
    g = torch.Generator(device=lay.x.device).manual_seed(12)
    dbias = torch.randn(m, generator=g, device=lay.x.device)
    dsc = tg.tg_score_grad(dbias, lay.scores, lay.kept, lay.prompts)
    dx = torch.zeros((n, d), dtype=torch.float32, device=lay.x.device)
    lib = tg.load()
    wsb = lib.tg_gate_backward_workspace_bytes(n, d, h, m)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=lay.x.device)
    f32 = torch.float32
    outs = [torch.empty(s, dtype=f32, device=lay.x.device) for s in ((h, d), (h,), (h,), (1,))]
    st = torch.cuda.current_stream().cuda_stream
    args = (1, lay.x.data_ptr(), n, d, lay.w1.data_ptr(), None if lay.b1 is None else lay.b1.data_ptr(),
            lay.w2.data_ptr(), h, dsc.data_ptr(), lay.kept.data_ptr(), m, dx.data_ptr(),
            *[t.data_ptr() for t in outs], ws.data_ptr(), ws.numel(), st)

    def call():
        if lib.tg_gate_backward(*args) != 0:
            raise RuntimeError(lib.tg_last_error().decode())

    call()
    us = pct(timed(call, reps), 0.5)
    fl = 3 * 2 * m * d * h
    return {"listed_rows": m, "us": round(us, 1), "algorithmic_tflops": round(fl / (us * 1e-6) / 1e12, 1),
            "frac_bf16_peak": round(fl / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def measure_dense_layer(torch, tg, lay, w, timed, pct, reps=10):
    """One Qwen3-1.7B-shaped decoder layer above the gate (RMSNorm, QKV, per-head
    Q/K norm + rotary embedding at the original positions, token-gated attention,
    output projection, SwiGLU MLP; random weights) over the 16k layer's kept rows,
    and the same layer over all 16384 rows (every row kept, zero bias) for
    comparison. Memory: the layer's device workspace plus its K/V cache and output
    (bf16), the part of the above-gate footprint that scales with the rows."""
    import ctypes
    from synthetic import Prompt, make_dense_layer
    from learned_token_pruning_layer_amd._lib import dense_weights, seq_array
    d, hq, hkv, dh, d_ff = lay.x.shape[1], lay.hq, lay.hkv, lay.head_dim, 6144
    wts = make_dense_layer(d, hq, hkv, dh, d_ff, seed=5, device=lay.x.device)
    lib = tg.load()
    desc = dense_weights(wts, d, hq, hkv, dh)

    def one(h, bias, pos, prompts):
        m = h.shape[0]
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        sa = seq_array(prompts)
        need = lib.tg_dense_layer_workspace_bytes(sa, len(prompts), ctypes.byref(desc))
        ws = torch.empty(need, dtype=torch.uint8, device=h.device)
        out = torch.empty_like(h)
        kc = torch.empty((m, hkv, dh), dtype=h.dtype, device=h.device)
        vc = torch.empty_like(kc)
        st = torch.cuda.current_stream().cuda_stream
        args = (1, h.data_ptr(), bias.data_ptr(), pos.data_ptr(), sa, len(prompts), ctypes.byref(desc),
                out.data_ptr(), kc.data_ptr(), vc.data_ptr(), ws.data_ptr(), need, st)

        def call():
            if lib.tg_dense_layer(*args) != 0:
                raise RuntimeError(lib.tg_last_error().decode())

        call()
        us = pct(timed(call, reps), 0.5)
        pairs = sum((p.k_doc + p.length - (p.doc_end - p.doc_begin)) * (p.k_doc + p.length - (p.doc_end - p.doc_begin)
                                                                        + 1) // 2 for p in prompts)
        fl = 2 * m * d * ((hq + 2 * hkv) * dh + hq * dh + 3 * d_ff) + 4 * dh * hq * pairs
        mem = need + (2 * kc.numel() + out.numel()) * 2
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        return {"rows": m, "us": round(us, 1), "tflops": round(fl / (us * 1e-6) / 1e12, 1),
                "row_scaled_bytes": int(mem), "peak_allocated_bytes": int(peak)}

    pruned = one(lay.hidden_kept if lay.hidden_kept is not None else lay.x[lay.kept.long()].contiguous(),
                 lay.bias_kept, lay.pos_kept, lay.prompts)
    n = w.x.shape[0]
    full = one(w.x, torch.zeros(n, dtype=torch.float32, device=w.x.device),
               torch.arange(n, dtype=torch.int32, device=w.x.device), [Prompt(0, n, 0, 0, 0)])
    return {"pruned": pruned, "unpruned": full, "speedup": round(full["us"] / pruned["us"], 2),
            "memory_ratio": round(full["row_scaled_bytes"] / pruned["row_scaled_bytes"], 2),
            "peak_memory_ratio": round(full["peak_allocated_bytes"] / max(1, pruned["peak_allocated_bytes"]), 2),
            "d_ff": d_ff,
            "memory_note": "peak_allocated_bytes: torch.cuda.max_memory_allocated over the call's own "
                           "allocations (workspace, K/V cache, output), inputs excluded"}


def measure_delta_scan(torch, tg, lay, timed, pct, reps=10):
    """The gated delta rule (the token mixer of a Gated-DeltaNet layer; 16 heads,
    dk = dv = 128, synthetic normalised q/k, decays in (0.9, 1)) over the 16k
    layer's 2384 kept rows, and over all 16384 rows for comparison. Algorithmic
    work of the recurrence: 8 dk dv flop per row and head (S k, the rank-1 update,
    S q)."""
    from synthetic import Prompt, make_delta_inputs
    from learned_token_pruning_layer_amd._lib import seq_array
    lib = tg.load()
    nh = 16
    res = {}
    for name, prompts, m in (("pruned", lay.prompts, lay.m), ("unpruned", [Prompt(0, lay.x.shape[0], 0, 0, 0)],
                                                               lay.x.shape[0])):
        a = make_delta_inputs([m], nh, 128, 128, seed=7, device=lay.x.device)
        sa = seq_array(prompts)
        need = lib.tg_delta_scan_workspace_bytes(sa, len(prompts), nh, 128, 128)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=lay.x.device)
        out = torch.empty_like(a["v"])
        st = torch.cuda.current_stream().cuda_stream
        args = (1, a["q"].data_ptr(), a["k"].data_ptr(), a["v"].data_ptr(), a["g"].data_ptr(), a["beta"].data_ptr(),
                sa, len(prompts), nh, 128, 128, None, out.data_ptr(), None, ws.data_ptr(), ws.numel(), st)

        def call():
            if lib.tg_gated_delta_scan(*args) != 0:
                raise RuntimeError(lib.tg_last_error().decode())

        call()
        us = pct(timed(call, reps), 0.5)
        res[name] = {"rows": m, "us": round(us, 1),
                     "recurrence_tflops": round(8 * 128 * 128 * nh * m / (us * 1e-6) / 1e12, 2)}
    res["speedup"] = round(res["unpruned"]["us"] / res["pruned"]["us"], 2)
    return res


def measure_configs(torch, tg, dev, timed, pct):
    """The other workloads, timed the same way (whole layer and attention
    alone, p50 of event-timed reps): the 32k budget sweep, 128k at 6.25%
    with the unpruned attention over all 131072 rows beside it, and the
    ragged 8-prompt batch feeding 4 above-gate layers."""
    from synthetic import SWEEP_FRACTIONS, Prompt, doc_budget, make_workload

    def causal_flops(prompts, hq, dh):
        return sum(4 * dh * hq * p.n_kept * (p.n_kept + 1) // 2 for p in prompts)

    def run_one(w, prompts, reps, attn_reps=None, decode=False):
        lay = tg.GatedPrefillLayer(w.x, w.w1, w.w2, prompts, w.layers, w.hq, w.hkv, w.head_dim)
        lay.run()
        t_layer = pct(timed(lay.run, reps), 0.5)
        t_attn = sum(pct(timed(lambda i=i: lay.attention(i), attn_reps or reps), 0.5) for i in range(len(w.layers)))
        fl = causal_flops(prompts, w.hq, w.head_dim) * len(w.layers)
        rec = {"kept_rows": lay.m, "layer_us": round(t_layer, 1), "attention_us": round(t_attn, 1),
               "attention_tflops": round(fl / (t_attn * 1e-6) / 1e12, 1)}
        if decode:
            rec["decode_one_token"] = measure_decode(torch, tg, lay, timed, pct)
        del lay
        return rec

    out = {}
    w = make_workload("sweep32k", device=dev)
    p0 = w.prompts[0]
    sweep = []
    for frac in SWEEP_FRACTIONS:
        k = doc_budget(frac, p0.n_doc)
        sweep.append({"keep": frac, "k_doc": k, **run_one(w, [p0._replace(k_doc=k)], 30)})
    out["sweep32k"] = {"n_rows": w.n_rows, "budgets": sweep}
    del w
    torch.cuda.empty_cache()
    w = make_workload("long128k", device=dev)
    p0 = w.prompts[0]
    pruned = run_one(w, w.prompts, 20, decode=True)
    lay = tg.GatedPrefillLayer(w.x, w.w1, w.w2, w.prompts, w.layers, w.hq, w.hkv, w.head_dim)
    lay.run()
    work = algorithmic_work(w, lay.m)
    kw = kernel_times(torch, lay, 20)
    evict = Evictor(torch, dev, read=True)
    kc = kernel_times(torch, lay, 10, evict=evict)
    evict.rbuf = None
    kcw = kernel_times(torch, lay, 10, evict=evict)
    del evict, lay
    pruned["kernels_us_warm"] = kw
    pruned["kernels_us_cold"] = kc
    pruned["kernels_us_cold_write_evicted"] = kcw
    pruned["kernel_rooflines_warm"] = rooflines_of(work, kw, "warm")
    pruned["kernel_rooflines_cold"] = rooflines_of(work, kc, "cold")
    pruned["kernel_rooflines_cold_write_evicted"] = rooflines_of(work, kcw, "cold_write_evicted")
    full = run_one(w, [p0._replace(k_doc=p0.n_doc)], 3, attn_reps=3, decode=True)
    out["long128k"] = {"n_rows": w.n_rows, "k_doc": p0.k_doc, **pruned,
                       "unpruned": {k: full[k] for k in ("kept_rows", "attention_us", "attention_tflops",
                                                         "decode_one_token")},
                       "unpruned_attention_over_pruned_layer": round(full["attention_us"] / pruned["layer_us"], 1)}
    del w
    torch.cuda.empty_cache()
    w = make_workload("ragged", device=dev)
    out["ragged"] = {"n_rows": w.n_rows, "prompts": len(w.prompts), "layers": len(w.layers),
                     **run_one(w, w.prompts, 20, decode=True),
                     "note": "layer_us: one gate, one select and one compaction for all prompts, then one "
                             "attention call per layer; attention_us sums the 4 layers"}
    del w
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.traffic_from:
        traffic_summary(*args.traffic_from)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "gpus_requested": args.gpus}))
        sys.exit(2)
    import torch

    import learned_token_pruning_layer_amd as tg
    from synthetic import make_workload

    torch.cuda.set_device(0)
    dev = "cuda:0"
    w = make_workload(args.workload, device=dev)
    layer = tg.GatedPrefillLayer(w.x, w.w1, w.w2, w.prompts, w.layers, w.hq, w.hkv, w.head_dim)
    m = layer.m
    work = algorithmic_work(w, m)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        layer.run()
    torch.cuda.synchronize()

    # Timed region: exactly `steps` whole-layer steps.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        layer.run()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps

    # Per-kernel durations: events between the four launches of each step.
    names = ["gate", "select", "compact", "attention"]
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for e in evs:
        e[0].record(stream)
        layer.gate()
        e[1].record(stream)
        layer.select()
        e[2].record(stream)
        layer.compact()
        e[3].record(stream)
        layer.attention(0)
        e[4].record(stream)
    torch.cuda.synchronize()
    per = {nm: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / args.steps * 1e3 for i, nm in enumerate(names)}

    # Dominant kernel alone, back to back: average launch duration.
    dom = max(per, key=per.get)
    call = {"gate": layer.gate, "select": layer.select, "compact": layer.compact,
            "attention": lambda: layer.attention(0)}[dom]
    for _ in range(10):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    dom_us = e0.elapsed_time(e1) / args.steps * 1e3

    def measured_traffic_of(kernel):
        return measured_traffic(kernel) if args.workload == "qwen16k" else None

    def roofline(kernel, us):
        wk = work[kernel]
        if kernel == "attention":
            ach = wk["flops"] / (us * 1e-6) / 1e12
            return dict(bound="mfma", achieved=round(ach, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                        frac=round(ach / PEAK_BF16_TFLOPS, 4), traffic=measured_traffic_of(kernel))
        ach = wk["bytes"] / (us * 1e-6) / 1e9
        return dict(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(ach / PEAK_HBM_GBS, 4), traffic=measured_traffic_of(kernel))

    attn_tflops = work["attention"]["flops"] / (per["attention"] * 1e-6) / 1e12
    rec = {
        "metric": METRIC,
        "value": round(ms_per_step, 5),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.workload],
                   "n_rows": w.n_rows, "kept_rows": m, "global_batch": 1, "seq_len": w.n_rows},
        "attn_tflops": round(attn_tflops, 2),
        "attn_frac_mfma_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "kernels_us": {k: round(v, 2) for k, v in per.items()},
        "kernel_rooflines": {k: dict(roofline(k, per[k]), cache="warm") for k in names if k != "select"},
        "roofline": dict(kernel=dom, launch_us=round(dom_us, 2), **roofline(dom, dom_us)),
        "wall_s_timed": round(wall, 4),
    }
    if args.calibrate_copy:
        a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
    if not args.no_extras:
        ex = measure_extras(torch, tg, layer, w, min(args.steps, 100), dev)
        gp, cp = ex["measured_peaks"]["bf16_gemm_8192_tflops"], ex["measured_peaks"]["device_copy_1gib_gbs_read_plus_write"]
        ex["fractions_vs_measured_peaks"] = {
            "attention_of_bf16_gemm": round(attn_tflops / gp, 4),
            **{f"{k}_of_copy": round(work[k]["bytes"] / (per[k] * 1e-6) / 1e9 / cp, 4) for k in ("gate", "compact")}}
        rec["extras"] = ex
    if not args.no_cpu_baseline:
        rec["cpu_baseline"], parity = cpu_baseline(w, args.cpu_budget_s, gpu_layer=layer)
        rec["parity"] = parity
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

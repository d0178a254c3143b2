"""fp64 CPU oracle for the TokenGate pruned-prefill layer.

TEST INFRASTRUCTURE. Only the test suite, the smoke check in
__graft_entry__ and the CPU-baseline leg of bench.py may import, call or
execute anything in this package. The HIP library and its Python binding
never import it, and it imports nothing from them: the two share no code,
constants or helpers. It is written to be read against the pages, not to
be fast.

Sources (pages about "TokenGate: Adapting LLMs for Fast and
Memory-Efficient Prefill with Learned Token Pruning"):

  [DE-prune] spke.com article (German), section
             "Wie hat TokenGate das Pruning von Tokens verstanden?":
             three-phase forward; a small MLP scores every token from its
             post-attention residual at the gate layer; a top-K selector
             keeps the best-scored tokens; layers above the gate see only
             the kept tokens and build no KV for the rest; only the
             document part of the prompt can be pruned, never the question.
  [DE-attn]  same article, section "Was ist token-gated Attention?":
             each kept token's score becomes a bias on the attention logits
             above the gate; a learnable per-head gain and a learnable
             temperature (the latter for queries that now see fewer keys).
  [DE-impl]  same article, section "Wie wird TokenGate implementiert?":
             a placeholder marks the prunable document; generation takes a
             kept-prefill-token budget; the attention kernel is a key-bias
             attention.
  [TH-how]   ai4bro.com post, section on how learned token pruning works
             (same three phases; query tokens are never pruned).
  [IT-keep]  ai.info news, section "TokenGate impara quali token mantenere":
             the component ranks tokens at an intermediate layer and sends
             only the kept tokens' representations upward.
  [TH-hybrid], [DE-hybrid], [IT-hybrid]  the sections of the same three
             pages on hybrid-attention models: TokenGate also prunes at a
             Gated-DeltaNet layer of the Qwen3.5 hybrid.

The pages fix the bias only qualitatively. The form used here, on both
sides, is: logit_ij = q_i.k_j / (sqrt(D) * tau) + g_h * logsigmoid(s_j) for
kept document keys, with bias 0 for keys outside the document span, and key
j visible to query i iff pos_j <= pos_i (original positions).

Readings taken where the pages are silent (each listed in the design notes):
  * gate MLP: Linear(d->H) -> SiLU -> Linear(H->1); optional biases b1, b2
    (default zero); the input is the raw residual;
  * ties in the top-K go to the lower row id; -0 equals +0; NaN ranks
    below every number;
  * kept rows are emitted in ascending row order, prompt by prompt;
  * one gain per query head, one scalar tau dividing only the q.k term;
  * query head h reads KV head floor(h * Hkv / Hq) (contiguous groups).

Parity pins: every function here is checked in tests/ against something
other than itself (brute force on tiny inputs, closed forms, invariants, or
a library routine it reduces to). None is unpinned.
"""

from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence

import numpy as np


def _f64(a) -> np.ndarray:
    """View any array-like (NumPy array, torch CPU tensor) as fp64 NumPy."""
    if hasattr(a, "detach"):
        a = a.detach().cpu()
        if str(a.dtype) in ("torch.bfloat16", "torch.float16"):
            a = a.float()
        a = a.numpy()
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Step 1: gate score.  [DE-prune], [TH-how], [IT-keep]
# ---------------------------------------------------------------------------

def sigmoid(z: np.ndarray) -> np.ndarray:
    """Logistic function 1 / (1 + e^-z), evaluated without overflow."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z)."""
    return z * sigmoid(z)


def gate_scores(x, w1, w2, b1=None, b2: float = 0.0, block_rows: int = 8192) -> np.ndarray:
    """Score every row r of the residual x[N, d]:

        h_r = W1 x_r + b1        (W1 is [H, d], the nn.Linear layout)
        s_r = w2 . SiLU(h_r) + b2

    Returns s[N] in fp64. Rows are processed in blocks only to bound memory.
    """
    w1 = _f64(w1)
    w2 = _f64(w2).reshape(-1)
    b1v = None if b1 is None else _f64(b1).reshape(-1)
    n = int(x.shape[0])
    out = np.empty(n, dtype=np.float64)
    for r0 in range(0, n, block_rows):
        xb = _f64(x[r0:r0 + block_rows])
        h = xb @ w1.T
        if b1v is not None:
            h = h + b1v
        out[r0:r0 + xb.shape[0]] = silu(h) @ w2 + float(b2)
    return out


# ---------------------------------------------------------------------------
# Step 2: top-K selection, document rows only.  [DE-prune], [TH-how], [DE-impl]
# ---------------------------------------------------------------------------

def _doc_rows(p) -> np.ndarray:
    return np.arange(p.start + p.doc_begin, p.start + p.doc_end, dtype=np.int64)


def select_topk(scores, prompts: Sequence) -> np.ndarray:
    """Kept row ids for every prompt, concatenated in prompt order.

    For each prompt: rank its document rows by score, highest first, ties
    to the lower row id, NaN below every number (-0 and +0 compare equal);
    keep the first k_doc of them; keep every row of the prompt outside the
    document span; emit the kept rows in ascending row order.
    """
    s = np.asarray(_f64(scores) if hasattr(scores, "detach") else scores)
    out: List[np.ndarray] = []
    for p in prompts:
        if not (0 <= p.doc_begin <= p.doc_end <= p.length):
            raise ValueError("document span outside the prompt")
        if not (0 <= p.k_doc <= p.doc_end - p.doc_begin):
            raise ValueError("k_doc outside [0, n_doc]")
        rows = np.arange(p.start, p.start + p.length, dtype=np.int64)
        doc = _doc_rows(p)
        sd = s[doc]
        is_nan = np.isnan(sd)
        neg = np.where(is_nan, 0.0, -sd.astype(np.float64))
        # np.lexsort sorts by its last key first: NaN flag, then -score,
        # then row id. It is a stable sort.
        order = np.lexsort((doc, neg, is_nan))
        keep_doc = doc[order[:p.k_doc]]
        in_doc = np.zeros(p.length, dtype=bool)
        in_doc[p.doc_begin:p.doc_end] = True
        keep = np.concatenate([rows[~in_doc], keep_doc])
        out.append(np.sort(keep))
    return np.concatenate(out) if out else np.zeros(0, dtype=np.int64)


def kept_rows(prompts: Iterable) -> int:
    """M = sum over prompts of k_doc + (length - n_doc)."""
    return int(sum(p.k_doc + p.length - (p.doc_end - p.doc_begin) for p in prompts))


# ---------------------------------------------------------------------------
# Step 3: compaction.  [DE-prune] (only kept tokens go up, no KV for the
# pruned), [IT-keep]; bias per [DE-attn] in the form stated above.
# ---------------------------------------------------------------------------

def logsigmoid(s) -> np.ndarray:
    """log(sigmoid(s)) = min(s, 0) - log1p(exp(-|s|)), in fp64."""
    s = np.asarray(s, dtype=np.float64)
    return np.minimum(s, 0.0) - np.log1p(np.exp(-np.abs(s)))


def prompt_of_rows(rows: np.ndarray, prompts: Sequence) -> np.ndarray:
    """Index of the prompt that holds each row."""
    starts = np.array([p.start for p in prompts], dtype=np.int64)
    return np.searchsorted(starts, rows, side="right") - 1


def compact(kept: np.ndarray, prompts: Sequence, tensors: Sequence = (), scores=None,
            pos=None):
    """Gather the kept rows.

    Returns (gathered, pos_kept, bias_kept):
      gathered[t] = tensors[t][kept]           (row gather, bit-exact)
      pos_kept[m] = pos[kept[m]], or kept[m] - start of its prompt when no
                    position array is given
      bias_kept[m]= logsigmoid(scores[kept[m]]) for document rows, else 0
    """
    kept = np.asarray(kept, dtype=np.int64)
    gathered = [t[kept] for t in tensors]
    pid = prompt_of_rows(kept, prompts)
    starts = np.array([p.start for p in prompts], dtype=np.int64)
    if pos is None:
        pos_kept = kept - starts[pid]
    else:
        pos_kept = np.asarray(pos)[kept].astype(np.int64)
    bias = np.zeros(len(kept), dtype=np.float64)
    if scores is not None and len(kept):
        db = np.array([p.start + p.doc_begin for p in prompts], dtype=np.int64)[pid]
        de = np.array([p.start + p.doc_end for p in prompts], dtype=np.int64)[pid]
        is_doc = (kept >= db) & (kept < de)
        sk = _f64(scores)[kept] if hasattr(scores, "detach") else np.asarray(scores, np.float64)[kept]
        bias[is_doc] = logsigmoid(sk[is_doc])
    return gathered, pos_kept, bias


# ---------------------------------------------------------------------------
# Step 4: token-gated attention.  [DE-attn], [DE-prune], [DE-impl]
# ---------------------------------------------------------------------------

def gated_attention(q, k, v, bias, pos, seg_lens: Sequence[int], hq: int, hkv: int,
                    gain, tau: float, rows: Optional[np.ndarray] = None,
                    block_rows: int = 256):
    """Token-gated causal attention over packed kept rows.

    q[M, hq, D], k/v[M, hkv, D], bias[M], pos[M], gain[hq]; the packed rows
    form consecutive segments (one per prompt) of lengths seg_lens. For
    segment rows i (queries) and j (keys) and query head h with KV head
    kv = floor(h * hkv / hq):

        l_ij  = q_i . k_j / (sqrt(D) * tau) + gain[h] * bias[j]
        J_i   = { j in the segment : pos[j] <= pos[i] }
        o_i   = sum_{j in J_i} softmax_j(l_i.) v_j
        lse_i = log sum_{j in J_i} exp(l_ij)

    Returns (o[M, hq, D], lse[hq, M]) in fp64. `rows`, if given, restricts
    the queries computed to those packed row ids (other outputs are NaN).
    """
    if hq % hkv:
        raise ValueError("hq must be a multiple of hkv")
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    b = _f64(bias).reshape(-1)
    ps = np.asarray(pos.detach().cpu().numpy() if hasattr(pos, "detach") else pos, dtype=np.int64)
    g = _f64(gain).reshape(-1)
    m_tot, _, dh = qd.shape
    scale = 1.0 / (math.sqrt(dh) * float(tau))
    o = np.full((m_tot, hq, dh), np.nan)
    lse = np.full((hq, m_tot), np.nan)
    want = None
    if rows is not None:
        want = np.zeros(m_tot, dtype=bool)
        want[np.asarray(rows, dtype=np.int64)] = True
    off = 0
    for ln in seg_lens:
        ln = int(ln)
        seg = slice(off, off + ln)
        q_rows = np.arange(off, off + ln)
        if want is not None:
            q_rows = q_rows[want[off:off + ln]]
        for h in range(hq):
            kvh = (h * hkv) // hq
            kh, vh = kd[seg, kvh, :], vd[seg, kvh, :]
            bh = g[h] * b[seg]
            for i0 in range(0, len(q_rows), block_rows):
                qi = q_rows[i0:i0 + block_rows]
                logits = (qd[qi, h, :] @ kh.T) * scale + bh[None, :]
                visible = ps[seg][None, :] <= ps[qi][:, None]
                logits = np.where(visible, logits, -np.inf)
                mx = logits.max(axis=1, keepdims=True)
                e = np.exp(logits - mx)
                den = e.sum(axis=1, keepdims=True)
                o[qi, h, :] = (e @ vh) / den
                lse[h, qi] = (mx + np.log(den))[:, 0]
        off += ln
    return o, lse


# ---------------------------------------------------------------------------
# Backward of token-gated attention, and the bias -> score chain.  [DE-attn]
# (the bias on the logits is what gives the gradient a path back to the
# scorer, like a mixture-of-experts router), [TH-how] (same: the kept
# tokens' scores become the bias so the gradient reaches the scorer).
# ---------------------------------------------------------------------------

def gated_attention_backward(q, k, v, bias, pos, seg_lens: Sequence[int], hq: int, hkv: int,
                             gain, tau: float, d_out, o=None):
    """Gradients of sum(d_out * o) through token-gated attention.

    Same inputs as gated_attention, plus d_out[M, hq, D]. With
    l_ij = q_i.k_j * c + gain[h] * bias[j], c = 1 / (sqrt(D) * tau), over
    visible keys, p = softmax_j(l), o_i = sum_j p_ij v_j:

        dv_j    = sum_{h in group, i} p_ij do_i
        dp_ij   = do_i . v_j
        ds_ij   = p_ij (dp_ij - sum_j' p_ij' dp_ij')     (= p_ij (dp_ij - do_i . o_i))
        dq_i    = c * sum_j ds_ij k_j
        dk_j    = c * sum_{h in group, i} ds_ij q_i
        dbias_j = sum_h gain[h] sum_i ds_ij
        dgain_h = sum_{i,j} ds_ij bias[j]
        dtau    = -(1/tau) * sum_{h,i,j} ds_ij (q_i.k_j * c)

    `o`, if given [M, hq, D], is the forward output handed to the backward
    (the attention call's stored result, e.g. rounded to bf16); the row term
    do_i . o_i is then taken from it, as a backward that receives the
    forward's output does, instead of from the exact p @ v.

    Returns dict(dq, dk, dv, dbias, dgain, dtau) in fp64, plus, for setting
    tolerances, the sizes of the terms the scalar gradients sum (they can
    cancel to far less): dtau_abs = (1/tau) sum |ds_ij q_i.k_j c|;
    dtau_mag = (1/tau) sum p_ij (|dp_ij| + |do_i . o_i|) |q_i.k_j c| (the
    same terms before ds is formed); dgain_abs[h] = sum_ij |ds_ij bias[j]|.
    """
    if hq % hkv:
        raise ValueError("hq must be a multiple of hkv")
    qd, kd, vd, dod = _f64(q), _f64(k), _f64(v), _f64(d_out)
    b = _f64(bias).reshape(-1)
    ps = np.asarray(pos.detach().cpu().numpy() if hasattr(pos, "detach") else pos, dtype=np.int64)
    g = _f64(gain).reshape(-1)
    m_tot, _, dh = qd.shape
    c = 1.0 / (math.sqrt(dh) * float(tau))
    dq = np.zeros_like(qd)
    dk = np.zeros_like(kd)
    dv = np.zeros_like(vd)
    dbias = np.zeros(m_tot)
    dgain = np.zeros(hq)
    dgain_abs = np.zeros(hq)
    dtau = 0.0
    dtau_abs = 0.0
    dtau_mag = 0.0
    od = None if o is None else _f64(o)
    off = 0
    for ln in seg_lens:
        ln = int(ln)
        seg = slice(off, off + ln)
        vis = ps[seg][None, :] <= ps[seg][:, None]          # [query, key]
        for h in range(hq):
            kvh = (h * hkv) // hq
            qk = qd[seg, h, :] @ kd[seg, kvh, :].T            # q_i . k_j
            logits = np.where(vis, qk * c + g[h] * b[seg][None, :], -np.inf)
            e = np.exp(logits - logits.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)
            o_h = p @ vd[seg, kvh, :] if od is None else od[seg, h, :]
            do = dod[seg, h, :]
            dp = do @ vd[seg, kvh, :].T
            row = (do * o_h).sum(axis=1, keepdims=True)
            ds = p * (dp - row)
            dv[seg, kvh, :] += p.T @ do
            dq[seg, h, :] += c * (ds @ kd[seg, kvh, :])
            dk[seg, kvh, :] += c * (ds.T @ qd[seg, h, :])
            dbias[seg] += g[h] * ds.sum(axis=0)
            dgain[h] += (ds.sum(axis=0) * b[seg]).sum()
            dgain_abs[h] += np.abs(ds * b[seg][None, :]).sum()
            dtau += -(1.0 / float(tau)) * (ds * qk * c).sum()
            dtau_abs += (1.0 / float(tau)) * np.abs(ds * qk * c).sum()
            dtau_mag += (1.0 / float(tau)) * (p * (np.abs(dp) + np.abs(row)) * np.abs(qk * c)).sum()
        off += ln
    return dict(dq=dq, dk=dk, dv=dv, dbias=dbias, dgain=dgain, dtau=dtau, dtau_abs=dtau_abs,
                dtau_mag=dtau_mag, dgain_abs=dgain_abs)


def score_grad(dbias_kept, scores, kept, prompts: Sequence) -> np.ndarray:
    """d(scores) from d(bias_kept): bias = logsigmoid(s) for kept document
    rows, whose derivative is sigmoid(-s); question rows carry a constant 0
    bias and pruned rows no bias at all, so both get 0."""
    s = _f64(scores).reshape(-1)
    db = _f64(dbias_kept).reshape(-1)
    kept = np.asarray(kept, dtype=np.int64)
    out = np.zeros_like(s)
    owner = prompt_of_rows(kept, prompts)
    for m, r in enumerate(kept):
        p = prompts[owner[m]]
        if p.start + p.doc_begin <= r < p.start + p.doc_end:
            out[r] = db[m] * sigmoid(-s[r])
    return out


def gate_backward(x, w1, w2, d_scores, rows=None, b1=None):
    """Gradients of sum_r d_scores[r] * s_r through the gate MLP, the last
    link of the path from the attention bias back to the scorer.

    With z_r = W1 x_r + b1, a_r = SiLU(z_r) and s_r = w2 . a_r + b2:

        dz_r  = d_scores[r] * w2 * SiLU'(z_r),   SiLU'(z) = sig(z) (1 + z (1 - sig(z)))
        dW1   = sum_r dz_r x_r^T        db1 = sum_r dz_r
        dw2   = sum_r d_scores[r] a_r   db2 = sum_r d_scores[r]
        dx_r  = W1^T dz_r

    The sums run over `rows` (every row if None); rows outside it are taken
    to have d_scores = 0. Returns dict(dx [len(rows), d] in the order of
    `rows`, dw1 [H, d], db1 [H], dw2 [H], db2) in fp64.
    """
    xd = _f64(x)
    w1d = _f64(w1)
    w2d = _f64(w2).reshape(-1)
    ds = _f64(d_scores).reshape(-1)
    n = xd.shape[0]
    idx = np.arange(n, dtype=np.int64) if rows is None else np.asarray(
        rows.detach().cpu().numpy() if hasattr(rows, "detach") else rows, dtype=np.int64)
    xr = xd[idx]
    z = xr @ w1d.T
    if b1 is not None:
        z = z + _f64(b1).reshape(-1)
    sg = sigmoid(z)
    a = z * sg
    dsr = ds[idx]
    dz = dsr[:, None] * w2d[None, :] * (sg * (1.0 + z * (1.0 - sg)))
    return dict(dx=dz @ w1d, dw1=dz.T @ xr, db1=dz.sum(axis=0), dw2=(dsr[:, None] * a).sum(axis=0),
                db2=float(dsr.sum()))


# ---------------------------------------------------------------------------
# Next step after prefill: decode over the pruned KV cache.  [DE-prune] (the
# layers above the gate build no KV for pruned tokens, so their cache holds
# only the kept rows), [DE-attn] (each kept token's bias sits on the
# attention logits of those layers), [DE-impl] (generation after a pruned
# prefill). Readings: the bias stays on the cached keys' logits while
# generating; newly generated tokens are not document tokens, so their bias
# is 0; causality by original position as in prefill.
# ---------------------------------------------------------------------------

def decode_attention(q_new, k, v, bias, pos, segs: Sequence, hq: int, hkv: int, gain, tau: float):
    """Attention of newly generated tokens over the pruned KV cache.

    segs: (start, length, n_new) per sequence: cache rows
    [start, start + length), whose last n_new rows are the new tokens
    (appended before the call, with their own bias and position).
    q_new[R, hq, D]: the new tokens' queries, sequence by sequence
    (R = sum n_new). For new token t of a sequence (cache row
    i = start + length - n_new + t) and query head h, kv = floor(h*hkv/hq):

        l_j = q . k_j / (sqrt(D) * tau) + gain[h] * bias[j],
              over cache rows j of the sequence with pos[j] <= pos[i]
        o   = sum_j softmax(l)_j v_j,   lse = log sum_j exp(l_j)

    Returns (o[R, hq, D], lse[hq, R]) in fp64, one query at a time.
    """
    if hq % hkv:
        raise ValueError("hq must be a multiple of hkv")
    qd, kd, vd = _f64(q_new), _f64(k), _f64(v)
    b = _f64(bias).reshape(-1)
    ps = np.asarray(pos.detach().cpu().numpy() if hasattr(pos, "detach") else pos, dtype=np.int64)
    g = _f64(gain).reshape(-1)
    n_out, _, dh = qd.shape
    scale = 1.0 / (math.sqrt(dh) * float(tau))
    o = np.zeros((n_out, hq, dh))
    lse = np.zeros((hq, n_out))
    r = 0
    for start, length, n_new in segs:
        start, length, n_new = int(start), int(length), int(n_new)
        if not (0 <= n_new <= length):
            raise ValueError("n_new outside [0, length]")
        keys = np.arange(start, start + length)
        for t in range(n_new):
            i = start + length - n_new + t
            vis = keys[ps[keys] <= ps[i]]
            for h in range(hq):
                kvh = (h * hkv) // hq
                logits = (kd[vis, kvh, :] @ qd[r, h, :]) * scale + g[h] * b[vis]
                mx = logits.max()
                e = np.exp(logits - mx)
                o[r, h, :] = (e @ vd[vis, kvh, :]) / e.sum()
                lse[h, r] = mx + math.log(e.sum())
            r += 1
    if r != n_out:
        raise ValueError("q_new rows do not match the segments' n_new")
    return o, lse


# ---------------------------------------------------------------------------
# The whole layer, in the pages' order.
# ---------------------------------------------------------------------------
# The full above-gate layer over the kept rows.  [DE-prune] (the layers above
# the gate process only the kept tokens and build no KV for the others),
# [IT-keep] (only the kept tokens' representations go up). The layer itself is
# the model's own decoder layer, unchanged: for the Qwen3 family, RMSNorm, a
# QKV projection, RMSNorm of every query and key head, rotary position
# embedding by the token's original position, attention (here token-gated),
# the output projection and a residual add, then RMSNorm, a SwiGLU MLP and a
# second residual add.
# ---------------------------------------------------------------------------

def rms_norm(x, w, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * w over the last axis."""
    xd = _f64(x)
    return xd / np.sqrt((xd * xd).mean(axis=-1, keepdims=True) + eps) * _f64(w)


def rope(x, pos, theta: float) -> np.ndarray:
    """Rotary embedding of x [M, heads, D] at positions pos [M]: element i of
    the first half pairs with element i + D/2 and the pair turns by the angle
    pos * theta^(-2i/D)."""
    xd = _f64(x)
    dh = xd.shape[-1]
    half = dh // 2
    inv = float(theta) ** (-2.0 * np.arange(half) / dh)
    ps = np.asarray(pos.detach().cpu().numpy() if hasattr(pos, "detach") else pos, dtype=np.float64)
    ang = ps[:, None] * inv[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = xd[..., :half], xd[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def linear(x, w, residual=None) -> np.ndarray:
    """x W^T (+ residual), W in the nn.Linear layout [out, in]."""
    y = _f64(x) @ _f64(w).T
    return y if residual is None else y + _f64(residual)


def swiglu(x, w_gate, w_up) -> np.ndarray:
    """SiLU(x Wg^T) * (x Wu^T), the gated input of the MLP's down projection."""
    return silu(linear(x, w_gate)) * linear(x, w_up)


def dense_layer(h, pos_kept, bias_kept, seg_lens: Sequence[int], w: dict, hq: int, hkv: int,
                head_dim: int) -> dict:
    """One decoder layer above the gate, over the kept rows h [M, d] at their
    original positions, with token-gated attention. w: ln1 [d], wqkv
    [(hq + 2 hkv) D, d] (q rows, then k, then v), q_norm [D], k_norm [D], wo
    [d, hq D], ln2 [d], w_gate [I, d], w_up [I, d], w_down [d, I], gain [hq],
    tau, eps, theta. Returns the layer output and the intermediates in fp64."""
    hd = _f64(h)
    m = hd.shape[0]
    dq = hq * head_dim
    dk = hkv * head_dim
    eps, theta = float(w["eps"]), float(w["theta"])
    a = rms_norm(hd, w["ln1"], eps)
    qkv = a @ _f64(w["wqkv"]).T
    q = rope(rms_norm(qkv[:, :dq].reshape(m, hq, head_dim), w["q_norm"], eps), pos_kept, theta)
    k = rope(rms_norm(qkv[:, dq:dq + dk].reshape(m, hkv, head_dim), w["k_norm"], eps), pos_kept, theta)
    v = qkv[:, dq + dk:].reshape(m, hkv, head_dim)
    o, _ = gated_attention(q, k, v, bias_kept, pos_kept, seg_lens, hq, hkv, w["gain"], w["tau"])
    h2 = linear(o.reshape(m, dq), w["wo"], hd)
    a2 = rms_norm(h2, w["ln2"], eps)
    mlp = swiglu(a2, w["w_gate"], w["w_up"])
    return dict(out=linear(mlp, w["w_down"], h2), h2=h2, q=q, k=k, v=v, attn=o, mlp=mlp)


# ---------------------------------------------------------------------------
# Pruning at a Gated-DeltaNet layer.  [TH-hybrid] ai4bro.com post, section on
# hybrid-attention models, [DE-hybrid] spke.com article, section on hybrid
# attention, [IT-hybrid] ai.info news, section on hybrid models: the gate can
# sit on a Gated-DeltaNet layer of the Qwen3.5 hybrid, and the layers above it
# then run on the kept tokens only. A Gated-DeltaNet layer's token mixer is
# the gated delta rule (its published definition), run here over the kept
# rows of each prompt in their order:
#     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
#     o_t = S_t q_t,
# with a state S [dv, dk] per prompt and head.
# ---------------------------------------------------------------------------

def gated_delta_scan(q, k, v, g, beta, seg_lens: Sequence[int], state0=None):
    """The gated delta rule over packed prompts. q, k [M, H, dk], v [M, H, dv],
    g (log decay) and beta [M, H]; state0 [n_prompts, H, dv, dk] or None
    (zero). Returns (o [M, H, dv], states [n_prompts, H, dv, dk]) in fp64.
    The product S (I - beta k k^T) is applied as S - beta (S k) k^T."""
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    gd, bd = _f64(g), _f64(beta)
    m_tot, nh, dk = kd.shape
    dv = vd.shape[2]
    o = np.zeros((m_tot, nh, dv))
    states = np.zeros((len(seg_lens), nh, dv, dk)) if state0 is None else _f64(state0).copy()
    off = 0
    for p, ln in enumerate(seg_lens):
        for t in range(off, off + int(ln)):
            for h in range(nh):
                sm = states[p, h]
                a, b = math.exp(gd[t, h]), bd[t, h]
                sm = a * (sm - b * np.outer(sm @ kd[t, h], kd[t, h])) + b * np.outer(vd[t, h], kd[t, h])
                states[p, h] = sm
                o[t, h] = sm @ qd[t, h]
        off += int(ln)
    return o, states


# ---------------------------------------------------------------------------

def gated_prefill(x, w1, w2, prompts: Sequence, layers: Sequence = (), b1=None, b2: float = 0.0,
                  hq: int = 0, hkv: int = 0, head_dim: int = 0, pos=None,
                  decision_dtype=None, scores=None, attn_rows=None) -> dict:
    """Gate -> select -> compact -> token-gated attention for every layer.

    layers: objects with .q [N, hq*D], .k/.v [N, hkv*D], .gain [hq], .tau.
    decision_dtype: if set (np.float32), the top-K decision is taken on the
    scores rounded to that type, the precision the GPU path decides in; the
    bias still uses the fp64 scores.
    scores: optional precomputed scores (skips the gate).
    """
    s = gate_scores(x, w1, w2, b1, b2) if scores is None else _f64(scores)
    s_dec = s if decision_dtype is None else s.astype(decision_dtype)
    kept = select_topk(s_dec, prompts)
    m = len(kept)
    seg_lens = [p.k_doc + p.length - (p.doc_end - p.doc_begin) for p in prompts]
    _, pos_kept, bias = compact(kept, prompts, (), s, pos)
    outs = []
    for layer in layers:
        (qk, kk, vk), _, _ = compact(kept, prompts, (layer.q, layer.k, layer.v))
        qk = _f64(qk).reshape(m, hq, head_dim)
        kk = _f64(kk).reshape(m, hkv, head_dim)
        vk = _f64(vk).reshape(m, hkv, head_dim)
        o, lse = gated_attention(qk, kk, vk, bias, pos_kept, seg_lens, hq, hkv, layer.gain,
                                 layer.tau, rows=attn_rows)
        outs.append((o, lse))
    return dict(scores=s, kept=kept, pos_kept=pos_kept, bias=bias, attn=outs, seg_lens=seg_lens)

"""Pure-Python brute-force definitions used to pin the oracle on tiny inputs.

Each function computes its result by the most literal route available
(nested loops, rank counting, the multiplicative form of the bias) rather
than by the oracle's NumPy formulation, so a slip in either shows up as a
disagreement.
"""

import math


def gate(x, w1, w2, b1=None, b2=0.0):
    """s_r = sum_h w2[h] * SiLU(sum_c w1[h][c] x[r][c] + b1[h]) + b2, with
    SiLU(a) written as a / (1 + e^-a)."""
    out = []
    for row in x:
        s = float(b2)
        for h in range(len(w1)):
            a = 0.0 if b1 is None else float(b1[h])
            for c in range(len(row)):
                a += float(w1[h][c]) * float(row[c])
            if a >= 0:
                silu = a / (1.0 + math.exp(-a))
            else:
                silu = a * math.exp(a) / (1.0 + math.exp(a))
            s += float(w2[h]) * silu
        out.append(s)
    return out


def ranks_before(a, ia, b, ib):
    """True if document row ia (score a) ranks before row ib (score b):
    higher score first, NaN last, ties to the lower row id."""
    an, bn = math.isnan(a), math.isnan(b)
    if an or bn:
        if an and bn:
            return ia < ib
        return bn
    if a != b:
        return a > b
    return ia < ib


def select(scores, prompts):
    """Row r of a prompt's document is kept iff fewer than k_doc document
    rows rank before it; rows outside the document are always kept."""
    kept = []
    for p in prompts:
        doc = range(p.start + p.doc_begin, p.start + p.doc_end)
        for r in range(p.start, p.start + p.length):
            if r not in doc:
                kept.append(r)
                continue
            before = sum(1 for r2 in doc if r2 != r and ranks_before(scores[r2], r2, scores[r], r))
            if before < p.k_doc:
                kept.append(r)
    return kept


def attention_multiplicative(q, k, v, s, is_doc, pos, seg_lens, hq, hkv, gain, tau):
    """o_i = sum_j w_ij v_j / sum_j w_ij with
    w_ij = exp(q_i.k_j / (sqrt(D) tau)) * sigmoid(s_j)^gain[h] for document
    keys and exp(q_i.k_j / (sqrt(D) tau)) for the rest, over visible keys
    (pos_j <= pos_i) of the same segment. Also returns log sum_j w_ij."""
    m = len(q)
    d = len(q[0][0])
    o = [[[0.0] * d for _ in range(hq)] for _ in range(m)]
    lse = [[0.0] * m for _ in range(hq)]
    off = 0
    for ln in seg_lens:
        for h in range(hq):
            kv = (h * hkv) // hq
            for i in range(off, off + ln):
                den = 0.0
                num = [0.0] * d
                for j in range(off, off + ln):
                    if pos[j] > pos[i]:
                        continue
                    dot = sum(q[i][h][c] * k[j][kv][c] for c in range(d))
                    w = math.exp(dot / (math.sqrt(d) * tau))
                    if is_doc[j]:
                        w *= (1.0 / (1.0 + math.exp(-s[j]))) ** gain[h]
                    den += w
                    for c in range(d):
                        num[c] += w * v[j][kv][c]
                for c in range(d):
                    o[i][h][c] = num[c] / den
                lse[h][i] = math.log(den)
        off += ln
    return o, lse


def decode_attention(q_new, k, v, bias, pos, segs, hq, hkv, gain, tau):
    """Pure-Python decode over a cache: for each new token (the last n_new
    rows of each segment) and head, o = sum_j w_j v_j / sum_j w_j with
    w_j = exp(q.k_j / (sqrt(D) tau) + gain[h] bias[j]) over cache rows
    j with pos[j] <= pos[new row]."""
    d = len(k[0][0])
    out, lse = [], [[] for _ in range(hq)]
    r = 0
    for start, length, n_new in segs:
        for t in range(n_new):
            i = start + length - n_new + t
            row = []
            for h in range(hq):
                kv = (h * hkv) // hq
                den, num = 0.0, [0.0] * d
                for j in range(start, start + length):
                    if pos[j] > pos[i]:
                        continue
                    dot = sum(q_new[r][h][c] * k[j][kv][c] for c in range(d))
                    w = math.exp(dot / (math.sqrt(d) * tau) + gain[h] * bias[j])
                    den += w
                    for c in range(d):
                        num[c] += w * v[j][kv][c]
                row.append([x / den for x in num])
                lse[h].append(math.log(den))
            out.append(row)
            r += 1
    return out, lse

"""The oracle's pins must catch plausible mistakes in the oracle itself.

Each case plants one mistake (a dropped term, a wrong sign, index or operand, a
wrong tie order) into a scratch copy of `oracle/tokengate.py`, on the CPU, and
runs the pin tests against that copy in a subprocess; at least one pin has to
fail. A case whose text no longer occurs in the oracle fails too, so the list
follows edits of the oracle.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (what the mistake is, text in the oracle, planted replacement)
MUTATIONS = [
    ("bias scaled by 1/tau as well", "* scale + bh[None, :]", "* scale + bh[None, :] / float(tau)"),
    ("gain of the KV head instead of the query head", "bh = g[h] * b[seg]", "bh = g[kvh] * b[seg]"),
    ("strict causal mask (a query does not see itself)", "<= ps[qi][:, None]", "< ps[qi][:, None]"),
    ("first gate bias dropped", "h = h + b1v", "h = h"),
    ("SiLU with the wrong sign", "return z * sigmoid(z)", "return z * sigmoid(-z)"),
    ("ties broken towards the higher row", "order = np.lexsort((doc, neg, is_nan))",
     "order = np.lexsort((-doc, neg, is_nan))"),
    ("query head mapped to the wrong KV head", "kvh = (h * hkv) // hq\n            kh, vh",
     "kvh = h % hkv\n            kh, vh"),
    ("scale 1/(D tau) instead of 1/(sqrt(D) tau)", "scale = 1.0 / (math.sqrt(dh) * float(tau))\n    o = np.full",
     "scale = 1.0 / (dh * float(tau))\n    o = np.full"),
    ("log-sigmoid with the wrong sign of the log term", "np.minimum(s, 0.0) - np.log1p",
     "np.minimum(s, 0.0) + np.log1p"),
    ("bias also on question keys", "bias[is_doc] = logsigmoid(sk[is_doc])", "bias[:] = logsigmoid(sk)"),
    ("keeps the lowest-scored rows", "keep_doc = doc[order[:p.k_doc]]",
     "keep_doc = doc[order[-p.k_doc:]] if p.k_doc else doc[:0]"),
    ("second gate bias dropped", "out[r0:r0 + xb.shape[0]] = silu(h) @ w2 + float(b2)",
     "out[r0:r0 + xb.shape[0]] = silu(h) @ w2"),
    ("decode: kept-token bias dropped", "* scale + g[h] * b[vis]", "* scale"),
    ("decode: a new token does not see itself", "vis = keys[ps[keys] <= ps[i]]", "vis = keys[ps[keys] < ps[i]]"),
    ("decode: queries placed at the first rows of the cache", "            i = start + length - n_new + t",
     "            i = start + t"),
    ("decode: query head mapped to the wrong KV head", "kvh = (h * hkv) // hq\n                logits",
     "kvh = h % hkv\n                logits"),
    ("decode: scale 1/(D tau)", "scale = 1.0 / (math.sqrt(dh) * float(tau))\n    o = np.zeros",
     "scale = 1.0 / (dh * float(tau))\n    o = np.zeros"),
    ("backward: softmax Jacobian without its row term", "ds = p * (dp - row)", "ds = p * dp"),
    ("backward: row term from the exact output although one is given",
     "o_h = p @ vd[seg, kvh, :] if od is None else od[seg, h, :]", "o_h = p @ vd[seg, kvh, :]"),
    ("backward: given output read at the KV head", "else od[seg, h, :]", "else od[seg, kvh, :]"),
    ("backward: dk without the logit scale", "dk[seg, kvh, :] += c * (ds.T @ qd[seg, h, :])",
     "dk[seg, kvh, :] += ds.T @ qd[seg, h, :]"),
    ("backward: bias gradient without the gain", "dbias[seg] += g[h] * ds.sum(axis=0)", "dbias[seg] += ds.sum(axis=0)"),
    ("backward: temperature gradient with the wrong sign", "dtau += -(1.0 / float(tau))", "dtau += (1.0 / float(tau))"),
    ("score gradient through sigmoid(+s)", "out[r] = db[m] * sigmoid(-s[r])", "out[r] = db[m] * sigmoid(s[r])"),
    ("gate backward: SiLU' taken as sigmoid", "(sg * (1.0 + z * (1.0 - sg)))", "(sg)"),
    ("gate backward: dz without w2", "dz = dsr[:, None] * w2d[None, :] * ", "dz = dsr[:, None] * "),
    ("gate backward: first bias left out of the recomputed pre-activation", "        z = z + _f64(b1).reshape(-1)\n    sg",
     "        z = z\n    sg"),
    ("gate backward: dw2 from the pre-activation", "dw2=(dsr[:, None] * a).sum(axis=0)", "dw2=(dsr[:, None] * z).sum(axis=0)"),
    ("rms norm without eps", "np.sqrt((xd * xd).mean(axis=-1, keepdims=True) + eps)",
     "np.sqrt((xd * xd).mean(axis=-1, keepdims=True))"),
    ("rope pairs adjacent elements", "x1, x2 = xd[..., :half], xd[..., half:]", "x1, x2 = xd[..., 0::2], xd[..., 1::2]"),
    ("rope turns the wrong way", "[x1 * c - x2 * s, x2 * c + x1 * s]", "[x1 * c + x2 * s, x2 * c - x1 * s]"),
    ("rope frequency exponent -i/D", "inv = float(theta) ** (-2.0 * np.arange(half) / dh)",
     "inv = float(theta) ** (-1.0 * np.arange(half) / dh)"),
    ("key heads left without their norm", "k = rope(rms_norm(qkv[:, dq:dq + dk].reshape(m, hkv, head_dim), w[\"k_norm\"], eps)",
     "k = rope(qkv[:, dq:dq + dk].reshape(m, hkv, head_dim)"),
    ("SiLU on the up projection instead of the gate", "return silu(linear(x, w_gate)) * linear(x, w_up)",
     "return linear(x, w_gate) * silu(linear(x, w_up))"),
    ("output projection without the residual", "h2 = linear(o.reshape(m, dq), w[\"wo\"], hd)",
     "h2 = linear(o.reshape(m, dq), w[\"wo\"])"),
    ("delta rule: decay applied after the new value is written",
     "sm = a * (sm - b * np.outer(sm @ kd[t, h], kd[t, h])) + b * np.outer(vd[t, h], kd[t, h])",
     "sm = a * (sm - b * np.outer(sm @ kd[t, h], kd[t, h]) + b * np.outer(vd[t, h], kd[t, h]))"),
    ("delta rule: erase term added instead of subtracted", "sm = a * (sm - b * np.outer(sm @ kd[t, h]",
     "sm = a * (sm + b * np.outer(sm @ kd[t, h]"),
    ("delta rule: output read from the state before the update", "                states[p, h] = sm\n                o[t, h] = sm @ qd[t, h]",
     "                o[t, h] = states[p, h] @ qd[t, h]\n                states[p, h] = sm"),
    ("second norm over the layer input instead of the attention residual", "a2 = rms_norm(h2, w[\"ln2\"], eps)",
     "a2 = rms_norm(hd, w[\"ln2\"], eps)"),
]


def _run_one(tmp_root, idx, old, new):
    """Plant one mistake into a scratch copy of the oracle and run the pins on it."""
    src = open(os.path.join(ROOT, "oracle", "tokengate.py")).read()
    if src.count(old) != 1:
        return None
    work = os.path.join(tmp_root, f"m{idx}")
    for d in ("oracle", "synthetic", "tests"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(work, d),
                        ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutations.py"))
    with open(os.path.join(work, "oracle", "tokengate.py"), "w") as f:
        f.write(src.replace(old, new))
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1", OMP_NUM_THREADS="1")
    return subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-x", "-q",
                           "-p", "no:cacheprovider", "-m", "not gpu"],
                          cwd=work, env=env, capture_output=True, text=True, timeout=900)


@pytest.fixture(scope="module")
def mutation_runs(tmp_path_factory):
    """Every planted mistake's pin run, several at a time (each is its own process)."""
    import concurrent.futures
    root = str(tmp_path_factory.mktemp("mutations"))
    workers = max(1, min(8, (os.cpu_count() or 2) - 1))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        futs = {m[0]: ex.submit(_run_one, root, i, m[1], m[2]) for i, m in enumerate(MUTATIONS)}
        return {k: f.result() for k, f in futs.items()}


@pytest.mark.parametrize("what,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(mutation_runs, what, old, new):
    r = mutation_runs[what]
    assert r is not None, f"mutation text not found once in the oracle: {old!r}"
    assert r.returncode != 0, f"planted mistake survived every pin: {what}\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
